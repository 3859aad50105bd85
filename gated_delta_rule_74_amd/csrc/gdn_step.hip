// Single-token decode step of the gated delta rule: one step of the
// recurrence from a carried fp32 state (the O(1)-state read/write of "GDN &
// MLA Mechanism Deep-Dive", Intuition; the delta rule of "HyMo-434M
// documentation portal", 01 GDN RECURRENCE).
//
// With r = h^T q, u = h^T k, s = k . q and alpha = exp(g A):
//   o  = alpha (r - beta s u) + beta s v
//   h' = alpha h + k (beta (v - alpha u))^T
// which is h' = alpha (h - beta k u^T) + beta k v^T followed by o = h'^T q,
// reading the state once and writing it once. Additive form: o = alpha r +
// beta s v, h' = alpha h + beta k v^T.
//
// One wave per (sequence, head); lane j owns value column j (and j + 64 when
// dv > 64), so every state row is one coalesced access across the wave and
// the reductions over the key index are plain per-lane sums in a fixed order.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

__device__ __forceinline__ float lane_bcast(float x, int i) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}

template <bool BF, int NCOL, bool KEEP>
__global__ __launch_bounds__(NTHR) void step_kernel(StepArgs a) {
    using S = typename Op<BF>::S;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nh = blockIdx.x * NWAVE + wave;
    if (nh >= a.N * a.H) return;
    const int h = nh % a.H, dk = a.dk, dv = a.dv;
    const S *q = (const S *)a.q + (size_t)nh * dk;
    const S *k = (const S *)a.k + (size_t)nh * dk;
    const S *v = (const S *)a.v + (size_t)nh * dv;
    S *o = (S *)a.o + (size_t)nh * dv;
    const float *hin = a.h_in ? a.h_in + (size_t)nh * dk * dv : nullptr;
    float *hout = a.h_out + (size_t)nh * dk * dv;

    const float A = -expf(a.A_log[h]);
    const float alpha = expf(a.g[nh] * A), beta = a.beta[nh];
    const float qa = lane < dk ? to_f(q[lane]) : 0.f, ka = lane < dk ? to_f(k[lane]) : 0.f;
    const float qb = lane + 64 < dk ? to_f(q[lane + 64]) : 0.f;
    const float kb = lane + 64 < dk ? to_f(k[lane + 64]) : 0.f;
    // s = k . q, butterfly sum (same value and order on every lane)
    float sk = qa * ka + qb * kb;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sk += __shfl_xor(sk, off, 64);

    int col[NCOL];
    bool ok[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
        col[c] = lane + 64 * c;
        ok[c] = col[c] < dv;
    }
    float r[NCOL], u[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) r[c] = u[c] = 0.f;

    constexpr int KR = KEEP ? 64 : 1;
    float hr[KR][NCOL];
    if (hin) {
        if (KEEP) {
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                if (i < dk) {
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) hr[i][c] = ok[c] ? hin[(size_t)i * dv + col[c]] : 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                if (i < dk) {
                    const float qi = lane_bcast(qa, i), ki = lane_bcast(ka, i);
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) {
                        r[c] += hr[i][c] * qi;
                        u[c] += hr[i][c] * ki;
                    }
                }
            }
        } else {
            for (int i = 0; i < dk; ++i) {
                const float qi = i < 64 ? lane_bcast(qa, i) : lane_bcast(qb, i - 64);
                const float ki = i < 64 ? lane_bcast(ka, i) : lane_bcast(kb, i - 64);
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                    const float x = ok[c] ? hin[(size_t)i * dv + col[c]] : 0.f;
                    r[c] += x * qi;
                    u[c] += x * ki;
                }
            }
        }
    }
    float w[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
        const float vj = ok[c] ? to_f(v[col[c]]) : 0.f;
        float oj;
        if (a.additive) {
            oj = alpha * r[c] + beta * sk * vj;
            w[c] = beta * vj;
        } else {
            oj = alpha * (r[c] - beta * sk * u[c]) + beta * sk * vj;
            w[c] = beta * (vj - alpha * u[c]);
        }
        if (ok[c]) o[col[c]] = from_f<BF>(oj);
    }
    if (KEEP) {
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            if (i < dk) {
                const float ki = lane_bcast(ka, i);
#pragma unroll
                for (int c = 0; c < NCOL; ++c)
                    if (ok[c]) hout[(size_t)i * dv + col[c]] = (hin ? alpha * hr[i][c] : 0.f) + ki * w[c];
            }
        }
    } else {
        for (int i = 0; i < dk; ++i) {
            const float ki = i < 64 ? lane_bcast(ka, i) : lane_bcast(kb, i - 64);
#pragma unroll
            for (int c = 0; c < NCOL; ++c) {
                if (ok[c]) {
                    const float x = hin ? hin[(size_t)i * dv + col[c]] : 0.f;
                    hout[(size_t)i * dv + col[c]] = alpha * x + ki * w[c];
                }
            }
        }
    }
}

template <bool BF> static hipError_t step_inst(const StepArgs &a, hipStream_t st) {
    const int grid = (a.N * a.H + NWAVE - 1) / NWAVE;
    const bool keep = a.dk <= 64;
    if (a.dv <= 64) {
        if (keep) hipLaunchKernelGGL((step_kernel<BF, 1, true>), dim3(grid), dim3(NTHR), 0, st, a);
        else hipLaunchKernelGGL((step_kernel<BF, 1, false>), dim3(grid), dim3(NTHR), 0, st, a);
    } else {
        if (keep) hipLaunchKernelGGL((step_kernel<BF, 2, true>), dim3(grid), dim3(NTHR), 0, st, a);
        else hipLaunchKernelGGL((step_kernel<BF, 2, false>), dim3(grid), dim3(NTHR), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, bool bf16, hipStream_t st) {
    return bf16 ? step_inst<true>(a, st) : step_inst<false>(a, st);
}

} // namespace gdn
