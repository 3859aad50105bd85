// Decode step of the gated delta rule: S consecutive tokens (S = 1: one
// step; S > 1: e.g. the draft tokens of a multi-token prediction) of the
// recurrence from a carried fp32 state (the O(1)-state read/write of "GDN &
// MLA Mechanism Deep-Dive", Intuition; the delta rule of "HyMo-434M
// documentation portal", 01 GDN RECURRENCE).
//
// With r = h^T q, u = h^T k, s = k . q and alpha = exp(g A):
//   o  = alpha (r - beta s u) + beta s v
//   h' = alpha h + k (beta (v - alpha u))^T
// which is h' = alpha (h - beta k u^T) + beta k v^T followed by o = h'^T q,
// reading the state once and writing it once per call: for S tokens the state
// stays in registers between tokens (heads up to 64 wide; wider heads read
// and write it per token). Additive form: o = alpha r + beta s v,
// h' = alpha h + beta k v^T.
//
// One wave per (sequence, head); lane j owns value column j (and j + 64 when
// dv > 64), so every state row is one coalesced access across the wave and
// the reductions over the key index are per-lane sums in a fixed order. With
// dk <= 64 the state stays in registers, and each token's q and k pass
// through the wave's own LDS so that every lane reads 4 key rows' values with
// one broadcast read; the sums run over eight interleaved row sets. Calls of
// 2 to 4 tokens on heads up to 64 wide load all their tokens' inputs first
// (step_pre_kernel).
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

__device__ __forceinline__ float lane_bcast(float x, int i) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}

// ONE: a single token per call (the loop below is then straight-line code and
// the state needs no registers beyond one token's update)
template <bool BF, int NCOL, bool KEEP, bool ONE>
__global__ __launch_bounds__(NTHR) void step_kernel(StepArgs a) {
    using S = typename Op<BF>::S;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nh = blockIdx.x * NWAVE + wave;
    if (nh >= a.N * a.H) return;
    const int seq = nh / a.H, h = nh % a.H, dk = a.dk, dv = a.dv;
    const float *hin = a.h_in ? a.h_in + (size_t)nh * dk * dv : nullptr;
    float *hout = a.h_out + (size_t)nh * dk * dv;
    const float A = -expf(a.A_log[h]);

    int col[NCOL];
    bool ok[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
        col[c] = lane + 64 * c;
        ok[c] = col[c] < dv;
    }
    // KEEP: the state rows stay in registers across the tokens of the call;
    // rows past dk hold zeros, so whole groups of 4 rows can be processed,
    // and each token's q and k go through the wave's LDS (4-row broadcasts)
    constexpr int KR = KEEP ? 64 : 1;
    constexpr int RS = 8; // interleaved row sets of the reductions (divides 64)
    __shared__ __attribute__((aligned(16))) float qk_s[NWAVE][2][64];
    float *qs = qk_s[wave][0], *ks = qk_s[wave][1];
    float hr[KR][NCOL];
    if (KEEP) {
#pragma unroll
        for (int i = 0; i < KR; ++i)
#pragma unroll
            for (int c = 0; c < NCOL; ++c) hr[i][c] = 0.f;
    }
    if (KEEP && hin) {
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            if (i < dk) {
#pragma unroll
                for (int c = 0; c < NCOL; ++c) hr[i][c] = ok[c] ? hin[(size_t)i * dv + col[c]] : 0.f;
            }
        }
    }
    bool have = hin != nullptr; // a state to decay (false: zero state)
    const int NT = ONE ? 1 : a.S; // tokens of this call
    for (int t = 0; t < NT; ++t) {
        // token t of sequence seq, head h ([N, S, H, *] layouts)
        const size_t tok = ((size_t)seq * NT + t) * a.H + h;
        const S *q = (const S *)a.q + tok * dk;
        const S *k = (const S *)a.k + tok * dk;
        const S *v = (const S *)a.v + tok * dv;
        S *o = (S *)a.o + tok * dv;
        const float *src = t == 0 ? hin : hout; // state before this token (not KEEP)

        const float alpha = expf(gate_of(a.g[tok], a.logits) * A), beta = gate_of(a.beta[tok], a.logits);
        const float qa = lane < dk ? to_f(q[lane]) : 0.f;
        const float qb = lane + 64 < dk ? to_f(q[lane + 64]) : 0.f;
        float ka = lane < dk ? to_f(k[lane]) : 0.f, kb = lane + 64 < dk ? to_f(k[lane + 64]) : 0.f;
        if (a.l2k) {
            // per-token key normalisation, k / sqrt(|k|^2 + KEY_EPS), in fp32
            float ss = ka * ka + kb * kb;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
            const float inv = 1.f / sqrtf(ss + KEY_EPS);
            ka *= inv;
            kb *= inv;
        }
        // s = k . q, butterfly sum (same value and order on every lane)
        float sk = qa * ka + qb * kb;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sk += __shfl_xor(sk, off, 64);
        if (KEEP) {
            // the wave reads back only what it wrote (in order after the
            // previous token's reads): no barrier beyond the wave's
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            qs[lane] = qa;
            ks[lane] = ka;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }

        float r[NCOL], u[NCOL];
#pragma unroll
        for (int c = 0; c < NCOL; ++c) r[c] = u[c] = 0.f;
        if (have) {
            if (KEEP) {
                // RS interleaved row sets, summed pairwise at the end
                float rs[RS][NCOL], us[RS][NCOL];
#pragma unroll
                for (int e = 0; e < RS; ++e)
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) rs[e][c] = us[e][c] = 0.f;
#pragma unroll
                for (int i = 0; i < KR; i += RS) {
                    if (i < dk) {
#pragma unroll
                        for (int e4 = 0; e4 < RS; e4 += 4) {
                            const float4 q4 = *(const float4 *)(qs + i + e4), k4 = *(const float4 *)(ks + i + e4);
                            const float qv[4] = {q4.x, q4.y, q4.z, q4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
#pragma unroll
                                for (int c = 0; c < NCOL; ++c) {
                                    rs[e4 + e][c] += hr[i + e4 + e][c] * qv[e];
                                    us[e4 + e][c] += hr[i + e4 + e][c] * kv[e];
                                }
                        }
                    }
                }
#pragma unroll
                for (int w2 = RS / 2; w2 > 0; w2 >>= 1)
#pragma unroll
                    for (int e = 0; e < w2; ++e)
#pragma unroll
                        for (int c = 0; c < NCOL; ++c) {
                            rs[e][c] += rs[e + w2][c];
                            us[e][c] += us[e + w2][c];
                        }
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                    r[c] = rs[0][c];
                    u[c] = us[0][c];
                }
            } else {
                for (int i = 0; i < dk; ++i) {
                    const float qi = i < 64 ? lane_bcast(qa, i) : lane_bcast(qb, i - 64);
                    const float ki = i < 64 ? lane_bcast(ka, i) : lane_bcast(kb, i - 64);
#pragma unroll
                    for (int c = 0; c < NCOL; ++c) {
                        const float x = ok[c] ? src[(size_t)i * dv + col[c]] : 0.f;
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
            if (a.D) oj += a.D[h] * vj; // skip term
            if (ok[c]) o[col[c]] = from_f<BF>(oj);
        }
        if (KEEP) {
#pragma unroll
            for (int i = 0; i < KR; i += 4) {
                if (i < dk) {
                    const float4 k4 = *(const float4 *)(ks + i);
                    const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int c = 0; c < NCOL; ++c)
                            hr[i + e][c] = (have ? alpha * hr[i + e][c] : 0.f) + kv[e] * w[c];
                }
            }
        } else {
            // each lane reads and writes only its own columns, so reading
            // hout here sees this lane's writes of the previous token
            for (int i = 0; i < dk; ++i) {
                const float ki = i < 64 ? lane_bcast(ka, i) : lane_bcast(kb, i - 64);
#pragma unroll
                for (int c = 0; c < NCOL; ++c) {
                    if (ok[c]) {
                        const float x = have ? src[(size_t)i * dv + col[c]] : 0.f;
                        hout[(size_t)i * dv + col[c]] = alpha * x + ki * w[c];
                    }
                }
            }
        }
        have = true;
    }
    if (KEEP) {
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            if (i < dk) {
#pragma unroll
                for (int c = 0; c < NCOL; ++c)
                    if (ok[c]) hout[(size_t)i * dv + col[c]] = hr[i][c];
            }
        }
    }
}

// Calls of 2 to 4 tokens with dk, dv <= 64: the same update as step_kernel
// with the state in registers, but every token's inputs are loaded before the
// first update, so the loads of later tokens do not wait behind the work of
// earlier ones (a separate kernel: folding this into step_kernel changed the
// single-token schedule for the worse).
constexpr int PRE_TOKENS = 4;
constexpr int PRE_RS = 8; // interleaved row sets of the reductions (divides 64)

template <bool BF> __global__ __launch_bounds__(NTHR) void step_pre_kernel(StepArgs a) {
    using S = typename Op<BF>::S;
    // q and k of every token of the wave's item, as 4-row broadcast reads
    __shared__ __attribute__((aligned(16))) float qk[NWAVE][2][PRE_TOKENS][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nh = blockIdx.x * NWAVE + wave;
    if (nh >= a.N * a.H) return;
    const int seq = nh / a.H, h = nh % a.H, dk = a.dk, dv = a.dv, NT = a.S;
    const float *hin = a.h_in ? a.h_in + (size_t)nh * dk * dv : nullptr;
    float *hout = a.h_out + (size_t)nh * dk * dv;
    const float A = -expf(a.A_log[h]);
    const bool ok = lane < dv;

    // rows past dk hold zeros, so whole groups of 4 rows can be processed
    float hr[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) hr[i] = (i < dk && hin && ok) ? hin[(size_t)i * dv + lane] : 0.f;
    // inputs of every token (lane: key index for q, k; value column for v)
    float gg[PRE_TOKENS], bb[PRE_TOKENS], vv[PRE_TOKENS];
    float(*qs)[64] = qk[wave][0], (*ks)[64] = qk[wave][1];
#pragma unroll
    for (int t = 0; t < PRE_TOKENS; ++t) {
        if (t < NT) {
            const size_t tok = ((size_t)seq * NT + t) * a.H + h;
            gg[t] = a.g[tok];
            bb[t] = a.beta[tok];
            qs[t][lane] = lane < dk ? to_f(((const S *)a.q)[tok * dk + lane]) : 0.f;
            float kl = lane < dk ? to_f(((const S *)a.k)[tok * dk + lane]) : 0.f;
            if (a.l2k) {
                float ss = kl * kl;
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                kl *= 1.f / sqrtf(ss + KEY_EPS);
            }
            ks[t][lane] = kl;
            vv[t] = ok ? to_f(((const S *)a.v)[tok * dv + lane]) : 0.f;
        }
    }
    // the wave reads back only what it wrote: no barrier beyond the wave's
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bool have = hin != nullptr;
#pragma unroll
    for (int t = 0; t < PRE_TOKENS; ++t) {
        if (t < NT) {
            const size_t tok = ((size_t)seq * NT + t) * a.H + h;
            const float alpha = expf(gate_of(gg[t], a.logits) * A), beta = gate_of(bb[t], a.logits);
            // s = k . q, and r = h^T q, u = h^T k over four interleaved row sets
            float sk = qs[t][lane] * ks[t][lane];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sk += __shfl_xor(sk, off, 64);
            float rs[PRE_RS], us[PRE_RS];
#pragma unroll
            for (int e = 0; e < PRE_RS; ++e) rs[e] = us[e] = 0.f;
            if (have) {
#pragma unroll
                for (int i = 0; i < 64; i += PRE_RS) {
                    if (i < dk) {
#pragma unroll
                        for (int e4 = 0; e4 < PRE_RS; e4 += 4) {
                            const float4 q4 = *(const float4 *)&qs[t][i + e4], k4 = *(const float4 *)&ks[t][i + e4];
                            const float qv[4] = {q4.x, q4.y, q4.z, q4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                rs[e4 + e] += hr[i + e4 + e] * qv[e];
                                us[e4 + e] += hr[i + e4 + e] * kv[e];
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int w2 = PRE_RS / 2; w2 > 0; w2 >>= 1)
#pragma unroll
                for (int e = 0; e < w2; ++e) {
                    rs[e] += rs[e + w2];
                    us[e] += us[e + w2];
                }
            const float r = rs[0], u = us[0];
            const float vj = vv[t];
            float oj, w;
            if (a.additive) {
                oj = alpha * r + beta * sk * vj;
                w = beta * vj;
            } else {
                oj = alpha * (r - beta * sk * u) + beta * sk * vj;
                w = beta * (vj - alpha * u);
            }
            if (a.D) oj += a.D[h] * vj; // skip term
            if (ok) ((S *)a.o)[tok * dv + lane] = from_f<BF>(oj);
#pragma unroll
            for (int i = 0; i < 64; i += 4) {
                if (i < dk) {
                    const float4 k4 = *(const float4 *)&ks[t][i];
                    hr[i] = (have ? alpha * hr[i] : 0.f) + k4.x * w;
                    hr[i + 1] = (have ? alpha * hr[i + 1] : 0.f) + k4.y * w;
                    hr[i + 2] = (have ? alpha * hr[i + 2] : 0.f) + k4.z * w;
                    hr[i + 3] = (have ? alpha * hr[i + 3] : 0.f) + k4.w * w;
                }
            }
            have = true;
        }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i)
        if (i < dk && ok) hout[(size_t)i * dv + lane] = hr[i];
}

template <bool BF, bool ONE> static hipError_t step_inst(const StepArgs &a, hipStream_t st) {
    const int grid = (a.N * a.H + NWAVE - 1) / NWAVE;
    const bool keep = a.dk <= 64;
    if (a.dv <= 64) {
        if (keep) hipLaunchKernelGGL((step_kernel<BF, 1, true, ONE>), dim3(grid), dim3(NTHR), 0, st, a);
        else hipLaunchKernelGGL((step_kernel<BF, 1, false, ONE>), dim3(grid), dim3(NTHR), 0, st, a);
    } else {
        if (keep) hipLaunchKernelGGL((step_kernel<BF, 2, true, ONE>), dim3(grid), dim3(NTHR), 0, st, a);
        else hipLaunchKernelGGL((step_kernel<BF, 2, false, ONE>), dim3(grid), dim3(NTHR), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, bool bf16, hipStream_t st) {
    if (a.S == 1) return bf16 ? step_inst<true, true>(a, st) : step_inst<false, true>(a, st);
    if (a.S <= PRE_TOKENS && a.dk <= 64 && a.dv <= 64) {
        const int grid = (a.N * a.H + NWAVE - 1) / NWAVE;
        if (bf16) hipLaunchKernelGGL(step_pre_kernel<true>, dim3(grid), dim3(NTHR), 0, st, a);
        else hipLaunchKernelGGL(step_pre_kernel<false>, dim3(grid), dim3(NTHR), 0, st, a);
        return hipGetLastError();
    }
    return bf16 ? step_inst<true, false>(a, st) : step_inst<false, false>(a, st);
}

} // namespace gdn
