// Chunked forward of the gated delta rule ("GDN & MLA Mechanism Deep-Dive",
// Step 5: closed form inside each 64-token chunk, state carried serially
// between chunks; the closed form is the WY/UT representation of the cited
// Gated Delta Net paper).
//
// One workgroup owns one (batch, head, block of BV value columns) and walks
// the chunks in order. Columns of the state are independent, so splitting
// d_v over workgroups multiplies the number of serial chains. Per chunk, with
// chunk-local cumulative log-decay gam and Gam_ij = exp(gam_i - gam_j), i >= j:
//   L  = strict_lower(diag(beta) (K K^T o Gam)),   Tm = (I + L)^{-1}
//   U  = Tm diag(beta) V,   Kw = Tm diag(beta e^gam) K
//   W  = U - Kw h
//   O  = diag(e^gam) Q h + ((Q K^T) o Gam) W
//   h <- e^{gam_last} h + (diag(e^{gam_last - gam}) K)^T W
// With the erase term off (additive write), Tm = I and W = diag(beta) V.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <bool BF, int D, int BV> struct FwdSmem {
    using S = typename Op<BF>::S;
    static constexpr int LDD = D + Op<BF>::PAD;
    static constexpr int LDC = C + Op<BF>::PAD;
    static constexpr int szCD = C * LDD * (int)sizeof(S);
    static constexpr int oK = 0;                                   // Ks  [C][LDD]
    static constexpr int oKT = oK + szCD;                          // KTs [D][LDC] (later scaled)
    static constexpr int oQ = oKT + D * LDC * (int)sizeof(S);      // Qs  [C][LDD]
    static constexpr int oVT = oQ + szCD;                          // VTs [BV][LDC]
    static constexpr int oR1 = oVT + BV * LDC * (int)sizeof(S);    // L fp32 -> Tb -> Kw
    static constexpr int szR1 = (C * LDF * 4 > szCD) ? C * LDF * 4 : szCD;
    static constexpr int oR2 = oR1 + szR1;                         // Tm fp32 -> Tk
    static constexpr int oP = oR2 + C * LDF * 4;                   // Ps  [C][LDC]
    static constexpr int oHT = oP + C * LDC * (int)sizeof(S);      // hTs [BV][LDD]
    static constexpr int oWT = oHT + BV * LDD * (int)sizeof(S);    // WTs [BV][LDC]
    static constexpr int oX = oWT + BV * LDC * (int)sizeof(S);     // solve scratch
    static constexpr int oGam = oX + 4 * 16 * 17 * 4;              // double[C]
    static constexpr int oEg = oGam + C * 8;                       // float[C]
    static constexpr int oEgn = oEg + C * 4;
    static constexpr int oBet = oEgn + C * 4;
    static constexpr int oG = oBet + C * 4;
    static constexpr int oMisc = oG + C * 4;
    static constexpr int SIZE = oMisc + 16;
    static_assert(C * LDC * (int)sizeof(S) <= szR1, "Tb must fit in R1");
    static_assert(C * LDC * (int)sizeof(S) <= C * LDF * 4, "Tk must fit in R2");
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

template <bool BF, int D, int BV>
__global__ __launch_bounds__(NTHR) void fwd_kernel(FwdArgs a) {
    using O = Op<BF>;
    using S = typename O::S;
    using L = FwdSmem<BF, D, BV>;
    constexpr int LDD = L::LDD, LDC = L::LDC;
    constexpr int DT = D / 16, VT = BV / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *KTs = (S *)(smem + L::oKT);
    S *Qs = (S *)(smem + L::oQ);
    S *VTs = (S *)(smem + L::oVT);
    float *Lm = (float *)(smem + L::oR1);
    S *Tb = (S *)(smem + L::oR1);
    S *Kws = (S *)(smem + L::oR1);
    float *Tm = (float *)(smem + L::oR2);
    S *Tk = (S *)(smem + L::oR2);
    S *Ps = (S *)(smem + L::oP);
    S *hTs = (S *)(smem + L::oHT);
    S *WTs = (S *)(smem + L::oWT);
    float *xs = (float *)(smem + L::oX);
    double *gam = (double *)(smem + L::oGam);
    float *eg = (float *)(smem + L::oEg);
    float *egn = (float *)(smem + L::oEgn);
    float *bet = (float *)(smem + L::oBet);
    float *gch = (float *)(smem + L::oG);
    float *misc = (float *)(smem + L::oMisc);

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int vb = lid % a.NVB, bh = lid / a.NVB;
    const int b = bh / s.H, h = bh % s.H;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv;
    const int v0 = vb * BV;
    const int nvc = min(BV, dv - v0); // valid value columns of this block
    const double A = -exp((double)s.A_log[h]);
    const S *q = (const S *)s.q;
    const S *k = (const S *)s.k;
    const S *v = (const S *)s.v;
    S *o = (S *)a.o;
    S *cs = (S *)a.cs;
    const bool veck = (dk % O::VEC) == 0, vecv = (dv % O::VEC) == 0;

    // state h[D][BV] (fp32) lives in the accumulators of the h-update product
    f32x4 accH[Tiles<DT, VT>::PW];
    for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
        accH[i][e] = (s.h0 && row < dk && col < nvc)
                         ? s.h0[((size_t)bh * dk + row) * dv + v0 + col]
                         : 0.f;
    });
    store_T<BF, DT, VT>(accH, hTs, LDD, wave, lane);

    for (int c = 0; c < s.NC; ++c) {
        const int t0 = c * C, n = min(C, T - t0);
        if (cs) {
            for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
                if (row < dk && col < nvc)
                    cs[(((size_t)bh * s.NC + c) * dk + row) * dv + v0 + col] = from_f<BF>(accH[i][e]);
            });
        }
        // ---- load the chunk
        if (tid < C) {
            const size_t gi = ((size_t)b * T + t0 + tid) * H + h;
            gch[tid] = (tid < n) ? s.g[gi] : 0.f;
            bet[tid] = (tid < n) ? s.beta[gi] : 0.f;
        }
        const size_t row0 = (size_t)b * T + t0;
        load_chunk<BF, D>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, veck, Ks, LDD, KTs, LDC, tid);
        load_chunk<BF, D>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, veck, Qs, LDD, nullptr, 0, tid);
        load_chunk<BF, BV>(v + (row0 * H + h) * dv + v0, (size_t)H * dv, n, nvc, vecv, nullptr, 0, VTs,
                           LDC, tid);
        __syncthreads();
        if (wave == 0) decay_prep(gch, A, n, lane, gam, eg, egn, misc);
        __syncthreads();

        // ---- Gram products, decay mask
        {
            f32x4 sk[4], sq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sk[i] = sq[i] = zero4();
            if (!s.additive) gemm<BF, 4, 4, D>(Ks, LDD, Ks, LDD, sk, wave, lane);
            gemm<BF, 4, 4, D>(Qs, LDD, Ks, LDD, sq, wave, lane);
            for_tiles<4, 4>(wave, lane, [&](int i, int e, int row, int col) {
                const float G = (row >= col) ? expf((float)(gam[row] - gam[col])) : 0.f;
                Lm[row * LDF + col] = (row > col) ? bet[row] * sk[i][e] * G : 0.f;
                Ps[row * LDC + col] = from_f<BF>(sq[i][e] * G);
            });
        }
        __syncthreads();

        // ---- Tm = (I + L)^{-1}
        if (!s.additive) {
            tri_inverse(Lm, Tm, xs, wave, lane);
        } else {
            for (int e = tid; e < C * C; e += NTHR) Tm[(e / C) * LDF + e % C] = (e / C == e % C) ? 1.f : 0.f;
            __syncthreads();
        }
        // Tb = Tm diag(beta) into R1, then Tk = Tm diag(beta e^gam) in place over Tm
        {
            float tv[C * C / NTHR];
#pragma unroll
            for (int m = 0; m < C * C / NTHR; ++m) {
                const int e = tid + m * NTHR, row = e / C, col = e % C;
                tv[m] = Tm[row * LDF + col];
                Tb[row * LDC + col] = from_f<BF>(tv[m] * bet[col]);
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < C * C / NTHR; ++m) {
                const int e = tid + m * NTHR, row = e / C, col = e % C;
                Tk[row * LDC + col] = from_f<BF>(tv[m] * bet[col] * eg[col]);
            }
        }
        __syncthreads();

        // ---- U = Tb V (kept in registers), Kw = Tk K (to LDS)
        f32x4 accW[Tiles<4, VT>::PW];
#pragma unroll
        for (int i = 0; i < Tiles<4, VT>::PW; ++i) accW[i] = zero4();
        gemm<BF, 4, VT, C>(Tb, LDC, VTs, LDC, accW, wave, lane);
        if (!s.additive) {
            f32x4 accK[Tiles<4, DT>::PW];
#pragma unroll
            for (int i = 0; i < Tiles<4, DT>::PW; ++i) accK[i] = zero4();
            gemm<BF, 4, DT, C>(Tk, LDC, KTs, LDC, accK, wave, lane);
            __syncthreads();
            store_N<BF, 4, DT>(accK, Kws, LDD, wave, lane);
        } else {
            __syncthreads();
        }
        // KTs <- K^T diag(e^{gam_last - gam})
        for (int e = tid; e < D * C; e += NTHR) {
            const int d = e / C, j = e % C;
            KTs[d * LDC + j] = from_f<BF>(to_f(KTs[d * LDC + j]) * egn[j]);
        }
        __syncthreads();

        // ---- W = U - Kw h  (serial chain, part 1)
        if (!s.additive) {
            f32x4 accX[Tiles<4, VT>::PW];
#pragma unroll
            for (int i = 0; i < Tiles<4, VT>::PW; ++i) accX[i] = zero4();
            gemm<BF, 4, VT, D>(Kws, LDD, hTs, LDD, accX, wave, lane);
#pragma unroll
            for (int i = 0; i < Tiles<4, VT>::PW; ++i) accW[i] -= accX[i];
        }
        store_T<BF, 4, VT>(accW, WTs, LDC, wave, lane);
        __syncthreads();

        // ---- O = diag(e^gam) Q h + P W
        if (o) {
            f32x4 accO[Tiles<4, VT>::PW];
#pragma unroll
            for (int i = 0; i < Tiles<4, VT>::PW; ++i) accO[i] = zero4();
            gemm<BF, 4, VT, D>(Qs, LDD, hTs, LDD, accO, wave, lane);
            for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) { accO[i][e] *= eg[row]; });
            gemm<BF, 4, VT, C>(Ps, LDC, WTs, LDC, accO, wave, lane);
            for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) {
                if (row < n && col < nvc) o[((row0 + row) * H + h) * dv + v0 + col] = from_f<BF>(accO[i][e]);
            });
        }
        // ---- h <- e^{gam_last} h + Ktilde^T W  (serial chain, part 2)
        {
            const float el = misc[0];
#pragma unroll
            for (int i = 0; i < Tiles<DT, VT>::PW; ++i) accH[i] *= el;
            gemm<BF, DT, VT, C>(KTs, LDC, WTs, LDC, accH, wave, lane);
        }
        __syncthreads();
        store_T<BF, DT, VT>(accH, hTs, LDD, wave, lane);
    }
    if (a.hT) {
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) a.hT[((size_t)bh * dk + row) * dv + v0 + col] = accH[i][e];
        });
    }
}

int pad_dim(int d, bool bf16) {
    int D = bf16 ? 32 : 16;
    while (D < d) D *= 2;
    return D;
}

int fwd_vblock(int D) { return D >= 64 ? 32 : 16; }

template <bool BF, int D> static hipError_t fwd_inst(const FwdArgs &a, hipStream_t st) {
    constexpr int BV = (D >= 64) ? 32 : 16;
    const int grid = a.s.B * a.s.H * a.NVB;
    hipLaunchKernelGGL((fwd_kernel<BF, D, BV>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs &a, bool bf16, int D, hipStream_t st) {
    if (bf16) {
        switch (D) {
        case 32: return fwd_inst<true, 32>(a, st);
        case 64: return fwd_inst<true, 64>(a, st);
        case 128: return fwd_inst<true, 128>(a, st);
        }
    } else {
        switch (D) {
        case 16: return fwd_inst<false, 16>(a, st);
        case 32: return fwd_inst<false, 32>(a, st);
        case 64: return fwd_inst<false, 64>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

} // namespace gdn
