// Chunked forward of the gated delta rule ("GDN & MLA Mechanism Deep-Dive",
// Step 5: closed form inside each 64-token chunk, state carried serially
// between chunks; the closed form is the WY/UT representation of the cited
// Gated Delta Net paper).
//
// Per chunk, with chunk-local cumulative log-decay gam and
// Gam_ij = exp(gam_i - gam_j) for i >= j:
//   L  = strict_lower(diag(beta) (K K^T o Gam)),   Tm = (I + L)^{-1}
//   U  = Tm diag(beta) V,   Kw = Tm diag(beta e^gam) K
//   W  = U - Kw h
//   O  = diag(e^gam) Q h + ((Q K^T) o Gam) W
//   h <- e^{gam_last} h + K^T diag(e^{gam_last - gam}) W
// With the erase term off (additive write), Tm = I and W = diag(beta) V.
//
// Two kernels. fwd_prep does everything that does not depend on the state,
// one workgroup per (batch, head, chunk), all chunks in parallel, and writes
// U, NK = -Kw and (when the backward will need it) Tm. fwd_chain walks the
// chunks in order for one (batch, head, block of value columns): per chunk
// only Q K^T, W, O and the state update remain, so the serial path is short.
#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// ------------------------------------------------------------------ prep

template <bool BF, int D> struct PrepSmem {
    using S = typename Op<BF>::S;
    static constexpr int LDD = D + Op<BF>::PAD;
    static constexpr int LDC = C + Op<BF>::PAD;
    static constexpr int mx(int x, int y) { return x > y ? x : y; }
    static constexpr int oK = 0;                                       // Ks [C][LDD] -> Tb [C][LDC]
    static constexpr int oKT = oK + mx(C * LDD, C * LDC) * (int)sizeof(S); // KT [D][LDC]
    static constexpr int oVT = oKT + D * LDC * (int)sizeof(S);        // VT [D][LDC]
    static constexpr int oL = oVT + D * LDC * (int)sizeof(S);         // L fp32 [C][LDF]
    static constexpr int oT = oL + C * LDF * 4;                       // Tm fp32 [C][LDF]
    static constexpr int oTk = oT + C * LDF * 4;                      // Tk [C][LDC]
    static constexpr int oX = oTk + C * LDC * (int)sizeof(S);         // solve scratch
    static constexpr int oGam = oX + 4 * 16 * 17 * 4;                 // double[C]
    static constexpr int oBet = oGam + C * 8;                         // float[C]
    static constexpr int oCk = oBet + C * 4;                          // beta e^gam
    static constexpr int SIZE = oCk + C * 4;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

// Store this wave's tiles of an [MT*16][NT*16] accumulator grid to a
// row-major global matrix (rows < nr, cols < nc), times `sign`.
template <bool BF, int MT, int NT>
__device__ __forceinline__ void store_global(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int nr,
                                             int nc, float sign, int wave, int lane) {
    for_tiles<MT, NT>(wave, lane, [&](int i, int e, int row, int col) {
        if (row < nr && col < nc) dst[(size_t)row * ld + col] = from_f<BF>(sign * acc[i][e]);
    });
}

template <bool BF, int D, bool VEC>
__global__ __launch_bounds__(NTHR) void fwd_prep_kernel(PrepArgs a) {
    using O = Op<BF>;
    using S = typename O::S;
    using L = PrepSmem<BF, D>;
    constexpr int LDD = L::LDD, LDC = L::LDC, DT = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *Tb = (S *)(smem + L::oK);
    S *KT = (S *)(smem + L::oKT);
    S *VT = (S *)(smem + L::oVT);
    float *Lm = (float *)(smem + L::oL);
    float *Tm = (float *)(smem + L::oT);
    S *Tk = (S *)(smem + L::oTk);
    float *xs = (float *)(smem + L::oX);
    double *gam2 = (double *)(smem + L::oGam);
    float *bet = (float *)(smem + L::oBet);
    float *ck = (float *)(smem + L::oCk);

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int c = lid % s.NC, bh = lid / s.NC;
    const int b = bh / s.H, h = bh % s.H;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv;
    const int t0 = c * C, n = min(C, T - t0);
    const size_t row0 = (size_t)b * T + t0;

    ChunkFrag<BF, D> fk, fv;
    fk.template fetch<VEC>((const S *)s.k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
    fv.template fetch<VEC>((const S *)s.v + (row0 * H + h) * dv, (size_t)H * dv, n, dv, tid);
    if (wave == 0) {
        const float gr = load_row_scalar(s.g + row0 * H + h, H, lane, n);
        const float br = load_row_scalar(s.beta + row0 * H + h, H, lane, n);
        const float g = lane < n ? gr : 0.f, be = lane < n ? br : 0.f;
        const Decay dc = decay_lane(g, -exp((double)s.A_log[h]) * LOG2E, lane);
        gam2[lane] = dc.gam2;
        bet[lane] = be;
        ck[lane] = be * dc.eg;
    }
    fk.stash(Ks, LDD, tid);
    fk.stash_T(KT, LDC, tid);
    fv.stash_T(VT, LDC, tid);
    __syncthreads();

    if (!s.additive) {
        f32x4 sk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sk[i] = zero4();
        gemm<BF, 4, 4, D>(Ks, LDD, Ks, LDD, sk, wave, lane);
        for_tiles<4, 4>(wave, lane, [&](int i, int e, int row, int col) {
            Lm[row * LDF + col] = (row > col) ? bet[row] * sk[i][e] * gamma_ij(gam2, row, col) : 0.f;
        });
        __syncthreads(); // L complete, Ks no longer read
        tri_inverse<BF, true, true, false>(Lm, Tm, xs, wave, lane, Tb, Tk, nullptr, LDC, bet, ck);
    } else {
        for (int e = tid; e < C * C; e += NTHR) {
            const int row = e / C, col = e % C;
            Tb[row * LDC + col] = from_f<BF>(row == col ? bet[col] : 0.f);
        }
        __syncthreads();
    }

    const size_t cbase = (size_t)bh * s.NC + c;
    // Tm of the chunk for the backward (row-major [64][64]; identity when
    // the erase term is off), one 16-byte store per thread and step. The
    // solve leaves the 16x16 blocks above the diagonal of Tm unwritten: they
    // are zero.
    if (a.Tsave) {
        S *dst = (S *)a.Tsave + cbase * C * C;
        constexpr int V = O::VEC;
        for (int e = tid * V; e < C * C; e += NTHR * V) {
            const int row = e / C, col = e % C;
            const bool upper = (col >> 4) > (row >> 4);
            union {
                uint4 u;
                S x[V];
            } pk;
#pragma unroll
            for (int j = 0; j < V; ++j)
                pk.x[j] = from_f<BF>(s.additive ? (row == col + j ? 1.f : 0.f)
                                                : (upper ? 0.f : Tm[row * LDF + col + j]));
            *reinterpret_cast<uint4 *>(dst + e) = pk.u;
        }
    }
    {
        f32x4 acc[Tiles<4, DT>::PW];
#pragma unroll
        for (int i = 0; i < Tiles<4, DT>::PW; ++i) acc[i] = zero4();
        gemm<BF, 4, DT, C>(Tb, LDC, VT, LDC, acc, wave, lane);
        store_global<BF, 4, DT>(acc, (S *)a.U + cbase * C * dv, dv, C, dv, 1.f, wave, lane);
    }
    if (!s.additive) {
        f32x4 acc[Tiles<4, DT>::PW];
#pragma unroll
        for (int i = 0; i < Tiles<4, DT>::PW; ++i) acc[i] = zero4();
        gemm<BF, 4, DT, C>(Tk, LDC, KT, LDC, acc, wave, lane);
        store_global<BF, 4, DT>(acc, (S *)a.NK + cbase * C * dk, dk, C, dk, -1.f, wave, lane);
    }
}

// ----------------------------------------------------------------- chain

template <bool BF, int D, int BV> struct FwdChainSmem {
    using S = typename Op<BF>::S;
    static constexpr int LDD = D + Op<BF>::PAD;
    static constexpr int LDC = C + Op<BF>::PAD;
    static constexpr int LDV = BV + Op<BF>::PAD;
    static constexpr int szCD = C * LDD * (int)sizeof(S);
    static constexpr int oK = 0;                                  // Ks  [C][LDD]
    static constexpr int oQ = oK + szCD;                          // Qs  [C][LDD]
    static constexpr int oNK = oQ + szCD;                         // NKs [C][LDD]  (-Kw)
    static constexpr int oU = oNK + szCD;                         // Us  [C][LDV]
    static constexpr int oP = oU + C * LDV * (int)sizeof(S);      // Pt  [C][LDC] (P transposed)
    static constexpr int oHT = oP + C * LDC * (int)sizeof(S);     // hTs [BV][LDD]
    static constexpr int oWT = oHT + BV * LDD * (int)sizeof(S);   // WT  [BV][LDC]
    static constexpr int oWTd = oWT + BV * LDC * (int)sizeof(S);  // WTd [BV][LDC] (rows * e^{gam_n-gam})
    static constexpr int oGam = oWTd + BV * LDC * (int)sizeof(S); // double[C]
    static constexpr int oEg = oGam + C * 8;
    static constexpr int oEgn = oEg + C * 4;
    static constexpr int oMisc = oEgn + C * 4;
    static constexpr int SIZE = oMisc + 16;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

template <bool BF, int D, int BV, bool VEC>
__global__ __launch_bounds__(NTHR) void fwd_chain_kernel(FwdChainArgs a) {
    using O = Op<BF>;
    using S = typename O::S;
    using L = FwdChainSmem<BF, D, BV>;
    constexpr int LDD = L::LDD, LDC = L::LDC, LDV = L::LDV;
    constexpr int DT = D / 16, VT = BV / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *Qs = (S *)(smem + L::oQ);
    S *NKs = (S *)(smem + L::oNK);
    S *Us = (S *)(smem + L::oU);
    S *Ps = (S *)(smem + L::oP);
    S *hTs = (S *)(smem + L::oHT);
    S *WT = (S *)(smem + L::oWT);
    S *WTd = (S *)(smem + L::oWTd);
    double *gam2 = (double *)(smem + L::oGam);
    float *eg = (float *)(smem + L::oEg);
    float *egn = (float *)(smem + L::oEgn);
    float *misc = (float *)(smem + L::oMisc);

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int vb = lid % a.NVB, bh = lid / a.NVB;
    const int b = bh / s.H, h = bh % s.H;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv;
    const int v0 = vb * BV, nvc = min(BV, dv - v0);
    const double A2 = -exp((double)s.A_log[h]) * LOG2E;
    const S *q = (const S *)s.q;
    const S *k = (const S *)s.k;
    const S *U = (const S *)a.U;
    const S *NK = (const S *)a.NK;
    S *o = (S *)a.o;
    S *cs = (S *)a.cs;

    // state h[D][BV] (fp32) lives in the accumulators of the h-update product
    f32x4 accH[Tiles<DT, VT>::PW];
    for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
        accH[i][e] = (s.h0 && row < dk && col < nvc) ? s.h0[((size_t)bh * dk + row) * dv + v0 + col] : 0.f;
    });
    store_T<BF, DT, VT>(accH, hTs, LDD, wave, lane);

    // inputs of the next chunk are fetched into registers during this one
    ChunkFrag<BF, D> fk, fq, fn;
    ChunkFrag<BF, BV> fu;
    float pg = 0.f;
    auto fetch = [&](int c) {
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = (size_t)b * T + t0, cb = (size_t)bh * s.NC + c;
        fk.template fetch<VEC>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        fq.template fetch<VEC>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        if (!s.additive) fn.template fetch<VEC>(NK + cb * C * dk, (size_t)dk, n, dk, tid);
        fu.template fetch<VEC>(U + cb * C * dv + v0, (size_t)dv, n, nvc, tid);
        pg = load_row_scalar(s.g + row0 * H + h, H, lane, n);
    };
    // O of a chunk is held in registers and written out during the next
    // chunk, after that chunk's inputs have arrived: stores are issued only
    // between consuming one prefetch and issuing the next, so waiting for
    // the inputs never waits for a store to complete
    f32x4 accO[Tiles<4, VT>::PW];
    auto store_o = [&](int c) {
        const int n = min(C, T - c * C);
        S *orow = o + (((size_t)b * T + c * C) * H + h) * dv + v0;
        for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < n && col < nvc) orow[(size_t)row * H * dv + col] = from_f<BF>(accO[i][e]);
        });
    };
    fetch(0);

    for (int c = 0; c < s.NC; ++c) {
        const int t0 = c * C, n = min(C, T - t0);
        wait_vmem();
        if (wave == 0) {
            const Decay dc = decay_lane(lane < n ? pg : 0.f, A2, lane);
            gam2[lane] = dc.gam2;
            eg[lane] = dc.eg;
            egn[lane] = dc.egn;
            if (lane == 0) misc[0] = dc.eglast;
        }
        fk.stash(Ks, LDD, tid);
        fq.stash(Qs, LDD, tid);
        if (!s.additive) fn.stash(NKs, LDD, tid);
        fu.stash(Us, LDV, tid);
        if (o && c > 0) store_o(c - 1);
        if (cs) {
            for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
                if (row < dk && col < nvc)
                    cs[(((size_t)bh * s.NC + c) * dk + row) * dv + v0 + col] = from_f<BF>(accH[i][e]);
            });
        }
        if (c + 1 < s.NC) fetch(c + 1);
        __syncthreads();

        // P = (Q K^T) o Gam (independent of the state)
        {
            f32x4 sq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sq[i] = zero4();
            gemm<BF, 4, 4, D>(Qs, LDD, Ks, LDD, sq, wave, lane);
            for_tiles<4, 4>(wave, lane, [&](int i, int e, int row, int col) { sq[i][e] *= gamma_ij(gam2, row, col); });
            store_T<BF, 4, 4>(sq, Ps, LDC, wave, lane);
        }
        // W = U - Kw h (serial chain, part 1)
        {
            f32x4 accW[Tiles<4, VT>::PW];
            for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) { accW[i][e] = to_f(Us[row * LDV + col]); });
            if (!s.additive) gemm<BF, 4, VT, D>(NKs, LDD, hTs, LDD, accW, wave, lane);
            store_T<BF, 4, VT>(accW, WT, LDC, wave, lane);
            store_T<BF, 4, VT>(accW, WTd, LDC, wave, lane, egn);
        }
        __syncthreads();

        // O = diag(e^gam) Q h + P W
        if (o) {
#pragma unroll
            for (int i = 0; i < Tiles<4, VT>::PW; ++i) accO[i] = zero4();
            gemm<BF, 4, VT, D>(Qs, LDD, hTs, LDD, accO, wave, lane);
            for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) { accO[i][e] *= eg[row]; });
            gemm<BF, 4, VT, C, true, false>(Ps, LDC, WT, LDC, accO, wave, lane);
        }
        // h <- e^{gam_last} h + K^T diag(e^{gam_last - gam}) W (serial chain, part 2)
        {
            const float el = misc[0];
#pragma unroll
            for (int i = 0; i < Tiles<DT, VT>::PW; ++i) accH[i] *= el;
            gemm<BF, DT, VT, C, true, false>(Ks, LDD, WTd, LDC, accH, wave, lane);
        }
        __syncthreads();
        store_T<BF, DT, VT>(accH, hTs, LDD, wave, lane);
    }
    if (o) store_o(s.NC - 1);
    if (a.hT) {
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) a.hT[((size_t)bh * dk + row) * dv + v0 + col] = accH[i][e];
        });
    }
}

// ---------------------------------------------------------------- launch

int pad_dim(int d, bool bf16) {
    int D = bf16 ? 32 : 16;
    while (D < d) D *= 2;
    return D;
}

int fwd_vblock(int D) { return D >= 64 ? 32 : 16; }

template <bool BF, int D> static hipError_t prep_inst(const PrepArgs &a, hipStream_t st) {
    const int grid = a.s.B * a.s.H * a.s.NC;
    if (vec_ok<BF>(a.s))
        hipLaunchKernelGGL((fwd_prep_kernel<BF, D, true>), dim3(grid), dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((fwd_prep_kernel<BF, D, false>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

template <bool BF, int D> static hipError_t chain_inst(const FwdChainArgs &a, hipStream_t st) {
    constexpr int BV = D >= 64 ? 32 : 16;
    const int grid = a.s.B * a.s.H * a.NVB;
    if (vec_ok<BF>(a.s))
        hipLaunchKernelGGL((fwd_chain_kernel<BF, D, BV, true>), dim3(grid), dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((fwd_chain_kernel<BF, D, BV, false>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fwd_prep(const PrepArgs &a, bool bf16, int D, hipStream_t st) {
    if (bf16) {
        switch (D) {
        case 32: return prep_inst<true, 32>(a, st);
        case 64: return prep_inst<true, 64>(a, st);
        case 128: return prep_inst<true, 128>(a, st);
        }
    } else {
        switch (D) {
        case 16: return prep_inst<false, 16>(a, st);
        case 32: return prep_inst<false, 32>(a, st);
        case 64: return prep_inst<false, 64>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_chain(const FwdChainArgs &a, bool bf16, int D, hipStream_t st) {
    if (fwd_vblock(D) * a.NVB < a.s.dv) return hipErrorInvalidValue;
    if (bf16) {
        switch (D) {
        case 32: return chain_inst<true, 32>(a, st);
        case 64: return chain_inst<true, 64>(a, st);
        case 128: return chain_inst<true, 128>(a, st);
        }
    } else {
        switch (D) {
        case 16: return chain_inst<false, 16>(a, st);
        case 32: return chain_inst<false, 32>(a, st);
        case 64: return chain_inst<false, 64>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

} // namespace gdn
