// Reverse-chunk backward of the chunked gated delta rule.
//
// The forward per chunk (chunk-local cumulative log-decay gam, Gam_ij =
// exp(gam_i - gam_j) for i >= j; see gdn_fwd.hip) is
//   L = strict_lower(diag(beta)(K K^T o Gam)), Tm = (I + L)^{-1}
//   U = Tm diag(beta) V,  Kw = Tm diag(beta e^gam) K,  W = U - Kw h
//   O = diag(e^gam) Q h + P W,  P = (Q K^T) o Gam (lower, diagonal included)
//   h' = e^{gam_n} h + Kt^T W,  Kt = diag(e^{gam_n - gam}) K
// Its reverse, given dO and dh' (gradient with respect to h'):
//   dW  = P^T dO + Kt dh'
//   dh  = e^{gam_n} dh' + Q^T diag(e^gam) dO - Kw^T dW          (serial chain)
//   dQ  = diag(e^gam) dO h^T + (dP o Gam) K,   dP = dO W^T
//   dKw = -dW h^T,  dV' = Tm^T dW,  dK' = Tm^T dKw,  dV = diag(beta) dV'
//   dL  = -(dV' U^T + dK' Kw^T) (strictly lower part)
// and, by associativity, dK' = -(Tm^T dW) h^T = -dV' h^T and
//   dL  = -dV' U^T + dV' (Kw h)^T = -dV' W^T,
// the forms the per-chunk kernel for heads up to 64 wide uses.
//   dK  = (dP o Gam)^T Q + diag(e^{gam_n - gam}) W dh'^T + diag(beta e^gam) dK'
//         + dS K + dS^T K,  dS = diag(beta)(dL o Gam)
//   dbeta_i = v_i . dV'_i + e^{gam_i} k_i . dK'_i + sum_j dL_ij (K K^T o Gam)_ij
//   dgam from every place gam enters (e^gam, e^{gam_n}, e^{gam_n - gam}, Gam);
//   dlam_r = sum_{i >= r} dgam_i;  dg = A dlam;  dA_log = sum_{b,t} g dg.
//
// Kernels: bwd_chain walks the chunks backwards per (batch, head, value
// block) carrying dh and stores dh' of every chunk; bwd_local recomputes a
// chunk's intermediates from the saved chunk-start state h and dh' and forms
// all local gradients, one workgroup per (batch, head, chunk); dA_reduce sums
// the per-chunk dA_log parts in a fixed order.
#include <atomic>
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// --------------------------------------------------------------- chain

template <bool BF, int D, int BV> struct ChainSmem {
    using S = typename Op<BF>::S;
    static constexpr int LDD = D + Op<BF>::PAD;
    static constexpr int LDC = C + Op<BF>::PAD;
    static constexpr int LDV = BV + Op<BF>::PAD;
    static constexpr int szCD = C * LDD * (int)sizeof(S);
    static constexpr int oK = 0;                                  // Ks  [C][LDD]
    static constexpr int oQ = oK + szCD;                          // Qs  [C][LDD]
    static constexpr int oQE = oQ + szCD;                         // Qe  [C][LDD] (rows * e^gam)
    static constexpr int oNK = oQE + szCD;                        // NKs [C][LDD] (-Kw)
    static constexpr int oDO = oNK + szCD;                        // dOs [C][LDV]
    static constexpr int oPT = oDO + C * LDV * (int)sizeof(S);    // Pt  [C][LDC] (P transposed)
    static constexpr int oDHT = oPT + C * LDC * (int)sizeof(S);   // dhT [BV][LDD]
    static constexpr int oDWT = oDHT + BV * LDD * (int)sizeof(S); // dWT [BV][LDC]
    static constexpr int oGam = oDWT + BV * LDC * (int)sizeof(S);
    static constexpr int oEgn = oGam + C * 8;
    static constexpr int oMisc = oEgn + C * 4;
    static constexpr int SIZE = oMisc + 16;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

template <bool BF, int D, int BV, bool VEC>
__global__ __launch_bounds__(NTHR) void bwd_chain_kernel(BwdChainArgs a) {
    using O = Op<BF>;
    using S = typename O::S;
    using L = ChainSmem<BF, D, BV>;
    constexpr int LDD = L::LDD, LDC = L::LDC, LDV = L::LDV;
    constexpr int DT = D / 16, VT = BV / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *Qs = (S *)(smem + L::oQ);
    S *Qe = (S *)(smem + L::oQE);
    S *NKs = (S *)(smem + L::oNK);
    S *dOs = (S *)(smem + L::oDO);
    S *PT = (S *)(smem + L::oPT);
    S *dHT = (S *)(smem + L::oDHT);
    S *dWT = (S *)(smem + L::oDWT);
    double *gam2 = (double *)(smem + L::oGam);
    float *egn = (float *)(smem + L::oEgn);
    float *misc = (float *)(smem + L::oMisc);

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv, NC = s.NC;
    // workgroup -> (batch-head, segment, value block); with maps the first
    // NVBM blocks carry dk identity columns (the linear part of the map) and
    // the segments are 1 .. nseg-1
    const bool maps = a.mode == 1;
    const int NVBM = maps ? (dk + BV - 1) / BV : 0;
    const int nvbe = a.NVB + NVBM, nsl = maps ? a.nseg - 1 : a.nseg;
    const int vbe = lid % nvbe, seg = (lid / nvbe) % nsl + (maps ? 1 : 0), bh = lid / (nvbe * nsl);
    const bool mblk = vbe < NVBM;
    const int v0 = (mblk ? vbe : vbe - NVBM) * BV, nvc = min(BV, (mblk ? dk : dv) - v0);
    const int c_lo = (int)((long long)seg * NC / a.nseg), c_hi = (int)((long long)(seg + 1) * NC / a.nseg);
    const int b = bh / s.H, h = bh % s.H;
    const double A2 = -exp((double)s.A_log[h]) * LOG2E;
    const S *q = (const S *)s.q;
    const S *k = (const S *)s.k;
    const S *dO = (const S *)a.dout;
    const S *NK = (const S *)a.NK;
    S *dhs = maps ? nullptr : (S *)a.dhs;

    // gradient at the end of the segment: dhT (last segment), the scan's
    // value, identity columns (maps, linear part) or zero
    const float *din = maps ? nullptr
                            : (seg == a.nseg - 1 ? (a.dhT ? a.dhT + (size_t)bh * dk * dv : nullptr)
                                                 : a.seg_dh + ((size_t)bh * a.nseg + seg) * dk * dv);
    f32x4 accDH[Tiles<DT, VT>::PW];
    for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
        const bool in = row < dk && col < nvc;
        accDH[i][e] = mblk ? ((in && row == v0 + col) ? 1.f : 0.f)
                           : ((din && in) ? din[(size_t)row * dv + v0 + col] : 0.f);
    });
    store_T<BF, DT, VT>(accDH, dHT, LDD, wave, lane);

    ChunkFrag<BF, D> fk, fq, fn;
    ChunkFrag<BF, BV> fo;
    fo.ok = 0; // identity columns take dO as zero: never fetched, stashed as zeros
    float pg = 0.f;
    auto fetch = [&](int c) {
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = (size_t)b * T + t0, cb = (size_t)bh * s.NC + c;
        fk.template fetch<VEC>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        if (!mblk) {
            fq.template fetch<VEC>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
            fo.template fetch<VEC>(dO + (row0 * H + h) * dv + v0, (size_t)H * dv, n, nvc, tid);
        }
        if (!s.additive) fn.template fetch<VEC>(NK + cb * C * dk, (size_t)dk, n, dk, tid);
        pg = load_row_scalar(s.g + row0 * H + h, H, lane, n);
    };
    if (c_hi > c_lo) fetch(c_hi - 1);

    for (int c = c_hi - 1; c >= c_lo; --c) {
        const int n = min(C, T - c * C);
        wait_vmem();
        // every wave computes the decay of its lane's row: the copy of Q
        // whose row j = lane is scaled by e^{gam_j} while it is stored
        const Decay dc = decay_lane(lane < n ? gate_of(pg, s.logits) : 0.f, A2, lane);
        if (wave == 0) {
            gam2[lane] = dc.gam2;
            egn[lane] = dc.egn;
            if (lane == 0) misc[0] = dc.eglast;
        }
        if (s.l2k) fk.normalize_rows(nullptr, tid);
        fk.stash(Ks, LDD, tid);
        if (!mblk) {
            fq.stash(Qs, LDD, tid);
            fq.stash_scaled(Qe, LDD, tid, dc.eg);
        }
        fo.stash(dOs, LDV, tid);
        if (!s.additive) fn.stash(NKs, LDD, tid);
        // stores go out between consuming one prefetch and issuing the next,
        // so waiting for the inputs never waits for a store
        // 4 consecutive rows d of one column v per lane: one 8-byte store
        // into the transposed [dv][dk] block when dk allows it
        {
            const int r16 = lane & 15, kq = lane >> 4;
#pragma unroll
            for (int i = 0; i < Tiles<DT, VT>::PW; ++i) {
                const int t = wave + NWAVE * i;
                if (Tiles<DT, VT>::N % NWAVE != 0 && t >= Tiles<DT, VT>::N) break;
                const int d0 = (t / VT) * 16 + 4 * kq, col = (t % VT) * 16 + r16;
                if (!dhs || col >= nvc) continue;
                S *dst = dhs + (((size_t)bh * s.NC + c) * dv + v0 + col) * dk + d0;
                if (BF && dk % 4 == 0) {
                    if (d0 < dk) {
                        uint2 u;
                        u.x = f2bf2(accDH[i][0], accDH[i][1]);
                        u.y = f2bf2(accDH[i][2], accDH[i][3]);
                        *reinterpret_cast<uint2 *>(dst) = u;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < dk) dst[e] = from_f<BF>(accDH[i][e]);
                }
            }
        }
        if (c > c_lo) fetch(c - 1);
        __syncthreads();

        // P^T and Q^T diag(e^gam) dO: independent of the chain (and zero for
        // identity columns, whose dO is zero)
        if (!mblk) {
            f32x4 sq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sq[i] = zero4();
            gemm<BF, 4, 4, D>(Qs, LDD, Ks, LDD, sq, wave, lane);
            for_tiles<4, 4>(wave, lane, [&](int i, int e, int row, int col) { sq[i][e] *= gamma_ij(gam2, row, col); });
            store_T<BF, 4, 4>(sq, PT, LDC, wave, lane);
        }
        f32x4 accQD[Tiles<DT, VT>::PW];
#pragma unroll
        for (int i = 0; i < Tiles<DT, VT>::PW; ++i) accQD[i] = zero4();
        if (!mblk) gemm<BF, DT, VT, C, true, true>(Qe, LDD, dOs, LDV, accQD, wave, lane);
        // dW = diag(e^{gam_n - gam}) K dh' + P^T dO (P^T is read after the barrier)
        f32x4 accW[Tiles<4, VT>::PW];
#pragma unroll
        for (int i = 0; i < Tiles<4, VT>::PW; ++i) accW[i] = zero4();
        gemm<BF, 4, VT, D>(Ks, LDD, dHT, LDD, accW, wave, lane);
        for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) { accW[i][e] *= egn[row]; });
        __syncthreads();
        if (!mblk) gemm<BF, 4, VT, C, false, true>(PT, LDC, dOs, LDV, accW, wave, lane);
        store_T<BF, 4, VT>(accW, dWT, LDC, wave, lane);
        __syncthreads();
        // dh = e^{gam_n} dh' + Q^T diag(e^gam) dO - Kw^T dW
        {
            const float el = misc[0];
#pragma unroll
            for (int i = 0; i < Tiles<DT, VT>::PW; ++i) accDH[i] = accDH[i] * el + accQD[i];
            if (!s.additive) gemm<BF, DT, VT, C, true, false>(NKs, LDD, dWT, LDC, accDH, wave, lane);
        }
        __syncthreads();
        store_T<BF, DT, VT>(accDH, dHT, LDD, wave, lane);
    }
    if (maps) {
        // [M | R] of this segment (index seg - 1): identity blocks fill the M columns
        float *dst = a.maps + ((size_t)bh * (a.nseg - 1) + seg - 1) * dk * (dk + dv) + (mblk ? v0 : dk + v0);
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) dst[(size_t)row * (dk + dv) + col] = accDH[i][e];
        });
    } else if (a.dh0 && seg == 0) {
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) a.dh0[((size_t)bh * dk + row) * dv + v0 + col] = accDH[i][e];
        });
    }
}

// ------------------------------------------------- wave-specialised chain
//
// bf16 path for head dims up to 64. One workgroup per (batch, head, block of
// BV value columns). Waves 0..VT-1 ("chain waves", VT = BV/16) each carry 16
// value columns of dh [D][16] in MFMA accumulators and run only
//   dW = diag(e^{gam_n - gam}) K dh' + X,   dh = e^{gam_n} dh' + Y + (-Kw)^T dW
// with X = P^T dO and Y = Q^T diag(e^gam) dO. With 16x16x16 products an
// accumulator tile is already the B operand of the next product over the
// same rows, so dW and dh never leave the wave's registers on the serial
// path. The eight helper waves that follow work ahead of the chain in two
// groups of four that swap roles every chunk: while the chain handles chunk
// c, the group that owns chunks of c's parity stages chunk c-2 into LDS and
// requests chunk c-4 (so its loads have two chunks' time to land), and the
// other group forms X and Y of chunk c-1.
// K, -Kw and the decay live three chunks in LDS, Q and dO two, X and Y two;
// one barrier per chunk hands them over. The chain waves store dh' of every
// chunk (bf16, transposed [dv][dk]) and the final dh themselves.

constexpr int BWS_HELPERS = 8;

template <int D, int BV> struct BwsSmem {
    static constexpr int LDD = D + 8;  // token rows [C][LDD]
    static constexpr int LDV = BV + 8; // dO rows [C][LDV]
    static constexpr int LDX = C + 4;  // X^T, Y^T [BV][LDX] fp32
    static constexpr int szCD = C * LDD * 2;
    static constexpr int szCV = C * LDV * 2;
    static constexpr int szX = BV * LDX * 4;
    static constexpr int szDec = C * 4 + C * 4 + 16; // gam (log2), e^{gam_n - gam}, e^{gam_n}
    static constexpr int oK = 0;                  // 3 x K
    static constexpr int oN = oK + 3 * szCD;      // 3 x -Kw
    static constexpr int oQ = oN + 3 * szCD;      // 2 x Q
    static constexpr int oO = oQ + 2 * szCD;      // 2 x dO
    static constexpr int oOe = oO + 2 * szCV;     // 2 x diag(e^gam) dO
    static constexpr int oX = oOe + 2 * szCV;     // 2 x X^T
    static constexpr int oY = oX + 2 * szX;       // 2 x Y^T
    static constexpr int oDec = oY + 2 * szX;     // 3 x decay
    static constexpr int SIZE = oDec + 3 * szDec;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

template <int D, int BV, bool VEC>
__global__ __launch_bounds__(64 * (BV / 16 + BWS_HELPERS)) void bwd_chain_ws_kernel(BwdChainArgs a) {
    constexpr int DT = D / 16, VT = BV / 16, KS = D / 32;
    constexpr int NHT = 64 * BWS_HELPERS; // helper threads
    using L = BwsSmem<D, BV>;
    constexpr int LDD = L::LDD, LDV = L::LDV, LDX = L::LDX;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    auto kbuf = [&](int i) { return (u16 *)(smem + L::oK + i * L::szCD); };
    auto nbuf = [&](int i) { return (u16 *)(smem + L::oN + i * L::szCD); };
    auto qbuf = [&](int i) { return (u16 *)(smem + L::oQ + i * L::szCD); };
    auto obuf = [&](int i) { return (u16 *)(smem + L::oO + i * L::szCV); };
    auto oebuf = [&](int i) { return (u16 *)(smem + L::oOe + i * L::szCV); };
    auto xbuf = [&](int i) { return (float *)(smem + L::oX + i * L::szX); };
    auto ybuf = [&](int i) { return (float *)(smem + L::oY + i * L::szX); };
    auto gam_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec); };
    auto egn_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec + C * 4); };
    auto el_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec + C * 8); };

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6;
    // per-lane indices are re-derived from an opaque copy of the thread index
    // at every chunk, so addresses built from them are formed where they are
    // used rather than hoisted out of the loop and held in registers
    int lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int vb = lid % a.NVB, bh = lid / a.NVB;
    const int b = bh / s.H, h = bh % s.H;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv, NC = s.NC, CN = NC - 1;
    const int V0 = vb * BV, nvc = min(BV, dv - V0);
    const bool chain = wave < VT;
    const bool add = s.additive != 0;
    const double A2 = -exp((double)s.A_log[h]) * LOG2E;

    // ---- chain-wave state: value columns V0 + v0 + (0..15)
    const int v0 = 16 * wave;
    f32x4 hacc[DT];
    u16 *dhs = (u16 *)a.dhs;

    // ---- helper-wave state; group gp (helpers 4gp..4gp+3) stages the chunks
    // of parity gp
    constexpr int NGT = NHT / 2; // threads of a group
    const int hw = wave - VT, gp = hw >> 2;
    int gtid = (tid - 64 * VT) & (NGT - 1);
    ChunkFrag<true, D, C, NGT> fk, fq, fn;
    ChunkFrag<true, BV, C, NGT> fo;
    float pg = 0.f;
    const u16 *q = (const u16 *)s.q, *k = (const u16 *)s.k, *dO = (const u16 *)a.dout;
    // additive: -Kw is never read; its loads repeat K so that every step
    // issues the same loads
    const u16 *NK = add ? nullptr : (const u16 *)a.NK;
    auto fetch = [&](int c) {
        c = max(c, 0); // past the first chunk: a harmless repeat of chunk 0
        const int n = min(C, T - c * C);
        const size_t row0 = (size_t)b * T + c * C, cb = (size_t)bh * NC + c;
        fk.template fetch<VEC>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, gtid);
        fq.template fetch<VEC>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, gtid);
        const bool kw = NK != nullptr;
        fn.template fetch<VEC>(kw ? NK + cb * C * dk : k + (row0 * H + h) * dk, kw ? (size_t)dk : (size_t)H * dk, n,
                               dk, gtid);
        fo.template fetch<VEC>(dO + (row0 * H + h) * dv + V0, (size_t)H * dv, n, nvc, gtid);
        pg = load_row_scalar(s.g + row0 * H + h, H, lane, n);
    };
    auto stash = [&](int c) {
        const int n = min(C, T - c * C), i3 = c % 3, i2 = c & 1;
        wait_vmem();
        const Decay dc = decay_lane(lane < n ? gate_of(pg, s.logits) : 0.f, A2, lane);
        if ((hw & 3) == 0) {
            gam_of(i3)[lane] = (float)dc.gam2;
            egn_of(i3)[lane] = dc.egn;
            if (lane == 0) el_of(i3)[0] = dc.eglast;
        }
        if (s.l2k) fk.normalize_rows(nullptr, gtid);
        fk.stash(kbuf(i3), LDD, gtid);
        if (!add) fn.stash(nbuf(i3), LDD, gtid);
        fq.stash(qbuf(i2), LDD, gtid);
        fo.stash(obuf(i2), LDV, gtid);
        fo.stash_scaled(oebuf(i2), LDV, gtid, dc.eg);
    };
    // X^T = dO^T P and Y^T = (diag(e^gam) dO)^T Q of chunk c, by the four
    // helpers of group hg: helpers 0 and 1 form P's column blocks {0, 3} and
    // {1, 2} (lower-triangular, so five 16 x 16 blocks each) and the X tiles
    // that need them, helpers 2 and 3 split the Y tiles
    auto xy = [&](int c, int hl) {
        const int i3 = c % 3, i2 = c & 1;
        const u16 *Ks = kbuf(i3), *Qs = qbuf(i2), *dOs = obuf(i2), *dOe = oebuf(i2);
        if (hl < 2) {
            if (add) return;
            const float *gm = gam_of(i3);
            float *XT = xbuf(i2);
            auto pcol = [&](auto JB) {
                constexpr int jb = decltype(JB)::value;
                const float gj = gm[16 * jb + r];
                f32x4 p[4];
#pragma unroll
                for (int ib = jb; ib < 4; ++ib) {
                    p[ib] = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 aq = *(const bf16x8 *)(Qs + (16 * ib + r) * LDD + 32 * ks + 8 * g);
                        const bf16x8 bk = *(const bf16x8 *)(Ks + (16 * jb + r) * LDD + 32 * ks + 8 * g);
                        p[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, p[ib], 0, 0, 0);
                    }
                }
                short4_t pb[4];
#pragma unroll
                for (int ib = jb; ib < 4; ++ib) {
                    // p[ib][e] = P[i = 16 ib + 4g + e][j = 16 jb + r]: decay and
                    // mask without branches
                    const float4 gv = *(const float4 *)(gm + 16 * ib + 4 * g);
                    const float gi[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float f = exp2_fast(gi[e] - gj);
                        p[ib][e] = (ib > jb || 4 * g + e >= r) ? p[ib][e] * f : 0.f;
                    }
                    pb[ib] = pack4(p[ib]);
                }
#pragma unroll
                for (int vx = 0; vx < VT; ++vx) {
                    f32x4 ax = zero4();
#pragma unroll
                    for (int ib = jb; ib < 4; ++ib) {
                        const short4_t ad = operand_tr4(dOs, LDV, 16 * ib, 16 * vx, lane);
                        ax = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ad, pb[ib], ax, 0, 0, 0);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) XT[(16 * vx + 4 * g + e) * LDX + 16 * jb + r] = ax[e];
                }
            };
            if (hl == 0) {
                pcol(std::integral_constant<int, 0>{});
                pcol(std::integral_constant<int, 3>{});
            } else {
                pcol(std::integral_constant<int, 1>{});
                pcol(std::integral_constant<int, 2>{});
            }
        } else {
            float *YT = ybuf(i2);
            constexpr int NY = DT * VT, HY = (NY + 1) / 2;
#pragma unroll
            for (int t0 = 0; t0 < HY; ++t0) {
                const int t = (hl - 2) * HY + t0;
                if (NY % 2 != 0 && t >= NY) break;
                const int vy = t / DT, db = t % DT;
                f32x4 ay = zero4();
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const short4_t ad = operand_tr4(dOe, LDV, 16 * ib, 16 * vy, lane);
                    const short4_t bq = operand_tr4(Qs, LDD, 16 * ib, 16 * db, lane);
                    ay = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ad, bq, ay, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) YT[(16 * vy + 4 * g + e) * LDX + 16 * db + r] = ay[e];
            }
        }
    };
    // one step of the chain on chunk c; dh' of chunk c goes out first
    auto chain_step = [&](int c) {
        const int i3 = c % 3, i2 = c & 1;
        const u16 *Ks = kbuf(i3), *NKs = nbuf(i3);
        const float *egn = egn_of(i3), *XT = xbuf(i2), *YT = ybuf(i2);
        const float el = el_of(i3)[0];
        short4_t hb[DT];
        const int v = v0 + r;
        u16 *dst = dhs + (((size_t)bh * NC + c) * dv + V0 + v) * dk;
#pragma unroll
        for (int kb = 0; kb < DT; ++kb) {
            hb[kb] = pack4(hacc[kb]);
            const int d0 = 16 * kb + 4 * g;
            if (v < nvc) {
                if (dk % 4 == 0) {
                    if (d0 < dk) *(short4_t *)(dst + d0) = hb[kb];
                } else {
                    const uint2 u = __builtin_bit_cast(uint2, hb[kb]);
                    const u16 x4[4] = {(u16)(u.x & 0xFFFF), (u16)(u.x >> 16), (u16)(u.y & 0xFFFF), (u16)(u.y >> 16)};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < dk) dst[d0 + e] = x4[e];
                }
            }
        }
        if (!add) {
            // dW = diag(e^{gam_n - gam}) K dh' + X
            f32x4 w[4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) w[tm] = zero4();
#pragma unroll
            for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const short4_t ak = *(const short4_t *)(Ks + (16 * tm + r) * LDD + 16 * kb + 4 * g);
                    w[tm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, hb[kb], w[tm], 0, 0, 0);
                }
            }
            short4_t wb[4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const float4 sc = *(const float4 *)(egn + 16 * tm + 4 * g);
                const float4 x = *(const float4 *)(XT + v * LDX + 16 * tm + 4 * g);
                wb[tm] = pack4(f32x4{w[tm][0] * sc.x + x.x, w[tm][1] * sc.y + x.y, w[tm][2] * sc.z + x.z,
                                     w[tm][3] * sc.w + x.w});
            }
            // dh = e^{gam_n} dh' + Y + (-Kw)^T dW
#pragma unroll
            for (int kb = 0; kb < DT; ++kb) {
                const float4 y = *(const float4 *)(YT + v * LDX + 16 * kb + 4 * g);
                hacc[kb] = f32x4{hacc[kb][0] * el + y.x, hacc[kb][1] * el + y.y, hacc[kb][2] * el + y.z,
                                 hacc[kb][3] * el + y.w};
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const short4_t an = operand_tr4(NKs, LDD, 16 * tm, 16 * kb, lane);
                    hacc[kb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(an, wb[tm], hacc[kb], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < DT; ++kb) {
                const float4 y = *(const float4 *)(YT + v * LDX + 16 * kb + 4 * g);
                hacc[kb] = f32x4{hacc[kb][0] * el + y.x, hacc[kb][1] * el + y.y, hacc[kb][2] * el + y.z,
                                 hacc[kb][3] * el + y.w};
            }
        }
    };

    // ---- prologue: dh at the end of the sequence (chain), first two chunks
    // requested (helpers)
    if (chain) {
#pragma unroll
        for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * kb + 4 * g + e, vv = v0 + r;
                hacc[kb][e] = (a.dhT && d < dk && vv < nvc) ? a.dhT[((size_t)bh * dk + d) * dv + V0 + vv] : 0.f;
            }
        }
    } else {
        fetch(((CN & 1) == gp) ? CN : CN - 1);
    }

    // the serial path issues first wherever it shares a SIMD with helpers
    if (chain) __builtin_amdgcn_s_setprio(3);
    // step c: chain on chunk c; helpers form X, Y of chunk c-1; the group of
    // c's parity stages chunk c-2 and requests chunk c-4
    for (int c = CN + 2; c >= 0; --c) {
        {
            int t = tid;
            asm volatile("" : "+v"(t));
            lane = t & 63;
            g = lane >> 4;
            r = lane & 15;
            gtid = (t - 64 * VT) & (NGT - 1);
        }
        if (chain) {
            if (c <= CN) chain_step(c);
        } else {
            if ((c & 1) == gp) {
                if (c - 2 >= 0 && c - 2 <= CN) stash(c - 2);
                fetch(c - 4);
            } else if (c - 1 >= 0 && c - 1 <= CN) {
                xy(c - 1, hw & 3);
            }
        }
        __syncthreads();
    }
    if (chain && a.dh0) {
#pragma unroll
        for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * kb + 4 * g + e, vv = v0 + r;
                if (d < dk && vv < nvc) a.dh0[((size_t)bh * dk + d) * dv + V0 + vv] = hacc[kb][e];
            }
        }
    }
}

// --------------------------------------------------------------- local
//
// Storage: inputs (K, Q, V, dO, -Kw, U, Tm, h^T, dh'^T) are stashed as they
// are in memory (token rows, transposed states, Tm rows); every product is
// stored once, transposed with packed writes ("t" suffix: Xt[col][row] =
// X[row][col]). Each product reads an operand straight or through the
// transposing LDS read, whichever its storage needs (gemm<..., ATR, BTR>).
// U and Tm come from the forward context, so no triangular solve runs here.
// Twelve LDS regions, some reused once a value is dead (Pn = phase n; the
// workgroup barrier that ends a phase separates the last read of a value
// from the first write of its successor):
//   RK K, RQ Q, RH h^T (P1-7), RU U (P1), RN -Kw (P1)
//   RPt Pt (P1-4) -> V (stashed in P5, read in P6) -> dSt (P7-8)
//   RWt Wt (P1-7)                     RdO dO (stashed in P1, P4-5) -> -dV't (P6-9)
//   Rdh dh'^T (stashed in P1, P4-5) -> partial sums (P9)
//   RdW dWt (P4-6)
//   RdPG (dP o Gam)^T (P5-6) -> dQ (P9)
//   RTm Tm (stashed in P5, P6) -> dK (P9)
// Every input is stashed once; dO and dh' (requested at the top of the
// chunk) are stashed at the end of P1, V and Tm at the end of P5, so each
// rides on a barrier that is there anyway.


template <bool BF, int D, int NW> struct LocalSmem {
    using S = typename Op<BF>::S;
    static constexpr int LDD = D + Op<BF>::PAD;
    static constexpr int LDC = C + Op<BF>::PAD;
    static constexpr int mx(int x, int y) { return x > y ? x : y; }
    static constexpr int sCD = C * LDD * (int)sizeof(S); // token rows [C][D]
    static constexpr int sDC = D * LDC * (int)sizeof(S); // [D][C]
    static constexpr int sDD = D * LDD * (int)sizeof(S); // state [D][D]
    static constexpr int sCC = C * LDC * (int)sizeof(S); // [C][C]
    static constexpr int sPart = (3 * C * (D / 16) + 3 * C * 4) * 4;
    static constexpr int oK = 0;
    static constexpr int oQ = oK + sCD;
    static constexpr int oH = oQ + sCD;
    static constexpr int oU = oH + sDD;
    static constexpr int oN = oU + sCD;
    static constexpr int oPt = oN + sCD;
    static constexpr int oWt = oPt + mx(sCC, sCD);
    static constexpr int odO = oWt + sDC;
    static constexpr int odh = odO + mx(sCD, sDC);
    static constexpr int odW = odh + mx(sDD, sPart);
    static constexpr int odPG = odW + sDC;
    static constexpr int oTm = odPG + mx(sCC, sCD);
    static constexpr int oGam = oTm + mx(sCC, sCD);
    static constexpr int oEg = oGam + NW * C * 8; // gam: one copy per wave
    static constexpr int oEgn = oEg + C * 4;
    static constexpr int oBet = oEgn + C * 4;
    static constexpr int oGch = oBet + C * 4;
    static constexpr int oMisc = oGch + C * 4;
    static constexpr int oRinv = oMisc + (16 + NW) * 4; // 1/|k| per row (normalised keys)
    static constexpr int SIZE = oRinv + C * 4;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

// EDGE: the layer edges (key normalisation, skip term, dD) are compiled in;
// the plain instantiation carries none of their code or registers
template <bool BF, int D, bool VEC, bool EDGE, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_local_kernel(BwdLocalArgs a) {
    static_assert(!EDGE || NW == DD_SLOTS, "one skip-term slot per wave");
    constexpr int NTL = 64 * NW; // threads
    using O = Op<BF>;
    using S = typename O::S;
    using L = LocalSmem<BF, D, NW>;
    constexpr int LDD = L::LDD, LDC = L::LDC, DT = D / 16;
    constexpr int PWC = Tiles<4, 4, NW>::PW, PWD = Tiles<4, DT, NW>::PW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *RQ = (S *)(smem + L::oQ);
    S *RH = (S *)(smem + L::oH);
    S *RU = (S *)(smem + L::oU);
    S *RN = (S *)(smem + L::oN);
    S *RPt = (S *)(smem + L::oPt);
    S *RWt = (S *)(smem + L::oWt);
    S *RdO = (S *)(smem + L::odO);
    S *Rdh = (S *)(smem + L::odh);
    S *RdW = (S *)(smem + L::odW);
    S *RdPG = (S *)(smem + L::odPG);
    S *RTm = (S *)(smem + L::oTm);
    double *gam = (double *)(smem + L::oGam);
    float *eg = (float *)(smem + L::oEg);
    float *egn = (float *)(smem + L::oEgn);
    float *bet = (float *)(smem + L::oBet);
    float *gch = (float *)(smem + L::oGch);
    float *misc = (float *)(smem + L::oMisc);
    float *rinvK = (float *)(smem + L::oRinv);

    const SeqArgs &s = a.s;
    const int tid0 = threadIdx.x;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv;
    const bool add = s.additive != 0;
    // Persistent blocks, each working through a list of chunks. Chunks are
    // numbered heads fastest (the rows of all heads of one token are adjacent
    // in memory). Block i runs on XCD i % 8; when the counts allow, each XCD
    // walks one contiguous eighth of the numbering with its blocks side by
    // side, so chunks that share cache lines run together on one XCD.
    const int NCH = s.B * H * s.NC, G = gridDim.x;
    const bool split = G % 8 == 0 && NCH % 8 == 0;
    const int per = split ? NCH / 8 : NCH;
    const int first = split ? ((int)blockIdx.x % 8) * per + (int)blockIdx.x / 8 : (int)blockIdx.x;
    const int lim = split ? ((int)blockIdx.x % 8 + 1) * per : NCH; // end of this block's range
    const int step = split ? G / 8 : G;
    // chunk lid = (b * NC + c) * H + h, advanced by `step` with carries
    struct Pos {
        int lid, h, c, b;
    };
    const int sh = step % H, sc = (step / H) % s.NC, sb = step / (H * s.NC);
    auto advance = [&](Pos p) {
        p.lid += step;
        p.h += sh;
        int cy = p.h >= H;
        p.h -= cy ? H : 0;
        p.c += sc + cy;
        cy = p.c >= s.NC;
        p.c -= cy ? s.NC : 0;
        p.b += sb + cy;
        return p;
    };

    // Global inputs are requested into registers well before their use: the
    // ones the first phases need (K, Q, h, U, -Kw, gates) while the previous
    // chunk finishes, the others at the top of the chunk itself.
    ChunkFrag<BF, D, C, NTL> fk, fq, fv, fo, fn, fu;
    ChunkFrag<BF, D, D, NTL> fh, fd;
    ChunkFrag<BF, C, C, NTL> ft;
    float gr = 0.f, br = 0.f, alr = 0.f;
    auto fetch_early = [&](const Pos &p, int tid, int lane) {
        const int h = p.h, c = p.c, b = p.b;
        const int n = min(C, T - c * C);
        const size_t row0 = (size_t)b * T + c * C, cb = ((size_t)b * H + h) * s.NC + c;
        fk.template fetch<VEC>((const S *)s.k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        fq.template fetch<VEC>((const S *)s.q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        fh.template fetch<VEC>((const S *)a.cs + cb * dk * dv, (size_t)dk, dv, dk, tid);
        fu.template fetch<VEC>((const S *)a.U + cb * C * dv, (size_t)dv, n, dv, tid);
        if (!add) fn.template fetch<VEC>((const S *)a.NK + cb * C * dk, (size_t)dk, n, dk, tid);
        alr = s.A_log[h];
        gr = load_row_scalar(s.g + row0 * H + h, H, lane, n);
        br = load_row_scalar(s.beta + row0 * H + h, H, lane, n);
    };
    if (first >= lim) return;
    Pos cur{first, first % H, (first / H) % s.NC, first / (H * s.NC)};
    fetch_early(cur, tid0, tid0 & 63);
    // a chunk's first inputs (K, Q, h, U, -Kw) go to LDS as soon as their
    // regions are free: before the loop for the first chunk, right after the
    // previous chunk's output stores for the others
    auto stash_inputs = [&](int tid) {
        if constexpr (EDGE) {
            if (s.l2k) fk.normalize_rows(rinvK, tid);
        }
        fk.stash(Ks, LDD, tid);
        fq.stash(RQ, LDD, tid);
        fh.stash(RH, LDD, tid);
        fu.stash(RU, LDD, tid);
        if (!add) fn.stash(RN, LDD, tid);
    };
    stash_inputs(tid0);
    for (;;) {
    // the thread index is hidden from the optimiser at the top of every
    // chunk, so per-lane addresses are formed where they are used instead of
    // being hoisted out of the loop and held in registers throughout
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6, lane = tid & 63;
    // this wave's [C][D] tiles of an LDS matrix with rows of LDD elements, in
    // the accumulator layout (bf16: one transposing read per tile)
    auto tiles_cd = [&](const S *X, f32x4 *out) {
        if constexpr (BF)
            load_tiles<4, DT, NW>(X, LDD, out, wave, lane);
        else
            for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) { out[i][e] = to_f(X[row * LDD + col]); });
    };
    const int h = cur.h, c = cur.c, b = cur.b;
    const int bh = b * H + h;
    const int t0 = c * C, n = min(C, T - t0);
    const double A = -exp((double)alr);
    const size_t row0 = (size_t)b * T + t0, cb = (size_t)bh * s.NC + c;
    fo.template fetch<VEC>((const S *)a.dout + (row0 * H + h) * dv, (size_t)H * dv, n, dv, tid);
    fd.template fetch<VEC>((const S *)a.dhs + cb * dk * dv, (size_t)dk, dv, dk, tid);
    ft.template fetch<VEC>((const S *)a.Tm + cb * C * C, (size_t)C, C, C, tid);
    fv.template fetch<VEC>((const S *)s.v + (row0 * H + h) * dv, (size_t)H * dv, n, dv, tid);

    // Contributions to dbeta and dgam, accumulated per lane at the (row, col)
    // positions this lane owns and reduced once at the end:
    //   rbD / rgD / rsD: row sums over [C][D] grids (dbeta, dgam, s_j)
    //   rbC: row sums, xgC: row sums minus column sums over [C][C] grids
    f32x4 rbD[PWD], rgD[PWD], rsD[PWD], rbC[PWC], xgC[PWC];
#pragma unroll
    for (int i = 0; i < PWD; ++i) rbD[i] = rgD[i] = rsD[i] = zero4();
#pragma unroll
    for (int i = 0; i < PWC; ++i) rbC[i] = xgC[i] = zero4();

    // ---- P1: gates, decay, K K^T and Q K^T; W = U - Kw h
    __syncthreads(); // K, Q, h, U, -Kw stashed
    // Gam, K K^T o Gam and P stay in registers at this lane's [C][C] positions
    f32x4 gC[PWC], kkg[PWC], pC[PWC];
    {
        f32x4 sk[PWC], sq[PWC];
#pragma unroll
        for (int i = 0; i < PWC; ++i) sk[i] = sq[i] = zero4();
        if (!add) gemm<BF, 4, 4, D, false, false, NW>(Ks, LDD, Ks, LDD, sk, wave, lane);
        gemm<BF, 4, 4, D, false, false, NW>(RQ, LDD, Ks, LDD, sq, wave, lane);
        // while the products run, every wave forms the chunk's decay (lane =
        // row) and keeps a copy of gam of its own; wave 0 publishes the rest
        const float gl = lane < n ? gate_of(gr, s.logits) : 0.f;
        const Decay dc = decay_lane(gl, A * LOG2E, lane);
        double *gw = gam + wave * C;
        gw[lane] = dc.gam2;
        if (wave == 0) {
            gch[lane] = gl;
            bet[lane] = lane < n ? gate_of(br, s.logits) : 0.f;
            eg[lane] = dc.eg;
            egn[lane] = dc.egn;
            if (lane == 0) misc[0] = dc.eglast;
        }
        for_tiles<4, 4, NW>(wave, lane, [&](int i, int e, int row, int col) {
            const float G = gamma_ij(gw, row, col);
            gC[i][e] = G;
            kkg[i][e] = (row > col) ? sk[i][e] * G : 0.f;
            pC[i][e] = sq[i][e] * G;
        });
        store_T<BF, 4, 4, NW>(pC, RPt, LDC, wave, lane); // Pt
    }
    {
        f32x4 accW[PWD];
        tiles_cd(RU, accW);
        if (!add) gemm<BF, 4, DT, D, false, false, NW>(RN, LDD, RH, LDD, accW, wave, lane); // + (-Kw) h
        store_T<BF, 4, DT, NW>(accW, RWt, LDC, wave, lane);                               // Wt
    }
    // dO and dh' into their own regions, and <h, dh'> from the register
    // fragments while both are held (one butterfly, one slot per wave)
    fo.stash(RdO, LDD, tid);
    fd.stash(Rdh, LDD, tid);
    {
        float hd = 0.f;
#pragma unroll
        for (int m = 0; m < fh.NIT; ++m) {
            typename ChunkFrag<BF, D, D, NTL>::U x, y;
            x.u = fh.item(m);
            y.u = fd.item(m);
#pragma unroll
            for (int e = 0; e < O::VEC; ++e) hd += to_f(x.s[e]) * to_f(y.s[e]);
        }
        hd = wave_sum(hd);
        if (lane == 0) misc[16 + wave] = hd;
    }
    __syncthreads(); // Pt, Wt, dO and dh' complete
    // ---- P4: dW = P^T dO + diag(e^{gam_n - gam}) K dh'
    {
        f32x4 accdW[PWD], accX[PWD];
#pragma unroll
        for (int i = 0; i < PWD; ++i) accdW[i] = accX[i] = zero4();
        gemm<BF, 4, DT, C, false, true, NW>(RPt, LDC, RdO, LDD, accdW, wave, lane); // P^T dO
        gemm<BF, 4, DT, D, false, false, NW>(Ks, LDD, Rdh, LDD, accX, wave, lane);  // K dh'
        for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) { accdW[i][e] += egn[row] * accX[i][e]; });
        store_T<BF, 4, DT, NW>(accdW, RdW, LDC, wave, lane); // dWt
    }
    __syncthreads();
    // ---- P5: dOh = dO h^T, dKt = W dh'^T, dP
    f32x4 accQ[PWD], accKd[PWD];
#pragma unroll
    for (int i = 0; i < PWD; ++i) accQ[i] = accKd[i] = zero4();
    gemm<BF, 4, DT, D, false, true, NW>(RdO, LDD, RH, LDD, accQ, wave, lane); // dO h^T
    {
        f32x4 accKt[PWD];
#pragma unroll
        for (int i = 0; i < PWD; ++i) accKt[i] = zero4();
        gemm<BF, 4, DT, D, true, true, NW>(RWt, LDC, Rdh, LDD, accKt, wave, lane); // W dh'^T
        // dK += diag(e^{gam_n - gam}) dKt ; s_j = e^{gam_n - gam_j} k_j . dKt_j
        f32x4 kt[PWD];
        tiles_cd(Ks, kt);
        for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) {
            const float x = egn[row] * accKt[i][e];
            accKd[i][e] = x;
            rsD[i][e] = x * kt[i][e];
        });
        // dP = dO W^T (lower incl. diagonal), dP o Gam -> RdPG
        {
            f32x4 accP[PWC];
#pragma unroll
            for (int i = 0; i < PWC; ++i) accP[i] = zero4();
            gemm<BF, 4, 4, D, false, true, NW>(RdO, LDD, RWt, LDC, accP, wave, lane);
            for_tiles<4, 4, NW>(wave, lane, [&](int i, int e, int row, int col) {
                const float dp = row >= col ? accP[i][e] : 0.f;
                xgC[i][e] += dp * pC[i][e]; // dP o P
                accP[i][e] = dp * gC[i][e];
            });
            store_T<BF, 4, 4, NW>(accP, RdPG, LDC, wave, lane); // dPGt
        }
        // Tm, and V where Pt was (last read in P4)
        ft.stash(RTm, LDC, tid);
        fv.stash(RPt, LDD, tid);
    }
    __syncthreads(); // dWt, dPGt, Tm and V complete; dO and dh' no longer read
    // ---- P6: dV' = Tm^T dW, dQ, dK += (dP o Gam)^T Q
    {
        f32x4 accV[PWD];
#pragma unroll
        for (int i = 0; i < PWD; ++i) accV[i] = zero4();
        gemm<BF, 4, DT, C, true, false, NW>(RTm, LDC, RdW, LDC, accV, wave, lane);
        // dQ = diag(e^gam) dO h^T + (dP o Gam) K, dK += (dP o Gam)^T Q
        {
            f32x4 qt[PWD];
            tiles_cd(RQ, qt);
            for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) {
                accQ[i][e] *= eg[row];
                rgD[i][e] += accQ[i][e] * qt[i][e]; // e^{gam_i} q_i . dOh_i
            });
        }
        gemm<BF, 4, DT, C, true, true, NW>(RdPG, LDC, Ks, LDD, accQ, wave, lane);
        gemm<BF, 4, DT, C, false, true, NW>(RdPG, LDC, RQ, LDD, accKd, wave, lane);
        {
            f32x4 vt[PWD];
            tiles_cd(RPt, vt);
            for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) {
                rbD[i][e] += vt[i][e] * accV[i][e]; // v_i . dV'_i
            });
        }
#pragma unroll
        for (int i = 0; i < PWD; ++i) accV[i] = -accV[i];
        store_T<BF, 4, DT, NW>(accV, RdO, LDC, wave, lane); // -dV't (also the source of dv)
    }
    __syncthreads(); // -dV't complete; V, Tm, dWt, dPGt no longer read
    // ---- P7: dK' = (-dV') h^T and its terms, dL = (-dV') W^T, dS
    if (!add) {
        {
            f32x4 accKp[PWD];
#pragma unroll
            for (int i = 0; i < PWD; ++i) accKp[i] = zero4();
            gemm<BF, 4, DT, D, true, true, NW>(RdO, LDC, RH, LDD, accKp, wave, lane);
            f32x4 kt[PWD];
            tiles_cd(Ks, kt);
            for_tiles<4, DT, NW>(wave, lane, [&](int i, int e, int row, int col) {
                const float kk = eg[row] * kt[i][e] * accKp[i][e]; // e^{gam_i} k_i . dK'_i
                rbD[i][e] += kk;
                rgD[i][e] += bet[row] * kk;
                accKd[i][e] += bet[row] * eg[row] * accKp[i][e];
            });
        }
        f32x4 accL[PWC];
#pragma unroll
        for (int i = 0; i < PWC; ++i) accL[i] = zero4();
        gemm<BF, 4, 4, D, true, true, NW>(RdO, LDC, RWt, LDC, accL, wave, lane);
        for_tiles<4, 4, NW>(wave, lane, [&](int i, int e, int row, int col) {
            const float dl = (row > col) ? accL[i][e] : 0.f;
            rbC[i][e] += dl * kkg[i][e];
            xgC[i][e] += dl * bet[row] * kkg[i][e]; // dL o L
            accL[i][e] = bet[row] * dl * gC[i][e];
        });
        store_T<BF, 4, 4, NW>(accL, RPt, LDC, wave, lane); // dSt
        __syncthreads();
        // ---- P8: dK += dS K + dS^T K
        gemm<BF, 4, DT, C, true, true, NW>(RPt, LDC, Ks, LDD, accKd, wave, lane);
        gemm<BF, 4, DT, C, false, true, NW>(RPt, LDC, Ks, LDD, accKd, wave, lane);
    }
    // every fragment is stashed and the products are done: request the first
    // inputs of the next chunk (the current one again after the last, so the
    // loads never depend on a branch)
    const Pos nxt = advance(cur);
    const bool more = nxt.lid < lim;
    fetch_early(more ? nxt : cur, tid, lane);
    // dQ and dK leave through LDS (dPGt and Tm were last read in P6): bf16
    // with 16-byte rows transposed, [D][C] like -dV't, so that one
    // transposing read hands a lane 16 bytes of an output row; otherwise
    // (and with the layer edges, whose key normalisation sums over rows) as
    // 16-byte rows
    constexpr bool TOUT = BF && VEC && !EDGE;
    if constexpr (TOUT) {
        store_T<BF, 4, DT, NW>(accQ, RdPG, LDC, wave, lane);
        store_T<BF, 4, DT, NW>(accKd, RTm, LDC, wave, lane);
    } else {
        store_N<BF, 4, DT, NW>(accQ, RdPG, LDD, wave, lane);
        store_N<BF, 4, DT, NW>(accKd, RTm, LDD, wave, lane);
    }
    // ---- P9: one fixed-order reduction of every dbeta / dgam contribution
    {
        // dh' was last read in P5
        float *pRbD = (float *)Rdh, *pRgD = pRbD + C * DT, *pRsD = pRgD + C * DT;
        float *pRbC = pRsD + C * DT, *pRgC = pRbC + C * 4, *pCgC = pRgC + C * 4;
        if constexpr (DT == 4) {
            // [C][D] and [C][C] tiles sit at the same places: add the row
            // contributions before the cross-lane sums
#pragma unroll
            for (int i = 0; i < PWD; ++i) {
                rbD[i] += rbC[i];
                rgD[i] += xgC[i];
            }
        } else {
            row_partials<4, 4, NW>(rbC, pRbC, wave, lane);
            row_partials<4, 4, NW>(xgC, pRgC, wave, lane);
        }
        row_partials<4, DT, NW>(rbD, pRbD, wave, lane);
        row_partials<4, DT, NW>(rgD, pRgD, wave, lane);
        row_partials<4, DT, NW>(rsD, pRsD, wave, lane);
        col_partials<4, 4, NW>(xgC, pCgC, wave, lane);
        __syncthreads();
        // dq, dk, dv rows of the chunk, written by waves 1.. while wave 0 forms
        // dbeta and dg: 16-byte stores (dv = -beta * (-dV'), from the
        // transposed -dV't). Edges: with normalised keys dk goes back
        // through the normalisation, dk = (dk_hat - k_hat (k_hat . dk_hat)) / |k|
        // (row dots over the lanes that hold a row); with the skip term dv
        // gains D_h do, and the chunk's share of dD_h (sum of do * v) goes to
        // one slot per wave.
        if constexpr (TOUT) {
            // units of 16 rows x 32 columns of dq, dk or dv, spread over
            // waves 1..: lane (g, r) stores row 16 mb + r, columns
            // 32 kb + 8 g .. + 7 (dv = -beta * (-dV'))
            constexpr int UPM = 4 * (D / 32);
            const int r16 = lane & 15, g4 = lane >> 4;
            if (wave > 0) {
                for (int u = wave - 1; u < 3 * UPM; u += NW - 1) {
                    const int mtx = u / UPM, mb = (u % UPM) & 3, kb = (u % UPM) >> 2;
                    const u16 *X = mtx == 0 ? (const u16 *)RdPG : (mtx == 1 ? (const u16 *)RTm : (const u16 *)RdO);
                    union {
                        bf16x8 b;
                        uint4 u;
                        u16 x[8];
                    } w;
                    w.b = operand_tr(X, LDC, 32 * kb, 16 * mb, lane);
                    const int j = 16 * mb + r16, c0 = 32 * kb + 8 * g4, dd = mtx == 2 ? dv : dk;
                    if (j < n && c0 < dd) {
                        if (mtx == 2) {
                            const float nb = -bet[j];
#pragma unroll
                            for (int e = 0; e < 8; ++e) w.x[e] = f2bf(nb * bf2f(w.x[e]));
                        }
                        S *dst = (S *)(mtx == 0 ? a.dq : (mtx == 1 ? a.dk : a.dv)) + (row0 * H + h) * dd;
                        *reinterpret_cast<uint4 *>(dst + (size_t)j * H * dd + c0) = w.u;
                    }
                }
            }
        } else if constexpr (!EDGE) {
            S *dq_out = (S *)a.dq + (row0 * H + h) * dk;
            S *dk_out = (S *)a.dk + (row0 * H + h) * dk;
            S *dv_out = (S *)a.dv + (row0 * H + h) * dv;
            constexpr int V = O::VEC, NG = D / V;
            if (wave == 0) {
            } else if (VEC) {
                for (int it = tid - 64; it < C * NG; it += NTL - 64) {
                    const int j = it / NG, c0 = (it % NG) * V;
                    if (j >= n) continue;
                    if (c0 < dk) {
                        *reinterpret_cast<uint4 *>(dq_out + (size_t)j * H * dk + c0) =
                            *reinterpret_cast<const uint4 *>(RdPG + j * LDD + c0);
                        *reinterpret_cast<uint4 *>(dk_out + (size_t)j * H * dk + c0) =
                            *reinterpret_cast<const uint4 *>(RTm + j * LDD + c0);
                    }
                    if (c0 < dv) {
                        union {
                            uint4 u;
                            S x[V];
                        } pk;
                        const float nb = -bet[j];
#pragma unroll
                        for (int e = 0; e < V; ++e) pk.x[e] = from_f<BF>(nb * to_f(RdO[(c0 + e) * LDC + j]));
                        *reinterpret_cast<uint4 *>(dv_out + (size_t)j * H * dv + c0) = pk.u;
                    }
                }
            } else {
                for (int it = tid - 64; it < C * D; it += NTL - 64) {
                    const int j = it / D, col = it % D;
                    if (j >= n) continue;
                    if (col < dk) {
                        dq_out[(size_t)j * H * dk + col] = RdPG[j * LDD + col];
                        dk_out[(size_t)j * H * dk + col] = RTm[j * LDD + col];
                    }
                    if (col < dv) dv_out[(size_t)j * H * dv + col] = from_f<BF>(-bet[j] * to_f(RdO[col * LDC + j]));
                }
            }
        } else {
            {
                S *dq_out = (S *)a.dq + (row0 * H + h) * dk;
                S *dk_out = (S *)a.dk + (row0 * H + h) * dk;
                S *dv_out = (S *)a.dv + (row0 * H + h) * dv;
                const S *do_in = (const S *)a.dout + (row0 * H + h) * dv;
                const S *v_in = (const S *)s.v + (row0 * H + h) * dv;
                const bool l2k = EDGE && s.l2k;
                const float *Dp = EDGE ? s.D : nullptr;
                float *dDp = EDGE ? a.dD_part : nullptr;
                const float Dh = Dp ? Dp[h] : 0.f;
                const bool edge_v = Dp || dDp; // do (and v) rows are needed
                float dsum = 0.f;
                constexpr int V = O::VEC, NG = D / V;
                union Pk {
                    uint4 u;
                    S x[V];
                };
                if (wave == 0) {
                } else if (VEC) {
                    for (int it = tid - 64; it < C * NG; it += NTL - 64) {
                        const int j = it / NG, c0 = (it % NG) * V;
                        Pk kd;
                        kd.u = *reinterpret_cast<const uint4 *>(RTm + j * LDD + c0);
                        if (l2k) {
                            Pk kh;
                            kh.u = *reinterpret_cast<const uint4 *>(Ks + j * LDD + c0);
                            float dot = 0.f;
#pragma unroll
                            for (int e = 0; e < V; ++e) dot += to_f(kh.x[e]) * to_f(kd.x[e]);
#pragma unroll
                            for (int off = NG / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
                            const float ri = rinvK[j];
#pragma unroll
                            for (int e = 0; e < V; ++e) kd.x[e] = from_f<BF>((to_f(kd.x[e]) - to_f(kh.x[e]) * dot) * ri);
                        }
                        if (j >= n) continue;
                        if (c0 < dk) {
                            *reinterpret_cast<uint4 *>(dq_out + (size_t)j * H * dk + c0) =
                                *reinterpret_cast<const uint4 *>(RdPG + j * LDD + c0);
                            *reinterpret_cast<uint4 *>(dk_out + (size_t)j * H * dk + c0) = kd.u;
                        }
                        if (c0 < dv) {
                            Pk pk, dov, vv;
                            const float nb = -bet[j];
                            if (edge_v) {
                                dov.u = *reinterpret_cast<const uint4 *>(do_in + (size_t)j * H * dv + c0);
                                vv.u = *reinterpret_cast<const uint4 *>(v_in + (size_t)j * H * dv + c0);
                            }
#pragma unroll
                            for (int e = 0; e < V; ++e) {
                                float x = nb * to_f(RdO[(c0 + e) * LDC + j]);
                                if (Dp) x += Dh * to_f(dov.x[e]);
                                if (dDp) dsum += to_f(dov.x[e]) * to_f(vv.x[e]);
                                pk.x[e] = from_f<BF>(x);
                            }
                            *reinterpret_cast<uint4 *>(dv_out + (size_t)j * H * dv + c0) = pk.u;
                        }
                    }
                } else {
                    for (int it = tid - 64; it < C * D; it += NTL - 64) {
                        const int j = it / D, col = it % D;
                        float kdv = to_f(RTm[j * LDD + col]);
                        if (l2k) {
                            const float khv = to_f(Ks[j * LDD + col]);
                            float dot = khv * kdv;
#pragma unroll
                            for (int off = D / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
                            kdv = (kdv - khv * dot) * rinvK[j];
                        }
                        if (j >= n) continue;
                        if (col < dk) {
                            dq_out[(size_t)j * H * dk + col] = RdPG[j * LDD + col];
                            dk_out[(size_t)j * H * dk + col] = from_f<BF>(kdv);
                        }
                        if (col < dv) {
                            float x = -bet[j] * to_f(RdO[col * LDC + j]);
                            if (edge_v) {
                                const float dd = to_f(do_in[(size_t)j * H * dv + col]);
                                if (Dp) x += Dh * dd;
                                if (dDp) dsum += dd * to_f(v_in[(size_t)j * H * dv + col]);
                            }
                            dv_out[(size_t)j * H * dv + col] = from_f<BF>(x);
                        }
                    }
                }
                if (dDp) {
                    dsum = wave_sum(dsum);
                    if (lane == 0) dDp[cb * DD_SLOTS + wave] = dsum;
                }
            }
        }
        if (wave == 0) {
            const int i = lane;
            float db = 0.f, dgm = 0.f, sj = 0.f;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                db += pRbD[i * DT + t];
                dgm += pRgD[i * DT + t];
                sj += pRsD[i * DT + t];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (DT != 4) {
                    db += pRbC[i * 4 + t];
                    dgm += pRgC[i * 4 + t];
                }
                dgm -= pCgC[i * 4 + t];
            }
            // gam_n enters through e^{gam_n} h and e^{gam_n - gam_j}: its gradient
            // e^{gam_n} <h, dh'> + sum_j s_j goes to the last row; -s_j to row j
            const float stot = wave_sum(sj);
            float hds = 0.f;
            for (int w = 0; w < NW; ++w) hds += misc[16 + w];
            dgm -= sj;
            if (i == C - 1) dgm += misc[0] * hds + stot;
            // dlam_r = sum_{i >= r} dgam_i = total - (prefix through r) + dgam_r
            const float pre = wave_prefix(dgm);
            const float x = lane_value(pre, 63) - pre + dgm;
            const float dg = (float)A * x;
            float p = (lane < n) ? gch[lane] * dg : 0.f;
            if (lane < n) {
                const size_t gi = (row0 + lane) * H + h;
                // with logit inputs, through the sigmoid: d/dx = s (1 - s) d/ds
                const float gs = gch[lane], bs = bet[lane];
                a.dg[gi] = s.logits ? dg * gs * (1.f - gs) : dg;
                a.dbeta[gi] = s.logits ? db * bs * (1.f - bs) : db;
            }
            p = wave_sum(p);
            if (lane == 0) a.dA_part[(size_t)bh * s.NC + c] = p;
        }
    }
    if (!more) break;
    cur = nxt;
    // the next chunk's first inputs: K was last read in P8, Q, h, U and -Kw
    // earlier, all before the partial-sum barrier; only the outputs with
    // normalised keys still read K and 1/|k|
    if constexpr (EDGE) __syncthreads();
    stash_inputs(tid);
    } // chunk loop
}

// --------------------------------------------------------------- wide local
//
// Local gradients of one chunk for head dims the LDS-resident kernel above
// does not hold (bf16 d > 64, fp32 d > 16): the same quantities and the same
// formulas, formed product by product. Every 64 x d and 64 x 64 intermediate
// goes to fp32 scratch of the workgroup's own (it stays in L2 between the
// phases); each product runs on fp32 MFMA tiles through LDS, 64-wide slices of
// the inner dimension at a time. Persistent workgroups over a fixed grid, so
// the scratch does not grow with the sequence.

constexpr int WIDE_GRID = 1024;
constexpr int WIDE_LD = 128;                                 // row stride of 64 x d scratch
constexpr int WIDE_SCRATCH = 5 * C * C + 7 * C * WIDE_LD;    // floats per workgroup
constexpr int WIDE_KS = 64;                                  // inner-dimension slice per staging
constexpr int WIDE_LDA = WIDE_KS + 4;                        // A slice [64][LDA]: rows 4 banks apart
constexpr int WIDE_LDB = WIDE_LD + 16;                       // B slice [KS][LDB]: rows 16 banks apart

// out = A (M x K) * B (K x N) for M <= 64, N <= 128; fa(m, k) and fb(k, n)
// fetch operands (only in range). The result is a grid of 16 x 16 tiles,
// row-major; wave w owns tiles w, w + 8, w + 16, w + 24, and in tile x lane
// l holds acc[x][y] = out[16 tm + 4 (l / 16) + y][16 tn + l % 16]
// (v_mfma_f32_16x16x4f32 layout). Ends with a barrier.
template <class FA, class FB>
__device__ __forceinline__ void wide_mm(int M, int N, int K, FA fa, FB fb, float *As, float *Bs, int tid,
                                        float (&acc)[4][4]) {
    const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kq = lane >> 4;
    const int TM = (M + 15) >> 4, TN = (N + 15) >> 4, NT = TM * TN, Np = 16 * TN;
    f32x4 c[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) c[x] = zero4();
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += WIDE_KS) {
        for (int e = tid; e < C * WIDE_KS; e += NTHR) {
            const int m = e / WIDE_KS, kk = e % WIDE_KS;
            As[m * WIDE_LDA + kk] = (m < M && k0 + kk < K) ? fa(m, k0 + kk) : 0.f;
        }
        for (int e = tid; e < WIDE_KS * Np; e += NTHR) {
            const int kk = e / Np, n = e % Np;
            Bs[kk * WIDE_LDB + n] = (n < N && k0 + kk < K) ? fb(k0 + kk, n) : 0.f;
        }
        __syncthreads();
        const int kn = min(WIDE_KS, K - k0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int t = wave + NWAVE * x;
            if (t < NT) {
                const int tm = t / TN, tn = t % TN;
                const float *ap = As + (16 * tm + r) * WIDE_LDA + kq;
                const float *bp = Bs + kq * WIDE_LDB + 16 * tn + r;
                for (int kk = 0; kk < kn; kk += 4)
                    c[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(ap[kk], bp[kk * WIDE_LDB], c[x], 0, 0, 0);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = c[x][y];
}

template <bool BF> __global__ __launch_bounds__(NTHR) void bwd_local_wide_kernel(BwdLocalArgs a) {
    using S = typename Op<BF>::S;
    __shared__ float As[C * WIDE_LDA];
    __shared__ float Bs[WIDE_KS * WIDE_LDB];
    __shared__ double gam[C];
    __shared__ float eg[C], egn[C], bet[C], gch[C], rk[C], red[NTHR];
    const SeqArgs &s = a.s;
    const int tid0 = threadIdx.x;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv, NC = s.NC;
    const bool add = s.additive != 0;
    float *sc = a.wide + (size_t)blockIdx.x * WIDE_SCRATCH;
    float *sP = sc, *sKG = sP + C * C, *sdP = sKG + C * C, *sdL = sdP + C * C, *sT = sdL + C * C;
    float *sW = sT + C * C, *sdW = sW + C * WIDE_LD, *sdOh = sdW + C * WIDE_LD, *sdKw = sdOh + C * WIDE_LD;
    float *sdKt = sdKw + C * WIDE_LD, *sdVp = sdKt + C * WIDE_LD, *sdKp = sdVp + C * WIDE_LD;
    const int NCH = s.B * H * NC;
    for (int lid = blockIdx.x; lid < NCH; lid += gridDim.x) {
        // the thread index is hidden from the optimiser per chunk, so per-lane
        // addresses are formed where they are used, not held across the loop
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int wave = tid >> 6, lane = tid & 63;
        // chunks numbered heads fastest (rows of all heads of a token are adjacent)
        const int h = lid % H, c = (lid / H) % NC, b = lid / (H * NC);
        const int bh = b * H + h, t0 = c * C, n = min(C, T - t0);
        const size_t row0 = (size_t)b * T + t0, cb = (size_t)bh * NC + c;
        const S *qb = (const S *)s.q + (row0 * H + h) * dk;
        const S *kb = (const S *)s.k + (row0 * H + h) * dk;
        const S *vb = (const S *)s.v + (row0 * H + h) * dv;
        const S *ob = (const S *)a.dout + (row0 * H + h) * dv;
        const S *hc = (const S *)a.cs + cb * dk * dv;  // h^T [dv][dk]
        const S *dhc = (const S *)a.dhs + cb * dk * dv; // dh'^T [dv][dk]
        const S *uc = (const S *)a.U + cb * C * dv;
        const S *nk = (const S *)a.NK + cb * C * dk;
        const S *tc = (const S *)a.Tm + cb * C * C;
        const size_t sq = (size_t)H * dk, sv = (size_t)H * dv;
        auto Q = [&](int i, int d) { return i < n ? to_f(qb[i * sq + d]) : 0.f; };
        // keys as the recurrence sees them (rk: 1 / |k| per row when normalised)
        auto K = [&](int i, int d) { return i < n ? to_f(kb[i * sq + d]) * rk[i] : 0.f; };
        auto V = [&](int i, int e) { return i < n ? to_f(vb[i * sv + e]) : 0.f; };
        auto dO = [&](int i, int e) { return i < n ? to_f(ob[i * sv + e]) : 0.f; };
        auto Hm = [&](int d, int e) { return to_f(hc[(size_t)e * dk + d]); };
        auto dH = [&](int d, int e) { return to_f(dhc[(size_t)e * dk + d]); };
        auto Um = [&](int i, int e) { return to_f(uc[(size_t)i * dv + e]); };
        auto NKm = [&](int i, int d) { return add ? 0.f : to_f(nk[(size_t)i * dk + d]); };
        auto Tmm = [&](int i, int j) { return to_f(tc[(size_t)i * C + j]); };
        auto Gm = [&](int i, int j) { return i >= j ? exp2_fast((float)(gam[i] - gam[j])) : 0.f; };
        const double A = -exp((double)s.A_log[h]);

        // ---- decay of the chunk (wave 0), gates
        if (wave == 0) {
            const float gr = load_row_scalar(s.g + row0 * H + h, H, lane, n);
            const float br = load_row_scalar(s.beta + row0 * H + h, H, lane, n);
            const float gl = lane < n ? gate_of(gr, s.logits) : 0.f;
            const Decay dcy = decay_lane(gl, A * LOG2E, lane);
            gam[lane] = dcy.gam2;
            eg[lane] = dcy.eg;
            egn[lane] = dcy.egn;
            bet[lane] = lane < n ? gate_of(br, s.logits) : 0.f;
            gch[lane] = gl;
            if (lane == 0) red[0] = dcy.eglast;
        }
        {
            // 1 / sqrt(|k|^2 + KEY_EPS) per row: eight lanes per row
            const int i = tid >> 3, gq = tid & 7;
            float ss = 0.f;
            if (s.l2k && i < n)
                for (int d = gq; d < dk; d += 8) {
                    const float x = to_f(kb[i * sq + d]);
                    ss += x * x;
                }
#pragma unroll
            for (int off = 4; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
            if (gq == 0) rk[i] = s.l2k ? 1.f / sqrtf(ss + KEY_EPS) : 1.f;
        }
        __syncthreads();
        const float eglast = red[0];
        float acc[4][4], acc2[4][4];
        // visit this lane's elements of an M x N product (wide_mm's layout)
        auto each = [&](int M, int N, auto f) {
            const int TN = (N + 15) >> 4, NT = ((M + 15) >> 4) * TN;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int t = wave + NWAVE * x;
                if (t < NT) {
                    const int i0 = 16 * (t / TN) + 4 * (lane >> 4), j = 16 * (t % TN) + (lane & 15);
#pragma unroll
                    for (int y = 0; y < 4; ++y)
                        if (i0 + y < M && j < N) f(i0 + y, j, x, y);
                }
            }
        };
        // ---- P = (Q K^T) o Gam (lower incl. diagonal); K K^T o Gam (strict)
        wide_mm(C, C, dk, Q, [&](int d, int j) { return K(j, d); }, As, Bs, tid, acc);
        each(C, C, [&](int i, int j, int x, int y) { sP[i * C + j] = acc[x][y] * Gm(i, j); });
        wide_mm(C, C, dk, K, [&](int d, int j) { return K(j, d); }, As, Bs, tid, acc);
        each(C, C, [&](int i, int j, int x, int y) { sKG[i * C + j] = (!add && i > j) ? acc[x][y] * Gm(i, j) : 0.f; });
        // ---- W = U + (-Kw) h
        wide_mm(C, dv, dk, NKm, Hm, As, Bs, tid, acc);
        each(C, dv, [&](int i, int e, int x, int y) { sW[i * WIDE_LD + e] = Um(i, e) + acc[x][y]; });
        __syncthreads();
        // ---- dW = P^T dO + diag(e^{gam_n - gam}) K dh'
        wide_mm(C, dv, C, [&](int i, int j) { return sP[j * C + i]; }, dO, As, Bs, tid, acc);
        wide_mm(C, dv, dk, K, dH, As, Bs, tid, acc2);
        each(C, dv, [&](int i, int e, int x, int y) { sdW[i * WIDE_LD + e] = acc[x][y] + egn[i] * acc2[x][y]; });
        __syncthreads();
        // ---- dOh = dO h^T; dKw = -dW h^T; dKt = W dh'^T; dP = dO W^T (lower)
        wide_mm(C, dk, dv, dO, [&](int e, int d) { return Hm(d, e); }, As, Bs, tid, acc);
        each(C, dk, [&](int i, int d, int x, int y) { sdOh[i * WIDE_LD + d] = acc[x][y]; });
        wide_mm(C, dk, dv, [&](int i, int e) { return sdW[i * WIDE_LD + e]; }, [&](int e, int d) { return Hm(d, e); },
                As, Bs, tid, acc);
        each(C, dk, [&](int i, int d, int x, int y) { sdKw[i * WIDE_LD + d] = add ? 0.f : -acc[x][y]; });
        wide_mm(C, dk, dv, [&](int i, int e) { return sW[i * WIDE_LD + e]; }, [&](int e, int d) { return dH(d, e); },
                As, Bs, tid, acc);
        each(C, dk, [&](int i, int d, int x, int y) { sdKt[i * WIDE_LD + d] = acc[x][y]; });
        wide_mm(C, C, dv, dO, [&](int e, int j) { return sW[j * WIDE_LD + e]; }, As, Bs, tid, acc);
        each(C, C, [&](int i, int j, int x, int y) { sdP[i * C + j] = i >= j ? acc[x][y] : 0.f; });
        __syncthreads();
        // ---- dV' = Tm^T dW, dK' = Tm^T dKw
        wide_mm(C, dv, C, [&](int i, int j) { return Tmm(j, i); }, [&](int j, int e) { return sdW[j * WIDE_LD + e]; },
                As, Bs, tid, acc);
        each(C, dv, [&](int i, int e, int x, int y) { sdVp[i * WIDE_LD + e] = acc[x][y]; });
        wide_mm(C, dk, C, [&](int i, int j) { return Tmm(j, i); }, [&](int j, int d) { return sdKw[j * WIDE_LD + d]; },
                As, Bs, tid, acc);
        each(C, dk, [&](int i, int d, int x, int y) { sdKp[i * WIDE_LD + d] = add ? 0.f : acc[x][y]; });
        __syncthreads();
        // ---- dL = -(dV' U^T + dK' Kw^T) = -dV' U^T + dK' (-Kw)^T, strictly lower
        wide_mm(C, C, dv, [&](int i, int e) { return sdVp[i * WIDE_LD + e]; }, [&](int e, int j) { return Um(j, e); },
                As, Bs, tid, acc);
        wide_mm(C, C, dk, [&](int i, int d) { return sdKp[i * WIDE_LD + d]; }, [&](int d, int j) { return NKm(j, d); },
                As, Bs, tid, acc2);
        each(C, C, [&](int i, int j, int x, int y) { sdL[i * C + j] = (!add && i > j) ? acc2[x][y] - acc[x][y] : 0.f; });
        __syncthreads();
        // dS + dS^T with dS = diag(beta)(dL o Gam), kept for the dK product
        for (int e = tid; e < C * C; e += NTHR) {
            const int i = e / C, j = e % C;
            sT[e] = bet[i] * sdL[i * C + j] * Gm(i, j) + bet[j] * sdL[j * C + i] * Gm(j, i);
        }
        __syncthreads();
        // ---- dQ = diag(e^gam) dO h^T + (dP o Gam) K
        wide_mm(C, dk, C, [&](int i, int j) { return sdP[i * C + j] * Gm(i, j); }, K, As, Bs, tid, acc);
        S *dq_out = (S *)a.dq + (row0 * H + h) * dk;
        each(C, dk, [&](int i, int d, int x, int y) {
            if (i < n) dq_out[i * sq + d] = from_f<BF>(eg[i] * sdOh[i * WIDE_LD + d] + acc[x][y]);
        });
        // ---- dK = (dP o Gam)^T Q + diag(e^{gam_n - gam}) dKt + diag(beta e^gam) dK' + (dS + dS^T) K
        wide_mm(C, dk, C, [&](int i, int j) { return sdP[j * C + i] * Gm(j, i); }, Q, As, Bs, tid, acc);
        wide_mm(C, dk, C, [&](int i, int j) { return sT[i * C + j]; }, K, As, Bs, tid, acc2);
        S *dk_out = (S *)a.dk + (row0 * H + h) * dk;
        if (!s.l2k) {
            each(C, dk, [&](int i, int d, int x, int y) {
                if (i < n)
                    dk_out[i * sq + d] = from_f<BF>(acc[x][y] + acc2[x][y] + egn[i] * sdKt[i * WIDE_LD + d] +
                                                    bet[i] * eg[i] * sdKp[i * WIDE_LD + d]);
            });
        } else {
            // gradient wrt the normalised keys into the free dKw scratch, then
            // back through the normalisation, dk = (dk_hat - k_hat (k_hat .
            // dk_hat)) / |k|, eight lanes per row
            each(C, dk, [&](int i, int d, int x, int y) {
                sdKw[i * WIDE_LD + d] = acc[x][y] + acc2[x][y] + egn[i] * sdKt[i * WIDE_LD + d] +
                                        bet[i] * eg[i] * sdKp[i * WIDE_LD + d];
            });
            __syncthreads();
            const int i = tid >> 3, gq = tid & 7;
            float dot = 0.f;
            for (int d = gq; d < dk; d += 8) dot += K(i, d) * sdKw[i * WIDE_LD + d];
#pragma unroll
            for (int off = 4; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
            if (i < n)
                for (int d = gq; d < dk; d += 8)
                    dk_out[i * sq + d] = from_f<BF>((sdKw[i * WIDE_LD + d] - K(i, d) * dot) * rk[i]);
        }
        // ---- dV = diag(beta) dV' (+ D_h dO with the skip term, whose dD_h
        // share, the sum of dO * V, goes to one slot per wave)
        S *dv_out = (S *)a.dv + (row0 * H + h) * dv;
        const float Dh = s.D ? s.D[h] : 0.f;
        float dsum = 0.f;
        for (int e = tid; e < n * dv; e += NTHR) {
            const int i = e / dv, f = e % dv;
            float x = bet[i] * sdVp[i * WIDE_LD + f];
            if (s.D) x += Dh * dO(i, f);
            if (a.dD_part) dsum += dO(i, f) * V(i, f);
            dv_out[i * sv + f] = from_f<BF>(x);
        }
        if (a.dD_part) {
            dsum = wave_sum(dsum);
            if (lane == 0) a.dD_part[cb * DD_SLOTS + wave] = dsum;
        }
        // ---- <h, dh'> in a fixed order
        float hd = 0.f;
        for (int e = tid; e < dk * dv; e += NTHR) hd += to_f(hc[e]) * to_f(dhc[e]);
        red[tid] = hd;
        __syncthreads();
        for (int w = NTHR / 2; w > 0; w >>= 1) {
            if (tid < w) red[tid] += red[tid + w];
            __syncthreads();
        }
        const float hds = red[0];
        // ---- dbeta and dgam per row. Every thread sums one eighth of a row
        // (row-contiguous reads of the scratch; the column sums of the C x C
        // term read along rows too), the eighths meet in LDS (As is free after
        // the last product) and wave 0 adds them in group order.
        {
            const int i = tid >> 3, gq = tid & 7;
            float qa = 0.f, qb = 0.f, qc = 0.f, qd = 0.f, qe = 0.f, qf = 0.f, qg = 0.f;
            for (int e = gq * 16; e < min(dv, gq * 16 + 16); ++e) qa += V(i, e) * sdVp[i * WIDE_LD + e];
            for (int d = gq * 16; d < min(dk, gq * 16 + 16); ++d) {
                qb += K(i, d) * sdKp[i * WIDE_LD + d];
                qc += Q(i, d) * sdOh[i * WIDE_LD + d];
                qd += K(i, d) * sdKt[i * WIDE_LD + d];
            }
            // Z = dP o P + diag(beta) (dL o (K K^T o Gam)): row sums minus column sums
            for (int j = gq * 8; j < gq * 8 + 8; ++j) {
                const float lk = sdL[i * C + j] * sKG[i * C + j];
                qe += lk;
                qf += sdP[i * C + j] * sP[i * C + j] + bet[i] * lk;
                qg += sdP[j * C + i] * sP[j * C + i] + bet[j] * sdL[j * C + i] * sKG[j * C + i];
            }
            float *pq = As; // [7][C][8]
            const float qv[7] = {qa, qb, qc, qd, qe, qf, qg};
#pragma unroll
            for (int u = 0; u < 7; ++u) pq[(u * C + i) * 8 + gq] = qv[u];
        }
        __syncthreads();
        if (wave == 0) {
            const int i = lane;
            const float *pq = As;
            float t[7];
#pragma unroll
            for (int u = 0; u < 7; ++u) {
                t[u] = 0.f;
                for (int gq = 0; gq < 8; ++gq) t[u] += pq[(u * C + i) * 8 + gq];
            }
            const float kdk = t[1];
            const float db = t[0] + eg[i] * kdk + t[4];
            float dgm = eg[i] * t[2] + bet[i] * eg[i] * kdk + t[5] - t[6];
            const float sj = egn[i] * t[3];
            const float stot = wave_sum(sj);
            dgm -= sj;
            if (i == C - 1) dgm += eglast * hds + stot;
            const float pre = wave_prefix(dgm);
            const float x = lane_value(pre, 63) - pre + dgm;
            const float dg = (float)A * x;
            float p = (lane < n) ? gch[lane] * dg : 0.f;
            if (lane < n) {
                const size_t gi = (row0 + lane) * H + h;
                // with logit inputs, through the sigmoid: d/dx = s (1 - s) d/ds
                const float gs = gch[lane], bs = bet[lane];
                a.dg[gi] = s.logits ? dg * gs * (1.f - gs) : dg;
                a.dbeta[gi] = s.logits ? db * bs * (1.f - bs) : db;
            }
            p = wave_sum(p);
            if (lane == 0) a.dA_part[cb] = p;
        }
        __syncthreads(); // LDS and scratch are reused by the next chunk
    }
}

// dA_log[h] = sum over (b, c) of part[b, h, c]: one workgroup per head,
// per-thread strided sums, then a fixed tree, so the order never changes.
__global__ __launch_bounds__(NTHR) void dA_reduce_kernel(const float *__restrict__ part,
                                                         float *__restrict__ dA, int B, int H, int NC) {
    __shared__ float red[NTHR];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int n = B * NC;
    float acc = 0.f;
    for (int i = tid; i < n; i += NTHR) {
        const int b = i / NC, c = i % NC;
        acc += part[((size_t)b * H + h) * NC + c];
    }
    red[tid] = acc;
    __syncthreads();
    for (int w = NTHR / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) dA[h] = red[0];
}

// --------------------------------------------------------------- launch

// value columns per workgroup of the reverse serial pass (16 for 128-wide
// heads: more workgroups share the chain, each carrying half the gradient);
// segmented launches take the forward's wider blocks
static int chain_vblock(bool, int D, bool segmented) {
    if (segmented) return fwd_vblock(D, true);
    return D == 64 ? 32 : 16;
}

template <bool BF, int D, int BV> static hipError_t chain_gen(const BwdChainArgs &a, hipStream_t st) {
    const int nvbe = a.NVB + (a.mode == 1 ? (a.s.dk + BV - 1) / BV : 0);
    const int nsl = a.mode == 1 ? a.nseg - 1 : a.nseg;
    const int grid = a.s.B * a.s.H * nsl * nvbe;
    if (vec_ok<BF>(a.s))
        hipLaunchKernelGGL((bwd_chain_kernel<BF, D, BV, true>), dim3(grid), dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<BF, D, BV, false>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

template <bool BF, int D> static hipError_t chain_inst(const BwdChainArgs &a, hipStream_t st) {
    constexpr int BV = D == 64 ? 32 : 16;
    const int grid = a.s.B * a.s.H * a.NVB;
    if (a.nseg < 1 || (a.mode == 1 && a.nseg < 2)) return hipErrorInvalidValue;
    if (a.nseg > 1) {
        const int bv = chain_vblock(BF, D, true);
        if (bv == 16) return chain_gen<BF, D, 16>(a, st);
        if constexpr (D >= 32)
            if (bv == 32) return chain_gen<BF, D, 32>(a, st);
        if constexpr (D >= 64)
            if (bv == 64) return chain_gen<BF, D, 64>(a, st);
        if constexpr (D >= 128)
            if (bv == 128) return chain_gen<BF, D, 128>(a, st);
        return hipErrorInvalidValue;
    }
    if constexpr (BF && D <= 64) {
        const dim3 block(64 * (BV / 16 + BWS_HELPERS));
        if (vec_ok<BF>(a.s))
            hipLaunchKernelGGL((bwd_chain_ws_kernel<D, BV, true>), dim3(grid), block, 0, st, a);
        else
            hipLaunchKernelGGL((bwd_chain_ws_kernel<D, BV, false>), dim3(grid), block, 0, st, a);
        return hipGetLastError();
    }
    if (vec_ok<BF>(a.s))
        hipLaunchKernelGGL((bwd_chain_kernel<BF, D, BV, true>), dim3(grid), dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<BF, D, BV, false>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_bwd_chain(const BwdChainArgs &a, bool bf16, int D, hipStream_t st) {
    if (chain_vblock(bf16, D, a.nseg > 1) * a.NVB < a.s.dv) return hipErrorInvalidValue;
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

// Blocks of a persistent kernel that are resident at once on the current
// device (compute units x blocks per unit), looked up once per device and
// kernel: KERNEL is the kernel itself, so every instance keeps its own cache.
template <auto KERNEL, int THREADS = NTHR> static hipError_t resident_blocks(int &out) {
    const auto kernel = KERNEL;
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int slot = dev & 63;
    int v = cache[slot].load(std::memory_order_relaxed);
    if (v <= 0) {
        int cus = 0, per = 0;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, THREADS, 0)) != hipSuccess) return e;
        v = cus * (per > 0 ? per : 1);
        cache[slot].store(v, std::memory_order_relaxed);
    }
    out = v;
    return hipSuccess;
}

// waves per local-gradient workgroup without the layer edges (with them: one
// skip-term slot per wave, DD_SLOTS). 16 waves (one tile per wave and
// product, at most 128 registers per lane) measured 0.44 ms against 0.32 for
// 8 at B8 H16 T4096 d56: 24 registers spilled, and no B operand is shared
#ifndef GDN_LOCAL_WAVES
#define GDN_LOCAL_WAVES 8
#endif

template <bool BF, int D, bool VEC, bool EDGE> static hipError_t local_launch(const BwdLocalArgs &a, hipStream_t st) {
    constexpr int NW = EDGE ? DD_SLOTS : GDN_LOCAL_WAVES;
    const int nch = a.s.B * a.s.H * a.s.NC;
    int grid = 0;
    const hipError_t e = resident_blocks<bwd_local_kernel<BF, D, VEC, EDGE, NW>, 64 * NW>(grid);
    if (e != hipSuccess) return e;
    grid = grid < nch ? grid : nch;
    hipLaunchKernelGGL((bwd_local_kernel<BF, D, VEC, EDGE, NW>), dim3(grid), dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

template <bool BF, int D> static hipError_t local_inst(const BwdLocalArgs &a, hipStream_t st) {
    const bool vec = vec_ok<BF>(a.s), edge = a.s.l2k || a.s.D || a.dD_part;
    if (edge) return vec ? local_launch<BF, D, true, true>(a, st) : local_launch<BF, D, false, true>(a, st);
    return vec ? local_launch<BF, D, true, false>(a, st) : local_launch<BF, D, false, false>(a, st);
}

template <bool BF> static hipError_t wide_inst(const BwdLocalArgs &a, hipStream_t st) {
    const int nch = a.s.B * a.s.H * a.s.NC;
    const int grid = nch < WIDE_GRID ? nch : WIDE_GRID;
    hipLaunchKernelGGL((bwd_local_wide_kernel<BF>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_bwd_local(const BwdLocalArgs &a, bool bf16, int D, hipStream_t st) {
    if (bf16) {
        switch (D) {
        case 32: return local_inst<true, 32>(a, st);
        case 64: return local_inst<true, 64>(a, st);
        case 128: return launch_bwd_local128(a, st);
        }
    } else {
        switch (D) {
        case 16: return local_inst<false, 16>(a, st);
        case 32:
        case 64: return a.wide ? wide_inst<false>(a, st) : hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

size_t bwd_wide_scratch_bytes(bool bf16, int D, int nchunks_total) {
    if (bf16 || D <= 16) return 0;
    const int grid = nchunks_total < WIDE_GRID ? nchunks_total : WIDE_GRID;
    return (size_t)grid * WIDE_SCRATCH * sizeof(float);
}

hipError_t launch_dA_reduce(const float *part, float *dA_log, int B, int H, int NC, hipStream_t st) {
    hipLaunchKernelGGL(dA_reduce_kernel, dim3(H), dim3(NTHR), 0, st, part, dA_log, B, H, NC);
    return hipGetLastError();
}

bool bwd_supported(bool bf16, int D) { return bf16 ? (D == 32 || D == 64 || D == 128) : (D == 16 || D == 32 || D == 64); }

int bwd_chain_vblock(bool bf16, int D, bool segmented) { return chain_vblock(bf16, D, segmented); }

} // namespace gdn
