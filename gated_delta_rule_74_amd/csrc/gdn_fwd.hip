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
    static constexpr int oK = 0;                                       // Ks [C][LDD]
    static constexpr int oTb = oK + C * LDD * (int)sizeof(S);         // Tb [C][LDC]
    static constexpr int oL = oTb + C * LDC * (int)sizeof(S);         // L^T, Tm, then V, fp32 [C][LDF]
    static constexpr int oX = oL + C * LDF * 4;                       // solve scratch
    static constexpr int oGam = oX + 4 * 16 * 17 * 4;                 // double[C]
    static constexpr int oBet = oGam + C * 8;                         // float[C]
    static constexpr int SIZE = oBet + C * 4;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
    static_assert(C * LDD * (int)sizeof(S) <= C * LDF * 4, "V fits the L^T / Tm area");
    // four workgroups per compute unit for bf16 heads up to 64 wide
    static_assert(!BF || D > 64 || 4 * SIZE <= 160 * 1024, "prep occupancy");
};

// X[row][0..D) *= sc(row) in place for the 16-byte pieces p0, p0 + np, ...
template <bool BF, int D, class F>
__device__ __forceinline__ void scale_rows(typename Op<BF>::S *X, int ld, F sc, int p0, int np) {
    using S = typename Op<BF>::S;
    constexpr int V = Op<BF>::VEC, NG = D / V;
    for (int it = p0; it < C * NG; it += np) {
        const int row = it / NG, c0 = (it % NG) * V;
        const float f = sc(row);
        union {
            uint4 u;
            S x[V];
        } pk;
        pk.u = *reinterpret_cast<const uint4 *>(X + row * ld + c0);
#pragma unroll
        for (int j = 0; j < V; ++j) pk.x[j] = from_f<BF>(to_f(pk.x[j]) * f);
        *reinterpret_cast<uint4 *>(X + row * ld + c0) = pk.u;
    }
}

// Store this wave's tiles of an [MT*16][NT*16] accumulator grid to a
// row-major global matrix (rows < nr, cols < nc), times `sign`.
template <bool BF, int MT, int NT>
__device__ __forceinline__ void store_global(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int nr,
                                             int nc, float sign, int wave, int lane) {
    for_tiles<MT, NT>(wave, lane, [&](int i, int e, int row, int col) {
        if (row < nr && col < nc) dst[(size_t)row * ld + col] = from_f<BF>(sign * acc[i][e]);
    });
}

// EDGE: keys normalised where they are loaded (compiled in only then)
template <bool BF, int D, bool VEC, bool EDGE>
__global__ __launch_bounds__(NTHR, 8) void fwd_prep_kernel(PrepArgs a) {
    using O = Op<BF>;
    using S = typename O::S;
    using L = PrepSmem<BF, D>;
    constexpr int LDD = L::LDD, LDC = L::LDC, DT = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    S *Ks = (S *)(smem + L::oK);
    S *Tb = (S *)(smem + L::oTb);
    float *Lm = (float *)(smem + L::oL);
    float *Tm = Lm;
    S *Vs = (S *)Lm; // V is staged once Tm has been stored out
    float *xs = (float *)(smem + L::oX);
    double *gam2 = (double *)(smem + L::oGam);
    float *bet = (float *)(smem + L::oBet);

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // heads fastest: the rows of all heads of one token are adjacent in
    // memory, so workgroups that share cache lines run together on one XCD
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid % s.H, c = a.c0 + (lid / s.H) % a.ncs, b = lid / (s.H * a.ncs);
    const int bh = b * s.H + h;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv;
    const int t0 = c * C, n = min(C, T - t0);
    const size_t row0 = (size_t)b * T + t0;

    // wave 0 requests the gates first, so the decay scan waits for them only
    // while the key and value rows are still in flight
    float gr = 0.f, br = 0.f, alg = 0.f;
    if (wave == 0) {
        gr = load_row_scalar(s.g + row0 * H + h, H, lane, n);
        br = load_row_scalar(s.beta + row0 * H + h, H, lane, n);
        alg = s.A_log[h];
    }
    ChunkFrag<BF, D> fk, fv;
    fk.template fetch<VEC>((const S *)s.k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
    fv.template fetch<VEC>((const S *)s.v + (row0 * H + h) * dv, (size_t)H * dv, n, dv, tid);
    if (wave == 0) {
        // first use of the gates here, after the row loads are issued
        asm volatile("" : "+v"(gr), "+v"(br), "+v"(alg));
        const float g = lane < n ? gate_of(gr, s.logits) : 0.f, be = lane < n ? gate_of(br, s.logits) : 0.f;
        const Decay dc = decay_lane(g, -exp((double)alg) * LOG2E, lane);
        gam2[lane] = dc.gam2;
        if (a.gam) a.gam[((size_t)bh * s.NC + c) * C + lane] = (float)dc.gam2;
        bet[lane] = be;
    }
    if constexpr (EDGE) {
        if (s.l2k) fk.normalize_rows(nullptr, tid);
    }
    fk.stash(Ks, LDD, tid);
    __syncthreads();

    // U = Tm (diag(beta) V) and -Kw = -Tm (diag(beta e^gam) K): the row
    // scales go onto V and K in LDS (K after K K^T has read it; V, kept in
    // registers until then, into the Tm area once Tm is stored out), so a
    // single operand copy Tb of Tm serves both products
    if (!s.additive) {
        f32x4 sk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sk[i] = zero4();
        gemm<BF, 4, 4, D>(Ks, LDD, Ks, LDD, sk, wave, lane);
        for_tiles<4, 4>(wave, lane, [&](int i, int e, int row, int col) {
            Lm[col * LDF + row] = (row > col) ? bet[row] * sk[i][e] * gamma_ij(gam2, row, col) : 0.f; // L^T
        });
        __syncthreads(); // L complete, K K^T done
        // waves 4..7 are idle during the diagonal solve: rows of K times
        // beta e^gam (the same e^gam the decay scan forms)
        if (wave >= 4)
            scale_rows<BF, D>(Ks, LDD, [&](int row) { return bet[row] * exp2_fast((float)gam2[row]); },
                              tid - 4 * 64, NTHR - 4 * 64);
        tri_inverse<BF>(Lm, xs, wave, lane, Tb, LDC);
    } else {
        for (int e = tid; e < C * C; e += NTHR) {
            const int row = e / C, col = e % C;
            Tb[row * LDC + col] = from_f<BF>(row == col ? 1.f : 0.f);
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
    __syncthreads(); // Tm read out: V (times beta) takes its place
    fv.stash_scaled(Vs, LDD, tid, bet[lane]);
    __syncthreads();
    f32x4 accU[Tiles<4, DT>::PW], accN[Tiles<4, DT>::PW];
#pragma unroll
    for (int i = 0; i < Tiles<4, DT>::PW; ++i) accU[i] = accN[i] = zero4();
    gemm<BF, 4, DT, C, false, true>(Tb, LDC, Vs, LDD, accU, wave, lane);
    if (!s.additive) gemm<BF, 4, DT, C, false, true>(Tb, LDC, Ks, LDD, accN, wave, lane);
    S *Ug = (S *)a.U + cbase * C * dv, *Ng = (S *)a.NK + cbase * C * dk;
    if constexpr (BF && 2 * C * D * (int)sizeof(S) <= C * LDF * 4) {
        // U and NK leave through the Tm area as 16-byte pieces of their
        // contiguous [64][d] blocks, once every wave has stored Tm out
        __syncthreads();
        S *Us = (S *)Lm, *Ns = Us + C * D;
#pragma unroll
        for (int i = 0; i < Tiles<4, DT>::PW; ++i) accN[i] = -accN[i];
        store_N<BF, 4, DT>(accU, Us, D, wave, lane);
        store_N<BF, 4, DT>(accN, Ns, D, wave, lane);
        __syncthreads();
        constexpr int V = O::VEC, NG = D / V;
        if (VEC) {
            for (int it = tid; it < C * NG; it += NTHR) {
                const int j = it / NG, c0 = (it % NG) * V;
                if (c0 < dv) *reinterpret_cast<uint4 *>(Ug + (size_t)j * dv + c0) = *reinterpret_cast<const uint4 *>(Us + j * D + c0);
                if (!s.additive && c0 < dk)
                    *reinterpret_cast<uint4 *>(Ng + (size_t)j * dk + c0) = *reinterpret_cast<const uint4 *>(Ns + j * D + c0);
            }
        } else {
            for (int it = tid; it < C * D; it += NTHR) {
                const int j = it / D, col = it % D;
                if (col < dv) Ug[(size_t)j * dv + col] = Us[j * D + col];
                if (!s.additive && col < dk) Ng[(size_t)j * dk + col] = Ns[j * D + col];
            }
        }
    } else {
        store_global<BF, 4, DT>(accU, Ug, dv, C, dv, 1.f, wave, lane);
        if (!s.additive) store_global<BF, 4, DT>(accN, Ng, dk, C, dk, -1.f, wave, lane);
    }
}

// ----------------------------------------------------------------- chain

// x + c y on eight packed bf16 values (fp32 arithmetic, one rounding)
__device__ __forceinline__ uint4 add_scaled_bf16x8(uint4 x, uint4 y, float c) {
    auto two = [&](uint32_t a, uint32_t b) {
        return f2bf2(bf2f((u16)(a & 0xFFFF)) + c * bf2f((u16)(b & 0xFFFF)), bf2f((u16)(a >> 16)) + c * bf2f((u16)(b >> 16)));
    };
    return uint4{two(x.x, y.x), two(x.y, y.y), two(x.z, y.z), two(x.w, y.w)};
}

// x + c y on one 16-byte vector of the operand type
template <bool BF> __device__ __forceinline__ uint4 add_scaled_vec(uint4 x, uint4 y, float c) {
    if constexpr (BF) {
        return add_scaled_bf16x8(x, y, c);
    } else {
        const float4 a = __builtin_bit_cast(float4, x), b = __builtin_bit_cast(float4, y);
        return __builtin_bit_cast(uint4, float4{a.x + c * b.x, a.y + c * b.y, a.z + c * b.z, a.w + c * b.w});
    }
}

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
    // O of a chunk [C][LDV] is staged over WT and WTd, which are free from the
    // end of one chunk's products to the W product of the next
    static_assert(C * LDV <= 2 * BV * LDC, "O staging fits the W area");
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
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv, NC = s.NC;
    // workgroup -> (batch-head, segment, value block); with maps the first
    // NVBM blocks carry dk identity columns (the linear part of the map)
    const bool maps = a.mode == 1;
    const int NVBM = maps ? (dk + BV - 1) / BV : 0;
    const int nvbe = a.NVB + NVBM, nsl = maps ? a.nseg - 1 : a.nseg;
    const int vbe = lid % nvbe, seg = (lid / nvbe) % nsl, bh = lid / (nvbe * nsl);
    const bool mblk = vbe < NVBM;
    const int v0 = (mblk ? vbe : vbe - NVBM) * BV, nvc = min(BV, (mblk ? dk : dv) - v0);
    const int c_lo = (int)((long long)seg * NC / a.nseg), c_hi = (int)((long long)(seg + 1) * NC / a.nseg);
    const int b = bh / s.H, h = bh % s.H;
    const double A2 = -exp((double)s.A_log[h]) * LOG2E;
    const S *q = (const S *)s.q;
    const S *k = (const S *)s.k;
    const S *U = (const S *)a.U;
    const S *NK = (const S *)a.NK;
    S *o = maps ? nullptr : (S *)a.o;
    S *cs = maps ? nullptr : (S *)a.cs;

    // state h[D][BV] (fp32) lives in the accumulators of the h-update product:
    // the segment's start state, identity columns (maps, linear part) or zero
    const float *hin = maps ? nullptr
                            : (seg == 0 ? (a.h_in ? a.h_in + (size_t)bh * dk * dv : nullptr)
                                        : a.seg_h + ((size_t)bh * a.nseg + seg) * dk * dv);
    f32x4 accH[Tiles<DT, VT>::PW];
    for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
        const bool in = row < dk && col < nvc;
        accH[i][e] = mblk ? ((in && row == v0 + col) ? 1.f : 0.f)
                          : ((hin && in) ? hin[(size_t)row * dv + v0 + col] : 0.f);
    });
    store_T<BF, DT, VT>(accH, hTs, LDD, wave, lane);

    // inputs of the next chunk are fetched into registers during this one
    ChunkFrag<BF, D> fk, fq, fn;
    ChunkFrag<BF, BV> fu;
    fu.ok = 0; // identity columns take U as zero: never fetched, stashed as zeros
    float pg = 0.f;
    auto fetch = [&](int c) {
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = (size_t)b * T + t0, cb = (size_t)bh * s.NC + c;
        fk.template fetch<VEC>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        if (o) fq.template fetch<VEC>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, tid);
        if (!s.additive) fn.template fetch<VEC>(NK + cb * C * dk, (size_t)dk, n, dk, tid);
        if (!mblk) fu.template fetch<VEC>(U + cb * C * dv + v0, (size_t)dv, n, nvc, tid);
        pg = gate_of(load_row_scalar(s.g + row0 * H + h, H, lane, n), s.logits);
    };
    // O of a chunk is written out during the next chunk, after that chunk's
    // inputs have arrived: stores are issued only between consuming one
    // prefetch and issuing the next, so waiting for the inputs never waits
    // for a store to complete. With 16-byte rows (VEC) O goes through LDS:
    // staged in tile layout once the chunk's products are done, then stored
    // as row pieces after the next chunk's first barrier; otherwise it is
    // held in registers and stored element by element.
    f32x4 accO[Tiles<4, VT>::PW];
    S *Os = WT; // [C][LDV]
    const float Dh = s.D ? s.D[h] : 0.f; // skip term o_t += D_h v_t
    auto store_o = [&](int c) {
        const int n = min(C, T - c * C);
        const size_t off = (((size_t)b * T + c * C) * H + h) * dv + v0;
        S *orow = o + off;
        const S *vrow = (const S *)s.v + off;
        if constexpr (VEC) {
            constexpr int V = O::VEC, NG = BV / V;
            for (int it = tid; it < C * NG; it += NTHR) {
                const int j = it / NG, c0 = (it % NG) * V;
                if (j >= n || c0 >= nvc) continue;
                const size_t x = (size_t)j * H * dv + c0;
                uint4 val = *reinterpret_cast<const uint4 *>(Os + j * LDV + c0);
                if (s.D) val = add_scaled_vec<BF>(val, *reinterpret_cast<const uint4 *>(vrow + x), Dh);
                *reinterpret_cast<uint4 *>(orow + x) = val;
            }
        } else {
            for_tiles<4, VT>(wave, lane, [&](int i, int e, int row, int col) {
                if (row < n && col < nvc) {
                    const size_t x = (size_t)row * H * dv + col;
                    orow[x] = from_f<BF>(s.D ? accO[i][e] + Dh * to_f(vrow[x]) : accO[i][e]);
                }
            });
        }
    };
    fetch(c_lo);

    for (int c = c_lo; c < c_hi; ++c) {
        const int t0 = c * C, n = min(C, T - t0);
        wait_vmem();
        if (wave == 0) {
            const Decay dc = decay_lane(lane < n ? pg : 0.f, A2, lane);
            gam2[lane] = dc.gam2;
            eg[lane] = dc.eg;
            egn[lane] = dc.egn;
            if (lane == 0) misc[0] = dc.eglast;
        }
        if (s.l2k) fk.normalize_rows(nullptr, tid);
        fk.stash(Ks, LDD, tid);
        if (o) fq.stash(Qs, LDD, tid);
        if (!s.additive) fn.stash(NKs, LDD, tid);
        fu.stash(Us, LDV, tid);
        if (!VEC && o && c > c_lo) store_o(c - 1);
        if (cs) {
            // chunk-start state, transposed [dv][dk]: a lane's 4 consecutive
            // key rows of one value column are contiguous (dk % 4 == 0 with
            // VEC): one 8-byte (bf16) or 16-byte (fp32) store
            if constexpr (VEC) {
                using TL = Tiles<DT, VT>;
                const int r = lane & 15, kq = lane >> 4;
#pragma unroll
                for (int i = 0; i < TL::PW; ++i) {
                    const int t = wave + NWAVE * i;
                    if (TL::N % NWAVE != 0 && t >= TL::N) break;
                    const int row = (t / VT) * 16 + 4 * kq, col = (t % VT) * 16 + r;
                    if (row < dk && col < nvc) {
                        S *dst = cs + (((size_t)bh * s.NC + c) * dv + v0 + col) * dk + row;
                        if constexpr (BF)
                            *reinterpret_cast<short4_t *>(dst) = pack4(accH[i]);
                        else
                            *reinterpret_cast<f32x4 *>(dst) = accH[i];
                    }
                }
            } else {
                for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
                    if (row < dk && col < nvc)
                        cs[(((size_t)bh * s.NC + c) * dv + v0 + col) * dk + row] = from_f<BF>(accH[i][e]);
                });
            }
        }
        if (c + 1 < c_hi) fetch(c + 1);
        __syncthreads();
        if (VEC && o && c > c_lo) {
            // O rows of the previous chunk out of the W area, which this
            // chunk's W product overwrites after the next barrier
            store_o(c - 1);
            __syncthreads();
        }

        // P = (Q K^T) o Gam (independent of the state; only the outputs need it)
        if (o) {
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
        if (VEC && o) store_N<BF, 4, VT>(accO, Os, LDV, wave, lane); // O staged for the next chunk
    }
    if (o && c_hi > c_lo) {
        if (VEC) __syncthreads(); // staged O rows complete
        store_o(c_hi - 1);
    }
    if (maps) {
        // [M | R] of this segment: identity blocks fill the M columns
        float *dst = a.maps + ((size_t)bh * (a.nseg - 1) + seg) * dk * (dk + dv) + (mblk ? v0 : dk + v0);
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) dst[(size_t)row * (dk + dv) + col] = accH[i][e];
        });
    } else if (a.hT && seg == a.nseg - 1) {
        for_tiles<DT, VT>(wave, lane, [&](int i, int e, int row, int col) {
            if (row < dk && col < nvc) a.hT[((size_t)bh * dk + row) * dv + v0 + col] = accH[i][e];
        });
    }
}

// Start states of the segments of a segmented pass, one workgroup per
// (batch-head, 16 value columns): x_0 = h0, x_{s+1} = M_s x_s + R_s with the
// maps [M | R] of the segments (reverse: from the last segment down), fp32,
// sums over the key index in order. Columns are independent, so each
// workgroup carries its own 16. Each step stages M (and the workgroup's R
// columns) in LDS from registers loaded two steps earlier.
__global__ __launch_bounds__(512) void range_scan_kernel(ScanArgs a) {
    constexpr int DK = 128, LDM = DK + 4, NT = 512, RPT = DK / (NT / 16); // rows per thread
    __shared__ __attribute__((aligned(16))) float Ms[DK * LDM];
    __shared__ float Rs[DK * 16];
    __shared__ __attribute__((aligned(16))) float hc[DK * 16];
    const int nvb = (a.dv + 15) / 16;
    const int bh = blockIdx.x / nvb, cb = blockIdx.x % nvb;
    const int dk = a.dk, dv = a.dv, ld = dk + dv, dk4 = (dk + 3) & ~3;
    const int tid = threadIdx.x, j = tid % 16, i0 = tid / 16, col = 16 * cb + j;
    const bool cin = col < dv;
    // x [k][16] for k < dk4 (rows dk .. dk4-1 stay zero), M rows zero-padded to dk4
    for (int i = i0; i < DK; i += NT / 16)
        hc[i * 16 + j] = (a.h0 && cin && i < dk) ? a.h0[((size_t)bh * dk + i) * dv + col] : 0.f;
    for (int e = tid; e < DK * LDM; e += NT) Ms[e] = 0.f;
    __syncthreads();
    // map of step it: forward the map of segment it, reverse that of segment
    // nseg-1-it (stored at index nseg-2-it)
    auto map_of = [&](int it) {
        return a.maps + ((size_t)bh * (a.nseg - 1) + (a.reverse ? a.nseg - 2 - it : it)) * dk * ld;
    };
    // M rows go through registers as 16-byte pieces when the row stride
    // allows, requested two steps ahead (two register sets taking turns), so
    // the serial chain of segments does not wait for memory
    const bool vec = (ld & 3) == 0 && (dk & 3) == 0;
    constexpr int PM = DK * (DK / 4) / NT; // 16-byte pieces of M per thread
    float4 pmA[PM], pmB[PM];
    float prA[RPT], prB[RPT];
    auto load_map = [&](int it, auto &pm, auto &pr) {
        const float *M = map_of(it);
#pragma unroll
        for (int r = 0; r < PM; ++r) {
            const int e = tid + NT * r, i = e / (dk / 4), k4 = (e % (dk / 4)) * 4;
            pm[r] = i < dk ? *reinterpret_cast<const float4 *>(M + (size_t)i * ld + k4) : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = i0 + (NT / 16) * r;
            pr[r] = (cin && i < dk) ? M[(size_t)i * ld + dk + col] : 0.f;
        }
    };
    // one step of the scan with the map staged from (pm, pr); returns true
    // after the last segment's start state is written
    auto step = [&](int it, auto &pm, auto &pr) {
        const int sg = a.reverse ? a.nseg - 1 - it : it;
        float *out = a.seg_h + ((size_t)bh * a.nseg + sg) * dk * dv;
        for (int i = i0; i < dk; i += NT / 16)
            if (cin) out[(size_t)i * dv + col] = hc[i * 16 + j];
        if (it == a.nseg - 1) return true;
        if (vec) {
#pragma unroll
            for (int r = 0; r < PM; ++r) {
                const int e = tid + NT * r, i = e / (dk / 4), k4 = (e % (dk / 4)) * 4;
                if (i < dk) *reinterpret_cast<float4 *>(Ms + i * LDM + k4) = pm[r];
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r) Rs[(i0 + (NT / 16) * r) * 16 + j] = pr[r];
        } else {
            const float *M = map_of(it);
            for (int e = tid; e < dk * dk; e += NT) Ms[(e / dk) * LDM + e % dk] = M[(size_t)(e / dk) * ld + e % dk];
            for (int i = i0; i < dk; i += NT / 16) Rs[i * 16 + j] = cin ? M[(size_t)i * ld + dk + col] : 0.f;
        }
        __syncthreads();
        if (vec && it + 2 < a.nseg - 1) load_map(it + 2, pm, pr);
        // rows i0 + 32 r of the new x: every 16-byte read of a row of M
        // serves four key steps, every read of x four rows
        float nx[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) nx[r] = 0.f;
        for (int kk = 0; kk < dk4; kk += 4) {
            const float x0 = hc[kk * 16 + j], x1 = hc[(kk + 1) * 16 + j];
            const float x2 = hc[(kk + 2) * 16 + j], x3 = hc[(kk + 3) * 16 + j];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const float4 m = *reinterpret_cast<const float4 *>(Ms + (i0 + (NT / 16) * r) * LDM + kk);
                nx[r] += m.x * x0;
                nx[r] += m.y * x1;
                nx[r] += m.z * x2;
                nx[r] += m.w * x3;
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = i0 + (NT / 16) * r;
            if (i < dk) hc[i * 16 + j] = Rs[i * 16 + j] + nx[r];
        }
        __syncthreads();
        return false;
    };
    if (vec && a.nseg > 1) load_map(0, pmA, prA);
    if (vec && a.nseg > 2) load_map(1, pmB, prB);
    for (int it = 0;; it += 2) {
        if (step(it, pmA, prA)) break;
        if (step(it + 1, pmB, prB)) break;
    }
}

hipError_t launch_fwd_scan(const ScanArgs &a, hipStream_t st) {
    if (a.dk > 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(range_scan_kernel, dim3(a.BH * ((a.dv + 15) / 16)), dim3(512), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------- wave-specialised chain
//
// bf16 path for head dims up to 64. One workgroup per (batch, head, block
// of BV value columns): the state's value columns evolve independently, so
// a block needs only its own columns of U, h, W and O (every block loads Q,
// K and -Kw and forms P). Waves 0..BV/16-1 ("chain waves") each carry 16
// value columns of the state h [D][16] in MFMA accumulators and run only
// the recurrence
//   W = U + NK h,   h <- e^{gam_n} h + K^T diag(e^{gam_n - gam}) W.
// With 16x16x16 products an accumulator tile (rows 4*(lane/16)+e, column
// lane%16) is already the B operand of a product over the same rows, so W
// and h stay in the wave's registers on the serial path: no barrier and no
// LDS round trip between the two products. The eight "helper" waves that
// follow split the rest: they stage the next chunk's inputs into LDS, form
// P = (Q K^T) o Gam and diag(e^gam) Q h for the current chunk, and finish
// O = ... + P W one chunk behind the chain (W arrives through LDS). Helper w
// owns chunk rows 16*(w%4).. and half of the block's value columns (and
// half of P's column blocks). One barrier per
// chunk hands the double-buffered LDS over. Helpers 0..3 issue every global
// load and helpers 4..7 store O (their own rows, and the rows helpers 0..3
// leave in LDS one chunk earlier), so the wait of a loading wave for its
// prefetch never includes stores; the chain waves store each chunk-start
// state from their registers.
//
// Chunk-start states go out transposed, [dv][dk] per chunk.

constexpr int WS_HELPERS = 8;

template <int D, int BV> struct WsSmem {
    static constexpr int VH = BV / 32; // value blocks per helper
    static constexpr int LDD = D + 8;  // token rows [C][LDD]; h^T [BV][LDD]
    static constexpr int LDC = C + 8;  // W^T [BV][LDC]
    static constexpr int LDP = 16 + 8; // P^T of one 16-row block [C][LDP]
    static constexpr int LDO = 16 * VH + 8;
    // 64-column blocks: each helper's O block (16 rows x 32 columns) is kept
    // transposed, [32][LDOT], in the same bytes as [16][LDO]
    static constexpr bool OT = VH == 2;
    static constexpr int LDOT = 16 + 4;
    static_assert(!OT || 32 * LDOT == 16 * LDO, "transposed O block fits its buffer");
    static constexpr int szCD = C * LDD * 2;
    static constexpr int szStage = 4 * szCD; // Q, K, -Kw, U
    static constexpr int szHX = BV * LDD * 2;
    static constexpr int szWX = BV * LDC * 2;
    static constexpr int szP = C * LDP * 2;
    static constexpr int szO = 16 * LDO * 2;
    static constexpr int szDec = 3 * C * 4 + 16; // gam (log2), e^gam, e^{gam_n-gam}, e^{gam_n}
    static constexpr int oStage = 0;
    static constexpr int oHX = oStage + 2 * szStage;
    static constexpr int oWX = oHX + 2 * szHX;
    static constexpr int oP = oWX + 2 * szWX;
    static constexpr int oO = oP + 2 * 4 * szP;
    static constexpr int oOA = oO + WS_HELPERS * szO; // O rows of helpers 0..3, two chunks
    static constexpr int oDec = oOA + 2 * 4 * szO;
    static constexpr int SIZE = oDec + 2 * szDec;
    static_assert(SIZE <= 160 * 1024, "LDS budget");
};

// EDGE: the layer edges (key normalisation, skip term) are compiled in; the
// plain instantiation carries none of their code, so its schedule is that of
// the recurrence alone
template <int D, int BV, bool VEC, bool EDGE>
__global__ __launch_bounds__(64 * (BV / 16 + WS_HELPERS)) void fwd_chain_ws_kernel(FwdChainArgs a) {
    constexpr int DT = D / 16, KS = D / 32, VT = BV / 16;
    constexpr int NLT = 64 * 4; // loading helper threads (helpers 0..3)
    using L = WsSmem<D, BV>;
    constexpr int LDD = L::LDD, LDC = L::LDC, LDP = L::LDP, LDO = L::LDO, VH = L::VH, LDOT = L::LDOT;
    constexpr bool OT = L::OT;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::SIZE];
    auto stage = [&](int st, int m) { return (u16 *)(smem + L::oStage + st * L::szStage + m * L::szCD); };
    auto hx = [&](int i) { return (u16 *)(smem + L::oHX + i * L::szHX); };
    auto wx = [&](int i) { return (u16 *)(smem + L::oWX + i * L::szWX); };
    auto pbuf = [&](int i, int ib) { return (u16 *)(smem + L::oP + (i * 4 + ib) * L::szP); };
    auto obuf = [&](int hw) { return (u16 *)(smem + L::oO + hw * L::szO); };
    auto obufA = [&](int c, int i) { return (u16 *)(smem + L::oOA + ((c & 1) * 4 + i) * L::szO); };
    auto gam_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec); };
    auto eg_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec + C * 4); };
    auto egn_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec + C * 8); };
    auto egl_of = [&](int i) { return (float *)(smem + L::oDec + i * L::szDec + C * 12); };

    const SeqArgs &s = a.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, r = lane & 15;
    // workgroup -> (batch-head, value block): the value blocks of one head
    // are neighbours, so they run on one XCD and share its cache for the
    // rows every block loads (q, k, -Kw)
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = lid / a.NVB, V0 = (lid % a.NVB) * BV;
    const int b = bh / s.H, h = bh % s.H;
    const int T = s.T, H = s.H, dk = s.dk, dv = s.dv, NC = s.NC, c0 = a.c0, c1 = a.c1;
    const int bcols = min(BV, dv - V0); // value columns of this block
    const bool chain = wave < VT;
    const bool add = s.additive != 0;

    // ---- chain-wave state: value columns V0 + v0 .. + 15 (block-local v0)
    const int v0 = 16 * wave;
    f32x4 hacc[DT];
    short4_t hb[DT];
    // ---- helper-wave state: rows 16*ib.., value blocks vb0..vb0+VH-1
    const int hw = wave - VT, htid = tid - 64 * VT;
    const int ib = hw & 3, half = hw >> 2, vb0 = half * VH;
    const bool loader = !chain && hw < 4;
    ChunkFrag<true, D, C, NLT> fq, fk, fn;
    ChunkFrag<true, BV, C, NLT> fu;
    float pg = 0.f;
    f32x4 accO[VH];
    const u16 *q = (const u16 *)s.q, *k = (const u16 *)s.k;
    const u16 *U = (const u16 *)a.U, *NK = (const u16 *)a.NK;
    u16 *o = (u16 *)a.o, *cs = (u16 *)a.cs;

    auto fetch = [&](int c) {
        const int n = min(C, T - c * C);
        const size_t row0 = (size_t)b * T + c * C, cb = (size_t)bh * NC + c;
        fq.template fetch<VEC>(q + (row0 * H + h) * dk, (size_t)H * dk, n, dk, htid);
        fk.template fetch<VEC>(k + (row0 * H + h) * dk, (size_t)H * dk, n, dk, htid);
        if (!add) fn.template fetch<VEC>(NK + cb * C * dk, (size_t)dk, n, dk, htid);
        fu.template fetch<VEC>(U + cb * C * dv + V0, (size_t)dv, n, bcols, htid);
        pg = a.gam[cb * C + lane];
    };
    auto stash = [&](int c) {
        const int st = c & 1;
        wait_vmem();
        fq.stash(stage(st, 0), LDD, htid);
        if constexpr (EDGE) {
            if (s.l2k) fk.normalize_rows(nullptr, htid);
        }
        fk.stash(stage(st, 1), LDD, htid);
        if (!add) fn.stash(stage(st, 2), LDD, htid);
        fu.stash(stage(st, 3), LDD, htid);
        if (hw == 0) {
            const float last = __shfl(pg, 63, 64);
            gam_of(st)[lane] = pg;
            eg_of(st)[lane] = exp2_fast(pg);
            egn_of(st)[lane] = exp2_fast(last - pg);
            if (lane == 0) egl_of(st)[0] = exp2_fast(last);
        }
    };

    // rows 16*bi.. and value blocks vb..vb+VH-1 of O of chunk cc, from LDS
    // (16 rows of LDO elements) to global
    // (with EDGE, the skip term o_t += D_h v_t is added to the rounded O rows
    // as they leave)
    auto store_o = [&](int cc, int bi, int vb, const u16 *Os) {
        const int n = min(C, T - cc * C);
        const int nr = min(16, n - 16 * bi), vlo = V0 + 16 * vb, nvc = min(16 * VH, dv - vlo);
        u16 *orow = o + (((size_t)b * T + cc * C + 16 * bi) * H + h) * dv + vlo;
        if constexpr (!EDGE) {
            if (OT && VEC) {
                // one transposing read: row r, columns 8g .. 8g + 7
                const int i = lane & 15, v = 8 * (lane >> 4);
                const bf16x8 x = operand_tr(Os, LDOT, 0, 0, lane);
                if (i < nr && v < nvc) *(bf16x8 *)(orow + (size_t)i * H * dv + v) = x;
            } else if (VEC) {
                for (int it = lane; it < 16 * 2 * VH; it += 64) {
                    const int i = it / (2 * VH), v = (it % (2 * VH)) * 8;
                    if (i < nr && v < nvc) *(uint4 *)(orow + (size_t)i * H * dv + v) = *(const uint4 *)(Os + i * LDO + v);
                }
            } else {
                for (int it = lane; it < 16 * 16 * VH; it += 64) {
                    const int i = it / (16 * VH), v = it % (16 * VH);
                    if (i < nr && v < nvc) orow[(size_t)i * H * dv + v] = OT ? Os[v * LDOT + i] : Os[i * LDO + v];
                }
            }
        } else {
            const u16 *vrow = (const u16 *)s.v + (orow - o);
            const float Dh = s.D ? s.D[h] : 0.f;
            if (VEC) {
                for (int it = lane; it < 16 * 2 * VH; it += 64) {
                    const int i = OT ? (lane & 15) : it / (2 * VH), v = OT ? 8 * (lane >> 4) : (it % (2 * VH)) * 8;
                    uint4 x;
                    if (OT)
                        x = __builtin_bit_cast(uint4, operand_tr(Os, LDOT, 0, 0, lane));
                    else
                        x = *(const uint4 *)(Os + i * LDO + v);
                    if (i < nr && v < nvc) {
                        if (s.D) x = add_scaled_bf16x8(x, *(const uint4 *)(vrow + (size_t)i * H * dv + v), Dh);
                        *(uint4 *)(orow + (size_t)i * H * dv + v) = x;
                    }
                }
            } else {
                for (int it = lane; it < 16 * 16 * VH; it += 64) {
                    const int i = it / (16 * VH), v = it % (16 * VH);
                    if (i < nr && v < nvc) {
                        const size_t x = (size_t)i * H * dv + v;
                        u16 val = OT ? Os[v * LDOT + i] : Os[i * LDO + v];
                        if (s.D) val = f2bf(bf2f(val) + Dh * bf2f(vrow[x]));
                        orow[x] = val;
                    }
                }
            }
        }
    };

    // ---- prologue: initial state (chain) and chunk 0 in LDS (helpers)
    if (chain) {
#pragma unroll
        for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * kb + 4 * g + e, v = V0 + v0 + r;
                hacc[kb][e] = (a.h_in && d < dk && v < dv) ? a.h_in[((size_t)bh * dk + d) * dv + v] : 0.f;
            }
            hb[kb] = pack4(hacc[kb]);
            *(short4_t *)(hx(c0 & 1) + (v0 + r) * LDD + 16 * kb + 4 * g) = hb[kb];
        }
    } else if (loader) {
        fetch(c0);
        stash(c0);
        if (c1 - c0 > 1) fetch(c0 + 1);
    }
    __syncthreads();

    for (int c = c0; c <= c1; ++c) {
        if (chain) {
            if (c < c1) {
                const int st = c & 1;
                const u16 *Ks = stage(st, 1), *NKs = stage(st, 2), *Us = stage(st, 3);
                // chunk-start state h_c out from the registers, transposed
                // [dv][dk]: 4 consecutive key rows of one value column per
                // lane (one 8-byte store when dk % 8 == 0, else per element)
                if (cs) {
                    u16 *dst = cs + ((size_t)bh * NC + c) * dv * dk;
                    const int v = V0 + v0 + r;
#pragma unroll
                    for (int kb = 0; kb < DT; ++kb) {
                        const int d = 16 * kb + 4 * g;
                        if (v < dv && d < dk) {
                            if (VEC) {
                                *(short4_t *)(dst + (size_t)v * dk + d) = hb[kb];
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (d + e < dk) dst[(size_t)v * dk + d + e] = (u16)hb[kb][e];
                            }
                        }
                    }
                }
                const float *egn = egn_of(st);
                const float el = egl_of(st)[0];
                // W = U + (-Kw) h
                f32x4 w[4];
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const short4_t u4 = operand_tr4(Us, LDD, 16 * tm, v0, lane);
                    const uint2 uu = __builtin_bit_cast(uint2, u4);
                    w[tm][0] = bf2f((u16)(uu.x & 0xFFFF));
                    w[tm][1] = bf2f((u16)(uu.x >> 16));
                    w[tm][2] = bf2f((u16)(uu.y & 0xFFFF));
                    w[tm][3] = bf2f((u16)(uu.y >> 16));
                }
                if (!add) {
#pragma unroll
                    for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
                        for (int tm = 0; tm < 4; ++tm) {
                            const short4_t an = *(const short4_t *)(NKs + (16 * tm + r) * LDD + 16 * kb + 4 * g);
                            w[tm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(an, hb[kb], w[tm], 0, 0, 0);
                        }
                    }
                }
                // W out for the helpers; W diag(e^{gam_n - gam}) stays here
                short4_t wb[4];
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    *(short4_t *)(wx(st) + (v0 + r) * LDC + 16 * tm + 4 * g) = pack4(w[tm]);
                    const float4 sc = *(const float4 *)(egn + 16 * tm + 4 * g);
                    wb[tm] = pack4(f32x4{w[tm][0] * sc.x, w[tm][1] * sc.y, w[tm][2] * sc.z, w[tm][3] * sc.w});
                }
                // h <- e^{gam_n} h + K^T (W diag(e^{gam_n - gam}))
#pragma unroll
                for (int kb = 0; kb < DT; ++kb) {
                    hacc[kb] *= el;
#pragma unroll
                    for (int tm = 0; tm < 4; ++tm) {
                        const short4_t ak = operand_tr4(Ks, LDD, 16 * tm, 16 * kb, lane);
                        hacc[kb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, wb[tm], hacc[kb], 0, 0, 0);
                    }
                    hb[kb] = pack4(hacc[kb]);
                    *(short4_t *)(hx((c + 1) & 1) + (v0 + r) * LDD + 16 * kb + 4 * g) = hb[kb];
                }
            }
        } else {
            // chunk c+1 into LDS (requested one chunk ago), chunk c+2 requested
            if (loader) {
                if (c + 1 < c1) stash(c + 1);
                if (c + 2 < c1) fetch(c + 2);
            } else if (o && c > c0 + 1) {
                // O rows helper hw - 4 finished one chunk ago
                store_o(c - 2, ib, 0, obufA(c - 2, hw - 4));
            }
            // finish O of the previous chunk: + P W
            if (o && c > c0) {
                const int pst = (c - 1) & 1;
                const u16 *Pt = pbuf(pst, ib), *WT = wx(pst);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 ap = operand_tr(Pt, LDP, 32 * ks, 0, lane);
#pragma unroll
                    for (int x = 0; x < VH; ++x) {
                        const bf16x8 bw = *(const bf16x8 *)(WT + (16 * (vb0 + x) + r) * LDC + 32 * ks + 8 * g);
                        accO[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bw, accO[x], 0, 0, 0);
                    }
                }
                // the 16 x 16*VH block goes out through LDS as 16-byte row
                // pieces; helpers 0..3 leave it for helpers 4..7
                u16 *Os = loader ? obufA(c - 1, hw) : obuf(hw);
#pragma unroll
                for (int x = 0; x < VH; ++x) {
                    if constexpr (OT) {
                        // four consecutive rows of one column: one 8-byte store
                        *(short4_t *)(Os + (16 * x + r) * LDOT + 4 * g) = pack4(accO[x]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) Os[(4 * g + e) * LDO + 16 * x + r] = f2bf(accO[x][e]);
                    }
                }
                if (!loader) store_o(c - 1, ib, vb0, Os);
            }
            // P's row block ib (storing helpers) and diag(e^gam) Q h
            if (o && c < c1) {
                const int st = c & 1;
                const u16 *Qs = stage(st, 0), *Ks = stage(st, 1), *HT = hx(st);
                const float *gam = gam_of(st);
                const float *eg = eg_of(st);
                bf16x8 aq[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) aq[ks] = *(const bf16x8 *)(Qs + (16 * ib + r) * LDD + 32 * ks + 8 * g);
                u16 *Pt = pbuf(st, ib);
                const float4 gi = *(const float4 *)(gam + 16 * ib + 4 * g);
                const float gil[4] = {gi.x, gi.y, gi.z, gi.w};
                // P is lower triangular over the chunk: of row block ib only
                // the column blocks 0..ib hold values. The storing helper of
                // the row block forms them and writes zeros for the others;
                // the loading helper, which also stages and requests the
                // chunks, forms none. (Handing the diagonal block of row
                // blocks 2 and 3 to the loading helpers, so that no helper
                // forms more than three, measured slower.)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    if (loader) break;
                    if (jb > ib) {
                        *(short4_t *)(Pt + (16 * jb + r) * LDP + 4 * g) = short4_t{0, 0, 0, 0};
                        continue;
                    }
                    f32x4 p = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 bk = *(const bf16x8 *)(Ks + (16 * jb + r) * LDD + 32 * ks + 8 * g);
                        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], bk, p, 0, 0, 0);
                    }
                    const int j = 16 * jb + r;
                    const float gj = gam[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p[e] = (16 * ib + 4 * g + e >= j) ? p[e] * exp2_fast(gil[e] - gj) : 0.f;
                    *(short4_t *)(Pt + j * LDP + 4 * g) = pack4(p);
                }
                const float4 sc = *(const float4 *)(eg + 16 * ib + 4 * g);
#pragma unroll
                for (int x = 0; x < VH; ++x) {
                    f32x4 y4 = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 bh8 = *(const bf16x8 *)(HT + (16 * (vb0 + x) + r) * LDD + 32 * ks + 8 * g);
                        y4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], bh8, y4, 0, 0, 0);
                    }
                    accO[x] = f32x4{y4[0] * sc.x, y4[1] * sc.y, y4[2] * sc.z, y4[3] * sc.w};
                }
            }
        }
        __syncthreads();
    }
    // the last O rows of helpers 0..3 (finished in the final iteration)
    if (o && !chain && !loader && c1 > c0) store_o(c1 - 1, ib, 0, obufA(c1 - 1, hw - 4));
    if (chain && a.hT) {
#pragma unroll
        for (int kb = 0; kb < DT; ++kb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * kb + 4 * g + e, v = V0 + v0 + r;
                if (d < dk && v < dv) a.hT[((size_t)bh * dk + d) * dv + v] = hacc[kb][e];
            }
        }
    }
}

// ---------------------------------------------------------------- launch

int pad_dim(int d, bool bf16) {
    int D = bf16 ? 32 : 16;
    while (D < d) D *= 2;
    return D;
}

// value columns per workgroup of the generic serial pass. Serial: 128-wide
// heads take 16 so that more workgroups share the chain (each carries part
// of the state), which measured faster on the long-context shape (16 heads).
// Segmented: the segments supply the parallelism, so wider blocks cut the
// work every block repeats (loading K and -Kw, forming P).
#ifndef GDN_SEG_BV
#define GDN_SEG_BV 128
#endif
int fwd_vblock(int D, bool segmented) {
    if (segmented) return D < GDN_SEG_BV ? D : GDN_SEG_BV;
    return D == 64 ? 32 : 16;
}

// Segments of the parallel scan: long sequences split into ranges of about
// SEG_CHUNKS chunks (at most 16 ranges); short ones stay serial.
#ifndef GDN_SEG_MAX
#define GDN_SEG_MAX 16
#endif
#ifndef GDN_SEG_CHUNKS
#define GDN_SEG_CHUNKS 32
#endif
int fwd_scan_segments(bool bf16, int D, int NC) {
    if (fwd_segmentable(bf16, D)) return 1; // the wave-specialised chain takes chunk ranges instead
    const int n = NC / GDN_SEG_CHUNKS;
    return n < 2 ? 1 : (n > GDN_SEG_MAX ? GDN_SEG_MAX : n);
}

bool fwd_segmentable(bool bf16, int D) { return bf16 && (D == 32 || D == 64); }

template <bool BF, int D> static hipError_t prep_inst(const PrepArgs &a, hipStream_t st) {
    const int grid = a.s.B * a.s.H * a.ncs;
    const bool vec = vec_ok<BF>(a.s);
    if (a.s.l2k)
        hipLaunchKernelGGL((vec ? fwd_prep_kernel<BF, D, true, true> : fwd_prep_kernel<BF, D, false, true>), dim3(grid),
                           dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((vec ? fwd_prep_kernel<BF, D, true, false> : fwd_prep_kernel<BF, D, false, false>),
                           dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

// Value columns per workgroup of the wave-specialised serial pass. Heads 64
// wide are split into two 32-column blocks: each workgroup then stages,
// multiplies and stores half of U, Qh and O (Q, K, -Kw and P are formed by
// both), which shortens the helpers' share of a chunk step, and the pass
// fills twice the compute units. At B8 H16 T4096 d56 the pass took 0.133 ms
// against 0.152 with one 64-column block (each run alone).
#ifndef GDN_WS_BV64
#define GDN_WS_BV64 32
#endif
constexpr int ws_vblock(int D) { return D == 64 ? GDN_WS_BV64 : D; }

int fwd_ws_blocks(int D, int dv) {
    const int bv = ws_vblock(D);
    return (dv + bv - 1) / bv;
}

template <int D> static hipError_t chain_ws_inst(const FwdChainArgs &a0, hipStream_t st) {
    constexpr int BV = ws_vblock(D);
    FwdChainArgs a = a0;
    a.NVB = (a.s.dv + BV - 1) / BV;
    const int grid = a.s.B * a.s.H * a.NVB;
    const int block = 64 * (BV / 16 + WS_HELPERS);
    const bool vec = vec_ok<true>(a.s), edge = a.s.l2k || a.s.D;
    if (vec && !edge)
        hipLaunchKernelGGL((fwd_chain_ws_kernel<D, BV, true, false>), dim3(grid), dim3(block), 0, st, a);
    else if (vec)
        hipLaunchKernelGGL((fwd_chain_ws_kernel<D, BV, true, true>), dim3(grid), dim3(block), 0, st, a);
    else if (!edge)
        hipLaunchKernelGGL((fwd_chain_ws_kernel<D, BV, false, false>), dim3(grid), dim3(block), 0, st, a);
    else
        hipLaunchKernelGGL((fwd_chain_ws_kernel<D, BV, false, true>), dim3(grid), dim3(block), 0, st, a);
    return hipGetLastError();
}

template <bool BF, int D, int BV> static hipError_t chain_bv(const FwdChainArgs &a, hipStream_t st) {
    const int nvbe = a.NVB + (a.mode == 1 ? (a.s.dk + BV - 1) / BV : 0);
    const int nsl = a.mode == 1 ? a.nseg - 1 : a.nseg;
    const int grid = a.s.B * a.s.H * nsl * nvbe;
    if (vec_ok<BF>(a.s))
        hipLaunchKernelGGL((fwd_chain_kernel<BF, D, BV, true>), dim3(grid), dim3(NTHR), 0, st, a);
    else
        hipLaunchKernelGGL((fwd_chain_kernel<BF, D, BV, false>), dim3(grid), dim3(NTHR), 0, st, a);
    return hipGetLastError();
}

template <bool BF, int D> static hipError_t chain_inst(const FwdChainArgs &a, hipStream_t st) {
    const int bv = fwd_vblock(D, a.nseg > 1);
    if (a.nseg < 1 || (a.mode == 1 && a.nseg < 2)) return hipErrorInvalidValue;
    if (bv == 16) return chain_bv<BF, D, 16>(a, st);
    if constexpr (D >= 32)
        if (bv == 32) return chain_bv<BF, D, 32>(a, st);
    if constexpr (D >= 64)
        if (bv == 64) return chain_bv<BF, D, 64>(a, st);
    if constexpr (D >= 128)
        if (bv == 128) return chain_bv<BF, D, 128>(a, st);
    return hipErrorInvalidValue;
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
    if (fwd_vblock(D, a.nseg > 1) * a.NVB < a.s.dv) return hipErrorInvalidValue;
    if (bf16) {
        switch (D) {
        case 32: return chain_ws_inst<32>(a, st);
        case 64: return chain_ws_inst<64>(a, st);
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
