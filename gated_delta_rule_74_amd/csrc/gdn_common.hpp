// Device building blocks shared by the gated delta rule kernels (gfx950).
//
// Conventions used by every kernel:
//  * a chunk is C = 64 tokens ("GDN & MLA Mechanism Deep-Dive", Step 5 and
//    the portal's "CHUNK 64"); a workgroup is 512 threads = 8 wave64s (two per SIMD,
//    so one wave's latency is covered by the other's work);
//  * matrices live in LDS row-major with a 16-byte row pad; a product
//    C += A * B reads A as [M][K] and B as its transpose BT = [N][K] (both
//    K-contiguous), so one 16-byte LDS read feeds one bf16 MFMA operand;
//  * 16x16 output tiles are spread over the 8 waves (tile t -> wave t % 8);
//    inside a tile, lane l holds column (l % 16) and rows 4*(l/16) .. +3,
//    the accumulator layout of v_mfma_f32_16x16x32_bf16 / _16x16x4_f32;
//  * operands are bf16 (inputs in bf16) or fp32 (inputs in fp32); state,
//    accumulators, decay factors and the triangular solve stay fp32, and the
//    in-chunk cumulative log-decay is summed in fp64 so that differences of
//    two prefix sums keep their precision.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int C = 64;
constexpr int NTHR = 512;
constexpr int NWAVE = 8;
// epsilon under the root of the per-token key normalisation
constexpr float KEY_EPS = 1e-6f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// 2^x on the hardware exp unit (x <= 0 here; results below 2^-126 may flush
// to zero, far below any tolerance).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr double LOG2E = 1.4426950408889634;

// Operand storage: bf16 bit patterns or fp32.
template <bool BF> struct Op;
template <> struct Op<true> {
    using S = u16;
    static constexpr int PAD = 8;    // 16 bytes
    static constexpr int KSTEP = 32; // K per MFMA
    static constexpr int KSUB = 8;   // K elements per lane per MFMA
    static constexpr int VEC = 8;    // elements per 16-byte global vector
};
template <> struct Op<false> {
    using S = float;
    static constexpr int PAD = 4;
    static constexpr int KSTEP = 4;
    static constexpr int KSUB = 1;
    static constexpr int VEC = 4;
};

__device__ __forceinline__ float to_f(u16 x) { return bf2f(x); }
__device__ __forceinline__ float to_f(float x) { return x; }
template <bool BF> __device__ __forceinline__ typename Op<BF>::S from_f(float x);
template <> __device__ __forceinline__ u16 from_f<true>(float x) { return f2bf(x); }
template <> __device__ __forceinline__ float from_f<false>(float x) { return x; }

__device__ __forceinline__ f32x4 mma(const u16 *a, const u16 *b, f32x4 acc) {
    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(a);
    const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const float *a, const float *b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Number of 16x16 tiles a wave owns for an MT x NT tile grid spread over NW
// waves (tile t -> wave t % NW).
template <int MT, int NT, int NW = NWAVE> struct Tiles {
    static constexpr int N = MT * NT;
    static constexpr int PW = (N + NW - 1) / NW;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// One MFMA operand (8 consecutive K values for row/column r = lane % 16 of a
// 16-wide block) read from an LDS matrix stored with K as its row index,
// X[k][m] (row stride ld): two transposing 64-bit reads. Lane s of k-group g
// points at X[k0 + 8g + s/4 (+4)][m0 + 4(s%4)]; the hardware hands lane
// 16g + j the values X[k0 + 8g + e][m0 + j], e = 0..3 (then 4..7).
__device__ __forceinline__ bf16x8 operand_tr(const u16 *X, int ld, int k0, int m0, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const u16 *p = X + (k0 + 8 * g + (sl >> 2)) * ld + m0 + 4 * (sl & 3);
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(p));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(p + 4 * ld));
    uint4 u;
    u.x = __builtin_bit_cast(uint2, lo).x;
    u.y = __builtin_bit_cast(uint2, lo).y;
    u.z = __builtin_bit_cast(uint2, hi).x;
    u.w = __builtin_bit_cast(uint2, hi).y;
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ short4_t pack4(f32x4 x) {
    uint2 u;
    u.x = f2bf2(x[0], x[1]);
    u.y = f2bf2(x[2], x[3]);
    return __builtin_bit_cast(short4_t, u);
}

// A lane's two 16x16x16 operand pieces (4 values each, from K blocks k0 and
// k1) as its 8 values of one 16x16x32 operand. A product sums over K in any
// order, so when both operands are joined the same way, one K = 32 step
// covering both blocks gives the sum of the two K = 16 steps, in half the
// instructions (gfx950 runs a K = 32 step in the time of a K = 16 one).
__device__ __forceinline__ bf16x8 join8(short4_t lo, short4_t hi) {
    uint4 u;
    u.x = __builtin_bit_cast(uint2, lo).x;
    u.y = __builtin_bit_cast(uint2, lo).y;
    u.z = __builtin_bit_cast(uint2, hi).x;
    u.w = __builtin_bit_cast(uint2, hi).y;
    return __builtin_bit_cast(bf16x8, u);
}

// One 16x16x16 operand from an LDS matrix stored with K as its row index,
// X[k][m]: lane 16g + j receives X[k0 + 4g + e][m0 + j], e = 0..3.
__device__ __forceinline__ short4_t operand_tr4(const u16 *X, int ld, int k0, int m0, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4 *)(X + (k0 + 4 * g + (sl >> 2)) * ld + m0 + 4 * (sl & 3)));
}

// acc[i] += A * B over K = KD for the tiles of this wave.
// A is stored [M][K] (ATR = false) or [K][M] (ATR = true); B is stored [N][K]
// (BTR = false, i.e. B transposed) or [K][N] (BTR = true). Row strides lda, ldb.
// KU > 0 limits the unrolling of the K loop (fewer operands in flight, for
// kernels short of registers); 0 unrolls it fully.
template <bool BF, int MT, int NT, int KD, bool ATR = false, bool BTR = false, int NW = NWAVE, int KU = 0>
__device__ __forceinline__ void gemm(const typename Op<BF>::S *A, int lda,
                                     const typename Op<BF>::S *B, int ldb, f32x4 *acc, int wave,
                                     int lane) {
    using O = Op<BF>;
    using TL = Tiles<MT, NT, NW>;
    static_assert(KD % O::KSTEP == 0, "contraction length must be a multiple of the MFMA K");
    constexpr int UNR = KU > 0 ? KU : KD / O::KSTEP;
    const int r = lane & 15, kq = lane >> 4;
    if constexpr (BF && NW % NT == 0 && TL::N % NW == 0 && TL::PW > 1) {
        // all tiles of this wave share the column block tn = wave % NT: read
        // each B operand once per K step and reuse it for every tile
        const int tn = wave % NT;
#pragma unroll UNR
        for (int k0 = 0; k0 < KD; k0 += O::KSTEP) {
            const bf16x8 bv = BTR ? operand_tr(B, ldb, k0, tn * 16, lane)
                                  : *reinterpret_cast<const bf16x8 *>(B + (tn * 16 + r) * ldb + k0 + kq * 8);
#pragma unroll
            for (int i = 0; i < TL::PW; ++i) {
                const int tm = (wave + NW * i) / NT;
                const bf16x8 av = ATR ? operand_tr(A, lda, k0, tm * 16, lane)
                                      : *reinterpret_cast<const bf16x8 *>(A + (tm * 16 + r) * lda + k0 + kq * 8);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const int tm = t / NT, tn = t % NT;
#pragma unroll UNR
        for (int k0 = 0; k0 < KD; k0 += O::KSTEP) {
            if constexpr (BF) {
                const bf16x8 av = ATR ? operand_tr(A, lda, k0, tm * 16, lane)
                                      : *reinterpret_cast<const bf16x8 *>(A + (tm * 16 + r) * lda + k0 + kq * 8);
                const bf16x8 bv = BTR ? operand_tr(B, ldb, k0, tn * 16, lane)
                                      : *reinterpret_cast<const bf16x8 *>(B + (tn * 16 + r) * ldb + k0 + kq * 8);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
            } else {
                const int k = k0 + kq;
                const float av = ATR ? A[k * lda + tm * 16 + r] : A[(tm * 16 + r) * lda + k];
                const float bv = BTR ? B[k * ldb + tn * 16 + r] : B[(tn * 16 + r) * ldb + k];
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i], 0, 0, 0);
            }
        }
    }
}

// Visit every element this wave owns in an MT x NT tile grid:
// f(i, e, row, col) with acc index i and element e in 0..3.
template <int MT, int NT, int NW = NWAVE, class F>
__device__ __forceinline__ void for_tiles(int wave, int lane, F &&f) {
    using TL = Tiles<MT, NT, NW>;
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const int tm = t / NT, tn = t % NT;
#pragma unroll
        for (int e = 0; e < 4; ++e) f(i, e, tm * 16 + 4 * kq + e, tn * 16 + r);
    }
}

// This wave's tiles of a bf16 [rows][cols] LDS matrix X (row stride ld) in
// the accumulator layout: lane 16g + r gets rows 16 tm + 4g .. + 3 of column
// 16 tn + r, one transposing 64-bit read per tile (X read as the [K][M]
// operand of a 16x16x16 product).
template <int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void load_tiles(const u16 *X, int ld, f32x4 *out, int wave, int lane) {
    using TL = Tiles<MT, NT, NW>;
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const short4_t v = operand_tr4(X, ld, 16 * (t / NT), 16 * (t % NT), lane);
        out[i] = f32x4{bf2f((u16)v[0]), bf2f((u16)v[1]), bf2f((u16)v[2]), bf2f((u16)v[3])};
    }
}

// The same tiles of a matrix held transposed, Xt[col][row]: the four rows
// a lane owns are adjacent, one 64-bit read per tile.
template <int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void load_tiles_t(const u16 *Xt, int ld, f32x4 *out, int wave, int lane) {
    using TL = Tiles<MT, NT, NW>;
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const short4_t v = *reinterpret_cast<const short4_t *>(Xt + (16 * (t % NT) + (lane & 15)) * ld +
                                                               16 * (t / NT) + 4 * (lane >> 4));
        out[i] = f32x4{bf2f((u16)v[0]), bf2f((u16)v[1]), bf2f((u16)v[2]), bf2f((u16)v[3])};
    }
}

// Store the tiles of this wave transposed: dst[col][row] (4 consecutive rows
// per lane become 4 consecutive elements).
// (optionally scaled per row by rs[row]).
template <bool BF, int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void store_T(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int wave,
                                        int lane, const float *rs = nullptr) {
    using TL = Tiles<MT, NT, NW>;
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const int tm = t / NT, tn = t % NT;
        const int row = tm * 16 + 4 * kq, col = tn * 16 + r;
        f32x4 x = acc[i];
        if (rs) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= rs[row + e];
        }
        if constexpr (BF) {
            uint2 w;
            w.x = f2bf2(x[0], x[1]);
            w.y = f2bf2(x[2], x[3]);
            *reinterpret_cast<uint2 *>(dst + col * ld + row) = w;
        } else {
            *reinterpret_cast<f32x4 *>(dst + col * ld + row) = x;
        }
    }
}

template <bool BF, int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void store_N(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int wave,
                                        int lane) {
    for_tiles<MT, NT, NW>(wave, lane, [&](int i, int e, int row, int col) {
        dst[row * ld + col] = from_f<BF>(acc[i][e]);
    });
}

// Register fragment of an NR-row tile [NR][DP] (a chunk of a [B,T,H,*]
// tensor, or a state matrix) in row-major global memory.
// fetch() issues the global loads (16-byte vectors; one item = one vector of
// one row), stash() writes the fragment to LDS (optionally row-scaled).
// Items are numbered row-major: consecutive lanes hold consecutive 16-byte
// pieces of a row, so the loads of one wave touch as few cache lines as the
// tile's row layout allows.
template <bool BF, int DP, int NR = C, int NT = NTHR> struct ChunkFrag {
    using S = typename Op<BF>::S;
    static constexpr int V = Op<BF>::VEC;
    static constexpr int NG = DP / V;
    static constexpr int NIT = (NR * NG + NT - 1) / NT;
    static constexpr bool FULL = (NR * NG) % NT == 0; // every thread's items exist
    union U {
        uint4 u;
        S s[V];
    };
    U r[NIT];
    uint32_t ok; // bit m: item m lies inside the tensor (else it reads as zero)

    // item it = row j, vector group cg (row-major)
    __device__ __forceinline__ static void pos(int it, int &j, int &cg) {
        j = it / NG;
        cg = it % NG;
    }

    // x: column 0 of row 0 of the tile, rs: elements between rows, n valid
    // rows (n >= 1), d valid columns. VEC: rows start on 16-byte boundaries
    // and d % V == 0. The vector path issues its loads without any per-lane
    // branch (out-of-range items read a clamped in-range address and are
    // masked in stash()), so they stay in flight until the data is stashed.
    template <bool VEC>
    __device__ __forceinline__ void fetch(const S *__restrict__ x, size_t rs, int n, int d, int tid) {
        ok = 0;
        if constexpr (VEC) {
#pragma unroll
            for (int m = 0; m < NIT; ++m) {
                const int it = tid + m * NT;
                int j, cg;
                pos(it, j, cg);
                const bool in = (FULL || j < NR) && j < n && cg * V < d;
                const int jj = min(j, n - 1), cc = min(cg * V, d - V);
                r[m].u = *reinterpret_cast<const uint4 *>(x + (size_t)jj * rs + cc);
                ok |= (in ? 1u : 0u) << m;
            }
        } else {
#pragma unroll
            for (int m = 0; m < NIT; ++m) {
                const int it = tid + m * NT;
                int j, cg;
                pos(it, j, cg);
                r[m].u = uint4{0u, 0u, 0u, 0u};
                if (!FULL && j >= NR) continue;
                if (j < n) {
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        if (cg * V + e < d) r[m].s[e] = x[(size_t)j * rs + cg * V + e];
                }
                ok |= 1u << m;
            }
        }
    }

    __device__ __forceinline__ uint4 item(int m) const {
        return ((ok >> m) & 1u) ? r[m].u : uint4{0u, 0u, 0u, 0u};
    }

    // Per-row L2 normalisation, k_hat = k / sqrt(|k|^2 + KEY_EPS): the NG
    // consecutive lanes that hold a row sum its squares with xor shuffles
    // (every lane takes part, items outside the tile count as zero), then
    // every item is rescaled and rounded back to the operand type. The lane
    // holding column group 0 of a row writes 1 / sqrt(|k|^2 + KEY_EPS) to
    // rinv[row] when rinv is given.
    __device__ __forceinline__ void normalize_rows(float *rinv, int tid) {
        static_assert(NT % 64 == 0 && 64 % NG == 0, "a row's lanes lie in one wave");
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            U x;
            x.u = item(m);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < V; ++e) ss += to_f(x.s[e]) * to_f(x.s[e]);
#pragma unroll
            for (int off = NG / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
            const float inv = 1.f / sqrtf(ss + KEY_EPS);
#pragma unroll
            for (int e = 0; e < V; ++e) x.s[e] = from_f<BF>(to_f(x.s[e]) * inv);
            r[m].u = x.u;
            int j, cg;
            pos(tid + m * NT, j, cg);
            if (rinv && cg == 0 && (FULL || j < NR)) rinv[j] = inv;
        }
    }

    // Straight copy to dst [NR][ldd].
    __device__ __forceinline__ void stash(S *dst, int ldd, int tid) const {
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            int j, cg;
            pos(tid + m * NT, j, cg);
            if (!FULL && j >= NR) continue;
            *reinterpret_cast<uint4 *>(dst + j * ldd + cg * V) = item(m);
        }
    }

    // Straight copy with row j scaled by the value `sc` holds in lane j
    // (NR == 64: every wave carries the 64 row scales, one per lane).
    __device__ __forceinline__ void stash_scaled(S *dst, int ldd, int tid, float sc) const {
        static_assert(NR == 64, "one row scale per lane");
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            int j, cg;
            pos(tid + m * NT, j, cg);
            const float rsc = __shfl(sc, j, 64);
            if (!FULL && j >= NR) continue;
            U val, out;
            val.u = item(m);
#pragma unroll
            for (int e = 0; e < V; ++e) out.s[e] = from_f<BF>(to_f(val.s[e]) * rsc);
            *reinterpret_cast<uint4 *>(dst + j * ldd + cg * V) = out.u;
        }
    }
};

// A gate from its input: the logistic sigmoid of a logit when the inputs are
// logits, else the input itself.
__device__ __forceinline__ float gate_of(float x, bool logit) { return logit ? 1.f / (1.f + expf(-x)) : x; }

// Wait until every vector memory access this wave issued has completed
// (s_waitcnt with vmcnt = 0 and the other counters left free). Placed where
// all prefetched registers are needed anyway, it also tells the compiler's
// wait tracking that no load into them is still outstanding, so later loads
// into the same registers are not held back behind stores.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A per-lane scalar of a chunk (g or beta of row `lane`), loaded from a
// clamped in-range address without a branch. The caller masks rows >= n
// where it uses the value, so the load can stay in flight until then.
__device__ __forceinline__ float load_row_scalar(const float *__restrict__ p, size_t stride, int lane,
                                                 int n) {
    return p[(size_t)min(lane, n - 1) * stride];
}

// Zero the padding of a [D][ld] LDS matrix outside [d0][d1].
template <bool BF, int D>
__device__ __forceinline__ void zero_pad(typename Op<BF>::S *m, int ld, int d0, int d1, int tid) {
    using S = typename Op<BF>::S;
    if (d0 == D && d1 == D) return;
    for (int e = tid; e < D * D; e += NTHR) {
        const int i = e / D, j = e % D;
        if (i >= d0 || j >= d1) m[i * ld + j] = S(0);
    }
}

// Per-chunk decay factors of row `lane` of a chunk. lam_r = g_r * A with
// A = -exp(A_log); the cumulative in-chunk log-decay is kept in the log2
// domain, gam2_i = log2(e) * sum_{r <= i} lam_r, summed in fp64 so that the
// difference of two prefix sums keeps its precision. Rows past the end of
// the sequence pass g = 0, so gam2 stays at its last valid value there.
// Every wave can run this on its own copy of the gates.
// Gam_ij = exp(gam_i - gam_j) for i >= j, else 0 (gam2 in LDS, log2 domain).
// Both reads and the exponential happen on every lane and the mask is a
// select, so no lane branches around LDS reads.
__device__ __forceinline__ float gamma_ij(const double *gam2, int i, int j) {
    const float f = exp2_fast((float)(gam2[i] - gam2[j]));
    return (i >= j) ? f : 0.f;
}

constexpr int LDF = C + 4; // row stride of fp32 C x C matrices

// T = (I + L)^{-1} for a strictly lower triangular 64 x 64 L, given as its
// transpose Lt[j][i] = L[i][j] (fp32, [C][LDF]). T is written over the lower
// triangle (diagonal blocks included) of the same array: the blocks of Lt the
// solve reads after the diagonal step lie strictly above the block diagonal,
// and each diagonal block is read whole into registers before it is
// overwritten. Diagonal 16 x 16 blocks by forward substitution, all four in
// wave 0 (lane group g = block g, lane = column); the step-i multipliers
// L[i+1..15][i] are one row of Lt, read two steps ahead so the LDS latency
// overlaps the updates. Off-diagonal blocks by block forward substitution
//   T_ij = -T_ii * sum_{k=j}^{i-1} L_ik T_kj
// level by level (i - j = 1, 2, 3) with fp32 MFMA; waves 0..3 do the work,
// one barrier per level. xs: 4 x 16 x 17 floats, one 16 x 17 tile per wave. Tb ([C][ldt]) receives T in the operand type as
// its blocks are produced, zeros above the block diagonal.
// Ends with a barrier.
template <bool BF>
__device__ __forceinline__ void tri_inverse(float *LT, float *xs, int wave, int lane, typename Op<BF>::S *Tb,
                                            int ldt) {
    const float *Lt = LT;
    float *Tm = LT;
    using S = typename Op<BF>::S;
    if (wave == 0) {
        const int c = lane & 15, o = 16 * (lane >> 4);
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
        // right-looking: once x_i is final, fold it into every later row
        auto ldrow = [&](int i, float4 *d) {
            const float *p = Lt + (o + i) * LDF + o;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) d[q4] = *reinterpret_cast<const float4 *>(p + 4 * q4);
        };
        float4 r0[4], r1[4], r2[4];
        ldrow(0, r0);
        ldrow(1, r1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 2 < 16) ldrow(i + 2, r2);
            const float l[16] = {r0[0].x, r0[0].y, r0[0].z, r0[0].w, r0[1].x, r0[1].y, r0[1].z, r0[1].w,
                                 r0[2].x, r0[2].y, r0[2].z, r0[2].w, r0[3].x, r0[3].y, r0[3].z, r0[3].w};
#pragma unroll
            for (int rr = i + 1; rr < 16; ++rr) x[rr] -= l[rr] * x[i];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                r0[q4] = r1[q4];
                r1[q4] = r2[q4];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Tm[(o + i) * LDF + o + c] = x[i];
            Tb[(o + i) * ldt + o + c] = from_f<BF>(x[i]);
        }
    } else if (wave < 4) {
        // zero the blocks right of the diagonal in block row wave - 1
        const int o = 16 * (wave - 1);
        for (int e = lane; e < 16 * 48; e += 64) {
            const int i = e / 48, cc = e % 48 + o + 16;
            if (cc < C) Tb[(o + i) * ldt + cc] = S(0);
        }
    }
    __syncthreads();
    const int r = lane & 15, kq = lane >> 4;
    float *X = xs + (wave & 3) * 16 * 17;
    for (int s = 1; s < 4; ++s) {
        const int bi = wave < 4 ? s + wave : 4, bj = wave; // block (bi, bj), bi - bj = s
        if (bi < 4) {
            f32x4 acc = zero4();
            for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4) {
                    const float a = Lt[(16 * bk + k0 + kq) * LDF + 16 * bi + r];
                    const float b = Tm[(16 * bk + k0 + kq) * LDF + 16 * bj + r];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) X[(4 * kq + e) * 17 + r] = acc[e];
        }
        // X is this wave's own: its LDS writes are ordered before the reads
        // below without a workgroup barrier
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (bi < 4) {
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) {
                const float a = Tm[(16 * bi + r) * LDF + 16 * bi + k0 + kq];
                const float b = X[(k0 + kq) * 17 + r];
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
            }
            const int col = 16 * bj + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * bi + 4 * kq + e;
                const float t = -acc[e];
                Tm[row * LDF + col] = t;
                Tb[row * ldt + col] = from_f<BF>(t);
            }
        }
        __syncthreads();
    }
}

// x moved from lane (l ^ 1) / (l ^ 2) / mirrored within 8 / mirrored within
// 16 lanes: data-parallel-primitive moves inside a 16-lane row.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF,
                                                                 0xF, true));
}

// x from the lane `CTRL` names, for the rows in ROWMASK only (other rows get 0).
template <int CTRL, int ROWMASK> __device__ __forceinline__ float dpp_rows(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK,
                                                                 0xF, false));
}

__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Sum over the 16 lanes of a row; every lane of the row gets the total.
__device__ __forceinline__ float sum16(float x) {
    x += dpp_f<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);  // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x); // row_half_mirror
    x += dpp_f<0x140>(x); // row_mirror
    return x;
}

// One reduce-scatter step over a 16-lane row: the lanes whose selecting bit
// is set keep the upper half of the N values they carry, the others the lower
// half, and each adds the partner lane's copy of the half it keeps (CTRL names
// a partner with the other selecting bit). With N == 1 the step is a plain add.
template <int CTRL, int N> __device__ __forceinline__ void rs_step(float *v, bool hi) {
    if constexpr (N == 1) {
        v[0] += dpp_f<CTRL>(v[0]);
    } else {
        constexpr int h = N / 2;
#pragma unroll
        for (int j = 0; j < h; ++j) {
            const float keep = hi ? v[j + h] : v[j], send = hi ? v[j] : v[j + h];
            v[j] = keep + dpp_f<CTRL>(send);
        }
    }
}

// Row sums of N values at once (N = 2, 4, 8 or 16; x[v] is this lane's
// value v): lane r of every 16-lane row ends with the sum over the row's
// lanes of value r % N. The bits of r that pick the value are settled from
// the highest down, each by a partner that differs in that bit and agrees in
// the bits already settled (lane 15 - r, r ^ 7, r ^ 2, r ^ 1); the remaining
// steps add lanes that hold the same value (rotations by 8 and 4). Costs
// 3(N - 1) + (4 - log2 N) instructions against 4N for N calls of sum16.
template <int N> __device__ __forceinline__ float rsum16(const float *x, int r) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "2, 4, 8 or 16 values");
    float v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = x[j];
    if constexpr (N == 16) {
        rs_step<0x140, 16>(v, r & 8); // row_mirror
        rs_step<0x141, 8>(v, r & 4);  // row_half_mirror
        rs_step<0x4E, 4>(v, r & 2);   // quad_perm [2,3,0,1]
        rs_step<0xB1, 2>(v, r & 1);   // quad_perm [1,0,3,2]
    } else if constexpr (N == 8) {
        rs_step<0x141, 8>(v, r & 4);
        rs_step<0x4E, 4>(v, r & 2);
        rs_step<0xB1, 2>(v, r & 1);
        rs_step<0x128, 1>(v, false); // row_ror:8
    } else if constexpr (N == 4) {
        rs_step<0x4E, 4>(v, r & 2);
        rs_step<0xB1, 2>(v, r & 1);
        rs_step<0x124, 1>(v, false); // row_ror:4
        rs_step<0x128, 1>(v, false);
    } else {
        rs_step<0xB1, 2>(v, r & 1);
        rs_step<0x4E, 1>(v, false);
        rs_step<0x124, 1>(v, false);
        rs_step<0x128, 1>(v, false);
    }
    return v[0];
}

// Sum over the 64 lanes (fixed order: row sums, then rows 0+1 and 2+3);
// the same value in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x = sum16(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets x_0 + ... +
// x_l): shifts inside 16-lane rows, then the row totals carried across rows.
__device__ __forceinline__ float wave_prefix(float x) {
    x += dpp_f<0x111>(x); // row_shr:1 (lanes shifted in from outside the row read 0)
    x += dpp_f<0x112>(x); // row_shr:2
    x += dpp_f<0x114>(x); // row_shr:4
    x += dpp_f<0x118>(x); // row_shr:8
    x += dpp_rows<0x142, 0xA>(x); // row_bcast:15 into rows 1 and 3
    x += dpp_rows<0x143, 0xC>(x); // row_bcast:31 into rows 2 and 3
    return x;
}

struct Decay {
    double gam2;  // log2 of the cumulative decay up to this row
    float eg;     // exp(gam_i)
    float egn;    // exp(gam_last - gam_i)
    float eglast; // exp(gam_last)
};

// fp64 value moved like dpp_f / dpp_rows (both 32-bit halves with the same
// control; lanes that read nothing get +0.0).
template <int CTRL, int ROWMASK, bool BC> __device__ __forceinline__ double dpp_d(double x) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROWMASK, 0xF, BC);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROWMASK, 0xF, BC);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Chunk decay for lane = row: gam2 = A2 * (g_0 + ... + g_lane) (log2 domain,
// fp64 inclusive scan with the same data-parallel moves as wave_prefix).
__device__ __forceinline__ Decay decay_lane(float g, double A2, int lane) {
    double s = (double)g * A2;
    s += dpp_d<0x111, 0xF, true>(s); // row_shr:1
    s += dpp_d<0x112, 0xF, true>(s); // row_shr:2
    s += dpp_d<0x114, 0xF, true>(s); // row_shr:4
    s += dpp_d<0x118, 0xF, true>(s); // row_shr:8
    s += dpp_d<0x142, 0xA, false>(s); // row_bcast:15 into rows 1 and 3
    s += dpp_d<0x143, 0xC, false>(s); // row_bcast:31 into rows 2 and 3
    const unsigned long long u = __builtin_bit_cast(unsigned long long, s);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 63);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 63);
    const double last = __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
    (void)lane;
    return Decay{s, exp2_fast((float)s), exp2_fast((float)(last - s)), exp2_fast((float)last)};
}

// Per-tile row sums of x (x[i][e] is this lane's value at (row, col) of tile
// i): the 16 lanes of a row group are summed inside their row, and one lane
// writes part[row * NT + tn]. Every (row, tn) slot has exactly one writer, so
// a later fixed-order sum over tn is deterministic. When every wave holds
// 1, 2 or 4 tiles, all of its values are reduced together (rsum16): lane r < 4PW
// then holds tile r / 4, row 4 kq + r % 4.
template <int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void row_partials(const f32x4 *x, float *part, int wave, int lane) {
    using TL = Tiles<MT, NT, NW>;
    const int r = lane & 15, kq = lane >> 4;
    if constexpr (TL::N % NW == 0 && (TL::PW == 1 || TL::PW == 2 || TL::PW == 4)) {
        constexpr int NV = 4 * TL::PW;
        float xs[NV];
#pragma unroll
        for (int i = 0; i < TL::PW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[4 * i + e] = x[i][e];
        const float s = rsum16<NV>(xs, r);
        if (r < NV) {
            const int t = wave + NW * (r >> 2);
            part[((t / NT) * 16 + 4 * kq + (r & 3)) * NT + t % NT] = s;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const int tm = t / NT, tn = t % NT;
        f32x4 s = x[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = sum16(s[e]);
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) part[(tm * 16 + 4 * kq + e) * NT + tn] = s[e];
        }
    }
}

// Per-tile column sums: part[col * MT + tm].
template <int MT, int NT, int NW = NWAVE>
__device__ __forceinline__ void col_partials(const f32x4 *x, float *part, int wave, int lane) {
    using TL = Tiles<MT, NT, NW>;
    const int r = lane & 15;
#pragma unroll
    for (int i = 0; i < TL::PW; ++i) {
        const int t = wave + NW * i;
        if (TL::N % NW != 0 && t >= TL::N) break;
        const int tm = t / NT, tn = t % NT;
        float s = (x[i][0] + x[i][1]) + (x[i][2] + x[i][3]);
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (lane < 16) part[(tn * 16 + r) * MT + tm] = s;
    }
}

// Workgroup -> logical index. Consecutive workgroups are dispatched round
// robin over the 8 XCDs; remap so that each XCD receives a contiguous range
// of logical indices (neighbouring heads share cache lines of q/k/v rows, and
// each XCD has its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    if (nblk % 8 != 0) return bid;
    return (bid % 8) * (nblk / 8) + bid / 8;
}

} // namespace gdn
