// Device building blocks shared by the gated delta rule kernels (gfx950).
//
// Conventions used by every kernel:
//  * a chunk is C = 64 tokens ("GDN & MLA Mechanism Deep-Dive", Step 5 and
//    the portal's "CHUNK 64"); a workgroup is 256 threads = 4 wave64s;
//  * matrices live in LDS row-major with a 16-byte row pad; a product
//    C += A * B reads A as [M][K] and B as its transpose BT = [N][K] (both
//    K-contiguous), so one 16-byte LDS read feeds one bf16 MFMA operand;
//  * 16x16 output tiles are spread over the 4 waves (tile t -> wave t % 4);
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
constexpr int NTHR = 256;
constexpr int NWAVE = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ u16 f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u16)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

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

// Number of 16x16 tiles a wave owns for an MT x NT tile grid.
template <int MT, int NT> struct Tiles {
    static constexpr int N = MT * NT;
    static constexpr int PW = (N + NWAVE - 1) / NWAVE;
};

// acc[i] += A * B over K = KD for the tiles of this wave.
// A: [M][lda] row-major, BT: [N][ldb] row-major (B transposed).
template <bool BF, int MT, int NT, int KD>
__device__ __forceinline__ void gemm(const typename Op<BF>::S *A, int lda,
                                     const typename Op<BF>::S *BT, int ldb, f32x4 *acc, int wave,
                                     int lane) {
    using O = Op<BF>;
    static_assert(KD % O::KSTEP == 0, "contraction length must be a multiple of the MFMA K");
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < Tiles<MT, NT>::PW; ++i) {
        const int t = wave + NWAVE * i;
        if (Tiles<MT, NT>::N % NWAVE != 0 && t >= Tiles<MT, NT>::N) break;
        const int tm = t / NT, tn = t % NT;
        const typename O::S *a = A + (tm * 16 + r) * lda + kq * O::KSUB;
        const typename O::S *b = BT + (tn * 16 + r) * ldb + kq * O::KSUB;
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += O::KSTEP) acc[i] = mma(a + k0, b + k0, acc[i]);
    }
}

// Visit every element this wave owns in an MT x NT tile grid:
// f(i, e, row, col) with acc index i and element e in 0..3.
template <int MT, int NT, class F>
__device__ __forceinline__ void for_tiles(int wave, int lane, F &&f) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < Tiles<MT, NT>::PW; ++i) {
        const int t = wave + NWAVE * i;
        if (Tiles<MT, NT>::N % NWAVE != 0 && t >= Tiles<MT, NT>::N) break;
        const int tm = t / NT, tn = t % NT;
#pragma unroll
        for (int e = 0; e < 4; ++e) f(i, e, tm * 16 + 4 * kq + e, tn * 16 + r);
    }
}

// Store the tiles of this wave transposed: dst[col][row] (4 consecutive rows
// per lane become 4 consecutive elements).
template <bool BF, int MT, int NT>
__device__ __forceinline__ void store_T(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int wave,
                                        int lane) {
    for_tiles<MT, NT>(wave, lane, [&](int i, int e, int row, int col) {
        dst[col * ld + row] = from_f<BF>(acc[i][e]);
    });
}

template <bool BF, int MT, int NT>
__device__ __forceinline__ void store_N(const f32x4 *acc, typename Op<BF>::S *dst, int ld, int wave,
                                        int lane) {
    for_tiles<MT, NT>(wave, lane, [&](int i, int e, int row, int col) {
        dst[row * ld + col] = from_f<BF>(acc[i][e]);
    });
}

// Load a C-row chunk of a [B,T,H,*] tensor (rows t0 .. t0+n-1 of one (b,h);
// `x` points at column 0 of row t0, `rs` elements between rows, d valid
// columns) into LDS, zero filled to C rows and DP columns. dst ([C][ldd])
// receives it as stored, dstT ([DP][ldt]) transposed; either may be null.
// When tscale is given the transposed copy gets row j multiplied by
// tscale[j]. `vec` selects 16-byte global loads; the caller sets it only when
// every row start and d are multiples of 16 bytes.
template <bool BF, int DP>
__device__ __forceinline__ void load_chunk(const typename Op<BF>::S *__restrict__ x, size_t rs,
                                           int n, int d, bool vec, typename Op<BF>::S *dst,
                                           int ldd, typename Op<BF>::S *dstT, int ldt, int tid,
                                           const float *tscale = nullptr) {
    using O = Op<BF>;
    using S = typename O::S;
    constexpr int V = O::VEC;
    if (vec) {
        constexpr int NG = DP / V; // vector groups per row
        for (int it = tid; it < C * NG; it += NTHR) {
            const int j = it / NG, cg = it % NG;
            union {
                uint4 u;
                S s[V];
            } val;
            if (j < n && cg * V < d)
                val.u = *reinterpret_cast<const uint4 *>(x + (size_t)j * rs + cg * V);
            else
                val.u = uint4{0u, 0u, 0u, 0u};
            if (dst) *reinterpret_cast<uint4 *>(dst + j * ldd + cg * V) = val.u;
            if (dstT) {
                const float sc = tscale ? tscale[j] : 1.f;
#pragma unroll
                for (int e = 0; e < V; ++e)
                    dstT[(cg * V + e) * ldt + j] = tscale ? from_f<BF>(to_f(val.s[e]) * sc) : val.s[e];
            }
        }
    } else {
        for (int it = tid; it < C * DP; it += NTHR) {
            const int j = it / DP, c = it % DP;
            const S val = (j < n && c < d) ? x[(size_t)j * rs + c] : S(0);
            if (dst) dst[j * ldd + c] = val;
            if (dstT) dstT[c * ldt + j] = tscale ? from_f<BF>(to_f(val) * tscale[j]) : val;
        }
    }
}

// Per-chunk decay factors. lam_r = g_r * A (A = -exp(A_log)), gam_i = sum of
// lam over the chunk up to i (fp64). Rows >= n get lam = 0, so gam stays at
// its last valid value. Writes gam (fp64), eg = exp(gam), egn = exp(gam_last -
// gam) and *eglast = exp(gam_last). Run by wave 0 only.
__device__ __forceinline__ void decay_prep(const float *__restrict__ gch, double A, int n, int lane,
                                           double *gam, float *eg, float *egn, float *eglast) {
    double s = (lane < n) ? (double)gch[lane] * A : 0.0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(s, off, 64);
        if (lane >= off) s += o;
    }
    const double last = __shfl(s, 63, 64);
    gam[lane] = s;
    eg[lane] = expf((float)s);
    egn[lane] = expf((float)(last - s));
    if (lane == 0) *eglast = expf((float)last);
}

constexpr int LDF = C + 4; // row stride of fp32 C x C matrices

// T = (I + L)^{-1} for a strictly lower triangular 64 x 64 L (fp32, [C][LDF]),
// written to Tm ([C][LDF]). Diagonal 16 x 16 blocks by forward substitution
// (one wave each), off-diagonal blocks by block forward substitution
//   T_ij = -T_ii * sum_{k=j}^{i-1} L_ik T_kj
// level by level (i - j = 1, 2, 3) with fp32 MFMA. xs: 4 x 16 x 17 floats.
// Ends with a barrier.
__device__ __forceinline__ void tri_inverse(const float *L, float *Tm, float *xs, int wave,
                                            int lane) {
    {
        const int c = lane & 15, o = 16 * wave;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= L[(o + i) * LDF + o + j] * x[j];
            x[i] = s;
        }
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) Tm[(o + i) * LDF + o + c] = x[i];
        }
        // zero the blocks right of the diagonal in this block row
        for (int e = lane; e < 16 * 48; e += 64) {
            const int i = e / 48, cc = e % 48 + 16 * (wave + 1);
            if (cc < C) Tm[(o + i) * LDF + cc] = 0.f;
        }
    }
    __syncthreads();
    const int r = lane & 15, kq = lane >> 4;
    float *X = xs + wave * 16 * 17;
    for (int s = 1; s < 4; ++s) {
        const int bi = s + wave, bj = wave; // block (bi, bj), bi - bj = s
        if (bi < 4) {
            f32x4 acc = zero4();
            for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4) {
                    const float a = L[(16 * bi + r) * LDF + 16 * bk + k0 + kq];
                    const float b = Tm[(16 * bk + k0 + kq) * LDF + 16 * bj + r];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) X[(4 * kq + e) * 17 + r] = acc[e];
        }
        __syncthreads();
        if (bi < 4) {
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) {
                const float a = Tm[(16 * bi + r) * LDF + 16 * bi + k0 + kq];
                const float b = X[(k0 + kq) * 17 + r];
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[(16 * bi + 4 * kq + e) * LDF + 16 * bj + r] = -acc[e];
        }
        __syncthreads();
    }
}

// Per-tile row sums of x (x[i][e] is this lane's value at (row, col) of tile
// i): the 16 lanes of a row group are summed by a butterfly, and lane r == 0
// writes part[row * NT + tn]. Every (row, tn) slot has exactly one writer, so
// a later fixed-order sum over tn is deterministic.
template <int MT, int NT>
__device__ __forceinline__ void row_partials(const f32x4 *x, float *part, int wave, int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < Tiles<MT, NT>::PW; ++i) {
        const int t = wave + NWAVE * i;
        if (Tiles<MT, NT>::N % NWAVE != 0 && t >= Tiles<MT, NT>::N) break;
        const int tm = t / NT, tn = t % NT;
        f32x4 s = x[i];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += __shfl_xor(s[e], off, 64);
        }
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) part[(tm * 16 + 4 * kq + e) * NT + tn] = s[e];
        }
    }
}

// Per-tile column sums: part[col * MT + tm].
template <int MT, int NT>
__device__ __forceinline__ void col_partials(const f32x4 *x, float *part, int wave, int lane) {
    const int r = lane & 15;
#pragma unroll
    for (int i = 0; i < Tiles<MT, NT>::PW; ++i) {
        const int t = wave + NWAVE * i;
        if (Tiles<MT, NT>::N % NWAVE != 0 && t >= Tiles<MT, NT>::N) break;
        const int tm = t / NT, tn = t % NT;
        float s = (x[i][0] + x[i][1]) + (x[i][2] + x[i][3]);
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (lane < 16) part[(tn * 16 + r) * MT + tm] = s;
    }
}

// Load a [d0][d1] state matrix (row-major in global, element type S) into
// LDS zero-padded to [D][D]: straight into dst ([D][ld]) and/or transposed
// into dstT ([D][ld]).
template <bool BF, int D>
__device__ __forceinline__ void load_state(const typename Op<BF>::S *__restrict__ x, int d0, int d1,
                                           typename Op<BF>::S *dst, typename Op<BF>::S *dstT,
                                           int ld, int tid) {
    using S = typename Op<BF>::S;
    for (int e = tid; e < D * D; e += NTHR) {
        const int i = e / D, j = e % D;
        const S val = (i < d0 && j < d1) ? x[(size_t)i * d1 + j] : S(0);
        if (dst) dst[i * ld + j] = val;
        if (dstT) dstT[j * ld + i] = val;
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
