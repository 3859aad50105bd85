// Host-side launch interface between the C ABI (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// gdn_fwd with a choice of streams: one_stream runs every launch on the
// caller's stream (no second stream is created or used). With ws_lookup set,
// ws is ignored: once every argument has passed validation, ws_lookup
// supplies the workspace (ws_bytes long, library-owned, so it aliases no
// argument).
gdn_status_t fwd_entry(const gdn_shape_t *s, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *A_log, const float *D, const float *h0, void *o, float *hT,
                       void *ctx,
                       void *ws, size_t ws_bytes, void *stream, bool one_stream,
                       gdn_status_t (*ws_lookup)(void *&ws));
// Sets the text gdn_last_error_detail() returns and passes st through.
gdn_status_t fail_detail(gdn_status_t st, const char *text);

struct SeqArgs {
    const void *q, *k, *v;
    const float *g, *beta, *A_log, *h0;
    int B, T, H, dk, dv, NC;
    int additive;
    int logits; // g and beta are logits (sigmoid applied where they are used)
    int l2k;    // keys are L2-normalised per token where they are loaded
    const float *D; // [H] skip weights (o_t += D_h v_t), or null
};

// Per-chunk products that do not depend on the state:
// U = Tm diag(beta) V  [B*H][NC][64][dv],  NK = -Tm diag(beta e^gam) K  [B*H][NC][64][dk],
// and (if Tsave is set) Tm itself [B*H][NC][64][64], row-major, for the backward.
struct PrepArgs {
    SeqArgs s;
    void *U, *NK;
    void *Tsave; // may be null
    float *gam;  // chunk-local cumulative log2-decay [B*H][NC][64], may be null
    int c0, ncs; // chunks c0 .. c0 + ncs - 1 of every (batch, head)
};

struct FwdChainArgs {
    SeqArgs s;
    const void *U, *NK;
    const float *gam; // from fwd_prep
    void *o;   // may be null (state-only pass)
    float *hT; // may be null
    void *cs;  // chunk-start states, transposed: [B,H,NC,dv,dk] in operand dtype; may be null
    int NVB;   // value-column blocks
    // chunk range of this launch and the fp32 state at chunk c0 ([B,H,dk,dv],
    // null: zero); hT receives the state after chunk c1 - 1. The general
    // chain kernel supports only the whole range with h_in == s.h0.
    int c0, c1;
    const float *h_in;
    // Segmented launches of the general chain kernel (the parallel scan over
    // chunk ranges): the chunks are split into nseg equal segments and the
    // grid covers (batch-head, segment, value block). mode 0: every segment
    // runs from its start state (h_in for segment 0, seg_h for the others),
    // writes o and cs for its chunks, and the last segment writes hT. mode 1
    // (maps): segments 0 .. nseg-2 run from a zero start over dk identity
    // columns (U taken as zero) and the value columns; their final states are
    // the segment's affine map [M | R] (h_end = M h_start + R), written to
    // maps [B*H][nseg-1][dk][dk+dv] fp32; nothing else is written.
    int nseg = 1, mode = 0;
    const float *seg_h = nullptr; // [B*H][nseg][dk][dv] fp32
    float *maps = nullptr;
};

// Start state of every segment from the segment maps: h_0 = h0 (zero when
// null), h_{s+1} = M_s h_s + R_s; seg_h [B*H][nseg][dk][dv] fp32.
// With reverse set, the backward's mirror: x_{nseg-1} = h0 (there: dhT),
// x_{s-1} = M_{s-1} x_s + R_{s-1} with the map of segment s at index s - 1.
struct ScanArgs {
    const float *maps; // [B*H][nseg-1][dk][dk+dv]
    const float *h0;   // [B*H][dk][dv] or null
    float *seg_h;
    int BH, nseg, dk, dv;
    int reverse = 0;
};

struct BwdChainArgs {
    SeqArgs s;
    const void *dout;
    const float *dhT; // may be null
    const void *NK;
    void *dhs;        // [B,H,NC,dv,dk]: gradient wrt the state after each chunk, transposed
    float *dh0;       // may be null
    int NVB;
    // Segmented launches of the general reverse chain (mirror of the
    // forward's): mode 0: segment s runs backwards from the gradient at its
    // end (dhT for the last segment, seg_dh for the others), writes dhs for
    // its chunks, and segment 0 writes dh0. mode 1 (maps): segments
    // 1 .. nseg-1 run from a zero end gradient over dk identity columns (dO
    // taken as zero) and the value columns; their final gradients are the
    // segment's map [M | R] (dh_start = M dh_end + R), written to maps
    // [B*H][nseg-1][dk][dk+dv] fp32 (segment s at index s - 1).
    int nseg = 1, mode = 0;
    const float *seg_dh = nullptr; // [B*H][nseg][dk][dv] fp32: gradient at the end of each segment
    float *maps = nullptr;
};

struct BwdLocalArgs {
    SeqArgs s;
    const void *dout;
    const void *cs;  // chunk-start states (transposed)
    const void *NK;
    const void *U;   // U of every chunk (forward context)
    const void *Tm;  // (I + L)^{-1} of every chunk (forward context)
    const void *dhs; // gradient wrt chunk-end states (transposed)
    void *dq, *dk, *dv;
    float *dg, *dbeta;
    float *dA_part;  // [B*H*NC]
    float *dD_part;  // [B*H*NC][DD_SLOTS] partial sums of do * v (skip term), or null
    float *wide;     // scratch of the wide-head kernel (null for the others)
};

// Slots per chunk of the skip term's partial sums (one per wave of the local
// gradient kernels), reduced in a fixed order.
constexpr int DD_SLOTS = 8;

struct StepArgs {
    const void *q, *k, *v;
    const float *g, *beta, *A_log, *h_in;
    float *h_out;
    void *o;
    int N, H, dk, dv, additive;
    int S; // tokens per sequence; q, k, v, o, g, beta are [N, S, H, *]
    int logits;
    int l2k;        // keys L2-normalised per token
    const float *D; // [H] skip weights, or null
};

// 16-byte vector loads are possible when every row of q/k/v (and of the
// per-chunk blocks) starts on a 16-byte boundary.
template <bool BF> inline bool vec_ok(const SeqArgs &s) {
    const int v = BF ? 8 : 4;
    return s.dk % v == 0 && s.dv % v == 0;
}

// Padded head dimension the kernels are instantiated for.
int pad_dim(int d, bool bf16);
int fwd_vblock(int D, bool segmented);
// segments of the parallel scan the general forward chain uses (1: serial)
int fwd_scan_segments(bool bf16, int D, int NC);
hipError_t launch_fwd_scan(const ScanArgs &a, hipStream_t st);
bool fwd_segmentable(bool bf16, int D); // chain launch accepts a chunk range
// workgroups per (batch, head) of the wave-specialised serial pass
int fwd_ws_blocks(int D, int dv);
int bwd_chain_vblock(bool bf16, int D, bool segmented);
bool bwd_supported(bool bf16, int D);
// Scratch bytes the local-gradient pass needs for this padded head dim (0
// when the LDS-resident kernel covers it).
size_t bwd_wide_scratch_bytes(bool bf16, int D, int nchunks_total);

hipError_t launch_fwd_prep(const PrepArgs &a, bool bf16, int D, hipStream_t st);
hipError_t launch_fwd_chain(const FwdChainArgs &a, bool bf16, int D, hipStream_t st);
hipError_t launch_bwd_chain(const BwdChainArgs &a, bool bf16, int D, hipStream_t st);
hipError_t launch_bwd_local(const BwdLocalArgs &a, bool bf16, int D, hipStream_t st);
// bf16 heads wider than 64 (padded to 128): the LDS-resident wide kernel
hipError_t launch_bwd_local128(const BwdLocalArgs &a, hipStream_t st);
hipError_t launch_dA_reduce(const float *part, float *dA_log, int B, int H, int NC, hipStream_t st);
hipError_t launch_step(const StepArgs &a, bool bf16, hipStream_t st);
// dst[0..n) = src[0..n), or zeros when src is null
hipError_t launch_copy_or_zero(float *dst, const float *src, size_t n, hipStream_t st);

} // namespace gdn
