// C ABI of libgdn.so: argument validation, workspace layout and kernel
// launches. The operation itself is described in include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "gdn_launch.hpp"

namespace {

thread_local char g_detail[256] = "";

gdn_status_t fail(gdn_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return st;
}

gdn_status_t ok() {
    g_detail[0] = 0;
    return GDN_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

size_t esize(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

struct Range {
    const void *p;
    size_t n;
    const char *name;
};

bool overlap(const Range &a, const Range &b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const char *pa = (const char *)a.p, *pb = (const char *)b.p;
    return pa < pb + b.n && pb < pa + a.n;
}

gdn_status_t check_aliasing(const Range *in, int nin, const Range *out, int nout) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j]))
                return fail(GDN_EINVAL, "output %s overlaps input %s", out[i].name, in[j].name);
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j]))
                return fail(GDN_EINVAL, "output %s overlaps output %s", out[i].name, out[j].name);
    }
    return GDN_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr uint32_t KNOWN_FLAGS = GDN_FLAG_ADDITIVE | GDN_FLAG_GATE_LOGITS | GDN_FLAG_L2NORM_K;

gdn_status_t check_shape(const gdn_shape_t *s) {
    if (!s) return fail(GDN_EINVAL, "shape is NULL");
    if (s->B < 1 || s->T < 0 || s->H < 1) return fail(GDN_EINVAL, "B and H must be >= 1, T >= 0");
    if (s->dk < 1 || s->dv < 1 || s->dk > 128 || s->dv > 128)
        return fail(GDN_EINVAL, "dk and dv must be in [1, 128]");
    if (s->dtype != GDN_F32 && s->dtype != GDN_BF16) return fail(GDN_EINVAL, "unknown dtype %d", s->dtype);
    if (s->chunk != 0 && s->chunk != 64) return fail(GDN_EUNSUPPORTED, "chunk must be 0 or 64");
    if (s->flags & ~KNOWN_FLAGS) return fail(GDN_EINVAL, "unknown flag bits 0x%x", s->flags);
    if (s->dtype == GDN_F32 && (s->dk > 64 || s->dv > 64))
        return fail(GDN_EUNSUPPORTED, "fp32 supports dk, dv <= 64");
    const double elems = (double)s->B * s->T * s->H * (s->dk > s->dv ? s->dk : s->dv);
    if (elems >= 2147483648.0 || (double)s->B * s->H >= 2147483648.0)
        return fail(GDN_EINVAL, "tensor too large");
    return GDN_OK;
}

int nchunks(const gdn_shape_t *s) { return (s->T + 63) / 64; }

size_t states_bytes(const gdn_shape_t *s) {
    return (size_t)s->B * s->H * nchunks(s) * s->dk * s->dv * esize(s->dtype);
}

// per-chunk 64 x d blocks of U (d = dv) or NK (d = dk)
size_t blocks_bytes(const gdn_shape_t *s, int d) {
    return (size_t)s->B * s->H * nchunks(s) * 64 * d * esize(s->dtype);
}

// forward context = [chunk-start states | NK | U | Tm], each 256-byte aligned
struct CtxLayout {
    size_t nk, u, t, total;
};
CtxLayout ctx_layout(const gdn_shape_t *s) {
    CtxLayout l;
    l.nk = align_up(states_bytes(s));
    l.u = l.nk + align_up(blocks_bytes(s, s->dk));
    l.t = l.u + align_up(blocks_bytes(s, s->dv));
    l.total = l.t + align_up(blocks_bytes(s, 64));
    return l;
}
size_t ctx_bytes(const gdn_shape_t *s) { return ctx_layout(s).total; }

gdn::SeqArgs seq(const gdn_shape_t *s, const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *A_log, const float *D, const float *h0) {
    gdn::SeqArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.A_log = A_log;
    a.h0 = h0;
    a.B = s->B;
    a.T = s->T;
    a.H = s->H;
    a.dk = s->dk;
    a.dv = s->dv;
    a.NC = nchunks(s);
    a.additive = (s->flags & GDN_FLAG_ADDITIVE) ? 1 : 0;
    a.logits = (s->flags & GDN_FLAG_GATE_LOGITS) ? 1 : 0;
    a.l2k = (s->flags & GDN_FLAG_L2NORM_K) ? 1 : 0;
    a.D = D;
    return a;
}

int pad_of(const gdn_shape_t *s) {
    return gdn::pad_dim(s->dk > s->dv ? s->dk : s->dv, s->dtype == GDN_BF16);
}

// Launch bracketing for gdn_time_launches().
thread_local void *const *g_events = nullptr;
thread_local int g_nevents = 0;
thread_local int g_launch = 0;
constexpr int KIND_LOG = 4096;
thread_local int8_t g_kinds[KIND_LOG];
thread_local int g_kind_n = 0; // launches logged by the last bracketing period
enum Kind { K_FWD_PREP = 0, K_FWD_CHAIN, K_BWD_CHAIN, K_BWD_LOCAL, K_DA_REDUCE, K_STEP, K_FWD_SCAN, K_BWD_SCAN };

template <class F> hipError_t timed(Kind kind, F &&launch, hipStream_t st) {
    const int i = g_launch;
    if (g_events && i < KIND_LOG) g_kinds[i] = (int8_t)kind;
    const bool on = g_events && 2 * i + 1 < g_nevents;
    if (on) {
        const hipError_t e = hipEventRecord((hipEvent_t)g_events[2 * i], st);
        if (e != hipSuccess) return e;
    }
    const hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (on) {
        const hipError_t e2 = hipEventRecord((hipEvent_t)g_events[2 * i + 1], st);
        if (e2 != hipSuccess) return e2;
    }
    if (g_events) ++g_launch;
    return hipSuccess;
}

gdn_status_t hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

} // namespace

extern "C" {

const char *gdn_status_string(gdn_status_t st) {
    switch (st) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_EUNSUPPORTED: return "unsupported configuration";
    case GDN_EWORKSPACE: return "workspace missing or too small";
    case GDN_EHIP: return "HIP error";
    }
    return "unknown status";
}

const char *gdn_last_error_detail(void) { return g_detail; }

int32_t gdn_launch_kind(int32_t i) {
    const int n = g_events ? g_launch : g_kind_n;
    if (i < 0 || i >= n || i >= KIND_LOG) return -1;
    return g_kinds[i];
}

int32_t gdn_time_launches(void *const *events, int32_t n) {
    const int32_t done = g_launch;
    g_kind_n = done;
    g_events = events;
    g_nevents = events ? n : 0;
    g_launch = 0;
    return done;
}

} // extern "C"

namespace {

// per-token log2-decay of every chunk (fp32), written by fwd_prep
size_t gam_bytes(const gdn_shape_t *s) { return (size_t)s->B * s->H * nchunks(s) * 64 * sizeof(float); }
// one fp32 state per (batch, head): hand-off between chunk ranges
size_t state32_bytes(const gdn_shape_t *s) { return (size_t)s->B * s->H * s->dk * s->dv * sizeof(float); }

// Segments of the parallel scan over chunk ranges for this shape (1: the
// serial passes need no scan scratch).
int scan_segments(const gdn_shape_t *s) {
    return gdn::fwd_scan_segments(s->dtype == GDN_BF16, pad_of(s), nchunks(s));
}
// Scan scratch: the maps [M | R] of all but the last segment, then the
// state at every segment boundary, fp32, per (batch, head).
size_t scan_maps_floats(const gdn_shape_t *s) {
    const int n = scan_segments(s);
    return n > 1 ? (size_t)s->B * s->H * (n - 1) * s->dk * (s->dk + s->dv) : 0;
}
// per-chunk partial sums of do * v for dD, one slot per wave
size_t dD_part_bytes(const gdn_shape_t *s) {
    return align_up((size_t)s->B * s->H * nchunks(s) * gdn::DD_SLOTS * sizeof(float));
}
size_t scan_bytes(const gdn_shape_t *s) {
    const int n = scan_segments(s);
    if (n <= 1) return 0;
    return align_up(scan_maps_floats(s) * 4) + align_up((size_t)s->B * s->H * n * s->dk * s->dv * 4);
}

} // namespace

extern "C" {

size_t gdn_fwd_workspace_size(const gdn_shape_t *s) {
    if (check_shape(s) != GDN_OK) return 0;
    return align_up(blocks_bytes(s, s->dv)) + align_up(blocks_bytes(s, s->dk)) + align_up(gam_bytes(s)) +
           align_up(state32_bytes(s)) + scan_bytes(s);
}

size_t gdn_fwd_context_size(const gdn_shape_t *s) {
    if (check_shape(s) != GDN_OK) return 0;
    return ctx_bytes(s);
}

size_t gdn_bwd_workspace_size(const gdn_shape_t *s) {
    if (check_shape(s) != GDN_OK) return 0;
    const size_t part = align_up((size_t)s->B * s->H * nchunks(s) * sizeof(float));
    const int nch = s->B * s->H * nchunks(s);
    const size_t wide = align_up(gdn::bwd_wide_scratch_bytes(s->dtype == GDN_BF16, pad_of(s), nch));
    return ctx_bytes(s) /* recomputed forward context */ + align_up(states_bytes(s)) /* dh per chunk */ + part +
           align_up(gam_bytes(s)) /* forward decay */ + align_up(state32_bytes(s)) /* forward hand-off */ +
           wide /* local-gradient scratch for wide heads */ + scan_bytes(s) /* scan scratch */ +
           dD_part_bytes(s) /* skip-term partial sums */;
}

} // extern "C"

namespace {

// Second stream and events of this thread for one device: the forward
// overlaps the prep of the next chunk range with the serial pass over the
// current one. Created on first use, kept for the life of the process.
constexpr int MAX_SEG = 8;
struct Aux {
    hipStream_t side = nullptr;
    hipEvent_t ev[MAX_SEG + 1] = {};
};
thread_local Aux g_aux[64];

// out = the current device's second stream, created here on first use. When
// it does not exist yet and `strm` is being captured into a graph, nothing is
// created (a stream or event made in the middle of a capture would be a side
// effect of the capture) and out = nullptr: the caller then runs on `strm` alone.
hipError_t aux_of_current(Aux *&out, hipStream_t strm) {
    out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    Aux &x = g_aux[dev];
    if (!x.side) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(strm, &cap) != hipSuccess) {
            (void)hipGetLastError(); // a failed query must not fail a later launch check
            return hipSuccess;
        }
        if (cap != hipStreamCaptureStatusNone) return hipSuccess;
        e = hipStreamCreateWithFlags(&x.side, hipStreamNonBlocking);
        if (e != hipSuccess) return e;
        for (hipEvent_t &ev : x.ev) {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
    }
    out = &x;
    return hipSuccess;
}

// Compute units of the current device, looked up once per device.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int v = cache[dev & 63].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev & 63].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Number of chunk ranges the forward is split into, so that the prep of one
// range runs beside the serial pass of the previous one. One range when the
// serial kernel cannot take a range, when the sequence is short, or when the
// serial pass alone takes more than half of the compute units: a serial
// workgroup holds most of a unit's LDS, so the prep then finds no room beside
// it and the ranges only add launches (at B8 H16 T4096 d56, 256 serial
// workgroups: 0.224 ms for the forward as one range, 0.25 as four).
#ifndef GDN_FWD_RANGES
#define GDN_FWD_RANGES 4
#endif
int fwd_segments(const gdn_shape_t *s, bool bf, int D) {
    if (!gdn::fwd_segmentable(bf, D)) return 1;
    const long long wgs = (long long)s->B * s->H * gdn::fwd_ws_blocks(D, s->dv);
    if (2 * wgs > device_cus()) return 1;
    const int n = nchunks(s) / 16;
    return n < 1 ? 1 : (n > GDN_FWD_RANGES ? GDN_FWD_RANGES : n);
}

// Forward pass into caller-provided buffers: U, NK (and Tm, γ) of every
// chunk, then the serial state pass (o may be null: states only). hs: fp32
// [B,H,dk,dv] hand-off state between chunk ranges. With one_stream (or when
// no second stream can be had) everything runs on `strm` as a single chunk
// range; the results are the same bit for bit, only the overlap is lost.
hipError_t run_forward(const gdn_shape_t *s, const gdn::SeqArgs &sa, bool bf, int D, void *U, void *NK,
                       void *Tsave, float *gam, float *hs, float *scan, void *o, float *hT, void *cs,
                       hipStream_t strm, bool one_stream = false) {
    const int NC = nchunks(s);
    int nseg = one_stream ? 1 : fwd_segments(s, bf, D);
    Aux *x = nullptr;
    if (nseg > 1) {
        const hipError_t e = aux_of_current(x, strm);
        if (e != hipSuccess) return e;
        if (!x) nseg = 1;
    }
    gdn::PrepArgs pa;
    pa.s = sa;
    pa.U = U;
    pa.NK = NK;
    pa.Tsave = Tsave;
    pa.gam = gam;
    gdn::FwdChainArgs fa;
    fa.s = sa;
    fa.U = U;
    fa.NK = NK;
    fa.gam = gam;
    fa.o = o;
    fa.cs = cs;
    const int nscan = scan_segments(s);
    const int BV = gdn::fwd_vblock(D, nscan > 1);
    fa.NVB = (s->dv + BV - 1) / BV;
    auto seg_lo = [&](int k) { return (int)((long long)k * NC / nseg); };
    hipError_t he;
    if (nseg == 1) {
        pa.c0 = 0;
        pa.ncs = NC;
        he = timed(K_FWD_PREP, [&] { return gdn::launch_fwd_prep(pa, bf, D, strm); }, strm);
        if (he != hipSuccess) return he;
        fa.c0 = 0;
        fa.c1 = NC;
        fa.h_in = sa.h0;
        fa.hT = hT;
        if (nscan > 1) {
            // parallel scan over chunk ranges: the maps of every range but
            // the last, the start state of every range, then every range
            // from its start state at once
            fa.nseg = nscan;
            fa.mode = 1;
            fa.maps = scan;
            he = timed(K_FWD_CHAIN, [&] { return gdn::launch_fwd_chain(fa, bf, D, strm); }, strm);
            if (he != hipSuccess) return he;
            gdn::ScanArgs sc;
            sc.maps = scan;
            sc.h0 = sa.h0;
            sc.seg_h = scan + align_up(scan_maps_floats(s) * 4) / 4;
            sc.BH = s->B * s->H;
            sc.nseg = nscan;
            sc.dk = s->dk;
            sc.dv = s->dv;
            he = timed(K_FWD_SCAN, [&] { return gdn::launch_fwd_scan(sc, strm); }, strm);
            if (he != hipSuccess) return he;
            fa.mode = 0;
            fa.maps = nullptr;
            fa.seg_h = sc.seg_h;
        }
        return timed(K_FWD_CHAIN, [&] { return gdn::launch_fwd_chain(fa, bf, D, strm); }, strm);
    }
    // fork: the second stream starts after the caller's earlier work
    if ((he = hipEventRecord(x->ev[0], strm)) != hipSuccess) return he;
    if ((he = hipStreamWaitEvent(x->side, x->ev[0], 0)) != hipSuccess) return he;
    pa.c0 = 0;
    pa.ncs = seg_lo(1);
    he = timed(K_FWD_PREP, [&] { return gdn::launch_fwd_prep(pa, bf, D, strm); }, strm);
    if (he != hipSuccess) return he;
    for (int k = 0; k < nseg; ++k) {
        if (k + 1 < nseg) {
            pa.c0 = seg_lo(k + 1);
            pa.ncs = seg_lo(k + 2) - pa.c0;
            he = timed(K_FWD_PREP, [&] { return gdn::launch_fwd_prep(pa, bf, D, x->side); }, x->side);
            if (he != hipSuccess) return he;
            if ((he = hipEventRecord(x->ev[k + 1], x->side)) != hipSuccess) return he;
        }
        if (k > 0 && (he = hipStreamWaitEvent(strm, x->ev[k], 0)) != hipSuccess) return he;
        fa.c0 = seg_lo(k);
        fa.c1 = seg_lo(k + 1);
        fa.h_in = k == 0 ? sa.h0 : hs;
        fa.hT = k + 1 == nseg ? hT : hs;
        he = timed(K_FWD_CHAIN, [&] { return gdn::launch_fwd_chain(fa, bf, D, strm); }, strm);
        if (he != hipSuccess) return he;
    }
    return hipSuccess; // the last range waited for the second stream's last launch
}

} // namespace

// An empty sequence (T = 0) runs no step of the recurrence: the final state
// is h0 (zero when h0 is NULL); backward, the gradient of h0 is dhT (zero when
// NULL) and dA_log is zero. Arrays whose extent has a factor T hold nothing and
// may be NULL; no workspace is used.
static gdn_status_t fwd_empty(const gdn_shape_t *s, const float *h0, float *hT, hipStream_t st) {
    const size_t sb = state32_bytes(s);
    if ((h0 && !aligned(h0, 4)) || (hT && !aligned(hT, 4)))
        return fail(GDN_EINVAL, "fp32 arrays must be 4-byte aligned");
    const Range in[] = {{h0, h0 ? sb : 0, "h0"}};
    const Range out[] = {{hT, hT ? sb : 0, "hT"}};
    gdn_status_t e = check_aliasing(in, 1, out, 1);
    if (e != GDN_OK || !hT) return e;
    return hip_status(gdn::launch_copy_or_zero(hT, h0, sb / 4, st), "gdn_fwd (empty sequence)");
}

static gdn_status_t bwd_empty(const gdn_shape_t *s, const float *D, const float *h0, const void *ctx,
                              const float *dhT, float *dA_log, float *dD, float *dh0, float *hT, hipStream_t st) {
    if (!dA_log) return fail(GDN_EINVAL, "a required pointer is NULL");
    if (ctx && hT) return fail(GDN_EINVAL, "hT can only be recomputed when ctx is NULL");
    const float *f32[] = {D, h0, dhT, dA_log, dD, dh0, hT};
    for (const float *p : f32)
        if (p && !aligned(p, 4)) return fail(GDN_EINVAL, "fp32 arrays must be 4-byte aligned");
    const size_t sb = state32_bytes(s);
    const size_t hb = (size_t)s->H * 4;
    const Range in[] = {{h0, h0 ? sb : 0, "h0"}, {dhT, dhT ? sb : 0, "dhT"}, {D, D ? hb : 0, "D"}};
    const Range out[] = {{dA_log, hb, "dA_log"}, {dD, dD ? hb : 0, "dD"}, {dh0, dh0 ? sb : 0, "dh0"},
                         {hT, hT ? sb : 0, "hT"}};
    gdn_status_t e = check_aliasing(in, 3, out, 4);
    if (e != GDN_OK) return e;
    hipError_t he = gdn::launch_copy_or_zero(dA_log, nullptr, (size_t)s->H, st);
    if (he == hipSuccess && dD) he = gdn::launch_copy_or_zero(dD, nullptr, (size_t)s->H, st);
    if (he == hipSuccess && dh0) he = gdn::launch_copy_or_zero(dh0, dhT, sb / 4, st);
    if (he == hipSuccess && hT) he = gdn::launch_copy_or_zero(hT, h0, sb / 4, st);
    return hip_status(he, "gdn_bwd (empty sequence)");
}



namespace gdn {

gdn_status_t fwd_entry(const gdn_shape_t *s, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *A_log, const float *D, const float *h0, void *o, float *hT,
                       void *ctx,
                       void *ws, size_t ws_bytes, void *stream, bool one_stream,
                       gdn_status_t (*ws_lookup)(void *&ws)) {
    gdn_status_t st = check_shape(s);
    if (st != GDN_OK) return st;
    if (s->T == 0) return fwd_empty(s, h0, hT, (hipStream_t)stream);
    if (!q || !k || !v || !g || !beta || !A_log)
        return fail(GDN_EINVAL, "q, k, v, g, beta and A_log must not be NULL");
    const void *vec[] = {q, k, v, o};
    for (const void *p : vec)
        if (!aligned(p, 16)) return fail(GDN_EINVAL, "q, k, v, o must be 16-byte aligned");
    const void *f32[] = {g, beta, A_log, D, h0, hT};
    for (const void *p : f32)
        if (p && !aligned(p, 4)) return fail(GDN_EINVAL, "fp32 arrays must be 4-byte aligned");
    if (ctx && !aligned(ctx, 256)) return fail(GDN_EINVAL, "ctx must be 256-byte aligned");
    const size_t need = gdn_fwd_workspace_size(s);
    if (!ws_lookup) {
        if (!ws || ws_bytes < need)
            return fail(GDN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        if (!aligned(ws, 256)) return fail(GDN_EINVAL, "workspace must be 256-byte aligned");
    } else if (ws_bytes < need) {
        return fail(GDN_EWORKSPACE, "workspace of %zu bytes needed, %zu available", need, ws_bytes);
    }
    const size_t e = esize(s->dtype), BTH = (size_t)s->B * s->T * s->H;
    const size_t sb = (size_t)s->B * s->H * s->dk * s->dv * 4;
    const Range in[] = {{q, BTH * s->dk * e, "q"},     {k, BTH * s->dk * e, "k"}, {v, BTH * s->dv * e, "v"},
                        {g, BTH * 4, "g"},             {beta, BTH * 4, "beta"},   {A_log, (size_t)s->H * 4, "A_log"},
                        {h0, h0 ? sb : 0, "h0"},       {D, D ? (size_t)s->H * 4 : 0, "D"}};
    const Range out[] = {{o, BTH * s->dv * e, "o"},
                         {hT, hT ? sb : 0, "hT"},
                         {ctx, ctx ? ctx_bytes(s) : 0, "ctx"},
                         {ws, ws_lookup ? 0 : need, "workspace"}};
    st = check_aliasing(in, 8, out, 4);
    if (st != GDN_OK) return st;
    // a workspace the library owns is looked up only once the call is known
    // to be valid (its lookup is the first device call)
    if (ws_lookup && (st = ws_lookup(ws)) != GDN_OK) return st;
    const bool bf = s->dtype == GDN_BF16;
    const int Dp = pad_of(s);
    char *w = (char *)ws, *c = (char *)ctx;
    const CtxLayout cl = ctx_layout(s);
    void *U = ctx ? c + cl.u : w;
    void *NK = ctx ? c + cl.nk : w + align_up(blocks_bytes(s, s->dv));
    void *Tsave = ctx ? c + cl.t : nullptr;
    float *gam = (float *)(w + align_up(blocks_bytes(s, s->dv)) + align_up(blocks_bytes(s, s->dk)));
    float *hs = (float *)((char *)gam + align_up(gam_bytes(s)));
    float *scan = (float *)((char *)hs + align_up(state32_bytes(s)));
    const gdn::SeqArgs sa = seq(s, q, k, v, g, beta, A_log, D, h0);
    return hip_status(
        run_forward(s, sa, bf, Dp, U, NK, Tsave, gam, hs, scan, o, hT, ctx, (hipStream_t)stream, one_stream),
        "gdn_fwd launch");
}

gdn_status_t fail_detail(gdn_status_t st, const char *text) { return fail(st, "%s", text); }

} // namespace gdn

extern "C" {

gdn_status_t gdn_fwd(const gdn_shape_t *s, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *A_log, const float *D, const float *h0, void *o, float *hT,
                     void *ctx, void *ws, size_t ws_bytes, void *stream) {
    return gdn::fwd_entry(s, q, k, v, g, beta, A_log, D, h0, o, hT, ctx, ws, ws_bytes, stream, false, nullptr);
}

gdn_status_t gdn_bwd(const gdn_shape_t *s, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *A_log, const float *D, const float *h0, const void *ctx,
                     const void *dout, const float *dhT, void *dq, void *dk, void *dv, float *dg,
                     float *dbeta, float *dA_log, float *dD, float *dh0, float *hT, void *ws, size_t ws_bytes,
                     void *stream) {
    gdn_status_t st = check_shape(s);
    if (st != GDN_OK) return st;
    if (s->T == 0) return bwd_empty(s, D, h0, ctx, dhT, dA_log, dD, dh0, hT, (hipStream_t)stream);
    if (!q || !k || !v || !g || !beta || !A_log || !dout || !dq || !dk || !dv || !dg || !dbeta || !dA_log)
        return fail(GDN_EINVAL, "a required pointer is NULL");
    if (ctx && hT) return fail(GDN_EINVAL, "hT can only be recomputed when ctx is NULL");
    const bool bf = s->dtype == GDN_BF16;
    const int Dp = pad_of(s);
    if (!gdn::bwd_supported(bf, Dp))
        return fail(GDN_EUNSUPPORTED, "backward not built for %s with head dim %d", bf ? "bf16" : "fp32",
                    s->dk > s->dv ? s->dk : s->dv);
    const void *vec[] = {q, k, v, dout, dq, dk, dv};
    for (const void *p : vec)
        if (!aligned(p, 16)) return fail(GDN_EINVAL, "q, k, v, do, dq, dk, dv must be 16-byte aligned");
    const void *f32[] = {g, beta, A_log, D, h0, dhT, dg, dbeta, dA_log, dD, dh0, hT};
    for (const void *p : f32)
        if (p && !aligned(p, 4)) return fail(GDN_EINVAL, "fp32 arrays must be 4-byte aligned");
    if (ctx && !aligned(ctx, 256)) return fail(GDN_EINVAL, "ctx must be 256-byte aligned");
    const size_t need = gdn_bwd_workspace_size(s);
    if (!ws || ws_bytes < need)
        return fail(GDN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(GDN_EINVAL, "workspace must be 256-byte aligned");
    const size_t e = esize(s->dtype), BTH = (size_t)s->B * s->T * s->H;
    const size_t sb = (size_t)s->B * s->H * s->dk * s->dv * 4;
    const Range in[] = {{q, BTH * s->dk * e, "q"},
                        {k, BTH * s->dk * e, "k"},
                        {v, BTH * s->dv * e, "v"},
                        {g, BTH * 4, "g"},
                        {beta, BTH * 4, "beta"},
                        {A_log, (size_t)s->H * 4, "A_log"},
                        {h0, h0 ? sb : 0, "h0"},
                        {ctx, ctx ? ctx_bytes(s) : 0, "ctx"},
                        {dout, BTH * s->dv * e, "do"},
                        {dhT, dhT ? sb : 0, "dhT"},
                        {D, D ? (size_t)s->H * 4 : 0, "D"},
                        {ws, need, "workspace"}};
    const Range out[] = {{dq, BTH * s->dk * e, "dq"},       {dk, BTH * s->dk * e, "dk"},
                         {dv, BTH * s->dv * e, "dv"},       {dg, BTH * 4, "dg"},
                         {dbeta, BTH * 4, "dbeta"},         {dA_log, (size_t)s->H * 4, "dA_log"},
                         {dh0, dh0 ? sb : 0, "dh0"},        {hT, hT ? sb : 0, "hT"},
                         {dD, dD ? (size_t)s->H * 4 : 0, "dD"}};
    st = check_aliasing(in, 12, out, 9);
    if (st != GDN_OK) return st;

    hipStream_t strm = (hipStream_t)stream;
    char *w = (char *)ws;
    char *wctx = w;
    char *dhs = wctx + ctx_bytes(s);
    float *part = (float *)(dhs + align_up(states_bytes(s)));
    float *gam = (float *)((char *)part + align_up((size_t)s->B * s->H * nchunks(s) * sizeof(float)));
    float *hs = (float *)((char *)gam + align_up(gam_bytes(s)));
    float *wide = (float *)((char *)hs + align_up(state32_bytes(s)));
    const bool has_wide = gdn::bwd_wide_scratch_bytes(bf, Dp, s->B * s->H * nchunks(s)) > 0;
    float *scan = (float *)((char *)wide + align_up(gdn::bwd_wide_scratch_bytes(bf, Dp, s->B * s->H * nchunks(s))));
    float *dD_part = (float *)((char *)scan + scan_bytes(s));
    const gdn::SeqArgs sa = seq(s, q, k, v, g, beta, A_log, D, h0);
    const CtxLayout cl = ctx_layout(s);
    hipError_t he;
    if (!ctx) {
        he = run_forward(s, sa, bf, Dp, wctx + cl.u, wctx + cl.nk, wctx + cl.t, gam, hs, scan, nullptr, hT, wctx,
                         strm);
        if (he != hipSuccess) return hip_status(he, "gdn_bwd forward recompute launch");
        ctx = wctx;
    }
    const void *cs = ctx;
    const void *NK = (const char *)ctx + cl.nk;
    gdn::BwdChainArgs ca;
    ca.s = sa;
    ca.dout = dout;
    ca.dhT = dhT;
    ca.NK = NK;
    ca.dhs = dhs;
    ca.dh0 = dh0;
    const int nscan = scan_segments(s);
    const int BVc = gdn::bwd_chain_vblock(bf, Dp, nscan > 1);
    ca.NVB = (s->dv + BVc - 1) / BVc;
    if (nscan > 1) {
        // parallel scan, mirror of the forward's: the maps of every range but
        // the first, the gradient at the end of every range (from dhT
        // backwards), then every range at once
        ca.nseg = nscan;
        ca.mode = 1;
        ca.maps = scan;
        he = timed(K_BWD_CHAIN, [&] { return gdn::launch_bwd_chain(ca, bf, Dp, strm); }, strm);
        if (he != hipSuccess) return hip_status(he, "gdn_bwd chain (maps) launch");
        gdn::ScanArgs sc;
        sc.maps = scan;
        sc.h0 = dhT;
        sc.seg_h = scan + align_up(scan_maps_floats(s) * 4) / 4;
        sc.BH = s->B * s->H;
        sc.nseg = nscan;
        sc.dk = s->dk;
        sc.dv = s->dv;
        sc.reverse = 1;
        he = timed(K_BWD_SCAN, [&] { return gdn::launch_fwd_scan(sc, strm); }, strm);
        if (he != hipSuccess) return hip_status(he, "gdn_bwd scan launch");
        ca.mode = 0;
        ca.maps = nullptr;
        ca.seg_dh = sc.seg_h;
    }
    he = timed(K_BWD_CHAIN, [&] { return gdn::launch_bwd_chain(ca, bf, Dp, strm); }, strm);
    if (he != hipSuccess) return hip_status(he, "gdn_bwd chain launch");
    gdn::BwdLocalArgs la;
    la.s = sa;
    la.dout = dout;
    la.cs = cs;
    la.NK = NK;
    la.U = (const char *)ctx + cl.u;
    la.Tm = (const char *)ctx + cl.t;
    la.dhs = dhs;
    la.dq = dq;
    la.dk = dk;
    la.dv = dv;
    la.dg = dg;
    la.dbeta = dbeta;
    la.dA_part = part;
    la.dD_part = dD ? dD_part : nullptr;
    la.wide = has_wide ? wide : nullptr;
    he = timed(K_BWD_LOCAL, [&] { return gdn::launch_bwd_local(la, bf, Dp, strm); }, strm);
    if (he != hipSuccess) return hip_status(he, "gdn_bwd local launch");
    he = timed(K_DA_REDUCE, [&] { return gdn::launch_dA_reduce(part, dA_log, s->B, s->H, nchunks(s), strm); }, strm);
    if (he != hipSuccess || !dD) return hip_status(he, "gdn_bwd dA_log launch");
    // dD[h]: the [B][H][NC][DD_SLOTS] partial sums read as NC * DD_SLOTS
    // terms per (batch, head), the layout the dA_log reduction walks
    he = timed(K_DA_REDUCE,
               [&] { return gdn::launch_dA_reduce(dD_part, dD, s->B, s->H, nchunks(s) * gdn::DD_SLOTS, strm); }, strm);
    return hip_status(he, "gdn_bwd dD launch");
}

// S = 0: no token, so the state is carried over unchanged (h_out = h_in,
// zeros when h_in is NULL); the token arrays may be NULL
static gdn_status_t step_empty(int32_t N, int32_t H, int32_t dk, int32_t dv, const float *h_in, float *h_out,
                               hipStream_t st) {
    if (!h_out) return fail(GDN_EINVAL, "a required pointer is NULL");
    if ((h_in && !aligned(h_in, 4)) || !aligned(h_out, 4)) return fail(GDN_EINVAL, "pointers must be 4-byte aligned");
    const size_t sb = (size_t)N * H * dk * dv * 4;
    if (h_in == h_out) return GDN_OK;
    if (h_in && overlap(Range{h_in, sb, "h_in"}, Range{h_out, sb, "h_out"}))
        return fail(GDN_EINVAL, "h_in and h_out overlap without being equal");
    return hip_status(gdn::launch_copy_or_zero(h_out, h_in, sb / 4, st), "gdn_step_tokens (no token)");
}

gdn_status_t gdn_step_tokens(int32_t N, int32_t S, int32_t H, int32_t dk, int32_t dv, int32_t dtype,
                             uint32_t flags, const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *A_log, const float *D, const float *h_in,
                             float *h_out, void *o, void *stream) {
    if (N < 0 || H < 1 || S < 0) return fail(GDN_EINVAL, "N, S must be >= 0 and H >= 1");
    if (dk < 1 || dv < 1 || dk > 128 || dv > 128) return fail(GDN_EINVAL, "dk and dv must be in [1, 128]");
    if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_EINVAL, "unknown dtype %d", dtype);
    if (flags & ~KNOWN_FLAGS) return fail(GDN_EINVAL, "unknown flag bits 0x%x", flags);
    if ((double)N * H * dk * dv >= 2147483648.0 || (double)N * S * H * (dk > dv ? dk : dv) >= 2147483648.0)
        return fail(GDN_EINVAL, "state or tokens too large");
    if (N == 0) return GDN_OK; // no sequence: nothing to read or write
    if (S == 0) return step_empty(N, H, dk, dv, h_in, h_out, (hipStream_t)stream);
    if (!q || !k || !v || !g || !beta || !A_log || !h_out || !o)
        return fail(GDN_EINVAL, "a required pointer is NULL");
    const void *all[] = {q, k, v, o, g, beta, A_log, D, h_in, h_out};
    for (const void *p : all)
        if (p && !aligned(p, 4)) return fail(GDN_EINVAL, "pointers must be 4-byte aligned");
    const size_t e = esize(dtype), NSH = (size_t)N * S * H, sb = (size_t)N * H * dk * dv * 4;
    const Range in[] = {{q, NSH * dk * e, "q"},        {k, NSH * dk * e, "k"},     {v, NSH * dv * e, "v"},
                        {g, NSH * 4, "g"},             {beta, NSH * 4, "beta"},    {A_log, (size_t)H * 4, "A_log"},
                        {h_in == h_out ? nullptr : h_in, sb, "h_in"},
                        {D, D ? (size_t)H * 4 : 0, "D"}};
    const Range out[] = {{h_out, sb, "h_out"}, {o, NSH * dv * e, "o"}};
    gdn_status_t st = check_aliasing(in, 8, out, 2);
    if (st != GDN_OK) return st;
    if (h_in && h_in != h_out && overlap(Range{h_in, sb, "h_in"}, Range{h_out, sb, "h_out"}))
        return fail(GDN_EINVAL, "h_in and h_out overlap without being equal");
    gdn::StepArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.A_log = A_log;
    a.h_in = h_in;
    a.h_out = h_out;
    a.o = o;
    a.N = N;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.additive = (flags & GDN_FLAG_ADDITIVE) ? 1 : 0;
    a.logits = (flags & GDN_FLAG_GATE_LOGITS) ? 1 : 0;
    a.l2k = (flags & GDN_FLAG_L2NORM_K) ? 1 : 0;
    a.D = D;
    a.S = S;
    return hip_status(timed(K_STEP, [&] { return gdn::launch_step(a, dtype == GDN_BF16, (hipStream_t)stream); }, (hipStream_t)stream),
                      "gdn_step launch");
}

gdn_status_t gdn_step(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t dtype, uint32_t flags,
                      const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const float *A_log, const float *D, const float *h_in, float *h_out, void *o,
                      void *stream) {
    return gdn_step_tokens(N, 1, H, dk, dv, dtype, flags, q, k, v, g, beta, A_log, D, h_in, h_out, o, stream);
}

} // extern "C"
