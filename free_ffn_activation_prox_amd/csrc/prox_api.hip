// Prox C ABI: host-side validation, workspace carve-up and launch sequence.
// Every check runs before the first launch, so an error return enqueues nothing.
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "prox.h"
#include "prox_internal.hpp"

using namespace prox;

namespace {

thread_local std::string g_err;

prox_status fail(prox_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

prox_status hip_fail(hipError_t e, const char* where) {
    return fail(PROX_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool kind_ok(int kind) {
    return kind == PROX_PROXY_INT8 || kind == PROX_PROXY_INT4_G128 || kind == PROX_PROXY_EXACT_BF16;
}

const char* shape_error(int d, int F, int kind) {
    if (!kind_ok(kind)) return "unknown proxy kind";
    if (d < 8 || d % 8) return "d_model must be a positive multiple of 8";
    if (F < 1) return "d_ff must be >= 1";
    if (kind == PROX_PROXY_INT4_G128 && d % kInt4Group) return "int4 group-128 proxy needs d_model % 128 == 0";
    return nullptr;
}

const char* limit_error(int d, int F) {
    if (d > PROX_MAX_D_MODEL) return "d_model above PROX_MAX_D_MODEL";
    if (F > PROX_MAX_D_FF) return "d_ff above PROX_MAX_D_FF";
    return nullptr;
}

struct ProxyGeom {
    int f_pad, groups, tile_ch;
    size_t row_stride, scale_offset, bytes;
};

ProxyGeom proxy_geom(int d, int F, int kind) {
    ProxyGeom g;
    g.tile_ch = tile_channels(kind);
    g.f_pad = f_pad_of(F, kind);
    if (kind == PROX_PROXY_EXACT_BF16) {      // no proxy: the weights rank themselves
        g.groups = 0;
        g.row_stride = g.scale_offset = g.bytes = 0;
        return g;
    }
    g.groups = kind == PROX_PROXY_INT8 ? 1 : d / kInt4Group;
    g.row_stride = kTileRowBytes;
    const size_t codes = (size_t)(g.f_pad / g.tile_ch) * d * kTileRowBytes;
    g.scale_offset = align_up(codes, 256);
    g.bytes = g.scale_offset + (size_t)2 * g.groups * g.f_pad * sizeof(float);
    return g;
}

ProxyView view_of(const prox_proxy* p) {
    ProxyView v;
    v.kind = p->kind;
    v.d = p->d_model;
    v.F = p->d_ff;
    v.f_pad = p->f_pad;
    v.groups = p->groups;
    v.codes = static_cast<const uint8_t*>(p->buf);
    v.scales = reinterpret_cast<const float*>(static_cast<const uint8_t*>(p->buf) + p->scale_offset);
    return v;
}

// Compute units of the current device (cached per device id).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// A tag per call for the Stage-1 arrival counters: counters left by any
// earlier call (this process or another, or never cleared) carry another tag.
uint32_t next_call_tag() {
    static std::atomic<uint32_t> tag{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
    return tag.fetch_add(1u, std::memory_order_relaxed);
}

}  // namespace

extern "C" int32_t prox_abi_version(void) { return PROX_ABI_VERSION; }

extern "C" size_t prox_proxy_bytes(int32_t d, int32_t F, int32_t kind) {
    if (shape_error(d, F, kind) || limit_error(d, F)) return 0;
    return proxy_geom(d, F, kind).bytes;
}

extern "C" size_t prox_workspace_bytes(int32_t d, int32_t F, int32_t batch, int32_t kind) {
    if (shape_error(d, F, kind) || limit_error(d, F)) return 0;
    if (batch < 1 || batch > PROX_MAX_BATCH) return 0;
    return ws_layout(d, F, batch < PROX_CHUNK_BATCH ? batch : PROX_CHUNK_BATCH, kind).total;
}

extern "C" prox_status prox_build_proxy(const prox_weights* w, int32_t kind, void* buf,
                                        size_t buf_bytes, prox_proxy* out, void* stream) {
    g_err.clear();
    if (!w || !out) return fail(PROX_E_INVALID, "null weights or output descriptor");
    if (!buf && kind != PROX_PROXY_EXACT_BF16) return fail(PROX_E_INVALID, "null proxy buffer");
    if (!w->w_gate_t || !w->w_up_t) return fail(PROX_E_INVALID, "null w_gate_t or w_up_t");
    if (const char* e = shape_error(w->d_model, w->d_ff, kind)) return fail(PROX_E_INVALID, "%s", e);
    if (const char* e = limit_error(w->d_model, w->d_ff)) return fail(PROX_E_UNSUPPORTED, "%s", e);
    if (!aligned(buf, 256)) return fail(PROX_E_INVALID, "proxy buffer must be 256-byte aligned");
    if (!aligned(w->w_gate_t, 16) || !aligned(w->w_up_t, 16))
        return fail(PROX_E_INVALID, "weights must be 16-byte aligned");
    const ProxyGeom g = proxy_geom(w->d_model, w->d_ff, kind);
    if (buf_bytes < g.bytes)
        return fail(PROX_E_INVALID, "proxy buffer too small: %zu < %zu", buf_bytes, g.bytes);
    prox_proxy p{};
    p.kind = kind;
    p.d_model = w->d_model;
    p.d_ff = w->d_ff;
    p.f_pad = g.f_pad;
    p.groups = g.groups;
    p.tile_ch = g.tile_ch;
    p.row_stride = g.row_stride;
    p.scale_offset = g.scale_offset;
    p.bytes = g.bytes;
    p.buf = buf;
    if (kind == PROX_PROXY_EXACT_BF16) {      // nothing to build
        *out = p;
        return PROX_OK;
    }
    hipError_t e = launch_build_proxy(static_cast<const uint16_t*>(w->w_gate_t),
                                      static_cast<const uint16_t*>(w->w_up_t), w->d_model,
                                      w->d_ff, view_of(&p), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "proxy build launch");
    *out = p;
    return PROX_OK;
}

namespace {

// Stage-2 rows of one forward: bf16 [F][d] each (qscale null), or int8 [F][d]
// each with their row scales qscale [3][F] (quantized Stage-2 weights).
struct S2Rows {
    const void* g;
    const void* u;
    const void* dn;
    const float* qscale;
};

prox_status forward_impl(const void* x, int32_t batch, int d, int F, const S2Rows& rows, const prox_proxy* p,
                         int32_t k_in, int32_t k_ff, float* y, uint8_t* mask, int32_t* idx, void* workspace,
                         size_t ws_bytes, const prox_taps* taps, void* stream) {
    if (!x || !p || !y || !workspace) return fail(PROX_E_INVALID, "null x, proxy, y or workspace");
    if (!p->buf && p->kind != PROX_PROXY_EXACT_BF16) return fail(PROX_E_INVALID, "null proxy buffer");
    if (const char* e = shape_error(d, F, p->kind)) return fail(PROX_E_INVALID, "%s", e);
    if (const char* e = limit_error(d, F)) return fail(PROX_E_UNSUPPORTED, "%s", e);
    if (batch < 1) return fail(PROX_E_INVALID, "batch must be >= 1");
    if (batch > PROX_MAX_BATCH) return fail(PROX_E_UNSUPPORTED, "batch above PROX_MAX_BATCH");
    if (k_in < 0 || k_in > d) return fail(PROX_E_INVALID, "k_in out of [0, d_model]");
    if (k_ff < 0 || k_ff > F) return fail(PROX_E_INVALID, "k_ff out of [0, d_ff]");
    if (p->kind == PROX_PROXY_EXACT_BF16 && k_in != d)
        return fail(PROX_E_INVALID, "exact mode keeps every input: k_in must equal d_model");
    if (p->kind == PROX_PROXY_EXACT_BF16 && rows.qscale)
        return fail(PROX_E_UNSUPPORTED, "exact mode computes h from the bf16 weights: no quantized Stage 2");
    if (p->d_model != d || p->d_ff != F) return fail(PROX_E_MISMATCH, "proxy shape differs from weights");
    const ProxyGeom g = proxy_geom(d, F, p->kind);
    if (p->f_pad != g.f_pad || p->groups != g.groups || p->tile_ch != g.tile_ch || p->row_stride != g.row_stride ||
        p->scale_offset != g.scale_offset || p->bytes != g.bytes)
        return fail(PROX_E_MISMATCH, "proxy descriptor is not the one prox_build_proxy writes");
    if (!aligned(x, 16) || !aligned(y, 16) || (p->kind != PROX_PROXY_EXACT_BF16 && !aligned(p->buf, 256)))
        return fail(PROX_E_INVALID, "misaligned x, y or proxy");
    if (!aligned(workspace, 256)) return fail(PROX_E_INVALID, "workspace must be 256-byte aligned");
    if (batch > PROX_CHUNK_BATCH) {
        // prefill: consecutive sub-batches, each a forward of its own over the
        // same workspace (stream order keeps them apart); taps per token
        // follow the sub-batch, the phase events time the last one
        const WsLayout Lc = ws_layout(d, F, PROX_CHUNK_BATCH, p->kind);
        if (ws_bytes < Lc.total) return fail(PROX_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, Lc.total);
        void* const* ev = (taps && taps->events && taps->event_mode == 0 && taps->n_events >= PROX_N_PHASES + 1)
                              ? taps->events : nullptr;
        if (ev) {
            hipError_t e = hipEventRecord((hipEvent_t)ev[0], (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "event record");
        }
        for (int c0 = 0; c0 < batch; c0 += PROX_CHUNK_BATCH) {
            const int nb = batch - c0 < PROX_CHUNK_BATCH ? batch - c0 : PROX_CHUNK_BATCH;
            const bool last = c0 + nb == batch;
            prox_taps t{};
            const prox_taps* tp = nullptr;
            if (taps) {
                t.in_idx = taps->in_idx ? taps->in_idx + (size_t)c0 * k_in : nullptr;
                t.key = taps->key ? taps->key + (size_t)c0 * F : nullptr;
                t.h_hat = taps->h_hat ? taps->h_hat + (size_t)c0 * F : nullptr;
                t.stream_idx = taps->stream_idx ? taps->stream_idx + (size_t)c0 * k_ff : nullptr;
                t.events = last ? taps->events : nullptr;
                t.n_events = last ? taps->n_events : 0;
                t.event_mode = taps->event_mode;
                tp = &t;
            }
            const prox_status st = forward_impl(static_cast<const uint16_t*>(x) + (size_t)c0 * d, nb, d, F, rows, p,
                                                k_in, k_ff, y + (size_t)c0 * d,
                                                mask ? mask + (size_t)c0 * F : nullptr,
                                                idx ? idx + (size_t)c0 * k_ff : nullptr, workspace, ws_bytes, tp,
                                                stream);
            if (st != PROX_OK) return st;
        }
        return PROX_OK;
    }
    const WsLayout L = ws_layout(d, F, batch, p->kind);
    if (ws_bytes < L.total) return fail(PROX_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);

    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const ProxyView pv = view_of(p);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    float* key = reinterpret_cast<float*>(ws + L.key);
    float* ypart = reinterpret_cast<float*>(ws + L.ypart);
    const int n_cu = device_cus();
    // per-token path: Stage-2 blocks on every compute unit up to d_model 4096,
    // on three quarters of them above (measured, µs per token: c2_s70 44.8 at
    // 256 blocks against 45.2 at 192; c4_b1_s70 152.3 at 192 against 153.8 at
    // 256, whose longer rows keep more bytes in flight per block)
    const int W2 = stage2_blocks(batch, k_ff, batch >= kBatchMin || d <= 4096 ? n_cu : n_cu * 3 / 4);

    // measurement events: mode 0 records events[i] on the stream at phase
    // boundary i; mode 1 hands phase i's pair (events[2i], events[2i + 1]) to
    // its kernels' launches (the guard clears them on every return)
    const int emode = taps ? taps->event_mode : 0;
    void* const* ev = (taps && taps->events && emode == 0 && taps->n_events >= PROX_N_PHASES + 1) ? taps->events
                                                                                                  : nullptr;
    void* const* kev = (taps && taps->events && emode == 1 && taps->n_events >= 2 * PROX_N_PHASES) ? taps->events
                                                                                                   : nullptr;
    struct EventsGuard {
        ~EventsGuard() { launch_events() = LaunchEvents{}; }
    } events_guard;
    auto mark = [&](int i) -> hipError_t {
        if (kev) {
            launch_events() = i < PROX_N_PHASES ? LaunchEvents{(hipEvent_t)kev[2 * i], (hipEvent_t)kev[2 * i + 1]}
                                                : LaunchEvents{};
            return hipSuccess;
        }
        return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
    };

    hipError_t e = mark(0);
    if (e != hipSuccess) return hip_fail(e, "event record");
    unsigned long long* tcnt = reinterpret_cast<unsigned long long*>(ws + L.tcnt);
    const uint16_t* wg = static_cast<const uint16_t*>(rows.g);
    const uint16_t* wu = static_cast<const uint16_t*>(rows.u);
    const uint16_t* wd = static_cast<const uint16_t*>(rows.dn);

    if (p->kind == PROX_PROXY_EXACT_BF16) {
        // exact mode: h of every channel (fp64), then the selection and the
        // W_down rows of the kept channels with h read back; per-token
        // kernels for any batch
        double* hx = reinterpret_cast<double*>(ws + L.hx);
        const int nb = n_cu / batch > 0 ? n_cu / batch : 1;
        const int W2x = stage2_blocks(batch, k_ff, d <= 4096 ? n_cu : n_cu * 3 / 4);
        unsigned long long* tl = taps ? (unsigned long long*)taps->timeline : nullptr;
        e = launch_exact_h(xb, batch, d, wg, wu, F, g.f_pad, nb, key, hx, taps ? taps->h_hat : nullptr,
                           taps ? taps->key : nullptr, taps ? taps->in_idx : nullptr, tl, s);
        if (e != hipSuccess) return hip_fail(e, "exact stage 1");
        if ((e = mark(1 + PROX_PHASE_STAGE1)) != hipSuccess) return hip_fail(e, "event record");
        e = launch_stage2(xb, wg, wu, wd, key, batch, d, F, g.f_pad, k_ff, W2x, idx, mask, ypart,
                          taps ? taps->stream_idx : nullptr, tl, 2, hx, nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "exact stage 2");
        if ((e = mark(1 + PROX_PHASE_STAGE2)) != hipSuccess) return hip_fail(e, "event record");
        e = launch_reduce_y(ypart, batch, d, W2x, y, s);
        if (e != hipSuccess) return hip_fail(e, "reduce y");
        if ((e = mark(1 + PROX_PHASE_REDUCE_Y)) != hipSuccess) return hip_fail(e, "event record");
        return PROX_OK;
    }

    if (rows.qscale) {
        // quantized Stage-2 weights: Stage 1 as for the bf16 rows (the
        // matrix-core proxy GEMM from kBatchMin tokens), Stage 2 with the
        // per-token kernel streaming int8 rows for every batch
        if (batch >= kBatchMin) {
            uint16_t* xm = reinterpret_cast<uint16_t*>(ws + L.xm);
            e = launch_xsel(xb, batch, d, k_in, xm, taps ? taps->in_idx : nullptr, s);
            if (e != hipSuccess) return hip_fail(e, "input selection");
            e = launch_proxy_batch(xm, batch, d, pv, reinterpret_cast<float*>(ws + L.bpart), tcnt, next_call_tag(),
                                   key, taps ? taps->h_hat : nullptr, taps ? taps->key : nullptr, s);
            if (e != hipSuccess) return hip_fail(e, "proxy GEMM");
        } else {
            const S1Geom g1 = s1_geom(k_in, F, p->kind, batch, n_cu);
            e = launch_stage1(xb, batch, d, k_in, pv, key, reinterpret_cast<double*>(ws + L.part), tcnt,
                              next_call_tag(), g1, taps ? taps->h_hat : nullptr, taps ? taps->key : nullptr,
                              taps ? taps->in_idx : nullptr, taps ? (unsigned long long*)taps->timeline : nullptr, s);
            if (e != hipSuccess) return hip_fail(e, "stage 1");
        }
        if ((e = mark(1 + PROX_PHASE_STAGE1)) != hipSuccess) return hip_fail(e, "event record");
        const int W2q = stage2_blocks(batch, k_ff, d <= 4096 ? n_cu : n_cu * 3 / 4);
        e = launch_stage2(xb, rows.g, rows.u, rows.dn, key, batch, d, F, g.f_pad, k_ff, W2q, idx, mask, ypart,
                          taps ? taps->stream_idx : nullptr, taps ? (unsigned long long*)taps->timeline : nullptr, 3,
                          nullptr, rows.qscale, s);
        if (e != hipSuccess) return hip_fail(e, "stage 2 (int8 rows)");
        if ((e = mark(1 + PROX_PHASE_STAGE2)) != hipSuccess) return hip_fail(e, "event record");
        e = launch_reduce_y(ypart, batch, d, W2q, y, s);
        if (e != hipSuccess) return hip_fail(e, "reduce y");
        if ((e = mark(1 + PROX_PHASE_REDUCE_Y)) != hipSuccess) return hip_fail(e, "event record");
        return PROX_OK;
    }

    if (batch >= kBatchMin) {
        // matrix-core path: input selection and proxy GEMM over the batch,
        // per-token channel selection, gate/up and down over the tokens' masks
        uint16_t* xm = reinterpret_cast<uint16_t*>(ws + L.xm);
        uint8_t* bmask = mask ? mask : ws + L.bmask;
        uint16_t* hb = reinterpret_cast<uint16_t*>(ws + L.hb);
        e = launch_xsel(xb, batch, d, k_in, xm, taps ? taps->in_idx : nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "input selection");
        e = launch_proxy_batch(xm, batch, d, pv, reinterpret_cast<float*>(ws + L.bpart), tcnt, next_call_tag(),
                               key, taps ? taps->h_hat : nullptr, taps ? taps->key : nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "proxy GEMM");
        if ((e = mark(1 + PROX_PHASE_STAGE1)) != hipSuccess) return hip_fail(e, "event record");
        e = launch_select(key, batch, d, F, g.f_pad, k_ff, W2, idx, bmask, s);
        if (e != hipSuccess) return hip_fail(e, "channel selection");
        int ks = 0;
        e = launch_stage2_batch(xb, wg, wu, wd, bmask, hb, batch, d, F, g.f_pad, ypart, &ks, s);
        if (e != hipSuccess) return hip_fail(e, "stage 2 (batch)");
        if ((e = mark(1 + PROX_PHASE_STAGE2)) != hipSuccess) return hip_fail(e, "event record");
        e = launch_reduce_y(ypart, batch, d, ks, y, s);
        if (e != hipSuccess) return hip_fail(e, "reduce y");
        if ((e = mark(1 + PROX_PHASE_REDUCE_Y)) != hipSuccess) return hip_fail(e, "event record");
        return PROX_OK;
    }

    const S1Geom g1 = s1_geom(k_in, F, p->kind, batch, n_cu);
    double* part = reinterpret_cast<double*>(ws + L.part);
    e = launch_stage1(xb, batch, d, k_in, pv, key, part, tcnt, next_call_tag(), g1,
                      taps ? taps->h_hat : nullptr, taps ? taps->key : nullptr,
                      taps ? taps->in_idx : nullptr, taps ? (unsigned long long*)taps->timeline : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "stage 1");
    if ((e = mark(1 + PROX_PHASE_STAGE1)) != hipSuccess) return hip_fail(e, "event record");
    e = launch_stage2(xb, wg, wu, wd, key, batch, d, F, g.f_pad, k_ff, W2, idx, mask, ypart,
                      taps ? taps->stream_idx : nullptr, taps ? (unsigned long long*)taps->timeline : nullptr, 1,
                      nullptr, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "stage 2");
    if ((e = mark(1 + PROX_PHASE_STAGE2)) != hipSuccess) return hip_fail(e, "event record");
    e = launch_reduce_y(ypart, batch, d, W2, y, s);
    if (e != hipSuccess) return hip_fail(e, "reduce y");
    if ((e = mark(1 + PROX_PHASE_REDUCE_Y)) != hipSuccess) return hip_fail(e, "event record");
    return PROX_OK;
}

}  // namespace

extern "C" prox_status prox_ffn_forward_taps(const void* x, int32_t batch, const prox_weights* w,
                                             const prox_proxy* p, int32_t k_in, int32_t k_ff,
                                             float* y, uint8_t* mask, int32_t* idx,
                                             void* workspace, size_t ws_bytes,
                                             const prox_taps* taps, void* stream) {
    g_err.clear();
    if (!w) return fail(PROX_E_INVALID, "null weights");
    if (!w->w_gate_t || !w->w_up_t || !w->w_down) return fail(PROX_E_INVALID, "null weight buffer");
    if (!aligned(w->w_gate_t, 16) || !aligned(w->w_up_t, 16) || !aligned(w->w_down, 16))
        return fail(PROX_E_INVALID, "misaligned weights");
    const S2Rows rows{w->w_gate_t, w->w_up_t, w->w_down, nullptr};
    return forward_impl(x, batch, w->d_model, w->d_ff, rows, p, k_in, k_ff, y, mask, idx, workspace, ws_bytes,
                        taps, stream);
}

// ---------------------------------------------------------------------------
// Quantized Stage-2 weights.
// ---------------------------------------------------------------------------
namespace {
size_t qweights_scale_offset(int d, int F) { return align_up((size_t)3 * F * d, 256); }
}  // namespace

extern "C" size_t prox_qweights_bytes(int32_t d, int32_t F) {
    if (shape_error(d, F, PROX_PROXY_INT8) || limit_error(d, F)) return 0;
    return qweights_scale_offset(d, F) + (size_t)3 * F * sizeof(float);
}

extern "C" prox_status prox_build_qweights(const prox_weights* w, void* buf, size_t buf_bytes, prox_qweights* out,
                                           void* stream) {
    g_err.clear();
    if (!w || !buf || !out) return fail(PROX_E_INVALID, "null weights, buffer or output descriptor");
    if (!w->w_gate_t || !w->w_up_t || !w->w_down) return fail(PROX_E_INVALID, "null weight buffer");
    const int d = w->d_model, F = w->d_ff;
    if (const char* e = shape_error(d, F, PROX_PROXY_INT8)) return fail(PROX_E_INVALID, "%s", e);
    if (const char* e = limit_error(d, F)) return fail(PROX_E_UNSUPPORTED, "%s", e);
    if (!aligned(buf, 256)) return fail(PROX_E_INVALID, "buffer must be 256-byte aligned");
    if (!aligned(w->w_gate_t, 16) || !aligned(w->w_up_t, 16) || !aligned(w->w_down, 16))
        return fail(PROX_E_INVALID, "misaligned weights");
    const size_t need = prox_qweights_bytes(d, F);
    if (buf_bytes < need) return fail(PROX_E_INVALID, "buffer too small: %zu < %zu", buf_bytes, need);
    prox_qweights q{};
    q.d_model = d;
    q.d_ff = F;
    q.scale_offset = qweights_scale_offset(d, F);
    q.bytes = need;
    q.buf = buf;
    uint8_t* b = static_cast<uint8_t*>(buf);
    hipError_t e = launch_build_qweights(static_cast<const uint16_t*>(w->w_gate_t),
                                         static_cast<const uint16_t*>(w->w_up_t),
                                         static_cast<const uint16_t*>(w->w_down), d, F, reinterpret_cast<int8_t*>(b),
                                         reinterpret_cast<float*>(b + q.scale_offset), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quantized weights build launch");
    *out = q;
    return PROX_OK;
}

extern "C" prox_status prox_ffn_forward_q8(const void* x, int32_t batch, const prox_qweights* q, const prox_proxy* p,
                                           int32_t k_in, int32_t k_ff, float* y, uint8_t* mask, int32_t* idx,
                                           void* workspace, size_t ws_bytes, const prox_taps* taps, void* stream) {
    g_err.clear();
    if (!q || !q->buf) return fail(PROX_E_INVALID, "null quantized weights");
    const int d = q->d_model, F = q->d_ff;
    if (const char* e = shape_error(d, F, PROX_PROXY_INT8)) return fail(PROX_E_INVALID, "%s", e);
    if (q->scale_offset != qweights_scale_offset(d, F) || q->bytes != prox_qweights_bytes(d, F) ||
        !aligned(q->buf, 256))
        return fail(PROX_E_MISMATCH, "quantized-weights descriptor is not the one prox_build_qweights writes");
    const uint8_t* b = static_cast<const uint8_t*>(q->buf);
    const size_t m = (size_t)F * d;
    const S2Rows rows{b, b + m, b + 2 * m, reinterpret_cast<const float*>(b + q->scale_offset)};
    return forward_impl(x, batch, d, F, rows, p, k_in, k_ff, y, mask, idx, workspace, ws_bytes, taps, stream);
}

extern "C" prox_status prox_ffn_forward(const void* x, int32_t batch, const prox_weights* w,
                                        const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                        uint8_t* mask, int32_t* idx, void* workspace,
                                        size_t ws_bytes, void* stream) {
    return prox_ffn_forward_taps(x, batch, w, p, k_in, k_ff, y, mask, idx, workspace, ws_bytes,
                                 nullptr, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is a fixed device array of this
// library, one copy per GPU, held until the process ends.  Its address on the
// current device comes from hipGetSymbolAddress the first time a call runs on
// that device (the array's name in host code is not a device address).
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = PROX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of `scratch` on the current device, or null (error set).
void* scratch_on_current_device(prox_status* st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *st = hip_fail(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *st = fail(PROX_E_UNSUPPORTED, "device id %d above the %d devices this library tracks", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *st = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t prox_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" prox_status prox_ffn_forward_noalloc(const void* x, int32_t batch, const prox_weights* w,
                                                const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                                uint8_t* mask, int32_t* idx, void* stream) {
    g_err.clear();
    if (!w || !p) return fail(PROX_E_INVALID, "null weights or proxy");
    const size_t need = prox_workspace_bytes(w->d_model, w->d_ff, batch, p->kind);
    if (need > kScratchBytes)
        return fail(PROX_E_UNSUPPORTED, "this shape needs a %zu-byte workspace, above the %zu-byte scratch of the "
                    "allocation-free forward; use prox_ffn_forward with a caller workspace", need, kScratchBytes);
    prox_status st = PROX_OK;
    void* ws = scratch_on_current_device(&st);
    if (!ws) return st;
    // need == 0 (invalid shape or batch): prox_ffn_forward_taps reports it
    return prox_ffn_forward_taps(x, batch, w, p, k_in, k_ff, y, mask, idx, ws, kScratchBytes, nullptr, stream);
}

extern "C" prox_status prox_quality(const uint8_t* mask_a, const uint8_t* mask_b, int32_t batch, int32_t d_ff,
                                    const float* y, const float* y_ref, int32_t d_model, int32_t* overlap,
                                    double* err, void* stream) {
    g_err.clear();
    if (batch < 1 || d_ff < 1 || d_model < 1) return fail(PROX_E_INVALID, "batch, d_ff and d_model must be >= 1");
    if ((!mask_a) != (!mask_b) || (!mask_a) != (!overlap))
        return fail(PROX_E_INVALID, "mask_a, mask_b and overlap must all be given or all be null");
    if ((!y) != (!y_ref) || (!y) != (!err))
        return fail(PROX_E_INVALID, "y, y_ref and err must all be given or all be null");
    if (!mask_a && !y) return fail(PROX_E_INVALID, "nothing to compare");
    hipError_t e = launch_quality(mask_a, mask_b, batch, d_ff, y, y_ref, d_model, overlap, err, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quality");
    return PROX_OK;
}

extern "C" const char* prox_status_str(int32_t st) {
    switch (st) {
        case PROX_OK: return "PROX_OK";
        case PROX_E_INVALID: return "PROX_E_INVALID";
        case PROX_E_UNSUPPORTED: return "PROX_E_UNSUPPORTED";
        case PROX_E_MISMATCH: return "PROX_E_MISMATCH";
        case PROX_E_WORKSPACE: return "PROX_E_WORKSPACE";
        case PROX_E_HIP: return "PROX_E_HIP";
        default: return "PROX_E_UNKNOWN";
    }
}

extern "C" const char* prox_last_error(void) { return g_err.c_str(); }
