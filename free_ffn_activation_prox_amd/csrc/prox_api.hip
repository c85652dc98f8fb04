// Prox C ABI: host-side validation, workspace carve-up and launch sequence.
// Every check runs before the first launch, so an error return enqueues nothing.
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
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

bool kind_ok(int kind) { return kind == PROX_PROXY_INT8 || kind == PROX_PROXY_INT4_G128; }

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
    return ws_layout(d, F, batch, kind).total;
}

extern "C" prox_status prox_build_proxy(const prox_weights* w, int32_t kind, void* buf,
                                        size_t buf_bytes, prox_proxy* out, void* stream) {
    g_err.clear();
    if (!w || !out || !buf) return fail(PROX_E_INVALID, "null weights, output descriptor or buffer");
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
    hipError_t e = launch_build_proxy(static_cast<const uint16_t*>(w->w_gate_t),
                                      static_cast<const uint16_t*>(w->w_up_t), w->d_model,
                                      w->d_ff, view_of(&p), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "proxy build launch");
    *out = p;
    return PROX_OK;
}

extern "C" prox_status prox_ffn_forward_taps(const void* x, int32_t batch, const prox_weights* w,
                                             const prox_proxy* p, int32_t k_in, int32_t k_ff,
                                             float* y, uint8_t* mask, int32_t* idx,
                                             void* workspace, size_t ws_bytes,
                                             const prox_taps* taps, void* stream) {
    g_err.clear();
    if (!x || !w || !p || !y || !workspace)
        return fail(PROX_E_INVALID, "null x, weights, proxy, y or workspace");
    if (!w->w_gate_t || !w->w_up_t || !w->w_down || !p->buf)
        return fail(PROX_E_INVALID, "null weight or proxy buffer");
    const int d = w->d_model, F = w->d_ff;
    if (const char* e = shape_error(d, F, p->kind)) return fail(PROX_E_INVALID, "%s", e);
    if (const char* e = limit_error(d, F)) return fail(PROX_E_UNSUPPORTED, "%s", e);
    if (batch < 1) return fail(PROX_E_INVALID, "batch must be >= 1");
    if (batch > PROX_MAX_BATCH) return fail(PROX_E_UNSUPPORTED, "batch above PROX_MAX_BATCH");
    if (k_in < 0 || k_in > d) return fail(PROX_E_INVALID, "k_in out of [0, d_model]");
    if (k_ff < 0 || k_ff > F) return fail(PROX_E_INVALID, "k_ff out of [0, d_ff]");
    if (p->d_model != d || p->d_ff != F) return fail(PROX_E_MISMATCH, "proxy shape differs from weights");
    const ProxyGeom g = proxy_geom(d, F, p->kind);
    if (p->f_pad != g.f_pad || p->groups != g.groups || p->tile_ch != g.tile_ch || p->row_stride != g.row_stride ||
        p->scale_offset != g.scale_offset || p->bytes != g.bytes)
        return fail(PROX_E_MISMATCH, "proxy descriptor is not the one prox_build_proxy writes");
    if (!aligned(x, 16) || !aligned(w->w_gate_t, 16) || !aligned(w->w_up_t, 16) ||
        !aligned(w->w_down, 16) || !aligned(y, 16) || !aligned(p->buf, 256))
        return fail(PROX_E_INVALID, "misaligned x, weights, y or proxy");
    if (!aligned(workspace, 256)) return fail(PROX_E_INVALID, "workspace must be 256-byte aligned");
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

    void* const* ev = (taps && taps->events && taps->n_events >= PROX_N_PHASES + 1) ? taps->events : nullptr;
    auto mark = [&](int i) -> hipError_t {
        return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
    };

    hipError_t e = mark(0);
    if (e != hipSuccess) return hip_fail(e, "event record");
    unsigned long long* tcnt = reinterpret_cast<unsigned long long*>(ws + L.tcnt);
    const uint16_t* wg = static_cast<const uint16_t*>(w->w_gate_t);
    const uint16_t* wu = static_cast<const uint16_t*>(w->w_up_t);
    const uint16_t* wd = static_cast<const uint16_t*>(w->w_down);

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
                      taps ? taps->in_idx : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "stage 1");
    if ((e = mark(1 + PROX_PHASE_STAGE1)) != hipSuccess) return hip_fail(e, "event record");
    e = launch_stage2(xb, wg, wu, wd, key, batch, d, F, g.f_pad, k_ff, W2, idx, mask, ypart, s);
    if (e != hipSuccess) return hip_fail(e, "stage 2");
    if ((e = mark(1 + PROX_PHASE_STAGE2)) != hipSuccess) return hip_fail(e, "event record");
    e = launch_reduce_y(ypart, batch, d, W2, y, s);
    if (e != hipSuccess) return hip_fail(e, "reduce y");
    if ((e = mark(1 + PROX_PHASE_REDUCE_Y)) != hipSuccess) return hip_fail(e, "event record");
    return PROX_OK;
}

extern "C" prox_status prox_ffn_forward(const void* x, int32_t batch, const prox_weights* w,
                                        const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                        uint8_t* mask, int32_t* idx, void* workspace,
                                        size_t ws_bytes, void* stream) {
    return prox_ffn_forward_taps(x, batch, w, p, k_in, k_ff, y, mask, idx, workspace, ws_bytes,
                                 nullptr, stream);
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
