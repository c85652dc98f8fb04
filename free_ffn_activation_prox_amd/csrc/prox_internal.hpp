// Host-side declarations shared by the Prox library's translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prox {

constexpr int kInt4Group = 128;
constexpr int kTileRowBytes = 128;   // bytes of one tile row of the proxy (one cache line)
constexpr int kMaxW2Total = 512;     // upper bound on Stage-2 blocks per launch (all tokens)
constexpr int kMaxS1Total = 512;     // upper bound on Stage-1 blocks per launch (all tokens)
constexpr int kPartChannels = 128;   // channels per partial-sum slot (the int4 tile width)
// Coarse histogram of the ranking keys that each Stage-2 block builds in LDS
// for its token: the bin of a key is its fp32 bit pattern >> 17 (keys are
// >= 0, so 14 bits: sign 0, exponent, 6 mantissa bits; 64 bins per binade).
constexpr int kGhShift = 17;
constexpr int kGhBins = 1 << (31 - kGhShift);
// Stage-2 LDS words holding the histogram (and 64 spare bins for keys past
// F), then the keys on their way from the coalesced load order to one run of
// PK per thread (NT runs of PK + 4 words), then (slow paths) every key of F.
inline __host__ __device__ int s2_keys_words(int F, int NT, int PK) {
    const int kw = (F + 64 + 3) & ~3;
    const int hw = kGhBins + 64;
    const int tw = NT * (PK + 4);
    const int m = kw > hw ? kw : hw;
    return m > tw ? m : tw;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// channels per proxy tile: int8 64, int4 128; exact mode (kind 3) has no
// proxy and pads the keys to 64 channels
inline int tile_channels(int kind) { return kind == 2 ? 128 : 64; }
inline int f_pad_of(int F, int kind) { return (int)align_up((size_t)F, (size_t)tile_channels(kind)); }

struct ProxyView {
    int kind;          // 1 int8, 2 int4
    int d, F, f_pad, groups;
    const uint8_t* codes;  // tile-major: [f_pad / tile_ch][d][128 B]
    const float* scales;   // gate [groups][f_pad] then up [groups][f_pad]
};

// Stage-2 blocks per token: about one block per compute unit over the batch.
inline int stage2_blocks_max(int batch) {
    int w = kMaxW2Total / batch;
    return w < 1 ? 1 : w;
}
inline int stage2_blocks(int batch, int k_ff, int n_cu) {
    int w = n_cu / batch;
    if (w > stage2_blocks_max(batch)) w = stage2_blocks_max(batch);
    if (w > k_ff) w = k_ff;
    return w < 1 ? 1 : w;
}

// Kept inputs per Stage-1 chunk (a multiple of 4).  Two chunks in flight
// per 8-lane slot: 4 rows put 64 KB in flight per compute unit, which
// measured faster than 8 or 12 rows (more requests only queue).
constexpr int kChunk = 4;

// Stage-1 work split: T = tiles * nch items (tile, chunk of kChunk kept
// inputs), nb1 blocks per token.
struct S1Geom {
    int tiles, nch, nb1;
};
inline int s1_blocks_max(int batch) {
    int w = kMaxS1Total / batch;
    return w < 1 ? 1 : w;
}
inline S1Geom s1_geom(int k_in, int F, int kind, int batch, int n_cu) {
    S1Geom g;
    g.tiles = f_pad_of(F, kind) / tile_channels(kind);
    g.nch = k_in > 0 ? (k_in + kChunk - 1) / kChunk : 1;
    int nb = n_cu / batch;
    if (nb > s1_blocks_max(batch)) nb = s1_blocks_max(batch);
    if (nb < 1) nb = 1;
    // int8 tiles are cheap enough per row to be bound by the stream: with no
    // more tiles than blocks each block takes one whole tile (no partial sums
    // to combine).  int4 rows cost more arithmetic per byte: its items are
    // spread over the blocks, in whole fractions of a tile when the tiles are
    // fewer than the blocks (no block then spans two tiles, so a block combines
    // split sums only at its end, never in the middle of its stream).
    if (kind == 1 && g.tiles < nb) nb = g.tiles;
    else if (g.tiles <= nb) nb = g.tiles * (nb / g.tiles);
    const long long T = (long long)g.tiles * g.nch;
    if (nb > T) nb = (int)T;
    g.nb1 = nb;
    return g;
}

// Batches of at least this many tokens take the matrix-core path (over the
// union of the tokens' rows and channels).  Measured crossover on the c3
// shape: at 4 tokens it takes 139 µs per layer against 158 µs for the
// per-token path, whose reads grow with every token.
constexpr int kBatchMin = 4;

// Row splits of the batched proxy GEMM (rows per split: whole 128-row groups).
struct PbSplit {
    int ks1, rps;
};
PbSplit proxy_batch_split(int d, int F, int kind);
// Channel slices of the batched down projection (chunk: rows per slice).
struct DnSplit {
    int KS, chunk;
};
DnSplit down_batch_split(int B, int d, int F);

// Workspace carve-up (byte offsets) for one (d, F, B, kind).  The batch
// regions (xm, bpart, bmask, hb) are empty below kBatchMin tokens.
struct WsLayout {
    size_t key, ypart, part, tcnt, xm, bpart, bmask, hb, hx, total;
};
inline WsLayout ws_layout(int d, int F, int B, int kind) {
    const int fp = f_pad_of(F, kind);
    const bool batch = B >= kBatchMin && kind != 3;   // exact mode runs the per-token kernels
    const size_t ks1 = batch ? (size_t)proxy_batch_split(d, F, kind).ks1 : 0;
    WsLayout L;
    size_t o = 0;
    L.key = o;    o = align_up(o + (size_t)B * fp * 4, 256);
    L.ypart = o;  o = align_up(o + (size_t)B * stage2_blocks_max(B) * d * 4, 256);
    L.part = o;   o = align_up(o + (size_t)B * (fp / tile_channels(kind) + s1_blocks_max(B)) * 2 * kPartChannels * 8, 256);
    L.tcnt = o;   o = align_up(o + (size_t)B * (fp / tile_channels(kind)) * 8, 256);
    L.xm = o;     o = align_up(o + (batch ? (size_t)B * d * 2 : 0), 256);
    L.bpart = o;  o = align_up(o + (ks1 > 1 ? ks1 * 2 * B * fp * 4 : 0), 256);
    L.bmask = o;  o = align_up(o + (batch ? (size_t)B * F : 0), 256);
    L.hb = o;     o = align_up(o + (batch ? (size_t)2 * B * fp * 2 : 0), 256);
    L.hx = o;     o = align_up(o + (kind == 3 ? (size_t)B * F * 8 : 0), 256);
    L.total = o;
    return L;
}

// Kernel-carried measurement events (event mode 1 of the taps), per host
// thread: while set, the next forward launch takes `start` at its start (and
// clears it) and every launch takes `stop` at its end, so after a phase the
// pair spans its first kernel's start to its last kernel's end.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents& launch_events() {
    static thread_local LaunchEvents e;
    return e;
}
// Every kernel of a forward is launched through here.
template <typename K, typename... Args>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
    LaunchEvents& e = launch_events();
    if (e.start || e.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, e.start, e.stop, 0u, args...);
        e.start = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
    }
}

// ---- launchers (prox_kernels.hip); all enqueue on `s` and return the launch status
hipError_t launch_build_proxy(const uint16_t* wg_t, const uint16_t* wu_t, int d, int F,
                              const ProxyView& p, hipStream_t s);
hipError_t launch_stage1(const uint16_t* x, int B, int d, int k_in, const ProxyView& p, float* key,
                         double* part, unsigned long long* tcnt, uint32_t gen,
                         const S1Geom& g, double* h_tap, float* key_tap, int32_t* in_idx_tap,
                         unsigned long long* tl, hipStream_t s);
// Stage 2 stream modes: 1 bf16 rows, 2 exact mode (h from hsrc [B][F], down
// rows only), 3 int8 rows (codes [F][d] each, qscale [3][F]).
hipError_t launch_stage2(const uint16_t* x, const void* wg_t, const void* wu_t, const void* wd, const float* key,
                         int B, int d, int F, int f_pad, int k_ff, int W2, int32_t* idx, uint8_t* mask, float* ypart,
                         int32_t* stream_tap, unsigned long long* tl, int mode, const double* hsrc,
                         const float* qscale, hipStream_t s);
hipError_t launch_reduce_y(const float* ypart, int B, int d, int W2, float* y, hipStream_t s);
// Stage-2 selection only: mask (required) and idx (nullable) from the keys.
hipError_t launch_select(const float* key, int B, int d, int F, int f_pad, int k_ff, int W2,
                         int32_t* idx, uint8_t* mask, hipStream_t s);

// Quantized Stage-2 weights: codes [3][F][d] int8, scales [3][F] fp32.
hipError_t launch_build_qweights(const uint16_t* wg_t, const uint16_t* wu_t, const uint16_t* wd, int d, int F,
                                 int8_t* codes, float* scales, hipStream_t s);

// ---- exact mode and diagnostics (prox_exact.hip)
hipError_t launch_exact_h(const uint16_t* x, int B, int d, const uint16_t* wg_t, const uint16_t* wu_t, int F,
                          int f_pad, int nb, float* key, double* hbuf, double* h_tap, float* key_tap,
                          int32_t* in_idx_tap, unsigned long long* tl, hipStream_t s);
hipError_t launch_quality(const uint8_t* ma, const uint8_t* mb, int B, int F, const float* y, const float* yr, int d,
                          int32_t* overlap, double* err, hipStream_t s);

// ---- batch launchers (prox_batch.hip)
hipError_t launch_xsel(const uint16_t* x, int B, int d, int k_in, uint16_t* xm, int32_t* in_idx,
                       hipStream_t s);
hipError_t launch_proxy_batch(const uint16_t* xm, int B, int d, const ProxyView& p, float* part,
                              unsigned long long* tcnt, uint32_t gen, float* key, double* h_tap,
                              float* key_tap, hipStream_t s);
// Gate/up and down over the tokens' masks; *ks_out = partial slices in ypart.
hipError_t launch_stage2_batch(const uint16_t* x, const uint16_t* wg_t, const uint16_t* wu_t,
                               const uint16_t* wd, const uint8_t* mask, uint16_t* hb, int B, int d,
                               int F, int f_pad, float* ypart, int* ks_out, hipStream_t s);

}  // namespace prox
