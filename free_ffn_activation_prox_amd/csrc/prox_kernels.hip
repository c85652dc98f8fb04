// Prox sparse SwiGLU FFN: gfx950 kernels of the single-token path (fewer than
// 4 tokens per call) and the one-time proxy build.
//
// One forward = three launches (Prox, Abstract; SwiGLU as in PrunePath, §2.1, Eq. (1)):
//   k_stage1  per (block, token): input selection (top-k_in of |x|, redone in
//             every block: x is a few KB), the block's share of the (channel
//             tile, kept-row chunk) items of the proxy GEMV, and for every
//             tile the block completes: h~ = silu(g~) u~ in fp64 and the fp32
//             ranking key |h~|
//   k_stage2  per (block, token): top-k of the keys (threshold bin from a
//             coarse LDS histogram, redone in every block), the block's share
//             of the kept channels, then for each of them the exact gate/up
//             dots over the dense x, h = silu(g) u and h * W_down row into the
//             block's partial y
//   k_reduce_y  y = fixed-order sum of the block partials
//
// Proxy layout (tile-major): the codes of one channel tile (64 channels int8,
// 128 channels int4) for input row i are one 128-byte line at
// (tile * d + i) * 128, so a block streams only the kept rows of its tile and
// every row it touches is exactly one cache line.
#include "prox_device.hpp"
#include "prox_internal.hpp"

namespace prox {

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
// Signed fields by shifts.  (__builtin_amdgcn_sbfe converted to double was
// lowered here as an unsigned conversion, so negative fields came out as
// ~4e9: every signed field below is extracted this way.)
__device__ __forceinline__ int sext8(uint32_t w, int c) { return (int)(w << (24 - 8 * c)) >> 24; }
__device__ __forceinline__ int sext4(uint32_t w, int c) { return (int)(w << (28 - 4 * c)) >> 28; }

// code = clamp(round-half-even(fp32(w / s)), -qmax, qmax); 0 when s == 0.
// The quotient is formed in fp64 and rounded once to fp32: for fp32 operands an
// fp64 quotient rounded to fp32 equals the correctly rounded fp32 quotient
// (53 >= 2 * 24 + 2), independent of fast-division compiler settings.
__device__ __forceinline__ int quant_code(float w, float s, float qmax) {
    if (!(s > 0.f)) return 0;
    float r = (float)((double)w / (double)s);
    float q = rintf(r);
    q = fminf(fmaxf(q, -qmax), qmax);
    return (int)q;
}

// ---------------------------------------------------------------------------
// Proxy build: scales.  grid (f_pad / 4, groups, 2), block 256: one wave per
// (channel, group, matrix); max |w| over the group, s = fp32(max / qmax).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_quant_scales(const uint16_t* __restrict__ wg_t,
                                                      const uint16_t* __restrict__ wu_t, int d,
                                                      int F, int f_pad, int groups, float qmax,
                                                      float* __restrict__ scales) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + wave;
    const int g = blockIdx.y, mat = blockIdx.z;
    if (j >= f_pad) return;
    const uint16_t* w = mat == 0 ? wg_t : wu_t;
    const int gs = d / groups;
    float amax = 0.f;
    if (j < F) {
        const uint16_t* row = w + (size_t)j * d + (size_t)g * gs;
        for (int i = lane; i < gs; i += kWave) amax = fmaxf(amax, fabsf(bf16_to_f32(row[i])));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if (lane == 0) {
        float s = (float)((double)amax / (double)qmax);
        scales[((size_t)mat * groups + g) * f_pad + j] = (j < F) ? s : 0.f;
    }
}

// Proxy build: codes.  grid (ceil(d / 256), f_pad / CB), block 256: thread = (input i,
// block of CB channels: 8 for int8, 16 for int4); reads W^T[j][i] (coalesced over
// i) and writes one 16-byte code block into the tile-major layout.
template <int KIND>
__global__ void __launch_bounds__(256) k_quant_codes(const uint16_t* __restrict__ wg_t,
                                                     const uint16_t* __restrict__ wu_t, int d,
                                                     int F, int f_pad, int groups,
                                                     const float* __restrict__ scales,
                                                     uint8_t* __restrict__ codes) {
    constexpr int CB = KIND == 1 ? 8 : 16;
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int cb = blockIdx.y;
    if (i >= d) return;
    const int g = i / (d / groups);
    const float qmax = KIND == 1 ? 127.f : 7.f;
    uint32_t pg[2] = {0, 0}, pu[2] = {0, 0};
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int j = cb * CB + c;
        float wgv = 0.f, wuv = 0.f;
        if (j < F) {
            wgv = bf16_to_f32(wg_t[(size_t)j * d + i]);
            wuv = bf16_to_f32(wu_t[(size_t)j * d + i]);
        }
        const int qg = quant_code(wgv, scales[(size_t)g * f_pad + j], qmax);
        const int qu = quant_code(wuv, scales[((size_t)groups + g) * f_pad + j], qmax);
        if (KIND == 1) {
            pg[c >> 2] |= (uint32_t)(qg & 0xff) << (8 * (c & 3));
            pu[c >> 2] |= (uint32_t)(qu & 0xff) << (8 * (c & 3));
        } else {
            pg[c >> 3] |= (uint32_t)(qg & 0xf) << (4 * (c & 7));
            pu[c >> 3] |= (uint32_t)(qu & 0xf) << (4 * (c & 7));
        }
    }
    const int tile = cb / 8, lb = cb % 8;
    uint4 v = make_uint4(pg[0], pg[1], pu[0], pu[1]);
    *reinterpret_cast<uint4*>(codes + ((size_t)tile * d + i) * kTileRowBytes + lb * 16) = v;
}

hipError_t launch_build_proxy(const uint16_t* wg_t, const uint16_t* wu_t, int d, int F,
                              const ProxyView& p, hipStream_t s) {
    float* scales = const_cast<float*>(p.scales);
    const float qmax = p.kind == 1 ? 127.f : 7.f;
    hipLaunchKernelGGL(k_quant_scales, dim3(p.f_pad / 4, p.groups, 2), dim3(256), 0, s, wg_t,
                       wu_t, d, F, p.f_pad, p.groups, qmax, scales);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint8_t* codes = const_cast<uint8_t*>(p.codes);
    if (p.kind == 1)
        hipLaunchKernelGGL(k_quant_codes<1>, dim3((d + 255) / 256, p.f_pad / 8), dim3(256), 0, s,
                           wg_t, wu_t, d, F, p.f_pad, p.groups, p.scales, codes);
    else
        hipLaunchKernelGGL(k_quant_codes<2>, dim3((d + 255) / 256, p.f_pad / 16), dim3(256), 0, s,
                           wg_t, wu_t, d, F, p.f_pad, p.groups, p.scales, codes);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantized Stage-2 weights: int8 codes of every row of W_gate^T, W_up^T and
// W_down, one fp32 scale per row (the proxy's rule: s = fp32(max|row| / 127),
// code = clamp(round-half-even(fp32(w / s)), -127, 127)).
// Scales: grid (ceil(F / 4), 3), block 256, one wave per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_qrow_scales(const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                                                     const uint16_t* __restrict__ w2, int d, int F,
                                                     float* __restrict__ scales) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + wave, m = blockIdx.y;
    if (j >= F) return;
    const uint16_t* row = (m == 0 ? w0 : (m == 1 ? w1 : w2)) + (size_t)j * d;
    float amax = 0.f;
    for (int i = lane; i < d; i += kWave) amax = fmaxf(amax, fabsf(bf16_to_f32(row[i])));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if (lane == 0) scales[(size_t)m * F + j] = (float)((double)amax / 127.0);
}

// Codes: grid (ceil(F * d / 8 / 256), 3), block 256; thread = 8 consecutive
// weights of one row (16 bytes in, 8 bytes out).
__global__ void __launch_bounds__(256) k_qrow_codes(const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                                                    const uint16_t* __restrict__ w2, int d, int F,
                                                    const float* __restrict__ scales, int8_t* __restrict__ codes) {
    const size_t n8 = (size_t)F * d / 8;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (e >= n8) return;
    const uint16_t* w = m == 0 ? w0 : (m == 1 ? w1 : w2);
    const size_t i0 = e * 8;
    const int j = (int)(i0 / d);
    const float s = scales[(size_t)m * F + j];
    const uint4 v = *reinterpret_cast<const uint4*>(w + i0);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float f = __uint_as_float(k & 1 ? (wd[k >> 1] & 0xffff0000u) : (wd[k >> 1] << 16));
        out[k >> 2] |= (uint32_t)(quant_code(f, s, 127.f) & 0xff) << (8 * (k & 3));
    }
    *reinterpret_cast<uint2*>(codes + (size_t)m * F * d + i0) = make_uint2(out[0], out[1]);
}

hipError_t launch_build_qweights(const uint16_t* wg_t, const uint16_t* wu_t, const uint16_t* wd, int d, int F,
                                 int8_t* codes, float* scales, hipStream_t s) {
    hipLaunchKernelGGL(k_qrow_scales, dim3((F + 3) / 4, 3), dim3(256), 0, s, wg_t, wu_t, wd, d, F, scales);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n8 = (size_t)F * d / 8;
    hipLaunchKernelGGL(k_qrow_codes, dim3((unsigned)((n8 + 255) / 256), 3), dim3(256), 0, s, wg_t, wu_t, wd, d, F,
                       scales, codes);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 1.  grid (NB1, B), block 512 (8 waves).
//
// Work items: (tile, chunk) pairs, tile-major, chunk = kChunk consecutive entries
// of the token's kept-input list.  int8 with no more tiles than blocks: one
// whole tile per block.  Otherwise block w takes items [w*T/NB1, (w+1)*T/NB1)
// of the T = tiles * nch items, so every compute unit streams the same number
// of proxy rows whatever the tile count; a tile split between blocks has its
// segment sums added, in block order, by the block that completes it.
//
// Input selection: thread t holds x[t*PX .. t*PX + PX - 1]; keys are the 15
// magnitude bits of the bf16 value (monotone in |x|, -0 == +0).  The list in
// LDS holds (index << 16 | bf16 bits) of the kept inputs: first those whose
// exponent is at most 5 above the threshold's, then the larger ones, each in
// index order (the GEMV sums over the list, so only the set matters).
//
// GEMV: row slot s (= 8 * wave + lane / 8, 64 slots) takes the segment's chunks
// s, s + 64, ...; lane % 8 picks a 16-byte block of the tile row (int8: 8 gate
// + 8 up codes; int4: 16 + 16).  int8 chunks whose x span at most 5 binades
// accumulate exactly in fp32 (see consume_chunk_i8) and the chunk sum is added
// to the fp64 accumulator; other chunks accumulate in fp64 directly.  int4
// accumulates in fp64 and scales each 128-input group's inner sum when the
// group changes.  The slots are reduced with lane shuffles and LDS in a fixed
// order, so the result is deterministic.
// ---------------------------------------------------------------------------
struct Stage1Args {
    const uint16_t* x;
    int d, k_in;
    ProxyView p;
    float* key;          // [B][f_pad]
    double* part;        // [B][tiles + nb1][2][128] segment partial sums
    unsigned long long* tcnt;   // [B][tiles] arrival counters: call tag << 32 | arrivals
    double* h_tap;       // [B][F] or null
    float* key_tap;      // [B][F] or null
    int32_t* in_idx_tap; // [B][k_in] or null
    int tiles, nch, nb1;
    uint32_t gen;        // tag of this call, distinct from earlier calls
    unsigned long long* tl;   // timeline stamps or null
};

constexpr int kS1Threads = 512;
// byte flags of the chunks after the kept-input list (k_in + 64 words) in the
// dynamic LDS: word offset
__host__ __device__ __forceinline__ int s1_flags_off(int k_in) { return (k_in + 64 + 3) & ~3; }
// int4: the group table after the flags, 16-byte aligned (word offset)
__host__ __device__ __forceinline__ int s1_table_off(int k_in) {
    return (s1_flags_off(k_in) + ((k_in + 3) / 4 + 16 + 3) / 4 + 3) & ~3;
}
constexpr int kSlots = 64;

// Items [i0, i1) of block w: i0 = w * T / nb1.  The block holding item i is the
// largest w with i0(w) <= i.  The segment of (tile, block) is stored at
// slot tile + block: along the tile-major item order both never decrease and
// at least one grows, so the slots are distinct and below tiles + nb1.
// (32-bit arithmetic: T = tiles * nch <= 512 * 4096 and nb1 <= 512 keep
// every product below 2^31.)
__device__ __forceinline__ int s1_item0(int w, int T, int nb1) { return split_point(w, T, nb1); }
__device__ __forceinline__ int s1_block_of(int i, int T, int nb1) {
    return (int)(((uint32_t)(i + 1) * (uint32_t)nb1 - 1u) / (uint32_t)T);
}


// h~ = silu(g~) u~ in fp64 (int8: per-channel scales applied here) and the
// fp32 ranking key |h~|.
__device__ __forceinline__ void stage1_score(const Stage1Args& a, int b, int j, double g, double u,
                                             float sg, float su) {
    if (j >= a.p.F) return;
    if (a.p.kind == 1) {
        g *= (double)sg;
        u *= (double)su;
    }
    const double h = g / (1.0 + exp(-g)) * u;
    const float kf = (float)fabs(h);
    a.key[(size_t)b * a.p.f_pad + j] = kf;
    if (a.h_tap) a.h_tap[(size_t)b * a.p.F + j] = h;
    if (a.key_tap) a.key_tap[(size_t)b * a.p.F + j] = kf;
}

// One chunk of <= kChunk kept rows for one lane: the packed list entries and the
// lane's 16-byte block of each tile row (buffer loads: tile offset scalar,
// row and block offset per lane).  Entries past the segment or the list read
// as x = 0 at an offset past the end of the codes, which the hardware returns
// as zeros without a memory access; the loads are unconditional so they stay
// in flight.
struct Chunk {
    uint32_t e[kChunk];
    uint4 v[kChunk];
    bool exact;          // x of the chunk span at most 5 binades, none subnormal
};

__device__ __forceinline__ void load_chunk(const uint32_t* list, const uint8_t* exact, int k_in, int ch,
                                           int ch_end, __amdgpu_buffer_rsrc_t codes, uint32_t codes_bytes,
                                           uint32_t tile_off, uint32_t lane_off, Chunk& c) {
    const int r0 = ch * kChunk;
    const int n = ch < ch_end ? min(kChunk, k_in - r0) : 0;
    // the entries in 16-byte LDS reads (a chunk past the list reads the
    // first entries, all masked; the list has 64 spare words past k_in)
    const int rr = n > 0 ? r0 : 0;
    uint32_t ev[kChunk];
#pragma unroll
    for (int g = 0; g < kChunk; g += 4) {
        const uint4 e4 = *reinterpret_cast<const uint4*>(list + rr + g);
        ev[g] = e4.x; ev[g + 1] = e4.y; ev[g + 2] = e4.z; ev[g + 3] = e4.w;
    }
    c.exact = n > 0 ? exact[ch] != 0 : true;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
        c.e[u] = u < n ? ev[u] : 0u;
        const uint32_t off = u < n ? (ev[u] >> 16) * (uint32_t)kTileRowBytes + lane_off : codes_bytes;
        c.v[u] = buf_load16(codes, off, tile_off);
    }
}

// 1 when the chunk's nonzero x span at most 5 binades and none is subnormal.
__device__ __forceinline__ bool chunk_exact32(const Chunk& c) {
    int lo = 255, hi = 0;
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
        const uint32_t r = c.e[u];
        const int e = (int)((r >> 7) & 0xffu);
        const bool zero = (r & 0x7fffu) == 0;       // +-0 contributes exactly 0
        ok = ok && (zero || e != 0);                 // subnormal x: take the fp64 path
        lo = zero ? lo : min(lo, e);
        hi = zero ? hi : max(hi, e);
    }
    return ok && hi - lo <= 5;
}

// Input selection.  Fills `list` with the k_in kept inputs: band B (exponent
// within e_lo .. e_lo + 5, e_lo = the threshold's exponent, not subnormal)
// first, then band A (the rest), each in index order; sc[16] = the band-B
// count, sc[17] = max(e_lo, 1).  Keys are 15 bits: a 2048-bin histogram of
// key >> 4 finds the threshold bin, a 16-bin histogram of the low 4 bits of
// the keys in that bin finds the threshold T itself (every thread scans those
// 16 bins), and one packed scan of (keys > T, keys == T) places every kept
// input, the first k_in - #(> T) keys equal to T in index order.  LDS: hist
// >= 2048 + 16 + 64 words.
template <int PX>
__device__ __forceinline__ void stage1_select(const Stage1Args& a, int b, uint32_t* list, uint32_t* hist, int* sc) {
    constexpr int NT = kS1Threads;
    const int t = threadIdx.x, lane = t & 63;
    const int d = a.d, k_in = a.k_in;
    uint32_t raw[PX];
    int key[PX];
    {
        bool valid[PX];
        load_u16_contig<PX>(a.x + (size_t)b * d, d, d, raw, valid);
#pragma unroll
        for (int q = 0; q < PX; ++q) key[q] = valid[q] ? (int)(raw[q] & 0x7fffu) : -1;   // past d: below every key
    }
    const bool all = k_in >= d;
    int T = -1, cgt = 0;                                   // keep-all: every valid key is above T
    if (!all && k_in > 0) {
        uint32_t* hist2 = hist + 2048;
        for (int i = t; i < 2048 + 16; i += NT) hist[i] = 0u;
        lds_barrier();
#pragma unroll
        for (int q = 0; q < PX; ++q) atomicAdd(&hist[key[q] >= 0 ? (key[q] >> 4) : 2048 + 16], 1u);
        lds_barrier();
        tl_mark(a.tl, 0, 4);
        uint32_t tb;
        static_assert(NT * 4 == 2048, "one 16-byte read of 4 bins per thread");
        find_bin4<NT>(hist, k_in, sc, tb, cgt);
#pragma unroll
        for (int q = 0; q < PX; ++q)
            if (key[q] >= 0 && (key[q] >> 4) == (int)tb) atomicAdd(&hist2[key[q] & 15], 1u);
        lds_barrier();
        // every thread: the 16 low-bit bins in four 16-byte reads, then the
        // same answer from registers
        uint32_t h16[16];
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
            const uint4 u = *reinterpret_cast<const uint4*>(hist2 + v);
            h16[v] = u.x; h16[v + 1] = u.y; h16[v + 2] = u.z; h16[v + 3] = u.w;
        }
        int cum = cgt;
        T = (int)(tb << 4);
        bool found = false;
#pragma unroll
        for (int v = 15; v >= 0; --v) {
            const int c = (int)h16[v];
            if (!found && cum + c >= k_in) {
                T = (int)(tb << 4) + v;
                found = true;
            }
            cum += found ? 0 : c;
        }
        cgt = cum;                                         // keys > T
    }
    tl_mark(a.tl, 0, 5);
    const int need = all ? 0 : k_in - cgt;                 // keys equal to T to keep
    int gt = 0, eq = 0;
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        gt += key[q] > T ? 1 : 0;
        eq += (key[q] == T && !all) ? 1 : 0;
    }
    uint32_t tot;
    // fewer than k_in <= 2^15 keys exceed T (keep-all: at most d keys, unpacked)
    const uint32_t pre = block_excl_scan_u32<NT>(all ? (uint32_t)gt : (((uint32_t)gt << 16) | (uint32_t)eq), sc, tot);
    // Which keys are kept, and the list order.  The kept inputs whose
    // exponent is at most 5 above the threshold's ("band B") come first, the
    // larger ones after, each part in index order: chunks of band B span at
    // most 5 binades, so they take the exact fp32 path, and a few large
    // outlier inputs cannot push whole chunks onto the fp64 path.
    bool on[PX];
    {
        int eb = all ? 0 : (int)(pre & 0xffffu);
        int pos = all ? (int)pre : (int)(pre >> 16) + min(eb, need);
#pragma unroll
        for (int q = 0; q < PX; ++q) {
            const bool e = key[q] == T && !all;
            on[q] = k_in > 0 && (key[q] > T || (e && eb < need));
            if (on[q] && a.in_idx_tap && blockIdx.x == 0) a.in_idx_tap[(size_t)b * k_in + pos] = t * PX + q;
            eb += e ? 1 : 0;
            pos += on[q] ? 1 : 0;
        }
    }
    // e_lo: the threshold's exponent (keep-all: the smallest exponent of a
    // normal input); band B = exponents e_lo .. e_lo + 5, band A = larger
    // exponents and subnormal inputs
    int e_lo = (T >> 7) & 0xff;
    if (all) {
        int m = 0;
#pragma unroll
        for (int q = 0; q < PX; ++q) {
            const int e = (key[q] >> 7) & 0xff;
            m = key[q] > 0 && e > 0 ? max(m, 255 - e) : m;
        }
        e_lo = 255 - block_max<NT>(m, sc);
    }
    const int e_hi = e_lo + 5;
    auto band_a = [&](int kq) {
        const int e = (kq >> 7) & 0xff;
        return e > e_hi || (e == 0 && (kq & 0x7f) != 0);
    };
    int nb = 0, na = 0;
#pragma unroll
    for (int q = 0; q < PX; ++q) {
        const bool big = band_a(key[q]);
        nb += on[q] && !big ? 1 : 0;
        na += on[q] && big ? 1 : 0;
    }
    uint32_t tot2;
    tl_mark(a.tl, 0, 6);
    const uint32_t pre2 = block_excl_scan_u32<NT>(((uint32_t)nb << 16) | (uint32_t)na, sc, tot2);
    if (k_in > 0) {
        int pb = (int)(pre2 >> 16), pa = (int)((uint32_t)tot2 >> 16) + (int)(pre2 & 0xffffu);
        uint32_t* dummy = list + k_in + lane;              // lanes with nothing to write
#pragma unroll
        for (int q = 0; q < PX; ++q) {
            const bool big = band_a(key[q]);
            *(on[q] ? list + (big ? pa : pb) : dummy) = ((uint32_t)(t * PX + q) << 16) | raw[q];
            pb += on[q] && !big ? 1 : 0;
            pa += on[q] && big ? 1 : 0;
        }
    }
    if (t == 0) {
        sc[16] = (int)(tot2 >> 16);                        // band-B entries (the list's first ones)
        sc[17] = max(e_lo, 1);                             // band B's unit exponent
    }
    lds_barrier();
}

// Each chunk's exactness flag (entries past k_in are empty), into LDS after
// the list.  The caller issues its first chunk loads before this and holds a
// barrier after it.
__device__ __forceinline__ void stage1_flags(const uint32_t* list, int k_in) {
    uint8_t* exact = reinterpret_cast<uint8_t*>(const_cast<uint32_t*>(list) + s1_flags_off(k_in));
    const int nch = (k_in + kChunk - 1) / kChunk;
    for (int ch = threadIdx.x; ch < nch; ch += kS1Threads) {
        Chunk c;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) c.e[u] = ch * kChunk + u < k_in ? list[ch * kChunk + u] : 0u;
        exact[ch] = chunk_exact32(c) ? 1 : 0;
    }
}

// Unsigned byte c of w as float (one conversion instruction).
__device__ __forceinline__ float ubyte_f(uint32_t w, int c) { return (float)((w >> (8 * c)) & 0xffu); }

// int8 chunk: 8 gate + 8 up channels of the lane.  Exact fp32 path: with the
// code bytes flipped by 0x80 each byte reads as q + 128 in [1, 255], so
// sum x*q = sum x*(q + 128) - 128 * sum x.  When the chunk's x span at most 5
// binades every x is an integer below 2^13 in units of 2^(e_lo - 7), every
// product below 2^21 and every partial sum below 2^24: all steps are exact,
// and so is the final difference (its value is the exact sum x*q).
__device__ __forceinline__ void consume_chunk_i8(const Chunk& c, double (&ag)[8], double (&au)[8]) {
    if (c.exact) {
        float sg[8], su[8], sx = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) sg[q] = su[q] = 0.f;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float xf = bf16f(c.e[u] & 0xffffu);
            sx += xf;
            const uint32_t gx = c.v[u].x ^ 0x80808080u, gy = c.v[u].y ^ 0x80808080u;
            const uint32_t ux = c.v[u].z ^ 0x80808080u, uy = c.v[u].w ^ 0x80808080u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sg[q] = fmaf(xf, ubyte_f(gx, q), sg[q]);
                sg[q + 4] = fmaf(xf, ubyte_f(gy, q), sg[q + 4]);
                su[q] = fmaf(xf, ubyte_f(ux, q), su[q]);
                su[q + 4] = fmaf(xf, ubyte_f(uy, q), su[q + 4]);
            }
        }
        const float corr = 128.f * sx;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            ag[q] += (double)(sg[q] - corr);
            au[q] += (double)(su[q] - corr);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const double xd = (double)bf16f(c.e[u] & 0xffffu);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ag[q] = fma(xd, (double)sext8(c.v[u].x, q), ag[q]);
                ag[q + 4] = fma(xd, (double)sext8(c.v[u].y, q), ag[q + 4]);
                au[q] = fma(xd, (double)sext8(c.v[u].z, q), au[q]);
                au[q + 4] = fma(xd, (double)sext8(c.v[u].w, q), au[q + 4]);
            }
        }
    }
}

// int4 chunk: 16 gate + 16 up channels of the lane; the inner sums of a
// 128-input group are scaled into og/ou when the row's group changes.
// int4: g~ = sum over groups of s_group * (sum over the group's rows of x q).
// A chunk whose x exponents span at most 5 binades sums its 8 products per
// channel exactly in fp32 (x has 8 significant bits, |q| <= 8, 8 terms: every
// partial sum is an integer below 2^21 in units of the smallest product's
// last bit); the sum is scaled in fp64 into the lane's totals.  Other chunks
// add x q s row by row in fp64 (x q is exact).  `sg`, `su` hold the current
// group's scales of the lane's 16 channels; they are reloaded when the group
// changes, which is rare because a slot takes consecutive kept rows.
struct I4State {
    int cur;
    float sg[16], su[16];
};

__device__ __forceinline__ void i4_set_group(I4State& st, int g, const float* sgp, const float* sup, int f_pad) {
    const float4* s4g = reinterpret_cast<const float4*>(sgp + (size_t)g * f_pad);
    const float4* s4u = reinterpret_cast<const float4*>(sup + (size_t)g * f_pad);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 fg = s4g[q], fu = s4u[q];
        st.sg[4 * q] = fg.x; st.sg[4 * q + 1] = fg.y; st.sg[4 * q + 2] = fg.z; st.sg[4 * q + 3] = fg.w;
        st.su[4 * q] = fu.x; st.su[4 * q + 1] = fu.y; st.su[4 * q + 2] = fu.z; st.su[4 * q + 3] = fu.w;
    }
    st.cur = g;
}

__device__ __forceinline__ void i4_flush(const I4State& st, float (&pg)[16], float (&pu)[16], double (&og)[16],
                                         double (&ou)[16]) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        og[q] = fma((double)pg[q], (double)st.sg[q], og[q]);
        ou[q] = fma((double)pu[q], (double)st.su[q], ou[q]);
        pg[q] = pu[q] = 0.f;
    }
}

__device__ __forceinline__ void consume_chunk_i4(const Chunk& c, const float* sgp, const float* sup, int f_pad,
                                                 I4State& st, double (&og)[16], double (&ou)[16]) {
    if (c.exact) {
        float pg[16], pu[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) pg[q] = pu[q] = 0.f;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            // an empty entry (past the run: x = 0, reads zeros) keeps the group
            const int g = c.e[u] ? (int)(c.e[u] >> 16) >> 7 : st.cur;
            if (g != st.cur) {
                if (st.cur >= 0) i4_flush(st, pg, pu, og, ou);
                i4_set_group(st, g, sgp, sup, f_pad);
            }
            const float xf = bf16f(c.e[u] & 0xffffu);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                pg[q] = fmaf(xf, (float)sext4(c.v[u].x, q), pg[q]);
                pg[q + 8] = fmaf(xf, (float)sext4(c.v[u].y, q), pg[q + 8]);
                pu[q] = fmaf(xf, (float)sext4(c.v[u].z, q), pu[q]);
                pu[q + 8] = fmaf(xf, (float)sext4(c.v[u].w, q), pu[q + 8]);
            }
        }
        if (st.cur >= 0) i4_flush(st, pg, pu, og, ou);
    } else {
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int g = c.e[u] ? (int)(c.e[u] >> 16) >> 7 : st.cur;
            if (g != st.cur) i4_set_group(st, g, sgp, sup, f_pad);
            if (st.cur < 0) continue;   // nothing kept yet: every entry is empty
            const float xf = bf16f(c.e[u] & 0xffffu);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // x q is exact in fp32 (8 + 4 significant bits)
                og[q] = fma((double)(xf * (float)sext4(c.v[u].x, q)), (double)st.sg[q], og[q]);
                og[q + 8] = fma((double)(xf * (float)sext4(c.v[u].y, q)), (double)st.sg[q + 8], og[q + 8]);
                ou[q] = fma((double)(xf * (float)sext4(c.v[u].z, q)), (double)st.su[q], ou[q]);
                ou[q + 8] = fma((double)(xf * (float)sext4(c.v[u].w, q)), (double)st.su[q + 8], ou[q + 8]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// int4 tile segment: kept-list entries [e0, e1) of one 128-channel tile.
//
// Band-B entries (the list's first nbB, index order): 16 lanes per kept row,
// lane (block bk, matrix m) reading the 8 bytes that hold the 16 codes of
// matrix m for channels 16 bk .. 16 bk + 15; a slot of 16 lanes streams a
// contiguous run of the segment's rows with kI4Ring rows in flight.  With
// every nibble flipped by 8 a code reads as q + 8 in 0..15, the nibbles split
// into bytes convert with one instruction each, and sum x q = sum x (q + 8) -
// 8 sum x.  Band-B inputs lie in the six binades e_u .. e_u + 5, so in units
// of 2^(e_u - 134) every x is an integer below 2^13, every x (q + 8) below
// 2^17 and every sum over one 128-row group below 2^24: the fp32 sums are
// exact.  When its run leaves a group a lane turns its sums into integers in
// those units and adds them to the group's row of an LDS table (integer adds:
// exact in any order).  After the stream thread t < 256 (matrix t / 128,
// channel t % 128) forms the sum over groups of s_group times the table entry
// in fp64, groups in ascending order.  The table holds kI4Win groups; a
// segment spanning more is taken kI4Win groups at a time.
//
// Band-A entries (larger or subnormal inputs, few) are summed in fp64 by the
// same 256 threads, x q exact in fp32 times the group scale, in list order.
// Returns, for t < 256, the segment's sum for the thread's (matrix, channel).
// ---------------------------------------------------------------------------
constexpr int kI4Ring = 8;
constexpr int kI4Win = 32;
constexpr int kI4TableWords = kI4Win * 256;

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_uint2(v.x, v.y);
}

// First entry in [lo, hi) whose row lies in group >= g (entries ascending).
__device__ __forceinline__ int i4_group_start(const uint32_t* list, int lo, int hi, int g) {
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)(list[mid] >> 23) < g) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void i4_flush(float (&pg)[16], float& sx, int gw, int m, int bk, int eu, int* table) {
    if (gw >= 0 && gw < kI4Win) {
        int* row = table + gw * 256 + m * 128 + 16 * bk;
#pragma unroll
        for (int c = 0; c < 16; ++c) atomicAdd(row + c, (int)ldexpf(pg[c] - 8.f * sx, 134 - eu));
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) pg[c] = 0.f;
    sx = 0.f;
}

template <int NT>
__device__ __forceinline__ double i4_segment(const Stage1Args& a, const uint32_t* list, int e0, int e1, int nbB,
                                             int eu, int tile, __amdgpu_buffer_rsrc_t crs, uint32_t codes_bytes,
                                             uint32_t tile_off, int* table) {
    constexpr int NS = NT / 16;                     // slots
    const int t = threadIdx.x;
    const int slot = t >> 4, bk = (t & 15) >> 1, m = t & 1;
    const uint32_t lane_off = (uint32_t)(bk * 16 + m * 8);
    const int f_pad = a.p.f_pad, groups = a.p.groups;
    const int tm = (t >> 7) & 1, tc = t & 127;      // the (matrix, channel) of thread t < 256
    const float* srow = a.p.scales + (size_t)tm * groups * f_pad + (size_t)tile * 128 + tc;

    // ---- band A, eight rows at a time (every load of a batch in flight)
    double acc_a = 0.0;
    const int a0 = max(e0, nbB), a1 = e1;
    if (t < 256) {
        const uint32_t word_off = (uint32_t)((tc >> 4) * 16 + tm * 8 + ((tc & 15) >> 3) * 4);
        for (int r0 = a0; r0 < a1; r0 += 8) {
            uint32_t wd[8];
            float sv[8], xv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = r0 + j;
                const bool ok = r < a1;
                const uint32_t e = ok ? list[r] : 0u;
                const int i = (int)(e >> 16);
                wd[j] = buf_load4(crs, ok ? (uint32_t)i * (uint32_t)kTileRowBytes + word_off : codes_bytes, tile_off);
                sv[j] = ok ? srow[(size_t)(i >> 7) * f_pad] : 0.f;
                xv[j] = __uint_as_float(e << 16);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc_a = fma((double)(xv[j] * (float)sext4(wd[j], tc & 7)), (double)sv[j], acc_a);
        }
    }

    // ---- band B
    double acc = 0.0;
    const int b0 = e0, b1 = max(e0, min(e1, nbB));
    if (b1 > b0) {
        const int gfirst = (int)(list[b0] >> 23), glast = (int)(list[b1 - 1] >> 23);
        for (int G0 = gfirst; G0 <= glast; G0 += kI4Win) {
            for (int i = t; i < kI4TableWords; i += NT) table[i] = 0;
            const int w0 = G0 > gfirst ? i4_group_start(list, b0, b1, G0) : b0;
            const int w1 = G0 + kI4Win <= glast ? i4_group_start(list, w0, b1, G0 + kI4Win) : b1;
            // this window's scales, needed after the stream (unconditional
            // loads: a group past the last one re-reads the last, and its
            // table entries are zero)
            float sw[kI4Win];
#pragma unroll
            for (int gw = 0; gw < kI4Win; ++gw) sw[gw] = srow[(size_t)min(G0 + gw, groups - 1) * f_pad];
            lds_barrier();                          // the table is clear
            const int n = w1 - w0;
            const int r0 = w0 + (int)((uint32_t)(slot * n) / (uint32_t)NS);      // this slot's run
            const int r1 = w0 + (int)((uint32_t)((slot + 1) * n) / (uint32_t)NS);
            // ring of kI4Ring rows: row r + kI4Ring is requested into the
            // slot of row r right after row r is consumed; the entries of the
            // next kI4Ring rows are read while the current ones are consumed
            // (two entry arrays, alternating).  Rows past the run have entry 0:
            // they read as x = 0 at an offset past the codes (zeros, no memory
            // access), so the loads are unconditional.
            auto entries = [&](int r, uint32_t (&en)[kI4Ring]) {
#pragma unroll
                for (int j = 0; j < kI4Ring; ++j) {
                    const int i = r + j;
                    const uint32_t e = list[min(i, r1)];     // r1 <= k_in: inside the list
                    en[j] = i < r1 ? e : 0u;
                }
            };
            auto request = [&](uint32_t e) {
                return buf_load8(crs, e != 0u ? (e >> 16) * (uint32_t)kTileRowBytes + lane_off : codes_bytes,
                                 tile_off);
            };
            float pg[16], sx = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) pg[c] = 0.f;
            int cur = r0 < r1 ? (int)(list[r0] >> 23) : G0;
            auto consume = [&](uint2 v, uint32_t e) {
                const float x = __uint_as_float(e << 16);
                const uint32_t wd[2] = {v.x, v.y};             // channels 0..7, 8..15
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    // nibbles flipped by 8 and split into bytes; the opaque
                    // moves keep each byte's conversion a single instruction
                    uint32_t lo = (wd[k] ^ 0x88888888u) & 0x0f0f0f0fu, hi = ((wd[k] >> 4) ^ 0x08888888u) & 0x0f0f0f0fu;
                    asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        pg[8 * k + 2 * q] = fmaf(x, ubyte_f(lo, q), pg[8 * k + 2 * q]);
                        pg[8 * k + 2 * q + 1] = fmaf(x, ubyte_f(hi, q), pg[8 * k + 2 * q + 1]);
                    }
                }
                sx += x;
                // the sums are final before the slot is reloaded, so the new
                // load can take the old registers
#pragma unroll
                for (int c = 0; c < 16; ++c) asm volatile("" : "+v"(pg[c]));
            };
            // one ring's worth of rows.  A row past the run (entry 0, group 0)
            // may flush the run's sums one row early and leave the lane on
            // group 0 with zero sums: harmless.  The branch holds no loads, so
            // the ring's loads stay in flight across it.
            auto half = [&](uint2 (&bv)[kI4Ring], const uint32_t (&ec)[kI4Ring], const uint32_t (&en)[kI4Ring]) {
#pragma unroll
                for (int j = 0; j < kI4Ring; ++j) {
                    const int g = (int)(ec[j] >> 23);
                    if (g != cur) {
                        i4_flush(pg, sx, cur - G0, m, bk, eu, table);
                        cur = g;
                    }
                    consume(bv[j], ec[j]);
                    bv[j] = request(en[j]);
                }
            };
            uint2 bv[kI4Ring];
            uint32_t ea[kI4Ring];
            entries(r0, ea);
#pragma unroll
            for (int j = 0; j < kI4Ring; ++j) {
                bv[j] = request(ea[j]);
                __builtin_amdgcn_sched_barrier(0);   // issue order = consumption order
            }
            for (int r = r0; r < r1; r += kI4Ring) {
                uint32_t eb[kI4Ring];
                entries(r + kI4Ring, eb);
                half(bv, ea, eb);
#pragma unroll
                for (int j = 0; j < kI4Ring; ++j) ea[j] = eb[j];
            }
            i4_flush(pg, sx, cur - G0, m, bk, eu, table);
            lds_barrier();                          // the table is complete
            if (t < 256) {
                double ws = 0.0;
#pragma unroll
                for (int gw = 0; gw < kI4Win; ++gw) ws = fma((double)table[gw * 256 + t], (double)sw[gw], ws);
                acc += ws;
            }
            lds_barrier();                          // read before the next window clears it
        }
    }
    return ldexp(acc, eu - 134) + acc_a;
}

template <int N>
__device__ __forceinline__ void settle_d(double (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]) : : "memory");
}

template <int KIND, int PX>
__global__ void __launch_bounds__(kS1Threads) k_stage1(Stage1Args a) {
    constexpr int TC = KIND == 1 ? 64 : 128;            // channels per tile
    constexpr int NV = KIND == 1 ? 8 : 16;               // channels per lane
    constexpr int NW = kS1Threads / kWave;
    extern __shared__ uint4 dyn_v[];               // 16-byte aligned (16-byte list reads)
    uint32_t* dyn = reinterpret_cast<uint32_t*>(dyn_v);
    __shared__ __align__(16) uint32_t hist[2048 + 16 + 64];
    __shared__ int sc[24];
    __shared__ double red[8][2][TC];
    __shared__ double gsum[2][TC];

    const int b = blockIdx.y, wb = blockIdx.x;
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int k_in = a.k_in, d = a.d, nch = a.nch;
    uint32_t* list = dyn;                         // [k_in + 64], then the chunks' exactness flags
    const uint8_t* xflags = reinterpret_cast<const uint8_t*>(dyn + s1_flags_off(k_in));
    int* i4_table = reinterpret_cast<int*>(dyn + s1_table_off(k_in));   // int4: [kI4Win][256]
    tl_mark(a.tl, 0, 0);
    stage1_select<PX>(a, b, list, hist, sc);
    tl_mark(a.tl, 0, 1);
    bool flags_done = false;     // the chunk flags are computed under the block's first loads

    const int T = a.tiles * nch;
    const int i0 = s1_item0(wb, T, a.nb1), i1 = s1_item0(wb + 1, T, a.nb1);
    const int slot = w * 8 + (l >> 3);
    const int cb = l & 7;
    const uint32_t codes_bytes = (uint32_t)a.tiles * (uint32_t)d * (uint32_t)kTileRowBytes;
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(a.p.codes, codes_bytes);
    const uint32_t lane_off = (uint32_t)cb * 16u;
    for (int tile = i0 / nch; tile * nch < i1; ++tile) {
        const int ca = max(i0, tile * nch) - tile * nch;
        const int ce = min(i1, (tile + 1) * nch) - tile * nch;
        const uint32_t tile_off = (uint32_t)tile * (uint32_t)d * (uint32_t)kTileRowBytes;
        // this segment's sums: thread t < 2 TC holds channel t % TC, gate (t < TC) or up
        double v = 0.0;
        float sgj = 0.f, suj = 0.f;
        if constexpr (KIND == 2) {
            v = i4_segment<kS1Threads>(a, list, ca * kChunk, min(ce * kChunk, k_in), sc[16], sc[17], tile, crs,
                                       codes_bytes, tile_off, i4_table);
            tl_mark(a.tl, 0, 2);
        } else {
        // int8 channel scales, requested now and used after the stream
        {
            const int j = tile * TC + (t % TC);             // < f_pad: always readable
            sgj = a.p.scales[j];
            suj = a.p.scales[(size_t)a.p.f_pad + j];
        }
        double ag[NV], au[NV];
#pragma unroll
        for (int c = 0; c < NV; ++c) ag[c] = au[c] = 0.0;

        // chunks ca + slot, + 64, ...: two chunks in flight per slot; the loop
        // has no exit from its middle and its loads are unconditional
        Chunk c0, c1;
        load_chunk(list, xflags, k_in, ca + slot, ce, crs, codes_bytes, tile_off, lane_off, c0);
        if (!flags_done) {
            stage1_flags(list, k_in);
            lds_barrier();
            flags_done = true;
            c0.exact = ca + slot < ce ? xflags[ca + slot] != 0 : true;
        }
        for (int ch = ca + slot; ch < ce; ch += 2 * kSlots) {
            load_chunk(list, xflags, k_in, ch + kSlots, ce, crs, codes_bytes, tile_off, lane_off, c1);
            consume_chunk_i8(c0, ag, au);
            settle_d(ag);
            settle_d(au);
            load_chunk(list, xflags, k_in, ch + 2 * kSlots, ce, crs, codes_bytes, tile_off, lane_off, c0);
            consume_chunk_i8(c1, ag, au);
            settle_d(ag);
            settle_d(au);
        }
        tl_mark(a.tl, 0, 2);
        // reduce the 8 row slots of the wave (lanes l ^ 8, l ^ 16, l ^ 32 share the
        // channel block), then the 8 waves, in a fixed order.  The slots are
        // added pairwise over lane bits 3, 4 and 5 with each level halving
        // what a lane keeps (bit 3 picks the matrix, bits 4 and 5 the channel
        // halves), so every lane ends with 2 of the wave's 128 sums; the
        // pairing, hence every rounding, is that of a full reduction over
        // the three lane bits.
        {
            const bool b3 = (l & 8) != 0, b4 = (l & 16) != 0, b5 = (l & 32) != 0;
            double w8[8], w4[4], w2[2];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const double send = b3 ? ag[c] : au[c];
                w8[c] = (b3 ? au[c] : ag[c]) + dpp_ror8(send);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const double send = b4 ? w8[c] : w8[c + 4];
                w4[c] = (b4 ? w8[c + 4] : w8[c]) + __shfl_xor(send, 16, kWave);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const double send = b5 ? w4[c] : w4[c + 2];
                w2[c] = (b5 ? w4[c + 2] : w4[c]) + __shfl_xor(send, 32, kWave);
            }
            const int ch = cb * NV + (b4 ? 4 : 0) + (b5 ? 2 : 0);
            red[w][b3 ? 1 : 0][ch] = w2[0];
            red[w][b3 ? 1 : 0][ch + 1] = w2[1];
        }
        lds_barrier();
        if (t < 2 * TC) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v += red[q][t / TC][t % TC];
        }
        }
        const int w0 = s1_block_of(tile * nch, T, a.nb1);
        const int w1 = s1_block_of((tile + 1) * nch - 1, T, a.nb1);
        bool last = true;
        if (w1 > w0) {
            // the tile is split: publish this segment, and the block that
            // completes the tile adds the segments in block order
            // (device-scope stores and loads: they are coherent across the
            // chip's L2 caches without writing back or invalidating whole
            // caches; the stores have completed before the arrival is counted)
            double* slot = a.part + ((size_t)b * (a.tiles + a.nb1) + tile) * 2 * kPartChannels;
            if (t < 2 * TC)
                __hip_atomic_store(&slot[((size_t)2 * wb + t / TC) * kPartChannels + t % TC], v,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
            __syncthreads();
            if (t == 0) sc[22] = tile_arrive(a.tcnt + (size_t)b * a.tiles + tile, a.gen, w1 - w0 + 1);
            lds_barrier();
            last = sc[22] != 0;
            if (last && t < 2 * TC) {
                v = 0.0;
                for (int w = w0; w <= w1; ++w)
                    v += __hip_atomic_load(&slot[((size_t)2 * w + t / TC) * kPartChannels + t % TC],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (last) {
            if (t < 2 * TC) gsum[t / TC][t % TC] = v;
            lds_barrier();
            if (t < TC) stage1_score(a, b, tile * TC + t, gsum[0][t], gsum[1][t], sgj, suj);
        }
        lds_barrier();   // `red` and `gsum` are rewritten by the next tile
    }
    tl_mark(a.tl, 0, 3);
    tl_flush(a.tl, 0);
}

template <int KIND, int PX>
static hipError_t go_stage1(const Stage1Args& a, int B, hipStream_t s) {
    const size_t dyn = KIND == 2 ? ((size_t)s1_table_off(a.k_in) + kI4TableWords) * 4
                                 : (size_t)s1_flags_off(a.k_in) * 4 + (size_t)((a.k_in + kChunk - 1) / kChunk + 16);
    auto fn = k_stage1<KIND, PX>;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    launch_kernel(fn, dim3(a.nb1, B), dim3(kS1Threads), dyn, s, a);
    return hipGetLastError();
}

template <int KIND>
static hipError_t stage1_px(const Stage1Args& a, int B, hipStream_t s) {
    const int per = (a.d + kS1Threads - 1) / kS1Threads;
    if (per <= 8) return go_stage1<KIND, 8>(a, B, s);
    if (per <= 16) return go_stage1<KIND, 16>(a, B, s);
    if (per <= 24) return go_stage1<KIND, 24>(a, B, s);
    return go_stage1<KIND, 32>(a, B, s);
}

hipError_t launch_stage1(const uint16_t* x, int B, int d, int k_in, const ProxyView& p, float* key,
                         double* part, unsigned long long* tcnt, uint32_t gen,
                         const S1Geom& g, double* h_tap, float* key_tap, int32_t* in_idx_tap,
                         unsigned long long* tl, hipStream_t s) {
    Stage1Args a{x, d, k_in, p, key, part, tcnt, h_tap, key_tap, in_idx_tap, g.tiles, g.nch, g.nb1, gen, tl};
    return p.kind == 1 ? stage1_px<1>(a, B, s) : stage1_px<2>(a, B, s);
}


// ---------------------------------------------------------------------------
// Stage 2.  grid (W2, B), block 512 (8 waves).  Block w of token b owns the
// channel range [w*F/W2, (w+1)*F/W2): it writes the mask bytes and idx
// entries of that range and the partial y over the kept channels in it.
//
// Sparse SwiGLU: thread t covers columns r*4096 + 8t .. +8 (r < R) of every
// row.  Channels go G at a time, double-buffered: the gate/up/down rows of the
// next group are in flight while the current group's gate/up dots (fp32) are
// reduced across the block, h = silu(g) u is formed and h * W_down row is
// accumulated into the thread's part of the block's partial y.
// ---------------------------------------------------------------------------
struct Stage2Args {
    const uint16_t* x;
    const uint16_t* wg_t;
    const uint16_t* wu_t;
    const uint16_t* wd;
    const float* key;     // [B][f_pad]
    int d, F, f_pad, k, W2;
    int32_t* idx;         // [B][k] or null
    uint8_t* mask;        // [B][F] or null
    float* ypart;         // [B][W2][d]
    int32_t* stream_tap;  // [B][k] or null: the channels the blocks stream, by share
    unsigned long long* tl;   // timeline stamps or null
    const double* hsrc;   // mode 2: exact h [B][F]
    const float* qscale;  // mode 3: row scales [3][F] (gate, up, down)
};

constexpr int kS2Threads = 512;

// Thread t covers columns r * 4096 + 8t .. +8 (r < R) of every row.  The rows a
// group holds, by stream mode:
//   1  bf16 gate, up and down rows (h computed here);
//   2  bf16 down rows; h of each channel read from memory (exact mode, where
//      Stage 1 computed the exact h of every channel);
//   3  int8 gate, up and down rows (8 bytes per thread per part) and the
//      rows' fp32 scales (quantized Stage-2 weights).
template <int MODE, int R, int G>
struct RowGroup {
    uint4 g[G][R], u[G][R], dn[G][R];
};
template <int R, int G>
struct RowGroup<2, R, G> {
    uint4 dn[G][R];
    float h[G];
};
template <int R, int G>
struct RowGroup<3, R, G> {
    uint2 g[G][R], u[G][R], dn[G][R];
    float sg[G], su[G], sd[G];
};

// Rows of list entries v0 .. v0 + G - 1 (buffer loads: the row offset is
// scalar, the column offset `voff` is this thread's).  Loads are unconditional
// so the compiler keeps them in flight: entries at or past `cnt` (their h is
// zeroed) and columns past d (x is 0 there) read at an offset past the end of
// the matrix, which the hardware returns as zeros without a memory access.
struct RowRsrc {
    __amdgpu_buffer_rsrc_t g, u, dn;
};
// Per-channel values the stream modes read from memory: h (mode 2, this
// token's [F]) or the rows' scales (mode 3, [F] each).
struct RowAux {
    const double* h;
    const float* sg;
    const float* su;
    const float* sd;
};


template <int MODE, int R, int G>
__device__ __forceinline__ void load_group(const RowRsrc& rs, const RowAux& aux, const uint16_t* chan, int v0,
                                           int cnt, uint32_t row_bytes, uint32_t oob, const uint32_t (&voff)[R],
                                           RowGroup<MODE, R, G>& rg) {
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const bool ok = v0 + q < cnt;
        const int j = __builtin_amdgcn_readfirstlane((int)chan[min(v0 + q, max(cnt - 1, 0))]);
        const uint32_t soff = (uint32_t)j * row_bytes;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t vo = ok ? voff[r] : oob;
            if constexpr (MODE == 1) {
                rg.g[q][r] = buf_load16(rs.g, vo, soff);
                rg.u[q][r] = buf_load16(rs.u, vo, soff);
                rg.dn[q][r] = buf_load16(rs.dn, vo, soff);
            } else if constexpr (MODE == 2) {
                rg.dn[q][r] = buf_load16(rs.dn, vo, soff);
            } else {
                rg.g[q][r] = buf_load8(rs.g, vo, soff);
                rg.u[q][r] = buf_load8(rs.u, vo, soff);
                rg.dn[q][r] = buf_load8(rs.dn, vo, soff);
            }
        }
        if constexpr (MODE == 2) rg.h[q] = (float)aux.h[j];
        if constexpr (MODE == 3) {
            rg.sg[q] = aux.sg[j];
            rg.su[q] = aux.su[j];
            rg.sd[q] = aux.sd[j];
        }
    }
}

// Materialise y here: no arithmetic on it moves across this point, and no
// memory access either.
template <int R>
__device__ __forceinline__ void settle(float (&y)[R][8]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(y[r][e]) : : "memory");
}

__device__ __forceinline__ float dot8(const float (&x)[8], uint4 v, float acc) {
    acc = fmaf(x[0], bf16_lo(v.x), acc); acc = fmaf(x[1], bf16_hi(v.x), acc);
    acc = fmaf(x[2], bf16_lo(v.y), acc); acc = fmaf(x[3], bf16_hi(v.y), acc);
    acc = fmaf(x[4], bf16_lo(v.z), acc); acc = fmaf(x[5], bf16_hi(v.z), acc);
    acc = fmaf(x[6], bf16_lo(v.w), acc); acc = fmaf(x[7], bf16_hi(v.w), acc);
    return acc;
}

__device__ __forceinline__ void axpy8(float h, uint4 v, float (&y)[8]) {
    y[0] = fmaf(h, bf16_lo(v.x), y[0]); y[1] = fmaf(h, bf16_hi(v.x), y[1]);
    y[2] = fmaf(h, bf16_lo(v.y), y[2]); y[3] = fmaf(h, bf16_hi(v.y), y[3]);
    y[4] = fmaf(h, bf16_lo(v.z), y[4]); y[5] = fmaf(h, bf16_hi(v.z), y[5]);
    y[6] = fmaf(h, bf16_lo(v.w), y[6]); y[7] = fmaf(h, bf16_hi(v.w), y[7]);
}

__device__ __forceinline__ float dot8_i8(const float (&x)[8], uint2 v, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(x[e], (float)sext8(v.x, e), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(x[4 + e], (float)sext8(v.y, e), acc);
    return acc;
}

__device__ __forceinline__ void axpy8_i8(float h, uint2 v, float (&y)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fmaf(h, (float)sext8(v.x, e), y[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[4 + e] = fmaf(h, (float)sext8(v.y, e), y[4 + e]);
}

// Gate/up dots of a group (fp32), reduced over the block's waves through LDS
// (`red` = this parity's [wave][2G] buffer), then h = silu(g) u for the
// `nvalid` leading entries and the W_down rows accumulated into y.  Mode 2
// takes h as read; mode 3 scales the integer-code dots by the rows' scales
// (g = s_g x.q_g, u = s_u x.q_u, and the down row s_d q_d).
template <int MODE, int R, int G>
__device__ __forceinline__ void consume_group(const RowGroup<MODE, R, G>& rg, const float (&xr)[R][8],
                                              float (&yacc)[R][8], int nvalid, float* red) {
    constexpr int NW = kS2Threads / kWave;
    float h[G];
    if constexpr (MODE == 2) {
#pragma unroll
        for (int q = 0; q < G; ++q) h[q] = q < nvalid ? rg.h[q] : 0.f;
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) axpy8(h[q], rg.dn[q][r], yacc[r]);
        return;
    } else {
        const int t = threadIdx.x, w = t >> 6, l = t & 63;
        float pg[G], pu[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float ga = 0.f, ua = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (MODE == 1) {
                    ga = dot8(xr[r], rg.g[q][r], ga);
                    ua = dot8(xr[r], rg.u[q][r], ua);
                } else {
                    ga = dot8_i8(xr[r], rg.g[q][r], ga);
                    ua = dot8_i8(xr[r], rg.u[q][r], ua);
                }
            }
            pg[q] = wave_sum(ga);
            pu[q] = wave_sum(ua);
        }
        if (l == 0) {
#pragma unroll
            for (int q = 0; q < G; ++q) {
                red[w * 2 * G + 2 * q] = pg[q];
                red[w * 2 * G + 2 * q + 1] = pu[q];
            }
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                gs += red[v * 2 * G + 2 * q];
                us += red[v * 2 * G + 2 * q + 1];
            }
            if constexpr (MODE == 3) {
                gs *= rg.sg[q];
                us *= rg.su[q];
            }
            h[q] = q < nvalid ? gs / (1.f + expf(-gs)) * us : 0.f;
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if constexpr (MODE == 1) axpy8(h[q], rg.dn[q][r], yacc[r]);
                else axpy8_i8(h[q] * rg.sd[q], rg.dn[q][r], yacc[r]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Stage 2 top-k.  A threshold bin (prefix at shift) splits the keys: those in
// higher bins are kept for certain ("certain"), those in the bin are
// "candidates".  The bin comes from a histogram of the keys' top 14 bits that
// the block builds in LDS (should its bins not add up, from a radix digit of
// the block's own keys).  Thread t owns channels t*PK .. t*PK + PK - 1 for the
// block-wide counts; the candidates go to LDS in index order and each gets
// its rank (key descending, index ascending), so a candidate is kept when its
// rank is below k - (certain keys).  Up to 64 candidates (the usual case: 64
// bins per binade leave a few dozen keys in the threshold bin) are ranked by
// one wave; more take block-wide passes.  The block's certain channels are
// listed and their first rows requested as soon as the bin is known, before
// the candidates are resolved.
//
// The list: certain channels of the range in index order, then its kept
// candidates in index order.  The first group holds the leading E = min(nc, G)
// certain entries; the rest follow G at a time, each group's rows in flight
// while the previous group is reduced and accumulated.
// ---------------------------------------------------------------------------
constexpr int kSmallCand = 128;   // candidates ranked by direct comparison up to this many
constexpr int kCandCap = 1024;    // candidates listed in LDS (more: the slow path)

template <int PK, int R, int G, int MODE>
__global__ void __launch_bounds__(kS2Threads) k_stage2(Stage2Args a) {
    // Keys per thread from 32 up are loaded coalesced and transposed through
    // LDS; fewer are loaded as each thread's own run directly (its 16-byte
    // loads span at most 96 bytes per lane, and the transposition would cost
    // more than it saves).
    constexpr bool kS2CoalescedKeys = PK >= 32;
    constexpr bool STREAM = MODE != 0;       // 0: selection only (mask and idx)
    constexpr int SM = STREAM ? MODE : 1;    // the stream code's mode (unused when MODE == 0)
    constexpr int NT = kS2Threads;
    constexpr int NW = NT / kWave;
    extern __shared__ uint4 dyn2v[];                     // 16-byte aligned
    uint32_t* dyn2 = reinterpret_cast<uint32_t*>(dyn2v);
    __shared__ uint32_t hist[2048 + 64];
    __shared__ int sc[24];
    __shared__ int wc[4][NW];
    __shared__ float red[2][NW * 2 * G];

    tl_mark(a.tl, 1, 0);
    const int w = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int F = a.F, k = a.k, W2 = a.W2;
    const int r0 = split_point(w, F, W2), r1 = split_point(w + 1, F, W2);
    const int L = r1 - r0;                                 // channels of this block's range
    uint32_t* keys = dyn2;                                 // [s2_keys_words(F, NT, PK)] the key histogram, then
                                                           // the keys' transposition, then every key (index order)
    uint32_t* cval = keys + s2_keys_words(F, NT, PK);      // [kCandCap + 64] candidate keys, index order
    uint16_t* cidx = reinterpret_cast<uint16_t*>(cval + kCandCap + 64);   // [kCandCap + 64] their channels
    uint16_t* kr = cidx + kCandCap + 64;                   // [kCandCap] rank among the kept candidates
    uint16_t* chan = kr + kCandCap;                        // [cap + 64] the block's list
    const float* keyb = a.key + (size_t)b * a.f_pad;

    constexpr uint32_t EB = MODE == 3 ? 1u : 2u;          // bytes per weight
    const uint32_t row_bytes = (uint32_t)a.d * EB;
    const uint32_t mat_bytes = (uint32_t)F * row_bytes;
    const RowRsrc rs{make_rsrc(a.wg_t, mat_bytes), make_rsrc(a.wu_t, mat_bytes), make_rsrc(a.wd, mat_bytes)};
    const RowAux aux{a.hsrc ? a.hsrc + (size_t)b * F : nullptr, a.qscale, a.qscale ? a.qscale + F : nullptr,
                     a.qscale ? a.qscale + 2 * (size_t)F : nullptr};
    uint32_t voff[R];
    uint4 xv[R];                    // this thread's 8 x values per row part, as loaded (converted
    float yacc[R][8];               // when the stream starts: nothing before it waits for them)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int col = r * 4096 + t * 8;
        voff[r] = col < a.d ? (uint32_t)col * EB : mat_bytes;   // past d: read as zeros
        xv[r] = make_uint4(0, 0, 0, 0);
        if (STREAM && col < a.d) xv[r] = *reinterpret_cast<const uint4*>(a.x + (size_t)b * a.d + col);
#pragma unroll
        for (int e = 0; e < 8; ++e) yacc[r][e] = 0.f;
    }
    const bool all = k >= F, none = k == 0;
    // the keys (from 32 per thread in the coalesced order, group g of thread t
    // = keys (g NT + t) 4 .. + 3: the histogram does not depend on which
    // thread holds a key; else thread t's own run), and the histogram of their
    // high bits cleared meanwhile
    uint32_t kb[PK];
    {
        bool valid[PK];
        if constexpr (kS2CoalescedKeys)
            load_u32_coal<PK, NT>(reinterpret_cast<const uint32_t*>(keyb), F, a.f_pad, kb, valid);
        else
            load_u32_contig<PK>(reinterpret_cast<const uint32_t*>(keyb), F, a.f_pad, kb, valid);
        if (!all && !none) {
#pragma unroll
            for (int v = 0; v < kGhBins / NT / 4; ++v)
                reinterpret_cast<uint4*>(keys)[v * NT + t] = make_uint4(0u, 0u, 0u, 0u);
        }
        // keys past F: negative as int, below every bin of a valid key; their
        // histogram bin (kGhBins + lane) is a spare word, one per lane
#pragma unroll
        for (int q = 0; q < PK; ++q) kb[q] = valid[q] ? kb[q] : 0x80000000u | ((uint32_t)(t & 63) << kGhShift);
    }
    // every key in LDS too (index order), for the slow paths (written after
    // the candidate count is known)
    auto keys_to_lds = [&]() {
        if (t * PK < F) {
#pragma unroll
            for (int q = 0; q < PK; q += 4)
                if (t * PK + q < F) *reinterpret_cast<uint4*>(keys + t * PK + q) = make_uint4(kb[q], kb[q + 1], kb[q + 2], kb[q + 3]);
        }
    };
    // the first NT channels of the range, one per thread
    const uint32_t own0 = t < L ? __float_as_uint(keyb[r0 + t]) : 0u;
    if (STREAM && t == 0) chan[0] = 0;                     // row 0 stands in for an empty list

    // ---- threshold bin: the block's key histogram (every key's top bits;
    // a key is a non-negative float, so its bit pattern orders like its
    // value), this thread's bins NB - 16 (t + 1) .. read back as 16-byte words
    SelectState st{0u, 0, 0, 0, 0};
    if (!all && !none) {
        lds_barrier();
        // keys past F land in the spare bins past the histogram (never read),
        // one per lane so they do not contend: no branch per key
#pragma unroll
        for (int q = 0; q < PK; ++q) atomicAdd(&keys[min(kb[q] >> kGhShift, (uint32_t)(kGhBins + 63))], 1u);
        lds_barrier();
        tl_mark(a.tl, 1, 4);
        // (the scans below hold barriers before keys_to_lds overwrites the histogram)
        if (!block_hist_bin_wave<NT, kGhBins>(keys, k, F, kGhShift, sc, st)) {
            bool valid[PK];
#pragma unroll
            for (int q = 0; q < PK; ++q) valid[q] = (int)kb[q] >= 0;
            st = block_coarse_bin<PK, NT>(kb, valid, k, 31, hist, sc);
        }
    }
    // ---- coalesced keys to one run per thread: thread t takes keys t PK ..
    // t PK + PK - 1 (the index-order ranks below come from one block scan of
    // the runs).  Through LDS (the histogram is no longer read): run t at word
    // t (PK + 4), so the 16-byte reads of the 64 lanes fall in distinct banks.
    if constexpr (kS2CoalescedKeys) {
#pragma unroll
        for (int g = 0; g < PK / 4; ++g) {
            const int j = (g * NT + t) * 4;                 // the 4 keys share one run (PK % 4 == 0)
            *reinterpret_cast<uint4*>(keys + j + 4 * (j / PK)) = make_uint4(kb[4 * g], kb[4 * g + 1],
                                                                            kb[4 * g + 2], kb[4 * g + 3]);
        }
        lds_barrier();
        const uint32_t sink = 0x80000000u | ((uint32_t)(t & 63) << kGhShift);
#pragma unroll
        for (int g = 0; g < PK / 4; ++g) {
            const uint4 u = *reinterpret_cast<const uint4*>(keys + t * (PK + 4) + 4 * g);
            const int j = t * PK + 4 * g;
            kb[4 * g] = j < F ? u.x : sink;
            kb[4 * g + 1] = j + 1 < F ? u.y : sink;
            kb[4 * g + 2] = j + 2 < F ? u.z : sink;
            kb[4 * g + 3] = j + 3 < F ? u.w : sink;
        }
    } else {
        // the thread's own run at the same place, for the candidate listing
        // below (each thread reads back only what it wrote: no barrier)
#pragma unroll
        for (int g = 0; g < PK / 4; ++g)
            *reinterpret_cast<uint4*>(keys + t * (PK + 4) + 4 * g) =
                make_uint4(kb[4 * g], kb[4 * g + 1], kb[4 * g + 2], kb[4 * g + 3]);
    }
    // bin of a key = (int)key >> shift: certain above cert_gt, candidate at
    // cand_eq (keep-all: every valid key certain; keep-none: nothing)
    const int shift = all || none ? 31 : st.shift;
    const int cert_gt = all ? -1 : (none ? 0x7fffffff : (int)st.prefix);
    const int cand_eq = all || none ? -2 : (int)st.prefix;
    auto is_cert = [&](uint32_t v) { return ((int)v >> shift) > cert_gt; };
    auto is_cand = [&](uint32_t v) { return ((int)v >> shift) == cand_eq; };

    // ---- this thread's certain / candidate keys as bit masks, then one
    // block scan of the counts: index-order rank of the thread's first
    // certain key (high half) and first candidate (low half)
    uint64_t cem = 0, cdm = 0;
#pragma unroll
    for (int q = 0; q < PK; ++q) {
        cem |= is_cert(kb[q]) ? (1ull << q) : 0ull;
        cdm |= is_cand(kb[q]) ? (1ull << q) : 0ull;
    }
    const int ncert_t = __popcll(cem), nd = __popcll(cdm);
    // both counts fit 16 bits (F <= 32768); the packed total may reach 2^31
    uint32_t tot;
    const uint32_t pre = block_excl_scan_u32<NT>(((uint32_t)ncert_t << 16) | (uint32_t)nd, sc, tot);
    const int ncand = (int)((uint32_t)tot & 0xffffu);
    const int C = (int)((uint32_t)tot >> 16);            // certain keys in all
    const int crank0 = (int)(pre >> 16), cp0 = (int)(pre & 0xffffu);
    tl_mark(a.tl, 1, 5);
    const bool listed = ncand <= kCandCap;                // candidates compacted (else the slow path)
    if (!listed || ncand > kSmallCand) keys_to_lds();     // the slow paths read every key from LDS
    // this block's share of the certain keys: ranks [c0, c1)
    const int c0 = split_point(w, C, W2), c1 = split_point(w + 1, C, W2);
    int nc = listed ? c1 - c0 : 0;
    if (listed) {
        // share: the certain keys of rank [c0, c1) into chan; candidates
        // (index order) into cidx / cval.  The loops visit only the set bits
        // of the thread's masks (the lowest first, so in index order); a
        // candidate's key is read back from the thread's run in LDS (after
        // keys_to_lds the run sits at t PK, else at t (PK + 4)).
        if (STREAM && crank0 < c1 && crank0 + ncert_t > c0) {
            int cr = crank0;
            for (uint64_t m = cem; m != 0ull && cr < c1; m &= m - 1ull, ++cr)
                if (cr >= c0) chan[cr - c0] = (uint16_t)(t * PK + __builtin_ctzll(m));
        }
        if (nd > 0) {
            const uint32_t* run = keys + (ncand > kSmallCand ? t * PK : t * (PK + 4));
            int cp = cp0;
            for (uint64_t m = cdm; m != 0ull; m &= m - 1ull, ++cp) {
                const int q = __builtin_ctzll(m);
                cidx[cp] = (uint16_t)(t * PK + q);
                cval[cp] = run[q];
            }
        }
    }
    if (t == r0 / PK) {                                    // counts before the range
        const int below = r0 - t * PK;                     // keys of this thread before r0
        const uint64_t lo = below >= 64 ? ~0ull : ((1ull << below) - 1);
        sc[16] = cp0 + __popcll(cdm & lo);
        sc[18] = crank0 + __popcll(cem & lo);
    }
    lds_barrier();
    tl_mark(a.tl, 1, 6);
    const int cs = sc[16];                                 // candidates before the range
    const int cert_before = sc[18];                        // certain keys before the range
    const int E = min(nc, G);
    RowGroup<SM, R, G> cur, nxt;
    if constexpr (STREAM) load_group<SM, R, G>(rs, aux, chan, 0, E, row_bytes, mat_bytes, voff, cur);

    int nks = 0, kc_before = 0, s0k = 0;
    if (listed && ncand <= kWave) {
        // ---- few candidates (the usual case): wave 0 ranks them (key
        // descending, index ascending), keeps the first k - C, and lists the
        // block's share of the kept ones; one barrier publishes the counts
        if (t < kWave) {
            const bool has = t < ncand;
            const uint32_t v = has ? cval[t] : 0u;
            int rank = 0;
            // eight lanes' keys per pass, so the reads are not one long
            // dependent chain
            for (int i0 = 0; i0 < ncand; i0 += 8) {
                uint32_t u[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = (uint32_t)__builtin_amdgcn_readlane((int)v, (i0 + e) & 63);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = i0 + e;
                    rank += (i < ncand && (u[e] > v || (u[e] == v && i < t))) ? 1 : 0;
                }
            }
            const bool kept = has && rank < st.krem;
            const uint64_t km = __ballot(kept);
            const int kcount = __popcll(km);
            const int s0 = split_point(w, kcount, W2), s1 = split_point(w + 1, kcount, W2);
            const int r = lanes_below(km);                 // rank among the kept, index order
            if (kept) {
                const uint16_t j = cidx[t];
                cidx[t] = (uint16_t)(j | 0x8000u);
                if (STREAM && r >= s0 && r < s1) chan[nc + r - s0] = j;
            }
            if (t == 0) {
                sc[12] = kcount;
                sc[13] = __popcll(km & (cs >= 64 ? ~0ull : ((1ull << cs) - 1)));
            }
        }
        lds_barrier();
        const int KC = sc[12];
        kc_before = sc[13];
        const int s0 = split_point(w, KC, W2), s1 = split_point(w + 1, KC, W2);
        nks = s1 - s0;
        s0k = s0;
        tl_mark(a.tl, 1, 7);
    } else if (listed) {
        // ---- resolve the candidates while those loads are in flight:
        // cidx[i] gets bit 15 when kept
        if (ncand > 0) {
            const int need = st.krem;                     // candidates to keep
            if (ncand <= kSmallCand) {
                // rank of candidate c = candidates before it in (key
                // descending, index ascending); S = NT / ncand (a power of
                // two, <= 64) consecutive lanes share candidate c, each
                // comparing every S-th candidate, then add their counts
                int S = 64;
                while (S * ncand > NT) S >>= 1;
                const int c = t / S, p = t & (S - 1);
                int rank = 0;
                const uint32_t v = c < ncand ? cval[c] : 0u;
                if (c < ncand) {
                    for (int i = p; i < ncand; i += S) {
                        const uint32_t u = cval[i];
                        rank += (u > v || (u == v && i < c)) ? 1 : 0;
                    }
                }
                for (int m = S >> 1; m >= 1; m >>= 1) rank += __shfl_xor(rank, m, 64);
                const bool kept = c < ncand && p == 0 && rank < need;
                lds_barrier();
                if (kept) cidx[c] |= 0x8000u;
            } else {
                // many candidates: remaining bits by histogram over the keys
                // of the threshold bin, then ties in index order
                SelectState s2 = st;
                s2.ncand = F;
                uint32_t T;
                int cgt;
                block_select_refine<NT>(s2, keys, T, cgt, hist, sc);
                const int eq_need = k - cgt;
                int eq_run = 0;
                for (int i0 = 0; i0 < ncand; i0 += NT) {
                    const int i = i0 + t;
                    const uint32_t v = i < ncand ? cval[i] : 0u;
                    bool p[1] = {i < ncand && v == T};
                    int pos[1], tt[1];
                    block_ballot_pos<kS2Threads, 1>(p, wc, pos, tt);
                    if (i < ncand && (v > T || (p[0] && eq_run + pos[0] < eq_need))) cidx[i] |= 0x8000u;
                    eq_run += tt[0];
                }
            }
            lds_barrier();
        }
        // ---- kept candidates: this block's share (ranks [s0, s1) among them,
        // in index order) goes after its certain entries; count those before
        // the range.  Ranks are found first, the writes follow (the shares of
        // later chunks need the totals of earlier ones only).
        int run = 0;
        for (int i0 = 0; i0 < ncand; i0 += NT) {
            const int i = i0 + t;
            const bool kept = i < ncand && (cidx[i] & 0x8000u) != 0;
            bool p[2] = {kept, kept && i < cs};
            int pos[2], tt[2];
            block_ballot_pos<kS2Threads, 2>(p, wc, pos, tt);
            if (i < ncand) kr[i] = (uint16_t)(run + pos[0]);   // rank among the kept
            run += tt[0];
            kc_before += tt[1];
        }
        const int KC = run;
        const int s0 = split_point(w, KC, W2), s1 = split_point(w + 1, KC, W2);
        nks = s1 - s0;
        s0k = s0;
        for (int i = t; i < ncand; i += NT) {
            const int r = kr[i];
            if (STREAM && (cidx[i] & 0x8000u) && r >= s0 && r < s1) chan[nc + r - s0] = cidx[i] & 0x7fffu;
        }
    } else {
        // ---- slow path (more candidates than the list holds): the exact
        // threshold over all keys, then every kept key's rank by one packed
        // scan; this block streams kept ranks [w*k/W2, (w+1)*k/W2)
        SelectState s2 = st;
        s2.ncand = F;
        uint32_t T;
        int cgt;
        block_select_refine<NT>(s2, keys, T, cgt, hist, sc);
        const int need = k - cgt;
        int gt = 0, eq = 0;
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            gt += (int)kb[q] >= 0 && kb[q] > T ? 1 : 0;
            eq += kb[q] == T ? 1 : 0;
        }
        uint32_t tk;
        const uint32_t pk = block_excl_scan_u32<NT>(((uint32_t)gt << 16) | (uint32_t)eq, sc, tk);
        int eb = (int)(pk & 0xffffu);
        int pos = (int)(pk >> 16) + min(eb, need);
        const int k0 = split_point(w, k, W2), k1 = split_point(w + 1, k, W2);
#pragma unroll
        for (int q = 0; q < PK; ++q) {
            const bool e = kb[q] == T;
            const bool on = ((int)kb[q] >= 0 && kb[q] > T) || (e && eb < need);
            if (STREAM && on && pos >= k0 && pos < k1) chan[pos - k0] = (uint16_t)(t * PK + q);
            const int j = t * PK + q;
            if (j >= r0 && j < r1) {
                if (on && a.idx) a.idx[(size_t)b * k + pos] = j;
                if (a.mask) a.mask[(size_t)b * F + j] = on ? 1 : 0;
            }
            eb += e ? 1 : 0;
            pos += on ? 1 : 0;
        }
        nc = k1 - k0;
    }
    const int kept_before = cert_before + kc_before;

    // ---- the range: kept flags, idx and mask (after the stream: nothing in
    // the stream depends on them)
    // (keys past the first NT of the range come from LDS: the threads' runs
    // at t (PK + 4), or every key in index order after keys_to_lds)
    auto write_range = [&]() {
    if (listed && (a.idx || a.mask)) {
        const bool idx_order = ncand > kSmallCand;
        int nk = 0, nd_run = 0;
        for (int c0r = 0; c0r < L; c0r += NT) {
            const int j = r0 + c0r + t;
            const bool in = c0r + t < L;
            const uint32_t v = c0r == 0 ? own0 : (in ? keys[idx_order ? j : (j / PK) * (PK + 4) + j % PK] : 0u);
            bool p1[1] = {in && is_cand(v)};
            int pos1[1], t1[1];
            block_ballot_pos<kS2Threads, 1>(p1, wc, pos1, t1);
            const bool kc = p1[0] && (cidx[cs + nd_run + pos1[0]] & 0x8000u) != 0;
            bool p2[1] = {in && (is_cert(v) || kc)};
            int pos2[1], t2[1];
            block_ballot_pos<kS2Threads, 1>(p2, wc, pos2, t2);
            if (p2[0] && a.idx) a.idx[(size_t)b * k + kept_before + nk + pos2[0]] = j;
            if (in && a.mask) a.mask[(size_t)b * F + j] = p2[0] ? 1 : 0;
            nd_run += t1[0];
            nk += t2[0];
        }
    }
    };
    const int n = nc + nks;
    lds_barrier();
    if constexpr (!STREAM) {         // selection only: mask and idx are written
        write_range();
        tl_flush(a.tl, 1);
        return;
    }
    if (a.stream_tap) {
        // the streamed list, at the ranks of the block's shares: certain keys
        // [c0, c1), then kept candidates at C + [s0, s1) (slow path: kept ranks
        // [k0, k1)); over all blocks, a permutation of the token's idx
        const int base1 = listed ? c0 : split_point(w, k, W2);
        for (int i = t; i < n; i += NT)
            a.stream_tap[(size_t)b * k + (i < nc ? base1 + i : C + s0k + (i - nc))] = chan[i];
    }

    // ---- sparse SwiGLU: group 0 = entries [0, E), then [E, n) G at a time.
    // The loads are unconditional and the loop has no exit from its middle:
    // on any path that merges pending and completed loads the compiler drains
    // every load and the overlap is lost.  After the last group, `cur` is
    // loaded past the list (zeros, no memory access) and left unused.
    tl_mark(a.tl, 1, 1);
    const int rest = n - E;
    const int groups = 1 + (rest + G - 1) / G;
    float xr[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        xr[r][0] = bf16_lo(xv[r].x); xr[r][1] = bf16_hi(xv[r].x);
        xr[r][2] = bf16_lo(xv[r].y); xr[r][3] = bf16_hi(xv[r].y);
        xr[r][4] = bf16_lo(xv[r].z); xr[r][5] = bf16_hi(xv[r].z);
        xr[r][6] = bf16_lo(xv[r].w); xr[r][7] = bf16_hi(xv[r].w);
    }
    int gi = 0;
    if (groups >= 2) {
        // the first two groups: the mask and idx of the block's range are
        // written while both are in flight
        load_group<SM, R, G>(rs, aux, chan, E, n, row_bytes, mat_bytes, voff, nxt);
        write_range();
        consume_group<SM, R, G>(cur, xr, yacc, E, red[0]);
        settle(yacc);
        load_group<SM, R, G>(rs, aux, chan, E + G, n, row_bytes, mat_bytes, voff, cur);
        consume_group<SM, R, G>(nxt, xr, yacc, min(G, rest), red[1]);
        settle(yacc);
        gi = 2;
    }
    for (; gi + 1 < groups; gi += 2) {
        load_group<SM, R, G>(rs, aux, chan, E + gi * G, n, row_bytes, mat_bytes, voff, nxt);
        consume_group<SM, R, G>(cur, xr, yacc, gi == 0 ? E : min(G, rest - (gi - 1) * G), red[0]);
        // The accumulation into y must finish before `cur` is reloaded: if the
        // compiler sinks it below the reloads, the old and new `cur` overlap
        // and the loop-carried registers need a copy that waits for the loads.
        settle(yacc);
        load_group<SM, R, G>(rs, aux, chan, E + (gi + 1) * G, n, row_bytes, mat_bytes, voff, cur);
        consume_group<SM, R, G>(nxt, xr, yacc, min(G, rest - gi * G), red[1]);
        settle(yacc);
    }
    if (gi < groups) consume_group<SM, R, G>(cur, xr, yacc, gi == 0 ? E : min(G, rest - (gi - 1) * G), red[0]);
    if (groups < 2) write_range();
    tl_mark(a.tl, 1, 2);
    float* dst = a.ypart + ((size_t)b * W2 + w) * a.d;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int col = r * 4096 + t * 8;
        if (col < a.d) {
            *reinterpret_cast<float4*>(dst + col) = make_float4(yacc[r][0], yacc[r][1], yacc[r][2], yacc[r][3]);
            *reinterpret_cast<float4*>(dst + col + 4) = make_float4(yacc[r][4], yacc[r][5], yacc[r][6], yacc[r][7]);
        }
    }
    tl_mark(a.tl, 1, 3);
    tl_flush(a.tl, 1);
}

template <int PK, int R, int G, int MODE>
static hipError_t go_stage2(const Stage2Args& a, int B, hipStream_t s) {
    // list length bound: ceil(C/W2) + ceil(KC/W2); selection only keeps no list
    const int cap = MODE != 0 ? (a.k + a.W2 - 1) / a.W2 + 2 : 0;
    const size_t dyn = (size_t)s2_keys_words(a.F, kS2Threads, PK) * 4 + ((size_t)kCandCap + 64) * 4 +
                       ((size_t)kCandCap * 2 + 64 + cap + 64) * 2;
    auto fn = k_stage2<PK, R, G, MODE>;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    launch_kernel(fn, dim3(a.W2, B), dim3(kS2Threads), dyn, s, a);
    return hipGetLastError();
}

template <int R, int G, int MODE>
static hipError_t stage2_pk(const Stage2Args& a, int B, hipStream_t s) {
    const int per = (a.F + kS2Threads - 1) / kS2Threads;
    if (per <= 4) return go_stage2<4, R, G, MODE>(a, B, s);
    if (per <= 8) return go_stage2<8, R, G, MODE>(a, B, s);
    if (per <= 16) return go_stage2<16, R, G, MODE>(a, B, s);
    if (per <= 24) return go_stage2<24, R, G, MODE>(a, B, s);
    if (per <= 32) return go_stage2<32, R, G, MODE>(a, B, s);
    if (per <= 40) return go_stage2<40, R, G, MODE>(a, B, s);
    if (per <= 48) return go_stage2<48, R, G, MODE>(a, B, s);
    if (per <= 56) return go_stage2<56, R, G, MODE>(a, B, s);
    return go_stage2<64, R, G, MODE>(a, B, s);
}

hipError_t launch_stage2(const uint16_t* x, const void* wg_t, const void* wu_t, const void* wd, const float* key,
                         int B, int d, int F, int f_pad, int k_ff, int W2, int32_t* idx, uint8_t* mask, float* ypart,
                         int32_t* stream_tap, unsigned long long* tl, int mode, const double* hsrc,
                         const float* qscale, hipStream_t s) {
    Stage2Args a{x, static_cast<const uint16_t*>(wg_t), static_cast<const uint16_t*>(wu_t),
                 static_cast<const uint16_t*>(wd), key, d, F, f_pad, k_ff, W2, idx, mask, ypart, stream_tap, tl,
                 hsrc, qscale};
    // channels per group: the fewest that keep the stream at its rate (more
    // rows in flight per block measured slower on the 4096 and 8192 shapes)
    if (mode == 2) {
        // exact mode streams one row per channel: more channels per group
        if (d <= 4096) return stage2_pk<1, 4, 2>(a, B, s);
        if (d <= 8192) return stage2_pk<2, 2, 2>(a, B, s);
        return stage2_pk<4, 1, 2>(a, B, s);
    }
    if (mode == 3) {
        if (d <= 4096) return stage2_pk<1, 2, 3>(a, B, s);
        if (d <= 8192) return stage2_pk<2, 1, 3>(a, B, s);
        return stage2_pk<4, 1, 3>(a, B, s);
    }
    if (d <= 4096) return stage2_pk<1, 2, 1>(a, B, s);
    if (d <= 8192) return stage2_pk<2, 1, 1>(a, B, s);
    return stage2_pk<4, 1, 1>(a, B, s);
}

hipError_t launch_select(const float* key, int B, int d, int F, int f_pad, int k_ff, int W2,
                         int32_t* idx, uint8_t* mask, hipStream_t s) {
    Stage2Args a{nullptr, nullptr, nullptr, nullptr, key, d, F, f_pad, k_ff, W2, idx, mask, nullptr, nullptr, nullptr,
                 nullptr, nullptr};
    return stage2_pk<1, 1, 0>(a, B, s);
}

// ---------------------------------------------------------------------------
// y = sum of the W2 block partials, fixed order.  grid (ceil(d / 16), B), block
// 256: thread (g = t / 4, c = t % 4) sums partials g, g + 64, ... of columns
// 4c .. 4c + 3 of the block's 16 (all of its loads in flight at once); the 16
// groups of a wave are combined by lane swaps (lanes 4 apart, then 8, 16, 32),
// the 4 waves through LDS, in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kRedCols = 16;
constexpr int kRedGroups = 64;
constexpr int kRedMax = kMaxW2Total / kRedGroups;   // partials per thread

__global__ void __launch_bounds__(256) k_reduce_y(const float* __restrict__ ypart, int d, int W2,
                                                  float* __restrict__ y) {
    __shared__ float4 acc[4][kRedCols / 4];
    const int b = blockIdx.y, t = threadIdx.x;
    const int g = t >> 2, c = t & 3;
    const int col = blockIdx.x * kRedCols + 4 * c;
    const bool in = col < d;                       // d % 8 == 0, so a quad is all in or all out
    const float* src = ypart + (size_t)b * W2 * d + (in ? col : 0);
    float4 v[kRedMax];
#pragma unroll
    for (int u = 0; u < kRedMax; ++u) {
        const int wv = g + u * kRedGroups;
        v[u] = wv < W2 ? *reinterpret_cast<const float4*>(src + (size_t)wv * d) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 s4 = v[0];
#pragma unroll
    for (int u = 1; u < kRedMax; ++u) {
        s4.x += v[u].x; s4.y += v[u].y; s4.z += v[u].z; s4.w += v[u].w;
    }
#pragma unroll
    for (int m = 4; m < kWave; m <<= 1) {
        s4.x += __shfl_xor(s4.x, m, kWave);
        s4.y += __shfl_xor(s4.y, m, kWave);
        s4.z += __shfl_xor(s4.z, m, kWave);
        s4.w += __shfl_xor(s4.w, m, kWave);
    }
    const int wv = t / kWave;
    if ((t & (kWave - 1)) < 4) acc[wv][c] = s4;
    __syncthreads();
    if (t < 4 && in) {
        float4 r = acc[0][c];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            const float4 o = acc[q][c];
            r.x += o.x; r.y += o.y; r.z += o.z; r.w += o.w;
        }
        *reinterpret_cast<float4*>(y + (size_t)b * d + col) = r;
    }
}

// The same sum for at most 32 partials (the matrix-core path's channel
// slices): block 256 = 64 column quads (256 columns) x 4 partial groups;
// thread (g = wave, q) sums partials g, g + 4, ... of quad q (every load in
// flight, each wave instruction one contiguous kilobyte of a partial), then
// the 4 groups are added through LDS in order.  One block per 256 columns
// and token instead of per 16, so a batch of tokens is one round of blocks.
constexpr int kRedFewMax = 32;
__global__ void __launch_bounds__(256) k_reduce_y_few(const float* __restrict__ ypart, int d, int W2,
                                                      float* __restrict__ y) {
    __shared__ float4 acc[4][64];
    const int b = blockIdx.y, t = threadIdx.x;
    const int q = t & 63, g = t >> 6;
    const int col = (blockIdx.x * 64 + q) * 4;
    const bool in = col < d;                       // d % 8 == 0: a quad is all in or all out
    const float* src = ypart + (size_t)b * W2 * d + (in ? col : 0);
    float4 v[kRedFewMax / 4];
#pragma unroll
    for (int u = 0; u < kRedFewMax / 4; ++u) {
        const int wv = g + 4 * u;
        v[u] = in && wv < W2 ? *reinterpret_cast<const float4*>(src + (size_t)wv * d) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 s4 = v[0];
#pragma unroll
    for (int u = 1; u < kRedFewMax / 4; ++u) {
        s4.x += v[u].x; s4.y += v[u].y; s4.z += v[u].z; s4.w += v[u].w;
    }
    acc[g][q] = s4;
    __syncthreads();
    if (g == 0 && in) {
        float4 r = acc[0][q];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            const float4 o = acc[i][q];
            r.x += o.x; r.y += o.y; r.z += o.z; r.w += o.w;
        }
        *reinterpret_cast<float4*>(y + (size_t)b * d + col) = r;
    }
}

hipError_t launch_reduce_y(const float* ypart, int B, int d, int W2, float* y, hipStream_t s) {
    if (W2 <= kRedFewMax)
        launch_kernel(k_reduce_y_few, dim3((d + 255) / 256, B), dim3(256), 0, s, ypart, d, W2, y);
    else
        launch_kernel(k_reduce_y, dim3((d + kRedCols - 1) / kRedCols, B), dim3(256), 0, s, ypart, d, W2, y);
    return hipGetLastError();
}

}  // namespace prox
