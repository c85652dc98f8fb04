// Device helpers shared by the Prox kernels (gfx950, wave64).
//
// Block-wide steps here synchronise with lds_barrier(): it waits for this
// wave's LDS operations only, so global loads issued earlier (prefetched
// weight rows) stay in flight across the barrier.  No kernel relies on a
// barrier to order global memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prox {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint32_t v16) { return __uint_as_float(v16 << 16); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- buffer loads: a scalar resource (base, byte size) + per-lane byte offset
// + scalar byte offset.  The hardware returns zeros past the size.  Rows that
// are uniform over a block then cost no per-lane address arithmetic.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Arrival at a split tile: the counter holds (call tag << 32 | arrivals).  The
// arrival that completes the tile stores 0 back, so every call leaves its
// counters clear (a replayed graph reuses one tag); a counter holding anything
// else with another tag (a workspace never cleared, an interrupted call)
// restarts at 1.  Returns 1 for the arrival that completes the tile.
__device__ __forceinline__ int tile_arrive(unsigned long long* cnt, uint32_t gen, int nseg) {
    unsigned long long cur = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const bool same = (cur >> 32) == gen || cur == 0ull;
        const unsigned long long nxt = same ? ((((unsigned long long)gen << 32) | (cur & 0xffffffffull)) + 1ull)
                                            : (((unsigned long long)gen << 32) | 1ull);
        if (__hip_atomic_compare_exchange_strong(cnt, &cur, nxt, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
            if ((int)(nxt & 0xffffffffull) != nseg) return 0;
            __hip_atomic_store(cnt, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return 1;
        }
    }
}

// Measurement hook: thread 0 of the block takes the 100 MHz real-time counter
// at one of eight points of kernel `kern` into LDS, and tl_flush copies the
// eight stamps to the timeline (layout [kern][1024 blocks][8 points], block =
// blockIdx.y * gridDim.x + blockIdx.x) when the block ends.  Point 0 clears
// the others first (a point not reached reads 0).  The stamps go through LDS
// so that a mark never waits behind the block's own weight loads in the
// vector memory queue.
__device__ __forceinline__ unsigned long long* tl_slots() {
    __shared__ unsigned long long slots[8];
    return slots;
}
__device__ __forceinline__ void tl_mark(unsigned long long* tl, int kern, int point) {
    (void)kern;
    if (tl && threadIdx.x == 0) {
        if (point == 0)
            for (int p = 1; p < 8; ++p) tl_slots()[p] = 0ull;
        tl_slots()[point] = __builtin_amdgcn_s_memrealtime();
    }
}
__device__ __forceinline__ void tl_flush(unsigned long long* tl, int kern) {
    if (tl && threadIdx.x == 0) {
        unsigned long long* dst = tl + ((size_t)kern * 1024 + blockIdx.y * gridDim.x + blockIdx.x) * 8;
        for (int p = 0; p < 8; ++p) dst[p] = tl_slots()[p];
    }
}

// floor(w * n / parts) in 32-bit arithmetic (the callers' products stay below
// 2^32: w <= parts <= 1024 and n < 2^22).  Operands that are uniform over the
// wave are moved to scalar registers first, so the division runs once per
// wave on the scalar unit instead of as a 64-lane sequence.
__device__ __forceinline__ int split_point(int w, int n, int parts) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_readfirstlane(w) * (uint32_t)__builtin_amdgcn_readfirstlane(n);
    return (int)(a / (uint32_t)__builtin_amdgcn_readfirstlane(parts));
}

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- cross-lane moves (DPP within rows of 16 lanes, permlane swaps across rows)
// dpp_ror<n>: lane i receives lane (i + n) mod 16 of its row.
template <int N>
__device__ __forceinline__ int dpp_ror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xf, 0xf, false); }
template <int N>
__device__ __forceinline__ float dpp_ror(float v) { return __int_as_float(dpp_ror<N>(__float_as_int(v))); }
// sum of the lane pairs (i, i ^ 16) / (i, i ^ 32): permlane swaps with both operands v
__device__ __forceinline__ int xor16_add(int v) {
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (int)r[0] + (int)r[1];
}
__device__ __forceinline__ int xor32_add(int v) {
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (int)r[0] + (int)r[1];
}
__device__ __forceinline__ float xor16_add(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ double dpp_ror8(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = dpp_ror<8>((int)(uint32_t)u), hi = dpp_ror<8>((int)(uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double xor16_add(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    auto lo = __builtin_amdgcn_permlane16_swap((int)(uint32_t)u, (int)(uint32_t)u, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((int)(uint32_t)(u >> 32), (int)(uint32_t)(u >> 32), false, false);
    const double a = __longlong_as_double((long long)(((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]));
    return a + b;
}
__device__ __forceinline__ double xor32_add(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    auto lo = __builtin_amdgcn_permlane32_swap((int)(uint32_t)u, (int)(uint32_t)u, false, false);
    auto hi = __builtin_amdgcn_permlane32_swap((int)(uint32_t)(u >> 32), (int)(uint32_t)(u >> 32), false, false);
    const double a = __longlong_as_double((long long)(((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]));
    return a + b;
}

// Wave-wide sum, every lane receives it.  Fixed order: ror 8, 4, 2, 1 inside
// each row of 16, then rows (0+1, 2+3), then halves.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_ror<8>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<1>(v);
    v = xor16_add(v);
    return xor32_add(v);
}

// Inclusive prefix sum over the wave (row_shr 1, 2, 4, 8, then row broadcasts),
// modulo 2^32 (callers pack two 16-bit counts into one word).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
    return x;
}

__device__ __forceinline__ int wave_max(int v) {
    v = max(v, dpp_ror<8>(v));
    v = max(v, dpp_ror<4>(v));
    v = max(v, dpp_ror<2>(v));
    v = max(v, dpp_ror<1>(v));
    {
        auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = max((int)r[0], (int)r[1]);
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = max((int)r[0], (int)r[1]);
    }
    return v;
}

// Exclusive prefix sum over the block in thread order, modulo 2^32; `total` =
// block sum.  `lds` holds >= 16 words.  Every thread of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, int* lds, uint32_t& total) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    uint32_t* l32 = reinterpret_cast<uint32_t*>(lds);
    if (lane == kWave - 1) l32[w] = incl;
    lds_barrier();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t c = l32[i];
        tot += c;
        off += i < w ? c : 0u;
    }
    lds_barrier();
    total = tot;
    return off + incl - v;
}

// The same for non-negative counts whose block total stays below 2^31.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* lds, int& total) {
    uint32_t tot;
    const uint32_t r = block_excl_scan_u32<NT>((uint32_t)v, lds, tot);
    total = (int)tot;
    return (int)r;
}

template <int NT>
__device__ __forceinline__ int block_max(int v, int* lds) {
    constexpr int NW = NT / kWave;
    v = wave_max(v);
    if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
    lds_barrier();
    int m = lds[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = max(m, lds[i]);
    lds_barrier();
    return m;
}

// Per-wave ballot counts of up to 4 predicates, then the block-wide exclusive
// positions (in thread order) and totals.  `wc` = [4][NT / 64] ints of LDS;
// ends with a barrier that makes `wc` reusable.
template <int NT, int NP>
__device__ __forceinline__ void block_ballot_pos(const bool (&p)[NP], int (*wc)[NT / kWave],
                                                 int (&pos)[NP], int (&tot)[NP]) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t m[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        m[i] = __ballot(p[i]);
        if (lane == 0) wc[i][wv] = __popcll(m[i]);
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        int off = 0, all = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const int c = wc[i][v];
            all += c;
            off += v < wv ? c : 0;
        }
        pos[i] = off + lanes_below(m[i]);
        tot[i] = all;
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------
// Keys with contiguous ownership: thread t holds elements t*P .. t*P + P - 1,
// read with 16-byte loads.  `readable` (a multiple of the vector width) bounds
// what may be read; elements at or beyond `n` are marked invalid.
// ---------------------------------------------------------------------------
template <int P>
__device__ __forceinline__ void load_u32_contig(const uint32_t* __restrict__ src, int n, int readable,
                                                uint32_t (&v)[P], bool (&valid)[P]) {
    static_assert(P % 4 == 0, "16-byte loads");
    const int base = (int)threadIdx.x * P;
#pragma unroll
    for (int q = 0; q < P; q += 4) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (base + q < readable) u = *reinterpret_cast<const uint4*>(src + base + q);
        v[q] = u.x; v[q + 1] = u.y; v[q + 2] = u.z; v[q + 3] = u.w;
    }
#pragma unroll
    for (int q = 0; q < P; ++q) valid[q] = base + q < n;
}

// Coalesced: 16-byte group g of thread t holds words (g * NT + t) * 4 .. + 3
// (each wave's load is one contiguous kilobyte).
template <int P, int NT>
__device__ __forceinline__ void load_u32_coal(const uint32_t* __restrict__ src, int n, int readable,
                                              uint32_t (&v)[P], bool (&valid)[P]) {
    static_assert(P % 4 == 0, "16-byte loads");
#pragma unroll
    for (int g = 0; g < P / 4; ++g) {
        const int i = (g * NT + (int)threadIdx.x) * 4;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (i < readable) u = *reinterpret_cast<const uint4*>(src + i);
        v[4 * g] = u.x; v[4 * g + 1] = u.y; v[4 * g + 2] = u.z; v[4 * g + 3] = u.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) valid[4 * g + e] = i + e < n;
    }
}

template <int P>
__device__ __forceinline__ void load_u16_contig(const uint16_t* __restrict__ src, int n, int readable,
                                                uint32_t (&v)[P], bool (&valid)[P]) {
    static_assert(P % 8 == 0, "16-byte loads");
    const int base = (int)threadIdx.x * P;
#pragma unroll
    for (int q = 0; q < P; q += 8) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (base + q < readable) u = *reinterpret_cast<const uint4*>(src + base + q);
        v[q] = u.x & 0xffffu; v[q + 1] = u.x >> 16;
        v[q + 2] = u.y & 0xffffu; v[q + 3] = u.y >> 16;
        v[q + 4] = u.z & 0xffffu; v[q + 5] = u.z >> 16;
        v[q + 6] = u.w & 0xffffu; v[q + 7] = u.w >> 16;
    }
#pragma unroll
    for (int q = 0; q < P; ++q) valid[q] = base + q < n;
}

// ---------------------------------------------------------------------------
// Block-wide radix selection pieces.  A threshold bin splits the keys: keys
// in higher bins are kept for certain, keys in the bin are candidates that the
// remaining (lower) bits and then the index order decide.  Every thread calls
// every step.
// ---------------------------------------------------------------------------
struct SelectState {
    uint32_t prefix;   // resolved high bits of the k-th largest key
    int shift;         // bits below the resolved ones
    int above;         // keys whose resolved bits exceed the prefix (all > T)
    int krem;          // k - above
    int ncand;         // candidates (keys whose resolved bits equal the prefix)
};

// Scan `nb` bins in descending order and find the one holding the krem-th key.
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int krem, int* sc,
                                         uint32_t& digit, int& above) {
    const int per = (nb + NT - 1) / NT;   // consecutive descending bins per thread
    int mine = 0;
    for (int q = 0; q < per; ++q) {
        const int r = threadIdx.x * per + q;
        if (r < nb) mine += (int)hist[nb - 1 - r];
    }
    int tot;
    int cum = block_excl_scan<NT>(mine, sc, tot);
    for (int q = 0; q < per; ++q) {
        const int r = threadIdx.x * per + q;
        if (r < nb) {
            const int c = (int)hist[nb - 1 - r];
            if (cum < krem && krem <= cum + c) {
                sc[20] = nb - 1 - r;
                sc[21] = cum;
            }
            cum += c;
        }
    }
    lds_barrier();
    digit = (uint32_t)sc[20];
    above = sc[21];
    lds_barrier();
}

// find_bin for nb = 4 * NT bins: thread t owns bins nb-1-4t .. nb-4-4t (one
// 16-byte LDS read; `hist` 16-byte aligned).
template <int NT>
__device__ __forceinline__ void find_bin4(const uint32_t* hist, int krem, int* sc, uint32_t& digit, int& above) {
    constexpr int nb = 4 * NT;
    const int t = threadIdx.x;
    const uint4 u = *reinterpret_cast<const uint4*>(hist + nb - 4 - 4 * t);
    const int c0 = (int)u.w, c1 = (int)u.z, c2 = (int)u.y, c3 = (int)u.x;   // descending bins
    int tot;
    const int cum = block_excl_scan<NT>(c0 + c1 + c2 + c3, sc, tot);
    if (cum < krem && krem <= cum + c0 + c1 + c2 + c3) {
        const int top = nb - 1 - 4 * t;
        if (krem <= cum + c0) { sc[20] = top; sc[21] = cum; }
        else if (krem <= cum + c0 + c1) { sc[20] = top - 1; sc[21] = cum + c0; }
        else if (krem <= cum + c0 + c1 + c2) { sc[20] = top - 2; sc[21] = cum + c0 + c1; }
        else { sc[20] = top - 3; sc[21] = cum + c0 + c1 + c2; }
    }
    lds_barrier();
    digit = (uint32_t)sc[20];
    above = sc[21];
    lds_barrier();
}

// The coarse digit from a histogram of the n valid keys: NB bins of
// key >> shift, thread t holding bins NB - (t + 1) * PER + i in c[i].  On
// success st holds the threshold bin (prefix), `above` = keys in higher bins
// and krem = k - above.  Returns false when the bins do not add up to n
// (a bin out of range, or a total that differs); the caller then ranks
// without them.  Requires 1 <= k <= n.
template <int NT, int NB>
__device__ __forceinline__ bool block_hist_bin_regs(const uint32_t (&c)[NB / NT], int k, int n, int shift, int* sc,
                                                    SelectState& st) {
    constexpr int PER = NB / NT;
    // Bins are checked one by one, so a thread's contribution is its true sum
    // (no wrap) or n + 1; the block total is n exactly when no bin is out of
    // range and the bins add up.
    uint32_t mine = 0;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        bad |= c[i] > (uint32_t)n;
        mine += c[i];
    }
    int tot;
    int cum = block_excl_scan<NT>(bad ? n + 1 : (int)min(mine, (uint32_t)n + 1u), sc, tot);
    if (tot != n) return false;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
        const int cnt = (int)c[i];
        if (cum < k && k <= cum + cnt) {
            sc[20] = NB - ((int)threadIdx.x + 1) * PER + i;
            sc[21] = cum;
        }
        cum += cnt;
    }
    lds_barrier();
    st = SelectState{(uint32_t)sc[20], shift, sc[21], k - sc[21], 0};
    lds_barrier();
    return true;
}

// The same from a histogram in LDS (`hist`, NB bins, 16-byte aligned) with
// the search spread over a wave: thread t sums bins NB - (t + 1) * PER ..
// NB - t * PER - 1, one block scan finds the thread whose bins hold the k-th
// largest key, and wave 0 finds the bin among that thread's PER bins with one
// wave scan (lane j <-> the j-th bin from the top).  No thread walks its bins
// one by one.  Same outputs and failure rule as block_hist_bin_regs.
template <int NT, int NB>
__device__ __forceinline__ bool block_hist_bin_wave(const uint32_t* hist, int k, int n, int shift, int* sc,
                                                    SelectState& st) {
    constexpr int PER = NB / NT;
    static_assert(PER % 4 == 0 && PER <= kWave, "16-byte reads; one lane per bin of a thread");
    const int t = threadIdx.x;
    uint32_t mine = 0, mx = 0;
    {
        const uint4* src = reinterpret_cast<const uint4*>(hist + NB - (t + 1) * PER);
#pragma unroll
        for (int v = 0; v < PER / 4; ++v) {
            const uint4 u = src[v];
            mine += u.x + u.y + u.z + u.w;
            mx = max(max(mx, max(u.x, u.y)), max(u.z, u.w));
        }
    }
    // a bin above n (a histogram that is not this token's) makes the total
    // differ from n; so does a sum that does not add up
    int tot;
    const int cum = block_excl_scan<NT>(mx > (uint32_t)n ? n + 1 : (int)min(mine, (uint32_t)n + 1u), sc, tot);
    if (tot != n) return false;
    if (cum < k && k <= cum + (int)mine) {
        sc[20] = t;
        sc[21] = cum;
    }
    lds_barrier();
    if (t < kWave) {
        const int ts = sc[20], cum0 = sc[21];
        const int bin = NB - 1 - ts * PER - t;
        const uint32_t cnt = t < PER ? hist[bin] : 0u;
        const uint32_t incl = wave_incl_scan(cnt);
        const uint64_t reach = __ballot(cum0 + (int)incl >= k);
        if (t == (int)__builtin_ctzll(reach)) {
            sc[22] = bin;
            sc[23] = cum0 + (int)(incl - cnt);
        }
    }
    lds_barrier();
    st = SelectState{(uint32_t)sc[22], shift, sc[23], k - sc[23], 0};
    return true;
}

// The coarse digit from the block's own keys: one radix digit of <= 11 bits
// in a window that starts at the highest bit set in any key (keys < 2^nbits).
// Same outputs as block_hist_bin_regs.  Requires 1 <= k <= number of valid keys.
template <int P, int NT>
__device__ __forceinline__ SelectState block_coarse_bin(const uint32_t (&key)[P], const bool (&valid)[P], int k,
                                        int nbits, uint32_t* hist, int* sc) {
    int kmax = 0;
#pragma unroll
    for (int q = 0; q < P; ++q) kmax = max(kmax, valid[q] ? (int)key[q] : 0);
    kmax = block_max<NT>(kmax, sc);
    int top = 32 - __clz(kmax);            // significant bits (0 when every key is 0)
    if (top > nbits) top = nbits;
    SelectState st{0u, top, 0, k, 0};       // bits at or above `top` are zero in every key
    if (top > 0) {
        const int dw = top >= 11 ? 11 : top;
        const int nb = 1 << dw;
        st.shift = top - dw;
        for (int b = threadIdx.x; b <= nb; b += NT) hist[b] = 0u;
        lds_barrier();
#pragma unroll
        for (int q = 0; q < P; ++q) atomicAdd(&hist[valid[q] ? (key[q] >> st.shift) : (uint32_t)nb], 1u);
        lds_barrier();
        uint32_t digit;
        find_bin<NT>(hist, nb, k, sc, digit, st.above);
        st.prefix = digit;
        st.krem = k - st.above;
    }
    return st;
}

// Remaining digits over the candidate array.  T = the k-th largest key,
// cgt = number of keys > T.
template <int NT>
__device__ __forceinline__ void block_select_refine(SelectState& st, const uint32_t* cand, uint32_t& T, int& cgt,
                                    uint32_t* hist, int* sc) {
    while (st.shift > 0) {
        const int dw = st.shift >= 11 ? 11 : st.shift;
        const int nb = 1 << dw;
        const int shift = st.shift - dw;
        for (int b = threadIdx.x; b < nb; b += NT) hist[b] = 0u;
        lds_barrier();
        for (int i = threadIdx.x; i < st.ncand; i += NT) {
            const uint32_t v = cand[i];
            if ((v >> st.shift) == st.prefix) atomicAdd(&hist[(v >> shift) & (nb - 1)], 1u);
        }
        lds_barrier();
        uint32_t digit;
        int ab;
        find_bin<NT>(hist, nb, st.krem, sc, digit, ab);
        st.above += ab;
        st.krem -= ab;
        st.prefix = (st.prefix << dw) | digit;
        st.shift = shift;
    }
    T = st.prefix;
    cgt = st.above;
}

}  // namespace prox
