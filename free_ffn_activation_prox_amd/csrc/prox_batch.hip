// Prox sparse SwiGLU FFN for batches of several tokens (gfx950 matrix cores).
//
// Each token keeps its own input set and its own channel mask (Prox, Abstract:
// Stage 1 ranks channels per token, one mask shared by the three projections;
// tokens are independent problems).  With several tokens most input rows and
// channels are kept by some token (at 8+ nearly all), so both stages become
// contractions over the union, run on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16):
//
//   input select  x~_b = x_b on its k_in largest |x| (lower index wins ties),
//                 0 elsewhere
//   proxy GEMM    g~ = X~ W~_gate, u~ = X~ W~_up over the quantized proxy.
//                 Codes are small integers and x is bf16, so every product is
//                 exact in fp32.  Four MFMAs (128 rows, one int4 group) chain
//                 in the fp32 accumulator, then the sum moves to fp64 (int4:
//                 times the group scale).  That fp32 sum of 128 exact
//                 products is not exact: its error is at most 127 * 2^-24 of
//                 the sum of the products' magnitudes (recursive summation;
//                 fewer roundings if the unit adds its 32 products at once).
//                 key = fp32(|silu(g~) u~|) with h~ formed in fp64.
//   selection     the per-token top-k_ff over the keys (the same kernel as the
//                 single-token path, selection only)
//   gate/up       G = X W_gate, U = X W_up over the channels some token keeps
//                 (PrunePath, §2.1, Eq. (1)); h = silu(g) u where the token
//                 keeps the channel, 0 elsewhere, stored as bf16 hi + lo
//   down          y = H W_down (COUNTDOWN, Abstract: y combines W_down rows
//                 weighted by h), hi and lo halves as two products, partial
//                 sums per channel slice, then the fixed-order reduction
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, r = l % 16, q = l / 16):
//   A[r][8q .. 8q + 7], B[8q .. 8q + 7][r], C[4q + i][r] for i < 4.
// The proxy codes and W_down are stored with the reduced dimension slowest,
// so their tiles are transposed through LDS on the way in.
#include "prox_device.hpp"
#include "prox_internal.hpp"

namespace prox {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Round to nearest even, finite inputs.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two rows' small integers -> one dword of two bf16 (row a low, row b high).
// The integers are exact in fp32 and in bf16, so the high half is the value.
__device__ __forceinline__ uint32_t pair_bf16(int qa, int qb) {
    return __builtin_amdgcn_perm(__float_as_uint((float)qb), __float_as_uint((float)qa), 0x07060302u);
}

// ===========================================================================
// Input selection: one block per token.  Thread t holds x[16t .. 16t + 15].
// Keys are |x| as bf16 bits (sign cleared, 15 bits), so the order of keys is
// the order of magnitudes.  T = the k-th largest key: a 2048-bin LDS
// histogram of key >> 4 gives its bin (one block scan), a 16-bin histogram of
// the low 4 bits of the keys in that bin gives T itself; keys above T are kept
// and keys equal to T are kept in index order until k are kept.
// ===========================================================================
constexpr int kXselPer = 16;   // keys per thread; blocks of d / 16 threads (d <= 16384)

template <int NT>
__global__ void __launch_bounds__(NT) k_xsel(const uint16_t* __restrict__ x, int d, int k,
                                                      uint16_t* __restrict__ xm, int32_t* __restrict__ in_idx) {
    __shared__ int sc[2][32];
    __shared__ uint32_t hist[2048 + 16];
    const int b = blockIdx.x, t = threadIdx.x;
    uint32_t v[kXselPer], key[kXselPer];
    bool valid[kXselPer];
    load_u16_contig<kXselPer>(x + (size_t)b * d, d, d, v, valid);
#pragma unroll
    for (int q = 0; q < kXselPer; ++q) key[q] = valid[q] ? (v[q] & 0x7fffu) : 0u;

    const bool all = k >= d, none = k <= 0;   // uniform over the block
    uint32_t T = 0;
    int cgt = 0;
    if (!all && !none) {
        for (int i = t; i < 2048 + 16; i += NT) hist[i] = 0u;
        lds_barrier();
#pragma unroll
        for (int q = 0; q < kXselPer; ++q)
            if (valid[q]) atomicAdd(&hist[key[q] >> 4], 1u);
        lds_barrier();
        uint32_t tb;
        int above;
        find_bin<NT>(hist, 2048, k, sc[0], tb, above);   // T's bin; `above` keys in higher bins
#pragma unroll
        for (int q = 0; q < kXselPer; ++q)
            if (valid[q] && (key[q] >> 4) == tb) atomicAdd(&hist[2048 + (key[q] & 15u)], 1u);
        lds_barrier();
        // every thread walks the 16 low-bit bins from the top
        int cum = above;
        bool found = false;
        T = tb << 4;
#pragma unroll
        for (int v2 = 15; v2 >= 0; --v2) {
            const int c = (int)hist[2048 + v2];
            if (!found && cum + c >= k) {
                T = (tb << 4) + (uint32_t)v2;
                found = true;
            }
            cum += found ? 0 : c;
        }
        cgt = cum;                                         // keys > T
    }
    const int need = k - cgt;   // keys equal to T that are kept, lowest indices first
    int neq = 0;
#pragma unroll
    for (int q = 0; q < kXselPer; ++q) neq += (valid[q] && key[q] == T) ? 1 : 0;
    int tot;
    int eq_before = block_excl_scan<NT>(neq, sc[0], tot);
    bool keep[kXselPer];
    int nk = 0;
#pragma unroll
    for (int q = 0; q < kXselPer; ++q) {
        const bool eq = valid[q] && key[q] == T;
        keep[q] = valid[q] && (all || (!none && (key[q] > T || (eq && eq_before < need))));
        eq_before += eq ? 1 : 0;
        nk += keep[q] ? 1 : 0;
    }
    int pos = block_excl_scan<NT>(nk, sc[1], tot);
    const int base = t * kXselPer;
#pragma unroll
    for (int q = 0; q < kXselPer; q += 8) {
        if (base + q < d) {
            uint32_t wv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wv[e] = (keep[q + 2 * e] ? v[q + 2 * e] : 0u) | ((keep[q + 2 * e + 1] ? v[q + 2 * e + 1] : 0u) << 16);
            *reinterpret_cast<uint4*>(xm + (size_t)b * d + base + q) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
    if (in_idx) {
#pragma unroll
        for (int q = 0; q < kXselPer; ++q)
            if (keep[q]) in_idx[(size_t)b * k + pos++] = base + q;
    }
}

hipError_t launch_xsel(const uint16_t* x, int B, int d, int k_in, uint16_t* xm, int32_t* in_idx,
                       hipStream_t s) {
    const int per_block = (d + kXselPer - 1) / kXselPer;
    if (per_block <= 256) launch_kernel(k_xsel<256>, dim3(B), dim3(256), 0, s, x, d, k_in, xm, in_idx);
    else if (per_block <= 512) launch_kernel(k_xsel<512>, dim3(B), dim3(512), 0, s, x, d, k_in, xm, in_idx);
    else launch_kernel(k_xsel<1024>, dim3(B), dim3(1024), 0, s, x, d, k_in, xm, in_idx);
    return hipGetLastError();
}

// ===========================================================================
// Proxy GEMM.  Block (tile, split): the tile's TC channels (64 int8 / 128
// int4) over rows [r0, r1) of the split, every token.  Wave w owns M-tile w
// (channels 16w .. 16w + 15 of the tile, gate and up) and works on its own:
// rows go 128 at a time ("stages"), lane l loads rows 2l and 2l + 1 of the
// wave's columns (int4: one 16-byte column block, int8: two), turns the codes
// into bf16 and writes them to the wave's LDS region transposed,
// [mat][channel][row], one dword (two rows) per write; the MFMA A operand (16
// channels x 8 rows per lane) is then one 16-byte LDS read.  A wave's LDS
// operations complete in order, so no barrier separates the writes from the
// reads.  B is x~ (token-major, rows contiguous), read from global memory.
// A stage is one 128-row group: its fp32 sums go to fp64 after the stage
// (int4: times the group's scales, which travel with the stage's loads).
// ===========================================================================
struct PbArgs {
    const uint16_t* xm;       // [B][d] x~
    const uint8_t* codes;     // [tiles][d][128 B]
    const float* scales;      // gate [groups][f_pad], up [groups][f_pad]
    int B, d, F, f_pad, groups, tiles, ks1, rps;
    float* part;              // [ks1][2][B][f_pad] split partial sums (ks1 > 1)
    unsigned long long* tcnt; // [tiles] arrival counters
    uint32_t gen;
    float* key;               // [B][f_pad]
    double* h_tap;            // [B][F] or null
    float* key_tap;           // [B][F] or null
};

// Cache policy of a buffer access (gfx950): bit 4 = sc1.  With it a store or
// load is coherent across the chip's L2 caches, like a device-scope atomic.
constexpr int kCoherent = 16;

constexpr int kPbRS = 136;    // LDS row stride of a transposed channel, in bf16 (128 + 8)
constexpr int kPbWave = 2 * 16 * kPbRS;   // bf16 per wave region

template <int KIND, int NG>
struct PbStage {
    uint4 c[KIND == 1 ? 4 : 2];   // rows 2l, 2l + 1 (int8: two column blocks each)
    uint4 x[4][NG];               // B operands of the stage's four K-steps
    float4 sg, su;                // int4: the group's scales of this lane's channels
};

__device__ __forceinline__ void pb_score(const PbArgs& a, int b, int j, double g, double u) {
    const double h = g / (1.0 + exp(-g)) * u;
    const float kf = (float)fabs(h);
    a.key[(size_t)b * a.f_pad + j] = kf;
    if (a.h_tap) a.h_tap[(size_t)b * a.F + j] = h;
    if (a.key_tap) a.key_tap[(size_t)b * a.F + j] = kf;
}

template <int KIND, int NG, int PD>
__global__ void __launch_bounds__(KIND == 1 ? 256 : 512) k_proxy_batch(PbArgs a) {
    constexpr int TC = KIND == 1 ? 64 : 128;   // channels of a tile
    constexpr int NW = TC / 16;                // waves (M-tiles)
    extern __shared__ uint4 pb_dyn[];
    __shared__ int flag;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int r = l & 15, q4 = l >> 4;
    uint16_t* buf = reinterpret_cast<uint16_t*>(pb_dyn) + w * kPbWave;
    const int tile = blockIdx.x / a.ks1, split = blockIdx.x % a.ks1;
    const int d = a.d;
    const int r0 = split * a.rps, r1 = min(d, r0 + a.rps);
    const int ch0 = tile * TC + 16 * w;        // this wave's first channel

    const uint32_t codes_bytes = (uint32_t)a.tiles * (uint32_t)d * kTileRowBytes;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, codes_bytes);
    const uint32_t tile_off = (uint32_t)tile * (uint32_t)d * kTileRowBytes;
    const uint32_t col_off = KIND == 1 ? 32u * w : 16u * w;
    const uint32_t x_bytes = (uint32_t)a.B * (uint32_t)d * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xm, x_bytes);
    uint32_t xrow[NG];   // byte offset of this lane's B-operand token row, or past the end
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int n = 16 * g + r;
        xrow[g] = n < a.B ? (uint32_t)n * (uint32_t)d * 2u : x_bytes;
    }
    const float* sg_base = a.scales + ch0 + 4 * q4;
    const float* su_base = sg_base + (size_t)a.groups * a.f_pad;

    auto load_stage = [&](int s, PbStage<KIND, NG>& st) {
        const int rb = r0 + 128 * s;
        if (KIND == 2) {
            const int gi = min(rb / 128, a.groups - 1);
            st.sg = *reinterpret_cast<const float4*>(sg_base + (size_t)gi * a.f_pad);
            st.su = *reinterpret_cast<const float4*>(su_base + (size_t)gi * a.f_pad);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = rb + 2 * l + h;
            const uint32_t off = row < r1 ? (uint32_t)row * kTileRowBytes + col_off : codes_bytes;
            if (KIND == 1) {
                st.c[2 * h] = buf_load16(rc, off, tile_off);
                st.c[2 * h + 1] = buf_load16(rc, row < r1 ? off + 16u : codes_bytes, tile_off);
            } else {
                st.c[h] = buf_load16(rc, off, tile_off);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = rb + 32 * ks + 8 * q4;
#pragma unroll
            for (int g = 0; g < NG; ++g)
                st.x[ks][g] = buf_load16(rx, (row < r1 && xrow[g] < x_bytes) ? xrow[g] + (uint32_t)row * 2u : x_bytes, 0);
        }
    };

    // code of channel c (0..15) of matrix mat in row h (0: row 2l, 1: row 2l + 1)
    auto code = [&](const PbStage<KIND, NG>& st, int h, int mat, int c) -> int {
        if (KIND == 1) {
            const uint4 v = st.c[2 * h + c / 8];
            const uint32_t wd = (mat == 0 ? ((c & 7) < 4 ? v.x : v.y) : ((c & 7) < 4 ? v.z : v.w));
            return __builtin_amdgcn_sbfe((int)wd, 8 * (c % 4), 8);
        } else {
            const uint4 v = st.c[h];
            const uint32_t wd = (mat == 0 ? (c < 8 ? v.x : v.y) : (c < 8 ? v.z : v.w));
            return __builtin_amdgcn_sbfe((int)wd, 4 * (c % 8), 4);
        }
    };
    // rows 2l, 2l + 1 of every channel -> one dword at [mat][channel][2l]
    auto store_stage = [&](const PbStage<KIND, NG>& st) {
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
#pragma unroll
            for (int c = 0; c < 16; ++c)
                *reinterpret_cast<uint32_t*>(buf + (mat * 16 + c) * kPbRS + 2 * l) =
                    pair_bf16(code(st, 0, mat, c), code(st, 1, mat, c));
    };

    f32x4_t acc[2][NG];
    double dacc[2][NG][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            acc[m][g] = zero4();
#pragma unroll
            for (int i = 0; i < 4; ++i) dacc[m][g][i] = 0.0;
        }

    auto mma_stage = [&](const PbStage<KIND, NG>& st) {
        uint4 av[4][2];   // every A operand of the stage first, then the products
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                av[ks][m] = *reinterpret_cast<const uint4*>(buf + (m * 16 + r) * kPbRS + 32 * ks + 8 * q4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int g = 0; g < NG; ++g) acc[m][g] = mfma16(av[ks][m], st.x[ks][g], acc[m][g]);
    };

    auto flush = [&](const PbStage<KIND, NG>& st) {
        const float s4[2][4] = {{st.sg.x, st.sg.y, st.sg.z, st.sg.w}, {st.su.x, st.su.y, st.su.z, st.su.w}};
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dacc[m][g][i] += KIND == 2 ? (double)acc[m][g][i] * (double)s4[m][i] : (double)acc[m][g][i];
                acc[m][g] = zero4();
            }
    };

    const int nst = (r1 - r0 + 127) / 128;
    PbStage<KIND, NG> ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
        load_stage(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);   // issue order = consumption order
    }
    // whole rounds of PD stages; stages past the split read zeros
    for (int s0 = 0; s0 < nst; s0 += PD) {
#pragma unroll
        for (int i = 0; i < PD; ++i) {
            store_stage(ring[i]);
            asm volatile("" ::: "memory");   // the LDS reads below follow the writes
            mma_stage(ring[i]);
            flush(ring[i]);
            __builtin_amdgcn_sched_barrier(0);
            load_stage(s0 + i + PD, ring[i]);
            __builtin_amdgcn_sched_barrier(0);
            // the waves read 16-byte pieces of the same 128-byte code lines;
            // kept within a stage of each other they find the lines still
            // in the L2 (no wait for memory here: loads stay in flight)
            asm volatile("s_barrier" ::: "memory");
        }
    }

    // this lane: gate / up of channels ch0 + 4 q4 + i, tokens 16 g + r
    if (a.ks1 > 1) {
        // publish this split's sums; the block that completes the tile adds the
        // splits in order.  The 16-byte stores and loads carry the sc1 cache
        // policy (the one the compiler gives device-scope atomics), which keeps
        // them coherent across the chip's L2 caches; the stores complete before
        // the arrival is counted.
        const uint32_t part_bytes = (uint32_t)a.ks1 * 2u * (uint32_t)a.B * (uint32_t)a.f_pad * 4u;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part, part_bytes);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int n = 16 * g + r;
                if (n < a.B) {
                    const uint32_t off =
                        ((((uint32_t)split * 2u + m) * (uint32_t)a.B + n) * (uint32_t)a.f_pad + ch0 + 4 * q4) * 4u;
                    const u32x4_t v = {__float_as_uint((float)dacc[m][g][0]), __float_as_uint((float)dacc[m][g][1]),
                                       __float_as_uint((float)dacc[m][g][2]), __float_as_uint((float)dacc[m][g][3])};
                    __builtin_amdgcn_raw_buffer_store_b128(v, rp, (int)off, 0, kCoherent);
                }
            }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
        __syncthreads();
        if (t == 0) flag = tile_arrive(a.tcnt + tile, a.gen, a.ks1);
        __syncthreads();
        if (!flag) return;
        // the splits in order; each split's 2 NG loads are in flight together
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) dacc[m][g][i] = 0.0;
        for (int sp = 0; sp < a.ks1; ++sp) {
            u32x4_t v[2][NG];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int n = 16 * g + r;
                    const uint32_t off =
                        ((((uint32_t)sp * 2u + m) * (uint32_t)a.B + n) * (uint32_t)a.f_pad + ch0 + 4 * q4) * 4u;
                    v[m][g] = n < a.B ? __builtin_amdgcn_raw_buffer_load_b128(rp, (int)off, 0, kCoherent)
                                      : u32x4_t{0u, 0u, 0u, 0u};
                }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    dacc[m][g][0] += (double)__uint_as_float(v[m][g].x);
                    dacc[m][g][1] += (double)__uint_as_float(v[m][g].y);
                    dacc[m][g][2] += (double)__uint_as_float(v[m][g].z);
                    dacc[m][g][3] += (double)__uint_as_float(v[m][g].w);
                }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = ch0 + 4 * q4 + i;
        if (j >= a.F) continue;
        double sg = 1.0, su = 1.0;
        if (KIND == 1) {
            sg = (double)a.scales[j];
            su = (double)a.scales[a.f_pad + j];
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int n = 16 * g + r;
            if (n < a.B) pb_score(a, n, j, dacc[0][g][i] * sg, dacc[1][g][i] * su);
        }
    }
}

// Row splits of the proxy GEMM: about kPbWaves waves over the chip (tiles x
// waves per tile x splits), splits of whole 128-row groups, at most
// kPbMaxSplits.  Depends on the shape only (the workspace is sized from it).
constexpr int kPbWaves = 1536;
constexpr int kPbMaxSplits = 8;

PbSplit proxy_batch_split(int d, int F, int kind) {
    const int tiles = f_pad_of(F, kind) / tile_channels(kind);
    const int waves = tiles * (kind == 1 ? 4 : 8);
    const int groups = (d + 127) / 128;
    int ks = (kPbWaves + waves - 1) / waves;
    if (ks > kPbMaxSplits) ks = kPbMaxSplits;
    if (ks > groups) ks = groups;
    if (ks < 1) ks = 1;
    const int gps = (groups + ks - 1) / ks;   // groups per split
    PbSplit r;
    r.rps = gps * 128;
    r.ks1 = (d + r.rps - 1) / r.rps;
    return r;
}

template <int KIND, int NG, int PD>
static hipError_t go_proxy_batch(const PbArgs& a, hipStream_t s) {
    constexpr int NW = KIND == 1 ? 4 : 8;
    const size_t dyn = (size_t)NW * kPbWave * 2;
    auto fn = k_proxy_batch<KIND, NG, PD>;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    launch_kernel(fn, dim3(a.tiles * a.ks1), dim3(NW * 64), dyn, s, a);
    return hipGetLastError();
}

template <int KIND>
static hipError_t proxy_batch_ng(const PbArgs& a, hipStream_t s) {
    const int ng = (a.B + 15) / 16;
    if (ng == 1) return go_proxy_batch<KIND, 1, 2>(a, s);
    if (ng == 2) return go_proxy_batch<KIND, 2, 2>(a, s);
    if (ng == 3) return go_proxy_batch<KIND, 3, 1>(a, s);
    return go_proxy_batch<KIND, 4, 1>(a, s);
}

hipError_t launch_proxy_batch(const uint16_t* xm, int B, int d, const ProxyView& p, float* part,
                              unsigned long long* tcnt, uint32_t gen, float* key, double* h_tap,
                              float* key_tap, hipStream_t s) {
    const PbSplit sp = proxy_batch_split(d, p.F, p.kind);
    PbArgs a{xm, p.codes, p.scales, B, d, p.F, p.f_pad, p.groups, p.f_pad / tile_channels(p.kind),
             sp.ks1, sp.rps, part, tcnt, gen, key, h_tap, key_tap};
    return p.kind == 1 ? proxy_batch_ng<1>(a, s) : proxy_batch_ng<2>(a, s);
}

// ===========================================================================
// Gate/up.  Block: 16·MTW channels j0 .. (the MFMA's M, MTW tiles of 16 per
// wave), every token (N, 16 per group), K = d split over the 4 waves, 64
// columns each per stage.  Weight rows and x are K-contiguous, so both
// operands are 16-byte buffer loads straight into registers; channels that no
// token keeps, tokens past B and columns past d read at an offset past the end
// (zeros, no traffic).  With two M-tiles per wave each x operand feeds four
// products.  Two K-steps per stage, PD stages in flight; the 4 waves' sums are
// added in LDS in a fixed order.
// ===========================================================================
struct GuArgs {
    const uint16_t* x;      // [B][d]
    const uint16_t* wg_t;   // [F][d]
    const uint16_t* wu_t;
    const uint8_t* mask;    // [B][F]
    uint16_t* hb;           // [2][B][f_pad] h as bf16 hi, lo
    int B, d, F, f_pad;
};

constexpr int kGuSteps = 2;

template <int NG, int MTW>
struct GuStage {
    uint4 g[kGuSteps][MTW], u[kGuSteps][MTW], x[kGuSteps][NG];
};

template <int NG, int MTW>
__global__ void __launch_bounds__(256) k_gateup_batch(GuArgs a) {
    constexpr int PD = MTW == 1 ? 4 : 3;   // stages in flight
    constexpr int CH = 16 * MTW;           // channels of the block
    __shared__ uint32_t used[CH];
    __shared__ uint8_t mk[16 * NG][CH];     // the tokens' mask bytes of the block's channels
    __shared__ float red[4][NG][2][4][64];
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int r = l & 15, q4 = l >> 4;
    const int j0 = blockIdx.x * CH;
    const int d = a.d;

    // the mask bytes of the block's channels (every load issued before the
    // first is waited for), then the channels that some token keeps
    {
        constexpr int NE = (16 * NG * CH + 255) / 256;
        uint8_t mv[NE];
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = t + 256 * u, n = e / CH, c = e % CH;
            mv[u] = (n < a.B && j0 + c < a.F) ? a.mask[(size_t)n * a.F + j0 + c] : (uint8_t)0;
        }
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = t + 256 * u;
            if (e < 16 * NG * CH) mk[e / CH][e % CH] = mv[u];
        }
    }
    __syncthreads();
    if (t < CH) {
        uint32_t any = 0;
        for (int n = 0; n < a.B; ++n) any |= mk[n][t];
        used[t] = any ? 1u : 0u;
    }
    __syncthreads();

    const uint32_t row_bytes = (uint32_t)d * 2u;
    const uint32_t w_bytes = (uint32_t)a.F * row_bytes, x_bytes = (uint32_t)a.B * row_bytes;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.wg_t, w_bytes), ru = make_rsrc(a.wu_t, w_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, x_bytes);
    uint32_t woff[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int j = j0 + 16 * mt + r;
        woff[mt] = (j < a.F && used[16 * mt + r]) ? (uint32_t)j * row_bytes : w_bytes;
    }
    uint32_t xoff[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int n = 16 * g + r;
        xoff[g] = n < a.B ? (uint32_t)n * row_bytes : x_bytes;
    }
    // wave w reads columns 64 w .. 64 w + 63 of each stage (whole 128-byte
    // lines of its rows), lane column 8 q4 in each of the two 32-wide steps
    const int kl = 64 * w + 8 * q4;
    constexpr int KS = 128 * kGuSteps;   // columns per stage (all 4 waves)

    auto load = [&](int s, GuStage<NG, MTW>& st) {
#pragma unroll
        for (int q = 0; q < kGuSteps; ++q) {
            const int k = KS * s + 32 * q + kl;
            const bool ok = k < d;   // d % 8 == 0: a lane's 8 columns are all in or all out
            const uint32_t kbytes = (uint32_t)k * 2u;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) {
                st.g[q][mt] = buf_load16(rg, ok && woff[mt] < w_bytes ? woff[mt] + kbytes : w_bytes, 0);
                st.u[q][mt] = buf_load16(ru, ok && woff[mt] < w_bytes ? woff[mt] + kbytes : w_bytes, 0);
            }
#pragma unroll
            for (int g = 0; g < NG; ++g)
                st.x[q][g] = buf_load16(rx, ok && xoff[g] < x_bytes ? xoff[g] + kbytes : x_bytes, 0);
        }
    };
    f32x4_t ag[MTW][NG], au[MTW][NG];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int g = 0; g < NG; ++g) ag[mt][g] = au[mt][g] = zero4();
    auto mma = [&](const GuStage<NG, MTW>& st) {
#pragma unroll
        for (int q = 0; q < kGuSteps; ++q)
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    ag[mt][g] = mfma16(st.g[q][mt], st.x[q][g], ag[mt][g]);
                    au[mt][g] = mfma16(st.u[q][mt], st.x[q][g], au[mt][g]);
                }
    };

    const int nst = (d + KS - 1) / KS;
    GuStage<NG, MTW> ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
        load(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);   // issue order = consumption order
    }
    // whole rounds of PD stages; stages past d read zeros.  The scheduling
    // barriers keep each refill right behind the products that free its
    // registers, so PD - 1 stages stay in flight.
    for (int s0 = 0; s0 < nst; s0 += PD) {
#pragma unroll
        for (int i = 0; i < PD; ++i) {
            mma(ring[i]);
            __builtin_amdgcn_sched_barrier(0);
            load(s0 + i + PD, ring[i]);
            __builtin_amdgcn_sched_barrier(0);
            // the 4 waves request adjacent 128-byte pieces of the same rows:
            // kept within a stage of each other (loads stay in flight)
            asm volatile("s_barrier" ::: "memory");
        }
    }
    // the 4 waves' K quarters, one M-tile at a time: channel j0 + 16 mt + 4 q4 + i, token 16 g + r
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        if (mt > 0) __syncthreads();   // `red` is reused
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[w][g][0][i][l] = ag[mt][g][i];
                red[w][g][1][i][l] = au[mt][g][i];
            }
        __syncthreads();
        // wave w finishes token groups w, w + 4, ...
        for (int g = w; g < NG; g += 4) {
            const int n = 16 * g + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jc = j0 + 16 * mt + 4 * q4 + i;
                // channels past F (up to the block's end) get h = 0: the down
                // projection reads h 8 channels at a time
                if (n < a.B) {
                    float gg = 0.f, uu = 0.f;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        gg += red[v][g][0][i][l];
                        uu += red[v][g][1][i][l];
                    }
                    float hv = gg / (1.f + expf(-gg)) * uu;
                    if (jc >= a.F || !mk[n][16 * mt + 4 * q4 + i]) hv = 0.f;
                    const uint32_t hi = bf16_rne(hv);
                    const uint32_t lo = bf16_rne(hv - __uint_as_float(hi << 16));
                    a.hb[(size_t)n * a.f_pad + jc] = (uint16_t)hi;
                    a.hb[((size_t)a.B + n) * a.f_pad + jc] = (uint16_t)lo;
                }
            }
        }
    }
}

// ===========================================================================
// Down.  Block (cx, ks): columns 128 cx .. + 128 and channel slice ks (rows
// [f0, f1), a multiple of 64 long), every token.  Rows go 64 at a time: each
// thread loads 4 rows of one 8-column block of W_down and writes them to LDS
// transposed, [column][row], so the B operand (one column, 8 rows per lane)
// is a 16-byte LDS read.  Wave w owns columns 32 w .. + 32 (two N-tiles); the
// A operand is h (hi, then lo) for 16 tokens x 8 channels, 16-byte loads from
// the [B][f_pad] arrays.  Partial y of slice ks goes to ypart[token][ks][col].
// ===========================================================================
struct DnArgs {
    const uint16_t* wd;     // [F][d]
    const uint16_t* hb;     // [2][B][f_pad]
    float* ypart;           // [B][KS][d]
    int B, d, F, f_pad, KS, chunk;
};

constexpr int kDnCols = 128;
constexpr int kDnRS = 72;

template <int NG>
struct DnStage {
    uint4 w[4];             // rows 4p .. 4p + 3 of this thread's column block
    uint4 h[2][NG][2];      // [K-step][token group][hi, lo]
};

template <int NG>
__global__ void __launch_bounds__(256) k_down_batch(DnArgs a) {
    constexpr int PD = NG == 1 ? 4 : (NG == 2 ? 3 : 2);   // stages in flight
    constexpr int TILE = kDnCols * kDnRS;      // bf16 per LDS buffer
    __shared__ uint4 lds_raw[2 * TILE / 8];
    uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int r = l & 15, q4 = l >> 4;
    const int c0 = blockIdx.x * kDnCols, ks = blockIdx.y;
    const int f0 = ks * a.chunk, f1 = min(a.F, f0 + a.chunk);
    const int d = a.d;
    const uint32_t row_bytes = (uint32_t)d * 2u, w_bytes = (uint32_t)a.F * row_bytes;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wd, w_bytes);
    const uint32_t h_bytes = 2u * (uint32_t)a.B * (uint32_t)a.f_pad * 2u;
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hb, h_bytes);
    // W loads: thread t -> column block cb (8 columns), rows 4p .. 4p + 3
    const int cb = t & 15, p = t >> 4;
    const bool col_ok = c0 + 8 * cb < d;   // d % 8 == 0
    const uint32_t col_off = (uint32_t)(c0 + 8 * cb) * 2u;
    uint32_t hrow[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int n = 16 * g + r;
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
            hrow[g][hl] = n < a.B ? ((uint32_t)hl * a.B + n) * (uint32_t)a.f_pad * 2u : h_bytes;
    }

    auto load_stage = [&](int s, DnStage<NG>& st) {
        const int rb = f0 + 64 * s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rb + 4 * p + i;
            st.w[i] = buf_load16(rw, (col_ok && row < f1) ? (uint32_t)row * row_bytes + col_off : w_bytes, 0);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int row = rb + 32 * kk + 8 * q4;
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    st.h[kk][g][hl] =
                        buf_load16(rh, (row < f1 && hrow[g][hl] < h_bytes) ? hrow[g][hl] + (uint32_t)row * 2u : h_bytes, 0);
        }
    };
    // 8 columns x 4 rows -> [column][rows 4p .. 4p + 3] (8 bytes per column)
    auto store_stage = [&](const DnStage<NG>& st, uint16_t* buf) {
        const int chunk = (p >> 1) ^ (cb & 7), sub = 4 * (p & 1);
        const uint32_t w0[4] = {st.w[0].x, st.w[0].y, st.w[0].z, st.w[0].w};
        const uint32_t w1[4] = {st.w[1].x, st.w[1].y, st.w[1].z, st.w[1].w};
        const uint32_t w2[4] = {st.w[2].x, st.w[2].y, st.w[2].z, st.w[2].w};
        const uint32_t w3[4] = {st.w[3].x, st.w[3].y, st.w[3].z, st.w[3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int wi = e / 2;
            // the column's bf16 from rows 0/1 and 2/3 (low half = the lower row)
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t lo01 = __builtin_amdgcn_perm(w1[wi], w0[wi], sel);
            const uint32_t lo23 = __builtin_amdgcn_perm(w3[wi], w2[wi], sel);
            *reinterpret_cast<uint2*>(buf + (8 * cb + e) * kDnRS + 8 * chunk + sub) = make_uint2(lo01, lo23);
        }
    };
    f32x4_t acc[2][NG];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[u][g] = zero4();
    auto mma_stage = [&](const DnStage<NG>& st, const uint16_t* buf) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int col = 32 * w + 16 * u + r;
                const int chunk = (4 * kk + q4) ^ ((col >> 3) & 7);
                const uint4 bv = *reinterpret_cast<const uint4*>(buf + col * kDnRS + 8 * chunk);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    acc[u][g] = mfma16(st.h[kk][g][0], bv, acc[u][g]);
                    acc[u][g] = mfma16(st.h[kk][g][1], bv, acc[u][g]);
                }
            }
        }
    };

    const int nst = (f1 - f0 + 63) / 64;
    DnStage<NG> ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
        load_stage(i, ring[i]);
        __builtin_amdgcn_sched_barrier(0);   // issue order = consumption order
    }
    for (int s0 = 0; s0 < nst; s0 += PD) {
#pragma unroll
        for (int i = 0; i < PD; ++i) {
            // alternate buffers by the global stage index: with an odd PD,
            // (i & 1) would give the last stage of a round and the first of
            // the next the same buffer, and a wave could overwrite it while
            // another still reads it (one barrier per stage only orders
            // stages that use different buffers)
            uint16_t* buf = lds + ((s0 + i) & 1) * TILE;
            store_stage(ring[i], buf);
            lds_barrier();
            mma_stage(ring[i], buf);
            load_stage(s0 + i + PD, ring[i]);
        }
    }
    // C[token 16 g + 4 q4 + i][column 32 w + 16 u + r]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = c0 + 32 * w + 16 * u + r;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 16 * g + 4 * q4 + i;
                if (n < a.B && c < d) a.ypart[((size_t)n * a.KS + ks) * d + c] = acc[u][g][i];
            }
    }
}

// Channel slices of the down projection: about 2 blocks per compute unit,
// whole 64-row stages, at most what the partial-sum region holds.
DnSplit down_batch_split(int B, int d, int F) {
    const int cols = (d + kDnCols - 1) / kDnCols;
    int ks = (512 + cols - 1) / cols;
    const int stages = (F + 63) / 64;
    if (ks > stages) ks = stages;
    if (ks > stage2_blocks_max(B)) ks = stage2_blocks_max(B);
    if (ks < 1) ks = 1;
    DnSplit r;
    r.chunk = (stages + ks - 1) / ks * 64;
    r.KS = (F + r.chunk - 1) / r.chunk;
    return r;
}

template <int NG>
static hipError_t go_gateup_down(const GuArgs& gu, const DnArgs& dn, hipStream_t s) {
    // two M-tiles per wave when x has two or more token groups (x operand reuse)
    constexpr int MTW = NG >= 2 ? 2 : 1;
    launch_kernel(k_gateup_batch<NG, MTW>, dim3((gu.F + 16 * MTW - 1) / (16 * MTW)), dim3(256), 0, s, gu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(k_down_batch<NG>, dim3((dn.d + kDnCols - 1) / kDnCols, dn.KS), dim3(256), 0, s, dn);
    return hipGetLastError();
}

hipError_t launch_stage2_batch(const uint16_t* x, const uint16_t* wg_t, const uint16_t* wu_t,
                               const uint16_t* wd, const uint8_t* mask, uint16_t* hb, int B, int d,
                               int F, int f_pad, float* ypart, int* ks_out, hipStream_t s) {
    const DnSplit sp = down_batch_split(B, d, F);
    *ks_out = sp.KS;
    GuArgs gu{x, wg_t, wu_t, mask, hb, B, d, F, f_pad};
    DnArgs dn{wd, hb, ypart, B, d, F, f_pad, sp.KS, sp.chunk};
    const int ng = (B + 15) / 16;
    if (ng == 1) return go_gateup_down<1>(gu, dn, s);
    if (ng == 2) return go_gateup_down<2>(gu, dn, s);
    if (ng == 3) return go_gateup_down<3>(gu, dn, s);
    return go_gateup_down<4>(gu, dn, s);
}

}  // namespace prox
