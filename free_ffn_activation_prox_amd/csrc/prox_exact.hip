// Exact-mask mode and quality diagnostics.
//
// Exact mode ranks the channels by the exact intermediate instead of a proxy:
// every input kept, the weights themselves as the proxy, so the mask is the
// top-k of |h| with h_j = silu(x . W_gate[:, j]) (x . W_up[:, j]) over every
// channel -- the selector Prox approximates ("Prox: ...", Abstract: the mask
// the intermediate state induces; "COUNTDOWN: ...", Abstract: selection on
// the actual coefficients).  Stage 1 here computes that h for every channel in
// fp64 (a bf16 x bf16 product is exact, the sums run in fp64) and its fp32
// ranking key; the usual Stage-2 selection then keeps the top k_ff and
// streams only their W_down rows, with h read back instead of recomputed.
//
// The diagnostics compare a forward with a reference: kept channels in common
// (mask recall = common / k_ff) and the relative L2 error of y.
#include "prox.h"
#include "prox_device.hpp"
#include "prox_internal.hpp"

namespace prox {

template <int N>
__device__ __forceinline__ double dpp_ror_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = dpp_ror<N>((int)(uint32_t)u), hi = dpp_ror<N>((int)(uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Wave-wide fp64 sum in a fixed order (ror 8, 4, 2, 1 in each row of 16, then
// rows pairwise); every lane receives it.
__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_ror_d<8>(v);
    v += dpp_ror_d<4>(v);
    v += dpp_ror_d<2>(v);
    v += dpp_ror_d<1>(v);
    return xor32_add(xor16_add(v));
}

__device__ __forceinline__ int wave_sum_i(int v) {
    v += dpp_ror<8>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<1>(v);
    return xor32_add(xor16_add(v));
}

constexpr int kExThreads = 256;
constexpr int kExParts = 8;     // 16-byte parts of a row in flight per lane and row

// grid (nb, B), block 256 (4 waves).  Wave gw = 4 * blockIdx.x + w takes
// channels gw, gw + 4 nb, ...  x is staged in LDS as fp32.  A lane reads
// 16-byte parts (8 weights) p = 64 u + lane of the gate and up rows, eight of
// each in flight, and accumulates x_i w_ij in fp64.
__global__ void __launch_bounds__(kExThreads) k_exact_h(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ wg_t,
                                                        const uint16_t* __restrict__ wu_t, int d, int F, int f_pad,
                                                        float* __restrict__ key, double* __restrict__ hbuf,
                                                        double* __restrict__ h_tap, float* __restrict__ key_tap,
                                                        int32_t* __restrict__ in_idx_tap,
                                                        unsigned long long* tl) {
    extern __shared__ float xs[];                 // [d]
    const int b = blockIdx.y, t = threadIdx.x, w = t >> 6, l = t & 63;
    tl_mark(tl, 0, 0);
    for (int i = t; i < d; i += kExThreads) {
        xs[i] = bf16f(x[(size_t)b * d + i]);
        if (in_idx_tap && blockIdx.x == 0) in_idx_tap[(size_t)b * d + i] = i;   // every input is kept
    }
    lds_barrier();
    tl_mark(tl, 0, 1);
    const int nparts = d / 8;
    const uint32_t mat_bytes = (uint32_t)F * (uint32_t)d * 2u;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(wg_t, mat_bytes), ru = make_rsrc(wu_t, mat_bytes);
    const int nw = 4 * gridDim.x;
    for (int j = 4 * blockIdx.x + w; j < F; j += nw) {
        const uint32_t soff = (uint32_t)j * (uint32_t)d * 2u;
        double ag = 0.0, au = 0.0;
        for (int p0 = 0; p0 < nparts; p0 += 64 * kExParts) {
            uint4 vg[kExParts], vu[kExParts];
#pragma unroll
            for (int u = 0; u < kExParts; ++u) {
                const int p = p0 + 64 * u + l;
                const uint32_t off = p < nparts ? (uint32_t)p * 16u : mat_bytes;   // past the row: zeros
                vg[u] = buf_load16(rg, off, soff);
                vu[u] = buf_load16(ru, off, soff);
            }
#pragma unroll
            for (int u = 0; u < kExParts; ++u) {
                const int p = p0 + 64 * u + l;
                float xv[8];
                if (p < nparts) {
                    const float4 x0 = *reinterpret_cast<const float4*>(xs + 8 * p);
                    const float4 x1 = *reinterpret_cast<const float4*>(xs + 8 * p + 4);
                    xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
                    xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xv[e] = 0.f;
                }
                const uint32_t gw4[4] = {vg[u].x, vg[u].y, vg[u].z, vg[u].w};
                const uint32_t uw4[4] = {vu[u].x, vu[u].y, vu[u].z, vu[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ag = fma((double)xv[2 * e], (double)bf16_lo(gw4[e]), ag);
                    ag = fma((double)xv[2 * e + 1], (double)bf16_hi(gw4[e]), ag);
                    au = fma((double)xv[2 * e], (double)bf16_lo(uw4[e]), au);
                    au = fma((double)xv[2 * e + 1], (double)bf16_hi(uw4[e]), au);
                }
            }
        }
        ag = wave_sum_d(ag);
        au = wave_sum_d(au);
        if (l == 0) {
            const double h = ag / (1.0 + exp(-ag)) * au;
            const float kf = (float)fabs(h);
            key[(size_t)b * f_pad + j] = kf;
            hbuf[(size_t)b * F + j] = h;
            if (h_tap) h_tap[(size_t)b * F + j] = h;
            if (key_tap) key_tap[(size_t)b * F + j] = kf;
        }
    }
    tl_mark(tl, 0, 3);
    tl_flush(tl, 0);
}

hipError_t launch_exact_h(const uint16_t* x, int B, int d, const uint16_t* wg_t, const uint16_t* wu_t, int F,
                          int f_pad, int nb, float* key, double* hbuf, double* h_tap, float* key_tap,
                          int32_t* in_idx_tap, unsigned long long* tl, hipStream_t s) {
    const size_t dyn = (size_t)d * 4;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)k_exact_h, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    launch_kernel(k_exact_h, dim3(nb, B), dim3(kExThreads), dyn, s, x, wg_t, wu_t, d, F, f_pad, key, hbuf,
                       h_tap, key_tap, in_idx_tap, tl);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quality diagnostics.  grid (B), block 256: token b's kept channels in common
// and the two squared L2 norms, each summed per thread then over the block in
// a fixed order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_quality(const uint8_t* __restrict__ ma, const uint8_t* __restrict__ mb,
                                                 int F, const float* __restrict__ y, const float* __restrict__ yr,
                                                 int d, int32_t* __restrict__ overlap, double* __restrict__ err) {
    __shared__ double red[2][4];
    __shared__ int redi[4];
    const int b = blockIdx.x, t = threadIdx.x, w = t >> 6;
    int common = 0;
    if (ma && mb)
        for (int j = t; j < F; j += 256) common += (ma[(size_t)b * F + j] != 0 && mb[(size_t)b * F + j] != 0) ? 1 : 0;
    double num = 0.0, den = 0.0;
    if (y && yr) {
        for (int c = t; c < d; c += 256) {
            const double r = (double)yr[(size_t)b * d + c];
            const double e = (double)y[(size_t)b * d + c] - r;
            num = fma(e, e, num);
            den = fma(r, r, den);
        }
    }
    num = wave_sum_d(num);
    den = wave_sum_d(den);
    common = wave_sum_i(common);
    if ((t & 63) == 0) {
        red[0][w] = num;
        red[1][w] = den;
        redi[w] = common;
    }
    __syncthreads();
    if (t == 0) {
        double n = 0.0, dd = 0.0;
        int c = 0;
        for (int q = 0; q < 4; ++q) {
            n += red[0][q];
            dd += red[1][q];
            c += redi[q];
        }
        if (overlap && ma && mb) overlap[b] = c;
        if (err && y && yr) err[b] = dd > 0.0 ? sqrt(n) / sqrt(dd) : sqrt(n);
    }
}

hipError_t launch_quality(const uint8_t* ma, const uint8_t* mb, int B, int F, const float* y, const float* yr, int d,
                          int32_t* overlap, double* err, hipStream_t s) {
    hipLaunchKernelGGL(k_quality, dim3(B), dim3(256), 0, s, ma, mb, F, y, yr, d, overlap, err);
    return hipGetLastError();
}

}  // namespace prox
