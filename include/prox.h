/*
 * prox.h — C ABI of the Prox sparse SwiGLU FFN decode path on MI355X (gfx950).
 *
 * The method ("Prox: Training-Free FFN Activation Sparsity via Approximate
 * Intermediate-Channel Salience in LLMs", Abstract) runs one SwiGLU FFN
 * (as defined in "PrunePath: Towards Highly Structured Sparse Language
 * Models", §2.1, Eq. (1)) in two stages per token:
 *
 *   Stage 1  keep the k_in largest |x_i| (input sparsity), run the kept inputs
 *            through quantized proxy copies of W_gate and W_up, form the
 *            approximate intermediate h~ = silu(g~) * u~, and keep the k_ff
 *            channels of largest |h~| as one mask shared by all three
 *            projections;
 *   Stage 2  compute the kept channels exactly over the dense x:
 *            h_j = silu(x . W_gate[:, j]) * (x . W_up[:, j]) and
 *            y = sum_j h_j * W_down[j, :] ("COUNTDOWN", Abstract: the output
 *            is a linear combination of W_down rows).
 *
 * Fixed choices: symmetric int8 per-output-channel proxy (or int4 with one
 * scale per group of 128 inputs and channel); scale = fp32(max|w| / qmax),
 * code = clamp(round-half-even(fp32(w / scale)), -qmax, qmax); equal
 * magnitudes are ranked by lower index in both selections; the channel
 * ranking key is |h~| rounded to fp32 from an fp64 accumulation.
 *
 * Conventions for every call:
 *  - "device" pointers are HIP device memory of the current device; "host"
 *    pointers are ordinary host memory.  The caller owns every buffer.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it; calls return before the GPU finishes.
 *  - All argument checks happen on the host before anything is enqueued; a
 *    call that returns an error has enqueued nothing.  HIP runtime errors
 *    (launch failures) return PROX_E_HIP; faults inside kernels surface on
 *    the stream (at the next synchronisation).
 *  - bf16 matrices are row-major with 16-byte aligned rows (d_model % 8 == 0)
 *    and 16-byte aligned base pointers.
 *  - Calls are thread-safe provided concurrent calls use distinct
 *    workspaces and outputs.  prox_last_error() is per host thread.
 */
#ifndef PROX_H
#define PROX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PROX_ABI_VERSION 1

typedef enum {
    PROX_OK = 0,
    PROX_E_INVALID = -1,     /* null pointer, size out of range, misaligned pointer */
    PROX_E_UNSUPPORTED = -2, /* valid request with no kernel plan (limits below)     */
    PROX_E_MISMATCH = -3,    /* proxy descriptor disagrees with weights or itself    */
    PROX_E_WORKSPACE = -4,   /* workspace smaller than prox_workspace_bytes()        */
    PROX_E_HIP = -5          /* HIP runtime error; see prox_last_error()             */
} prox_status;

typedef enum {
    PROX_PROXY_INT8 = 1,      /* one fp32 scale per output channel, codes in [-127, 127]        */
    PROX_PROXY_INT4_G128 = 2  /* one fp32 scale per (128 inputs, channel), codes in [-7, 7]     */
} prox_proxy_kind;

/* Limits of this build: 8 <= d_model <= 16384, d_model % 8 == 0 (int4: % 128);
 * 1 <= d_ff <= 32768; 1 <= batch <= 64. */
#define PROX_MAX_D_MODEL 16384
#define PROX_MAX_D_FF 32768
#define PROX_MAX_BATCH 64

/* The three bf16 weight matrices of one SwiGLU FFN, all device, all [d_ff][d_model]:
 *   w_gate_t row j = W_gate[:, j]   (the gate weight stored output-major)
 *   w_up_t   row j = W_up[:, j]
 *   w_down   row j = W_down[j, :]   (the page's W_down in R^{d_ff x d}) */
typedef struct {
    int32_t d_model;
    int32_t d_ff;
    const void* w_gate_t;
    const void* w_up_t;
    const void* w_down;
} prox_weights;

/* Descriptor of a proxy built by prox_build_proxy (host struct, device buffer).
 * Channels are grouped in tiles of tile_ch channels (64 for int8, 128 for
 * int4); f_pad = d_ff rounded up to a whole tile.  Layout of buf (bytes):
 *   codes  tile-major, [f_pad / tile_ch][d_model][row_stride = 128]: the 128
 *          bytes of (tile, input row i) are 8 blocks of 16 bytes; block b holds
 *          int8: gate codes of channels 8b..8b+7, then their up codes;
 *          int4: gate codes of channels 16b..16b+15 (channel 2t in the low
 *          nibble of byte t), then their up codes.
 *   scales at scale_offset: fp32 gate[groups][f_pad] then up[groups][f_pad],
 *          groups = 1 (int8) or d_model / 128 (int4).
 * Padding channels d_ff .. f_pad-1 have zero codes and zero scales. */
typedef struct {
    int32_t kind;
    int32_t d_model;
    int32_t d_ff;
    int32_t f_pad;
    int32_t groups;
    int32_t tile_ch;
    size_t row_stride;
    size_t scale_offset;
    size_t bytes;
    void* buf;
} prox_proxy;

/* Kernels of one forward, in launch order (measurement hook below). */
#define PROX_PHASE_STAGE1 0   /* input selection + proxy GEMV + ranking keys */
#define PROX_PHASE_STAGE2 1   /* channel top-k + exact sparse SwiGLU, partial y */
#define PROX_PHASE_REDUCE_Y 2 /* sum of the partial y */
#define PROX_N_PHASES 3

/* Optional intermediate outputs of prox_ffn_forward_taps (device, nullable each):
 *   in_idx [batch][k_in]   kept inputs of Stage 1, ascending
 *   key    [batch][d_ff]   fp32 ranking key |h~_j|
 *   h_hat  [batch][d_ff]   fp64 approximate intermediate h~_j (signed)
 * Measurement hook (host, nullable): `events` holds n_events >= PROX_N_PHASES + 1
 * hipEvent_t handles (as void*) created by the caller; events[0] is recorded on
 * the stream before the first launch and events[p + 1] after phase p.  A phase
 * is one kernel below 4 tokens per call; from 4 tokens stage 1 is the input
 * selection and the proxy GEMM, stage 2 the channel selection, gate/up and
 * down projections.                                                          */
typedef struct {
    int32_t* in_idx;
    float* key;
    double* h_hat;
    void* const* events;
    int32_t n_events;
    int32_t reserved;
} prox_taps;

/* ABI version compiled into the library (PROX_ABI_VERSION). */
int32_t prox_abi_version(void);

/* Bytes a proxy of this shape and kind needs; 0 if the arguments are invalid. */
size_t prox_proxy_bytes(int32_t d_model, int32_t d_ff, int32_t kind);

/* Build the proxy of w->w_gate_t and w->w_up_t ("quantized proxy weights",
 * Prox, Abstract) into the caller's device buffer `buf` (buf_bytes >=
 * prox_proxy_bytes, 256-byte aligned) and fill the host descriptor `out`.
 * One-time, training-free transform of the weights; the codes are bit-exact
 * with the scale/code rule stated at the top of this header. */
prox_status prox_build_proxy(const prox_weights* w, int32_t kind, void* buf, size_t buf_bytes,
                             prox_proxy* out, void* stream);

/* Workspace bytes prox_ffn_forward needs for this shape, batch and kind
 * (an upper bound over k_in, k_ff); 0 if the arguments are invalid. */
size_t prox_workspace_bytes(int32_t d_model, int32_t d_ff, int32_t batch, int32_t kind);

/* One sparse FFN forward for `batch` tokens (Prox, Abstract: Stage 1 then
 * Stage 2, one mask per token shared by the three projections).
 *   x      device bf16 [batch][d_model]
 *   w, p   weights and a proxy built from the same w_gate_t / w_up_t
 *   k_in   inputs kept in Stage 1, 0 <= k_in <= d_model
 *   k_ff   channels kept, 0 <= k_ff <= d_ff
 *   y      device fp32 [batch][d_model], written (not accumulated)
 *   mask   device uint8 [batch][d_ff] 0/1, nullable
 *   idx    device int32 [batch][k_ff] kept channels ascending, nullable
 *   workspace  device, >= prox_workspace_bytes(d_model, d_ff, batch, kind),
 *          256-byte aligned.  Scratch only: its contents on entry do not
 *          change the result, and it need not be cleared.  Calls that
 *          share a workspace must not overlap in time.                    */
prox_status prox_ffn_forward(const void* x, int32_t batch, const prox_weights* w,
                             const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                             uint8_t* mask, int32_t* idx, void* workspace, size_t ws_bytes,
                             void* stream);

/* prox_ffn_forward plus the intermediate outputs in `taps` (nullable). */
prox_status prox_ffn_forward_taps(const void* x, int32_t batch, const prox_weights* w,
                                  const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                  uint8_t* mask, int32_t* idx, void* workspace, size_t ws_bytes,
                                  const prox_taps* taps, void* stream);

/* Static text for a status code. */
const char* prox_status_str(int32_t status);

/* Text of the last error on this host thread ("" if none). */
const char* prox_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PROX_H */
