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

#define PROX_ABI_VERSION 4

typedef enum {
    PROX_OK = 0,
    PROX_E_INVALID = -1,     /* null pointer, size out of range, misaligned pointer */
    PROX_E_UNSUPPORTED = -2, /* valid request with no kernel plan (limits below)     */
    PROX_E_MISMATCH = -3,    /* proxy descriptor disagrees with weights or itself    */
    PROX_E_WORKSPACE = -4,   /* workspace smaller than prox_workspace_bytes()        */
    PROX_E_HIP = -5          /* HIP runtime error; see prox_last_error()             */
} prox_status;

typedef enum {
    PROX_PROXY_INT8 = 1,       /* one fp32 scale per output channel, codes in [-127, 127]        */
    PROX_PROXY_INT4_G128 = 2,  /* one fp32 scale per (128 inputs, channel), codes in [-7, 7]     */
    PROX_PROXY_EXACT_BF16 = 3  /* exact-mask mode: no proxy; every input kept (k_in = d_model)
                                  and the channels ranked by the exact |h| computed from the bf16
                                  weights themselves (the selector the proxies approximate)      */
} prox_proxy_kind;

/* Limits of this build: 8 <= d_model <= 16384, d_model % 8 == 0 (int4: % 128);
 * 1 <= d_ff <= 32768; 1 <= batch <= 4096.  Batches above PROX_CHUNK_BATCH
 * tokens (prefill) run as consecutive sub-batches of at most that many
 * tokens within the call, sharing one workspace sized for one sub-batch. */
#define PROX_MAX_D_MODEL 16384
#define PROX_MAX_D_FF 32768
#define PROX_MAX_BATCH 4096
#define PROX_CHUNK_BATCH 64

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
 * Measurement hook (host, nullable): `events` holds hipEvent_t handles (as
 * void*) created by the caller, used in one of two ways (`event_mode`):
 *   0  n_events >= PROX_N_PHASES + 1: events[0] is recorded on the stream
 *      before the first launch and events[p + 1] after phase p (the interval
 *      also holds the dispatch of the phase's first kernel);
 *   1  n_events >= 2 * PROX_N_PHASES: the kernels themselves carry the events
 *      (hipExtLaunchKernel): events[2p] takes the start of phase p's first
 *      kernel and events[2p + 1] the end of its last one, so one kernel's
 *      interval is its execution alone.  A phase with no kernel leaves its
 *      pair unrecorded.
 * A phase is one kernel below 4 tokens per call; from 4 tokens stage 1 is the
 * input selection and the proxy GEMM, stage 2 the channel selection, gate/up
 * and down projections.  Above PROX_CHUNK_BATCH tokens the events time the
 * last sub-batch (mode 0: events[0] is still recorded before the first).  The
 * other taps cover every token.
 *   stream_idx [batch][k_ff]  below 4 tokens per call only (untouched from 4):
 *          the channels whose rows the Stage-2 blocks actually stream, each
 *          block's list at the ranks of its share; over all blocks a
 *          permutation of idx when no channel is lost or streamed twice.
 *   timeline [2][1024][8]  below 4 tokens per call only: the GPU's 100 MHz
 *          real-time counter, stored by each block of Stage 1 (index 0) and
 *          Stage 2 (index 1; block = token * blocks per token + block) at
 *          points 0 start, 1 selection done, 2 stream done (Stage 1: of its
 *          last tile), 3 end, and inside the selections: Stage 1 4 histogram
 *          built, 5 threshold found, 6 first scan done; Stage 2 4 histogram
 *          built, 5 keys classified, 6 lists written, 7 candidates ranked.  */
typedef struct {
    int32_t* in_idx;
    float* key;
    double* h_hat;
    void* const* events;
    int32_t n_events;
    int32_t event_mode;
    int32_t* stream_idx;
    uint64_t* timeline;
} prox_taps;

/* ABI version compiled into the library (PROX_ABI_VERSION). */
int32_t prox_abi_version(void);

/* Bytes a proxy of this shape and kind needs; 0 if the arguments are invalid
 * (and for PROX_PROXY_EXACT_BF16, which needs no buffer). */
size_t prox_proxy_bytes(int32_t d_model, int32_t d_ff, int32_t kind);

/* Build the proxy of w->w_gate_t and w->w_up_t ("quantized proxy weights",
 * Prox, Abstract) into the caller's device buffer `buf` (buf_bytes >=
 * prox_proxy_bytes, 256-byte aligned) and fill the host descriptor `out`.
 * One-time, training-free transform of the weights; the codes are bit-exact
 * with the scale/code rule stated at the top of this header.
 * PROX_PROXY_EXACT_BF16: nothing is built or enqueued; `buf` may be NULL and
 * the descriptor only records the shape (bytes = 0). */
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

/* With a PROX_PROXY_EXACT_BF16 descriptor (exact-mask mode) k_in must equal
 * d_model (PROX_E_INVALID otherwise): Stage 1 computes h_j = silu(x . W_gate[:, j])
 * (x . W_up[:, j]) for every channel in fp64 and ranks fp32(|h_j|); Stage 2
 * keeps the top k_ff and streams only their W_down rows, with h read back.
 * The per-token kernels run for every batch size.  k_ff = d_ff gives the
 * dense FFN. */

/* prox_ffn_forward plus the intermediate outputs in `taps` (nullable). */
prox_status prox_ffn_forward_taps(const void* x, int32_t batch, const prox_weights* w,
                                  const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                  uint8_t* mask, int32_t* idx, void* workspace, size_t ws_bytes,
                                  const prox_taps* taps, void* stream);

/* ---- Quantized Stage-2 weights ---------------------------------------------
 * "Prox: ...", Abstract: the method is compatible with quantization.  Every
 * row of W_gate^T, W_up^T (the weights of one channel) and W_down (the output
 * direction of one channel) as int8 codes with one fp32 scale per row, by
 * the int8 proxy's rule (scale = fp32(max|row| / 127), code =
 * clamp(round-half-even(fp32(w / scale)), -127, 127)); Stage 2 then streams
 * d_model bytes per row instead of 2 * d_model.  Stage 1 is unchanged (its
 * proxy is built from the bf16 weights).
 * Layout of buf (device): codes gate [d_ff][d_model], up, down (int8), then
 * at scale_offset fp32 scales gate [d_ff], up [d_ff], down [d_ff].          */
typedef struct {
    int32_t d_model;
    int32_t d_ff;
    size_t scale_offset;
    size_t bytes;
    void* buf;
} prox_qweights;

/* Bytes of the quantized weights of this shape (d_model % 8 == 0 and the
 * limits above); 0 if the arguments are invalid. */
size_t prox_qweights_bytes(int32_t d_model, int32_t d_ff);

/* Quantize w's three bf16 matrices into the caller's device buffer `buf`
 * (buf_bytes >= prox_qweights_bytes, 256-byte aligned); fills the host
 * descriptor `out`.  One-time, stream-ordered. */
prox_status prox_build_qweights(const prox_weights* w, void* buf, size_t buf_bytes, prox_qweights* out,
                                void* stream);

/* prox_ffn_forward_taps with the Stage-2 rows taken from `q` (int8 rows and
 * scales): g_j = s_g,j (x . q_g,j), u_j likewise, h_j = silu(g_j) u_j and
 * y = sum over the kept j of h_j s_d,j q_d,j.  Stage 1 and every other
 * argument as prox_ffn_forward_taps (taps nullable); the workspace is the one
 * prox_workspace_bytes gives for the proxy's kind.  The per-token Stage-2
 * kernel runs for every batch.  PROX_E_UNSUPPORTED for an exact-mode proxy. */
prox_status prox_ffn_forward_q8(const void* x, int32_t batch, const prox_qweights* q, const prox_proxy* p,
                                int32_t k_in, int32_t k_ff, float* y, uint8_t* mask, int32_t* idx,
                                void* workspace, size_t ws_bytes, const prox_taps* taps, void* stream);

/* ---- Allocation-free forward ----------------------------------------------
 * For callers that cannot allocate device memory around a forward (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * prox_ffn_forward with the workspace taken from a fixed device array of the
 * library, PROX_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, allocated when the
 * library is loaded and held until the process ends.  No call allocates.
 *   Arguments as prox_ffn_forward, without the workspace.
 *   Returns PROX_E_UNSUPPORTED (nothing enqueued) when this shape and batch
 *   need more workspace than the array holds (prox_workspace_bytes above
 *   PROX_NOALLOC_SCRATCH_BYTES), PROX_E_HIP if the array's address on the
 *   current device cannot be found; otherwise as prox_ffn_forward.
 *   Every call on one GPU uses that GPU's array: calls that overlap in time
 *   on one GPU (other streams, other host threads) race and must not be
 *   issued.  The array keeps the last call's contents; the forward needs
 *   none of it cleared (as for any workspace).                               */
#define PROX_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Bytes of the allocation-free forward's scratch array (per GPU). */
size_t prox_noalloc_scratch_bytes(void);

prox_status prox_ffn_forward_noalloc(const void* x, int32_t batch, const prox_weights* w,
                                     const prox_proxy* p, int32_t k_in, int32_t k_ff, float* y,
                                     uint8_t* mask, int32_t* idx, void* stream);

/* ---- Quality diagnostics (not part of the forward) --------------------------
 * For each token b < batch, on device data:
 *   overlap[b] = number of channels j < d_ff with mask_a[b][j] != 0 and
 *                mask_b[b][j] != 0 (kept channels in common: the mask recall
 *                of a proxy against the exact-mask mode is overlap / k_ff);
 *   err[b]     = ||y[b] - y_ref[b]||_2 / ||y_ref[b]||_2 in fp64 (the numerator
 *                alone when y_ref[b] is 0), e.g. a sparse forward against the
 *                dense FFN (exact mode with k_ff = d_ff).
 * mask_a, mask_b: uint8 [batch][d_ff]; y, y_ref: fp32 [batch][d_model];
 * overlap int32 [batch]; err fp64 [batch]; all device.  Each triple (masks +
 * overlap, ys + err) is given or null as a whole, at least one of them.    */
prox_status prox_quality(const uint8_t* mask_a, const uint8_t* mask_b, int32_t batch, int32_t d_ff,
                         const float* y, const float* y_ref, int32_t d_model, int32_t* overlap,
                         double* err, void* stream);

/* ---- Measurement helper (not part of the forward) ---------------------------
 * Read-stream probe: reads the first bytes / 16 * 16 bytes of the device
 * buffer `buf` (16-byte aligned) with `blocks` blocks of 512 threads, each
 * block one contiguous part, 16-byte loads, eight in flight per thread
 * (64 KB per block), and writes one word per thread to the
 * device array sink[blocks * 512] (so the loads are not removed).  Timing it
 * gives the HBM read rate a plain stream reaches, the practical ceiling the
 * forward's rate is compared with.  PROX_E_INVALID for a null or misaligned
 * buffer, bytes < 16 or blocks < 1.                                         */
prox_status prox_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* Static text for a status code. */
const char* prox_status_str(int32_t status);

/* Text of the last error on this host thread ("" if none). */
const char* prox_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PROX_H */
