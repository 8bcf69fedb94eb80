/*
 * gdn2.h -- C ABI of the MI355X (gfx950) Gated DeltaNet-2 recurrence library.
 *
 * The operation is the GDN-2 state update of the page "Why NVIDIA Gated
 * DeltaNet-2 separates erase and write gates" (axbrief.com), section
 * "Gated Delta Rule-2: channel-wise separation of erase and write", its
 * recurrence equation:
 *
 *     S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *     o_t = S_t^T q_t                       (read-out after the update)
 *
 * S is dk x dv (rows are key channels), alpha_t = exp(log_alpha_t) is a decay
 * per key channel, b_t in [0,1]^dk is the erase gate (key side) and
 * w_t in [0,1]^dv the write gate (value side).  There is no query scale.
 *
 * The calls: a chunk-parallel forward over whole sequences (the same page,
 * section "Gated Delta Rule-2", gives the chunk size of 64 used by the fused
 * training kernels), the same forward from gate logits (activations formed in
 * the kernels), the same forward over packed sequences of different
 * lengths, its backward pass (vector-Jacobian product; the same section: the
 * gates enter the gradient inner products, so the backward is derived with
 * them), a single-token recurrent decode step (the page's opening section:
 * decoding keeps a constant-size state), and the mixer's fused elementwise
 * passes on either side of the recurrence.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (HIP global memory) of the current
 *     device, contiguous and row-major in the layouts stated below, and
 *     16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously; the caller keeps every buffer alive until the
 *     stream has passed the call.
 *   - The library never allocates, frees or synchronises and keeps no reference
 *     after returning.  Its only global state is the per-device address of the
 *     fixed array gdn2_chunk_bwd_noalloc works in, looked up once under a lock;
 *     every other call is reentrant.
 *   - All validation happens before anything is enqueued.  On any error the
 *     call returns a non-zero status and writes nothing.  A launch rejected by
 *     the HIP runtime returns GDN2_ERR_HIP.  Faults inside a kernel surface at
 *     the caller's next synchronisation, as for any HIP kernel.
 *   - Inputs are not range-checked on the device: log_alpha must be finite and
 *     <= 0; b and w are expected in [0,1] (values outside are used as given).
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Chunk length of the chunk-parallel forward (tokens per chunk). */
#define GDN2_CHUNK 64

/* Element type of q, k, v, b, w (`dtype`) and of o (`o_dtype`).  Arithmetic
 * inside is fp32 either way; log_alpha and the state are always float32. */
typedef enum gdn2_dtype {
    GDN2_DTYPE_F32 = 0,
    GDN2_DTYPE_BF16 = 1
} gdn2_dtype_t;

typedef enum gdn2_status {
    GDN2_OK = 0,
    GDN2_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN2_ERR_SHAPE = 2,       /* a size is < 1 or too large for 32-bit indexing of a row */
    GDN2_ERR_UNSUPPORTED = 3, /* (dk, dv, dtype) is not built into this library */
    GDN2_ERR_MISALIGNED = 4,  /* a tensor pointer is not 16-byte aligned */
    GDN2_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    GDN2_ERR_WORKSPACE = 6,   /* the workspace is NULL or smaller than required */
    GDN2_ERR_HIP = 7          /* the HIP runtime rejected a query or a launch */
} gdn2_status_t;

/*
 * gdn2_chunk_fwd -- forward over B sequences of T tokens and H heads.
 *
 *   q, k, b       [B, T, H, dk]  dtype        query, key, erase gate
 *   v, w          [B, T, H, dv]  dtype        value, write gate
 *   log_alpha     [B, T, H, dk]  float32      log of the per-channel decay
 *   initial_state [B, H, dk, dv] float32      S_0, or NULL for zeros
 *   o             [B, T, H, dv]  o_dtype      out: o_t = S_t^T q_t
 *   final_state   [B, H, dk, dv] float32      out: S_T, or NULL to skip;
 *                                             may be the same pointer as
 *                                             initial_state (updated in place)
 *
 * T may be any value >= 1 (a last partial chunk is handled exactly).
 * Built combinations: dtype BF16 with (dk, dv) = (64, 64) or (128, 128);
 * dtype F32 with (64, 64).  o_dtype is F32, or equal to dtype: with bf16
 * inputs an F32 output keeps the fp32 accumulation all the way out, a BF16
 * output rounds it once on the store.  Others return GDN2_ERR_UNSUPPORTED.
 * o must not overlap any input; final_state must not overlap any input other
 * than an identical initial_state.  H * dk and H * dv (the elements between
 * consecutive tokens of one tensor) must be below 2^22, else GDN2_ERR_SHAPE.
 * workspace / workspace_bytes select the implementation.  With a workspace of
 * at least gdn2_chunk_fwd_split_workspace_bytes(...) bytes (device memory owned by
 * the caller, 256-byte aligned, overlapping no argument; its contents on entry
 * do not matter and on return are unspecified) the forward runs as two kernels
 * per batch of chunks: one forms every chunk's state-independent quantities in
 * parallel, the other carries the state through the chunks.  With
 * workspace = NULL and workspace_bytes = 0 it runs as one fused kernel (same
 * results within the parity bar, no workspace).  A workspace passed where the
 * two-kernel form does not exist, or a shorter one, returns GDN2_ERR_WORKSPACE.
 * gdn2_chunk_fwd_workspace_bytes says which form is faster for a shape.
 */
gdn2_status_t gdn2_chunk_fwd(const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* initial_state, void* o, float* final_state,
                             int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * gdn2_chunk_fwd_logits -- gdn2_chunk_fwd with the gate activations done in
 * the kernels: it takes the projections' outputs instead of the activated
 * decay and gates.  The erase and write gates are sigmoids of projections of
 * the token (page "Why NVIDIA Gated DeltaNet-2 separates erase and write
 * gates", axbrief.com, section "Gated Delta Rule-2"); the decay takes the
 * same form (alpha = sigmoid(a), so log alpha = log sigmoid(a)).  Forming the
 * activation inside the recurrence kernel so that no full-sequence activation
 * tensor is stored is the "gate-in-kernel" fusion of page "CARVE:
 * Content-Aware Recurrent with Value Efficiency for Chunk-Parallel Linear
 * Attention" (gist.science), section 2.3 "Key-Axis Decay and Fusion".
 *
 *   a_logit       [B, T, H, dk]  dtype        decay logits: alpha = sigmoid(a)
 *   b_logit       [B, T, H, dk]  dtype        erase-gate logits: b = sigmoid(.)
 *   w_logit       [B, T, H, dv]  dtype        write-gate logits: w = sigmoid(.)
 *
 * Every other argument, the workspace rule (gdn2_chunk_fwd_workspace_bytes
 * applies unchanged) and every error are as for gdn2_chunk_fwd.  dtype must be
 * BF16 (dk = dv = 64 or 128), else GDN2_ERR_UNSUPPORTED.  The activations are
 * formed in fp32 from the bf16 logits; a logit below about -88 gives a decay
 * or gate of exactly 0.
 */
gdn2_status_t gdn2_chunk_fwd_logits(const void* q, const void* k, const void* v,
                                    const void* a_logit, const void* b_logit, const void* w_logit,
                                    const float* initial_state, void* o, float* final_state,
                                    int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                    gdn2_dtype_t dtype, gdn2_dtype_t o_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * gdn2_chunk_fwd_split_workspace_bytes -- bytes of device workspace that the
 * two-kernel form of gdn2_chunk_fwd needs for these sizes on the current device:
 * the chunk records of one batch of about a thousand (sequence, head, chunk)
 * triples, 68,608 bytes each at dk = dv = 128 (44,032 at 64), plus one fp32
 * state [B, H, dk, dv].  When the (sequence, head) chains (one workgroup of
 * the state pass each) fill at most half of the device's compute units and the
 * sequences hold at least 32 chunks, the form instead cuts every sequence into
 * segments walked in
 * parallel and joined through their state transitions: it then needs every
 * chunk's record plus, per (sequence, head), a [dk][2 dv] fp32 transition for
 * every segment but the last and a [dk][dv] fp32 start state for every
 * segment.  The
 * two-kernel form exists for BF16 inputs with dk = dv = 64 or 128; for every
 * other combination (and for sizes out of range) this returns 0.
 */
size_t gdn2_chunk_fwd_split_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                            gdn2_dtype_t dtype);

/*
 * gdn2_chunk_fwd_workspace_bytes -- the workspace to pass to gdn2_chunk_fwd for
 * its faster form on the current device: the two-kernel form's size (as above)
 * when the fused kernel's chains, one per (sequence, head, 64 value columns),
 * are fewer than the device's compute units, else 0 (run with workspace = NULL,
 * workspace_bytes = 0: the fused kernel).
 */
size_t gdn2_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdn2_dtype_t dtype);

/*
 * gdn2_chunk_fwd_varlen -- the same forward over N sequences of different
 * lengths packed along one token axis (prefill of a serving batch).
 *
 *   q, k, b       [total_T, H, dk]  dtype
 *   v, w          [total_T, H, dv]  dtype
 *   log_alpha     [total_T, H, dk]  float32
 *   cu_seqlens    [N + 1]           int64, DEVICE memory, 8-byte aligned:
 *                                   sequence n holds tokens
 *                                   [cu_seqlens[n], cu_seqlens[n + 1])
 *   initial_state [N, H, dk, dv]    float32, or NULL for zeros
 *   o             [total_T, H, dv]  o_dtype
 *   final_state   [N, H, dk, dv]    float32 or NULL; may equal initial_state
 *
 * The offsets are expected to be non-decreasing with cu_seqlens[0] = 0 and
 * cu_seqlens[N] = total_T (they are in device memory and are not read on the
 * host).  Each sequence's range is clamped into [0, total_T] on the device, so
 * any offsets keep every access inside the tensors; tokens outside every
 * sequence are left unwritten in o.  A sequence of length 0 passes its initial
 * state (or zeros) through to final_state.  The final states are laid out as
 * gdn2_decode_step's state, so decoding continues from them directly.
 * N >= 1, total_T >= 0; everything else as for gdn2_chunk_fwd (supported
 * shapes and dtypes, alignment, aliasing; cu_seqlens must not overlap o or
 * final_state).
 */
gdn2_status_t gdn2_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                    const float* log_alpha, const void* b, const void* w,
                                    const float* initial_state, void* o, float* final_state,
                                    const int64_t* cu_seqlens, int64_t N, int64_t total_T,
                                    int64_t H, int64_t dk, int64_t dv, gdn2_dtype_t dtype,
                                    gdn2_dtype_t o_dtype, void* stream);

/*
 * gdn2_decode_step -- one recurrent step for N independent sequences.
 *
 *   q, k, b       [N, H, dk]     dtype
 *   v, w          [N, H, dv]     dtype
 *   log_alpha     [N, H, dk]     float32
 *   state         [N, H, dk, dv] float32      read and updated in place
 *   o             [N, H, dv]     o_dtype      out: o = S_new^T q
 *
 * Built combinations: dtype BF16 or F32 with (dk, dv) = (64, 64) or (128, 128);
 * o_dtype is F32 or equal to dtype.
 * o must not overlap any input or the state.
 */
gdn2_status_t gdn2_decode_step(const void* q, const void* k, const void* v,
                               const float* log_alpha, const void* b, const void* w,
                               float* state, void* o, int64_t N, int64_t H, int64_t dk,
                               int64_t dv, gdn2_dtype_t dtype, gdn2_dtype_t o_dtype,
                               void* stream);

/*
 * gdn2_chunk_bwd_workspace_bytes -- bytes of device workspace gdn2_chunk_bwd
 * needs for these sizes (NC = ceil(T / 64)): 4 * (2 B H NC dk dv +
 * 2 B T H dv + B H NC R), each of the five parts rounded up to 256 bytes, where
 * R = 2*64*64 + 5*64*dk + 64*dv + dk rounded up to a multiple of 64 (one record
 * of chunk-local quantities per chunk).  Returns 0 if the sizes overflow or dk
 * or dv exceeds 2^20.
 */
size_t gdn2_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv);

/*
 * gdn2_chunk_bwd -- backward pass of gdn2_chunk_fwd: the gradients of
 * L = sum(d_o * o) + sum(d_final_state * S_T) with respect to every input.
 *
 *   q, k, v, log_alpha, b, w, initial_state   as for gdn2_chunk_fwd (dtype)
 *   d_o            [B, T, H, dv]  float32     upstream gradient of o
 *   d_final_state  [B, H, dk, dv] float32     upstream gradient of S_T, or NULL
 *                                             for zeros
 *   dq, dk, db     [B, T, H, dk]  float32     out
 *   dv, dw         [B, T, H, dv]  float32     out
 *   dlog_alpha     [B, T, H, dk]  float32     out
 *   d_initial_state [B, H, dk, dv] float32    out: gradient of S_0, or NULL to
 *                                             skip (zeros S_0 when
 *                                             initial_state is NULL)
 *   workspace      device memory of at least
 *                  gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv) bytes,
 *                  16-byte aligned, owned by the caller; its contents on entry
 *                  do not matter and on return are unspecified
 *
 * The call re-runs the forward to recover the state entering every chunk, so
 * it needs neither o nor any saved state.  Built combinations and the limits
 * on sizes are those of gdn2_chunk_fwd (B, T >= 1).  No output may overlap
 * another output, an input or the workspace, and the workspace may not
 * overlap an input (GDN2_ERR_ALIAS); a missing or short workspace returns
 * GDN2_ERR_WORKSPACE.
 */
gdn2_status_t gdn2_chunk_bwd(const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* initial_state, const float* d_o,
                             const float* d_final_state, float* dq, float* dk, float* dv,
                             float* dlog_alpha, float* db, float* dw, float* d_initial_state,
                             void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                             int64_t H, int64_t dk_dim, int64_t dv_dim, gdn2_dtype_t dtype,
                             void* stream);

/* Bytes of the device array that gdn2_chunk_bwd_noalloc uses as its workspace (64 MiB). */
#define GDN2_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gdn2_chunk_bwd_noalloc -- gdn2_chunk_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training loops,
 * harnesses that forbid hipMalloc): the same gradients, computed by the same
 * kernels, with the workspace taken from a fixed array of GDN2_SCRATCH_BYTES
 * inside the library instead of from the caller.  Nothing is allocated or freed.
 *
 *   arguments       as for gdn2_chunk_bwd, without workspace / workspace_bytes
 *
 * Calls whose gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv) exceeds
 * GDN2_SCRATCH_BYTES return GDN2_ERR_WORKSPACE (for example B = 1, H = 16,
 * dk = dv = 128 fits up to T = 576).  Each GPU the library runs on holds its own
 * array from the first call on that device until the process ends; the first
 * call on a device looks up the array's address (GDN2_ERR_HIP if that fails).
 * Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents: calls that may run at the same time on one GPU (different streams,
 * different host threads without ordering) race and must not overlap.  No part
 * of the array needs clearing: every call writes each slot before reading it.
 */
gdn2_status_t gdn2_chunk_bwd_noalloc(const void* q, const void* k, const void* v,
                                     const float* log_alpha, const void* b, const void* w,
                                     const float* initial_state, const float* d_o,
                                     const float* d_final_state, float* dq, float* dk, float* dv,
                                     float* dlog_alpha, float* db, float* dw,
                                     float* d_initial_state, int64_t B, int64_t T, int64_t H,
                                     int64_t dk_dim, int64_t dv_dim, gdn2_dtype_t dtype,
                                     void* stream);

/*
 * gdn2_mixer_prep -- the elementwise steps between the layer's projections and
 * the recurrence, in one pass (page "Why NVIDIA Gated DeltaNet-2 separates
 * erase and write gates", the section on the layer's architecture: query and
 * key through a short causal convolution, SiLU and L2 normalisation, value
 * through the convolution and SiLU; section "Gated Delta Rule-2": erase and
 * write gates are sigmoids of projections):
 *
 *   q = xq' / sqrt(|xq'|^2 + eps),  xq' = SiLU(conv(xq))   (norm over dk)
 *   k likewise from xk;  v = SiLU(conv(xv))
 *   b = sigmoid(xb),  w = sigmoid(xw),  log_alpha = log sigmoid(xa)
 *
 *   xq, xk, xb, xa  [B, T, H, dk]  dtype   projection outputs (pre-activation)
 *   xv, xw          [B, T, H, dv]  dtype
 *   conv_q, conv_k  [H * dk, 4]    float32 depthwise causal taps: tap j of a
 *   conv_v          [H * dv, 4]    float32 channel multiplies its input at token
 *                                          t - 3 + j; tokens before 0 are zero
 *   q, k, b         [B, T, H, dk]  dtype   out
 *   v, w            [B, T, H, dv]  dtype   out
 *   log_alpha       [B, T, H, dk]  float32 out (<= 0)
 *
 * The sigmoid form of the decay is this library's reading: the pages give the
 * decay no activation.  Built: dtype BF16 or F32 with dk = dv = 64 or 128.  No
 * output may overlap an input or another output.  eps >= 0.
 * With b, w and log_alpha all NULL only q, k and v are formed (xb, xw and xa
 * are then not read and may be NULL): the gates are left to
 * gdn2_chunk_fwd_logits, which activates them inside the recurrence kernels.
 * Some but not all of b, w, log_alpha NULL returns GDN2_ERR_NULL.
 */
gdn2_status_t gdn2_mixer_prep(const void* xq, const void* xk, const void* xv, const void* xb,
                              const void* xw, const void* xa, const float* conv_q,
                              const float* conv_k, const float* conv_v, void* q, void* k,
                              void* v, void* b, void* w, float* log_alpha, int64_t B, int64_t T,
                              int64_t H, int64_t dk, int64_t dv, float eps, gdn2_dtype_t dtype,
                              void* stream);

/*
 * gdn2_mixer_out -- the layer output from the recurrence output, in one pass
 * (same page and section: RMS normalisation and a SiLU output gate):
 *
 *   y = o / sqrt(mean(o^2) + eps) * gamma * SiLU(z)      (mean over dv)
 *
 *   o      [B, T, H, dv]  o_dtype  recurrence output (F32, or equal to dtype)
 *   z      [B, T, H, dv]  dtype    output-gate projection
 *   gamma  [dv]           float32  norm weight, shared by the heads
 *   y      [B, T, H, dv]  dtype    out; must not overlap o, z or gamma
 *
 * Built: dtype BF16 or F32 with dv = 64 or 128.  eps >= 0.
 */
gdn2_status_t gdn2_mixer_out(const void* o, const void* z, const float* gamma, void* y, int64_t B,
                             int64_t T, int64_t H, int64_t dv, float eps, gdn2_dtype_t dtype,
                             gdn2_dtype_t o_dtype, void* stream);

/* 1 if gdn2_chunk_fwd and gdn2_chunk_fwd_varlen (which = 0), gdn2_decode_step
 * (which = 1), gdn2_chunk_bwd (which = 2) or gdn2_mixer_prep and gdn2_mixer_out
 * (which = 3) support (dk, dv, dtype), else 0. */
int gdn2_supported(int which, int64_t dk, int64_t dv, gdn2_dtype_t dtype);

/* Static, NUL-terminated description of a status code. */
const char* gdn2_status_string(gdn2_status_t status);

/* Static version string of the library. */
const char* gdn2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
