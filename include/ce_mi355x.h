/*
 * ce_mi355x.h -- C ABI of the MI355X (gfx950) token-level softmax
 * cross-entropy library: forward, backward, and the fused forward+backward
 * that writes the gradient over the logits; around it, the LM-head projection
 * fused with the loss (ce_linear_*), RMS layer normalisation (ce_rmsnorm_*)
 * and the rotary position embedding with position ids (ce_rope), each
 * declared below with the passage that defines it.
 *
 * The operation.  The pages name a "Fast Cross Entropy" kernel (PyPI page
 * "fms-acceleration-foak 0.7.4", kernel list) that replaces a causal LM's
 * cross-entropy loss (fms-acceleration PR #79, "Bug Fix to Model Patcher":
 * FastCrossEntropyLoss is patched in for the model's loss) and is used for full
 * fine-tuning, LoRA and padding-free packed batches (fms-hf-tuning PR #280,
 * "Notes on FastKernels").  It computes, for each logit row x[0..V) with label
 * y, the textbook softmax cross-entropy:
 *
 *   lse   = log sum_j exp(x_j)                      (stable: max subtracted)
 *   loss  = lse - x_y                               (nats)
 *   L     = sum over valid rows of loss / n_valid   (token mean: PR #280,
 *                                                    "Early Version Of This
 *                                                    Plugin", per-token averaging)
 *   grad_j = (dloss / n_valid) * (exp(x_j - lse) - [j == y])
 *
 * A row whose label equals ignore_index is not valid: its loss is 0, its
 * gradient row is +0, and it is not counted in n_valid.  The default
 * ignore_index of the callers is -100.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a device pointer owned by the caller; the
 *     library allocates no memory and keeps no pointer after return.
 *   - The library links the HIP runtime and nothing else.  In a process that
 *     also uses PyTorch (which ships its own copy of the runtime), load this
 *     library after PyTorch: loaded first, it brings up the system runtime,
 *     in which PyTorch's device pointers are not valid (a launch then fails
 *     with CE_ERR_HIP).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream).  No entry point synchronises the stream or reads device data on
 *     the host; outputs are valid once the stream work completes, and inputs
 *     must stay alive until then.
 *   - logits: n_rows rows of `vocab` elements of `dtype`, row i starting at
 *     element i * ld (ld >= vocab).  The pointer must be aligned to the element
 *     size; any 16-byte misalignment is handled.
 *   - labels: n_rows int64 class indices.
 *   - Host-checkable errors return a nonzero code before anything is enqueued.
 *     A HIP launch failure returns CE_ERR_HIP.
 *   - Errors only the device can see are OR-ed into the status word (see
 *     CE_STATUS_*): a label outside [0, vocab) that is not ignore_index makes
 *     that row's loss and gradient NaN, still counts the row in n_valid, and
 *     sets CE_STATUS_LABEL_RANGE.
 *   - Calls that share a workspace must be ordered (same stream, or joined by
 *     events); calls with different workspaces are independent.
 *   - Results are deterministic: the same inputs give the same bits.
 *   - Precision: bf16/fp16 inputs are computed in fp32 and the gradient is
 *     rounded once to the input format (nearest-even, subnormals kept); fp32
 *     inputs are computed in fp64 and rounded once to fp32 (each entry point
 *     below states its own arithmetic).
 */
#ifndef CE_MI355X_H
#define CE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CE_ABI_VERSION 5

/* element formats of logits and gradients */
enum ce_dtype { CE_DTYPE_F32 = 0, CE_DTYPE_BF16 = 1, CE_DTYPE_F16 = 2 };

/* return codes */
enum ce_error {
  CE_OK = 0,
  CE_ERR_INVALID_ARG = 1, /* bad size, stride, pointer or alignment */
  CE_ERR_DTYPE = 2,       /* unknown dtype */
  CE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than ce_workspace_bytes() */
  CE_ERR_UNSUPPORTED = 4, /* a valid request this library does not serve */
  CE_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
  CE_ERR_SCRATCH = 6      /* more workspace than ce_fwd_bwd_inplace_noalloc's static scratch */
};

/* bits OR-ed into the status word by the kernels */
#define CE_STATUS_LABEL_RANGE 0x1u  /* some label outside [0, vocab) and not ignore_index */
#define CE_STATUS_SYNC_TIMEOUT 0x2u /* a bounded inter-workgroup wait gave up: outputs invalid */

/* ABI version of the loaded library (CE_ABI_VERSION it was built with). */
int ce_abi_version(void);

/*
 * Test hook for the bounded inter-workgroup wait of the token mean (the mean
 * over valid tokens, fms-hf-tuning PR #280, "Early Version Of This Plugin",
 * needs the batch's valid-token count before any gradient is scaled, so the
 * single-launch kernels wait for partial counts published by other
 * workgroups).  spin_limit > 0 replaces the default number of polls before a
 * wait gives up (0 restores it); extra_counters > 0 makes every poller also
 * wait for that many partial-count words that no workgroup publishes, so each
 * wait expires after spin_limit polls and every workgroup still exits.  A call
 * whose wait expired reports CE_STATUS_SYNC_TIMEOUT, writes NaN to loss_mean
 * and NaN gradients for its valid rows; ce_workspace_init then makes the
 * workspace ready again.  Process-wide; affects launches made after it
 * returns.  Returns CE_ERR_INVALID_ARG for negative values or
 * extra_counters > 64.
 */
int ce_debug_sync_override(int spin_limit, int extra_counters);

/* Static text for a return code or status bit. */
const char* ce_error_string(int code);

/*
 * Bytes of device workspace the calls below need for this shape (0 < result;
 * the same value serves ce_forward and ce_fwd_bwd_inplace).  chunk as below.
 * Returns 0 for arguments that every entry point would reject.
 */
size_t ce_workspace_bytes(int64_t n_rows, int64_t vocab, int64_t chunk, int dtype);

/*
 * Prepare a workspace for first use (zero-fills it on `stream`).  Must be
 * called once after allocating a workspace; every successful call leaves the
 * workspace ready for the next one.  Also recovers a workspace after a call
 * that reported CE_STATUS_SYNC_TIMEOUT.
 */
int ce_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass.
 *   chunk         vocabulary slab width for the per-chunk log-sum-exp merge
 *                 (lse = M + log sum_c exp(lse_c - M), M = max_c lse_c; PR #79
 *                 "TODO": chunked loss) of rows too wide to be held on chip
 *                 (> 131072 bf16/fp16 or > 65536 fp32 elements); 0 = 65536
 *                 (fp32: 32768).  A row that fits on chip is read once
 *                 whatever chunk is: its workgroup merges (max, sum) partials
 *                 of many lanes, a finer partition of the same merge.  In
 *                 ce_fwd_bwd_inplace, 16-byte-aligned bf16/fp16 rows of
 *                 65537..131072 elements with chunk = 65536 reduce the two
 *                 chunks separately and merge their (max, sum) on chip.
 *                 The result does not depend on chunk beyond rounding.
 *   loss_mean     out, 1 float: L (NaN when n_valid == 0).
 *   loss_rows     out, n_rows floats: per-row loss (0 for ignored rows).
 *   lse_rows      out or NULL, n_rows doubles: per-row lse (0 for ignored rows).
 *   pcomp_rows    out or NULL, n_rows doubles: 1 - softmax(x)_y, the complement
 *                 of the label's probability, computed without cancellation
 *                 (0 for ignored rows).  ce_backward needs lse and pcomp; they
 *                 are kept in fp64 so that a backward of fp32 logits can round
 *                 its gradient as tightly as the fused call does.
 *   n_valid       out, 1 int32.
 *   status        out or NULL, 1 uint32: CE_STATUS_* bits of this call.
 * logits is not modified.
 */
int ce_forward(const void* logits, int64_t ld, const int64_t* labels, int64_t n_rows,
               int64_t vocab, int dtype, int64_t ignore_index, int64_t chunk,
               float* loss_mean, float* loss_rows, double* lse_rows, double* pcomp_rows,
               int32_t* n_valid, uint32_t* status, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Backward pass from the forward's saved per-row lse and pcomp:
 *   grad_j = s * exp(x_j - lse)  (j != y),   grad_y = -s * pcomp,
 *   s = dloss / n_valid;  ignored rows get +0.
 *   dloss     device float or NULL (= 1.0): the upstream gradient of L.
 *   n_valid   device int32 from the forward.
 *   grad      n_rows rows of `vocab` elements of dtype, row i at i * grad_ld.
 *             May be the logits buffer itself (in place, grad_ld == ld); if it
 *             is a different buffer it must not overlap logits
 *             (CE_ERR_INVALID_ARG).  Its alignment and stride are free (element
 *             aligned): the kernel writes whole 16-byte vectors of the
 *             gradient rows and assembles each vector's logits from the
 *             16-byte blocks they straddle when the two layouts differ.
 */
int ce_backward(const void* logits, int64_t ld, const int64_t* labels, const double* lse_rows,
                const double* pcomp_rows, const int32_t* n_valid, const float* dloss,
                int64_t n_rows, int64_t vocab, int dtype, int64_t ignore_index, void* grad,
                int64_t grad_ld, void* stream);

/*
 * Fused forward + backward: the outputs of ce_forward, and the gradient of
 * dloss * L written over the logits.  With no chunking and rows that fit on
 * chip (vocab <= 131072 for bf16/fp16, <= 65536 for fp32) this is one kernel
 * that reads every valid row once and writes every row once; ignored rows are
 * written without being read.  dloss: device float or NULL (= 1.0).
 */
int ce_fwd_bwd_inplace(void* logits, int64_t ld, const int64_t* labels, int64_t n_rows,
                       int64_t vocab, int dtype, int64_t ignore_index, int64_t chunk,
                       const float* dloss, float* loss_mean, float* loss_rows, double* lse_rows,
                       double* pcomp_rows, int32_t* n_valid, uint32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * ce_fwd_bwd_inplace without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * ce_fwd_bwd_inplace; its workspace is a static device array of 8 MiB per GPU
 * inside the library (enough for n_rows up to about one million unchunked
 * rows: header 1 KiB + 8 bytes per row, plus the slab partials of rows wider
 * than on-chip capacity), looked up and zero-filled on `stream` on the first
 * call on each device and held until the process ends.  Calls no allocating
 * routine.  Requests whose ce_workspace_bytes() exceeds 8 MiB return
 * CE_ERR_SCRATCH before anything is enqueued.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (unordered streams,
 * concurrent host threads without ordering) race and must be avoided.
 */
int ce_fwd_bwd_inplace_noalloc(void* logits, int64_t ld, const int64_t* labels, int64_t n_rows,
                               int64_t vocab, int dtype, int64_t ignore_index, int64_t chunk,
                               const float* dloss, float* loss_mean, float* loss_rows, double* lse_rows,
                               double* pcomp_rows, int32_t* n_valid, uint32_t* status, void* stream);

/*
 * LM-head projection followed by the cross-entropy above, forward and
 * backward.  The pages compare the plain kernel with a fused linear
 * cross-entropy (PyPI page "fms-acceleration-foak 0.7.4", "Running Liger
 * Kernel Benchmarks"), list fused cross-entropy among the kernels to come
 * (fms-hf-tuning PR #280, "Notes on FastKernels") and leave a chunked loss as
 * a to-do (fms-acceleration PR #79, "TODO").  With hidden states
 * h [n_rows, hidden_size] and the weight W [vocab, hidden_size] of a bias-free
 * linear layer:
 *
 *   logits      = h W^T
 *   L, loss_rows, n_valid, status  as ce_forward on those logits
 *   grad_hidden = g W,  grad_weight = g^T h,  g = dloss * dL/dlogits
 *
 * bf16 / fp16: every product runs on the matrix cores of this library's own
 * kernels (16-bit inputs, fp32 accumulation, no other library).  The logits
 * are never stored: each 256 x 256 tile of them stays in the registers of
 * the workgroup that computed it, whose epilogue takes per row the tile's
 * max m and stores the tile's exponentials e = exp(x - m) (times 2^14 for
 * fp16), rounded to dtype, with 0 at the label's column, where g goes, and
 * per row the tile's shift and label-excluded sum of e -- the statistics of
 * 256-column chunks.  A second kernel merges each row's pairs into its
 * log-sum-exp (fixed order), writes loss_rows (fp32: lse - x_y, or
 * log1p(S / e^{x_y}) when p_y > 1/2) and turns the row's e into
 * g = dloss (softmax - onehot) / n_valid by its tiles' factors, rounded to
 * dtype again (the label's element, -dloss (1 - p_y) / n_valid, once).
 * g is held scaled by 2^k (k = 0 for bf16; for fp16, k puts dloss / n_valid
 * near 2^14 so that g stays in range) and the two backward products remove
 * the scale before rounding grad_hidden and grad_weight once to dtype.
 * Sums are in a fixed order: repeated calls give identical bits.
 * Fast operand loads (16-byte direct-to-LDS) need hidden and weight rows
 * 16-byte aligned (pointer and ld * element size) and hidden_size a multiple
 * of 8; other layouts load element by element (same results, slower).
 * chunk_rows is not used.  vocab above 2097152 (8192 tiles of 256) gives
 * CE_ERR_UNSUPPORTED.
 * fp32: chunk_rows rows at a time (0 = 1024; rounded up to a multiple of 64,
 * and up so that there are at most 4096 chunks): the chunk's fp32 logits by
 * an fp32 tiled product, its loss and gradient by the kernels of
 * ce_fwd_bwd_inplace (fp64 arithmetic) with the token mean over the whole
 * batch, then the two backward products in fp32 (grad_weight accumulated
 * over the chunks in place).
 *   hidden        n_rows rows of hidden_size elements of dtype, row i at
 *                 i * ld_hidden (ld_hidden >= hidden_size).
 *   weight        vocab rows of hidden_size elements, row v at v * ld_weight.
 *   labels        n_rows int64 class indices in [0, vocab) or ignore_index.
 *   dloss         device float or NULL (= 1.0): the upstream gradient of L.
 *   loss_mean, loss_rows, n_valid, status: as ce_forward (loss_rows required).
 *   grad_hidden   out or NULL (not computed): n_rows rows, stride ld_grad_hidden.
 *   grad_weight   out or NULL: vocab rows, stride ld_grad_weight (all zeros when
 *                 n_rows == 0).
 *   workspace     ce_linear_workspace_bytes(...) bytes, 256-byte aligned,
 *                 owned by this function for the call (calls on one
 *                 workspace must not overlap).  bf16 / fp16: a 256-byte
 *                 header (the call's scale and status), g (n_rows x vocab
 *                 rounded up to 8, dtype), two floats per row and 256-column
 *                 tile, the label logits (n_rows floats) and, when the rows
 *                 are too few to fill the chip with dL/dh's tiles, fp32
 *                 partial sums of dL/dh over up to 16 vocabulary ranges;
 *                 nothing in it carries over between calls.  fp32: a chunk's cross-entropy
 *                 workspace (zeroed at the start of every call), the chunk's
 *                 fp32 logits and per-chunk counts.
 * Errors: as ce_fwd_bwd_inplace; n_rows, hidden_size, vocab or a leading
 * dimension of 2^31 or more, hidden or weight of 2^31 bytes or more (the
 * loads use 32-bit buffer offsets), and for fp32 or the element-wise loads
 * also (n_rows + 256) x vocab elements of 2^31 bytes or more, give
 * CE_ERR_UNSUPPORTED; a failed launch gives CE_ERR_HIP.
 */
size_t ce_linear_workspace_bytes(int64_t n_rows, int64_t hidden_size, int64_t vocab, int64_t chunk_rows,
                                 int dtype);
int ce_linear_fwd_bwd(const void* hidden, int64_t ld_hidden, const void* weight, int64_t ld_weight,
                      const int64_t* labels, int64_t n_rows, int64_t hidden_size, int64_t vocab, int dtype,
                      int64_t ignore_index, int64_t chunk_rows, const float* dloss, float* loss_mean,
                      float* loss_rows, int32_t* n_valid, uint32_t* status, void* grad_hidden,
                      int64_t ld_grad_hidden, void* grad_weight, int64_t ld_grad_weight, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * RMS layer normalisation, forward and backward.  The pages list "Fast RMS
 * LayerNorm" among the package's kernels (PyPI page "fms-acceleration-foak
 * 0.7.4", kernel list) and patch it in for a model's RMSNorm class (same page,
 * the model-patcher rule that replaces GraniteRMSNorm's forward;
 * fms-hf-tuning PR #280, "Notes on FastKernels").  Per row x[0..hidden):
 *
 *   rstd = 1 / sqrt(mean_j x_j^2 + eps),   y_j = w_j x_j rstd
 *   dx_j = rstd (w_j dy_j - x^_j mean_k(x^_k w_k dy_k)),   x^ = x rstd
 *   dw_j = sum over rows of dy_j x^_j
 *
 * bf16 / fp16 compute in fp32 and round once; fp32 computes y and dx in fp64.
 * x, y, dy, dx: n_rows rows of hidden elements of dtype, row i at i * ld_*;
 * every row pointer 16-byte aligned (pointers and ld * element size multiples
 * of 16) and hidden a multiple of 8 (16-bit) or 4 (fp32), else
 * CE_ERR_UNSUPPORTED.  weight, dweight: hidden elements of dtype.  rstd:
 * n_rows floats, written by the forward and read by the backward.
 * Forward: hidden up to 16384 (16-bit) / 8192 (fp32); eps >= 0; y may be x
 * itself (same stride: each row is read whole before it is written).  The
 * 16-bit sum of squares runs in fp32 and is redone in fp64 when it overflows
 * or falls below 2^-100; with eps = 0, a row whose root mean square is below
 * 2^-128 gives rstd = inf.
 * Backward: hidden up to 16384 (16-bit) / 8192 (fp32); dx may be dy itself
 * (same stride); dweight is summed over the rows in fixed order
 * (deterministic) through a workspace of ce_rmsnorm_workspace_bytes() bytes
 * (256-byte aligned, no preparation needed, contents overwritten: not a
 * cross-entropy workspace that is still in use); dweight is all zeros when
 * n_rows == 0.  Errors: CE_ERR_DTYPE, CE_ERR_INVALID_ARG (negative sizes,
 * ld < hidden, NULL pointers, eps < 0 or NaN, aliasing with another stride,
 * dweight misaligned for dtype), CE_ERR_UNSUPPORTED (shape or alignment not
 * served), CE_ERR_WORKSPACE, CE_ERR_HIP (launch failure); nothing is written
 * on an error return.
 */
size_t ce_rmsnorm_workspace_bytes(int64_t n_rows, int64_t hidden, int dtype);
int ce_rmsnorm_forward(const void* x, int64_t ld_x, const void* weight, int64_t n_rows, int64_t hidden, int dtype,
                       float eps, void* y, int64_t ld_y, float* rstd, void* stream);
int ce_rmsnorm_backward(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* weight,
                        const float* rstd, int64_t n_rows, int64_t hidden, int dtype, void* dx, int64_t ld_dx,
                        void* dweight, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Rotary position embedding with per-token position ids.
 *
 * The pages list "Fast RoPE" among the package's kernels (PyPI page
 * "fms-acceleration-foak 0.7.4", kernel list) and note that it takes no
 * position ids (same page, known issues; fms-hf-tuning PR #280, "Notes on
 * FastKernels"); padding-free packed batches need them (positions restart at
 * each packed sequence).  For token t at position p = positions[t] and every
 * head of q and k, with D = head_dim and pairs i = 0 .. D/2-1 formed by
 * elements i and i + D/2:
 *
 *   theta = p * base^(-2 i / D)     (negated when inverse = 1)
 *   y_i       = x_i cos(theta) - x_{i+D/2} sin(theta)
 *   y_{i+D/2} = x_{i+D/2} cos(theta) + x_i sin(theta)
 *
 * inverse = 1 is the rotation back, i.e. the backward: dq = rope(dq_out, -theta).
 * q: q_heads heads of head_dim elements per token, element (t, h, j) at
 * q + (t * q_ld_token + h * q_ld_head + j) * element size; q_out has the same
 * strides and may be q itself (in place); likewise k (k_heads = 0: no k, the
 * pointers may be NULL).  positions: n_tokens int64 values.  Angles are
 * computed in fp64; 16-bit formats rotate in fp32 and round once, fp32 data
 * rotates in fp64.  The (token, head) segments must not overlap
 * (CE_ERR_INVALID_ARG).  Served: head_dim / 2 a multiple of 8 (16-bit) or 4
 * (fp32) and head_dim <= 256; pointers and strides * element size multiples of
 * 16 bytes; one token's heads spanning under 2 GiB (else CE_ERR_UNSUPPORTED).
 * Errors: CE_ERR_DTYPE, CE_ERR_INVALID_ARG (negative sizes, odd or < 2
 * head_dim, base not finite and positive, inverse not 0/1, NULL pointers,
 * overlapping segments), CE_ERR_UNSUPPORTED, CE_ERR_HIP; nothing is written on
 * an error return.  n_tokens = 0 (or no heads) returns CE_OK without reading any
 * pointer.  One kernel launch on `stream`; nothing is allocated.
 */
int ce_rope(const void* q, void* q_out, int64_t q_ld_token, int64_t q_ld_head, int64_t q_heads, const void* k,
            void* k_out, int64_t k_ld_token, int64_t k_ld_head, int64_t k_heads, const int64_t* positions,
            int64_t n_tokens, int64_t head_dim, double base, int inverse, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CE_MI355X_H */
