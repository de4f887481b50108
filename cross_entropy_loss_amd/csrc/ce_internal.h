// ce_internal.h -- entry points shared by the library's translation units and
// not exported from it (hidden visibility; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

extern "C" {

// The cross-entropy step of the LM-head path on one chunk: fp32 logits in
// (rows 16-byte aligned), loss rows and the token mean of the chunk out, and
// the gradient of dloss * L written to a separate bf16 / fp16 buffer (rows
// 8-byte aligned) in fp32 arithmetic.  Arguments as ce_fwd_bwd_inplace; the
// workspace is that of ce_workspace_bytes(n_rows, vocab, 0, CE_DTYPE_F32).
// Returns CE_ERR_UNSUPPORTED unless vocab is a multiple of 4 and at most
// 65536 with 16-byte aligned logits rows and 8-byte aligned gradient rows; the
// caller then takes the in-place fp32 path and a cast.
__attribute__((visibility("hidden"))) int ce_lin_chunk_f32_to16(
    const float* logits, int64_t ld, const int64_t* labels, int64_t n_rows, int64_t vocab, int out_dtype,
    int64_t ignore_index, const float* dloss, float* loss_mean, float* loss_rows, int32_t* n_valid, uint32_t* status,
    void* grad, int64_t grad_ld, void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // extern "C"
