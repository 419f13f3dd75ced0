// bf16 MFMA path of the covariance accumulation (cov_mfma.hip).
#pragma once
#include "lrc_internal.h"

namespace lrc {

// Shapes the MFMA path handles (rows of 16 bytes; head width a multiple of 32).
bool cov_mfma_shape_ok(int64_t d_in, int64_t d_out, int32_t n_blocks);
// Shape plus pointer/leading-dimension alignment of the actual call.
bool cov_mfma_supported(lrc_dtype x_t, const void *X, int64_t ldx, const void *W, int64_t ldw, int64_t d_in,
                        int64_t d_out, int32_t n_blocks);
size_t cov_mfma_workspace(int64_t n_tok, int64_t d_in, int has_w, int64_t d_out, int32_t n_blocks);
lrc_status cov_mfma_run(const CovArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

}  // namespace lrc
