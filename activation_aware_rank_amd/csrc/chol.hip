// Curvature-weighted variant (LASER page, method 1): Cholesky factor and triangular products /
// solves with it.  Filled in by a later change; until then these report LRC_ERR_UNIMPLEMENTED.
#include "lrc_internal.h"

namespace lrc {

size_t cholesky_workspace(int64_t) { return 0; }

lrc_status cholesky_run(double *, int64_t, int64_t, void *, size_t, int32_t *, hipStream_t) {
    return fail(LRC_ERR_UNIMPLEMENTED, "lrc_cholesky is not implemented in this build");
}

lrc_status trmm_run(int, int, int64_t, int64_t, const double *, int64_t, double *, int64_t, hipStream_t) {
    return fail(LRC_ERR_UNIMPLEMENTED, "lrc_trmm is not implemented in this build");
}

lrc_status trsm_run(int, int, int64_t, int64_t, const double *, int64_t, double *, int64_t, hipStream_t) {
    return fail(LRC_ERR_UNIMPLEMENTED, "lrc_trsm is not implemented in this build");
}

}  // namespace lrc
