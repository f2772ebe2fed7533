// Rank-r factor refresh (KVCMAS Eq. 7, App. B.1 "Factorization and Measurement").
#include "kvc_internal.h"

namespace kvc {

size_t svd_workspace_bytes(int n_mats, int rows, int cols, int rank, int oversample) {
  (void)n_mats; (void)rows; (void)cols; (void)rank; (void)oversample;
  return 256;
}

hipError_t svd_refresh(const float*, int, int, int, int, void*, void*, int, float*, int, int, uint64_t, void*, size_t,
                       hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvc
