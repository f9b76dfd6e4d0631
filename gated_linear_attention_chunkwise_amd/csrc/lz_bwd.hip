// lz_bwd.hip -- backward pass (placeholder until the kernels land).
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {

size_t bwd_workspace_bytes(int B, int H, int L, int M, int D) {
  (void)B; (void)H; (void)L; (void)M; (void)D;
  return 0;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int D, hipStream_t st) {
  (void)a; (void)dtype; (void)D; (void)st;
  return hipErrorNotSupported;
}

}  // namespace lz
