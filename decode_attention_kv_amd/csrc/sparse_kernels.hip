// Top-k sparse MLA-style decode (placeholder until the MFMA kernel lands).
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

size_t sparse_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_sparse(const void*, const void*, const int32_t*, int, int, int, int, int, int,
                         float, float*, float*, void*, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dakv
