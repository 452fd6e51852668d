// kvq_pca.hip — projection (PCA) variants of encode / decode / score.
#include "kvq_device.h"
#include "kvq_kernels.h"

namespace kvq {

hipError_t launch_encode_pca(int, int, int, bool, bool, const EncodeArgs&, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvq
