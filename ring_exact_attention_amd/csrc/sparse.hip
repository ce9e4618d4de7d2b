// Attention over gathered candidates ("AnnAttention", faiss_block_attention).
#include "common.h"
#include "launch.h"

namespace rea {

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream) {
  (void)a;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace rea
