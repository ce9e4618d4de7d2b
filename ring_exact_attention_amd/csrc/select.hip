// Exact top-n block selection ("AnnAttention", select_block, with exact inner
// products in place of the approximate index).
#include "common.h"
#include "launch.h"

namespace rea {

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  (void)a;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace rea
