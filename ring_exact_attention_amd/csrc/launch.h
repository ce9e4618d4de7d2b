// Internal launchers (host side), one per kernel family.  The C-ABI layer validates
// the public parameters, fills the argument structs and calls these.
#pragma once

#include "common.h"

namespace rea {

// dtype: 0 = bf16, 1 = fp32.  Head dims (q/k D, v Dv) with kernels built for them.
bool head_dims_supported(int dtype, int D, int Dv);
hipError_t launch_fwd(int dtype, const FwdArgs& a, hipStream_t stream);
int fwd_tile_rows(int dtype);

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t stream);
int bwd_q_tile_rows(int dtype);
int bwd_k_tile_rows(int dtype);

hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream);
hipError_t launch_sparse_bwd(const SparseBwdArgs& a, hipStream_t stream);

}  // namespace rea
