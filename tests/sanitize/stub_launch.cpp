// Host-only stand-ins for the kernel launchers, so that the C-ABI layer (api.cpp) can be
// built without device code under AddressSanitizer / UndefinedBehaviorSanitizer.  Each
// launcher checks the argument struct the validation produced and returns success.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace rea {
int launches = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launcher received inconsistent arguments: %s\n", what);
    abort();
  }
}
hipError_t launch_fwd(int, const FwdArgs& a, hipStream_t) {
  expect(a.B > 0 && a.Sq > 0 && a.Hq % a.Hkv == 0 && a.G == a.Hq / a.Hkv, "fwd shape");
  expect(a.kv_block >= 1 && a.n_vblocks * a.kv_block == a.Skv, "fwd ring blocks");
  ++launches;
  return hipSuccess;
}
int fwd_tile_rows(int dtype) { return dtype == 0 ? 32 : 128; }
hipError_t launch_bwd(int, const BwdArgs& a, hipStream_t) {
  expect(a.B > 0 && a.Hq % a.Hkv == 0 && a.kv_splits >= 1 && a.G % a.kv_splits == 0, "bwd shape");
  expect(a.Dvec != nullptr && a.lse2 != nullptr && (a.kv_splits == 1) == (a.dkv_part == nullptr), "bwd workspace");
  ++launches;
  return hipSuccess;
}
int bwd_q_tile_rows(int dtype) { return dtype == 0 ? 32 : 128; }
int bwd_k_tile_rows(int) { return 128; }
hipError_t launch_select(const SelectArgs& a, hipStream_t) {
  expect(a.nblk == a.Skv / a.bs && a.nsplit >= 1 && (a.nsplit == 1 || (a.part_s && a.part_c)), "select");
  ++launches;
  return hipSuccess;
}
hipError_t launch_sparse(const SparseArgs& a, hipStream_t) {
  expect(a.E == 512 && a.top_n >= 1 && a.q_pos0 + a.S <= a.Skv, "sparse");
  ++launches;
  return hipSuccess;
}
hipError_t launch_sparse_bwd(const SparseBwdArgs& a, hipStream_t) {
  expect(a.E == 512 && a.Dvec && a.lse2, "sparse bwd");
  ++launches;
  return hipSuccess;
}
}
