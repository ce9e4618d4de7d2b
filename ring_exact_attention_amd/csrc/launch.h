// Internal launchers (host side), one per kernel family.  The C-ABI layer validates
// the public parameters, fills the argument structs and calls these.
#pragma once

#include "common.h"

namespace rea {

// dtype: 0 = bf16, 1 = fp32.  Head dims (q/k D, v Dv) with kernels built for them.
inline bool head_dims_supported(int dtype, int D, int Dv) {
  if (dtype == 0) return (D == Dv && (D == 32 || D == 64 || D == 128)) || (D == 128 && Dv == 64);
  return (D == Dv && (D == 32 || D == 64)) || (D == 64 && Dv == 32);
}
hipError_t launch_fwd(int dtype, const FwdArgs& a, hipStream_t stream);
int fwd_tile_rows(int dtype);

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t stream);
int bwd_q_tile_rows(int dtype);
int bwd_k_tile_rows(int dtype);

hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

// Work split of the gathered sparse forward: tokens per workgroup (32, halved while the
// grid would have fewer than 512 workgroups, down to 1) and, when the grid is still
// below 256 workgroups and a workspace is given, workgroups per token group over the
// group's 32-row steps (window blocks, then the union of selected blocks).
inline void sparse_plan(int B, int S, int window, int sel_block, int top_n, bool workspace, int& tpw,
                        int& ksplit) {
  tpw = 32;
  while (tpw > 1 && (long long)B * ((S + tpw - 1) / tpw) < 512) tpw >>= 1;
  ksplit = 1;
  const long long wg = (long long)B * ((S + tpw - 1) / tpw);
  if (!workspace || wg <= 0 || wg >= 256) return;
  const long long nwin = (window + tpw - 1 + 31) / 32, nsub = (sel_block + 31) / 32;
  const long long ent = (long long)tpw * top_n < 512 ? (long long)tpw * top_n : 512;
  long long ks = 256 / wg;
  if (ks > nwin + ent * nsub) ks = nwin + ent * nsub;
  ksplit = ks < 1 ? 1 : (int)ks;
}

// Workgroups per query block of block_select.  While the grid would have fewer than 256
// workgroups (a few tokens, e.g. decoding), each query block's chunks of 64 candidate
// blocks are shared out over several workgroups whose top-n lists a merge kernel
// combines (at most 64 list entries per token).
inline int select_splits(int B, int S, int q_pos0, int bs, int nblk, int top_n) {
  if (B <= 0 || S <= 0 || bs <= 0 || top_n < 1 || top_n > 16) return 1;
  const long long nqb = (long long)(q_pos0 + S - 1) / bs - q_pos0 / bs + 1;
  const long long wg = (long long)B * nqb;
  if (wg >= 256) return 1;
  long long ns = 256 / wg;
  const long long chunks = (nblk + 63) / 64;
  if (ns > chunks) ns = chunks;
  if (ns > 64 / top_n) ns = 64 / top_n;
  return ns < 1 ? 1 : (int)ns;
}
hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream);

// Sets this thread's attn_last_error() message and returns `code`.
int report_error(int code, const char* msg);
hipError_t launch_sparse_bwd(const SparseBwdArgs& a, hipStream_t stream);

}  // namespace rea
