// Exact top-n block selection ("AnnAttention", select_block, with exact inner products
// in place of the approximate index).
//
// block_means: mean of each full block of bs key rows, in fp64 (exact for bf16 rows).
// block_select: one workgroup per (batch, query block i).  The bs tokens of the block
// score the candidate blocks c < i in chunks of 64: each thread holds a tile of
// bs/16 tokens x 4 candidates of fp64 dot products over the embedding, the chunk's
// scores go to LDS, and one thread per token merges them into its running top-n
// list (score descending; on equal scores the earlier, lower index stays ahead).
// The list is written sorted ascending with -1 padding first.
#include "common.h"
#include "launch.h"

namespace rea {

__global__ __launch_bounds__(256) void block_means_kernel(SelectArgs a) {
  const int c = blockIdx.x % a.nblk, b = blockIdx.x / a.nblk;
  const __bf16* kp = (const __bf16*)a.k + ((size_t)b * a.S + (size_t)c * a.bs) * a.E;
  double* mp = a.means + ((size_t)b * a.nblk + c) * a.E;
  for (int e = threadIdx.x; e < a.E; e += 256) {
    double s = 0.0;
    for (int r = 0; r < a.bs; ++r) s += (double)(float)kp[(size_t)r * a.E + e];
    mp[e] = s / (double)a.bs;
  }
}

template <int BS>
__global__ __launch_bounds__(256) void block_select_kernel(SelectArgs a) {
  constexpr int TPT = BS / 16;            // tokens per thread
  constexpr int CPT = 4;                  // candidates per thread
  constexpr int CH = 16 * CPT;            // candidates per chunk
  constexpr int NMAX = 16;                // largest top_n
  __shared__ __attribute__((aligned(16))) __bf16 sq[32768];   // BS * E <= 32768 (host-checked)
  __shared__ double ssc[BS][CH + 1];

  const int nqb = (a.S + BS - 1) / BS;
  const int i = blockIdx.x % nqb, b = blockIdx.x / nqb;
  const int tid = threadIdx.x;
  const int t0 = i * BS;
  const int ntok = min(BS, a.S - t0);
  const int ncand = min(i, a.nblk);

  // top-n state of token `tid` (threads 0..BS-1)
  double best_s[NMAX];
  int best_c[NMAX];
#pragma unroll
  for (int j = 0; j < NMAX; ++j) {
    best_s[j] = -INFINITY;
    best_c[j] = -1;
  }
  int kept = 0;

  if (ncand > 0) {
    // stage the block's query rows (bf16) in LDS
    const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.S + t0) * a.E;
    const int chunks = ntok * a.E / 8;
    for (int c = tid; c < chunks; c += 256)
      *(u32x4*)&sq[c * 8] = *(const u32x4*)(qp + (size_t)c * 8);
    for (int c = chunks + tid; c < BS * a.E / 8; c += 256) *(u32x4*)&sq[c * 8] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    const int tg = tid / 16, cg = tid % 16;
    const double* mbase = a.means + (size_t)b * a.nblk * a.E;
    for (int c0 = 0; c0 < ncand; c0 += CH) {
      double acc[TPT][CPT];
#pragma unroll
      for (int x = 0; x < TPT; ++x)
#pragma unroll
        for (int y = 0; y < CPT; ++y) acc[x][y] = 0.0;
      const double* mrow[CPT];
#pragma unroll
      for (int y = 0; y < CPT; ++y) {
        const int c = min(c0 + cg * CPT + y, ncand - 1);
        mrow[y] = mbase + (size_t)c * a.E;
      }
      for (int e = 0; e < a.E; ++e) {
        double mv[CPT];
#pragma unroll
        for (int y = 0; y < CPT; ++y) mv[y] = mrow[y][e];
#pragma unroll
        for (int x = 0; x < TPT; ++x) {
          const double qv = (double)(float)sq[(tg * TPT + x) * a.E + e];
#pragma unroll
          for (int y = 0; y < CPT; ++y) acc[x][y] = fma(qv, mv[y], acc[x][y]);
        }
      }
#pragma unroll
      for (int x = 0; x < TPT; ++x)
#pragma unroll
        for (int y = 0; y < CPT; ++y) ssc[tg * TPT + x][cg * CPT + y] = acc[x][y];
      __syncthreads();
      if (tid < ntok) {
        const int nc = min(CH, ncand - c0);
        for (int y = 0; y < nc; ++y) {
          const double s = ssc[tid][y];
          const int c = c0 + y;
          // insert (s, c) if it beats the current last kept entry; candidates arrive
          // in ascending index order, so an equal score never displaces an entry.
          if (kept < a.top_n || s > best_s[a.top_n - 1]) {
            int pos = kept < a.top_n ? kept : a.top_n - 1;
            while (pos > 0 && s > best_s[pos - 1]) {
              best_s[pos] = best_s[pos - 1];
              best_c[pos] = best_c[pos - 1];
              --pos;
            }
            best_s[pos] = s;
            best_c[pos] = c;
            if (kept < a.top_n) ++kept;
          }
        }
      }
      __syncthreads();
    }
  }

  if (tid < ntok) {
    // sort the kept indices ascending (insertion sort on <= 16 entries)
    for (int x = 1; x < kept; ++x) {
      const int v = best_c[x];
      int y = x - 1;
      while (y >= 0 && best_c[y] > v) {
        best_c[y + 1] = best_c[y];
        --y;
      }
      best_c[y + 1] = v;
    }
    int32_t* out = a.idx + ((size_t)b * a.S + t0 + tid) * a.top_n;
    const int pad = a.top_n - kept;
    for (int j = 0; j < a.top_n; ++j) out[j] = j < pad ? -1 : best_c[j - pad];
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.nblk > 0)
    hipLaunchKernelGGL(block_means_kernel, dim3((unsigned)(a.B * a.nblk)), dim3(256), 0, stream, a);
  const int nqb = (a.S + a.bs - 1) / a.bs;
  const dim3 grid((unsigned)(a.B * nqb));
  switch (a.bs) {
    case 16: hipLaunchKernelGGL(block_select_kernel<16>, grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL(block_select_kernel<32>, grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(block_select_kernel<64>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rea
