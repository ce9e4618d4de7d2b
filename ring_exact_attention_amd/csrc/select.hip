// Exact top-n block selection ("AnnAttention", select_block, with exact inner products
// in place of the approximate index).
//
// block_means: mean of each full block of bs key rows, in fp64 (exact for bf16 rows).
// block_select: one workgroup per (batch, block i of query positions; query row r sits
// at position q_pos0 + r of the key sequence, so decoding a few new tokens against a
// key cache is the same call).  The block's tokens score the candidate blocks
// c < i in chunks of 64 (16 per wavefront) with fp64 MFMA
// (bf16 queries are exact in fp64), the chunk's scores go to LDS, and one thread per
// token merges them into its running top-n list kept in LDS (score descending; on
// equal scores the earlier, lower index stays ahead).  The list is written sorted
// ascending with -1 padding first.
#include "common.h"
#include "launch.h"

namespace rea {

__global__ __launch_bounds__(256) void block_means_kernel(SelectArgs a) {
  const int c = blockIdx.x % a.nblk, b = blockIdx.x / a.nblk;
  const __bf16* kp = (const __bf16*)a.k + ((size_t)b * a.Skv + (size_t)c * a.bs) * a.E;
  double* mp = a.means + ((size_t)b * a.nblk + c) * a.E;
  for (int e = threadIdx.x; e < a.E; e += 256) {
    double s = 0.0;
    for (int r = 0; r < a.bs; ++r) s += (double)(float)kp[(size_t)r * a.E + e];
    mp[e] = s / (double)a.bs;
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Scores by v_mfma_f64_16x16x4_f64 (A: lane l holds A[l % 16][l / 16]; B: B[l / 16][l % 16];
// D: lane l, register r holds D[l / 16 + 4r][l % 16]).  The contraction index of the
// 4 MFMAs of one 16-wide slice is e = 16m + 4(l / 16) + s, so each lane reads 4
// consecutive embedding values per operand.  Tokens are the rows, candidates the columns.
template <int BS>
__global__ __launch_bounds__(256) void block_select_kernel(SelectArgs a) {
  constexpr int TB = BS / 16;             // 16-token blocks
  constexpr int CH = 64;                  // candidates per chunk (16 per wave)
  constexpr int NMAX = 16;                // largest top_n
  extern __shared__ __attribute__((aligned(16))) __bf16 sq[];   // BS * E (dynamic, <= 64 KiB)
  __shared__ double ssc[BS][CH + 1];
  __shared__ double best_s[BS][NMAX];
  __shared__ int best_c[BS][NMAX];

  const int first = a.q_pos0 / BS;
  const int nqb = (a.q_pos0 + a.S - 1) / BS - first + 1;
  const int i = first + blockIdx.x % nqb, b = blockIdx.x / nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int p0 = max(i * BS, a.q_pos0);                      // first query position of the block
  const int t0 = p0 - a.q_pos0;                               // its query row
  const int ntok = min((i + 1) * BS, a.q_pos0 + a.S) - p0;
  const int ncand = min(i, a.nblk);
  int kept = 0;                           // list length of token `tid` (threads < BS)

  if (ncand > 0) {
    const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.S + t0) * a.E;
    const int chunks = ntok * a.E / 8;
    for (int c = tid; c < chunks; c += 256)
      *(u32x4*)&sq[c * 8] = *(const u32x4*)(qp + (size_t)c * 8);
    for (int c = chunks + tid; c < BS * a.E / 8; c += 256) *(u32x4*)&sq[c * 8] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    const double* mbase = a.means + (size_t)b * a.nblk * a.E;
    const int col = lane & 15, grp = lane >> 4;
    for (int c0 = 0; c0 < ncand; c0 += CH) {
      const int cand = min(c0 + 16 * wave + col, ncand - 1);
      const double* mrow = mbase + (size_t)cand * a.E + 4 * grp;
      f64x4 acc[TB];
#pragma unroll
      for (int x = 0; x < TB; ++x) acc[x] = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int e0 = 0; e0 < a.E; e0 += 16) {
        const f64x4 mv = *(const f64x4*)(mrow + e0);
#pragma unroll
        for (int x = 0; x < TB; ++x) {
          const u32x2 qu = *(const u32x2*)&sq[(16 * x + col) * a.E + e0 + 4 * grp];
          const double q0 = bf16_lo(qu[0]), q1 = bf16_hi(qu[0]), q2 = bf16_lo(qu[1]), q3 = bf16_hi(qu[1]);
          acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q0, mv[0], acc[x], 0, 0, 0);
          acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q1, mv[1], acc[x], 0, 0, 0);
          acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q2, mv[2], acc[x], 0, 0, 0);
          acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q3, mv[3], acc[x], 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < TB; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) ssc[16 * x + grp + 4 * r][16 * wave + col] = acc[x][r];
      __syncthreads();
      if (tid < ntok) {
        const int nc = min(CH, ncand - c0);
        for (int y = 0; y < nc; ++y) {
          const double sc = ssc[tid][y];
          const int c = c0 + y;
          // insert (sc, c) if it beats the last kept entry; candidates arrive in
          // ascending index order, so an equal score never displaces an entry.
          if (kept < a.top_n || sc > best_s[tid][a.top_n - 1]) {
            int pos = kept < a.top_n ? kept : a.top_n - 1;
            while (pos > 0 && sc > best_s[tid][pos - 1]) {
              best_s[tid][pos] = best_s[tid][pos - 1];
              best_c[tid][pos] = best_c[tid][pos - 1];
              --pos;
            }
            best_s[tid][pos] = sc;
            best_c[tid][pos] = c;
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
      const int v = best_c[tid][x];
      int y = x - 1;
      while (y >= 0 && best_c[tid][y] > v) {
        best_c[tid][y + 1] = best_c[tid][y];
        --y;
      }
      best_c[tid][y + 1] = v;
    }
    int32_t* out = a.idx + ((size_t)b * a.S + t0 + tid) * a.top_n;
    const int pad = a.top_n - kept;
    for (int j = 0; j < a.top_n; ++j) out[j] = j < pad ? -1 : best_c[tid][j - pad];
  }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.nblk > 0)
    hipLaunchKernelGGL(block_means_kernel, dim3((unsigned)(a.B * a.nblk)), dim3(256), 0, stream, a);
  if (a.S == 0) return hipGetLastError();
  const int nqb = (a.q_pos0 + a.S - 1) / a.bs - a.q_pos0 / a.bs + 1;
  const dim3 grid((unsigned)(a.B * nqb));
  const size_t lds = (size_t)a.bs * a.E * sizeof(__bf16);
  switch (a.bs) {
    case 16: hipLaunchKernelGGL(block_select_kernel<16>, grid, dim3(256), lds, stream, a); break;
    case 32: hipLaunchKernelGGL(block_select_kernel<32>, grid, dim3(256), lds, stream, a); break;
    case 64: hipLaunchKernelGGL(block_select_kernel<64>, grid, dim3(256), lds, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rea
