// Exact top-n block selection ("AnnAttention", select_block, with exact inner products
// in place of the approximate index).
//
// block_means: mean of each full block of bs key rows, in fp64 (exact for bf16 rows).
// block_select: one workgroup per (batch, block i of query positions; query row r sits
// at position q_pos0 + r of the key sequence, so decoding a few new tokens against a
// key cache is the same call).  The block's tokens score the candidate blocks
// c < i in chunks of 64 (16 per wavefront) with fp64 MFMA (bf16 queries are exact in
// fp64), the chunk's scores go to LDS, and each token's running top-n list (in LDS,
// score descending; on equal scores the lower index ahead) absorbs the chunk in one
// parallel step: a wavefront per token ranks the candidates that beat the list's last
// entry against the list and each other and writes every survivor to its rank.  The
// list is written sorted ascending with -1 padding first.
#include "common.h"
#include "launch.h"

namespace rea {

// One workgroup per (batch, block): a thread sums 8 consecutive columns over every
// RG-th row of the block (16-byte loads; RG = 256 / (E / 8) row groups), the row groups
// are added in LDS.  All partial sums of bf16 values are exact in fp64, so the order
// does not change the mean.
__global__ __launch_bounds__(256) void block_means_kernel(SelectArgs a) {
  __shared__ double part[256 * 8];
  const int wg = wg_index(a.rev_order), c = wg % a.nblk, b = wg / a.nblk;
  const __bf16* kp = (const __bf16*)a.k + ((size_t)b * a.Skv + (size_t)c * a.bs) * a.E;
  double* mp = a.means + ((size_t)b * a.nblk + c) * a.E;
  const int cpr = a.E / 8;                               // 16-byte chunks per row (8 .. 128)
  const int rg = 256 / cpr;                               // row groups (2 .. 32)
  const int tid = threadIdx.x, g = tid / cpr, ch = tid - g * cpr;
  double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (g < rg) {
    for (int r = g; r < a.bs; r += rg) {
      const u32x4 u = *(const u32x4*)(kp + (size_t)r * a.E + 8 * ch);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s[2 * w] += (double)bf16_lo(u[w]);
        s[2 * w + 1] += (double)bf16_hi(u[w]);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) part[x * 256 + tid] = s[x];
  __syncthreads();
  for (int e = tid; e < a.E; e += 256) {
    const int ch2 = e / 8, x = e % 8;
    double t = 0.0;
    for (int g2 = 0; g2 < rg; ++g2) t += part[x * 256 + g2 * cpr + ch2];
    mp[e] = t / (double)a.bs;
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// The wavefront's maximum of x, in every lane: DPP within each row of 16 lanes (quad
// swaps, then the half-row and row mirrors), then the row-swapping permutes; all VALU,
// where a shuffle through ds_bpermute puts an LDS round trip on each of the six steps.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16_f32(float x) {   // lane i's value from lane i ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32_f32(float x) {   // ... from lane i ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));    // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4E>(x));    // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));   // row_half_mirror: the two quads of each 8 lanes
  x = fmaxf(x, dpp_f32<0x140>(x));   // row_mirror: the two halves of each 16-lane row
  x = fmaxf(x, xor16_f32(x));
  x = fmaxf(x, xor32_f32(x));
  return x;
}

// Lane y's value of x (y uniform across the wavefront).
__device__ __forceinline__ double read_lane_f64(double x, int y) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, y);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), y);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Row pitch (elements) of the queries staged in LDS: padded by 8 so that the 16 rows one
// MFMA operand read touches fall in different banks, unless that would pass 64 KiB.
__host__ __device__ inline int sq_pitch(int bs, int E) { return bs * (E + 8) * 2 <= 65536 ? E + 8 : E; }

// Scores by v_mfma_f64_16x16x4_f64 (A: lane l holds A[l % 16][l / 16]; B: B[l / 16][l % 16];
// D: lane l, register r holds D[l / 16 + 4r][l % 16]).  The contraction index of the
// 4 MFMAs of one 16-wide slice is e = 16m + 4(l / 16) + s, so each lane reads 4
// consecutive embedding values per operand.  Tokens are the rows, candidates the columns.
template <int BS>
__global__ __launch_bounds__(256) void block_select_kernel(SelectArgs a) {
  constexpr int TB = BS / 16;             // 16-token blocks
  constexpr int CH = 64;                  // candidates per chunk (16 per wave)
  constexpr int NMAX = 16;                // largest top_n
  extern __shared__ __attribute__((aligned(16))) __bf16 sq[];   // BS rows of sq_pitch (dynamic)
  __shared__ double ssc[BS][CH + 1];
  __shared__ double best_s[BS][NMAX];
  __shared__ int best_c[BS][NMAX];

  const int first = a.q_pos0 / BS;
  const int nqb = (a.q_pos0 + a.S - 1) / BS - first + 1;
  const int ns = a.nsplit, wg = wg_index(a.rev_order), split = wg % ns, qb = wg / ns;
  // longest first: query block i scores i candidates, so the grid walks i downwards (all
  // sequences of the batch at each i) and the short blocks fill in behind the long ones
  const int i = first + (nqb - 1 - qb / a.B), b = qb % a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int p0 = max(i * BS, a.q_pos0);                      // first query position of the block
  const int t0 = p0 - a.q_pos0;                               // its query row
  const int ntok = min((i + 1) * BS, a.q_pos0 + a.S) - p0;
  const int ncand = min(i, a.nblk);
  // this workgroup's share of the candidates: whole chunks [c_begin, c_end)
  const int nch = (ncand + CH - 1) / CH, cps = (nch + ns - 1) / ns;
  const int c_begin = min(ncand, split * cps * CH), c_end = min(ncand, (split + 1) * cps * CH);

  if (c_begin < c_end) {
    const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.S + t0) * a.E;
    const int pitch = sq_pitch(BS, a.E), cpr = a.E / 8;
    for (int c = tid; c < BS * cpr; c += 256) {
      const int t = c / cpr, ch = c - t * cpr;
      u32x4 u = {0u, 0u, 0u, 0u};
      if (t < ntok) u = *(const u32x4*)(qp + (size_t)t * a.E + 8 * ch);
      *(u32x4*)&sq[t * pitch + 8 * ch] = u;
    }
    __syncthreads();

    const double* mbase = a.means + (size_t)b * a.nblk * a.E;
    const int col = lane & 15, grp = lane >> 4;
    for (int c0 = c_begin; c0 < c_end; c0 += CH) {
      const int cand = min(c0 + 16 * wave + col, ncand - 1);
      const double* mrow = mbase + (size_t)cand * a.E + 4 * grp;
      f64x4 acc[TB];
#pragma unroll
      for (int x = 0; x < TB; ++x) acc[x] = f64x4{0.0, 0.0, 0.0, 0.0};
      // The candidate's means stream through a ring of PF 16-wide slices loaded PF slices
      // ahead (a past-the-end slice rereads slice 0), so the L2 latency overlaps the MFMAs.
      constexpr int PF = 8;
      f64x4 mv[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) mv[u] = *(const f64x4*)(mrow + (16 * u < a.E ? 16 * u : 0));
      for (int e0 = 0; e0 < a.E; e0 += 16 * PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int e = e0 + 16 * u, en = e + 16 * PF;
          const f64x4 m4 = mv[u];
          mv[u] = *(const f64x4*)(mrow + (en < a.E ? en : 0));
          if (e < a.E) {
#pragma unroll
            for (int x = 0; x < TB; ++x) {
              if (16 * x >= ntok) break;                   // no token in this 16-row tile
              const u32x2 qu = *(const u32x2*)&sq[(16 * x + col) * pitch + e + 4 * grp];
              const double q0 = bf16_lo(qu[0]), q1 = bf16_hi(qu[0]), q2 = bf16_lo(qu[1]), q3 = bf16_hi(qu[1]);
              acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q0, m4[0], acc[x], 0, 0, 0);
              acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q1, m4[1], acc[x], 0, 0, 0);
              acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q2, m4[2], acc[x], 0, 0, 0);
              acc[x] = __builtin_amdgcn_mfma_f64_16x16x4f64(q3, m4[3], acc[x], 0, 0, 0);
            }
          }
        }
      }
#pragma unroll
      for (int x = 0; x < TB; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) ssc[16 * x + grp + 4 * r][16 * wave + col] = acc[x][r];
      __syncthreads();
      // Merge the chunk into each token's list.  Before the chunk the list holds
      // kept0 = min(n, c0 - c_begin) entries.  Lane y carries candidate c0 + y; those not above
      // the last entry of a full list cannot place (ties go to the lower index).  A
      // survivor's rank counts the list entries >= it and the survivors above it (or
      // equal with a lower index); list entry e moves down by the survivors above it.
      {
        const int n = a.top_n, nc = min(CH, c_end - c0), kept0 = min(n, c0 - c_begin);
        for (int t = wave; t < ntok; t += 4) {
          const bool cval = lane < nc;
          const double v = cval ? ssc[t][lane] : 0.0;
          double thr = kept0 < n ? -INFINITY : best_s[t][n - 1];
          bool surv = cval && v > thr;
          if (kept0 == 0 && nc > n) {
            // Empty list (a share's first chunk): only the chunk's n largest scores can
            // enter it, so keep the candidates at or above the n-th largest (counted with
            // multiplicity; ties at it survive and are ranked by index below) instead of
            // ranking all of them against each other.  The cut is taken on the scores
            // rounded to fp32, which keeps their order (a >= b gives f(a) >= f(b)): the n-th
            // largest rounded score is the rounding of the n-th largest score, so every
            // candidate at or above the latter passes; the few more that round to the same
            // value are ranked exactly below and drop out there.
            const float vf = (float)v;
            float cut = INFINITY;
            int cnt = 0;
            for (int it = 0; it < n && cnt < n; ++it) {
              cut = wave_max_f32(cval && vf < cut ? vf : -INFINITY);
              cnt += __popcll(__ballot(cval && vf == cut));
            }
            surv = cval && vf >= cut;
          }
          const uint64_t P = __ballot(surv);
          if (P == 0) continue;                          // nothing enters: the list stays
          const bool is_l = lane < kept0;
          const double ls = is_l ? best_s[t][lane] : 0.0;
          const int lc = is_l ? best_c[t][lane] : 0;
          int rc = 0, rl = lane;
          for (int e = 0; e < kept0; ++e) rc += read_lane_f64(ls, e) >= v ? 1 : 0;
          for (uint64_t m = P; m; m &= m - 1) {
            const int y = __builtin_ctzll(m);
            const double w = read_lane_f64(v, y);
            rc += (w > v || (w == v && y < lane)) ? 1 : 0;
            rl += w > ls ? 1 : 0;
          }
          if (surv && rc < n) {
            best_s[t][rc] = v;
            best_c[t][rc] = c0 + lane;
          }
          if (is_l && rl < n) {
            best_s[t][rl] = ls;
            best_c[t][rl] = lc;
          }
        }
      }
      __syncthreads();
    }
  }

  if (ns > 1 && tid < ntok) {
    // a share of the candidates: the list as ranked (index -1 = empty) for the merge
    const int kept = min(a.top_n, c_end - c_begin);
    const size_t base = ((size_t)(b * a.S + t0 + tid) * ns + split) * a.top_n;
    for (int j = 0; j < a.top_n; ++j) {
      a.part_s[base + j] = j < kept ? best_s[tid][j] : -INFINITY;
      a.part_c[base + j] = j < kept ? best_c[tid][j] : -1;
    }
  } else if (tid < ntok) {
    const int kept = min(a.top_n, ncand);
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

// Combines the nsplit partial lists of each token (disjoint candidate ranges), one
// wavefront per token: an entry's rank counts the entries that beat it (a higher score,
// or an equal one with a lower index -- the order one workgroup's merge keeps); ranks
// below top_n are kept and written ascending by index after the -1 padding.
__global__ __launch_bounds__(256) void block_select_merge_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const long long tok = (long long)wg_index(a.rev_order) * 4 + wave_id();
  if (tok >= (long long)a.B * a.S) return;               // the whole wavefront
  const int n = a.top_n, ne = a.nsplit * n;
  double s = -INFINITY;
  int c = -1;
  if (lane < ne) {
    s = a.part_s[tok * ne + lane];
    c = a.part_c[tok * ne + lane];
  }
  const bool valid = c >= 0;
  int rank = 0;
  for (uint64_t m = __ballot(valid); m; m &= m - 1) {
    const int y = __builtin_ctzll(m);
    const double w = read_lane_f64(s, y);
    const int cy = __builtin_amdgcn_readlane(c, y);
    rank += (w > s || (w == s && cy < c)) ? 1 : 0;
  }
  const bool keep = valid && rank < n;
  const uint64_t K = __ballot(keep);
  int pos = 0;                                            // among the kept, by index
  for (uint64_t m = K; m; m &= m - 1) pos += __builtin_amdgcn_readlane(c, __builtin_ctzll(m)) < c ? 1 : 0;
  int32_t* out = a.idx + tok * n;
  const int pad = n - __popcll(K);
  if (keep) out[pad + pos] = c;
  if (lane < pad) out[lane] = -1;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.nblk > 0)
    hipLaunchKernelGGL(block_means_kernel, dim3((unsigned)(a.B * a.nblk)), dim3(256), 0, stream, a);
  if (a.S == 0) return hipGetLastError();
  const int nqb = (a.q_pos0 + a.S - 1) / a.bs - a.q_pos0 / a.bs + 1;
  const dim3 grid((unsigned)(a.B * nqb * a.nsplit));
  const size_t lds = (size_t)a.bs * sq_pitch(a.bs, a.E) * sizeof(__bf16);
  switch (a.bs) {
    case 16: hipLaunchKernelGGL(block_select_kernel<16>, grid, dim3(256), lds, stream, a); break;
    case 32: hipLaunchKernelGGL(block_select_kernel<32>, grid, dim3(256), lds, stream, a); break;
    case 64: hipLaunchKernelGGL(block_select_kernel<64>, grid, dim3(256), lds, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.nsplit > 1) {
    const long long toks = (long long)a.B * a.S;
    hipLaunchKernelGGL(block_select_merge_kernel, dim3((unsigned)((toks + 3) / 4)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rea
