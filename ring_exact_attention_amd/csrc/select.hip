// Exact top-n block selection ("AnnAttention", select_block, with exact inner products
// in place of the approximate index).
//
// block_means: mean of each full block of bs key rows, in fp64 (exact for bf16 rows),
// with its two bf16 parts and its norm.
// Selection: one workgroup per (batch, block i of query positions; query row r sits at
// position q_pos0 + r of the key sequence, so decoding a few new tokens against a key
// cache is the same call).  Up to 256 key blocks (and 256 or more query blocks),
// block_select_bf16_kernel scores all candidates c < i in bf16 with an error bound and
// scores in fp64 only those the bound leaves undecided.  Otherwise block_select_kernel
// scores the candidates in chunks of
// 64 (16 per wavefront) with fp64 MFMA (bf16 queries are exact in fp64), the chunk's
// scores go to LDS, and each token's running top-n list (in LDS, score descending; on
// equal scores the lower index ahead) absorbs the chunk in one parallel step: a
// wavefront per token ranks the candidates that beat the list's last entry against the
// list and each other and writes every survivor to its rank.  Either way the list is
// written sorted ascending with -1 padding first.
#include "common.h"
#include "launch.h"

namespace rea {

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

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double xor16_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const auto l = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
  const auto h = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const bool odd = ((threadIdx.x >> 4) & 1) != 0;
  return __longlong_as_double((long long)(((unsigned long long)(odd ? h[0] : h[1]) << 32) | (odd ? l[0] : l[1])));
}
__device__ __forceinline__ double xor32_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const auto l = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const bool up = (threadIdx.x & 32) != 0;
  return __longlong_as_double((long long)(((unsigned long long)(up ? h[0] : h[1]) << 32) | (up ? l[0] : l[1])));
}
// Wavefront sum / maximum of doubles, the same value in every lane (partners add the same
// two values, so the order is fixed): quad swaps, half-row and row mirrors, row swaps.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);
  x += dpp_f64<0x4E>(x);
  x += dpp_f64<0x141>(x);
  x += dpp_f64<0x140>(x);
  x += xor16_f64(x);
  x += xor32_f64(x);
  return x;
}
__device__ __forceinline__ double wave_max_f64(double x) {
  x = fmax(x, dpp_f64<0xB1>(x));
  x = fmax(x, dpp_f64<0x4E>(x));
  x = fmax(x, dpp_f64<0x141>(x));
  x = fmax(x, dpp_f64<0x140>(x));
  x = fmax(x, xor16_f64(x));
  x = fmax(x, xor32_f64(x));
  return x;
}
__device__ __forceinline__ int wave_min_i32(int x) {
  x = min(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = min(x, (int)(((threadIdx.x >> 4) & 1) ? r16[0] : r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  x = min(x, (int)((threadIdx.x & 32) ? r32[0] : r32[1]));
  return x;
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// One workgroup per (batch, block): a thread sums 8 consecutive columns over every
// RG-th row of the block (16-byte loads; RG = 256 / (E / 8) row groups), the row groups
// are added in LDS.  All partial sums of bf16 values are exact in fp64, so the order
// does not change the mean.
__global__ __launch_bounds__(256) void block_means_kernel(SelectArgs a) {
  __shared__ double part[256 * 8];
  const int nm = a.mto - a.mfrom;                       // blocks per sequence this call
  const int wg = wg_index(a.rev_order), c = a.mfrom + wg % nm, b = wg / nm;
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
  // The mean, its two bf16 parts (the second the rounding of what the first leaves; the
  // difference is exact in fp64) and the sum of squares for the norm.
  const size_t plane = (size_t)a.B * a.nblk * a.E;
  uint16_t* sp = a.msplit + ((size_t)b * a.nblk + c) * a.E;
  double sq2 = 0.0;
  for (int e = tid; e < a.E; e += 256) {
    const int ch2 = e / 8, x = e % 8;
    double t = 0.0;
    for (int g2 = 0; g2 < rg; ++g2) t += part[x * 256 + g2 * cpr + ch2];
    t /= (double)a.bs;
    mp[e] = t;
    sq2 = fma(t, t, sq2);
    double r = t;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint16_t h = bf16_bits_rne((float)r);
      sp[k * plane + e] = h;
      r -= (double)__uint_as_float((uint32_t)h << 16);
    }
  }
  __syncthreads();
  part[tid] = sq2;
  __syncthreads();
  if (tid < 64) {
    const double t = wave_sum_f64(part[tid] + part[tid + 64] + part[tid + 128] + part[tid + 192]);
    const float nf = (float)sqrt(t);
    if (tid == 0) a.mnorm[(size_t)b * a.nblk + c] = __uint_as_float(__float_as_uint(nf) + 1u);   // one ulp up
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Order-preserving integer key of a float (the sign-magnitude bits mapped to two's
// complement; -0 sorts below +0) and its inverse.
__device__ __forceinline__ int f32_key(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_f32(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }
// Wavefront maximum of ints, uniform: DPP within each 16-lane row (quad swaps, half-row
// and row mirrors), then lane 15 of rows 0 and 2 into rows 1 and 3 and lane 31 into rows
// 2 and 3 (row broadcasts; rows outside the mask see the minimum), read from lane 63.
// Four independent maxima, their steps interleaved (each step's DPP waits for the
// previous step's write; the other three values fill that wait).
__device__ __forceinline__ void wave_max4_i32(int (&x)[4]) {
#define REA_DPP_MAX4(CTRL, RM)                                                              \
  _Pragma("unroll") for (int u = 0; u < 4; ++u)                                            \
      x[u] = max(x[u], __builtin_amdgcn_update_dpp(INT_MIN, x[u], CTRL, RM, 0xF, false));
  REA_DPP_MAX4(0xB1, 0xF)
  REA_DPP_MAX4(0x4E, 0xF)
  REA_DPP_MAX4(0x141, 0xF)
  REA_DPP_MAX4(0x140, 0xF)
  REA_DPP_MAX4(0x142, 0xA)
  REA_DPP_MAX4(0x143, 0xC)
#undef REA_DPP_MAX4
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = __builtin_amdgcn_readlane(x[u], 63);
}
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0xB1, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x4E, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x141, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x140, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
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

// Top-n selection with approximate scores and an error bound, for up to 256 candidate
// blocks.  With the means written as m = h + d + r (two bf16 parts, |r| <= 2^-17 |m|), the
// scores s~ = q . (h + d) come from bf16 MFMA with fp32 accumulation.  The products are
// exact in fp32 and each of the 2 E / 16 instructions adds at most 17 roundings of at
// most 2^-23 of a partial sum (even if they truncate), so
//   |s~ - s| <= (2 E/16 * 17 * 2^-23 (1 + 2^-8) + 2^-17) sum_e |q_e| |m_e|,
// and sum_e |q_e| |m_e| <= |q| |m| (Cauchy-Schwarz; 2^-12.8 |q| |m| at E = 512).  Eb, 1.25
// times that with |q| and max|m| rounded up, bounds it with room for the fp32 rounding
// of the thresholds below.  With v_n >= v_n+1 the n-th
// and (n+1)-th largest s~ (counted with multiplicity):
//   * s~_c > v_n+1 + 2 Eb: at most n candidates have s~ > v_n+1, and every candidate that
//     ties or beats c has s > v_n+1 + Eb, hence s~ > v_n+1: c is in the top n;
//   * s~_c < v_n - 2 Eb: the n candidates with s~ >= v_n all have s > s_c: c is out;
//   * the rest (usually none) get exact fp64 scores, and the top n - k of them (by score,
//     then lower index) join the k sure ones: leaving out candidates that are out does
//     not change the order of the others.
// The set is the exact top n (ties to the lower index) of the exact fp64 scores.
// One workgroup per (batch, query block), no candidate split; the scores of all
// candidates sit in LDS.  BS tokens, four wavefronts: scoring takes 32 candidates per
// wavefront pass (v_mfma_f32_32x32x16_bf16, 32 tokens x 32 candidates; at most two passes
// per wavefront, held in registers until every wavefront is done with the queries, whose
// LDS the scores then take over), the selection one wavefront per token (lane y holds
// candidates y, y + 64, y + 128, y + 192).
constexpr int kSelFastMax = 256;
// floats per token row of scores: padded against bank conflicts of the score stores,
// except with 64 tokens, where the padding would take the table past 64 KiB
__host__ __device__ constexpr int sel_score_pitch(int bs) { return bs >= 64 ? kSelFastMax : kSelFastMax + 4; }
__host__ __device__ inline size_t sel_fast_lds(int bs, int E) {
  const size_t q = (size_t)bs * sq_pitch(bs, E) * 2, sc = (size_t)bs * sel_score_pitch(bs) * 4;
  return q > sc ? q : sc;
}

template <int BS>
__global__ __launch_bounds__(256, 4) void block_select_bf16_kernel(SelectArgs a) {
  constexpr int NC = kSelFastMax;
  constexpr int TT = (BS + 31) / 32;      // 32-token tiles
  constexpr int SP = sel_score_pitch(BS);
  constexpr int NT = NC / 32 / 4;         // candidate tiles per wavefront
  extern __shared__ __attribute__((aligned(16))) char sel_lds[];   // queries, then scores
  __bf16* const sq = (__bf16*)sel_lds;                              // BS rows of sq_pitch
  float (*const ssc)[SP] = (float (*)[SP])sel_lds;                  // BS rows of SP
  __shared__ float snq[BS];

  const int first = a.q_pos0 / BS;
  const int nqb = (a.q_pos0 + a.S - 1) / BS - first + 1;
  const int qb = wg_index(a.rev_order);
  const int i = first + (nqb - 1 - qb / a.B), b = qb % a.B;   // longest first
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int p0 = max(i * BS, a.q_pos0);
  const int t0 = p0 - a.q_pos0;
  const int ntok = min((i + 1) * BS, a.q_pos0 + a.S) - p0;
  const int ncand = min(i, a.nblk);
  const int pitch = sq_pitch(BS, a.E), cpr = a.E / 8;

  const __bf16* qp = (const __bf16*)a.q + ((size_t)b * a.S + t0) * a.E;
  for (int c = tid; c < BS * cpr; c += 256) {
    const int t = c / cpr, ch = c - t * cpr;
    u32x4 u = {0u, 0u, 0u, 0u};
    if (t < ntok) u = *(const u32x4*)(qp + (size_t)t * a.E + 8 * ch);
    *(u32x4*)&sq[t * pitch + 8 * ch] = u;
  }
  __syncthreads();

  // |q| per token (fp32 sum of squares; its relative error, below E 2^-24, is covered by
  // the 2^-8 it is scaled up by) and the largest |m| among the candidates.
  for (int t = wave; t < ntok; t += 4) {
    float ss = 0.f;
    for (int ch = lane; ch < cpr; ch += 64) {
      const u32x4 u = *(const u32x4*)&sq[t * pitch + 8 * ch];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ss = fmaf(bf16_lo(u[w]), bf16_lo(u[w]), ss);
        ss = fmaf(bf16_hi(u[w]), bf16_hi(u[w]), ss);
      }
    }
    ss += dpp_f32<0xB1>(ss);
    ss += dpp_f32<0x4E>(ss);
    ss += dpp_f32<0x141>(ss);
    ss += dpp_f32<0x140>(ss);
    ss += xor16_f32(ss);
    ss += xor32_f32(ss);
    if (lane == 0) snq[t] = sqrtf(ss) * (1.f + 1.f / 256.f);
  }
  float mmax = 0.f;
  for (int c = lane; c < ncand; c += 64) mmax = fmaxf(mmax, a.mnorm[(size_t)b * a.nblk + c]);
  mmax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_max_f32(mmax))));

  // Approximate scores of the candidates, 32 per wavefront pass.
  const size_t plane = (size_t)a.B * a.nblk * a.E;
  const uint16_t* sp0 = a.msplit + (size_t)b * a.nblk * a.E;
  const int ntile = (ncand + 31) / 32, nks = a.E / 16;
  f32x16 acc[NT][TT];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int x = 0; x < TT; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[it][x][r] = 0.f;
  // The wavefront's NA active tiles (candidates 32 ct .. of ct = wave, wave + 4) share one
  // k-step loop, so their loads are in flight together; the two parts of k-steps
  // ks .. ks + PF - 1 are loaded ahead of their MFMAs (PF = 8 / NA).
  auto score = [&](auto na_c) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_c)::value, PF = 8 / NA;
    const uint16_t* mrow[NA];
#pragma unroll
    for (int it = 0; it < NA; ++it)
      mrow[it] = sp0 + (size_t)min(32 * (wave + 4 * it) + li, ncand - 1) * a.E + 8 * lh;
    u32x4 mb[PF][NA][2];
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int it = 0; it < NA; ++it)
#pragma unroll
        for (int k = 0; k < 2; ++k) mb[u][it][k] = *(const u32x4*)(mrow[it] + k * plane + 16 * (u < nks ? u : 0));
    // nks is a multiple of 4, not always of PF: k-steps past the end are skipped
    for (int ks0 = 0; ks0 < nks; ks0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int ks = ks0 + u, kn = ks + PF < nks ? ks + PF : 0;
        if (ks >= nks) break;
        u32x4 m3[NA][2];
#pragma unroll
        for (int it = 0; it < NA; ++it)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            m3[it][k] = mb[u][it][k];
            mb[u][it][k] = *(const u32x4*)(mrow[it] + k * plane + 16 * kn);
          }
#pragma unroll
        for (int x = 0; x < TT; ++x) {
          const int row = 32 * x + li;
          u32x4 qu = {0u, 0u, 0u, 0u};
          if (BS >= 32 || row < BS) qu = *(const u32x4*)&sq[row * pitch + 16 * ks + 8 * lh];
          const bf16x8 qa = as_bf16x8(qu);
#pragma unroll
          for (int it = 0; it < NA; ++it)
#pragma unroll
            for (int k = 0; k < 2; ++k) acc[it][x] = mfma32(qa, as_bf16x8(m3[it][k]), acc[it][x]);
        }
      }
    }
  };
  static_assert(NT == 2, "a wavefront scores at most two 32-candidate tiles");
  if (wave + 4 < ntile) score(IntConst<2>{});
  else if (wave < ntile) score(IntConst<1>{});
  __syncthreads();                                 // the queries' LDS becomes the scores'
  // lane (candidate li) holds tokens 8g + 4lh + e of each 32-token tile
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const int ct = wave + 4 * it;
    if (ct >= ntile) continue;
#pragma unroll
    for (int x = 0; x < TT; ++x)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 32 * x + 8 * g + 4 * lh + e;
          if (BS >= 32 || row < BS) ssc[row][32 * ct + li] = acc[it][x][4 * g + e];
        }
  }
  __syncthreads();

  const int n = a.top_n;
  const double* mean0 = a.means + (size_t)b * a.nblk * a.E;
  // error bound per unit of |q| max|m| (the rounding count above, with a quarter of room)
  const float ceb = 1.25f * (2.f * (float)(a.E / 16) * 17.f * 0x1p-23f * (1.f + 0x1p-8f) + 0x1p-17f);
  bool valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) valid[j] = lane + 64 * j < ncand;
  // Four tokens of this wavefront at a time (t = wave + 4 (4 g + u)), their rounds
  // interleaved so that one token's reductions fill the others' latencies.
  for (int g0 = wave; g0 < ntok; g0 += 16) {
    constexpr int U = 4;
    float v[U][4], vn[U], vn1[U], eb[U];
    int kv[U][4], cnt[U];
    bool all_exact[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(g0 + 4 * u, ntok - 1);
      bool fin = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[u][j] = valid[j] ? ssc[t][lane + 64 * j] : -INFINITY;
        kv[u][j] = valid[j] ? f32_key(v[u][j]) : INT_MIN;   // below every score's key
        if (valid[j] && !__builtin_isfinite(v[u][j])) fin = false;
      }
      const float nq = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, snq[t])));
      eb[u] = ceb * nq * mmax + 1e-30f;
      all_exact[u] = __ballot(!fin) != 0 || !__builtin_isfinite(eb[u]);
      vn[u] = vn1[u] = 0.f;
      // tokens past the block's end, short lists and the exact fallback need no rounds
      cnt[u] = (g0 + 4 * u >= ntok || ncand <= n || all_exact[u]) ? n + 1 : 0;
    }
    // v_n and v_n+1 of each token, counted with multiplicity (ncand > n finite scores, so
    // every round finds a value and a token is done within n + 1 rounds).  The rounds run
    // on integer keys of the scores (same order; -0 below +0, which leaves v_n and v_n+1
    // the same numbers), so the maxima need no NaN handling and end in scalar registers;
    // a round's maximum is taken out of the keys (set to the minimum) once counted.
    // (Everything here is uniform: no branches inside a round, and the four tokens'
    // reductions interleave.)
    int vnk[U], vn1k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vnk[u] = vn1k[u] = 0;
    for (int r = 0; r <= n && (cnt[0] <= n || cnt[1] <= n || cnt[2] <= n || cnt[3] <= n); ++r) {
      int mx[U];
#pragma unroll
      for (int u = 0; u < U; ++u) mx[u] = max(max(kv[u][0], kv[u][1]), max(kv[u][2], kv[u][3]));
      wave_max4_i32(mx);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int m = mx[u];
        const bool live = cnt[u] <= n;
        int ce = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool eq = kv[u][j] == m;
          ce += __builtin_popcountll(__builtin_amdgcn_ballot_w64(eq));
          kv[u][j] = eq && live ? INT_MIN : kv[u][j];
        }
        vnk[u] = (live && cnt[u] < n && cnt[u] + ce >= n) ? m : vnk[u];
        vn1k[u] = (live && cnt[u] + ce >= n + 1) ? m : vn1k[u];
        cnt[u] += live ? ce : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vn[u] = key_f32(vnk[u]);
      vn1[u] = key_f32(vn1k[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = g0 + 4 * u;
      if (t >= ntok) break;
      uint64_t chosen[4] = {0, 0, 0, 0};
      if (ncand <= n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) chosen[j] = __ballot(valid[j]);
      } else {
        const float hi = all_exact[u] ? INFINITY : vn1[u] + 2.f * eb[u];
        const float lo = all_exact[u] ? -INFINITY : vn[u] - 2.f * eb[u];
        bool amb[4];
        uint64_t ambm = 0;
        int k = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool in = valid[j] && v[u][j] > hi;
          amb[j] = valid[j] && !in && (all_exact[u] || v[u][j] >= lo);   // NaN scores: all exact
          chosen[j] = __ballot(in);
          k += __popcll(chosen[j]);
          ambm |= __ballot(amb[j]);
        }
        if (ambm != 0) {
          cold_path();
          // exact scores of the undecided candidates: a wavefront dot product each, the
          // token's query held as fp64 (E <= 1024: at most 16 values per lane)
          double qx[16];
          const __bf16* qt = qp + (size_t)t * a.E + lane;
#pragma unroll
          for (int x = 0; x < 16; ++x) qx[x] = lane + 64 * x < a.E ? (double)(float)qt[64 * x] : 0.0;
          double sx[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            for (uint64_t m = __ballot(amb[j]); m; m &= m - 1) {
              const int y = __builtin_ctzll(m);
              const double* mr = mean0 + (size_t)(y + 64 * j) * a.E + lane;
              double mv[16];
#pragma unroll
              for (int x = 0; x < 16; ++x) mv[x] = lane + 64 * x < a.E ? mr[64 * x] : 0.0;
              double d = 0.0;
#pragma unroll
              for (int x = 0; x < 16; ++x) d = fma(qx[x], mv[x], d);
              d = wave_sum_f64(d);
              if (lane == y) sx[j] = d;
            }
          }
          // the best n - k of them, one per round: highest score, then lowest index
          bool taken[4] = {false, false, false, false};
          for (int r = k; r < n; ++r) {
            double bs = -INFINITY;
            int bc = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (amb[j] && !taken[j] && (bc == 0x7fffffff || sx[j] > bs)) {
                bs = sx[j];
                bc = lane + 64 * j;
              }
            const double best = wave_max_f64(bs);
            const int win = wave_min_i32(bc != 0x7fffffff && bs == best ? bc : 0x7fffffff);
            if (win == 0x7fffffff) break;
            if ((win & 63) == lane) taken[win >> 6] = true;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) chosen[j] |= __ballot(taken[j]);
        }
      }
      // ascending candidate index (j-major, then lane), after the -1 padding
      int32_t* out = a.idx + ((size_t)b * a.S + t0 + t) * n;
      int nch = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) nch += __popcll(chosen[j]);
      const int pad = n - nch;
      int before = pad;
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((chosen[j] >> lane) & 1ull) out[before + __popcll(chosen[j] & below)] = lane + 64 * j;
        before += __popcll(chosen[j]);
      }
      if (lane < pad) out[lane] = -1;
    }
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
  if (a.mto > a.mfrom)
    hipLaunchKernelGGL(block_means_kernel, dim3((unsigned)(a.B * (a.mto - a.mfrom))), dim3(256), 0, stream, a);
  if (a.S == 0) return hipGetLastError();
  const int nqb = (a.q_pos0 + a.S - 1) / a.bs - a.q_pos0 / a.bs + 1;
  if (a.nblk <= kSelFastMax && a.nsplit == 1) {
    // all candidates of a query block fit the LDS score table: one workgroup per block.
    // (A grid of fewer than 256 query blocks -- decoding -- takes the split fp64 path
    // instead: a few workgroups scoring all candidates each wait on their loads longer
    // than the split's workgroups take to score their shares.)
    const dim3 grid((unsigned)(a.B * nqb));
    const size_t lds = sel_fast_lds(a.bs, a.E);
    switch (a.bs) {
      case 16: hipLaunchKernelGGL(block_select_bf16_kernel<16>, grid, dim3(256), lds, stream, a); break;
      case 32: hipLaunchKernelGGL(block_select_bf16_kernel<32>, grid, dim3(256), lds, stream, a); break;
      case 64: hipLaunchKernelGGL(block_select_bf16_kernel<64>, grid, dim3(256), lds, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
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
