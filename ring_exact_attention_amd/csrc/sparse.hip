// Attention over gathered candidates ("AnnAttention", faiss_block_attention).
//
// Every token t attends to a list of slots: a window of W keys ending at t (positions
// before 0 are zero vectors), then the bs rows of each of its top_n selected blocks
// (block index -1 reads token 0 for every row, as the page clamps negative item
// indices).  One softmax over all slots, no mask; logits are q . k / sqrt(E).
//
// gfx950 mapping: one wavefront per token, each lane owning 8 of the E = 512
// embedding values (16 bytes of every row, so a row load is one coalesced 1 KB
// access per wave).  Rows are taken 32 at a time: each lane keeps 32 partial dots and
// a butterfly reduce-scatter over the 64 lanes (halving the values at every exchange)
// leaves row r's full dot in lanes 2r and 2r+1 after 32 exchanges.  Logits go to LDS;
// the max / exp / sum run over LDS; a second pass accumulates p * v in fp32.
#include "common.h"
#include "launch.h"

namespace rea {

constexpr int kSpE = 512;            // joint embedding (8 bf16 per lane)
constexpr int kSpMaxSlots = 64 + 16 * 64;
constexpr int kSpWaves = 4;

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m); }

__global__ __launch_bounds__(256) void sparse_fwd_kernel(SparseArgs a) {
  __shared__ int spos[kSpWaves][kSpMaxSlots];
  __shared__ float sdot[kSpWaves][kSpMaxSlots];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long tok_raw = (long long)blockIdx.x * kSpWaves + wave;   // b * S + t
  const bool valid = tok_raw < (long long)a.B * a.S;                   // tail waves compute token 0
  const long long tok = valid ? tok_raw : 0;                          // and store nothing
  const int b = (int)(tok / a.S), t = (int)(tok % a.S);
  const int W = a.window, bs = a.sel_block, n = a.top_n;
  const int nslots = W + n * bs;

  // slot positions (-1 = zero padding)
  const int32_t* sel = a.sel + tok * n;
  for (int s = lane; s < nslots; s += 64) {
    int p;
    if (s < W) {
      p = t - W + 1 + s;
      if (p < 0) p = -1;
    } else {
      const int j = (s - W) / bs, r = (s - W) % bs;
      const int c = sel[j];
      p = c < 0 ? 0 : c * bs + r;
      if (p >= a.S) p = a.S - 1;        // indices are < S/bs by contract; keep reads in bounds
    }
    spos[wave][s] = p;
  }
  __syncthreads();

  const __bf16* kb = (const __bf16*)a.k + (size_t)b * a.S * kSpE + 8 * lane;
  const __bf16* vb = (const __bf16*)a.v + (size_t)b * a.S * kSpE + 8 * lane;
  const u32x4 qu = *(const u32x4*)((const __bf16*)a.q + (size_t)tok * kSpE + 8 * lane);
  float qf[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    qf[2 * w] = bf16_lo(qu[w]);
    qf[2 * w + 1] = bf16_hi(qu[w]);
  }

  // pass 1: dots of q with every slot row, 32 rows at a time
  for (int g = 0; g < nslots; g += 32) {
    float part[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int s = g + r;
      const int p = s < nslots ? spos[wave][s] : -1;
      float acc = 0.f;
      if (p >= 0) {
        const u32x4 ku = *(const u32x4*)(kb + (size_t)p * kSpE);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc = fmaf(qf[2 * w], bf16_lo(ku[w]), acc);
          acc = fmaf(qf[2 * w + 1], bf16_hi(ku[w]), acc);
        }
      }
      part[r] = acc;
    }
    // butterfly reduce-scatter: after the exchange at distance m (32, 16, 8, 4, 2)
    // each lane keeps the half of its values selected by its lane bit, summed with
    // the partner's; lane L ends with row L >> 1, then one more exchange at distance 1.
#pragma unroll
    for (int half = 16, m = 32; half >= 1; half >>= 1, m >>= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int r = 0; r < half; ++r) {
        const float keep = upper ? part[r + half] : part[r];
        const float send = upper ? part[r] : part[r + half];
        part[r] = keep + shfl_xor_f(send, m);
      }
    }
    const float dot = part[0] + shfl_xor_f(part[0], 1);
    const int s = g + (lane >> 1);
    if ((lane & 1) == 0 && s < nslots) sdot[wave][s] = dot;
  }
  __syncthreads();

  // softmax statistics over all slots
  float mx = -INFINITY;
  for (int s = lane; s < nslots; s += 64) mx = fmaxf(mx, sdot[wave][s]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, m));
  float sum = 0.f;
  for (int s = lane; s < nslots; s += 64) {
    const float p = fast_exp2((sdot[wave][s] - mx) * a.scale_log2);
    sdot[wave][s] = p;
    sum += p;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += shfl_xor_f(sum, m);
  __syncthreads();

  // pass 2: o = sum_s p_s v_s / sum
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int g = 0; g < nslots; g += 8) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int s = g + r;
      if (s < nslots) {
        const int p = spos[wave][s];
        if (p >= 0) {
          const float ps = sdot[wave][s];
          const u32x4 vu = *(const u32x4*)(vb + (size_t)p * kSpE);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o[2 * w] = fmaf(ps, bf16_lo(vu[w]), o[2 * w]);
            o[2 * w + 1] = fmaf(ps, bf16_hi(vu[w]), o[2 * w + 1]);
          }
        }
      }
    }
  }
  const float inv = 1.f / sum;
  u32x4 ou;
#pragma unroll
  for (int w = 0; w < 4; ++w) ou[w] = pack_bf16x2(o[2 * w] * inv, o[2 * w + 1] * inv);
  if (!valid) return;
  *(u32x4*)((__bf16*)a.o + (size_t)tok * kSpE + 8 * lane) = ou;
  if (lane == 0) {
    a.m[tok] = mx * a.scale;
    a.l[tok] = sum;
  }
}

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream) {
  const long long ntok = (long long)a.B * a.S;
  const unsigned blocks = (unsigned)((ntok + kSpWaves - 1) / kSpWaves);
  hipLaunchKernelGGL(sparse_fwd_kernel, dim3(blocks), dim3(64 * kSpWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rea
