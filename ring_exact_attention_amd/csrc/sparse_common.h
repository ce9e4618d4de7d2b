// Shared pieces of the gathered block-sparse kernels ("AnnAttention",
// faiss_block_attention): the joint embedding, the 32-token work unit and the per-unit
// union of selected blocks.
#pragma once

#include "common.h"

namespace rea {

constexpr int kSpE = 512;            // joint embedding (8 bf16 per lane)
constexpr int kUQ = 32;              // tokens per workgroup
constexpr int kUDW = 128;            // embedding slice per wavefront
constexpr int kUPITCH = kUDW + 32;   // slice row pitch (elements): conflict-free tr reads
constexpr int kUMaxEnt = 512;        // 32 tokens x top_n (<= 16)

// Float offset of group g (four values) of lane `lane` in a wave's partial score tile
// (an f32x16 per lane) exchanged through LDS.  Consecutive lanes take consecutive
// 16-byte slots, so 16 lanes cover 256 contiguous bytes: no bank conflicts, where a
// lane-major layout (16 floats per lane) puts every fourth lane on the same banks.
__device__ __forceinline__ int part_off(int lane, int g) { return 4 * (64 * g + lane); }

// Workgroup barrier over LDS only: this wave's LDS operations complete, then s_barrier
// (the memory clobber keeps LDS accesses on their side of it).  __syncthreads also waits
// for every vector memory load in flight (its release fence covers the loads that write
// LDS), which in the walks below are the next step's gathers.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Unit index (b * n_per_seq + unit) of workgroup wg.  Workgroups are dispatched
// round-robin over the 8 XCDs (wg % 8), each with its own L2; with xcd_seq > 0 every XCD
// takes the units of one sequence (xcd_seq XCDs share a sequence, taking its units in
// turn), so the rows a unit gathers on an XCD all come from that sequence.
__device__ __forceinline__ int xcd_unit(int wg, int n_per_seq, int xcd_seq) {
  if (xcd_seq <= 0) return wg;
  const int x = wg & 7, r = wg >> 3;
  return (x / xcd_seq) * n_per_seq + r * xcd_seq + (x % xcd_seq);
}
// Token groups later in a sequence see more earlier blocks, so their unions are longer
// (S 8192, top 8: a few steps for the first group, ~176 for the last), and the walks that
// go through them in ascending order end on a tail of the longest ones.  This takes each
// sequence's units from the last one down.
__device__ __forceinline__ int longest_first(int u, int n_per_seq) {
  const int b = u / n_per_seq;
  return b * n_per_seq + (n_per_seq - 1 - (u - b * n_per_seq));
}
// XCDs per sequence for B sequences of n_per_seq units each (0 = plain order).
__host__ __device__ inline int xcd_per_seq(int B, long long n_per_seq) {
  return (B >= 1 && B <= 8 && 8 % B == 0 && n_per_seq % (8 / B) == 0) ? 8 / B : 0;
}
constexpr int kUSentinel = 0x7fffffff;

// The selections of tokens t0 .. min(t0 + 32, tend) - 1 of sequence b (S tokens): their
// (block, token) pairs are sorted by block in LDS, the distinct blocks go to
// ublk[0 .. nu) in ascending order (-1 first), and ucnt[u][t / 4] byte t % 4 counts how
// often token t0 + t lists block u.  scratch: 3 * kUMaxEnt ints of LDS.  Called by all
// 256 threads; returns nu.
__device__ __forceinline__ int build_union(const int32_t* sel, int S, int tend, int n, int b, int t0,
                                           int* scratch, uint32_t (*ucnt)[kUQ / 4], int* ublk, int* s_nu) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int ne = kUQ * n;
  // entries sorted: the group's tokens x n, rounded up to a power of two (>= 64)
  const int cnt = max(0, min(kUQ, tend - t0));
  int SZ = 64;
  while (SZ < cnt * n) SZ <<= 1;
  int* skey = scratch;
  int* stok = skey + kUMaxEnt;
  for (int k = tid; k < SZ; k += 256) {
    int key = kUSentinel, tok = 0;
    if (k < ne) {
      const int t = k / n, j = k % n;
      if (t0 + t < tend) {
        const int c = sel[((size_t)b * S + t0 + t) * n + j];
        key = c < 0 ? -1 : c;
        tok = t;
      }
    }
    skey[k] = key;
    stok[k] = tok;
  }
  __syncthreads();
  for (int size = 2; size <= SZ; size <<= 1) {                // bitonic sort by key
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int k = tid; k < SZ / 2; k += 256) {
        const int lo = 2 * k - (k & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int ka = skey[lo], kb = skey[hi];
        if ((ka > kb) == up) {
          skey[lo] = kb;
          skey[hi] = ka;
          const int ta = stok[lo];
          stok[lo] = stok[hi];
          stok[hi] = ta;
        }
      }
      __syncthreads();
    }
  }
  if (wave == 0) {                                             // union index of each entry
    int* suid = stok + kUMaxEnt;
    int running = 0;
    for (int c0 = 0; c0 < SZ; c0 += 64) {
      const int k = c0 + lane;
      const int key = skey[k];
      const bool first = key != kUSentinel && (k == 0 || skey[k - 1] != key);
      const uint64_t mask = __ballot(first);
      const int before = __popcll(mask & ((1ull << lane) - 1));
      suid[k] = running + before + (first ? 0 : -1);
      if (first) ublk[running + before] = key;
      running += __popcll(mask);
    }
    if (lane == 0) *s_nu = running;
  }
  for (int k = tid; k < SZ * (kUQ / 4); k += 256) ((uint32_t*)ucnt)[k] = 0u;
  __syncthreads();
  {
    const int* suid = stok + kUMaxEnt;
    for (int k = tid; k < SZ; k += 256)
      if (skey[k] != kUSentinel) atomicAdd(&ucnt[suid[k]][stok[k] >> 2], 1u << (8 * (stok[k] & 3)));
  }
  __syncthreads();
  return *s_nu;
}

}  // namespace rea
