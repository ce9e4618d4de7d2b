// Tile scheduling shared by the dense kernels: which key tiles a query tile visits
// (and in which order), which query tiles a key tile is visited by, and the mapping
// of workgroup ids to (batch, head, tile) that keeps GQA groups on one XCD.
#pragma once

#include "common.h"

namespace rea {

// Key tiles of width BN visited by a set of query rows whose visible keys lie in
// [jlo, jhi] (inclusive, already clipped to [0, Skv)).  Keys are cut into virtual
// ring blocks of kvb rows; the blocks are visited in ring order starting at block
// `diag` and descending modulo nvb (the key block a ring member holds at step idx is
// (rank - idx) mod N).  Inside a block, tiles start at the block start and step by BN;
// `kend` is the end of the tile's block, so a tile never reaches into the next block.
template <int BN>
struct KeyTileIter {
  int nvb, kvb, idx, diag;
  int jlo, jhi;
  int ts, e, bend;

  __device__ __forceinline__ void init(int nvb_, int kvb_, int diag_, int jlo_, int jhi_) {
    nvb = nvb_; kvb = kvb_; diag = diag_; idx = 0;
    jlo = jlo_; jhi = jhi_;
    ts = 0; e = 0; bend = 0;
  }
  __device__ __forceinline__ bool next_block() {
    while (idx < nvb) {
      int vb = diag - idx;
      if (vb < 0) vb += nvb;
      ++idx;
      const int b0 = vb * kvb, b1 = b0 + kvb;
      const int s = max(b0, jlo), en = min(b1, jhi + 1);
      if (s < en) {
        ts = b0 + ((s - b0) / BN) * BN;
        e = en;
        bend = b1;
        return true;
      }
    }
    return false;
  }
  __device__ __forceinline__ bool next(int& tile_start, int& kend) {
    if (ts >= e) {
      if (!next_block()) return false;
    }
    tile_start = ts;
    kend = min(ts + BN, bend);
    ts += BN;
    return true;
  }
};

// Query tiles of height BQ that see a set of keys whose visible rows lie in [ilo, ihi].
// Rows are cut into virtual blocks of qvb rows; blocks are visited starting at `diag`
// and ascending modulo nvb (in the ring's backward pass a key block and its gradient
// travel forward, meeting query block (j + idx) mod N at step idx).
template <int BQ>
struct QueryTileIter {
  int nvb, qvb, idx, diag;
  int ilo, ihi;
  int ts, e, bend;

  __device__ __forceinline__ void init(int nvb_, int qvb_, int diag_, int ilo_, int ihi_) {
    nvb = nvb_; qvb = qvb_; diag = diag_; idx = 0;
    ilo = ilo_; ihi = ihi_;
    ts = 0; e = 0; bend = 0;
  }
  __device__ __forceinline__ bool next_block() {
    while (idx < nvb) {
      int vb = diag + idx;
      if (vb >= nvb) vb -= nvb;
      ++idx;
      const int b0 = vb * qvb, b1 = b0 + qvb;
      const int s = max(b0, ilo), en = min(b1, ihi + 1);
      if (s < en) {
        ts = b0 + ((s - b0) / BQ) * BQ;
        e = en;
        bend = b1;
        return true;
      }
    }
    return false;
  }
  __device__ __forceinline__ bool next(int& tile_start, int& rend) {
    if (ts >= e) {
      if (!next_block()) return false;
    }
    tile_start = ts;
    rend = min(ts + BQ, bend);
    ts += BQ;
    return true;
  }
};

// Workgroup id -> (batch, q head, tile index).  Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8), each with its own L2.  When the (batch, kv head) groups
// divide evenly over the XCDs, all q heads of one group -- which read the same K/V --
// are placed on the same XCD.  `reverse` visits tiles from the last one down
// (longest-first when later query tiles see more keys).
__device__ __forceinline__ void map_task(int bid, int n_tiles, int B, int Hq, int Hkv, int G,
                                         int xcd_groups, bool reverse, int& b, int& hq, int& t) {
  if (xcd_groups > 0) {
    const int x = bid & 7, r = bid >> 3;
    const int per_t = xcd_groups * G;
    t = r / per_t;
    const int rem = r - t * per_t;
    const int gl = rem / G, hh = rem - gl * G;
    const int grp = x + 8 * gl;                 // b * Hkv + hkv
    b = grp / Hkv;
    hq = (grp - b * Hkv) * G + hh;
  } else {
    const int per_t = B * Hq;
    t = bid / per_t;
    const int rem = bid - t * per_t;
    b = rem / Hq;
    hq = rem - b * Hq;
  }
  if (reverse) t = n_tiles - 1 - t;
}

// Same for kernels that own one kv head (the dk/dv pass): id -> (batch, kv head, tile).
__device__ __forceinline__ void map_kv_task(int bid, int n_tiles, int B, int Hkv, int xcd_groups,
                                            bool reverse, int& b, int& hkv, int& t) {
  if (xcd_groups > 0) {
    const int x = bid & 7, r = bid >> 3;
    t = r / xcd_groups;
    const int gl = r - t * xcd_groups;
    const int grp = x + 8 * gl;
    b = grp / Hkv;
    hkv = grp - b * Hkv;
  } else {
    const int per_t = B * Hkv;
    t = bid / per_t;
    const int rem = bid - t * per_t;
    b = rem / Hkv;
    hkv = rem - b * Hkv;
  }
  if (reverse) t = n_tiles - 1 - t;
}

// LDS layouts of a row-major bf16 tile with D columns, chosen per access pattern so that
// no pattern has bank conflicts (64 banks x 4 bytes; measured on gfx950):
//   kRowRead:  rows read as 16-byte MFMA operands (16 lanes = 16 rows, same column) ->
//              pitch D + 8 elements (272 B at D = 128: 16 rows land on 16 distinct 16-byte
//              bank groups);
//   kTrRead:   rows read with ds_read_b64_tr_b16 (32 lanes = 4 rows x 64 bytes) -> pitch
//              D + 32 (320 B: 4 consecutive rows start 64 bytes apart modulo 256);
//   kBothRead: both patterns.  At D = 128, rows go in groups of four at a 320-byte pitch
//              and each group starts 16 bytes further round the banks (group pitch 1296 B),
//              which satisfies both conditions with offsets that stay linear in the row
//              for row steps that are multiples of 4.  Otherwise pitch D + 32.
// Row stores of 16-byte chunks (16 lanes per row) are conflict-free in all three.
enum TileKind { kRowRead = 0, kTrRead = 1, kBothRead = 2 };

template <int D, int KIND>
struct TileLayout {
  static constexpr bool kGrouped = (KIND == kBothRead && D == 128);
  static constexpr int PITCH = kGrouped ? 160 : (KIND == kRowRead ? D + 8 : D + 32);
  static constexpr int GROUP = kGrouped ? 4 * PITCH + 8 : 4 * PITCH;   // elements per 4 rows
  static constexpr int elems(int rows) { return (rows / 4) * GROUP; }  // rows % 4 == 0
  // element offset of (row, col); row steps that are multiples of 4 add (step / 4) * GROUP
  __device__ static __forceinline__ int idx(int row, int col) {
    return (row >> 2) * GROUP + (row & 3) * PITCH + col;
  }
  static constexpr int rows(int step) { return (step / 4) * GROUP; }   // step % 4 == 0
};

}  // namespace rea
