// Shared device-side definitions for the gfx950 attention kernels.
//
// Everything here is plain HIP for CDNA4: 64-wide wavefronts, bf16 MFMA with fp32
// accumulation, LDS staging.  The kernel argument structs are filled by the host
// layer (api.cpp) after it has validated the C-ABI parameters.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace rea {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPosInf = 1 << 30;   // "unbounded" key offset (positions are validated < 2^29)

// Forward kernel arguments (dense path).
struct FwdArgs {
  int rev_order;      // nonzero: workgroups take the grid's tasks in reverse order (see wg_index)
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;         // NULL, or bf16 like o: the fp32 output's rounding residual
  float* m;
  float* l;
  float* acc;
  int B, Sq, Skv, Hq, Hkv, G, D;
  int Dv;             // head dim of v and o (may differ from D, the q/k head dim)
  int has_sink;       // softmax with a sink term exp(z_h) in each row's denominator
  const float* sink;  // [Hq] sink logits z_h (natural units); NULL with has_sink: z = 0
  // Additive logit bias (natural units) or NULL: element (b, hq, i, j) at
  // bias[b*bs_b + hq*bs_h + i*bs_i + j*bs_j] (a zero stride broadcasts).  It enters the
  // raw dot products as bias / scale.
  const float* bias;
  long long bs_b, bs_h, bs_i, bs_j;
  float inv_scale;
  int bias_vec4;      // rows readable as 16-byte vectors (unit key stride, aligned)
  // Dropout: pair (i, j) of (b, hq) dropped iff bit j % 32 of word
  // drop[b*ds_b + hq*ds_h + i*ds_i + j/32] is set; NULL = none.
  const uint32_t* drop;
  long long ds_b, ds_h, ds_i;
  // Visibility of (row i, key j): lo_off <= (j - i) + delta <= hi_off, with
  // delta = kv_pos0 - q_pos0 and j < Skv.
  int delta;
  int lo_off;
  int hi_off;
  float scale;        // natural-units logit scale
  float scale_log2;   // scale * log2(e)
  int kv_block;       // rows per virtual ring block (>= 1)
  int n_vblocks;      // Skv / kv_block
  int carry_in;
  int finalize;
  int n_qtiles;       // ceil(Sq / BM)
  int xcd_groups;     // (B*Hkv) / 8 when the XCD-aware order applies, else 0
  // bf16 workgroup shape (set by the launcher): gh q heads of one GQA group x
  // rows_wg query rows, gh * rows_wg = 256; n_hg = Hq / gh head groups.
  int gh, gh_shift, rows_wg, n_hg;
};

// Backward kernel arguments (dense path).
struct BwdArgs {
  int rev_order;      // nonzero: workgroups take the grid's tasks in reverse order (see wg_index)
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;   // NULL, or o's low part (bf16 like o): D_i uses o + o_lo
  const void* dout;
  const float* m;
  const float* l;
  void* dq;
  void* dk;
  void* dv;
  float* Dvec;        // [B, Hq, Sq] workspace: rowsum(dO * o)
  float* lse2;        // [B, Hq, Sq] workspace: m*log2(e) + log2(l)  (log2 units)
  int B, Sq, Skv, Hq, Hkv, G, D;
  int Dv;             // head dim of v, o, dout, dv
  int has_sink;       // as in FwdArgs: the LSE includes exp(z_h)
  const float* sink;  // [Hq] or NULL (z = 0)
  float* dsink;       // [Hq] output dL/dz_h (learnable sink), or NULL
  const float* bias;  // as in FwdArgs
  long long bs_b, bs_h, bs_i, bs_j;
  float inv_scale;
  int bias_vec4;
  const uint32_t* drop;  // as in FwdArgs
  long long ds_b, ds_h, ds_i;
  int delta, lo_off, hi_off;
  float scale, scale_log2;
  int kv_block, n_vblocks;     // virtual key blocks (ring order of the dq pass)
  int q_vblock, n_qvblocks;    // virtual query blocks (ring order of the dk/dv pass)
  int n_qtiles, n_ktiles;      // grid sizes: query tiles (dq), key tiles (dk/dv)
  int xcd_groups;              // (B*Hkv)/8 for the XCD-aware dq order, else 0
  int xcd_kv_groups;           // same for the dk/dv grid (over B * Hkv * kv_splits)
  int kv_splits;               // dk/dv workgroups per (key tile, kv head), each taking
                               // G / kv_splits q heads (bf16 only; 1 = no split)
  float* dkv_part;             // kv_splits > 1: fp32 partials [ns,B,Skv,Hkv,D] ++ [ns,B,Skv,Hkv,Dv]
  int stages;                  // bit 0: D/LSE pre-pass, bit 1: dq, bit 2: dk/dv
  int accumulate;              // dq, dk, dv (and dsink) are fp32 and this call adds into them
  // bf16 dq workgroup shape (set by the launcher), as in FwdArgs; fused_stats: the dq
  // kernel computes D and the LSE itself (and stores them for the dk/dv pass).
  int gh, gh_shift, rows_wg, n_hg, fused_stats;
};

struct SelectArgs {
  int rev_order;      // nonzero: workgroups take the grid's tasks in reverse order (see wg_index)
  const void* q;
  const void* k;
  int32_t* idx;
  double* means;      // [B, nblk, E] workspace
  int B, S, E, bs, top_n, nblk;   // S: query rows; nblk = Skv / bs full key blocks
  int Skv, q_pos0;    // key rows; position of query row 0 in the key sequence
  int nsplit;         // workgroups per query block, each over a share of the candidates
  double* part_s;     // nsplit > 1: [B, S, nsplit, top_n] partial lists (score, index;
  int32_t* part_c;    //   index -1 = empty), combined by block_select_merge_kernel
  uint16_t* msplit;   // [2, B, nblk, E] the means as sums of two bf16 parts (hi, lo)
  float* mnorm;       // [B, nblk] Euclidean norm of each mean, rounded up
  int mfrom, mto;     // blocks whose means this call computes: [mfrom, mto)
};

struct SparseArgs {
  int rev_order;      // nonzero: workgroups take the grid's tasks in reverse order (see wg_index)
  const void* q;
  const void* k;
  const void* v;
  const int32_t* sel;
  void* o;
  float* m;
  float* l;
  int B, S, E, top_n, sel_block, window;
  float scale_log2, scale;
  int Skv, q_pos0;    // key / value rows; position of query row 0 among them
  int tpw;            // tokens per workgroup (power of two <= 32; set by the launcher)
  int ksplit;         // workgroups per token group, each over a share of its 32-row steps
  int xcd_seq;        // > 0: XCDs per sequence of the XCD-aware group order (set by the launcher)
  float* part;        // ksplit > 1: [B, S, ksplit, 512 + 4] partial numerator, max, sum, pad
};

// Most selectable blocks (S / sel_block) for which the sparse backward builds its block
// masks (the building kernel holds 2 x 8 x that many words of LDS).
constexpr int kMaskMaxSel = 1024;

// Backward of the gathered block-sparse attention.
struct SparseBwdArgs {
  int rev_order;      // nonzero: workgroups take the grid's tasks in reverse order (see wg_index)
  const void* q;
  const void* k;
  const void* v;
  const int32_t* sel;
  const void* o;
  const void* dout;
  const float* m;
  const float* l;
  void* dq;
  void* dk;
  void* dv;
  float* Dvec;        // [B, S] workspace: rowsum(dO * o)
  float* lse2;        // [B, S] workspace: m*log2(e) + log2(l)
  // 2 x [B, nsel, nwords] workspace (or null): in the first plane, bit t % 32 of word
  // (b, c, t / 32) is set when token t lists block c (a -1 entry counts for block 0); in
  // the second, when its code for c (count | count of -1 entries << 8) is not 1.
  // nsel = S / sel_block, nwords = ceil(S / 32)
  uint32_t* lmask;
  int nsel, nwords;
  int B, S, E, top_n, sel_block, window;
  float scale_log2, scale;
};

// ---------------------------------------------------------------- device helpers

// Task index of this workgroup: its id in dispatch order, or (rev != 0) counted from the
// end of the grid.  No workgroup depends on another's progress or on the order of their
// writes, so a launch with the order reversed must give bitwise the same results; tests
// run both (the host sets rev from the ATTN_REVERSE_WORKGROUPS environment variable).
__device__ __forceinline__ int wg_index(int rev) {
  return rev ? (int)(gridDim.x - 1u - blockIdx.x) : (int)blockIdx.x;
}

// Sum of x over each aligned group of N lanes (N = 2, 4, 8 or 16), in every lane of the
// group: DPP quad swaps, then the half-row and row mirrors (VALU only; a shuffle goes
// through an LDS permute).
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "groups of 2 to 16 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  if constexpr (N >= 4) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  if constexpr (N >= 16) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// A compile-time int passed to a generic lambda (e.g. the buffer of an unrolled step).
template <int V>
struct IntConst {
  static constexpr int value = V;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw additive bias (without the 1/scale factor) for the 16 score registers of one lane
// of a 32x32 MFMA tile: register r holds index x = first + 8(r>>2) + (r&3) along the
// register dimension (keys in the forward and dq kernels, query rows in dk/dv); p points
// at the bias of the lane's own row (or key), st is the stride along x.  An x beyond
// `last` reads element `safe` instead (an in-range index; the caller masks those scores),
// so the loads carry no branches and are waited for together where d is first used.
// vec4 (st == 1, p 16-byte aligned, first and safe multiples of 4 and every in-range
// group of 4 whole): four 16-byte loads instead of 16 scalar ones.
__device__ __forceinline__ void bias_fetch16(f32x16& d, const float* p, long long st, int first, int last,
                                             int safe, bool vec4) {
  if (vec4) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int x0 = first + 8 * g;
      const f32x4 v = *(const f32x4*)(p + (x0 <= last ? x0 : safe));
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * g + e] = v[e];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int x = first + 8 * (r >> 2) + (r & 3);
      d[r] = p[(long long)(x <= last ? x : safe) * st];
    }
  }
}

// Dropout words of a tile of 32(NR - 1) keys starting at key ts: the NR words of the
// query row (p, nw of them; words past the row are clamped -- their keys are masked
// anyway) that cover the tile, loaded ahead; drop_bits_tile() aligns them where they are used (so the
// loads are not waited for at once).
// A tile that starts on a 32-key boundary needs only the first NR - 1 words (ts is
// wave-uniform, so the last load is skipped for the whole wave).
template <int NR>
__device__ __forceinline__ void drop_fetch_tile(uint32_t (&dwr)[NR], const uint32_t* p, int nw, int ts) {
  const int k0 = ts >> 5;
#pragma unroll
  for (int i = 0; i < NR - 1; ++i) dwr[i] = p[min(k0 + i, nw - 1)];
  dwr[NR - 1] = (ts & 31) ? p[min(k0 + NR - 1, nw - 1)] : 0u;
}
// Register r of 32-key half mb of a lane holds key ts + 32mb + 8(r>>2) + 4lh + (r&3): bit
// 8(r>>2) + (r&3) of dwl[mb] set = dropped.
template <int NL>
__device__ __forceinline__ void drop_bits_tile(uint32_t (&dwl)[NL], const uint32_t (&dwr)[NL + 1], int ts, int lh) {
  const uint32_t sh = (uint32_t)ts & 31u;
#pragma unroll
  for (int i = 0; i < NL; ++i)                    // keys ts + 32i .. ts + 32i + 31
    dwl[i] = __builtin_amdgcn_alignbit(dwr[i + 1], dwr[i], sh) >> (4 * lh);
}
// x, or -inf where bit `bit` of w is set: the sign-extended bit selects the bits of -inf
// (a bitfield extract and a bitfield insert).
__device__ __forceinline__ float drop_if(float x, uint32_t w, int bit) {
  const int m = __builtin_amdgcn_sbfe((int)w, bit, 1);           // 0 or -1
  return __int_as_float((m & (int)0xff800000) | (~m & __float_as_int(x)));
}
__device__ __forceinline__ void drop_apply16(f32x16& s, uint32_t w) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = drop_if(s[r], w, 8 * (r >> 2) + (r & 3));
}
// Whether pair (row i, key j) is dropped (j < Skv, i < Sq).
__device__ __forceinline__ bool dropped(const uint32_t* drop, long long base, long long ds_i, int i, int j) {
  return (drop[base + (long long)i * ds_i + (j >> 5)] >> (j & 31)) & 1u;
}

// log2 of (l * 2^mm + 2^zz) for a row's key statistics (mm = m * log2 e, l relative to
// m) and a sink logit zz in log2 units, without overflow; +inf when the row sees no key.
__device__ __forceinline__ float lse2_with_sink(float mm, float l, float zz) {
  if (!(l > 0.f)) return INFINITY;
  const float M = fmaxf(mm, zz);
  return M + log2f(l * exp2f(mm - M) + exp2f(zz - M));
}

// Value held by the lane in the other half of the wavefront (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const bool lo = (threadIdx.x & 63) < 32;
  return __uint_as_float(lo ? r[1] : r[0]);
}

// Two floats -> two bf16 (round to nearest even) packed in one dword; a single
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2v p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Marks a rarely taken branch: an opaque statement cannot be speculated, so the
// compiler keeps the branch instead of computing its body unconditionally.
__device__ __forceinline__ void cold_path() { asm volatile(""); }

// Index of this thread's wavefront in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Raw buffer resource over `bytes` bytes at `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Resource for the bytes [start, total) of a region: offsets used with it are relative
// to `start` and range-checked against the rest of the region.  All arguments must be
// the same on every lane; they are moved to scalar registers explicitly, since a
// resource the compiler cannot prove uniform makes it loop over lanes at every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_at(const void* base, uint32_t total,
                                                               uint32_t start) {
  const uint64_t addr = (uint64_t)(uintptr_t)base + start;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(total > start ? total - start : 0u);
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
}

// Direct global -> LDS copy (gfx950 buffer_load_dwordx4 ... lds): each active lane
// reads 16 bytes at voff and writes them to lds + 16 * lane.  `lds` must be the same on
// every lane.  Completion is tracked by vmcnt (wait_vmcnt0 before the data is read).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0,
                                           0, 0);
}
// s_waitcnt vmcnt(0), leaving the other counters alone.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16-byte load at base + voffset + soffset (bytes); zero when voffset is out of range.
// The range check covers voffset only, so callers keep soffset at zero and move a tile's
// start into the resource (make_rsrc_at).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j points at 4 consecutive
// 16-bit values (row j of a 16 x 4 block); lane i receives column i % 4 of rows
// i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.
typedef short short4v __attribute__((ext_vector_type(4)));
// The pointer is cast to the LDS address space directly (not through an integer), so
// the compiler still sees which LDS array it reads: it then does not hold the read
// behind copies in flight into other arrays.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  typedef __attribute__((address_space(3))) short4v lds_s4;
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ bf16x8 join_bf16x8(u32x2 lo, u32x2 hi) {
  const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(u);
}

// Clamp an int64 to the int32 range used for key offsets.
__host__ __device__ inline int clamp_i32(long long x) {
  return x > kPosInf ? kPosInf : (x < -kPosInf ? -kPosInf : (int)x);
}

}  // namespace rea
