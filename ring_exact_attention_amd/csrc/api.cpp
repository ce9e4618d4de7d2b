// C-ABI entry points of libattn.so (declared in include/attn.h).
//
// Every argument is validated here, on the host, before anything is launched; a
// failed check returns a status code and leaves a thread-local message.  Nothing in
// this file allocates device memory: scratch comes in through the caller's workspace.
#include "attn.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
int ok() {
  g_err.clear();
  return ATTN_OK;
}

constexpr long long kMaxLen = 1LL << 28;    // rows per call
constexpr long long kMaxPos = 1LL << 27;    // |global position of row 0|
constexpr long long kMaxSlice = (1LL << 32) - 256;   // bytes of one batch element of a tensor
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

std::string fmt(const char* f, long long a, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

// A validated dense (or sparse) problem.
struct Problem {
  int dtype = 0, B = 0, Sq = 0, Skv = 0, Hq = 0, Hkv = 0, D = 0, Dv = 0, G = 1;
  int delta = 0, lo_off = -rea::kPosInf, hi_off = rea::kPosInf;
  float scale = 1.f;
  int kv_block = 1, n_vblocks = 0, q_vblock = 1, n_qvblocks = 0;
  bool carry_in = false, finalize = true;
  int has_sink = 0;
  const float* sink = nullptr;
  float* dsink = nullptr;
  const float* bias = nullptr;
  long long bias_stride[4] = {0, 0, 0, 0};
  bool bias_vec4 = false;
  const uint32_t* drop = nullptr;
  long long drop_stride[3] = {0, 0, 0};
  void* o_lo = nullptr;
};

static_assert(offsetof(attn_params, softmax_type) == ATTN_PARAMS_V1_SIZE,
              "a version-1 attn_params is the current one without its softmax fields");
static_assert(offsetof(attn_params, bias) == ATTN_PARAMS_V2_SIZE,
              "a version-2 attn_params is the current one without its bias fields");
static_assert(offsetof(attn_params, drop_mask) == ATTN_PARAMS_V3_SIZE,
              "a version-3 attn_params is the current one without its dropout fields");
static_assert(offsetof(attn_params, o_lo) == ATTN_PARAMS_V4_SIZE,
              "a version-4 (or 5) attn_params is the current one without o_lo");

// The caller's params in the current layout: an earlier version's struct reads with its
// missing fields zero (ATTN_SOFTMAX_VANILLA, no bias, no dropout, no o_lo).  Other sizes pass through for the
// size check.
// First field of every params struct: read with memcpy, since a caller's struct of an
// unknown or older version may be shorter than the current type.
uint32_t struct_size_of(const void* p) {
  uint32_t n = 0;
  memcpy(&n, p, sizeof n);
  return n;
}

// The size field is read with memcpy: an older caller's struct is shorter than
// attn_params, so no member of it is accessed through the current type.
const attn_params* current_layout(const attn_params* p, attn_params& tmp) {
  if (!p) return p;
  const uint32_t n = struct_size_of(p);
  if (n != ATTN_PARAMS_V1_SIZE && n != ATTN_PARAMS_V2_SIZE && n != ATTN_PARAMS_V3_SIZE &&
      n != ATTN_PARAMS_V4_SIZE)
    return p;
  memset(&tmp, 0, sizeof tmp);
  memcpy(&tmp, p, n);
  tmp.struct_size = sizeof(attn_params);
  return &tmp;
}

int check_dense(const attn_params* p, bool bwd, Problem& r) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (struct_size_of(p) != sizeof(attn_params))
    return fail(ATTN_ERR_INVALID_ARG, fmt("params->struct_size is %lld, this library expects %lld",
                                          (long long)struct_size_of(p), (long long)sizeof(attn_params)));
  if (p->dtype != ATTN_BF16 && p->dtype != ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, fmt("dtype %lld is not supported (ATTN_BF16 or ATTN_F32)", p->dtype));
  if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_kv < 0)
    return fail(ATTN_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_kv must be >= 0");
  if (p->seqlen_q > kMaxLen || p->seqlen_kv > kMaxLen)
    return fail(ATTN_ERR_UNSUPPORTED, fmt("sequence lengths above %lld are not supported", kMaxLen));
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "num_q_heads and num_kv_heads must be > 0");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(ATTN_ERR_INVALID_ARG, fmt("num_q_heads (%lld) must be a multiple of num_kv_heads (%lld)",
                                          p->num_q_heads, p->num_kv_heads));
  const int D = p->head_dim;
  if (p->head_dim_v < 0) return fail(ATTN_ERR_INVALID_ARG, "head_dim_v must be >= 0 (0 = head_dim)");
  const int Dv = p->head_dim_v > 0 ? p->head_dim_v : D;
  if (!rea::head_dims_supported(p->dtype == ATTN_BF16 ? 0 : 1, D, Dv))
    return fail(ATTN_ERR_UNSUPPORTED, fmt("head_dim %lld / head_dim_v %lld are not supported for this dtype "
                                          "(bf16: 32/32, 64/64, 128/128, 128/64; f32: 32/32, 64/64, 64/32)",
                                          D, Dv));
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_ERR_INVALID_ARG, "window_left and window_right must be >= -1 (-1 = unbounded)");
  if (p->causal && p->window_right > 0)
    return fail(ATTN_ERR_INVALID_ARG, "a causal mask accepts window_right of -1 or 0 only");
  if (p->q_pos0 < -kMaxPos || p->q_pos0 > kMaxPos || p->kv_pos0 < -kMaxPos || p->kv_pos0 > kMaxPos)
    return fail(ATTN_ERR_UNSUPPORTED, fmt("|q_pos0|, |kv_pos0| above %lld are not supported", kMaxPos));
  if (std::isinf(p->scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (p->query_chunk < 0 || p->key_chunk < 0 || p->kv_block < 0)
    return fail(ATTN_ERR_INVALID_ARG, "query_chunk, key_chunk and kv_block must be >= 0");
  if (p->query_chunk > 0 && p->seqlen_q % p->query_chunk != 0)
    return fail(ATTN_ERR_INVALID_ARG, fmt("query_chunk (%lld) must divide seqlen_q (%lld)",
                                          p->query_chunk, p->seqlen_q));
  if (p->key_chunk > 0 && p->seqlen_kv % p->key_chunk != 0)
    return fail(ATTN_ERR_INVALID_ARG, fmt("key_chunk (%lld) must divide seqlen_kv (%lld)",
                                          p->key_chunk, p->seqlen_kv));
  if (p->kv_block > 0 && p->seqlen_kv % p->kv_block != 0)
    return fail(ATTN_ERR_INVALID_ARG, fmt("kv_block (%lld) must divide seqlen_kv (%lld)",
                                          p->kv_block, p->seqlen_kv));
  if (p->softmax_type != ATTN_SOFTMAX_VANILLA && p->softmax_type != ATTN_SOFTMAX_OFF_BY_ONE &&
      p->softmax_type != ATTN_SOFTMAX_LEARNABLE)
    return fail(ATTN_ERR_INVALID_ARG, fmt("softmax_type %lld is not one of the ATTN_SOFTMAX_* values",
                                          p->softmax_type));
  if (p->softmax_type == ATTN_SOFTMAX_LEARNABLE && (!p->sink || ((uintptr_t)p->sink & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_SOFTMAX_LEARNABLE needs sink: [num_q_heads] fp32 on the device");
  if (p->dsink && ((uintptr_t)p->dsink & 3u)) return fail(ATTN_ERR_INVALID_ARG, "dsink must be 4-byte aligned");
  if (p->bias) {
    if ((uintptr_t)p->bias & 3u) return fail(ATTN_ERR_INVALID_ARG, "bias must be 4-byte aligned");
    for (int d = 0; d < 4; ++d)
      if (p->bias_stride[d] < 0 || p->bias_stride[d] > (1LL << 40))
        return fail(ATTN_ERR_INVALID_ARG, "bias_stride entries must be in [0, 2^40]");
  }
  if (p->drop_mask) {
    if ((uintptr_t)p->drop_mask & 3u) return fail(ATTN_ERR_INVALID_ARG, "drop_mask must be 4-byte aligned");
    for (int d = 0; d < 3; ++d)
      if (p->drop_stride[d] < 0 || p->drop_stride[d] > (1LL << 40))
        return fail(ATTN_ERR_INVALID_ARG, "drop_stride entries must be in [0, 2^40]");
  }
  if (p->o_lo) {
    if (p->dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "o_lo applies to bf16 tensors only (must be NULL)");
    if (!aligned16(p->o_lo)) return fail(ATTN_ERR_INVALID_ARG, "o_lo must be 16-byte aligned");
  }
  const uint32_t fwd_flags = ATTN_CARRY_IN | ATTN_NO_FINALIZE;
  const uint32_t bwd_flags = ATTN_BWD_SKIP_DQ | ATTN_BWD_SKIP_DKDV | ATTN_BWD_REUSE_STATS | ATTN_BWD_ACCUMULATE;
  if (p->flags & ~(fwd_flags | bwd_flags)) return fail(ATTN_ERR_INVALID_ARG, "unknown bits in flags");
  if (bwd && (p->flags & fwd_flags))
    return fail(ATTN_ERR_INVALID_ARG, "attn_bwd flags: only the ATTN_BWD_* flags apply");
  if (!bwd && (p->flags & bwd_flags))
    return fail(ATTN_ERR_INVALID_ARG, "attn_fwd flags: the ATTN_BWD_* flags do not apply");

  r.dtype = p->dtype;
  r.B = p->batch;
  r.Sq = p->seqlen_q;
  r.Skv = p->seqlen_kv;
  r.Hq = p->num_q_heads;
  r.Hkv = p->num_kv_heads;
  r.D = D;
  r.Dv = Dv;
  r.G = r.Hq / r.Hkv;
  r.delta = (int)(p->kv_pos0 - p->q_pos0);
  // A window wider than any distance between rows is the same as no window.
  const long long wl = p->window_left > kMaxLen * 2 ? -1 : p->window_left;
  const long long wr = p->window_right > kMaxLen * 2 ? -1 : p->window_right;
  r.lo_off = wl >= 0 ? -(int)wl : -rea::kPosInf;
  int hi = rea::kPosInf;
  if (p->causal) hi = 0;
  if (wr >= 0 && wr < hi) hi = (int)wr;
  r.hi_off = hi;
  r.scale = (p->scale > 0.f) ? p->scale : 1.f / std::sqrt((float)D);
  r.kv_block = p->kv_block > 0 ? p->kv_block : (r.Skv > 0 ? r.Skv : 1);
  r.n_vblocks = r.Skv / r.kv_block;
  r.q_vblock = (r.Sq > 0 && r.Sq % r.kv_block == 0) ? r.kv_block : (r.Sq > 0 ? r.Sq : 1);
  r.n_qvblocks = r.Sq / r.q_vblock;
  const long long esize = r.dtype == ATTN_BF16 ? 2 : 4;
  if ((long long)r.Sq * r.Hq * D * esize > kMaxSlice || (long long)r.Skv * r.Hkv * D * esize > kMaxSlice)
    return fail(ATTN_ERR_UNSUPPORTED, fmt("one batch element of q or k/v exceeds %lld bytes", kMaxSlice));
  // (head_dim_v <= head_dim for every supported pair, so o, dout and v are no larger.)
  r.carry_in = (p->flags & ATTN_CARRY_IN) != 0;
  r.finalize = (p->flags & ATTN_NO_FINALIZE) == 0;
  r.has_sink = p->softmax_type != ATTN_SOFTMAX_VANILLA;
  r.sink = p->softmax_type == ATTN_SOFTMAX_LEARNABLE ? p->sink : nullptr;
  r.dsink = p->softmax_type == ATTN_SOFTMAX_LEARNABLE ? p->dsink : nullptr;
  r.bias = p->bias;
  for (int d = 0; d < 4; ++d) r.bias_stride[d] = p->bias_stride[d];
  r.drop = p->drop_mask;
  for (int d = 0; d < 3; ++d) r.drop_stride[d] = p->drop_stride[d];
  r.o_lo = p->o_lo;
  // Rows of the bias read as 16-byte vectors by the bf16 kernels: unit key stride, every
  // row start 16-byte aligned, and key tiles that start at multiples of 4 keys.
  r.bias_vec4 = r.bias && r.bias_stride[3] == 1 && ((uintptr_t)r.bias & 15u) == 0 &&
                r.bias_stride[0] % 4 == 0 && r.bias_stride[1] % 4 == 0 && r.bias_stride[2] % 4 == 0 &&
                r.Skv % 4 == 0 && r.kv_block % 4 == 0;
  return ATTN_OK;
}

// Testing knob: with ATTN_REVERSE_WORKGROUPS=1 in the environment every kernel takes its
// grid's tasks in reverse order (results must not change; see wg_index in common.h).
int reverse_order() {
  const char* e = getenv("ATTN_REVERSE_WORKGROUPS");
  return e && e[0] == '1' ? 1 : 0;
}

int check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(ptr)) return fail(ATTN_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return ATTN_OK;
}

int xcd_groups(int B, int Hkv) { return ((long long)B * Hkv) % 8 == 0 ? (B * Hkv) / 8 : 0; }

// dk/dv workgroups per (key tile, kv head).  With a causal (or right-window) mask and no
// left window, the key tiles near the start of the sequence see many more query rows
// than those near the end; when there are few workgroups (B * Hkv * key tiles well under
// a few per CU), the longest ones set the kernel time.  Sharing a group's q heads out
// over ns workgroups (fp32 partials, summed by a small reduction) evens this out.
int dkdv_splits(const Problem& r) {
  if (r.dtype != ATTN_BF16 || r.G < 2) return 1;
  if (!(r.lo_off == -rea::kPosInf && r.hi_off < rea::kPosInf)) return 1;
  const int bk = rea::bwd_k_tile_rows(r.dtype);
  const long long wgs = (long long)((r.Skv + bk - 1) / bk) * r.B * r.Hkv;
  int ns = 1;
  while (ns < r.G && r.G % (2 * ns) == 0 && wgs * ns < 2048) ns *= 2;
  return ns;
}

int hip_status(hipError_t e) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, std::string("HIP error: ") + hipGetErrorString(e));
  return ok();
}

// Checks shared by the gathered block-sparse forward and backward (sel_idx != NULL).
int check_sparse(const attn_params* p) {
  if (struct_size_of(p) != sizeof(attn_params))
    return fail(ATTN_ERR_INVALID_ARG, "params->struct_size does not match this library");
  if (p->head_dim_v != 0 && p->head_dim_v != p->head_dim)
    return fail(ATTN_ERR_UNSUPPORTED, "sparse mode needs head_dim_v = 0 (the joint embedding)");
  if (p->softmax_type != ATTN_SOFTMAX_VANILLA)
    return fail(ATTN_ERR_UNSUPPORTED, "sparse mode has no sink softmax");
  if (p->bias) return fail(ATTN_ERR_UNSUPPORTED, "sparse mode has no bias");
  if (p->drop_mask) return fail(ATTN_ERR_UNSUPPORTED, "sparse mode has no dropout mask");
  if (p->o_lo) return fail(ATTN_ERR_UNSUPPORTED, "sparse mode has no o_lo (its backward forms D from fp32 probabilities)");
  if (p->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "sparse mode supports bf16 only");
  if (p->num_q_heads != 1 || p->num_kv_heads != 1)
    return fail(ATTN_ERR_INVALID_ARG, "sparse mode takes the joint embedding: num_q_heads = num_kv_heads = 1");
  if (p->head_dim != 512) return fail(ATTN_ERR_UNSUPPORTED, "sparse mode supports head_dim (embed) 512");
  if (p->batch < 0 || p->seqlen_q < 0 || p->q_pos0 < 0 || p->q_pos0 + p->seqlen_q > p->seqlen_kv)
    return fail(ATTN_ERR_INVALID_ARG, "sparse mode needs 0 <= q_pos0 and q_pos0 + seqlen_q <= seqlen_kv");
  if (p->seqlen_kv > kMaxLen || (long long)p->seqlen_kv * 512 * 2 > kMaxSlice)
    return fail(ATTN_ERR_UNSUPPORTED, "sequence too long");
  if (p->top_n < 1 || p->top_n > 16) return fail(ATTN_ERR_INVALID_ARG, "top_n must be in 1..16");
  if (p->sel_block != 16 && p->sel_block != 32 && p->sel_block != 64)
    return fail(ATTN_ERR_UNSUPPORTED, "sel_block must be 16, 32 or 64");
  if (p->sparse_window < 1 || p->sparse_window > 64)
    return fail(ATTN_ERR_INVALID_ARG, "sparse_window must be in 1..64");
  if (p->flags) return fail(ATTN_ERR_INVALID_ARG, "sparse mode takes no flags");
  if (std::isinf(p->scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  return ATTN_OK;
}

// Gathered block-sparse forward (sel_idx != NULL).
int sparse_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o, float* m,
               float* l, float* work, void* stream) {
  int st0 = check_sparse(p);
  if (st0) return st0;
  if (p->batch == 0 || p->seqlen_q == 0) return ok();
  int st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(m, "m")) || (st = check_ptr(l, "l")))
    return st;
  if (work && ((uintptr_t)work & (kAlign - 1)) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "the sparse forward's workspace (acc) must be 256-byte aligned");
  rea::SparseArgs a{};
  a.rev_order = reverse_order();
  a.part = work;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sel = p->sel_idx;
  a.o = o;
  a.m = m;
  a.l = l;
  a.B = p->batch;
  a.S = p->seqlen_q;
  a.Skv = p->seqlen_kv;
  a.q_pos0 = (int)p->q_pos0;
  a.E = p->head_dim;
  a.top_n = p->top_n;
  a.sel_block = p->sel_block;
  a.window = p->sparse_window;
  a.scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt((float)a.E);
  a.scale_log2 = a.scale * rea::kLog2e;
  return hip_status(rea::launch_sparse(a, (hipStream_t)stream));
}

// The two block masks of the sparse dk/dv kernel (which tokens list each block, and which
// of those with a code other than 1) take 2 * B * (S / 32) * ceil(S / 32) words; past
// kSparseMaskMax bytes, or past rea::kMaskMaxSel blocks (the LDS of the kernel that
// builds them), they are left out and that kernel scans every token's selections.
constexpr size_t kSparseMaskMax = (size_t)64 << 20;
size_t sparse_mask_bytes(const attn_params* p) {
  if (p->batch <= 0 || p->seqlen_q <= 0 || p->sel_block <= 0) return 0;
  const size_t S = (size_t)p->seqlen_q, nsel = S / (size_t)p->sel_block;
  if (nsel > (size_t)rea::kMaskMaxSel) return 0;
  const size_t bytes = 2 * (size_t)p->batch * nsel * ((S + 31) / 32) * sizeof(uint32_t);
  return bytes <= kSparseMaskMax ? bytes : 0;
}

size_t sparse_bwd_workspace(const attn_params* p) {
  const size_t n = (size_t)(p->batch > 0 ? p->batch : 0) * (p->seqlen_q > 0 ? p->seqlen_q : 0) * sizeof(float);
  const size_t mask = sparse_mask_bytes(p);
  return 2 * align_up(n > 0 ? n : 1) + (mask > 0 ? align_up(mask) : 0);
}

// Gradient of the gathered block-sparse attention (sel_idx != NULL).
int sparse_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* m, const float* l, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_sparse(p);
  if (st) return st;
  if (p->sel_block != 32)
    return fail(ATTN_ERR_UNSUPPORTED, "the sparse backward supports sel_block 32");
  if (p->seqlen_kv != p->seqlen_q || p->q_pos0 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "the sparse backward needs seqlen_q == seqlen_kv and q_pos0 == 0");
  if (p->batch == 0 || p->seqlen_q == 0) return ok();
  const size_t need = sparse_bwd_workspace(p);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                        (long long)(workspace ? workspace_bytes : 0)));
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(dout, "dout")) || (st = check_ptr(m, "m")) ||
      (st = check_ptr(l, "l")) || (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) ||
      (st = check_ptr(dv, "dv")))
    return st;
  rea::SparseBwdArgs a{};
  a.rev_order = reverse_order();
  a.q = q;
  a.k = k;
  a.v = v;
  a.sel = p->sel_idx;
  a.o = o;
  a.dout = dout;
  a.m = m;
  a.l = l;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t n = (size_t)p->batch * p->seqlen_q * sizeof(float);
  a.Dvec = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + align_up(n));
  a.lmask = sparse_mask_bytes(p) > 0 ? (uint32_t*)((char*)workspace + 2 * align_up(n)) : nullptr;
  a.nsel = p->seqlen_q / p->sel_block;
  a.nwords = (p->seqlen_q + 31) / 32;
  a.B = p->batch;
  a.S = p->seqlen_q;
  a.E = p->head_dim;
  a.top_n = p->top_n;
  a.sel_block = p->sel_block;
  a.window = p->sparse_window;
  a.scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt((float)a.E);
  a.scale_log2 = a.scale * rea::kLog2e;
  return hip_status(rea::launch_sparse_bwd(a, (hipStream_t)stream));
}

}  // namespace

namespace rea {
// Status reporting for entry points defined in other translation units.
int report_error(int code, const char* msg) { return fail(code, msg); }
}  // namespace rea

extern "C" {

const char* attn_last_error(void) { return g_err.c_str(); }

uint32_t attn_abi_version(void) { return ATTN_PARAMS_VERSION; }

int attn_fwd(const attn_params* p_in, const void* q, const void* k, const void* v, void* o, float* m,
             float* l, float* acc, void* stream) {
  attn_params tmp;
  const attn_params* p = current_layout(p_in, tmp);
  if (p && struct_size_of(p) == sizeof(attn_params) && p->sel_idx)
    return sparse_fwd(p, q, k, v, o, m, l, acc, stream);
  Problem r;
  int st = check_dense(p, false, r);
  if (st) return st;
  if (r.B == 0 || r.Sq == 0) return ok();
  if ((st = check_ptr(q, "q")) || (st = check_ptr(m, "m")) || (st = check_ptr(l, "l"))) return st;
  if (r.Skv > 0 && ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")))) return st;
  if (r.finalize && (st = check_ptr(o, "o"))) return st;
  if ((r.carry_in || !r.finalize) && (st = check_ptr(acc, "acc (needed by ATTN_CARRY_IN / ATTN_NO_FINALIZE)")))
    return st;
  rea::FwdArgs a{};
  a.rev_order = reverse_order();
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_lo = r.finalize ? r.o_lo : nullptr;
  a.m = m;
  a.l = l;
  a.acc = acc;
  a.B = r.B;
  a.Sq = r.Sq;
  a.Skv = r.Skv;
  a.Hq = r.Hq;
  a.Hkv = r.Hkv;
  a.G = r.G;
  a.D = r.D;
  a.Dv = r.Dv;
  a.has_sink = r.has_sink;
  a.sink = r.sink;
  a.bias = r.bias;
  a.bs_b = r.bias_stride[0];
  a.bs_h = r.bias_stride[1];
  a.bs_i = r.bias_stride[2];
  a.bs_j = r.bias_stride[3];
  a.bias_vec4 = r.bias_vec4 ? 1 : 0;
  a.drop = r.drop;
  a.ds_b = r.drop_stride[0];
  a.ds_h = r.drop_stride[1];
  a.ds_i = r.drop_stride[2];
  a.inv_scale = 1.f / r.scale;
  a.delta = r.delta;
  a.lo_off = r.lo_off;
  a.hi_off = r.hi_off;
  a.scale = r.scale;
  a.scale_log2 = r.scale * rea::kLog2e;
  a.kv_block = r.kv_block;
  a.n_vblocks = r.n_vblocks;
  a.carry_in = r.carry_in;
  a.finalize = r.finalize;
  const int bm = rea::fwd_tile_rows(r.dtype);
  a.n_qtiles = (r.Sq + bm - 1) / bm;
  a.xcd_groups = r.dtype == ATTN_BF16 ? xcd_groups(r.B, r.Hkv) : 0;
  if ((long long)a.n_qtiles * r.B * r.Hq >= (1LL << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  return hip_status(rea::launch_fwd(r.dtype, a, (hipStream_t)stream));
}

size_t attn_fwd_workspace_bytes(const attn_params* p_in) {
  attn_params tmp;
  const attn_params* p = current_layout(p_in, tmp);
  if (!p || struct_size_of(p) != sizeof(attn_params) || !p->sel_idx) return 0;
  const std::string saved = g_err;
  if (check_sparse(p) != ATTN_OK) return 0;
  g_err = saved;
  int tpw = 0, ks = 1;
  rea::sparse_plan(p->batch, p->seqlen_q, p->sparse_window, p->sel_block, p->top_n, true, tpw, ks);
  if (ks <= 1) return 0;
  return align_up((size_t)p->batch * p->seqlen_q * ks * (512 + 4) * sizeof(float));
}

size_t attn_bwd_workspace_bytes(const attn_params* p_in) {
  attn_params tmp;
  const attn_params* p = current_layout(p_in, tmp);
  if (p && struct_size_of(p) == sizeof(attn_params) && p->sel_idx) {
    const std::string saved = g_err;
    if (struct_size_of(p) != sizeof(attn_params) || check_sparse(p) != ATTN_OK) return 0;
    g_err = saved;
    return sparse_bwd_workspace(p);
  }
  Problem r;
  const std::string saved = g_err;
  if (!p || check_dense(p, true, r) != ATTN_OK) return 0;
  g_err = saved;
  const size_t n = (size_t)r.B * r.Hq * r.Sq * sizeof(float);
  const int ns = dkdv_splits(r);
  const size_t part = ns > 1 ? (size_t)ns * r.B * r.Skv * r.Hkv * (r.D + r.Dv) * sizeof(float) : 0;
  return 2 * align_up(n > 0 ? n : 1) + (part ? align_up(part) : 0);
}

int attn_bwd(const attn_params* p_in, const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* m, const float* l, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
  attn_params tmp;
  const attn_params* p = current_layout(p_in, tmp);
  if (p && struct_size_of(p) == sizeof(attn_params) && p->sel_idx)
    return sparse_bwd(p, q, k, v, o, dout, m, l, dq, dk, dv, workspace, workspace_bytes, stream);
  Problem r;
  int st = check_dense(p, true, r);
  if (st) return st;
  if (r.B == 0 || (r.Sq == 0 && r.Skv == 0)) return ok();
  const size_t need = attn_bwd_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                        (long long)(workspace ? workspace_bytes : 0)));
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const bool do_pre = !(p->flags & ATTN_BWD_REUSE_STATS);
  const bool do_dq = !(p->flags & ATTN_BWD_SKIP_DQ);
  const bool do_dkdv = !(p->flags & ATTN_BWD_SKIP_DKDV);
  if (r.Sq > 0 && ((st = check_ptr(q, "q")) || (st = check_ptr(dout, "dout"))))
    return st;
  if (r.Sq > 0 && do_pre && ((st = check_ptr(o, "o")) || (st = check_ptr(m, "m")) || (st = check_ptr(l, "l"))))
    return st;
  if (r.Sq > 0 && do_dq && (st = check_ptr(dq, "dq"))) return st;
  if (r.Skv > 0 && ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")))) return st;
  if (r.Skv > 0 && do_dkdv && ((st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))) return st;
  rea::BwdArgs a{};
  a.rev_order = reverse_order();
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_lo = r.o_lo;
  a.dout = dout;
  a.m = m;
  a.l = l;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t n = (size_t)r.B * r.Hq * r.Sq * sizeof(float);
  a.Dvec = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + align_up(n > 0 ? n : 1));
  a.B = r.B;
  a.Sq = r.Sq;
  a.Skv = r.Skv;
  a.Hq = r.Hq;
  a.Hkv = r.Hkv;
  a.G = r.G;
  a.D = r.D;
  a.Dv = r.Dv;
  a.has_sink = r.has_sink;
  a.sink = r.sink;
  a.bias = r.bias;
  a.bs_b = r.bias_stride[0];
  a.bs_h = r.bias_stride[1];
  a.bs_i = r.bias_stride[2];
  a.bs_j = r.bias_stride[3];
  a.bias_vec4 = r.bias_vec4 ? 1 : 0;
  a.drop = r.drop;
  a.ds_b = r.drop_stride[0];
  a.ds_h = r.drop_stride[1];
  a.ds_i = r.drop_stride[2];
  a.inv_scale = 1.f / r.scale;
  a.delta = r.delta;
  a.lo_off = r.lo_off;
  a.hi_off = r.hi_off;
  a.scale = r.scale;
  a.scale_log2 = r.scale * rea::kLog2e;
  a.kv_block = r.kv_block;
  a.n_vblocks = r.n_vblocks;
  a.q_vblock = r.q_vblock;
  a.n_qvblocks = r.n_qvblocks;
  const int bq = rea::bwd_q_tile_rows(r.dtype), bk = rea::bwd_k_tile_rows(r.dtype);
  a.n_qtiles = (r.Sq + bq - 1) / bq;
  a.n_ktiles = (r.Skv + bk - 1) / bk;
  a.xcd_groups = r.dtype == ATTN_BF16 ? xcd_groups(r.B, r.Hkv) : 0;
  a.kv_splits = dkdv_splits(r);
  a.xcd_kv_groups = r.dtype == ATTN_BF16 ? xcd_groups(r.B, r.Hkv * a.kv_splits) : 0;
  a.dkv_part = a.kv_splits > 1 ? (float*)((char*)workspace + 2 * align_up(n > 0 ? n : 1)) : nullptr;
  a.stages = (do_pre ? 1 : 0) | (do_dq ? 2 : 0) | (do_dkdv ? 4 : 0);
  a.accumulate = (p->flags & ATTN_BWD_ACCUMULATE) ? 1 : 0;
  a.dsink = r.Sq > 0 ? r.dsink : nullptr;
  if ((long long)a.n_qtiles * r.B * r.Hq >= (1LL << 31)) return fail(ATTN_ERR_UNSUPPORTED, "problem too large");
  return hip_status(rea::launch_bwd(r.dtype, a, (hipStream_t)stream));
}

// The caller's select params in the current layout (version 1: seqlen_kv = seqlen,
// q_pos0 = 0).  Other sizes pass through for the size check.
const select_params* current_select_layout(const select_params* p, select_params& tmp) {
  if (!p) return p;
  if (struct_size_of(p) != SELECT_PARAMS_V1_SIZE) return p;
  memset(&tmp, 0, sizeof tmp);
  memcpy(&tmp, p, SELECT_PARAMS_V1_SIZE);
  tmp.struct_size = sizeof(select_params);
  return &tmp;
}

// Key rows of a select call (seqlen_kv, or seqlen when 0).
int select_kv_rows(const select_params* p) { return p->seqlen_kv > 0 ? p->seqlen_kv : p->seqlen; }

size_t block_select_workspace_bytes(const select_params* p_in) {
  select_params tmp;
  const select_params* p = current_select_layout(p_in, tmp);
  if (!p || struct_size_of(p) != sizeof(select_params) || p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 ||
      p->embed <= 0 || p->block_size <= 0)
    return 0;
  const size_t nblk = (size_t)(select_kv_rows(p) / p->block_size);
  const size_t n = (size_t)p->batch * nblk * p->embed * sizeof(double);
  // block means, their bf16 parts and norms, then (split selection) the partial top-n lists
  const size_t nb = (size_t)p->batch * nblk;
  const int ns = rea::select_splits(p->batch, p->seqlen, p->q_pos0, p->block_size, (int)nblk, p->top_n);
  const size_t parts = ns > 1 ? (size_t)p->batch * p->seqlen * ns * p->top_n : 0;
  const size_t ns3 = 2 * nb * p->embed * sizeof(uint16_t), nn = nb * sizeof(float);
  return align_up(n > 0 ? n : 1) + align_up(ns3 > 0 ? ns3 : 1) + align_up(nn > 0 ? nn : 1) +
         (parts ? align_up(parts * sizeof(double)) + align_up(parts * sizeof(int32_t)) : 0);
}

int block_select(const select_params* p_in, const void* q, const void* k, int32_t* idx, void* workspace,
                 size_t workspace_bytes, void* stream) {
  select_params tmp;
  const select_params* p = current_select_layout(p_in, tmp);
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (struct_size_of(p) != sizeof(select_params))
    return fail(ATTN_ERR_INVALID_ARG, "params->struct_size does not match this library");
  if (p->means_cached < 0 || (p->block_size > 0 && p->means_cached > select_kv_rows(p) / p->block_size))
    return fail(ATTN_ERR_INVALID_ARG, "params->means_cached must be in 0 .. seqlen_kv / block_size");
  if (p->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "block_select supports bf16 inputs");
  if (p->batch < 0 || p->seqlen < 0 || p->seqlen_kv < 0 || p->q_pos0 < 0)
    return fail(ATTN_ERR_INVALID_ARG, "batch, seqlen, seqlen_kv and q_pos0 must be >= 0");
  const int skv = select_kv_rows(p);
  if ((long long)p->q_pos0 + p->seqlen > skv)
    return fail(ATTN_ERR_INVALID_ARG, "q_pos0 + seqlen must not exceed seqlen_kv");
  if (skv > kMaxLen) return fail(ATTN_ERR_UNSUPPORTED, "sequence too long");
  if (p->embed <= 0 || p->embed % 64 != 0 || p->embed > 1024)
    return fail(ATTN_ERR_UNSUPPORTED, "embed must be a multiple of 64 up to 1024");
  if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return fail(ATTN_ERR_UNSUPPORTED, "block_size must be 16, 32 or 64");
  if ((long long)p->embed * p->block_size > 32768)
    return fail(ATTN_ERR_UNSUPPORTED, "embed * block_size above 32768 is not supported");
  if (p->top_n < 1 || p->top_n > 16) return fail(ATTN_ERR_INVALID_ARG, "top_n must be in 1..16");
  if (p->batch == 0 || p->seqlen == 0) return ok();
  int st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(idx, "idx"))) return st;
  const size_t need = block_select_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, fmt("workspace of %lld bytes needed, %lld given", (long long)need,
                                        (long long)(workspace ? workspace_bytes : 0)));
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  rea::SelectArgs a{};
  a.rev_order = reverse_order();
  a.q = q;
  a.k = k;
  a.idx = idx;
  a.means = (double*)workspace;
  a.B = p->batch;
  a.S = p->seqlen;
  a.Skv = skv;
  a.q_pos0 = p->q_pos0;
  a.E = p->embed;
  a.bs = p->block_size;
  a.top_n = p->top_n;
  a.nblk = skv / p->block_size;
  // Means needed: candidates of query block i are the blocks c < min(i, nblk), and the
  // last query block of the call is (q_pos0 + S - 1) / bs; the first means_cached are
  // already in the workspace.
  a.mto = std::min(a.nblk, (a.q_pos0 + a.S - 1) / a.bs);
  a.mfrom = std::min(p->means_cached, a.mto);
  a.nsplit = rea::select_splits(a.B, a.S, a.q_pos0, a.bs, a.nblk, a.top_n);
  {
    const size_t nm = (size_t)a.B * a.nblk * a.E * sizeof(double), nb = (size_t)a.B * a.nblk;
    char* w = (char*)workspace + align_up(nm > 0 ? nm : 1);
    const size_t ns3 = 2 * nb * a.E * sizeof(uint16_t), nn = nb * sizeof(float);
    a.msplit = (uint16_t*)w;
    w += align_up(ns3 > 0 ? ns3 : 1);
    a.mnorm = (float*)w;
    w += align_up(nn > 0 ? nn : 1);
    if (a.nsplit > 1) {
      const size_t parts = (size_t)a.B * a.S * a.nsplit * a.top_n;
      a.part_s = (double*)w;
      a.part_c = (int32_t*)((char*)a.part_s + align_up(parts * sizeof(double)));
    }
  }
  return hip_status(rea::launch_select(a, (hipStream_t)stream));
}

}  // extern "C"
