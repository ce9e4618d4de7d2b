/*
 * attn.h -- C ABI of libattn.so: blockwise exact softmax attention for gfx950 (MI355X).
 *
 * The operation (sources are web pages, cited by title and section):
 *   * "bpt.py" (llm_large_context): ring attention over blockwise attention.  Query
 *     and key chunks are scored, masked with global chunk offsets, and folded into a
 *     carried running max / numerator / denominator (``_blockwise_attention_fwd``,
 *     ``_ring_attention_fwd``); the backward pass recomputes the probabilities from the
 *     saved max and denominator (``_blockwise_attention_bwd``, ``_ring_attention_bwd``).
 *   * "JAX: Single-GPU Attention with TransformerEngine", section 1: BSHD layout, grouped
 *     query heads (q head h reads kv head h / (Hq/Hkv)), and the causal sliding-window
 *     mask ``_make_causal_swa_mask``; "Other attention knobs": ``scale_factor``.
 *   * "AnnAttention" (StudyExchange), "Core code": per-token top-n selection of earlier
 *     key blocks by their mean (``select_block``) and attention over the gathered
 *     window ++ selected blocks (``faiss_block_attention``).
 *
 * Conventions shared by every entry point:
 *   * All tensor arguments are DEVICE pointers (memory of the current HIP device),
 *     dense and row-major, allocated and owned by the caller.  The library allocates
 *     no device memory and keeps no pointer after a call returns.
 *   * BSHD layout: q, dq are [B, Sq, Hq, D]; k, dk are [B, Skv, Hkv, D]; v, dv are
 *     [B, Skv, Hkv, Dv]; o, dout are [B, Sq, Hq, Dv], with Dv = head_dim_v (= D unless
 *     set).  Statistics m, l are fp32 [B, Hq, Sq].  The carry ``acc`` is fp32
 *     [B, Sq, Hq, Dv].
 *   * ``stream`` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; nothing is synchronised.  Buffers must stay alive until the
 *     stream work completes.
 *   * Arguments are checked on the host before anything is launched.  A failed check
 *     returns ATTN_ERR_INVALID_ARG / ATTN_ERR_UNSUPPORTED / ATTN_ERR_WORKSPACE and
 *     launches nothing; a failed launch returns ATTN_ERR_HIP.  attn_last_error() then
 *     describes the problem.  A batch of 0 (or Sq = 0) is a successful no-op.
 *   * One batch element's slice of any tensor (S x H x D elements) must stay under
 *     4 GiB: the kernels address each slice with 32-bit byte offsets.  Larger slices
 *     return ATTN_ERR_UNSUPPORTED.
 *   * Testing knob: with ATTN_REVERSE_WORKGROUPS=1 in the environment (read at every
 *     call), every kernel takes the tasks of its grid in reverse order.  Results are
 *     bitwise the same: no workgroup depends on another's progress or write order.
 */
#ifndef RING_EXACT_ATTENTION_ATTN_H_
#define RING_EXACT_ATTENTION_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,   /* malformed arguments (NULL pointer, bad size, ...) */
  ATTN_ERR_UNSUPPORTED = -2,   /* well-formed but not built (head_dim, dtype, ...)  */
  ATTN_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than required           */
  ATTN_ERR_HIP = -4            /* the HIP runtime reported an error                  */
} attn_status;

typedef enum {
  ATTN_BF16 = 0,               /* q, k, v, o, dout, dq, dk, dv are bfloat16 */
  ATTN_F32 = 1                 /* ... are float32                           */
} attn_dtype;

/* attn_params.flags */
enum {
  /* Read m, l, acc as the incoming carry instead of starting from
   * m = -inf, l = 0, acc = 0 (one ring step resumes where the previous one stopped;
   * "bpt.py", ``_ring_attention_fwd`` threads (max, numerator, denominator) through
   * its scan). */
  ATTN_CARRY_IN = 1u,
  /* Leave the carry unnormalised in m, l, acc and do not write o (a ring step that is
   * not the last one). */
  ATTN_NO_FINALIZE = 2u,
  /* attn_bwd only: compute part of the backward pass.  dq is owned by the query
   * block and dk/dv by the key block ("bpt.py", _ring_attention_bwd keeps dq local
   * and passes dk, dv along the ring), so an owner may want only its share. */
  ATTN_BWD_SKIP_DQ = 8u,       /* do not compute dq (dq may be NULL)                  */
  ATTN_BWD_SKIP_DKDV = 16u,    /* do not compute dk, dv (both may be NULL)            */
  ATTN_BWD_REUSE_STATS = 32u,  /* the workspace already holds D and the log-sum-exp
                                  written by an earlier attn_bwd call with the same
                                  params, o, dout, m and l: do not recompute them     */
  /* attn_bwd only: dq, dk, dv are fp32 buffers (same shapes, whatever the element type of
   * q) and this call adds its gradients into them, as does dsink.  One ring step of the
   * backward pass ("bpt.py", _ring_attention_bwd carries fp32 dq, dk, dv through its scan:
   * dq stays with the query block while dk, dv travel with the key block and gather the
   * contributions of every query block they meet): call attn_bwd once per (query block,
   * key block) pair with that pair's q_pos0 / kv_pos0, adding into the query block's dq and
   * the key block's dk, dv. */
  ATTN_BWD_ACCUMULATE = 64u
};

/* attn_params.softmax_type ("JAX: Single-GPU Attention with TransformerEngine", "Other
 * attention knobs": softmax_type "off_by_one" or "learnable").  A sink adds exp(z_h) to
 * the denominator of every row's softmax of q head h and nothing to its numerator (as
 * one more key with logit z_h, in the units of the scaled logits, and a zero value):
 *   o_i = sum_j exp(s_ij) v_j / (exp(z_h) + sum_j exp(s_ij)).
 * OFF_BY_ONE is z_h = 0 (the "1 + sum" softmax); LEARNABLE reads z_h from params.sink and
 * attn_bwd can return dL/dz_h.  m and l stay the statistics of the keys alone; the sink
 * enters only when the output is finalised, so carried ring steps are unchanged. */
enum {
  ATTN_SOFTMAX_VANILLA = 0,
  ATTN_SOFTMAX_OFF_BY_ONE = 1,
  ATTN_SOFTMAX_LEARNABLE = 2
};

/* 2: softmax_type, sink, dsink appended; 3: bias, bias_stride appended; 4: drop_mask,
 * drop_stride appended; 5: select_params.reserved became means_cached (0, the value it
 * had to hold, keeps the earlier behaviour); 6: o_lo appended.  Structs of the earlier
 * sizes are still accepted: the missing fields read as zero (ATTN_SOFTMAX_VANILLA, no
 * bias, no dropout, no o_lo). */
#define ATTN_PARAMS_VERSION 6u
#define ATTN_PARAMS_V1_SIZE 104u
#define ATTN_PARAMS_V2_SIZE 128u
#define ATTN_PARAMS_V3_SIZE 168u
#define ATTN_PARAMS_V4_SIZE 200u   /* versions 4 and 5 */

typedef struct attn_params {
  uint32_t struct_size;        /* = sizeof(attn_params); versioning of the ABI        */
  int32_t dtype;               /* attn_dtype                                           */
  int32_t batch;               /* B >= 0                                               */
  int32_t seqlen_q;            /* Sq >= 0 (rows of q in this call)                     */
  int32_t seqlen_kv;           /* Skv >= 0 (rows of k, v in this call)                 */
  int32_t num_q_heads;         /* Hq > 0                                               */
  int32_t num_kv_heads;        /* Hkv > 0, Hq % Hkv == 0 (GQA group G = Hq / Hkv)      */
  int32_t head_dim;            /* D: 32, 64 or 128 (dense); 512 (sparse mode)         */
  int64_t q_pos0;              /* global position of q row 0 (chunk index start times
                                  chunk size in "bpt.py")                              */
  int64_t kv_pos0;             /* global position of k/v row 0                         */
  int32_t causal;              /* 1: key position <= query position                    */
  int32_t window_left;         /* -1 = unbounded, else key >= query - left (inclusive) */
  int32_t window_right;        /* -1 = unbounded, else key <= query + right; with
                                  causal only -1 or 0 is accepted                      */
  float scale;                 /* logit scale; <= 0 selects 1/sqrt(head_dim)          */
  int32_t query_chunk;         /* 0 = Sq; otherwise must divide Sq                     */
  int32_t key_chunk;           /* 0 = Skv; otherwise must divide Skv                   */
  int32_t kv_block;            /* virtual ring block: 0 = Skv (one block); otherwise
                                  must divide Skv.  Key blocks are visited in ring
                                  order starting at the block holding the query tile's
                                  own position and descending (mod the block count).  */
  uint32_t flags;              /* attn_fwd: ATTN_CARRY_IN | ATTN_NO_FINALIZE;
                                  attn_bwd: ATTN_BWD_SKIP_DQ | ATTN_BWD_SKIP_DKDV |
                                  ATTN_BWD_REUSE_STATS | ATTN_BWD_ACCUMULATE            */
  /* Gathered block-sparse mode ("AnnAttention", faiss_block_attention): when sel_idx
   * is non-NULL, attn_fwd attends each token to a zero-padded window of
   * sparse_window keys ending at the token, followed by the sel_block rows of each of
   * its top_n selected blocks (an index of -1 reads token 0 for every row), with one
   * softmax over all slots and no mask.  A block whose rows run past the end of the
   * key sequence is outside the operation (block_select never produces one, and the
   * page's gather is undefined for it); the kernels' range-checked reads then see zero
   * rows (logit 0, value 0, no gradient), nothing is read out of bounds and no error is
   * returned.  Requires bf16, Hq = Hkv = 1, head_dim = the
   * joint embedding (512), causal/window/flags/kv_block unused.  Query row r sits at
   * position q_pos0 + r of the Skv key / value rows (q_pos0 >= 0, q_pos0 + Sq <= Skv):
   * the whole sequence (Sq = Skv, q_pos0 = 0) or new tokens against a cache.  The
   * backward requires Sq = Skv and q_pos0 = 0.                                       */
  const int32_t* sel_idx;      /* [B, Sq, top_n] device, from block_select             */
  int32_t top_n;               /* 1..16                                                */
  int32_t sel_block;           /* rows per selected block (32)                         */
  int32_t sparse_window;       /* 1..64                                                */
  /* Head dim of v (and so of o, dout, dv and the carry acc) when it differs from the
   * q/k head dim: the DeepSeek-style MLA case of "JAX: Single-GPU Attention with
   * TransformerEngine", section 4 (q/k 128, v 64).  0 = head_dim.  Pairs built:
   * bf16 32/32, 64/64, 128/128, 128/64; f32 32/32, 64/64, 64/32; others return
   * ATTN_ERR_UNSUPPORTED.  The default scale stays 1/sqrt(head_dim).  Sparse mode
   * requires 0.                                                                     */
  int32_t head_dim_v;
  int32_t softmax_type;        /* ATTN_SOFTMAX_*; sparse mode requires VANILLA          */
  const float* sink;           /* LEARNABLE: [Hq] fp32 device, sink logits z_h          */
  float* dsink;                /* attn_bwd with LEARNABLE: [Hq] fp32 device output
                                  dL/dz_h summed over the batch and this call's query
                                  rows, written by calls that compute dq (added into
                                  with ATTN_BWD_ACCUMULATE; it depends on the query
                                  rows only, so pass it on one call per query block);
                                  NULL = not wanted                                     */
  /* Additive logit bias ("bpt.py": ring_attention / blockwise_attn take a bias that
   * broadcasts to (batch, heads, q_len, kv_len) and is added to the scaled logits;
   * the page passes no gradient to it, and neither does attn_bwd).  fp32 device, in the
   * units of the scaled logits; element (b, hq, i, j) -- this call's query row i and
   * key row j -- is bias[b*s0 + hq*s1 + i*s2 + j*s3] with s = bias_stride (elements,
   * >= 0; 0 broadcasts that dimension).  -inf removes a pair like the mask.  NULL = none.
   * Dense mode only.  Gradient accuracy: with a bias, P and dS enter dv and dk as bf16
   * pairs (high part and rounded low part), since a bias can give a few keys most of the
   * attention of hundreds of (row, head) pairs; the bias backward's dk/dv kernel runs
   * two more matrix products per step for that.  Checked within the bf16 bound
   * 2e-2 + 2^-8 |ref|: key padding (0 / -inf), key-shared N(0,1) biases over random
   * shapes (with o_lo; at N(0,4) one GQA-16 shape leaves the bound on 3 dk elements by
   * 2 %), per-row / per-head / full biases, and a dense N(0,1) bias [1, 1, S, S] on a
   * causal S = 8192 ring of 16 heads.                                                    */
  const float* bias;
  int64_t bias_stride[4];
  /* Dropout ("bpt.py": _blockwise_attention_fwd / _bwd draw a Bernoulli(attn_pdrop) array
   * over (batch, heads, q_len, kv_len) that _chunk_attention_bias adds to the logits times
   * the dtype's most negative value): a dropped pair leaves the softmax like a masked one
   * and the others are not rescaled.  The caller draws the array and passes it packed:
   * pair (i, j) of (b, hq) -- this call's query row i and key row j -- is dropped iff
   * bit j % 32 of word drop_mask[b*d0 + hq*d1 + i*d2 + j/32] is set, d = drop_stride
   * (32-bit words, >= 0; 0 broadcasts that dimension).  The same array must be given to
   * attn_fwd and attn_bwd.  NULL = no dropout.  Dense mode only.                         */
  const uint32_t* drop_mask;
  int64_t drop_stride[3];
  /* Low part of the output ("bpt.py": the forward keeps the output from before its cast
   * to the input dtype as a residual, and the backward takes each row's dot product of
   * dout with that output, D_i).  bf16 [B, Sq, Hq, head_dim_v] device, 16-byte aligned,
   * laid out like o; caller-owned.  attn_fwd (bf16, dense, a call that finalises) writes
   * o_lo = bf16(o32 - o) beside o = bf16(o32), o32 being the fp32 output, so o + o_lo
   * holds o32 to about 16 bits.  attn_bwd forms D_i from o + o_lo.  NULL in attn_fwd:
   * not written; NULL in attn_bwd: D_i from o alone, which puts the output's bf16
   * rounding into dq and dk through D (past the bf16 bound by a few percent where a key
   * collects several hundred (row, head) pairs, e.g. a GQA group of 8 under a causal
   * window of 100).  Must be NULL for fp32 tensors and in sparse mode (whose backward
   * forms D_i from o, or from its fp32 probabilities where rows of -1 entries gather
   * the gradients of many slots).                                                      */
  void* o_lo;
} attn_params;

/* 2: seqlen_kv and q_pos0 appended (a version-1 struct of SELECT_PARAMS_V1_SIZE bytes
 * means seqlen_kv = seqlen, q_pos0 = 0). */
#define SELECT_PARAMS_V1_SIZE 32u

typedef struct select_params {
  uint32_t struct_size;        /* = sizeof(select_params)                              */
  int32_t dtype;               /* ATTN_BF16                                            */
  int32_t batch;               /* B >= 0                                               */
  int32_t seqlen;              /* Sq >= 0: query rows                                  */
  int32_t embed;               /* E = heads * head_dim, multiple of 64, <= 1024        */
  int32_t block_size;          /* 16, 32 or 64                                         */
  int32_t top_n;               /* 1..16                                                */
  /* Leading full key blocks whose means the workspace already holds from an earlier call
   * on the same key rows (same k pointer contents for those rows, batch, embed,
   * block_size and seqlen_kv), as the page's index keeps the means of completed blocks
   * across decoding steps: 0 <= means_cached <= seqlen_kv / block_size; those blocks'
   * means are not recomputed.  0 = compute every mean the call needs.  The caller owns
   * the promise: means of rows that changed since are used as they are.              */
  int32_t means_cached;
  /* Decoding ("AnnAttention" in inference mode: new tokens against the key cache).
   * Query row r sits at position q_pos0 + r of a key sequence of seqlen_kv rows;
   * 0 = seqlen (the whole sequence, q_pos0 = 0).  q_pos0 + seqlen <= seqlen_kv.      */
  int32_t seqlen_kv;
  int32_t q_pos0;              /* >= 0                                                 */
} select_params;

/*
 * attn_fwd -- exact softmax attention forward, one GPU's share of the ring.
 * ("bpt.py": _ring_attention_fwd / _blockwise_attention_fwd; masking as in
 * _chunk_attention_bias and the TransformerEngine page's _make_causal_swa_mask.)
 *
 *   s_ij = scale * q_i . k_j over visible pairs, where query row i sits at q_pos0 + i,
 *   key row j at kv_pos0 + j, and (i, j) is visible iff
 *   (causal => kpos <= qpos) and (right >= 0 => kpos <= qpos + right) and
 *   (left >= 0 => kpos >= qpos - left).
 *   Writes m_i = max_j s_ij (natural-log units), l_i = sum_j exp(s_ij - m_i), and
 *   o_i = sum_j exp(s_ij - m_i) v_j / l_i rounded to the element type.  A row with no
 *   visible key gets o = 0, m = -inf, l = 0.
 *
 *   q, k, v   [in]  element type per params->dtype, BSHD.
 *   o         [out] [B, Sq, Hq, D]; may be NULL only with ATTN_NO_FINALIZE.
 *   m, l      [in/out] fp32 [B, Hq, Sq]; inputs only with ATTN_CARRY_IN.
 *   acc       [in/out] fp32 [B, Sq, Hq, D] unnormalised numerator; required (and only
 *             used) with ATTN_CARRY_IN or ATTN_NO_FINALIZE, else may be NULL.
 *             With ATTN_NO_FINALIZE the stored (m, l, acc) satisfy
 *             acc_i = sum_j exp(s_ij - m_i) v_j over all blocks seen so far.
 * In sparse mode (sel_idx != NULL) m and l hold the max logit and the softmax sum
 * over the token's slots, and acc is NULL or the workspace of attn_fwd_workspace_bytes.
 */
int attn_fwd(const attn_params* params, const void* q, const void* k, const void* v,
             void* o, float* m, float* l, float* acc, void* stream);

/* Bytes of optional device workspace the sparse forward (params->sel_idx != NULL) can
 * use, passed as attn_fwd's acc argument (256-byte aligned, contents overwritten): with
 * it, a call with few tokens (decoding) shares each token group's 32-row steps out over
 * several workgroups and combines their partial results; acc = NULL runs without the
 * split.  0 when the call would not split, for dense params, and for invalid params. */
size_t attn_fwd_workspace_bytes(const attn_params* params);

/*
 * attn_bwd -- gradients of attn_fwd's output, recomputing the probabilities from the
 * saved statistics ("bpt.py": _blockwise_attention_bwd / _ring_attention_bwd):
 *   D_i = dO_i . o_i,  P_ij = exp(s_ij - m_i) / l_i,  dS_ij = P_ij (dO_i . v_j - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i,
 * with dk, dv summed over the q heads that share a kv head.
 *
 *   q, k, v, o, dout [in] as in attn_fwd (o = attn_fwd's output, dout = dL/do).
 *   m, l             [in] fp32 [B, Hq, Sq] written by attn_fwd.
 *   dq [out] [B, Sq, Hq, D]; dk, dv [out] [B, Skv, Hkv, D] (element type of q; fp32 and
 *                    added into with ATTN_BWD_ACCUMULATE).
 *   workspace        device scratch of at least attn_bwd_workspace_bytes(params)
 *                    bytes (256-byte aligned); its contents are overwritten.
 * flags: 0 or a combination of the ATTN_BWD_* flags.  The result is bitwise
 * reproducible run to run.
 *
 * Gathered block-sparse mode (params->sel_idx != NULL, the same params as the sparse
 * attn_fwd call, sel_block 32): the gradient of "AnnAttention"'s
 * faiss_block_attention.  Per token t with slots j (window ++ selected blocks),
 * dS_tj = P_tj (dO_t . v_j - D_t) and dq_t = scale sum_j dS_tj k_j; every slot that
 * reads a sequence row p passes scale dS_tj q_t to dk_p and P_tj dO_t to dv_p (the -1
 * clamp makes row 0 collect those slots; zero pads and rows past the end pass nothing).
 * q, k, v, o, dout, dq, dk, dv are bf16 [B, S, 512]; m, l fp32 [B, S] from the sparse
 * forward; flags must be 0.  The workspace holds D and the log-sum-exp per token and,
 * while they take at most 64 MiB and S / 32 <= 1024, two bit masks per (batch, block)
 * over the tokens (which list the block; which of those need their slots re-read); past
 * that limit attn_bwd_workspace_bytes leaves them out and the kernels scan every
 * token's selections instead, with the same result.
 */
int attn_bwd(const attn_params* params, const void* q, const void* k, const void* v,
             const void* o, const void* dout, const float* m, const float* l,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
             void* stream);

/* Bytes of device workspace attn_bwd needs for these params (0 if params invalid). */
size_t attn_bwd_workspace_bytes(const attn_params* params);

/*
 * attn_bwd_noalloc -- attn_bwd (dense mode) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, result and flags as attn_bwd, without the workspace: the
 * scratch lives in a static device array of ATTN_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the library's load until the process ends.  Nothing is
 * allocated.
 *   * Params whose attn_bwd_workspace_bytes exceeds ATTN_NOALLOC_SCRATCH_BYTES return
 *     ATTN_ERR_WORKSPACE (nothing launched); use attn_bwd with a workspace for them.
 *   * All calls on one GPU share that GPU's array, which keeps the last call's contents
 *     (nothing in it needs to start at zero: every call writes what it reads, except that
 *     ATTN_BWD_REUSE_STATS reads the statistics left by the previous call on this GPU).
 *     Calls that overlap on one GPU (other streams, other threads) race on it.
 *   * Sparse mode (sel_idx != NULL) returns ATTN_ERR_UNSUPPORTED.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_bwd_noalloc(const attn_params* params, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* m, const float* l,
                     void* dq, void* dk, void* dv, void* stream);

/*
 * block_select -- exact top-n block selection ("AnnAttention", select_block, with the
 * approximate index replaced by exact inner products):
 *   mean_c = average of key rows c*bs .. c*bs+bs-1 (full blocks), in fp64;
 *   a token t in block i = t / bs scores the blocks c < i by q_t . mean_c (fp64),
 *   keeps the top min(top_n, i) by (score descending, block index ascending), pads
 *   with -1 and sorts ascending (so -1 entries come first).
 *
 *   q          [in]  bf16 [B, Sq, E] (BSHD with the heads flattened: E = H * D), row r at
 *                    position q_pos0 + r.
 *   k          [in]  bf16 [B, Skv, E] (Skv = seqlen_kv, or Sq when 0).
 *   idx        [out] int32 [B, Sq, top_n].
 * A block's mean is a function of its rows, so recomputing the means from the key cache
 * at every decoding step equals the page's index that gains one mean per completed block.
 *   workspace  device scratch of at least block_select_workspace_bytes(params) bytes
 *              (256-byte aligned; contents overwritten): the fp64 block means, each
 *              mean as two bf16 parts and its norm and, when only a few query blocks
 *              are selected for (decoding), the partial top-n lists of the workgroups
 *              that share a block's candidates.
 * With up to 256 key blocks and 256 or more query blocks the scores are first taken in
 * bf16 (the two parts) and only the candidates that an error bound leaves undecided are
 * scored in fp64; the indices are those of the exact fp64 scores either way.
 */
int block_select(const select_params* params, const void* q, const void* k, int32_t* idx,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace block_select needs (0 if params invalid). */
size_t block_select_workspace_bytes(const select_params* params);

/* Message of the last failed call on this thread ("" after a success). */
const char* attn_last_error(void);

/* ATTN_PARAMS_VERSION the library was built with. */
uint32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RING_EXACT_ATTENTION_ATTN_H_ */
