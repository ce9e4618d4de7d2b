// Forward pass of blockwise exact attention on gfx950.
//
// Method ("bpt.py", _blockwise_attention_fwd inside _ring_attention_fwd): a query tile
// walks the key tiles it can see, in ring order over the virtual key blocks, keeping a
// running max m, denominator l and unnormalised numerator acc; each tile rescales the
// carry by exp(m_old - m_new) before adding exp(s - m_new) and exp(s - m_new) V.  Masks
// follow _chunk_attention_bias (causal) and the TransformerEngine page's
// _make_causal_swa_mask (window), on global positions.
//
// gfx950 mapping (bf16): one workgroup = 8 wavefronts (one per CU, two per SIMD); each
// wave owns 32 query rows of one q head, and the workgroup covers gh heads of one GQA
// group x 256/gh rows, so all eight waves read the same K/V tiles.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane owns one query row
// (a column of the accumulator), the row max / sum need one cross-half exchange, and
// P^T is already the B operand of O^T = V^T P^T.
//
// K and V tiles of 64 keys are copied straight from HBM/L2 into LDS (buffer loads with
// an LDS destination, rows past the end read as zero), three stages deep, with layouts
// chosen so that neither operand read has bank conflicts: K rows at an odd number of
// 16-byte slots (row-operand reads), V rows at 20 slots (ds_read_b64_tr_b16 reads, four
// rows cover all banks).
//
// The two waves of a SIMD alternate between an MFMA block (S of tile t and O += P V of
// tile t-1) and a VALU block (mask, row max, exp, row sum of tile t): waves 0-3 run the
// MFMA block while waves 4-7 run the VALU block, and the roles swap at every workgroup
// barrier, so the matrix unit of each SIMD is fed by one wave while the other does its
// softmax arithmetic.
//
// Accumulation is fp32; exp uses v_exp_f32 on logits pre-scaled by scale*log2(e).  The
// carry is rescaled only when a row max grows by more than 2^8 (exact: numerator and
// denominator share the stale reference), and the stored statistics use the exact max.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace rea {

template <int D, int DV, int NW_>
struct FwdCfg {
  static constexpr int NW = NW_;                   // wavefronts per workgroup (8 or 4)
  static constexpr bool PP = NW == 8;              // ping-pong between the two waves of a SIMD
  // keys per tile: 64 with the ping-pong; 32 with 4 waves, whose windowed rows need
  // about 160 keys per 32-row block (five 32-key tiles instead of three of 64)
  static constexpr int BN = PP ? 64 : 32;
  static constexpr int NMB = BN / 32;              // 32-key blocks per tile
  static constexpr int KS = D / 16;                // k-steps of S^T over d
  static constexpr int DB = DV / 32;               // 32-row blocks of O^T
  static constexpr int DC = D / 8;                 // 16-byte chunks per Q / K row
  static constexpr int DCV = DV / 8;               // ... per V / O row
  static constexpr int KRS = DC + 1;               // K row pitch in 16-byte slots (odd)
  static constexpr int VRS = DCV == 4 ? 4 : (DCV == 8 ? 12 : 20);   // V row pitch, slots
  static constexpr int KI = (BN * KRS + 63) / 64;  // 64-lane copy instructions per K tile
  static constexpr int VI = (BN * VRS + 63) / 64;  // ... per V tile
  static constexpr int NI = (KI + VI + NW - 1) / NW;   // per wave per tile
  static constexpr int KB = KI * 1024, VB = VI * 1024;
  // 8 waves: three stages, each holding K and V of one tile.  4 waves (two workgroups
  // per CU, so at most 80 KB each): two K slots and two V slots, V copied one tile
  // behind K (K of tile t+1 and V of tile t are copied during step t).
  static constexpr int STAGE = KB + VB;
  // The prologue stages each wave's 32 Q rows (2D bytes each) from QOFF on, past what
  // step 0's copies touch; the epilogue stages O rows (2DV + 16 bytes) from 0.
  static constexpr int QOFF = PP ? STAGE : KB;
  static constexpr int cmax(int x, int y) { return x > y ? x : y; }
  static constexpr int LDS = cmax(cmax((PP ? 3 : 2) * STAGE, QOFF + NW * 32 * 2 * D), NW * 32 * (2 * DV + 16));
  static constexpr int kaddr(int slot) { return PP ? slot * STAGE : slot * KB; }
  static constexpr int vaddr(int slot) { return PP ? slot * STAGE + KB : 2 * KB + slot * VB; }
};

// Rows of the scores may grow by this much (log2 units) before the carry is rescaled.
constexpr float kRescaleThreshold = 8.0f;

// EX: extra logit terms compiled in -- bit 0 an additive bias, bit 1 a dropout mask.
template <int D, int DV, int NW, int EX>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, DV, NW>;
  constexpr bool BIAS = (EX & 1) != 0, DROP = (EX & 2) != 0;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

  int b, hg, qt;
  map_task(wg_index(a.rev_order), a.n_qtiles, a.B, a.n_hg, a.Hkv, a.G >> a.gh_shift, a.xcd_groups, a.hi_off < kPosInf,
           b, hg, qt);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int grp = wave >> 2;                       // 0: MFMA block in the first half-step
  const int hq = (hg << a.gh_shift) + (wave & (a.gh - 1));
  const int hkv = hq / a.G;
  const int wg_row0 = qt * a.rows_wg;
  const int row0 = wg_row0 + 32 * (wave >> a.gh_shift);
  const int row = row0 + li;
  const bool row_ok = row < a.Sq;

  const size_t q_rs = (size_t)a.Hq * D;            // elements between q rows
  const size_t o_rs = (size_t)a.Hq * DV;           // ... between o (and carry) rows
  const uint32_t k_rs_b = (uint32_t)a.Hkv * D * 2;            // bytes between key rows
  const uint32_t v_rs_b = (uint32_t)a.Hkv * DV * 2;           // bytes between value rows
  const size_t kv_row0 = (size_t)b * a.Skv * a.Hkv + hkv;
  const uint32_t k_bytes = a.Skv > 0 ? (uint32_t)(a.Skv - 1) * k_rs_b + D * 2 : 0;
  const uint32_t v_bytes = a.Skv > 0 ? (uint32_t)(a.Skv - 1) * v_rs_b + DV * 2 : 0;
  const __bf16* kbase = (const __bf16*)a.k + kv_row0 * D;
  const __bf16* vbase = (const __bf16*)a.v + kv_row0 * DV;

  // Q^T as B operands: lane (li, lh) holds q[row][16kk + 8lh .. +7]; loaded through LDS
  // (see the prologue) so that the HBM reads cover whole rows.
  bf16x8 qreg[C::KS];

  // O^T accumulators: acc[db][r] = O[row][32db + 8(r>>2) + 4lh + (r&3)], unnormalised,
  // relative to m_used.  m_true is the exact running max.
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_used = -INFINITY, m_true = -INFINITY;   // log2 units of the scaled logits
  float l_part = 0.f;                              // this lane's half of the denominator
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  float* accp = a.acc ? a.acc + ((size_t)b * a.Sq + row) * o_rs + (size_t)hq * DV : nullptr;
  if (a.carry_in && row_ok) {
    const float mi = a.m[stat];
    m_used = m_true = mi * kLog2e;
    l_part = lh == 0 ? a.l[stat] : 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v4 = *(const f32x4*)(accp + 32 * db + 8 * g + 4 * lh);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * g + e] = v4[e];
      }
  }

  // Keys visible to any row of this workgroup: j in [i - delta + lo_off, i - delta + hi_off].
  const int r_last_wg = min(wg_row0 + a.rows_wg, a.Sq) - 1;
  const int jlo = max(0, wg_row0 - a.delta + a.lo_off);
  const int jhi = min(a.Skv - 1, r_last_wg - a.delta + a.hi_off);
  int diag = (wg_row0 - a.delta);
  diag = diag < 0 ? 0 : diag / a.kv_block;
  if (diag >= a.n_vblocks) diag = a.n_vblocks - 1;
  KeyTileIter<C::BN> it;
  it.init(a.n_vblocks, a.kv_block, diag, jlo, jhi);

  const bool wave_on = row0 < a.Sq;
  const int w_last = min(row0 + 31, a.Sq - 1);
  const int w_jmin_lo = row0 - a.delta + a.lo_off;
  const int w_jmin_hi = w_last - a.delta + a.lo_off;
  const int w_jmax_lo = row0 - a.delta + a.hi_off;
  const int w_jmax_hi = w_last - a.delta + a.hi_off;
  const int my_jmin = row - a.delta + a.lo_off;
  const int my_jmax = row - a.delta + a.hi_off;

  // Tile copies: instruction n (0 <= n < KI + VI) fills bytes [1024n', 1024n' + 1024) of
  // a K slot (n' = n < KI) or a V slot (n' = n - KI); lane l of it carries 16-byte slot
  // 64n' + l of the tile, i.e. row slot / pitch, chunk slot % pitch (padding slots are
  // skipped).  Wave w issues instructions w, w + NW, ...  One call copies K of tile ts_k
  // (when do_k) into K slot sk and V of tile ts_v (when do_v) into V slot sv.
  uint32_t voff[C::NI];
  bool vld[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int n = wave + C::NW * i;
    const bool is_k = n < C::KI;
    const int pitch = is_k ? C::KRS : C::VRS;
    const int slot = 64 * (is_k ? n : n - C::KI) + lane;
    const int r = slot / pitch, ch = slot - r * pitch;
    vld[i] = n < C::KI + C::VI && ch < (is_k ? C::DC : C::DCV) && r < C::BN;
    voff[i] = (uint32_t)r * (is_k ? k_rs_b : v_rs_b) + 16u * ch;
  }
  auto issue = [&](bool do_k, int ts_k, int sk, bool do_v, int ts_v, int sv) {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc_at(kbase, k_bytes, __builtin_amdgcn_readfirstlane((uint32_t)ts_k * k_rs_b));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc_at(vbase, v_bytes, __builtin_amdgcn_readfirstlane((uint32_t)ts_v * v_rs_b));
    char* const kb = lds + C::kaddr(sk);
    char* const vb = lds + C::vaddr(sv) - C::KB;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int n = wave + C::NW * i;
      if (n < C::KI) {
        if (do_k && vld[i]) dma16(rk, kb + 1024 * n, voff[i]);
      } else if (n < C::KI + C::VI) {
        if (do_v && vld[i]) dma16(rv, vb + 1024 * n, voff[i]);
      }
    }
  };

  // Operand offsets (bytes within a slot).  K rows as A operands of S^T; V^T by
  // transposed reads: lane (g = lane/16, j = lane%16) points at
  // V[16c + 4(g>>1) + j/4 (+8)][32db + 16(g&1) + 4(j%4) ..+3].
  const int tg = lane >> 4, tj = lane & 15;
  const int k_off = li * (16 * C::KRS) + 16 * lh;
  const int v_off = (4 * (tg >> 1) + (tj >> 2)) * (16 * C::VRS) + 32 * (tg & 1) + 8 * (tj & 3);

  f32x16 s[C::NMB];
  bf16x8 pb[2 * C::NMB];                           // P^T of the last softmax, B operands
  bool s_valid = false, p_valid = false;

  // With a bias, s holds the raw bias of the next tile whose S is computed (loaded as
  // soon as the previous scores are consumed, so the loads overlap other work); the S
  // MFMAs accumulate onto bias / scale.  Keys past the tile's end read key ts instead
  // and are masked with the rest.
  const float* const brow =
      BIAS ? a.bias + b * a.bs_b + hq * a.bs_h + (long long)min(row, a.Sq - 1) * a.bs_i : nullptr;
  // Dropout bits of the same tile (dwl), fetched with it and applied before the row max.
  const uint32_t* const drow =
      DROP ? a.drop + b * a.ds_b + hq * a.ds_h + (long long)min(row, a.Sq - 1) * a.ds_i : nullptr;
  const int drop_nw = (a.Skv + 31) >> 5;
  uint32_t dwr[C::NMB + 1] = {};
  auto bias_load = [&](int ts, int kend) {
    if constexpr (BIAS) {
      const int last = min(kend, a.Skv) - 1;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
        bias_fetch16(s[mb], brow, a.bs_j, ts + 32 * mb + 4 * lh, last, ts, a.bias_vec4 != 0);
    }
    if constexpr (DROP) drop_fetch_tile(dwr, drow, drop_nw, ts);
  };

  // MFMA block: S^T of tile ts_s (K in slot st_s) and O^T += V^T P^T for the tile whose
  // V is in slot st_p.
  auto mfma_block = [&](bool do_s, int ts_s, int kend_s, int st_s, int st_p) {
    __builtin_amdgcn_s_setprio(1);
    s_valid = false;
    if (do_s && wave_on && !(ts_s > w_jmax_hi || min(kend_s, a.Skv) - 1 < w_jmin_lo)) {
      s_valid = true;
      const char* kt = lds + C::kaddr(st_s) + k_off;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = BIAS ? s[mb][r] * a.inv_scale : 0.f;
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
        for (int mb = 0; mb < C::NMB; ++mb) {
          const bf16x8 ka = *(const bf16x8*)(kt + mb * 32 * 16 * C::KRS + 32 * kk);
          s[mb] = mfma32(ka, qreg[kk], s[mb]);
        }
    }
    if (p_valid) {
      const char* vt = lds + C::vaddr(st_p) + v_off;
#pragma unroll
      for (int c = 0; c < 2 * C::NMB; ++c)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const char* vp0 = vt + c * 16 * 16 * C::VRS + 64 * db;
          const bf16x8 va = join_bf16x8(lds_read_tr16((const __bf16*)vp0),
                                        lds_read_tr16((const __bf16*)(vp0 + 8 * 16 * C::VRS)));
          acc[db] = mfma32(va, pb[c], acc[db]);
        }
      p_valid = false;
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // VALU block: mask, max, (lazy) rescale of the carry, P = exp2(S - m), row sums.
  auto softmax_block = [&](int ts, int kend) {
    if (!s_valid) return;
    const int tend = min(kend, a.Skv);            // keys >= tend are not in this visit
    const bool full = ts >= w_jmin_hi && ts + C::BN - 1 <= w_jmax_lo && ts + C::BN <= tend;
    if (!full) {
      cold_path();
      // key j = ts + 4lh + koff is visible iff jlo_v <= j <= jhi_v: one unsigned compare
      const int jlo_v = max(my_jmin, ts), jhi_v = min(my_jmax, tend - 1);
      const uint32_t span = (uint32_t)(jhi_v - jlo_v);
      const int base = ts + 4 * lh - jlo_v;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * mb + 8 * (r >> 2) + (r & 3);
          if (jhi_v < jlo_v || (uint32_t)(base + koff) > span) s[mb][r] = -INFINITY;
        }
    }
    if constexpr (DROP) {
      uint32_t dwl[C::NMB];
      drop_bits_tile(dwl, dwr, ts, lh);
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) drop_apply16(s[mb], dwl[mb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = fmaxf(mx, other_half(mx));
    const float mt = mx * a.scale_log2;            // this tile's row max (log2 units)
    m_true = fmaxf(m_true, mt);
    if (__ballot(mt > m_used + kRescaleThreshold)) {
      cold_path();
      const float m_new = fmaxf(m_used, mt);
      const float alpha = fast_exp2(m_used - (m_new == -INFINITY ? 0.f : m_new));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_used = m_new;
    }
    const float m_ref = (m_used == -INFINITY) ? 0.f : m_used;
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = fast_exp2(fmaf(s[mb][8 * ks + 2 * w], a.scale_log2, -m_ref));
          const float p1 = fast_exp2(fmaf(s[mb][8 * ks + 2 * w + 1], a.scale_log2, -m_ref));
          rs += p0 + p1;
          w4[w] = pack_bf16x2(p0, p1);
        }
        pb[2 * mb + ks] = as_bf16x8(w4);
      }
    l_part += rs;
    p_valid = true;
  };

  // Pipeline (8 waves).  Step t has two halves separated by workgroup barriers:
  //   group 0: [mfma_block: S of t, PV of t-1] | [softmax of t]
  //   group 1: [softmax of t-1]                | [mfma_block: S of t, PV of t-1]
  // Tile t+1 is copied into its stage during step t (the stage last held tile t-2).
  // Both groups run the same number of steps, hence of barriers.
  int ts_c = 0, ke_c = 0, ts_p = 0, ke_p = 0;
  bool have_c = it.next(ts_c, ke_c), have_p = false;
  // Prologue: this wave's 32 Q rows are copied whole (16 lanes per row) into LDS that no
  // copy of step 0 touches and read back in the operand layout; K (and V, with 8 waves)
  // of tile 0 go to slot 0.
  constexpr int RPI = 64 / C::DC;                  // Q rows per copy instruction
  char* const qs = lds + C::QOFF + wave * (32 * 2 * D);
  {
    const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (uint32_t)(q_rs * 2) + (uint32_t)hq * D * 2);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc_at((const __bf16*)a.q + (size_t)b * a.Sq * q_rs, (uint32_t)a.Sq * (uint32_t)(q_rs * 2), so);
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i)
      dma16(rq, qs + 1024 * i, (uint32_t)(RPI * i + lane / C::DC) * (uint32_t)(q_rs * 2) + 16u * (lane % C::DC));
  }
  if (have_c) issue(true, ts_c, 0, C::PP, ts_c, 0);
  wait_vmcnt0();
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) qreg[kk] = *(const bf16x8*)(qs + li * (2 * D) + 32 * kk + 16 * lh);
  __syncthreads();                                 // the Q rows' LDS is refilled from step 0 on
  if constexpr (!C::PP) {
    // 4 waves, one per SIMD (the other workgroup on the CU supplies the second wave):
    // step t runs [S of t, PV of t-1] then the softmax of t, while K of t+1 and V of t
    // are copied (K slot (t+1)&1 last held tile t-1, V slot t&1 tile t-2).
    int sk = 0;                                    // K slot of the current tile
    if (have_c) bias_load(ts_c, ke_c);
    while (have_c || have_p) {
      int ts_n = 0, ke_n = 0;
      const bool have_n = have_c && it.next(ts_n, ke_n);
      issue(have_n, ts_n, sk ^ 1, have_c, ts_c, sk);
      mfma_block(have_c, ts_c, ke_c, sk, sk ^ 1);
      softmax_block(ts_c, ke_c);
      if (have_n) bias_load(ts_n, ke_n);
      wait_vmcnt0();
      __syncthreads();
      have_p = have_c; ts_p = ts_c; ke_p = ke_c;
      have_c = have_n; ts_c = ts_n; ke_c = ke_n;
      sk ^= 1;
    }
  } else {
    int st_c = 0, st_p = 0;
    if (grp == 0) {
      if (have_c) bias_load(ts_c, ke_c);
      while (have_c || have_p) {
        int ts_n = 0, ke_n = 0;
        const bool have_n = have_c && it.next(ts_n, ke_n);
        const int st_n = st_c == 2 ? 0 : st_c + 1;
        if (have_n) issue(true, ts_n, st_n, true, ts_n, st_n);
        mfma_block(have_c, ts_c, ke_c, st_c, st_p);
        __syncthreads();
        softmax_block(ts_c, ke_c);
        if (have_n) bias_load(ts_n, ke_n);
        wait_vmcnt0();
        __syncthreads();
        have_p = have_c; ts_p = ts_c; ke_p = ke_c; st_p = st_c;
        have_c = have_n; ts_c = ts_n; ke_c = ke_n; st_c = st_n;
      }
    } else {
      while (have_c || have_p) {
        int ts_n = 0, ke_n = 0;
        const bool have_n = have_c && it.next(ts_n, ke_n);
        const int st_n = st_c == 2 ? 0 : st_c + 1;
        if (have_n) issue(true, ts_n, st_n, true, ts_n, st_n);
        softmax_block(ts_p, ke_p);
        if (have_c) bias_load(ts_c, ke_c);
        __syncthreads();
        mfma_block(have_c, ts_c, ke_c, st_c, st_p);
        wait_vmcnt0();
        __syncthreads();
        have_p = have_c; ts_p = ts_c; ke_p = ke_c; st_p = st_c;
        have_c = have_n; ts_c = ts_n; ke_c = ke_n; st_c = st_n;
      }
    }
  }

  // Normalise the statistics to the exact max: l_true = l_used * 2^(m_used - m_true).
  const float l_used = l_part + other_half(l_part);
  const float corr = (m_true == -INFINITY) ? 0.f : fast_exp2(m_used - m_true);
  if (a.finalize) {
    // O through LDS (this wave's 32 rows at 2D + 16 bytes, in the now idle stages; all
    // reads of the stages ended at the loop's last barrier), then stored as whole rows.
    // A sink adds exp(z) to the denominator (relative to m_used, like l_used); a row with
    // no visible key keeps O = 0.
    float den = l_used;
    if (a.has_sink && m_used != -INFINITY) den += fast_exp2(fmaf(a.sink ? a.sink[hq] : 0.f, kLog2e, -m_used));
    const float inv = den > 0.f ? 1.f / den : 0.f;
    constexpr int OP = 2 * DV + 16, RPO = 64 / C::DCV;
    char* const os = lds + wave * (32 * OP);
    const size_t o_off = ((size_t)b * a.Sq + row0) * o_rs + (size_t)hq * DV;
    // The low part x - bf16(x) of each output, rounded to bf16, goes straight from the
    // registers to o_lo (8 bytes per lane, the two lanes of a row 16 contiguous bytes).
    __bf16* const lrow = a.o_lo ? (__bf16*)a.o_lo + o_off + (size_t)li * o_rs : nullptr;
    const bool lo_ok = a.o_lo != nullptr && row0 + li < a.Sq;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w, wl;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float x0 = acc[db][4 * g + 2 * h] * inv, x1 = acc[db][4 * g + 2 * h + 1] * inv;
          w[h] = pack_bf16x2(x0, x1);
          wl[h] = pack_bf16x2(x0 - bf16_lo(w[h]), x1 - bf16_hi(w[h]));
        }
        *(u32x2*)(os + li * OP + 2 * (32 * db + 8 * g + 4 * lh)) = w;
        if (lo_ok) *(u32x2*)(lrow + 32 * db + 8 * g + 4 * lh) = wl;
      }
    __bf16* ob = (__bf16*)a.o + o_off;
#pragma unroll
    for (int i = 0; i < 32 / RPO; ++i) {
      const int r = RPO * i + lane / C::DCV, ch = lane % C::DCV;
      const u32x4 v = *(const u32x4*)(os + r * OP + 16 * ch);
      if (row0 + r < a.Sq) *(u32x4*)(ob + (size_t)r * o_rs + 8 * ch) = v;
    }
  }
  if (row_ok) {
    if (!a.finalize) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[db][4 * g + e] * corr;
          *(f32x4*)(accp + 32 * db + 8 * g + 4 * lh) = v4;
        }
    }
    if (lh == 0) {
      a.m[stat] = (m_true == -INFINITY) ? -INFINITY : m_true * kLn2;
      a.l[stat] = l_used * corr;
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// A plain, exact-in-fp32 kernel for float32 inputs (small head dims): one thread per
// query row, key tiles staged in LDS, per-tile online softmax.  Same masking,
// ring order and carry conventions as the bf16 kernel.
template <int D, int DV>
__global__ __launch_bounds__(128) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BM = 128, BN = 32;
  __shared__ float sK[BN][D + 1];
  __shared__ float sV[BN][DV + 1];
  int b, hq, qt;
  map_task(wg_index(a.rev_order), a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, 0, false, b, hq, qt);
  const int hkv = hq / a.G;
  const int tid = threadIdx.x;
  const int row = qt * BM + tid;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D, k_rs = (size_t)a.Hkv * D;
  const size_t o_rs = (size_t)a.Hq * DV, v_rs = (size_t)a.Hkv * DV;
  const float* qp = (const float*)a.q + (size_t)b * a.Sq * q_rs + (size_t)hq * D;
  const float* kp = (const float*)a.k + (size_t)b * a.Skv * k_rs + (size_t)hkv * D;
  const float* vp = (const float*)a.v + (size_t)b * a.Skv * v_rs + (size_t)hkv * DV;

  float qr[D], acc[DV];
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = row_ok ? qp[(size_t)row * q_rs + d] : 0.f;
#pragma unroll
  for (int d = 0; d < DV; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  float* accp = a.acc ? a.acc + ((size_t)b * a.Sq + row) * o_rs + (size_t)hq * DV : nullptr;
  if (a.carry_in && row_ok) {
    m_run = a.m[stat] * kLog2e;
    l_run = a.l[stat];
#pragma unroll
    for (int d = 0; d < DV; ++d) acc[d] = accp[d];
  }
  const int wg_row0 = qt * BM;
  const int r_last = min(wg_row0 + BM, a.Sq) - 1;
  const int jlo = max(0, wg_row0 - a.delta + a.lo_off);
  const int jhi = min(a.Skv - 1, r_last - a.delta + a.hi_off);
  int diag = wg_row0 - a.delta;
  diag = diag < 0 ? 0 : diag / a.kv_block;
  if (diag >= a.n_vblocks) diag = a.n_vblocks - 1;
  KeyTileIter<BN> it;
  it.init(a.n_vblocks, a.kv_block, diag, jlo, jhi);
  const int my_jmin = row - a.delta + a.lo_off, my_jmax = row - a.delta + a.hi_off;

  int ts, kend;
  while (it.next(ts, kend)) {
    const int tend = min(kend, a.Skv);
    for (int c = tid; c < BN * D; c += BM) {
      const int r = c / D, d = c % D, j = ts + r;
      sK[r][d] = j < a.Skv ? kp[(size_t)j * k_rs + d] : 0.f;
    }
    for (int c = tid; c < BN * DV; c += BM) {
      const int r = c / DV, d = c % DV, j = ts + r;
      sV[r][d] = j < a.Skv ? vp[(size_t)j * v_rs + d] : 0.f;
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < BN; ++r) {
      const int j = ts + r;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qr[d], sK[r][d], dot);
      if (a.bias && j < tend) dot = fmaf(a.bias[b * a.bs_b + hq * a.bs_h + (long long)min(row, a.Sq - 1) * a.bs_i +
                                                (long long)j * a.bs_j], a.inv_scale, dot);
      const bool drop = a.drop && j < tend && dropped(a.drop, b * a.ds_b + hq * a.ds_h, a.ds_i, min(row, a.Sq - 1), j);
      s[r] = (j < my_jmin || j > my_jmax || j >= tend || drop) ? -INFINITY : dot * a.scale_log2;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DV; ++d) acc[d] *= alpha;
#pragma unroll
    for (int r = 0; r < BN; ++r) {
      const float p = fast_exp2(s[r] - m_ref);
      l_run += p;
#pragma unroll
      for (int d = 0; d < DV; ++d) acc[d] = fmaf(p, sV[r][d], acc[d]);
    }
    m_run = m_new;
    __syncthreads();
  }
  if (row_ok) {
    if (a.finalize) {
      float den = l_run;
      if (a.has_sink && m_run != -INFINITY) den += fast_exp2(fmaf(a.sink ? a.sink[hq] : 0.f, kLog2e, -m_run));
      const float inv = den > 0.f ? 1.f / den : 0.f;
      float* op = (float*)a.o + ((size_t)b * a.Sq + row) * o_rs + (size_t)hq * DV;
#pragma unroll
      for (int d = 0; d < DV; ++d) op[d] = acc[d] * inv;
    } else {
#pragma unroll
      for (int d = 0; d < DV; ++d) accp[d] = acc[d];
    }
    a.m[stat] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
    a.l[stat] = l_run;
  }
}

// Smallest number of query rows a workgroup covers (for the host-side size checks).
int fwd_tile_rows(int dtype) { return dtype == 0 ? 32 : 128; }

// Workgroup shape of the bf16 forward: 8 waves (ping-pong, one workgroup per CU) when
// a query tile sees many keys; 4 waves (two workgroups per CU, 32-key tiles) when every
// row sees a window under 1024 keys, where a work item is only a few tiles long and the
// second workgroup hides the load of one item's Q and the store of its O behind the
// other's tiles (measured ahead up to windows of about 1000 keys, level at 1500-3000).
static bool fwd_use_w4(const FwdArgs& a) {
  return a.lo_off > -kPosInf && a.hi_off < kPosInf && (long long)a.hi_off - a.lo_off < 1024;
}

template <int D, int DV, int EX>
static void launch_fwd_ex(const FwdArgs& a, bool w4, dim3 grid, dim3 block, hipStream_t stream) {
  if (w4)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, 4, EX>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, 8, EX>), grid, block, 0, stream, a);
}

template <int D, int DV>
static void launch_fwd_bf16(FwdArgs a, bool w4, hipStream_t stream) {
  // gh = q heads per workgroup: the largest power of two <= NW dividing the GQA group.
  const int nw = w4 ? 4 : 8, max_shift = w4 ? 2 : 3;
  a.gh_shift = 0;
  while (a.gh_shift < max_shift && a.G % (2 << a.gh_shift) == 0) ++a.gh_shift;
  a.gh = 1 << a.gh_shift;
  a.rows_wg = (32 * nw) >> a.gh_shift;
  a.n_hg = a.Hq >> a.gh_shift;
  a.n_qtiles = (a.Sq + a.rows_wg - 1) / a.rows_wg;
  const dim3 grid((unsigned)a.n_qtiles * a.B * a.n_hg), block(64 * nw);
  // extra logit terms compiled in: bit 0 bias, bit 1 dropout
  switch ((a.bias ? 1 : 0) | (a.drop ? 2 : 0)) {
    case 1: launch_fwd_ex<D, DV, 1>(a, w4, grid, block, stream); break;
    case 2: launch_fwd_ex<D, DV, 2>(a, w4, grid, block, stream); break;
    case 3: launch_fwd_ex<D, DV, 3>(a, w4, grid, block, stream); break;
    default: launch_fwd_ex<D, DV, 0>(a, w4, grid, block, stream);
  }
}

hipError_t launch_fwd(int dtype, const FwdArgs& args, hipStream_t stream) {
  if (!head_dims_supported(dtype, args.D, args.Dv)) return hipErrorInvalidValue;
  const int dd = args.D * 1000 + args.Dv;
  if (dtype == 0) {
    const bool w4 = fwd_use_w4(args);
    switch (dd) {
      case 32032: launch_fwd_bf16<32, 32>(args, w4, stream); break;
      case 64064: launch_fwd_bf16<64, 64>(args, w4, stream); break;
      case 128128: launch_fwd_bf16<128, 128>(args, w4, stream); break;
      case 128064: launch_fwd_bf16<128, 64>(args, w4, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const FwdArgs& a = args;
    const dim3 grid((unsigned)a.n_qtiles * a.B * a.Hq), block(128);
    switch (dd) {
      case 32032: hipLaunchKernelGGL((fwd_f32_kernel<32, 32>), grid, block, 0, stream, a); break;
      case 64064: hipLaunchKernelGGL((fwd_f32_kernel<64, 64>), grid, block, 0, stream, a); break;
      case 64032: hipLaunchKernelGGL((fwd_f32_kernel<64, 32>), grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace rea
