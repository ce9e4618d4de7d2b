// Backward pass of blockwise exact attention on gfx950.
//
// Method ("bpt.py", _blockwise_attention_bwd inside _ring_attention_bwd): with the
// saved max and denominator the probabilities are recomputed per tile,
//   P = exp(s - m) / l,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * o),
//   dq += scale dS K,  dk += scale dS^T Q,  dv += P^T dO.
// On the ring, dq stays with its query block while dk/dv travel with their key block;
// here one kernel owns a query tile's dq (looping over its key tiles in ring order)
// and another owns a key tile's dk/dv (looping over the query tiles of every q head
// of its GQA group), so nothing is accumulated with atomics and the result is
// bitwise reproducible.
//
// Kernels: bwd_pre (D and the log2-domain LSE), bwd_dq (per 128-row query tile:
// S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T) and bwd_dkdv (per 128-key tile:
// S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS), all on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Tiles are fetched with raw buffer
// loads (rows past the end read as zero) into row-major LDS tiles at a pitch of D + 32
// elements; transposed operands come from the same tiles through ds_read_b64_tr_b16.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace rea {

// ------------------------------------------------------------------ pre pass
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int LPR = D / EPC;               // lanes per row
  constexpr int RPB = 256 / LPR;             // rows per block
  const int tid = threadIdx.x;
  const long long rowg = (long long)wg_index(a.rev_order) * RPB + tid / LPR;   // row of [B, Sq, Hq]
  const int sub = tid % LPR;
  const long long nrows = (long long)a.B * a.Sq * a.Hq;
  float part = 0.f;
  if (rowg < nrows) {
    const u32x4 ou = *(const u32x4*)((const T*)a.o + rowg * D + sub * EPC);
    const u32x4 gu = *(const u32x4*)((const T*)a.dout + rowg * D + sub * EPC);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        part = fmaf(bf16_lo(ou[w]), bf16_lo(gu[w]), part);
        part = fmaf(bf16_hi(ou[w]), bf16_hi(gu[w]), part);
      } else {
        part = fmaf(__uint_as_float(ou[w]), __uint_as_float(gu[w]), part);
      }
    }
    if constexpr (sizeof(T) == 2) {
      if (a.o_lo) {   // the output's low part: D_i from the fp32 output, not its bf16 rounding
        const u32x4 lu = *(const u32x4*)((const T*)a.o_lo + rowg * D + sub * EPC);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          part = fmaf(bf16_lo(lu[w]), bf16_lo(gu[w]), part);
          part = fmaf(bf16_hi(lu[w]), bf16_hi(gu[w]), part);
        }
      }
    }
  }
  part = sum_lanes<LPR>(part);
  if (rowg < nrows && sub == 0) {
    const int h = (int)(rowg % a.Hq);
    const long long bs = rowg / a.Hq;
    const int s = (int)(bs % a.Sq), b = (int)(bs / a.Sq);
    const size_t st = ((size_t)b * a.Hq + h) * a.Sq + s;
    a.Dvec[st] = part;
    const float l = a.l[st], m = a.m[st];
    if (a.has_sink)
      a.lse2[st] = lse2_with_sink(m * kLog2e, l, (a.sink ? a.sink[h] : 0.f) * kLog2e);
    else
      a.lse2[st] = (l > 0.f) ? fmaf(m, kLog2e, log2f(l)) : INFINITY;
  }
}

// ------------------------------------------------------------------ dq (bf16)
// One workgroup = 8 wavefronts (one per CU, two per SIMD), each owning 32 query rows of
// one q head; the workgroup covers gh heads of one GQA group x 256/gh rows and walks
// their key tiles in ring order.  Transposed form, so each lane owns one query row:
//   S^T = K Q^T, dP^T = V dO^T (A operands: K, V tiles in LDS; B: Q, dO in registers),
//   P^T = exp2(S^T scale log2e - lse2_i), dS^T = P^T (dP^T - D_i) (lane-local stats),
//   dQ^T += K^T dS^T with the transposed K operand read by ds_read_b64_tr_b16.
// K/V tiles are copied straight into LDS, three stages deep.  K is read both as rows
// and transposed, so its rows go in groups of four at the transposed-read pitch with one
// extra 16-byte slot per group; V is read as rows only (odd slot pitch).  As in the
// forward kernel, waves 0-3 and 4-7 alternate between the MFMA block (S, dP of tile t;
// dQ of tile t-1) and the VALU block (P and dS of tile t) at every barrier.
// With fused_stats the kernel also computes D_i = rowsum(dO * O) and lse2_i from m, l
// and stores them for the dk/dv pass.
template <int D, int DV, int NW_>
struct BwdQCfg {
  static constexpr int NW = NW_;                  // 8: ping-pong, one workgroup per CU; 4: two per CU
  static constexpr bool PP = NW == 8;
  static constexpr int BN = PP ? 64 : 32;        // keys per tile (32: windowed rows, see the forward)
  static constexpr int NMB = BN / 32;             // 32-key blocks per tile
  static constexpr int NS = PP ? 3 : 2;           // stages of (K, V) tiles
  static constexpr int KS = D / 16;               // k-steps of S^T (over the q/k head dim)
  static constexpr int KSV = DV / 16;             // k-steps of dP^T (over the v head dim)
  static constexpr int DB = D / 32;
  static constexpr int DC = D / 8;                // 16-byte chunks per Q / K / dQ row
  static constexpr int DCV = DV / 8;              // ... per V / O / dO row
  static constexpr int P4 = DC == 4 ? 4 : (DC == 8 ? 12 : 20);    // K row pitch in a group (slots)
  static constexpr int G4 = 4 * P4 + 1;                            // K group pitch (slots)
  static constexpr int VRS = DCV + 1;                              // V row pitch (slots)
  static constexpr int KI = ((BN / 4) * G4 + 63) / 64;             // copy instructions per K tile
  static constexpr int VI = (BN * VRS + 63) / 64;
  static constexpr int NI = (KI + VI + NW - 1) / NW;
  static constexpr int STAGE = (KI + VI) * 1024;
  // LDS: NS stages, enough room from STAGE on for each wave's 32 Q (or dO) rows in the
  // prologue and from 0 for its 32 dQ rows (2D + 16 bytes each) in the epilogue, then the
  // per-row D values.
  static constexpr int cmax(int x, int y) { return x > y ? x : y; }
  static constexpr int MAIN = cmax(cmax(NS * STAGE, STAGE + NW * 32 * 2 * D), NW * 32 * (2 * D + 16));
};

// EX: extra logit terms compiled in -- bit 0 an additive bias, bit 1 a dropout mask.
template <int D, int DV, int NW, int EX>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq_bf16_kernel(BwdArgs a) {
  using C = BwdQCfg<D, DV, NW>;
  constexpr bool BIAS = (EX & 1) != 0, DROP = (EX & 2) != 0;
  static_assert(DV <= D, "the v head dim may not exceed the q/k head dim");
  __shared__ __attribute__((aligned(1024))) char lds[C::MAIN + C::NW * 32 * 4];

  int b, hg, qt;
  map_task(wg_index(a.rev_order), a.n_qtiles, a.B, a.n_hg, a.Hkv, a.G >> a.gh_shift, a.xcd_groups, a.hi_off < kPosInf,
           b, hg, qt);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int grp = wave >> 2;
  const int hq = (hg << a.gh_shift) + (wave & (a.gh - 1));
  const int hkv = hq / a.G;
  const int wg_row0 = qt * a.rows_wg;
  const int row0 = wg_row0 + 32 * (wave >> a.gh_shift);
  const int row = row0 + li;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D;            // elements between q / dq rows
  const size_t o_rs = (size_t)a.Hq * DV;           // ... between o / dout rows
  const uint32_t k_rs_b = (uint32_t)a.Hkv * D * 2, v_rs_b = (uint32_t)a.Hkv * DV * 2;
  const size_t kv_row0 = (size_t)b * a.Skv * a.Hkv + hkv;
  const uint32_t k_bytes = a.Skv > 0 ? (uint32_t)(a.Skv - 1) * k_rs_b + D * 2 : 0;
  const uint32_t v_bytes = a.Skv > 0 ? (uint32_t)(a.Skv - 1) * v_rs_b + DV * 2 : 0;
  const __bf16* kbase = (const __bf16*)a.k + kv_row0 * D;
  const __bf16* vbase = (const __bf16*)a.v + kv_row0 * DV;

  // Q^T and dO^T as B operands (lane (li, lh) holds x[row][16kk + 8lh .. +7]) and the row
  // statistics; filled in the prologue below.
  bf16x8 qreg[C::KS], doreg[C::KSV];
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  float lse2 = INFINITY, Di = 0.f;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int r_last_wg = min(wg_row0 + a.rows_wg, a.Sq) - 1;
  const int jlo = max(0, wg_row0 - a.delta + a.lo_off);
  const int jhi = min(a.Skv - 1, r_last_wg - a.delta + a.hi_off);
  int diag = wg_row0 - a.delta;
  diag = diag < 0 ? 0 : diag / a.kv_block;
  if (diag >= a.n_vblocks) diag = a.n_vblocks - 1;
  KeyTileIter<C::BN> it;
  it.init(a.n_vblocks, a.kv_block, diag, jlo, jhi);

  const bool wave_on = row0 < a.Sq;
  const int w_last = min(row0 + 31, a.Sq - 1);
  const int w_jmin_lo = row0 - a.delta + a.lo_off, w_jmin_hi = w_last - a.delta + a.lo_off;
  const int w_jmax_lo = row0 - a.delta + a.hi_off, w_jmax_hi = w_last - a.delta + a.hi_off;
  const int my_jmin = row - a.delta + a.lo_off, my_jmax = row - a.delta + a.hi_off;

  // Tile copies: instruction n of a stage fills bytes [1024n, 1024n + 1024); lane l of it
  // carries slot 64n' + l of the K tile (n' = n; grouped rows) or the V tile (n' = n - KI).
  uint32_t voff[C::NI];
  bool vld[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int n = wave + C::NW * i;
    int r, ch;
    bool ok;
    if (n < C::KI) {
      const int slot = 64 * n + lane;
      const int q4 = slot / C::G4, rem = slot - q4 * C::G4;
      const int k4 = rem / C::P4;
      ch = rem - k4 * C::P4;
      r = 4 * q4 + k4;
      ok = k4 < 4;
    } else {
      const int slot = 64 * (n - C::KI) + lane;
      r = slot / C::VRS;
      ch = slot - r * C::VRS;
      ok = ch < C::DCV;
    }
    vld[i] = ok && n < C::KI + C::VI && ch < C::DC && r < C::BN;
    voff[i] = (uint32_t)r * (n < C::KI ? k_rs_b : v_rs_b) + 16u * ch;
  }
  auto issue = [&](int ts, int stage) {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc_at(kbase, k_bytes, __builtin_amdgcn_readfirstlane((uint32_t)ts * k_rs_b));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc_at(vbase, v_bytes, __builtin_amdgcn_readfirstlane((uint32_t)ts * v_rs_b));
    char* sb = lds + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int n = wave + C::NW * i;
      if (n < C::KI + C::VI) {
        if (vld[i]) dma16(n < C::KI ? rk : rv, sb + 1024 * n, voff[i]);
      }
    }
  };

  // Operand offsets (bytes within a stage).  K row (li, 8lh..) for S^T; transposed K:
  // lane (g = lane/16, j = lane%16) points at K[16c + 4(g>>1) + j/4 (+8)][32db + 16(g&1) + 4(j%4)];
  // V row (li, 8lh..) for dP^T.
  const int tg = lane >> 4, tj = lane & 15;
  const int k_off = (li >> 2) * (16 * C::G4) + (li & 3) * (16 * C::P4) + 16 * lh;
  const int kt_off = (tg >> 1) * (16 * C::G4) + (tj >> 2) * (16 * C::P4) + 32 * (tg & 1) + 8 * (tj & 3);
  const int v_off = C::KI * 1024 + li * (16 * C::VRS) + 16 * lh;

  f32x16 s[C::NMB], dp[C::NMB];
  bf16x8 dsb[2 * C::NMB];                                   // dS^T of the last VALU block, B operands
  bool s_valid = false, ds_valid = false;

  // With a bias, s holds the raw bias of the next tile whose S is computed (loaded once
  // the previous scores are consumed); the S MFMAs accumulate onto bias / scale.
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

  auto mfma_block = [&](bool do_s, int ts_s, int kend_s, int st_s, int st_p) {
    __builtin_amdgcn_s_setprio(1);
    s_valid = false;
    if (do_s && wave_on && !(ts_s > w_jmax_hi || min(kend_s, a.Skv) - 1 < w_jmin_lo)) {
      s_valid = true;
      const char* kt = lds + st_s * C::STAGE + k_off;
      const char* vt = lds + st_s * C::STAGE + v_off;
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mb][r] = BIAS ? s[mb][r] * a.inv_scale : 0.f;
          dp[mb][r] = 0.f;
        }
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
        for (int mb = 0; mb < C::NMB; ++mb) {
          s[mb] = mfma32(*(const bf16x8*)(kt + mb * 8 * 16 * C::G4 + 32 * kk), qreg[kk], s[mb]);
          if (kk < C::KSV)
            dp[mb] = mfma32(*(const bf16x8*)(vt + mb * 32 * 16 * C::VRS + 32 * kk), doreg[kk], dp[mb]);
        }
    }
    if (ds_valid) {
      const char* kp = lds + st_p * C::STAGE + kt_off;
#pragma unroll
      for (int c = 0; c < 2 * C::NMB; ++c)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const char* kp0 = kp + c * 4 * 16 * C::G4 + 64 * db;
          const bf16x8 ka = join_bf16x8(lds_read_tr16((const __bf16*)kp0),
                                        lds_read_tr16((const __bf16*)(kp0 + 2 * 16 * C::G4)));
          acc[db] = mfma32(ka, dsb[c], acc[db]);
        }
      ds_valid = false;
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto valu_block = [&](int ts, int kend) {
    if (!s_valid) return;
    const int tend = min(kend, a.Skv);
    const bool full = ts >= w_jmin_hi && ts + C::BN - 1 <= w_jmax_lo && ts + C::BN <= tend;
    if constexpr (DROP) {
      uint32_t dwl[C::NMB];
      drop_bits_tile(dwl, dwr, ts, lh);
#pragma unroll
      for (int mb = 0; mb < C::NMB; ++mb) drop_apply16(s[mb], dwl[mb]);
    }
    if (!full) {
      cold_path();
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
#pragma unroll
    for (int mb = 0; mb < C::NMB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r0 = 8 * ks + 2 * w;
          const float p0 = fast_exp2(fmaf(s[mb][r0], a.scale_log2, -lse2));
          const float p1 = fast_exp2(fmaf(s[mb][r0 + 1], a.scale_log2, -lse2));
          w4[w] = pack_bf16x2(p0 * (dp[mb][r0] - Di), p1 * (dp[mb][r0 + 1] - Di));
        }
        dsb[2 * mb + ks] = as_bf16x8(w4);
      }
    ds_valid = true;
  };

  // Prologue.  Q, dO (and O for D) rows are read whole, 16 lanes per row, so that every
  // HBM access covers full cache lines: Q and then dO pass through LDS (from stage 1 on) into
  // the operand layout; O stays in registers in the row layout for the dot product.
  int ts_c = 0, ke_c = 0, ts_p = 0, ke_p = 0;
  bool have_c = it.next(ts_c, ke_c), have_p = false;
  {
    // Q rows: RPI per copy instruction (DC lanes each), NQ instructions for 32 rows;
    // dO and O rows likewise with the v head dim (RPO, NO).
    constexpr int RPI = 64 / C::DC, NQ = 32 / RPI;
    constexpr int RPO = 64 / C::DCV, NO = 32 / RPO;
    char* const qs = lds + C::STAGE + wave * (32 * 2 * D);
    const uint32_t q_rs_b = (uint32_t)q_rs * 2, o_rs_b = (uint32_t)o_rs * 2;
    const int rr = lane / C::DC, rc = lane % C::DC;
    const int orr = lane / C::DCV, orc = lane % C::DCV;
    auto rsrc_rows = [&](const void* tensor, size_t rs) {
      const uint32_t rs_b = (uint32_t)rs * 2;
      const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)row0 * rs_b + (uint32_t)(rs / a.Hq) * hq * 2);
      return make_rsrc_at((const __bf16*)tensor + (size_t)b * a.Sq * rs, (uint32_t)a.Sq * rs_b, so);
    };
    const bool fused = a.fused_stats != 0;
    // the row's statistics are loaded now, with the first copies, rather than after the
    // dO rows have landed (a third round trip to memory)
    float l_in = 0.f, m_in = 0.f, lse_in = INFINITY, d_in = 0.f;
    if (row_ok) {
      if (fused) {
        l_in = a.l[stat];
        m_in = a.m[stat];
      } else {
        lse_in = a.lse2[stat];
        d_in = a.Dvec[stat];
      }
    }
    u32x4 orow[NO];                                // O: row RPO*i + lane/DCV, chunk lane%DCV
    if (fused) {
      const __amdgpu_buffer_rsrc_t ro = rsrc_rows(a.o, o_rs);
#pragma unroll
      for (int i = 0; i < NO; ++i) orow[i] = buf_load16(ro, (uint32_t)(RPO * i + orr) * o_rs_b + 16u * orc, 0);
    }
    {
      const __amdgpu_buffer_rsrc_t rq = rsrc_rows(a.q, q_rs);
#pragma unroll
      for (int i = 0; i < NQ; ++i) dma16(rq, qs + 1024 * i, (uint32_t)(RPI * i + rr) * q_rs_b + 16u * rc);
    }
    if (have_c) issue(ts_c, 0);
    wait_vmcnt0();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) qreg[kk] = *(const bf16x8*)(qs + li * (2 * D) + 32 * kk + 16 * lh);
    __syncthreads();                               // (this wave's rows only, but keep the copies ordered)
    {
      const __amdgpu_buffer_rsrc_t rg = rsrc_rows(a.dout, o_rs);
#pragma unroll
      for (int i = 0; i < NO; ++i) dma16(rg, qs + 1024 * i, (uint32_t)(RPO * i + orr) * o_rs_b + 16u * orc);
    }
    // The output's low part, when given, in the same round trip as dO (O's rows layout).
    u32x4 lrow[NO];
    const bool with_lo = fused && a.o_lo != nullptr;
    if (with_lo) {
      const __amdgpu_buffer_rsrc_t rl = rsrc_rows(a.o_lo, o_rs);
#pragma unroll
      for (int i = 0; i < NO; ++i) lrow[i] = buf_load16(rl, (uint32_t)(RPO * i + orr) * o_rs_b + 16u * orc, 0);
    }
    wait_vmcnt0();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < C::KSV; ++kk) doreg[kk] = *(const bf16x8*)(qs + li * (2 * DV) + 32 * kk + 16 * lh);
    if (fused) {
      // D_i = sum_d dO[i][d] O[i][d] over the DCV lanes holding row i, then moved to lane i.
      float* const sd = (float*)(lds + C::MAIN) + wave * 32;
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        const u32x4 gu = *(const u32x4*)(qs + (RPO * i + orr) * (2 * DV) + 16 * orc);
        float part = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          part = fmaf(bf16_lo(orow[i][w]), bf16_lo(gu[w]), part);
          part = fmaf(bf16_hi(orow[i][w]), bf16_hi(gu[w]), part);
        }
        if (with_lo) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            part = fmaf(bf16_lo(lrow[i][w]), bf16_lo(gu[w]), part);
            part = fmaf(bf16_hi(lrow[i][w]), bf16_hi(gu[w]), part);
          }
        }
        part = sum_lanes<C::DCV>(part);
        if (orc == 0) sd[RPO * i + orr] = part;
      }
      Di = sd[li];
      const float l = l_in, m = m_in;
      if (a.has_sink)
        lse2 = lse2_with_sink(m * kLog2e, l, (a.sink ? a.sink[hq] : 0.f) * kLog2e);
      else
        lse2 = (l > 0.f) ? fmaf(m, kLog2e, log2f(l)) : INFINITY;
      if (row_ok && lh == 0) {
        a.Dvec[stat] = Di;
        a.lse2[stat] = lse2;
      }
    } else if (row_ok) {
      lse2 = lse_in;
      Di = d_in;
    }
    if (!row_ok) Di = 0.f;
    __syncthreads();                               // stage 1 on is refilled from step 0 on
  }
  if constexpr (!C::PP) {
    // 4 waves, one per SIMD (the other workgroup on the CU supplies the second wave):
    // step t runs S, dP of tile t, then dS, then dQ += K^T dS of the same tile, while tile
    // t+1 is copied into the other stage (which held tile t-1).
    int st = 0;
    if (have_c) bias_load(ts_c, ke_c);
    while (have_c) {
      int ts_n = 0, ke_n = 0;
      const bool have_n = it.next(ts_n, ke_n);
      if (have_n) issue(ts_n, st ^ 1);
      mfma_block(true, ts_c, ke_c, st, st);
      valu_block(ts_c, ke_c);
      if (have_n) bias_load(ts_n, ke_n);
      mfma_block(false, ts_c, ke_c, st, st);
      wait_vmcnt0();
      __syncthreads();
      have_c = have_n; ts_c = ts_n; ke_c = ke_n;
      st ^= 1;
    }
  } else {
    int st_c = 0, st_p = 0;
    if (grp == 0) {
      if (have_c) bias_load(ts_c, ke_c);
      while (have_c || have_p) {
        int ts_n = 0, ke_n = 0;
        const bool have_n = have_c && it.next(ts_n, ke_n);
        const int st_n = st_c == C::NS - 1 ? 0 : st_c + 1;
        if (have_n) issue(ts_n, st_n);
        mfma_block(have_c, ts_c, ke_c, st_c, st_p);
        __syncthreads();
        valu_block(ts_c, ke_c);
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
        const int st_n = st_c == C::NS - 1 ? 0 : st_c + 1;
        if (have_n) issue(ts_n, st_n);
        valu_block(ts_p, ke_p);
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

  if (a.accumulate) {
    // fp32 dq of the caller, added into: lane (li, lh) holds dq[row][32db + 8g + 4lh .. +3]
    if (row_ok) {
      float* dqp = (float*)a.dq + ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* p = (f32x4*)(dqp + 32 * db + 8 * g + 4 * lh);
          f32x4 v = *p;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += acc[db][4 * g + e] * a.scale;
          *p = v;
        }
    }
    return;
  }
  // dQ through LDS (this wave's rows at 2D + 16 bytes in the idle stages; all reads of the
  // stages ended at the loop's last barrier), then stored as whole rows.
  {
    constexpr int OP = 2 * D + 16, RPI = 64 / C::DC;
    char* const os = lds + wave * (32 * OP);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * g] * a.scale, acc[db][4 * g + 1] * a.scale);
        w[1] = pack_bf16x2(acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale);
        *(u32x2*)(os + li * OP + 2 * (32 * db + 8 * g + 4 * lh)) = w;
      }
    __bf16* ob = (__bf16*)a.dq + ((size_t)b * a.Sq + row0) * q_rs + (size_t)hq * D;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + lane / C::DC, ch = lane % C::DC;
      const u32x4 v = *(const u32x4*)(os + r * OP + 16 * ch);
      if (row0 + r < a.Sq) *(u32x4*)(ob + (size_t)r * q_rs + 8 * ch) = v;
    }
  }
}

// ------------------------------------------------------------------ dk, dv (bf16)
// One workgroup = 128 keys of one (batch, kv head), 32 per wavefront, with K and V in
// registers.  It walks every q head of the GQA group and, for each, the 32-row query
// steps that can see its keys (ring order over the virtual query blocks).  Per step:
//   S = Q K^T, dP = dO V^T (A operands: row-major Q, dO tiles; B: K, V in registers),
//   P = exp2(S scale log2e - lse2_i), dS = P (dP - D_i),
//   dV^T += dO^T P, dK^T += Q^T dS with transposed dO / Q operands via ds_read_b64_tr_b16.
template <int D, int DV>
struct BwdKVCfg {
  static constexpr int BK = 128;                  // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 32;                   // query rows per step
  static constexpr int KS = D / 16;               // k-steps of S (q/k head dim)
  static constexpr int KSV = DV / 16;             // k-steps of dP (v head dim)
  static constexpr int DB = D / 32;               // 32-column blocks of dK
  static constexpr int DBV = DV / 32;             // ... of dV
  using QL = TileLayout<D, kBothRead>;            // Q tile: row operands and transposed
  using GL = TileLayout<DV, kBothRead>;           // dO tile: the same with the v head dim
  using VL = TileLayout<DV, kRowRead>;            // V tile: row operands
  static constexpr int DC = D / 8, DCV = DV / 8;  // 16-byte chunks per Q / dO row
  static constexpr int VCPT = BK * DCV / 256;     // 16-byte chunks of the V tile per thread
  // Step tiles are copied straight into LDS: 16-byte slot s of a tile is row
  // 4 (s / GS) + (s % GS) / PS, chunk (s % GS) % PS; padding slots are skipped.
  static constexpr int QPS = QL::PITCH / 8, QGS = QL::GROUP / 8, QSL = QL::elems(BQ) / 8;
  static constexpr int GPS = GL::PITCH / 8, GGS = GL::GROUP / 8, GSL = GL::elems(BQ) / 8;
  static constexpr int QI = (QSL + 63) / 64, GI = (GSL + 63) / 64;   // 64-lane copies per tile
  static constexpr int NI = (QI + GI + 3) / 4;                       // per wave
  static constexpr int QB = QI * 1024, GB = GI * 1024;               // bytes per tile buffer
};

// EX: extra logit terms compiled in -- bit 0 an additive bias, bit 1 a dropout mask.
template <int D, int DV, int EX>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_bf16_kernel(BwdArgs a) {
  using C = BwdKVCfg<D, DV>;
  constexpr bool BIAS = (EX & 1) != 0, DROP = (EX & 2) != 0;
  static_assert(DV <= D, "the v head dim may not exceed the q/k head dim");
  // Q and dO tiles of a step, two buffers each (the next step's rows are copied in while
  // the current step runs).  Each buffer is an array of its own and the step loop is
  // unrolled by two, so the compiler can tell the buffer being read from the one being
  // copied into and does not hold the step's LDS reads behind the copies.
  __shared__ __attribute__((aligned(1024))) char sQb0[C::QB];
  __shared__ __attribute__((aligned(1024))) char sQb1[C::QB];
  __shared__ __attribute__((aligned(1024))) char sGb0[C::GB];
  __shared__ __attribute__((aligned(1024))) char sGb1[C::GB];
  __shared__ __attribute__((aligned(16))) __bf16 sVk[C::VL::elems(C::BK)];   // this workgroup's V rows
  __shared__ __attribute__((aligned(16))) float sLse[2][C::BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BQ];
  // dropout words of a step: [wave][row], one 32-key word per wave (staged like Q, dO)
  __shared__ __attribute__((aligned(16))) uint32_t sDrop[2][DROP ? 4 * C::BQ : 1];

  // Workgroup id -> (batch, kv head, key tile) and the split: with kv_splits = ns > 1 the
  // G q heads of the group are shared out over ns workgroups (G / ns heads each), which
  // write fp32 partial dk, dv that bwd_dkdv_reduce_kernel sums.
  int b, hv, kt;
  map_kv_task(wg_index(a.rev_order), a.n_ktiles, a.B, a.Hkv * a.kv_splits, a.xcd_kv_groups, false, b, hv, kt);
  const int hkv = hv / a.kv_splits, split = hv - hkv * a.kv_splits;
  const int g_per = a.G / a.kv_splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int k0 = kt * C::BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + li;
  const bool key_ok = key < a.Skv;
  const size_t k_rs = (size_t)a.Hkv * D, v_rs = (size_t)a.Hkv * DV;
  const uint32_t q_rs_b = (uint32_t)a.Hq * D * 2, g_rs_b = (uint32_t)a.Hq * DV * 2;
  const size_t koff = ((size_t)b * a.Skv + key) * k_rs + (size_t)hkv * D;
  const size_t voff = ((size_t)b * a.Skv + key) * v_rs + (size_t)hkv * DV;
  const uint32_t q_bytes = a.Sq > 0 ? (uint32_t)a.Sq * q_rs_b : 0;
  const uint32_t g_bytes = a.Sq > 0 ? (uint32_t)a.Sq * g_rs_b : 0;
  const __bf16* qbase = (const __bf16*)a.q + (size_t)b * a.Sq * a.Hq * D;
  const __bf16* gbase = (const __bf16*)a.dout + (size_t)b * a.Sq * a.Hq * DV;

  // K stays in registers (B operand of S = Q K^T); V goes to LDS once (B operand of
  // dP = dO V^T, re-read every step) to keep the register count within two waves per SIMD.
  bf16x8 kreg[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (key_ok) u = *(const u32x4*)((const __bf16*)a.k + koff + 16 * kk + 8 * lh);
    kreg[kk] = as_bf16x8(u);
  }
  {
    const uint32_t v_rs_b = (uint32_t)v_rs * 2;
    const size_t v_base = ((size_t)b * a.Skv + k0) * v_rs + (size_t)hkv * DV;
    const int rows = min(C::BK, a.Skv - k0);
    const __amdgpu_buffer_rsrc_t rvk =
        make_rsrc((const __bf16*)a.v + v_base, (uint32_t)(rows - 1) * v_rs_b + DV * 2);
#pragma unroll
    for (int u = 0; u < C::VCPT; ++u) {
      const int c = tid + 256 * u, r = c / C::DCV, ch = c % C::DCV;
      *(u32x4*)&sVk[C::VL::idx(r, 8 * ch)] = buf_load16(rvk, (uint32_t)r * v_rs_b + 16u * ch, 0);
    }
  }
  f32x16 dk[C::DB], dv[C::DBV];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = 0.f;
#pragma unroll
  for (int db = 0; db < C::DBV; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[db][r] = 0.f;

  // Rows that can see some key of this workgroup: i in [j + delta - hi_off, j + delta - lo_off].
  const int k_last = min(k0 + C::BK, a.Skv) - 1;
  const int ilo = max(0, k0 + a.delta - a.hi_off);
  const int ihi = min(a.Sq - 1, k_last + a.delta - a.lo_off);
  int diag = k0 + a.delta;
  diag = diag < 0 ? 0 : diag / a.q_vblock;
  const int nqvb = a.n_qvblocks;
  if (diag >= nqvb) diag = nqvb - 1;
  // One row block and a left window: the walk is phased so that neighbouring key tiles
  // read the query rows they share at about the same time.  With n step tiles, it starts
  // at the tile whose index (row / BQ) is a multiple of n and wraps round; away from the
  // sequence ends every key tile has the same n, so a row is reached at the same
  // position (row / BQ mod n) of every walk that reads it, and the L2 the neighbours share
  // serves all but its first read.  The walk is presented to the iterator as two row
  // blocks, [mid, 2 mid) visited before [0, mid).
  int it_nvb = nqvb, it_qvb = a.q_vblock, it_diag = diag;
  if (nqvb == 1 && a.lo_off > -kPosInf && ilo <= ihi) {
    const int t0 = ilo / C::BQ, n = ihi / C::BQ - t0 + 1;
    const int first = (n - t0 % n) % n;
    const int mid = (t0 + first) * C::BQ;
    if (first > 0 && 2 * mid > ihi) {
      it_nvb = 2;
      it_qvb = mid;
      it_diag = 1;
    }
  }
  QueryTileIter<C::BQ> qit;
  int hh = split * g_per;
  const int hh_end = hh + g_per;
  qit.init(it_nvb, it_qvb, it_diag, ilo, ihi);
  auto next_step = [&](int& hq_o, int& qs, int& rend) -> bool {
    while (hh < hh_end) {
      if (qit.next(qs, rend)) {
        hq_o = hkv * a.G + hh;
        return true;
      }
      ++hh;
      qit.init(it_nvb, it_qvb, it_diag, ilo, ihi);
    }
    return false;
  };

  const bool wave_on = kw0 < a.Skv;
  const int w_klast = kw0 + 31;

  // Step tile copies: instruction n fills bytes [1024n, 1024n + 1024) of the Q buffer
  // (n < QI) or of the dO buffer (n - QI); lane l carries 16-byte slot 64n' + l.  Wave w
  // issues instructions w, w + 4, ...
  uint32_t cpo[C::NI];
  bool cpv[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int n = wave + 4 * i;
    const bool is_q = n < C::QI;
    const int sl = 64 * (is_q ? n : n - C::QI) + lane;
    const int gs = is_q ? C::QGS : C::GGS, ps = is_q ? C::QPS : C::GPS;
    const int grp = sl / gs, rem = sl - grp * gs, k4 = rem / ps, ch = rem - k4 * ps;
    const int r = 4 * grp + k4;
    cpv[i] = n < C::QI + C::GI && k4 < 4 && ch < (is_q ? C::DC : C::DCV) && r < C::BQ;
    cpo[i] = (uint32_t)r * (is_q ? q_rs_b : g_rs_b) + 16u * ch;
  }
  float lbuf = 0.f;
  uint32_t dbuf = 0u;
  auto load_step = [&](int hq_, int qs, int buf) {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc_at(
        qbase, q_bytes, __builtin_amdgcn_readfirstlane((uint32_t)qs * q_rs_b + (uint32_t)hq_ * D * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc_at(
        gbase, g_bytes, __builtin_amdgcn_readfirstlane((uint32_t)qs * g_rs_b + (uint32_t)hq_ * DV * 2));
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int n = wave + 4 * i;
      if (n < C::QI) {
        if (cpv[i]) dma16(rq, (buf ? sQb1 : sQb0) + 1024 * n, cpo[i]);
      } else if (n < C::QI + C::GI) {
        if (cpv[i]) dma16(rg, (buf ? sGb1 : sGb0) + 1024 * (n - C::QI), cpo[i]);
      }
    }
    if (tid < 2 * C::BQ) {
      const int i = tid & (C::BQ - 1), row = qs + i;
      const size_t st = ((size_t)b * a.Hq + hq_) * a.Sq + row;
      lbuf = row < a.Sq ? (tid < C::BQ ? a.lse2[st] : a.Dvec[st]) : (tid < C::BQ ? INFINITY : 0.f);
    }
    if constexpr (DROP) {
      if (tid < 4 * C::BQ) {   // word of row qs + tid % BQ for the keys of wave tid / BQ
        const int i = min(qs + (tid % C::BQ), a.Sq - 1);
        const int kw = min(k0 + 32 * (tid / C::BQ), a.Skv - 1) >> 5;
        dbuf = a.drop[b * a.ds_b + hq_ * a.ds_h + (long long)i * a.ds_i + kw];
      }
    }
  };
  // After this wave's copies of a step have landed: its row statistics (and dropout words).
  auto store_step = [&](int buf) {
    if (tid < C::BQ) sLse[buf][tid] = lbuf;
    else if (tid < 2 * C::BQ) sD[buf][tid - C::BQ] = lbuf;
    if constexpr (DROP) {
      if (tid < 4 * C::BQ) sDrop[buf][tid] = dbuf;
    }
  };
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_off = C::QL::idx(4 * (tg >> 1) + (tj >> 2), 16 * (tg & 1) + 4 * (tj & 3));
  const int gtr_off = C::GL::idx(4 * (tg >> 1) + (tj >> 2), 16 * (tg & 1) + 4 * (tj & 3));
  const int q_off = C::QL::idx(li, 8 * lh);
  const int g_off = C::GL::idx(li, 8 * lh);
  const int v_off = C::VL::idx(wave * 32 + li, 8 * lh);

  // With a bias, S accumulates onto bias / scale.  A bias without a row stride (bs_i == 0,
  // e.g. key padding) is one value per lane and q head, fetched a step ahead (bkey);
  // otherwise the step's 16 row values are read into s at the top of the step, before the
  // next step's copies are issued.  Rows past the step's end read row qs and are masked.
  const bool bias_rows = BIAS && a.bs_i != 0;
  auto bias_ptr = [&](int hq_) {
    return a.bias + b * a.bs_b + hq_ * a.bs_h + (long long)min(key, a.Skv - 1) * a.bs_j;
  };
  float bkey = 0.f;
  int hq = 0, qs = 0, rend = 0;
  bool have = next_step(hq, qs, rend);
  if (have) {
    load_step(hq, qs, 0);
    wait_vmcnt0();
    store_step(0);
    if (BIAS && !bias_rows) bkey = *bias_ptr(hq);
  }
  __syncthreads();
  // One query step on buffer CUR (the next step's rows go to the other one).
  auto step = [&](auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    int nhq = 0, nqs = 0, nrend = 0;
    const bool nhave = next_step(nhq, nqs, nrend);

    const int qe = min(rend, a.Sq);   // rows >= qe are not part of this step
    // pair (i, j) visible iff lo_off <= j - i + delta <= hi_off
    const int dmin = kw0 - (qs + C::BQ - 1) + a.delta;   // smallest j - i + delta in the step
    const int dmax = w_klast - qs + a.delta;             // largest
    const bool empty = !wave_on || dmax < a.lo_off || dmin > a.hi_off || qs >= qe;
    f32x16 s;
    if ((BIAS || DROP) && !empty) {
      if (bias_rows) {
        bias_fetch16(s, bias_ptr(hq), a.bs_i, qs + 4 * lh, qe - 1, qs, false);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = BIAS ? bkey : 0.f;
      }
      if constexpr (DROP) {
        // dropped pairs start the S accumulation at -inf: lane (key li) holds rows
        // 8g + 4lh + e of the step, bit li of their words
        const uint32_t* dw = &sDrop[cur][wave * C::BQ];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 w4 = *(const u32x4*)(dw + 8 * g + 4 * lh);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * g + e] = drop_if(s[4 * g + e], w4[e], li);
        }
      }
    }
    if (nhave) load_step(nhq, nqs, cur ^ 1);
    if (BIAS && !bias_rows && nhave) bkey = *bias_ptr(nhq);
    if (!empty) {
      const bool full = dmin >= a.lo_off && dmax <= a.hi_off && qs + C::BQ <= qe;
      const __bf16* qt_ = (const __bf16*)(cur ? sQb1 : sQb0);
      const __bf16* gt_ = (const __bf16*)(cur ? sGb1 : sGb0);
      f32x16 dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = (BIAS || DROP) ? s[r] * a.inv_scale : 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        s = mfma32(*(const bf16x8*)&qt_[q_off + 16 * kk], kreg[kk], s);
        if (kk < C::KSV) {
          const bf16x8 vb = *(const bf16x8*)&sVk[v_off + 16 * kk];
          dp = mfma32(*(const bf16x8*)&gt_[g_off + 16 * kk], vb, dp);
        }
      }
      if (!full) {
        cold_path();
        // row i = qs + 4lh + ioff is visible iff ilo_v <= i <= ihi_v (rows that see key)
        const int ilo_v = max(key + a.delta - a.hi_off, qs);
        const int ihi_v = min(key + a.delta - a.lo_off, qe - 1);
        const uint32_t span = (uint32_t)(ihi_v - ilo_v);
        const int base = qs + 4 * lh - ilo_v;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ioff = 8 * (r >> 2) + (r & 3);
          if (ihi_v < ilo_v || (uint32_t)(base + ioff) > span) s[r] = -INFINITY;
        }
      }
      // lane (key li) holds query rows i = 8g + 4lh + e, r = 4g + e
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lse4 = *(const f32x4*)&sLse[cur][8 * g + 4 * lh];
        const f32x4 d4 = *(const f32x4*)&sD[cur][8 * g + 4 * lh];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float p = fast_exp2(fmaf(s[r], a.scale_log2, -lse4[e]));
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]);
        }
      }
      // P and dS as the B operands of dV^T += dO^T P and dK^T += Q^T dS, 8 keys' worth
      // of query rows (one k-step) at a time.  With a bias they also enter through their
      // low parts x - bf16(x): a bias can give a few keys most of the attention of many
      // (row, head) pairs, and their dV and dK then sum hundreds of large terms whose
      // bf16 roundings alone would leave the bf16 bound.  That form packs each k-step
      // just before its products, which keeps it within the register budget.
      auto products = [&](int ks, const u32x4& pw, const u32x4& sw) {
        const bf16x8 pbf = as_bf16x8(pw), sbf = as_bf16x8(sw);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          if (db < C::DBV) {
            const int o0 = gtr_off + C::GL::rows(16 * ks) + 32 * db, o1 = o0 + C::GL::rows(8);
            const bf16x8 ga = join_bf16x8(lds_read_tr16(&gt_[o0]), lds_read_tr16(&gt_[o1]));
            dv[db] = mfma32(ga, pbf, dv[db]);
          }
          const int o0 = tr_off + C::QL::rows(16 * ks) + 32 * db, o1 = o0 + C::QL::rows(8);
          const bf16x8 qa = join_bf16x8(lds_read_tr16(&qt_[o0]), lds_read_tr16(&qt_[o1]));
          dk[db] = mfma32(qa, sbf, dk[db]);
        }
      };
      if constexpr (BIAS) {
        // (P's pair and its dV products first, then dS's pair and its dK products: only
        // one pair is live at a time.)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 hw, lw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = s[8 * ks + 2 * w], p1 = s[8 * ks + 2 * w + 1];
            hw[w] = pack_bf16x2(p0, p1);
            lw[w] = pack_bf16x2(p0 - bf16_lo(hw[w]), p1 - bf16_hi(hw[w]));
          }
#pragma unroll
          for (int db = 0; db < C::DBV; ++db) {
            const int o0 = gtr_off + C::GL::rows(16 * ks) + 32 * db, o1 = o0 + C::GL::rows(8);
            const bf16x8 ga = join_bf16x8(lds_read_tr16(&gt_[o0]), lds_read_tr16(&gt_[o1]));
            dv[db] = mfma32(ga, as_bf16x8(hw), dv[db]);
            dv[db] = mfma32(ga, as_bf16x8(lw), dv[db]);
          }
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float d0 = dp[8 * ks + 2 * w], d1 = dp[8 * ks + 2 * w + 1];
            hw[w] = pack_bf16x2(d0, d1);
            lw[w] = pack_bf16x2(d0 - bf16_lo(hw[w]), d1 - bf16_hi(hw[w]));
          }
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int o0 = tr_off + C::QL::rows(16 * ks) + 32 * db, o1 = o0 + C::QL::rows(8);
            const bf16x8 qa = join_bf16x8(lds_read_tr16(&qt_[o0]), lds_read_tr16(&qt_[o1]));
            dk[db] = mfma32(qa, as_bf16x8(hw), dk[db]);
            dk[db] = mfma32(qa, as_bf16x8(lw), dk[db]);
          }
        }
      } else {
        u32x4 pb[2], sb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[ks][w] = pack_bf16x2(s[8 * ks + 2 * w], s[8 * ks + 2 * w + 1]);
            sb[ks][w] = pack_bf16x2(dp[8 * ks + 2 * w], dp[8 * ks + 2 * w + 1]);
          }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) products(ks, pb[ks], sb[ks]);
      }
    }
    if (nhave) {
      wait_vmcnt0();                 // this wave's copies of the next step have landed
      store_step(cur ^ 1);
    }
    __syncthreads();
    hq = nhq;
    qs = nqs;
    rend = nrend;
    have = nhave;
  };
  while (have) {
    step(IntConst<0>{});
    if (!have) break;
    step(IntConst<1>{});
  }

  if (key_ok && a.kv_splits > 1) {
    // fp32 partials of this split: [ns, B, Skv, Hkv, D] then [ns, B, Skv, Hkv, Dv]
    const size_t nk = (size_t)a.B * a.Skv * k_rs, nv = (size_t)a.B * a.Skv * v_rs;
    float* pk = a.dkv_part + split * nk + koff;
    float* pv = a.dkv_part + a.kv_splits * nk + split * nv + voff;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = dk[db][4 * g + e] * a.scale;
        *(f32x4*)(pk + 32 * db + 8 * g + 4 * lh) = w;
      }
#pragma unroll
    for (int db = 0; db < C::DBV; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = dv[db][4 * g + e];
        *(f32x4*)(pv + 32 * db + 8 * g + 4 * lh) = w;
      }
  } else if (key_ok && a.accumulate) {
    // fp32 dk, dv of the caller, added into
    float* kop = (float*)a.dk + koff;
    float* vop = (float*)a.dv + voff;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4* p = (f32x4*)(kop + 32 * db + 8 * g + 4 * lh);
        f32x4 w = *p;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += dk[db][4 * g + e] * a.scale;
        *p = w;
      }
#pragma unroll
    for (int db = 0; db < C::DBV; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4* p = (f32x4*)(vop + 32 * db + 8 * g + 4 * lh);
        f32x4 w = *p;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] += dv[db][4 * g + e];
        *p = w;
      }
  } else if (key_ok) {
    __bf16* kop = (__bf16*)a.dk + koff;
    __bf16* vop = (__bf16*)a.dv + voff;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk;
        wk[0] = pack_bf16x2(dk[db][4 * g] * a.scale, dk[db][4 * g + 1] * a.scale);
        wk[1] = pack_bf16x2(dk[db][4 * g + 2] * a.scale, dk[db][4 * g + 3] * a.scale);
        *(u32x2*)(kop + 32 * db + 8 * g + 4 * lh) = wk;
      }
#pragma unroll
    for (int db = 0; db < C::DBV; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wv;
        wv[0] = pack_bf16x2(dv[db][4 * g], dv[db][4 * g + 1]);
        wv[1] = pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3]);
        *(u32x2*)(vop + 32 * db + 8 * g + 4 * lh) = wv;
      }
  }
}

// Sum of the kv_splits fp32 partials of dk (n_k elements) and dv (n_v elements), in split
// order (so the result is bitwise reproducible), rounded once to bf16 (or, accumulating,
// added into the caller's fp32 dk, dv).  4 elements per thread; n_k and n_v are multiples
// of 4 (head dims are multiples of 32).
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* part, int ns, long long n_k,
                                                              long long n_v, void* dk, void* dv, int rev,
                                                              int accumulate) {
  const long long i = 4 * ((long long)wg_index(rev) * 256 + threadIdx.x);
  if (i >= n_k + n_v) return;
  const bool is_k = i < n_k;
  const float* src = is_k ? part + i : part + ns * n_k + (i - n_k);
  const long long stride = is_k ? n_k : n_v;
  f32x4 s = *(const f32x4*)src;
  for (int j = 1; j < ns; ++j) {
    const f32x4 t = *(const f32x4*)(src + j * stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += t[e];
  }
  if (accumulate) {          // fp32 outputs of the caller, added into
    f32x4* p = (f32x4*)(is_k ? (float*)dk + i : (float*)dv + (i - n_k));
    f32x4 o = *p;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += s[e];
    *p = o;
    return;
  }
  u32x2 w;
  w[0] = pack_bf16x2(s[0], s[1]);
  w[1] = pack_bf16x2(s[2], s[3]);
  *(u32x2*)(is_k ? (__bf16*)dk + i : (__bf16*)dv + (i - n_k)) = w;
}

// Gradient of the learnable sink logits: dz_h = -sum over (b, i) of P_sink,i * D_i, with
// P_sink,i = exp(z_h - LSE_i) (the LSE includes the sink) and D_i = rowsum(dO * O), both
// left in the workspace by the D / LSE pass.  One workgroup per q head; each thread sums
// a fixed strided subset and the workgroup a fixed tree, so the result is reproducible.
__global__ __launch_bounds__(256) void bwd_sink_grad_kernel(BwdArgs a) {
  __shared__ float red[256];
  const int h = wg_index(a.rev_order), tid = threadIdx.x;
  const float zz = a.sink[h] * kLog2e;
  float acc = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const size_t base = ((size_t)b * a.Hq + h) * a.Sq;
    for (int i = tid; i < a.Sq; i += 256) acc -= exp2f(zz - a.lse2[base + i]) * a.Dvec[base + i];
  }
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) a.dsink[h] = a.accumulate ? a.dsink[h] + red[0] : red[0];
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 kernels (small head dims): one thread per query row for dq, one thread
// per key row for dk/dv; tiles of the other side staged in LDS.
template <int D, int DV>
__global__ __launch_bounds__(128) void bwd_dq_f32_kernel(BwdArgs a) {
  constexpr int BM = 128, BN = 32;
  __shared__ float sK[BN][D + 1], sV[BN][DV + 1];
  int b, hq, qt;
  map_task(wg_index(a.rev_order), a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, 0, false, b, hq, qt);
  const int hkv = hq / a.G, tid = threadIdx.x;
  const int row = qt * BM + tid;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D, k_rs = (size_t)a.Hkv * D;
  const size_t o_rs = (size_t)a.Hq * DV, v_rs = (size_t)a.Hkv * DV;
  const size_t qoff = ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
  const size_t goff = ((size_t)b * a.Sq + row) * o_rs + (size_t)hq * DV;
  const float* kp = (const float*)a.k + (size_t)b * a.Skv * k_rs + (size_t)hkv * D;
  const float* vp = (const float*)a.v + (size_t)b * a.Skv * v_rs + (size_t)hkv * DV;
  float qr[D], gr[DV], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = row_ok ? ((const float*)a.q)[qoff + d] : 0.f;
    acc[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DV; ++d) gr[d] = row_ok ? ((const float*)a.dout)[goff + d] : 0.f;
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  const float lse2 = row_ok ? a.lse2[stat] : INFINITY;
  const float Di = row_ok ? a.Dvec[stat] : 0.f;
  const int wg_row0 = qt * BM, r_last = min(wg_row0 + BM, a.Sq) - 1;
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
    for (int r = 0; r < BN; ++r) {
      const int j = ts + r;
      if (j < my_jmin || j > my_jmax || j >= tend) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], sK[r][d], s);
#pragma unroll
      for (int d = 0; d < DV; ++d) dp = fmaf(gr[d], sV[r][d], dp);
      // rows past the end (not stored) read the last row's bias / dropout bits
      const int rc = min(row, a.Sq - 1);
      if (a.bias)
        s = fmaf(a.bias[b * a.bs_b + hq * a.bs_h + (long long)rc * a.bs_i + (long long)j * a.bs_j], a.inv_scale, s);
      if (a.drop && dropped(a.drop, b * a.ds_b + hq * a.ds_h, a.ds_i, rc, j)) s = -INFINITY;
      const float p = fast_exp2(fmaf(s, a.scale_log2, -lse2));
      const float ds = p * (dp - Di);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, sK[r][d], acc[d]);
    }
    __syncthreads();
  }
  if (row_ok) {
    float* op = (float*)a.dq + qoff;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = (a.accumulate ? op[d] : 0.f) + acc[d] * a.scale;
  }
}

template <int D, int DV, int EX>
__global__ __launch_bounds__(128) void bwd_dkdv_f32_kernel(BwdArgs a) {
  constexpr int BK = 128, BQ = 32;
  __shared__ float sQ[BQ][D + 1], sG[BQ][DV + 1], sL[BQ], sDv[BQ];
  int b, hkv, kt;
  map_kv_task(wg_index(a.rev_order), a.n_ktiles, a.B, a.Hkv, 0, false, b, hkv, kt);
  const int tid = threadIdx.x;
  const int key = kt * BK + tid;
  const bool key_ok = key < a.Skv;
  const size_t q_rs = (size_t)a.Hq * D, k_rs = (size_t)a.Hkv * D;
  const size_t o_rs = (size_t)a.Hq * DV, v_rs = (size_t)a.Hkv * DV;
  const size_t koff = ((size_t)b * a.Skv + key) * k_rs + (size_t)hkv * D;
  const size_t voff = ((size_t)b * a.Skv + key) * v_rs + (size_t)hkv * DV;
  float kr[D], vr[DV], dk[D], dv[DV];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = key_ok ? ((const float*)a.k)[koff + d] : 0.f;
    dk[d] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DV; ++d) {
    vr[d] = key_ok ? ((const float*)a.v)[voff + d] : 0.f;
    dv[d] = 0.f;
  }
  const int k0 = kt * BK, k_last = min(k0 + BK, a.Skv) - 1;
  const int ilo = max(0, k0 + a.delta - a.hi_off);
  const int ihi = min(a.Sq - 1, k_last + a.delta - a.lo_off);
  int diag = k0 + a.delta;
  diag = diag < 0 ? 0 : diag / a.q_vblock;
  const int nqvb = a.n_qvblocks;
  if (diag >= nqvb) diag = nqvb - 1;
  for (int hh = 0; hh < a.G; ++hh) {
    const int hq = hkv * a.G + hh;
    const float* qp = (const float*)a.q + (size_t)b * a.Sq * q_rs + (size_t)hq * D;
    const float* gp = (const float*)a.dout + (size_t)b * a.Sq * o_rs + (size_t)hq * DV;
    QueryTileIter<BQ> qit;
    qit.init(nqvb, a.q_vblock, diag, ilo, ihi);
    int qs, rend;
    while (qit.next(qs, rend)) {
      const int qe = min(rend, a.Sq);
      for (int c = tid; c < BQ * D; c += BK) {
        const int r = c / D, d = c % D, row = qs + r;
        sQ[r][d] = row < a.Sq ? qp[(size_t)row * q_rs + d] : 0.f;
      }
      for (int c = tid; c < BQ * DV; c += BK) {
        const int r = c / DV, d = c % DV, row = qs + r;
        sG[r][d] = row < a.Sq ? gp[(size_t)row * o_rs + d] : 0.f;
      }
      if (tid < BQ) {
        const int row = qs + tid;
        const size_t st = ((size_t)b * a.Hq + hq) * a.Sq + row;
        sL[tid] = row < a.Sq ? a.lse2[st] : INFINITY;
        sDv[tid] = row < a.Sq ? a.Dvec[st] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < BQ; ++r) {
        const int i = qs + r;
        const int dd = key - i + a.delta;
        if (i >= qe || dd < a.lo_off || dd > a.hi_off) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(sQ[r][d], kr[d], s);
#pragma unroll
        for (int d = 0; d < DV; ++d) dp = fmaf(sG[r][d], vr[d], dp);
        // keys past the end (not stored) read the last key's bias / dropout bits
        const int kc = min(key, a.Skv - 1);
        if ((EX & 1) && a.bias)
          s = fmaf(a.bias[b * a.bs_b + hq * a.bs_h + (long long)i * a.bs_i + (long long)kc * a.bs_j], a.inv_scale, s);
        if ((EX & 2) && a.drop && dropped(a.drop, b * a.ds_b + hq * a.ds_h, a.ds_i, i, kc)) s = -INFINITY;
        const float p = fast_exp2(fmaf(s, a.scale_log2, -sL[r]));
        const float ds = p * (dp - sDv[r]);
#pragma unroll
        for (int d = 0; d < D; ++d) dk[d] = fmaf(ds, sQ[r][d], dk[d]);
#pragma unroll
        for (int d = 0; d < DV; ++d) dv[d] = fmaf(p, sG[r][d], dv[d]);
      }
      __syncthreads();
    }
  }
  if (key_ok) {
#pragma unroll
    for (int d = 0; d < D; ++d) ((float*)a.dk)[koff + d] = (a.accumulate ? ((float*)a.dk)[koff + d] : 0.f) + dk[d] * a.scale;
#pragma unroll
    for (int d = 0; d < DV; ++d) ((float*)a.dv)[voff + d] = (a.accumulate ? ((float*)a.dv)[voff + d] : 0.f) + dv[d];
  }
}

// Smallest number of query rows a dq workgroup covers (for the host-side size checks).
int bwd_q_tile_rows(int dtype) { return dtype == 0 ? 32 : 128; }
int bwd_k_tile_rows(int dtype) { return dtype == 0 ? BwdKVCfg<128, 128>::BK : 128; }

template <typename T, int D>
static void launch_pre(const BwdArgs& a, hipStream_t stream) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  constexpr int RPB = 256 / LPR;
  const long long nrows = (long long)a.B * a.Sq * a.Hq;
  const unsigned blocks = (unsigned)((nrows + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, a);
}

// Workgroup shape of the bf16 dq kernel.  The 4-wave form (32-key tiles, two workgroups
// per CU) measured faster for every window tried (128 to 3000 keys wide) and for causal
// attention with fewer than 8 q heads per kv head; with 8 or more heads sharing each K/V
// tile, or with dropout (whose words cost more loads per key in 32-key tiles), the 8-wave
// ping-pong is ahead.
static bool dq_use_w4(const BwdArgs& a) {
  return (a.lo_off > -kPosInf && a.hi_off < kPosInf) || (a.G < 8 && a.drop == nullptr);
}

hipError_t launch_bwd(int dtype, const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  dim3 gq((unsigned)a.n_qtiles * a.B * a.Hq), bq(128);
  // bf16 dq workgroups: 8 waves (ping-pong, one per CU) or 4 waves (two per CU), chosen
  // by dq_use_w4; gh q heads of one GQA group x 32 * waves / gh rows.
  const bool w4 = dq_use_w4(a);
  if (dtype == 0) {
    const int nw = w4 ? 4 : 8, max_shift = w4 ? 2 : 3;
    a.gh_shift = 0;
    while (a.gh_shift < max_shift && a.G % (2 << a.gh_shift) == 0) ++a.gh_shift;
    a.gh = 1 << a.gh_shift;
    a.rows_wg = (32 * nw) >> a.gh_shift;
    a.n_hg = a.Hq >> a.gh_shift;
    a.n_qtiles = (a.Sq + a.rows_wg - 1) / a.rows_wg;
    gq = dim3((unsigned)a.n_qtiles * a.B * a.n_hg);
    bq = dim3(64 * nw);
  }
  const dim3 gk((unsigned)a.n_ktiles * a.B * a.Hkv * a.kv_splits), bk(dtype == 0 ? 256 : 128);
  const bool has_q = gq.x > 0, has_k = gk.x > 0;
  const bool want_pre = has_q && (a.stages & 1), dq = has_q && (a.stages & 2), dkdv = has_k && (a.stages & 4);
  // The bf16 dq kernel computes D and the LSE itself when they are needed.
  a.fused_stats = (dtype == 0 && want_pre && dq) ? 1 : 0;
  const bool pre = want_pre && !a.fused_stats;
  const int ex = (a.bias ? 1 : 0) | (a.drop ? 2 : 0);   // extra logit terms compiled in
  // D and the LSE: rows of o and dout have the v head dim.
#define REA_BWD(T, DD, DDV, DQ_LAUNCH, DKV)                                       \
  do {                                                                          \
    if (pre) launch_pre<T, DDV>(a, stream);                                     \
    if (dq) DQ_LAUNCH;                                                          \
    if (dkdv) {                                                                 \
      switch (ex) {                                                             \
        case 1: hipLaunchKernelGGL((DKV<DD, DDV, 1>), gk, bk, 0, stream, a); break; \
        case 2: hipLaunchKernelGGL((DKV<DD, DDV, 2>), gk, bk, 0, stream, a); break; \
        case 3: hipLaunchKernelGGL((DKV<DD, DDV, 3>), gk, bk, 0, stream, a); break; \
        default: hipLaunchKernelGGL((DKV<DD, DDV, 0>), gk, bk, 0, stream, a);      \
      }                                                                         \
      if (a.kv_splits > 1) {                                                    \
        const long long nk = (long long)a.B * a.Skv * a.Hkv * a.D;              \
        const long long nv = (long long)a.B * a.Skv * a.Hkv * a.Dv;             \
        const unsigned blocks = (unsigned)((nk + nv + 1023) / 1024);            \
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3(blocks), dim3(256), 0,  \
                           stream, a.dkv_part, a.kv_splits, nk, nv,             \
                           a.dk, a.dv, a.rev_order, a.accumulate);              \
      }                                                                         \
    }                                                                           \
  } while (0)
#define REA_DQ_BF16_EX(DD, DDV, EXV)                                                          \
  do {                                                                                     \
    if (w4) hipLaunchKernelGGL((bwd_dq_bf16_kernel<DD, DDV, 4, EXV>), gq, bq, 0, stream, a); \
    else hipLaunchKernelGGL((bwd_dq_bf16_kernel<DD, DDV, 8, EXV>), gq, bq, 0, stream, a);    \
  } while (0)
#define REA_DQ_BF16(DD, DDV)                                        \
  do {                                                              \
    switch (ex) {                                                   \
      case 1: REA_DQ_BF16_EX(DD, DDV, 1); break;                    \
      case 2: REA_DQ_BF16_EX(DD, DDV, 2); break;                    \
      case 3: REA_DQ_BF16_EX(DD, DDV, 3); break;                    \
      default: REA_DQ_BF16_EX(DD, DDV, 0);                          \
    }                                                               \
  } while (0)
#define REA_DQ_F32(DD, DDV) hipLaunchKernelGGL((bwd_dq_f32_kernel<DD, DDV>), gq, bq, 0, stream, a)
  if (!head_dims_supported(dtype, a.D, a.Dv)) return hipErrorInvalidValue;
  const int dd = a.D * 1000 + a.Dv;
  if (dtype == 0) {
    switch (dd) {
      case 32032: REA_BWD(__bf16, 32, 32, REA_DQ_BF16(32, 32), bwd_dkdv_bf16_kernel); break;
      case 64064: REA_BWD(__bf16, 64, 64, REA_DQ_BF16(64, 64), bwd_dkdv_bf16_kernel); break;
      case 128128: REA_BWD(__bf16, 128, 128, REA_DQ_BF16(128, 128), bwd_dkdv_bf16_kernel); break;
      case 128064: REA_BWD(__bf16, 128, 64, REA_DQ_BF16(128, 64), bwd_dkdv_bf16_kernel); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (dd) {
      case 32032: REA_BWD(float, 32, 32, REA_DQ_F32(32, 32), bwd_dkdv_f32_kernel); break;
      case 64064: REA_BWD(float, 64, 64, REA_DQ_F32(64, 64), bwd_dkdv_f32_kernel); break;
      case 64032: REA_BWD(float, 64, 32, REA_DQ_F32(64, 32), bwd_dkdv_f32_kernel); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef REA_DQ_F32
  // The sink gradient needs D and the LSE of every row: after the pass that wrote them.
  if (a.dsink && a.sink && has_q && (want_pre || dq))
    hipLaunchKernelGGL(bwd_sink_grad_kernel, dim3(a.Hq), dim3(256), 0, stream, a);
#undef REA_DQ_BF16
#undef REA_DQ_BF16_EX
#undef REA_BWD
  return hipGetLastError();
}

}  // namespace rea
