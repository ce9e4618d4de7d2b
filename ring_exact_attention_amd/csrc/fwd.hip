// Forward pass of blockwise exact attention on gfx950.
//
// Method ("bpt.py", _blockwise_attention_fwd inside _ring_attention_fwd): a query tile
// walks the key tiles it can see, in ring order over the virtual key blocks, keeping a
// running max m, denominator l and unnormalised numerator acc; each tile rescales the
// carry by exp(m_old - m_new) before adding exp(s - m_new) and exp(s - m_new) V.  Masks
// follow _chunk_attention_bias (causal) and the TransformerEngine page's
// _make_causal_swa_mask (window), on global positions.
//
// gfx950 mapping (bf16): one workgroup = 4 wavefronts = 128 query rows of one
// (batch, q head); each wave owns 32 rows.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so that each lane owns one query row
// (column of the accumulator): the row max / sum need one cross-half exchange, and
// the probabilities P^T are already in the B-operand layout of O^T = V^T P^T.
// K and V tiles are fetched with raw buffer loads (rows past the end read as zero) and
// staged row-major in LDS at a pitch of D + 32 elements, double-buffered through
// registers.  K feeds S^T with 16-byte reads; the transposed V operand of O^T is read
// with ds_read_b64_tr_b16, in the key order of the score accumulator.  Both read
// patterns are free of LDS bank conflicts at that pitch.
// Accumulation is fp32; exp uses v_exp_f32 on logits pre-scaled by scale*log2(e).  The
// carry is rescaled only when a row max grows by more than 2^8 (exact: numerator and
// denominator share the stale reference), and the stored statistics use the exact max.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace rea {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;                   // query rows per workgroup
  static constexpr int BN = 64;                    // keys per tile
  static constexpr int KS = D / 16;                // k-steps of S^T over d
  static constexpr int DB = D / 32;                // 32-row blocks of O^T
  using KL = TileLayout<D, kRowRead>;              // K tile: read as row operands
  using VL = TileLayout<D, kTrRead>;               // V tile: read transposed
  static constexpr int DC = D / 8;                 // 16-byte chunks per row
  static constexpr int LPT = BN * DC / 256;        // 16-byte chunks per thread per tile and tensor
};

// Rows of the scores may grow by this much (log2 units) before the carry is rescaled.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][C::KL::elems(C::BN)];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][C::VL::elems(C::BN)];

  int b, hq, qt;
  map_task(blockIdx.x, a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, a.xcd_groups, a.hi_off < kPosInf, b, hq, qt);
  const int hkv = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int wg_row0 = qt * C::BM;
  const int row0 = wg_row0 + wave * 32;
  const int row = row0 + li;
  const bool row_ok = row < a.Sq;

  const size_t q_rs = (size_t)a.Hq * D;
  const uint32_t kv_rs_b = (uint32_t)a.Hkv * D * 2;           // bytes between key rows
  const __bf16* qp = (const __bf16*)a.q + (size_t)b * a.Sq * q_rs + (size_t)hq * D;
  const size_t kv_base = ((size_t)b * a.Skv * a.Hkv + hkv) * D;
  const uint32_t kv_bytes = a.Skv > 0 ? (uint32_t)(a.Skv - 1) * kv_rs_b + D * 2 : 0;
  const __bf16* kbase = (const __bf16*)a.k + kv_base;
  const __bf16* vbase = (const __bf16*)a.v + kv_base;

  // Q^T as B operands: lane (li, lh) holds q[row][16kk + 8lh .. +7].
  bf16x8 qreg[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (row_ok) u = *(const u32x4*)(qp + (size_t)row * q_rs + 16 * kk + 8 * lh);
    qreg[kk] = as_bf16x8(u);
  }

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
  float* accp = a.acc ? a.acc + ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D : nullptr;
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
  const int r_last_wg = min(wg_row0 + C::BM, a.Sq) - 1;
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

  // Staging: thread t moves 16-byte chunks c = t + 256u (row c / DC, chunk c % DC).
  u32x4 kbuf[C::LPT], vbuf[C::LPT];
  uint32_t goff[C::LPT];
  constexpr int RPU = 256 / C::DC;                  // rows per staging round (multiple of 4)
#pragma unroll
  for (int u = 0; u < C::LPT; ++u) goff[u] = (uint32_t)(tid / C::DC + RPU * u) * kv_rs_b + 16u * (tid % C::DC);
  const int kl0 = C::KL::idx(tid / C::DC, 8 * (tid % C::DC));
  const int vl0 = C::VL::idx(tid / C::DC, 8 * (tid % C::DC));
  auto load_tile = [&](int ts) {
    const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)ts * kv_rs_b);   // uniform
    const __amdgpu_buffer_rsrc_t rk = make_rsrc_at(kbase, kv_bytes, so);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc_at(vbase, kv_bytes, so);
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      kbuf[u] = buf_load16(rk, goff[u], 0);
      vbuf[u] = buf_load16(rv, goff[u], 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      *(u32x4*)&sK[buf][kl0 + C::KL::rows(RPU * u)] = kbuf[u];
      *(u32x4*)&sV[buf][vl0 + C::VL::rows(RPU * u)] = vbuf[u];
    }
  };
  // Transposed V operand: lane (group g = lane/16, j = lane%16) points at
  // V[16c + 4(g>>1) + j/4 (+8)][32db + 16(g&1) + 4(j%4) ..+3].
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_off = C::VL::idx(4 * (tg >> 1) + (tj >> 2), 16 * (tg & 1) + 4 * (tj & 3));
  const int k_off = C::KL::idx(li, 8 * lh);

  int ts = 0, kend = 0;
  bool have = it.next(ts, kend);
  if (have) {
    load_tile(ts);
    store_tile(0);
  }
  __syncthreads();
  int cur = 0;
  while (have) {
    int nts = 0, nkend = 0;
    const bool nhave = it.next(nts, nkend);
    if (nhave) load_tile(nts);

    const int tend = min(kend, a.Skv);            // keys >= tend are not in this visit
    const bool empty = !wave_on || ts > w_jmax_hi || tend - 1 < w_jmin_lo;
    if (!empty) {
      const bool full = ts >= w_jmin_hi && ts + C::BN - 1 <= w_jmax_lo && ts + C::BN <= tend;
      const __bf16* kt = sK[cur];
      const __bf16* vt = sV[cur];
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)        // two independent accumulation chains
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 ka = *(const bf16x8*)&kt[k_off + C::KL::rows(32 * mb) + 16 * kk];
          s[mb] = mfma32(ka, qreg[kk], s[mb]);
        }
      if (!full) {
        cold_path();
        // key j = ts + 4lh + koff is visible iff jlo_v <= j <= jhi_v: one unsigned compare
        const int jlo_v = max(my_jmin, ts), jhi_v = min(my_jmax, tend - 1);
        const uint32_t span = (uint32_t)(jhi_v - jlo_v);
        const int base = ts + 4 * lh - jlo_v;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = 32 * mb + 8 * (r >> 2) + (r & 3);
            if (jhi_v < jlo_v || (uint32_t)(base + koff) > span) s[mb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = fmaxf(mx, other_half(mx));
      const float mt = mx * a.scale_log2;          // this tile's row max (log2 units)
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
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[mb][r], a.scale_log2, -m_ref));
          s[mb][r] = p;
          rs += p;
        }
      l_part += rs;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 pb;
#pragma unroll
          for (int w = 0; w < 4; ++w) pb[w] = pack_bf16x2(s[mb][8 * ks + 2 * w], s[mb][8 * ks + 2 * w + 1]);
          const bf16x8 pbf = as_bf16x8(pb);
          const int c = 2 * mb + ks;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const __bf16* vp0 = &vt[tr_off + C::VL::rows(16 * c) + 32 * db];
            const bf16x8 va = join_bf16x8(lds_read_tr16(vp0), lds_read_tr16(vp0 + C::VL::rows(8)));
            acc[db] = mfma32(va, pbf, acc[db]);
          }
        }
    }

    if (nhave) store_tile(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    ts = nts;
    kend = nkend;
    have = nhave;
  }

  // Normalise the statistics to the exact max: l_true = l_used * 2^(m_used - m_true).
  const float l_used = l_part + other_half(l_part);
  const float corr = (m_true == -INFINITY) ? 0.f : fast_exp2(m_used - m_true);
  if (row_ok) {
    if (a.finalize) {
      const float inv = l_used > 0.f ? 1.f / l_used : 0.f;
      __bf16* op = (__bf16*)a.o + ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
          *(u32x2*)(op + 32 * db + 8 * g + 4 * lh) = w;
        }
    } else {
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
template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BM = 128, BN = 32;
  __shared__ float sK[BN][D + 1];
  __shared__ float sV[BN][D + 1];
  int b, hq, qt;
  map_task(blockIdx.x, a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, 0, false, b, hq, qt);
  const int hkv = hq / a.G;
  const int tid = threadIdx.x;
  const int row = qt * BM + tid;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D, kv_rs = (size_t)a.Hkv * D;
  const float* qp = (const float*)a.q + (size_t)b * a.Sq * q_rs + (size_t)hq * D;
  const float* kp = (const float*)a.k + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;
  const float* vp = (const float*)a.v + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;

  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = row_ok ? qp[(size_t)row * q_rs + d] : 0.f;
    acc[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  float* accp = a.acc ? a.acc + ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D : nullptr;
  if (a.carry_in && row_ok) {
    m_run = a.m[stat] * kLog2e;
    l_run = a.l[stat];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = accp[d];
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
      sK[r][d] = j < a.Skv ? kp[(size_t)j * kv_rs + d] : 0.f;
      sV[r][d] = j < a.Skv ? vp[(size_t)j * kv_rs + d] : 0.f;
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
      s[r] = (j < my_jmin || j > my_jmax || j >= tend) ? -INFINITY : dot * a.scale_log2;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int r = 0; r < BN; ++r) {
      const float p = fast_exp2(s[r] - m_ref);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sV[r][d], acc[d]);
    }
    m_run = m_new;
    __syncthreads();
  }
  if (row_ok) {
    if (a.finalize) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      float* op = (float*)a.o + ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
#pragma unroll
      for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) accp[d] = acc[d];
    }
    a.m[stat] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
    a.l[stat] = l_run;
  }
}

int fwd_tile_rows(int dtype) { return dtype == 0 ? FwdCfg<128>::BM : 128; }

hipError_t launch_fwd(int dtype, const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.n_qtiles * a.B * a.Hq), block256(256), block128(128);
  if (dtype == 0) {
    switch (a.D) {
      case 32: hipLaunchKernelGGL(fwd_bf16_kernel<32>, grid, block256, 0, stream, a); break;
      case 64: hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block256, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block256, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.D) {
      case 32: hipLaunchKernelGGL(fwd_f32_kernel<32>, grid, block128, 0, stream, a); break;
      case 64: hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block128, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace rea
