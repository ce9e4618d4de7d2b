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
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
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
  const long long rowg = (long long)blockIdx.x * RPB + tid / LPR;   // row of [B, Sq, Hq]
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
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if (rowg < nrows && sub == 0) {
    const int h = (int)(rowg % a.Hq);
    const long long bs = rowg / a.Hq;
    const int s = (int)(bs % a.Sq), b = (int)(bs / a.Sq);
    const size_t st = ((size_t)b * a.Hq + h) * a.Sq + s;
    a.Dvec[st] = part;
    const float l = a.l[st], m = a.m[st];
    a.lse2[st] = (l > 0.f) ? fmaf(m, kLog2e, log2f(l)) : INFINITY;
  }
}

// ------------------------------------------------------------------ dq (bf16)
template <int D>
struct BwdQCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KROW = D + 8;
  static constexpr int TROW = BN + 8;
  static constexpr int KG = BN * D / 2048;
  static constexpr int DC = D / 8;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(BwdArgs a) {
  using C = BwdQCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][C::BN * C::KROW];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][C::BN * C::KROW];
  __shared__ __attribute__((aligned(16))) __bf16 sKt[2][D * C::TROW];

  int b, hq, qt;
  map_task(blockIdx.x, a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, a.xcd_groups, a.hi_off < kPosInf, b, hq, qt);
  const int hkv = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int wg_row0 = qt * C::BM;
  const int row0 = wg_row0 + wave * 32;
  const int row = row0 + li;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D, kv_rs = (size_t)a.Hkv * D;
  const size_t qoff = ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
  const __bf16* kp = (const __bf16*)a.k + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;
  const __bf16* vp = (const __bf16*)a.v + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;

  bf16x8 qreg[C::KS], doreg[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    u32x4 u = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (row_ok) {
      u = *(const u32x4*)((const __bf16*)a.q + qoff + 16 * kk + 8 * lh);
      g = *(const u32x4*)((const __bf16*)a.dout + qoff + 16 * kk + 8 * lh);
    }
    qreg[kk] = as_bf16x8(u);
    doreg[kk] = as_bf16x8(g);
  }
  const size_t stat = ((size_t)b * a.Hq + hq) * a.Sq + row;
  const float lse2 = row_ok ? a.lse2[stat] : INFINITY;
  const float Di = row_ok ? a.Dvec[stat] : 0.f;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int r_last_wg = min(wg_row0 + C::BM, a.Sq) - 1;
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

  u32x4 kbuf[C::KG], vbuf[C::KG];
  const int t_dc = tid % C::DC, t_kg = tid / C::DC;
  auto load_tile = [&](int ts) {
#pragma unroll
    for (int r = 0; r < C::KG; ++r) {
      const int j = ts + C::KG * t_kg + r;
      const bool ok = j < a.Skv;
      kbuf[r] = ok ? *(const u32x4*)(kp + (size_t)j * kv_rs + 8 * t_dc) : u32x4{0u, 0u, 0u, 0u};
      vbuf[r] = ok ? *(const u32x4*)(vp + (size_t)j * kv_rs + 8 * t_dc) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::KG; ++r) {
      const int j = C::KG * t_kg + r;
      *(u32x4*)&sK[buf][j * C::KROW + 8 * t_dc] = kbuf[r];
      *(u32x4*)&sV[buf][j * C::KROW + 8 * t_dc] = vbuf[r];
    }
    const int slot = perm_slot(C::KG * t_kg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16* dst = &sKt[buf][(8 * t_dc + e) * C::TROW + slot];
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      if constexpr (C::KG == 4) {
        u32x2 pr;
        pr[0] = __builtin_amdgcn_perm(kbuf[1][w], kbuf[0][w], sel);
        pr[1] = __builtin_amdgcn_perm(kbuf[3][w], kbuf[2][w], sel);
        *(u32x2*)dst = pr;
      } else if constexpr (C::KG == 2) {
        *(uint32_t*)dst = __builtin_amdgcn_perm(kbuf[1][w], kbuf[0][w], sel);
      } else {
        const uint32_t x = (e & 1) ? (kbuf[0][w] >> 16) : (kbuf[0][w] & 0xffffu);
        *(uint16_t*)dst = (uint16_t)x;
      }
    }
  };

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
    const int tend = min(kend, a.Skv);
    const bool empty = !wave_on || ts > w_jmax_hi || tend - 1 < w_jmin_lo;
    if (!empty) {
      const bool full = ts >= w_jmin_hi && ts + C::BN - 1 <= w_jmax_lo && ts + C::BN <= tend;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mb][r] = 0.f;
          dp[mb][r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
          const int off = (32 * mb + li) * C::KROW + 16 * kk + 8 * lh;
          s[mb] = mfma32(*(const bf16x8*)&sK[cur][off], qreg[kk], s[mb]);
          dp[mb] = mfma32(*(const bf16x8*)&sV[cur][off], doreg[kk], dp[mb]);
        }
      }
      if (!full) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = ts + 32 * mb + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (j < my_jmin || j > my_jmax || j >= tend) s[mb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[mb][r], a.scale_log2, -lse2));
          s[mb][r] = p * (dp[mb][r] - Di);
        }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int mb = c >> 1, ks = c & 1;
        u32x4 pb;
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[w] = pack_bf16x2(s[mb][8 * ks + 2 * w], s[mb][8 * ks + 2 * w + 1]);
        const bf16x8 pbf = as_bf16x8(pb);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 ka = *(const bf16x8*)&sKt[cur][(32 * db + li) * C::TROW + 16 * c + 8 * lh];
          acc[db] = mfma32(ka, pbf, acc[db]);
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

  if (row_ok) {
    __bf16* op = (__bf16*)a.dq + qoff;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * g] * a.scale, acc[db][4 * g + 1] * a.scale);
        w[1] = pack_bf16x2(acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale);
        *(u32x2*)(op + 32 * db + 8 * g + 4 * lh) = w;
      }
  }
}

// ------------------------------------------------------------------ dk, dv (bf16)
template <int D>
struct BwdKVCfg {
  static constexpr int BK = 128;                  // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 32;                   // query rows per step
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QROW = D + 8;
  static constexpr int TROW = BQ + 8;
  static constexpr int DC = D / 8;
  static constexpr int NCH = BQ * DC;             // 16-byte chunks per tensor per step
  static constexpr int CPT = (NCH + 255) / 256;   // chunks per thread
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(BwdArgs a) {
  using C = BwdKVCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][C::BQ * C::QROW];
  __shared__ __attribute__((aligned(16))) __bf16 sG[2][C::BQ * C::QROW];
  __shared__ __attribute__((aligned(16))) __bf16 sQt[2][D * C::TROW];
  __shared__ __attribute__((aligned(16))) __bf16 sGt[2][D * C::TROW];
  __shared__ __attribute__((aligned(16))) float sLse[2][C::BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BQ];

  int b, hkv, kt;
  map_kv_task(blockIdx.x, a.n_ktiles, a.B, a.Hkv, a.xcd_kv_groups, false, b, hkv, kt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int k0 = kt * C::BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + li;
  const bool key_ok = key < a.Skv;
  const size_t q_rs = (size_t)a.Hq * D, kv_rs = (size_t)a.Hkv * D;
  const size_t koff = ((size_t)b * a.Skv + key) * kv_rs + (size_t)hkv * D;

  bf16x8 kreg[C::KS], vreg[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    u32x4 u = {0u, 0u, 0u, 0u}, w = {0u, 0u, 0u, 0u};
    if (key_ok) {
      u = *(const u32x4*)((const __bf16*)a.k + koff + 16 * kk + 8 * lh);
      w = *(const u32x4*)((const __bf16*)a.v + koff + 16 * kk + 8 * lh);
    }
    kreg[kk] = as_bf16x8(u);
    vreg[kk] = as_bf16x8(w);
  }
  f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // Rows that can see some key of this workgroup: i in [j + delta - hi_off, j + delta - lo_off].
  const int k_last = min(k0 + C::BK, a.Skv) - 1;
  const int ilo = max(0, k0 + a.delta - a.hi_off);
  const int ihi = min(a.Sq - 1, k_last + a.delta - a.lo_off);
  int diag = k0 + a.delta;
  diag = diag < 0 ? 0 : diag / a.q_vblock;
  const int nqvb = a.n_qvblocks;
  if (diag >= nqvb) diag = nqvb - 1;
  QueryTileIter<C::BQ> qit;
  int hh = 0;
  qit.init(nqvb, a.q_vblock, diag, ilo, ihi);
  auto next_step = [&](int& hq_o, int& qs, int& rend) -> bool {
    while (hh < a.G) {
      if (qit.next(qs, rend)) {
        hq_o = hkv * a.G + hh;
        return true;
      }
      ++hh;
      qit.init(nqvb, a.q_vblock, diag, ilo, ihi);
    }
    return false;
  };

  const bool wave_on = kw0 < a.Skv;
  const int w_klast = kw0 + 31;

  u32x4 qbuf[C::CPT], gbuf[C::CPT];
  float lbuf = 0.f;
  auto load_step = [&](int hq_, int qs) {
    const __bf16* qp = (const __bf16*)a.q + (size_t)b * a.Sq * q_rs + (size_t)hq_ * D;
    const __bf16* gp = (const __bf16*)a.dout + (size_t)b * a.Sq * q_rs + (size_t)hq_ * D;
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int c = tid + 256 * u;
      const int i = c / C::DC, col = (c % C::DC) * 8;
      const int row = qs + i;
      const bool ok = c < C::NCH && row < a.Sq;
      qbuf[u] = ok ? *(const u32x4*)(qp + (size_t)row * q_rs + col) : u32x4{0u, 0u, 0u, 0u};
      gbuf[u] = ok ? *(const u32x4*)(gp + (size_t)row * q_rs + col) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2 * C::BQ) {
      const int i = tid & (C::BQ - 1), row = qs + i;
      const size_t st = ((size_t)b * a.Hq + hq_) * a.Sq + row;
      lbuf = row < a.Sq ? (tid < C::BQ ? a.lse2[st] : a.Dvec[st]) : (tid < C::BQ ? INFINITY : 0.f);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int c = tid + 256 * u;
      if (c < C::NCH) {
        const int i = c / C::DC, col = (c % C::DC) * 8;
        *(u32x4*)&sQ[buf][i * C::QROW + col] = qbuf[u];
        *(u32x4*)&sG[buf][i * C::QROW + col] = gbuf[u];
        const int slot = perm_slot(i);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t qv = (e & 1) ? (qbuf[u][w] >> 16) : (qbuf[u][w] & 0xffffu);
          const uint32_t gv = (e & 1) ? (gbuf[u][w] >> 16) : (gbuf[u][w] & 0xffffu);
          *(uint16_t*)&sQt[buf][(col + e) * C::TROW + slot] = (uint16_t)qv;
          *(uint16_t*)&sGt[buf][(col + e) * C::TROW + slot] = (uint16_t)gv;
        }
      }
    }
    if (tid < C::BQ) sLse[buf][tid] = lbuf;
    else if (tid < 2 * C::BQ) sD[buf][tid - C::BQ] = lbuf;
  };

  int hq = 0, qs = 0, rend = 0;
  bool have = next_step(hq, qs, rend);
  if (have) {
    load_step(hq, qs);
    store_step(0);
  }
  __syncthreads();
  int cur = 0;
  while (have) {
    int nhq = 0, nqs = 0, nrend = 0;
    const bool nhave = next_step(nhq, nqs, nrend);
    if (nhave) load_step(nhq, nqs);

    const int qe = min(rend, a.Sq);   // rows >= qe are not part of this step
    // pair (i, j) visible iff lo_off <= j - i + delta <= hi_off
    const int dmin = kw0 - (qs + C::BQ - 1) + a.delta;   // smallest j - i + delta in the step
    const int dmax = w_klast - qs + a.delta;             // largest
    const bool empty = !wave_on || dmax < a.lo_off || dmin > a.hi_off || qs >= qe;
    if (!empty) {
      const bool full = dmin >= a.lo_off && dmax <= a.hi_off && qs + C::BQ <= qe;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        const int off = li * C::QROW + 16 * kk + 8 * lh;
        s = mfma32(*(const bf16x8*)&sQ[cur][off], kreg[kk], s);
        dp = mfma32(*(const bf16x8*)&sG[cur][off], vreg[kk], dp);
      }
      // lane (key li) holds query rows i = 8g + 4lh + e, r = 4g + e
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lse4 = *(const f32x4*)&sLse[cur][8 * g + 4 * lh];
        const f32x4 d4 = *(const f32x4*)&sD[cur][8 * g + 4 * lh];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float x = s[r];
          if (!full) {
            const int i = qs + 8 * g + 4 * lh + e;
            const int dd = key - i + a.delta;
            if (dd < a.lo_off || dd > a.hi_off || i >= qe) x = -INFINITY;
          }
          const float p = fast_exp2(fmaf(x, a.scale_log2, -lse4[e]));
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 pb, sb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pb[w] = pack_bf16x2(s[8 * ks + 2 * w], s[8 * ks + 2 * w + 1]);
          sb[w] = pack_bf16x2(dp[8 * ks + 2 * w], dp[8 * ks + 2 * w + 1]);
        }
        const bf16x8 pbf = as_bf16x8(pb), sbf = as_bf16x8(sb);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int off = (32 * db + li) * C::TROW + 16 * ks + 8 * lh;
          dv[db] = mfma32(*(const bf16x8*)&sGt[cur][off], pbf, dv[db]);
          dk[db] = mfma32(*(const bf16x8*)&sQt[cur][off], sbf, dk[db]);
        }
      }
    }
    if (nhave) store_step(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    hq = nhq;
    qs = nqs;
    rend = nrend;
    have = nhave;
  }

  if (key_ok) {
    __bf16* kop = (__bf16*)a.dk + koff;
    __bf16* vop = (__bf16*)a.dv + koff;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk[db][4 * g] * a.scale, dk[db][4 * g + 1] * a.scale);
        wk[1] = pack_bf16x2(dk[db][4 * g + 2] * a.scale, dk[db][4 * g + 3] * a.scale);
        wv[0] = pack_bf16x2(dv[db][4 * g], dv[db][4 * g + 1]);
        wv[1] = pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3]);
        *(u32x2*)(kop + 32 * db + 8 * g + 4 * lh) = wk;
        *(u32x2*)(vop + 32 * db + 8 * g + 4 * lh) = wv;
      }
  }
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 kernels (small head dims): one thread per query row for dq, one thread
// per key row for dk/dv; tiles of the other side staged in LDS.
template <int D>
__global__ __launch_bounds__(128) void bwd_dq_f32_kernel(BwdArgs a) {
  constexpr int BM = 128, BN = 32;
  __shared__ float sK[BN][D + 1], sV[BN][D + 1];
  int b, hq, qt;
  map_task(blockIdx.x, a.n_qtiles, a.B, a.Hq, a.Hkv, a.G, 0, false, b, hq, qt);
  const int hkv = hq / a.G, tid = threadIdx.x;
  const int row = qt * BM + tid;
  const bool row_ok = row < a.Sq;
  const size_t q_rs = (size_t)a.Hq * D, kv_rs = (size_t)a.Hkv * D;
  const size_t qoff = ((size_t)b * a.Sq + row) * q_rs + (size_t)hq * D;
  const float* kp = (const float*)a.k + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;
  const float* vp = (const float*)a.v + (size_t)b * a.Skv * kv_rs + (size_t)hkv * D;
  float qr[D], gr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = row_ok ? ((const float*)a.q)[qoff + d] : 0.f;
    gr[d] = row_ok ? ((const float*)a.dout)[qoff + d] : 0.f;
    acc[d] = 0.f;
  }
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
      sK[r][d] = j < a.Skv ? kp[(size_t)j * kv_rs + d] : 0.f;
      sV[r][d] = j < a.Skv ? vp[(size_t)j * kv_rs + d] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < BN; ++r) {
      const int j = ts + r;
      if (j < my_jmin || j > my_jmax || j >= tend) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qr[d], sK[r][d], s);
        dp = fmaf(gr[d], sV[r][d], dp);
      }
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
    for (int d = 0; d < D; ++d) op[d] = acc[d] * a.scale;
  }
}

template <int D>
__global__ __launch_bounds__(128) void bwd_dkdv_f32_kernel(BwdArgs a) {
  constexpr int BK = 128, BQ = 32;
  __shared__ float sQ[BQ][D + 1], sG[BQ][D + 1], sL[BQ], sDv[BQ];
  int b, hkv, kt;
  map_kv_task(blockIdx.x, a.n_ktiles, a.B, a.Hkv, 0, false, b, hkv, kt);
  const int tid = threadIdx.x;
  const int key = kt * BK + tid;
  const bool key_ok = key < a.Skv;
  const size_t q_rs = (size_t)a.Hq * D, kv_rs = (size_t)a.Hkv * D;
  const size_t koff = ((size_t)b * a.Skv + key) * kv_rs + (size_t)hkv * D;
  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = key_ok ? ((const float*)a.k)[koff + d] : 0.f;
    vr[d] = key_ok ? ((const float*)a.v)[koff + d] : 0.f;
    dk[d] = 0.f;
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
    const float* gp = (const float*)a.dout + (size_t)b * a.Sq * q_rs + (size_t)hq * D;
    QueryTileIter<BQ> qit;
    qit.init(nqvb, a.q_vblock, diag, ilo, ihi);
    int qs, rend;
    while (qit.next(qs, rend)) {
      const int qe = min(rend, a.Sq);
      for (int c = tid; c < BQ * D; c += BK) {
        const int r = c / D, d = c % D, row = qs + r;
        sQ[r][d] = row < a.Sq ? qp[(size_t)row * q_rs + d] : 0.f;
        sG[r][d] = row < a.Sq ? gp[(size_t)row * q_rs + d] : 0.f;
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
        for (int d = 0; d < D; ++d) {
          s = fmaf(sQ[r][d], kr[d], s);
          dp = fmaf(sG[r][d], vr[d], dp);
        }
        const float p = fast_exp2(fmaf(s, a.scale_log2, -sL[r]));
        const float ds = p * (dp - sDv[r]);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dk[d] = fmaf(ds, sQ[r][d], dk[d]);
          dv[d] = fmaf(p, sG[r][d], dv[d]);
        }
      }
      __syncthreads();
    }
  }
  if (key_ok) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      ((float*)a.dk)[koff + d] = dk[d] * a.scale;
      ((float*)a.dv)[koff + d] = dv[d];
    }
  }
}

int bwd_q_tile_rows(int dtype) { return dtype == 0 ? BwdQCfg<128>::BM : 128; }
int bwd_k_tile_rows(int dtype) { return dtype == 0 ? BwdKVCfg<128>::BK : 128; }

template <typename T, int D>
static void launch_pre(const BwdArgs& a, hipStream_t stream) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  constexpr int RPB = 256 / LPR;
  const long long nrows = (long long)a.B * a.Sq * a.Hq;
  const unsigned blocks = (unsigned)((nrows + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, a);
}

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t stream) {
  const dim3 gq((unsigned)a.n_qtiles * a.B * a.Hq), gk((unsigned)a.n_ktiles * a.B * a.Hkv);
  const bool has_q = gq.x > 0, has_k = gk.x > 0;
  const bool pre = has_q && (a.stages & 1), dq = has_q && (a.stages & 2), dkdv = has_k && (a.stages & 4);
  const dim3 bb(dtype == 0 ? 256 : 128);
#define REA_BWD(T, DD, DQ, DKV)                                                  \
  do {                                                                          \
    if (pre) launch_pre<T, DD>(a, stream);                                      \
    if (dq) hipLaunchKernelGGL(DQ<DD>, gq, bb, 0, stream, a);                   \
    if (dkdv) hipLaunchKernelGGL(DKV<DD>, gk, bb, 0, stream, a);                \
  } while (0)
  if (dtype == 0) {
    switch (a.D) {
      case 32: REA_BWD(__bf16, 32, bwd_dq_bf16_kernel, bwd_dkdv_bf16_kernel); break;
      case 64: REA_BWD(__bf16, 64, bwd_dq_bf16_kernel, bwd_dkdv_bf16_kernel); break;
      case 128: REA_BWD(__bf16, 128, bwd_dq_bf16_kernel, bwd_dkdv_bf16_kernel); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.D) {
      case 32: REA_BWD(float, 32, bwd_dq_f32_kernel, bwd_dkdv_f32_kernel); break;
      case 64: REA_BWD(float, 64, bwd_dq_f32_kernel, bwd_dkdv_f32_kernel); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef REA_BWD
  return hipGetLastError();
}

}  // namespace rea
