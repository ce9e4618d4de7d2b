// Backward pass of the attention over gathered candidates ("AnnAttention",
// faiss_block_attention: the model trains through it).
//
// Token t attends to its slots j (window of W keys ending at t, zero vectors before
// position 0; then the bs rows of each selected block, -1 reading token 0).  With the
// forward's statistics, P(t, j) = exp(s_tj - LSE_t) and
//   D_t = dO_t . O_t,  dP(t, j) = dO_t . v_j,  dS(t, j) = P(t, j) (dP(t, j) - D_t),
//   dq_t = scale sum_j dS(t, j) k_j,
// and every slot j that reads sequence row p passes scale dS(t, j) q_t to dk_p and
// P(t, j) dO_t to dv_p (duplicates and the -1 clamp to token 0 add up; zero pads pass
// nothing).  Slots of one token that read the same row have the same logit, so they are
// handled together with a weight w(t, row) = the number of such slots.
//
// Two kernels, both owner-computes (no atomics, bitwise reproducible):
//  * sparse_bwd_dq_kernel -- one workgroup per 32 consecutive tokens, walking the same
//    deduplicated union of selected blocks and window blocks as the forward kernel.
//    D_t = dO_t . O_t from the stored output, except in a unit whose tokens have -1
//    entries: there the bs clamped slots of each entry all pass their gradient to row 0,
//    so row 0 collects P (dP - D) with weights up to bs * top_n, and the rounding of the
//    stored bf16 output would show; such a unit first walks its blocks once to form
//    D_t = sum_j P(t, j) dP(t, j) from fp32 values (equal in exact arithmetic).  D_t and
//    the LSE go to the workspace for the dk/dv kernel;
//  * sparse_bwd_dkdv_kernel -- one workgroup per 32-row key tile (one selection block,
//    bs = 32): the tokens whose window covers the tile, then every token that selected
//    the block (found by scanning the selections in token order), and for the tile at
//    position 0 the tokens with -1 entries, whose bs clamped slots all read row 0.
// Both split the embedding E = 512 over their four waves (128 each) and sum the partial
// score tiles through LDS, as the forward kernel does.
#include "common.h"
#include "launch.h"
#include "sparse_common.h"
#include "tiles.h"

namespace rea {

__global__ __launch_bounds__(256, 1) void sparse_bwd_dq_kernel(SparseBwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sS[4][64 * 16];   // partial scores per wave
  __shared__ __attribute__((aligned(16))) float sP[4][64 * 16];   // partial dP per wave
  // K slices, stored by rows (lane = row) and read transposed: the grouped layout keeps
  // both patterns free of bank conflicts (also the setup scratch)
  using KL = TileLayout<kUDW, kBothRead>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[4][KL::elems(kUQ)];
  // V slices by rows at a 272-byte pitch (conflict-free row reads), copied straight from
  // the gathered rows: nine 1 KB copies per wave, the last one partly into the padding
  using VL = TileLayout<kUDW, kRowRead>;
  constexpr int kVRowSlots = VL::PITCH / 8;                      // 16-byte slots per row
  constexpr int kVCopies = (kUQ * kVRowSlots + 63) / 64;
  __shared__ __attribute__((aligned(16))) __bf16 sV[4][kVCopies * 512];
  __shared__ uint32_t ucnt[kUMaxEnt][kUQ / 4];
  __shared__ int ublk[kUMaxEnt];
  __shared__ int s_nu;
  __shared__ float sDp[4][kUQ];
  // dS of the step as bf16, [token][key] at a 34-word row pitch (conflict-free B-operand
  // reads), and each token's log2-LSE and D
  constexpr int kDsPitch = 34;
  __shared__ __attribute__((aligned(16))) uint32_t sDS[kUQ * kDsPitch];
  __shared__ float sTokLse[kUQ], sTokD[kUQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int nqb = (a.S + kUQ - 1) / kUQ;
  const int u = longest_first(xcd_unit(wg_index(a.rev_order), nqb, xcd_per_seq(a.B, nqb)), nqb);
  const int b = u / nqb, t0 = (u % nqb) * kUQ;
  const int n = a.top_n, bs = a.sel_block, W = a.window;

  const int nu = build_union(a.sel, a.S, a.S, n, b, t0, (int*)&sK[0][0], ucnt, ublk, &s_nu);

  const int nwin = (W + kUQ - 1 + 31) / 32;
  // 32-row steps per selected block: bs is 16, 32 or 64 (checked by the host), so a
  // step's entry and sub-block come from a shift and a mask rather than a division
  const int nsub_sh = bs > 32 ? 1 : 0, nsub = 1 << nsub_sh;
  const int nsteps = nwin + nu * nsub;
  const int wstart = t0 - W + 1;
  const uint32_t row_b = (uint32_t)kSpE * 2;
  const size_t bbase = (size_t)b * a.S * kSpE;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const __bf16*)a.k + bbase, (uint32_t)a.S * row_b);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)a.v + bbase, (uint32_t)a.S * row_b);
  const int e0 = kUDW * wave;
  const int tok = t0 + li;
  const bool tok_ok = tok < a.S;

  // Q^T and dO^T slices as B operands (lane (li, lh): token li, e0 + 16kk + 8lh ..+7);
  // dO . O over this wave's slice for D_t.
  bf16x8 qreg[kUDW / 16], doreg[kUDW / 16];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < kUDW / 16; ++kk) {
    u32x4 uq = {0u, 0u, 0u, 0u}, ug = uq, uo = uq;
    if (tok_ok) {
      const size_t off = bbase + (size_t)tok * kSpE + e0 + 16 * kk + 8 * lh;
      uq = *(const u32x4*)((const __bf16*)a.q + off);
      ug = *(const u32x4*)((const __bf16*)a.dout + off);
      uo = *(const u32x4*)((const __bf16*)a.o + off);
    }
    qreg[kk] = as_bf16x8(uq);
    doreg[kk] = as_bf16x8(ug);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = fmaf(bf16_lo(ug[w]), bf16_lo(uo[w]), dpart);
      dpart = fmaf(bf16_hi(ug[w]), bf16_hi(uo[w]), dpart);
    }
  }
  dpart += other_half(dpart);
  if (lh == 0) sDp[wave][li] = dpart;
  __syncthreads();
  const size_t st = (size_t)b * a.S + (tok_ok ? tok : 0);
  // union blocks are sorted ascending, so a -1 entry in this unit shows as ublk[0] = -1
  const bool exact_d = nu > 0 && ublk[0] < 0;
  float lse2 = INFINITY;
  if (tok_ok) {
    const float l = a.l[st];
    lse2 = l > 0.f ? fmaf(a.m[st], kLog2e, log2f(l)) : INFINITY;
  }

  auto row_pos = [&](int step, int r) -> int {      // sequence row of row r of a step
    if (step < nwin) return wstart + 32 * step + r;    // negative: zero pad (reads 0)
    const int u = (step - nwin) >> nsub_sh, h = (step - nwin) & (nsub - 1);
    const int c = ublk[u];
    return c < 0 ? 0 : c * bs + 32 * h + r;
  };
  // K rows as A operands in registers: lane (li, lh) holds row li, e0 + 16kk + 8lh ..+7.
  // An A-operand load puts 32 rows in flight, 32 bytes of each, and the load path serves
  // about one cache line per clock, so issuing these gathers had become the longest part
  // of a step; V rows therefore go straight into this wave's LDS rows instead (16 lanes
  // per row: an instruction moves four whole rows) and are read back as A operands.
  // Both loads are issued unconditionally (a step past the end reads out of range), so a
  // step's single wait counts exactly.
  u32x4 kbuf[kUDW / 16];
  auto load_k = [&](int step) {
    const int pk = step < nsteps ? row_pos(step, li) : -1;
#pragma unroll
    for (int kk = 0; kk < kUDW / 16; ++kk)
      kbuf[kk] = buf_load16(rk, (uint32_t)pk * row_b + 2u * (e0 + 16 * kk + 8 * lh), 0);
  };
  auto dma_v = [&](int step) {
    const bool live = step < nsteps;
    bool all0 = false;
    int base = 0;
    if (live && step < nwin) {
      base = wstart + 32 * step;
    } else if (live) {
      const int c = ublk[(step - nwin) >> nsub_sh];
      all0 = c < 0;
      base = c * bs + 32 * ((step - nwin) & (nsub - 1));
    }
#pragma unroll
    for (int n = 0; n < kVCopies; ++n) {
      const int j = 64 * n + lane, r = j / kVRowSlots, ch = j - kVRowSlots * r;
      const int pv = all0 ? 0 : base + r;
      const bool ok = live && ch < 16 && r < kUQ;
      dma16(rv, &sV[wave][512 * n], ok ? (uint32_t)pv * row_b + 2u * (e0 + 8 * ch) : 0xffffffffu);
    }
  };

  f32x16 acc[kUDW / 32];                             // dQ^T slice: 4 blocks of 32 e x 32 tokens
#pragma unroll
  for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_off = KL::idx(4 * (tg >> 1) + (tj >> 2), 16 * (tg & 1) + 4 * (tj & 3));

  // pass 0 (units with -1 entries only) accumulates D_t from P and dP; pass 1 uses D_t
  // for dS and dQ.
  //
  // A step: each wave forms partial S and dP tiles over its embedding slice and writes
  // them to LDS; after a barrier wave w sums the four partials of tokens 8w .. 8w + 7
  // only (lane: token T = 8w + lane / 8, key rows 4q .. 4q + 3 with q = lane % 8), forms
  // P and dS for them and writes dS as bf16; after a second barrier every wave reads the
  // whole dS tile as the B operand of dQ^T += K^T dS^T.  Next step's partials are written
  // only after every wave has passed the second barrier, i.e. finished its sums; the K
  // slice in LDS is private to its wave.
  const float Dt = tok_ok ? (sDp[0][li] + sDp[1][li]) + (sDp[2][li] + sDp[3][li]) : 0.f;
  if (wave == 0 && lh == 0) {
    sTokLse[li] = lse2;
    sTokD[li] = Dt;
    if (!exact_d && tok_ok) {
      a.Dvec[st] = Dt;
      a.lse2[st] = lse2;
    }
  }
  const int rT = 8 * wave + (lane >> 3), rq = lane & 7;       // reduce phase: token, key quad
  const int rtok = t0 + rT;
  const bool rtok_ok = rtok < a.S;
  const int rsrc = part_off(rT + 32 * (rq & 1), rq >> 1);      // its four values in a partial tile
  float dsum = 0.f;
  for (int pass = exact_d ? 0 : 1; pass < 2; ++pass) {
    load_k(0);
    dma_v(0);
    for (int step = 0; step < nsteps; ++step) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      // this step's K rows and V slice have landed (the memory clobber keeps the V reads
      // below the wait)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int kk = 0; kk < kUDW / 16; ++kk) {
        s = mfma32(as_bf16x8(kbuf[kk]), qreg[kk], s);
        dp = mfma32(*(const bf16x8*)&sV[wave][VL::idx(li, 16 * kk + 8 * lh)], doreg[kk], dp);
      }

#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 s4 = {s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
        const f32x4 p4 = {dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3]};
        *(f32x4*)&sS[wave][part_off(lane, g)] = s4;
        *(f32x4*)&sP[wave][part_off(lane, g)] = p4;
      }
      if (pass == 1) {
#pragma unroll
        for (int kk = 0; kk < kUDW / 16; ++kk) *(u32x4*)&sK[wave][KL::idx(li, 16 * kk + 8 * lh)] = kbuf[kk];
      }
      // the dP MFMAs have consumed this wave's reads of its V slice; issued after this
      // step's other LDS stores, which the compiler would otherwise hold back until the
      // copies land (the wait and clobber keep the copies after the reads)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_v(step + 1);
      lds_barrier();                                   // partial tiles written
      load_k(step + 1);

      // reduce phase: token rT, key rows 4 rq + e of the step
      f32x4 sr = *(const f32x4*)&sS[0][rsrc], pr = *(const f32x4*)&sP[0][rsrc];
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) {
        const f32x4 s4 = *(const f32x4*)&sS[w2][rsrc];
        const f32x4 p4 = *(const f32x4*)&sP[w2][rsrc];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sr[e] += s4[e];
          pr[e] += p4[e];
        }
      }
      float wt[4];
      if (step < nwin) {
        const int p0 = wstart + 32 * step + 4 * rq;
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[e] = (rtok_ok && p0 + e >= rtok - W + 1 && p0 + e <= rtok) ? 1.f : 0.f;
      } else {
        const int u = (step - nwin) >> nsub_sh, h = (step - nwin) & (nsub - 1);
        const float cnt = (float)((ucnt[u][rT >> 2] >> (8 * (rT & 3))) & 0xffu);
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[e] = 32 * h + 4 * rq + e < bs ? cnt : 0.f;
      }
      const float lseT = sTokLse[rT];
      if (pass == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum = fmaf(wt[e] * fast_exp2(fmaf(sr[e], a.scale_log2, -lseT)), pr[e], dsum);
      } else {
        const float DT = sTokD[rT];
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = wt[e] * fast_exp2(fmaf(sr[e], a.scale_log2, -lseT));
          ds[e] = pe * (pr[e] - DT);
        }
        u32x2 w2v;
        w2v[0] = pack_bf16x2(ds[0], ds[1]);
        w2v[1] = pack_bf16x2(ds[2], ds[3]);
        *(u32x2*)&sDS[rT * kDsPitch + 2 * rq] = w2v;
      }
      lds_barrier();                                   // dS tile written
      if (pass == 1) {
        // B operand for keys 16 ks + {4 lh .. 4 lh + 3, 8 + 4 lh .. 8 + 4 lh + 3} of token
        // li: the key order of the transposed K reads below
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t* dr = &sDS[li * kDsPitch + 8 * ks + 2 * lh];
          const u32x2 lo = *(const u32x2*)dr, hi = *(const u32x2*)(dr + 4);
          const u32x4 pb = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 dsb = as_bf16x8(pb);
#pragma unroll
          for (int db = 0; db < kUDW / 32; ++db) {
            const __bf16* kp0 = &sK[wave][tr_off + KL::rows(16 * ks) + 32 * db];
            const bf16x8 ka = join_bf16x8(lds_read_tr16(kp0), lds_read_tr16(kp0 + KL::rows(8)));
            acc[db] = mfma32(ka, dsb, acc[db]);
          }
        }
      }
    }
    if (pass == 0) {
      // D of token rT: the sum over its eight key-quad lanes
      float d = dsum;
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      d += __shfl_xor(d, 4);
      if (rq == 0) {
        sTokD[rT] = rtok_ok ? d : 0.f;
        if (rtok_ok) {
          const size_t rst = (size_t)b * a.S + rtok;
          a.Dvec[rst] = d;
          a.lse2[rst] = sTokLse[rT];
        }
      }
      __syncthreads();
    }
  }

  if (tok_ok) {
    __bf16* op = (__bf16*)a.dq + bbase + (size_t)tok * kSpE + e0;
#pragma unroll
    for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * g] * a.scale, acc[db][4 * g + 1] * a.scale);
        w[1] = pack_bf16x2(acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale);
        *(u32x2*)(op + 32 * db + 8 * g + 4 * lh) = w;
      }
  }
}

// ---------------------------------------------------------------------------------
// dk, dv: one workgroup per 32-row key tile (selection block c = tile index, bs = 32).
// A lane owns one key row (B operand of S = Q K^T and dP = dO V^T, K and V slices in
// registers); tiles of 32 tokens are gathered into LDS (row-major Q and dO slices, read
// as rows for S / dP and transposed for dV^T += dO^T P and dK^T += Q^T dS).
constexpr int kSpScan = 4;           // tokens per thread in one pass of the selection scan
constexpr int kSpList = 256 * kSpScan + 32;   // pending token list (a scan pass + leftover)

__global__ __launch_bounds__(256, 1) void sparse_bwd_dkdv_kernel(SparseBwdArgs a) {
  using QL = TileLayout<kUDW, kBothRead>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[4][QL::elems(kUQ)];
  __shared__ __attribute__((aligned(16))) __bf16 sG[4][QL::elems(kUQ)];
  __shared__ __attribute__((aligned(16))) float sS[4][64 * 16];
  __shared__ __attribute__((aligned(16))) float sP[4][64 * 16];
  __shared__ __attribute__((aligned(16))) float sLse[kUQ];
  __shared__ __attribute__((aligned(16))) float sD[kUQ];
  __shared__ float sWa[kUQ], sWb[kUQ];               // per token: weight of every row / extra on row 0
  __shared__ int sTok[kUQ];
  // P and dS of the tile as bf16 hi and lo parts, [key][token] at a 34-word row pitch
  constexpr int kTPitch = 34;
  __shared__ __attribute__((aligned(16))) uint32_t sPD[4][32 * kTPitch];
  __shared__ int lstT[kSpList];
  __shared__ int lstC[kSpList];                      // count | (count of -1 entries) << 8
  __shared__ int sWaveN[4];
  __shared__ int s_npend;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int nkt = (a.S + 31) / 32;
  const int u = xcd_unit(wg_index(a.rev_order), nkt, xcd_per_seq(a.B, nkt));
  const int b = u / nkt, c = u % nkt;
  const int r0 = 32 * c;
  const int n = a.top_n, W = a.window;
  const int e0 = kUDW * wave;
  const uint32_t row_b = (uint32_t)kSpE * 2;
  const size_t bbase = (size_t)b * a.S * kSpE;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)a.q + bbase, (uint32_t)a.S * row_b);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc((const __bf16*)a.dout + bbase, (uint32_t)a.S * row_b);
  const int key = r0 + li;
  const bool key_ok = key < a.S;

  bf16x8 kreg[kUDW / 16], vreg[kUDW / 16];
#pragma unroll
  for (int kk = 0; kk < kUDW / 16; ++kk) {
    u32x4 uk = {0u, 0u, 0u, 0u}, uv = uk;
    if (key_ok) {
      const size_t off = bbase + (size_t)key * kSpE + e0 + 16 * kk + 8 * lh;
      uk = *(const u32x4*)((const __bf16*)a.k + off);
      uv = *(const u32x4*)((const __bf16*)a.v + off);
    }
    kreg[kk] = as_bf16x8(uk);
    vreg[kk] = as_bf16x8(uv);
  }
  f32x16 dk[kUDW / 32], dv[kUDW / 32];
#pragma unroll
  for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_off = QL::idx(4 * (tg >> 1) + (tj >> 2), 16 * (tg & 1) + 4 * (tj & 3));
  const int q_off = QL::idx(li, 8 * lh);

  // One tile of up to 32 tokens: tokfn(i) -> (token or -1, weight of every row, extra
  // weight on row 0); with `win` the weight is instead 1 for the rows in the token's
  // window.  Gathers the tokens' Q / dO slices and statistics, then accumulates this
  // tile's part of dK^T and dV^T.  Outside the window pass a weight stands for several
  // slots (up to bs * top_n on row 0 under the -1 clamp), so P and dS enter the MFMAs as
  // a bf16 pair hi + lo: one bf16 rounding of the merged weight would cost as much as
  // that many roundings of the separate slots.
  // A tile's gathered rows in registers (32 tokens x 16 chunks of 16 bytes per tensor
  // per wave: 8 per lane) and the statistics of token tid < 32; gathered one tile ahead
  // where the next tile's tokens are already listed, so the gather's latency overlaps the
  // current tile's work.
  struct Gathered {
    u32x4 q[8], g[8];
    float lse, d, wa, wb;
    int t;
  };
  auto gather = [&](auto tokfn, Gathered& G) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int cidx = lane + 64 * u, i = cidx >> 4, ch = cidx & 15;
      float wa, wb;
      const int t = tokfn(i, wa, wb);
      const uint32_t off = t >= 0 ? (uint32_t)t * row_b + 2u * (e0 + 8 * ch) : 0xffffffffu;
      G.q[u] = buf_load16(rq, off, 0);
      G.g[u] = buf_load16(rg, off, 0);
    }
    G.lse = INFINITY;
    G.d = 0.f;
    G.wa = 0.f;
    G.wb = 0.f;
    G.t = -1;
    if (tid < kUQ) {
      float wa, wb;
      const int t = tokfn(tid, wa, wb);
      const size_t st = (size_t)b * a.S + (t >= 0 ? t : 0);
      if (t >= 0) {
        G.lse = a.lse2[st];
        G.d = a.Dvec[st];
        G.wa = wa;
        G.wb = wb;
      }
      G.t = t;
    }
  };
  // Stores a gathered tile to LDS (the previous tile's reads ended at its last barrier).
  auto store = [&](const Gathered& G) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int cidx = lane + 64 * u, i = cidx >> 4, ch = cidx & 15;
      *(u32x4*)&sQ[wave][QL::idx(i, 8 * ch)] = G.q[u];
      *(u32x4*)&sG[wave][QL::idx(i, 8 * ch)] = G.g[u];
    }
    if (tid < kUQ) {
      sLse[tid] = G.lse;
      sD[tid] = G.d;
      sWa[tid] = G.wa;
      sWb[tid] = G.wb;
      sTok[tid] = G.t;
    }
  };
  // The tile's work once its rows are in LDS; `next` (if any) is gathered meanwhile.
  auto compute = [&](bool win, auto&& next) {
    lds_barrier();
    next();
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < kUDW / 16; ++kk) {
      s = mfma32(*(const bf16x8*)&sQ[wave][q_off + 16 * kk], kreg[kk], s);
      dp = mfma32(*(const bf16x8*)&sG[wave][q_off + 16 * kk], vreg[kk], dp);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 s4 = {s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
      const f32x4 p4 = {dp[4 * g], dp[4 * g + 1], dp[4 * g + 2], dp[4 * g + 3]};
      *(f32x4*)&sS[wave][part_off(lane, g)] = s4;
      *(f32x4*)&sP[wave][part_off(lane, g)] = p4;
    }
    lds_barrier();
    // Reduce-scatter: wave w sums the four partials of keys 8w .. 8w + 7 only (lane: key
    // rK = 8w + lane / 8, tokens 4 rq .. 4 rq + 3 with rq = lane % 8), forms P and dS as
    // bf16 hi + lo parts and shares them; after the next barrier every wave reads the
    // whole tiles as B operands, in the token order of its transposed Q / dO reads.
    {
      const int rK = 8 * wave + (lane >> 3), rq = lane & 7;
      const int rkey = r0 + rK;
      const int rsrc = part_off(rK + 32 * (rq & 1), rq >> 1);
      f32x4 sr = *(const f32x4*)&sS[0][rsrc], pr = *(const f32x4*)&sP[0][rsrc];
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) {
        const f32x4 s4 = *(const f32x4*)&sS[w2][rsrc];
        const f32x4 p4 = *(const f32x4*)&sP[w2][rsrc];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sr[e] += s4[e];
          pr[e] += p4[e];
        }
      }
      const f32x4 lse4 = *(const f32x4*)&sLse[4 * rq];
      const f32x4 d4 = *(const f32x4*)&sD[4 * rq];
      float pv[4], dv4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * rq + e;
        const int t = sTok[i];
        const float w = win ? ((t >= 0 && rkey >= t - W + 1 && rkey <= t) ? 1.f : 0.f)
                            : sWa[i] + (rK == 0 ? sWb[i] : 0.f);
        const float p = rkey < a.S ? w * fast_exp2(fmaf(sr[e], a.scale_log2, -lse4[e])) : 0.f;
        pv[e] = p;
        dv4[e] = p * (pr[e] - d4[e]);
      }
      const int o = rK * kTPitch + 2 * rq;
      u32x2 ph, sh;
      ph[0] = pack_bf16x2(pv[0], pv[1]);
      ph[1] = pack_bf16x2(pv[2], pv[3]);
      sh[0] = pack_bf16x2(dv4[0], dv4[1]);
      sh[1] = pack_bf16x2(dv4[2], dv4[3]);
      *(u32x2*)&sPD[0][o] = ph;
      *(u32x2*)&sPD[1][o] = sh;
      if (!win) {
        u32x2 pl, sl;
        pl[0] = pack_bf16x2(pv[0] - bf16_lo(ph[0]), pv[1] - bf16_hi(ph[0]));
        pl[1] = pack_bf16x2(pv[2] - bf16_lo(ph[1]), pv[3] - bf16_hi(ph[1]));
        sl[0] = pack_bf16x2(dv4[0] - bf16_lo(sh[0]), dv4[1] - bf16_hi(sh[0]));
        sl[1] = pack_bf16x2(dv4[2] - bf16_lo(sh[1]), dv4[3] - bf16_hi(sh[1]));
        *(u32x2*)&sPD[2][o] = pl;
        *(u32x2*)&sPD[3][o] = sl;
      }
    }
    lds_barrier();
    // B operand of tile k: key li, tokens 16 ks + {4 lh .. 4 lh + 3, 8 + 4 lh .. + 3}
    auto bop = [&](int k, int ks) -> bf16x8 {
      const uint32_t* r = &sPD[k][li * kTPitch + 8 * ks + 2 * lh];
      const u32x2 lo = *(const u32x2*)r, hi = *(const u32x2*)(r + 4);
      const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
      return as_bf16x8(w);
    };
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pbf = bop(0, ks), sbf = bop(1, ks);
      bf16x8 plf = pbf, slf = sbf;
      if (!win) {
        plf = bop(2, ks);
        slf = bop(3, ks);
      }
#pragma unroll
      for (int db = 0; db < kUDW / 32; ++db) {
        const int o0 = tr_off + QL::rows(16 * ks) + 32 * db, o1 = o0 + QL::rows(8);
        const bf16x8 ga = join_bf16x8(lds_read_tr16(&sG[wave][o0]), lds_read_tr16(&sG[wave][o1]));
        const bf16x8 qa = join_bf16x8(lds_read_tr16(&sQ[wave][o0]), lds_read_tr16(&sQ[wave][o1]));
        dv[db] = mfma32(ga, pbf, dv[db]);
        dk[db] = mfma32(qa, sbf, dk[db]);
        if (!win) {
          dv[db] = mfma32(ga, plf, dv[db]);
          dk[db] = mfma32(qa, slf, dk[db]);
        }
      }
    }
    lds_barrier();                                   // LDS tiles are rewritten by the next tile
  };

  // 1. Window slots: token t reads rows t - W + 1 .. t, so the tile's rows are read by
  //    tokens r0 .. r0 + 31 + W - 1, one slot per (token, row) pair in its window.
  const int wend = min(a.S, r0 + 32 + W - 1);
  Gathered G;
  for (int tw = r0; tw < wend; tw += kUQ) {
    gather([&](int i, float& wa, float& wb) -> int {
      const int t = tw + i;
      wa = 0.f;
      wb = 0.f;
      return t < wend ? t : -1;
    }, G);
    store(G);
    compute(true, [] {});
  }

  // 2. Selected slots: tokens that list block c (each listing = bs slots, one per row),
  //    and for the tile at position 0 the -1 entries (bs slots that all read row 0).
  //    Every token is scanned, in order, so any selection (not only block_select's,
  //    which lists strictly earlier blocks) is handled, and the order is fixed.
  if (tid == 0) s_npend = 0;
  lds_barrier();
  // A pass covers 256 * kSpScan tokens: thread tid takes the consecutive tokens
  // base0 + kSpScan tid + k (k < kSpScan), whose selections are contiguous, so with top_n a
  // multiple of 4 they come in 16-byte loads (kSpScan top_n / 4 per thread instead of
  // kSpScan top_n); the entries are appended in token order (lane-major, then k).
  const bool vec_sel = (n & 3) == 0 && ((uintptr_t)a.sel & 15) == 0;
  const bool scan_blk = c < a.S / a.sel_block;
  // With top_n <= 8 the next pass's pieces are loaded into registers before this pass's
  // tiles run (the barriers are LDS-only, so the loads stay in flight through them).
  const bool pf_sel = vec_sel && n <= 8;
  u32x4 selpf[kSpScan][2];
  bool selpf_ok = false;
  auto sel_fetch = [&](int base0) {
    const int tb = base0 + kSpScan * tid;
    selpf_ok = scan_blk && tb + kSpScan <= a.S;
    const int32_t* rowp = a.sel + ((size_t)b * a.S + (selpf_ok ? tb : 0)) * n;
#pragma unroll
    for (int k = 0; k < kSpScan; ++k)
#pragma unroll
      for (int j4 = 0; j4 < 2; ++j4)
        if (selpf_ok && 4 * j4 < n) selpf[k][j4] = *(const u32x4*)(rowp + k * n + 4 * j4);
  };
  // With the block masks a thread reads two words for its four tokens (listed; listed
  // with a code other than 1) and the selections of only the tokens in the second; the
  // next pass's words are loaded before the current pass's tiles run.
  const size_t mplane = (size_t)a.B * a.nsel * a.nwords;
  const uint32_t* mrow = a.lmask && scan_blk ? a.lmask + ((size_t)b * a.nsel + c) * a.nwords : nullptr;
  // pw: word (base0 / 32 + lane % 32) of the pass, so that every wave sees all of the
  // pass's 32 words and all four skip a pass that lists no token, together
  uint32_t mw1 = 0u, mw2 = 0u, pw = 0u;
  auto mask_fetch = [&](int base0) {
    const int tb = base0 + kSpScan * tid;
    const int pwi = (base0 >> 5) + (lane & 31);
    mw1 = mw2 = pw = 0u;
    if (tb < a.S) {
      mw1 = mrow[tb >> 5];
      mw2 = mrow[mplane + (tb >> 5)];
    }
    if (pwi < a.nwords) pw = mrow[pwi];
  };
  if (mrow) mask_fetch(0);
  if (pf_sel && !mrow) sel_fetch(0);
  // (a tile past the last whole block is listed by no token: no pass)
  for (int base0 = 0; base0 < (scan_blk ? a.S : 0); base0 += 256 * kSpScan) {
    int code[kSpScan];                                 // count | (count of -1 entries) << 8
    const int tb = base0 + kSpScan * tid;              // this thread's first token
    const int32_t* rowp = a.sel + ((size_t)b * a.S + (tb < a.S ? tb : 0)) * n;
    if (mrow && __ballot(pw != 0u) == 0) {
      mask_fetch(base0 + 256 * kSpScan);               // no token of this pass lists the block
      continue;
    }
    if (mrow) {
      // tb is a multiple of 4, so the four tokens' bits sit in one word of each mask
      const uint32_t bits = (mw1 >> (tb & 31)) & 0xfu, odd = (mw2 >> (tb & 31)) & 0xfu;
#pragma unroll
      for (int k = 0; k < kSpScan; ++k) {
        code[k] = (bits >> k) & 1u;
        if ((odd >> k) & 1u) {
          const int32_t* row = rowp + k * n;
          int cnt = 0, neg = 0;
          for (int j = 0; j < n; ++j) {
            const int e = row[j];
            cnt += e == c;
            neg += e < 0;
          }
          code[k] = cnt | ((c != 0 ? 0 : neg) << 8);
        }
      }
      mask_fetch(base0 + 256 * kSpScan);
    } else if (pf_sel && selpf_ok) {
#pragma unroll
      for (int k = 0; k < kSpScan; ++k) {
        int cnt = 0, neg = 0;
#pragma unroll
        for (int j4 = 0; j4 < 2; ++j4)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int e = 4 * j4 < n ? (int)selpf[k][j4][x] : c + 1;
            cnt += e == c;
            neg += e < 0;
          }
        code[k] = cnt | ((c != 0 ? 0 : neg) << 8);
      }
    } else if (vec_sel && scan_blk && tb + kSpScan <= a.S) {
      int cnt[kSpScan], neg[kSpScan];
#pragma unroll
      for (int k = 0; k < kSpScan; ++k) cnt[k] = neg[k] = 0;
      // kSpScan * n entries, n / 4 16-byte pieces per token
      for (int j4 = 0; j4 < n / 4; ++j4) {
#pragma unroll
        for (int k = 0; k < kSpScan; ++k) {
          const u32x4 e4 = *(const u32x4*)(rowp + k * n + 4 * j4);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            cnt[k] += (int)e4[x] == c;
            neg[k] += (int)e4[x] < 0;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kSpScan; ++k) code[k] = cnt[k] | ((c != 0 ? 0 : neg[k]) << 8);
    } else {
#pragma unroll
      for (int k = 0; k < kSpScan; ++k) {
        const int t = tb + k;
        const bool scan = t < a.S && scan_blk;
        const int32_t* row = rowp + k * n;
        int e[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) e[j] = scan && j < n ? row[j] : c + 1;
        int cnt = 0, neg = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          cnt += e[j] == c;
          neg += e[j] < 0;
        }
        code[k] = cnt | ((c != 0 ? 0 : neg) << 8);
      }
    }
    if (pf_sel && !mrow) sel_fetch(base0 + 256 * kSpScan);
    // position: entries of the lanes below, then of this lane's earlier tokens
    const uint64_t below = (1ull << lane) - 1;
    int pre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kSpScan; ++k) {
      const uint64_t mk = __ballot(code[k] != 0);
      pre += __popcll(mk & below);
      tot += __popcll(mk);
    }
    if (lane == 0) sWaveN[wave] = tot;
    lds_barrier();
    const int npend = s_npend;
    int pos = npend + pre;
    for (int w2 = 0; w2 < wave; ++w2) pos += sWaveN[w2];
#pragma unroll
    for (int k = 0; k < kSpScan; ++k) {
      if (code[k] != 0) {
        lstT[pos] = tb + k;
        lstC[pos] = code[k];
        ++pos;
      }
    }
    const int have = npend + sWaveN[0] + sWaveN[1] + sWaveN[2] + sWaveN[3];
    lds_barrier();
    int head = 0;
    auto listed = [&](int h) {
      return [&, h](int i, float& wa, float& wb) -> int {
        const int e = lstC[h + i];
        wa = (float)(e & 0xff);
        wb = (float)(32 * (e >> 8));
        return lstT[h + i];
      };
    };
    if (have - head >= kUQ) gather(listed(head), G);
    while (have - head >= kUQ) {
      store(G);
      const bool more = have - head >= 2 * kUQ;
      compute(false, [&] {
        if (more) gather(listed(head + kUQ), G);
      });
      head += kUQ;
    }
    // move the leftover (< 32 entries) to the front
    int lt = 0, lc = 0;
    if (tid < have - head) {
      lt = lstT[head + tid];
      lc = lstC[head + tid];
    }
    lds_barrier();
    if (tid < have - head) {
      lstT[tid] = lt;
      lstC[tid] = lc;
    }
    if (tid == 0) s_npend = have - head;
    lds_barrier();
  }
  const int rest = s_npend;
  if (rest > 0) {
    gather([&](int i, float& wa, float& wb) -> int {
      if (i >= rest) {
        wa = 0.f;
        wb = 0.f;
        return -1;
      }
      const int e = lstC[i];
      wa = (float)(e & 0xff);
      wb = (float)(32 * (e >> 8));
      return lstT[i];
    }, G);
    store(G);
    compute(false, [] {});
  }

  if (key_ok) {
    __bf16* kop = (__bf16*)a.dk + bbase + (size_t)key * kSpE + e0;
    __bf16* vop = (__bf16*)a.dv + bbase + (size_t)key * kSpE + e0;
#pragma unroll
    for (int db = 0; db < kUDW / 32; ++db)
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

// Builds the two block masks, one workgroup per 256 tokens (eight 32-token words per
// block): each thread marks, for its token, every distinct block c < nsel it lists (a -1
// entry counting for block 0) in the first mask, and in the second too when its code for
// c is not 1 (listed twice or more, or block 0 with -1 entries); the workgroup's words,
// zeros included, are then written out, so no word needs clearing beforehand and none is
// written twice.  LDS: 2 x 8 x nsel words (dynamic).
__global__ __launch_bounds__(256) void sparse_mask_kernel(SparseBwdArgs a) {
  extern __shared__ uint32_t smask[];                // [2][8][nsel]
  const int tid = threadIdx.x;
  const int nchunk = (a.S + 255) / 256;
  const int b = blockIdx.x / nchunk, t0 = (blockIdx.x - b * nchunk) * 256;
  const int ns = a.nsel, n = a.top_n;
  for (int i = tid; i < 2 * 8 * ns; i += 256) smask[i] = 0u;
  __syncthreads();
  const int t = t0 + tid;
  if (t < a.S) {
    const int32_t* row = a.sel + ((size_t)b * a.S + t) * n;
    int e[16];
    int neg = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      e[j] = j < n ? row[j] : -2;
      neg += (j < n && e[j] < 0) ? 1 : 0;
    }
    const uint32_t bit = 1u << (tid & 31);
    uint32_t* w1 = smask + (tid >> 5) * ns;
    uint32_t* w2 = smask + 8 * ns + (tid >> 5) * ns;
    bool zero_listed = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= n || e[j] < 0 || e[j] >= ns) continue;
      bool first = true;
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < n && e[i] == e[j]) {
          first = first && i >= j;
          ++cnt;
        }
      if (!first) continue;
      if (e[j] == 0) zero_listed = true;
      atomicOr(&w1[e[j]], bit);
      if ((cnt | (e[j] == 0 ? neg << 8 : 0)) != 1) atomicOr(&w2[e[j]], bit);
    }
    if (neg > 0 && !zero_listed && ns > 0) {
      atomicOr(&w1[0], bit);
      atomicOr(&w2[0], bit);
    }
  }
  __syncthreads();
  // word (plane, g, c) of the workgroup goes to plane * (B nsel nwords) + (b nsel + c) nwords
  // + t0 / 32 + g; consecutive threads take consecutive g
  const size_t plane = (size_t)a.B * ns * a.nwords;
  const int g0 = t0 >> 5;
  for (int i = tid; i < 2 * 8 * ns; i += 256) {
    const int g = i & 7, rest = i >> 3, c = rest % ns, pl = rest / ns;
    if (g0 + g < a.nwords) a.lmask[pl * plane + ((size_t)b * ns + c) * a.nwords + g0 + g] = smask[(pl * 8 + g) * ns + c];
  }
}

hipError_t launch_sparse_bwd(const SparseBwdArgs& a, hipStream_t stream) {
  const unsigned nqb = (unsigned)((a.S + kUQ - 1) / kUQ);
  if (a.lmask && a.nsel > 0) {
    const unsigned nchunk = (unsigned)((a.S + 255) / 256);
    hipLaunchKernelGGL(sparse_mask_kernel, dim3((unsigned)a.B * nchunk), dim3(256),
                       (size_t)2 * 8 * a.nsel * sizeof(uint32_t), stream, a);
  }
  hipLaunchKernelGGL(sparse_bwd_dq_kernel, dim3((unsigned)a.B * nqb), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(sparse_bwd_dkdv_kernel, dim3((unsigned)a.B * nqb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rea
