// Attention over gathered candidates ("AnnAttention", faiss_block_attention).
//
// Every token t attends to a list of slots: a window of W keys ending at t (positions
// before 0 are zero vectors), then the bs rows of each of its top_n selected blocks
// (block index -1 reads token 0 for every row, as the page clamps negative item
// indices).  One softmax over all slots, no mask; logits are q . k / sqrt(E).
//
#include "common.h"
#include "launch.h"
#include "sparse_common.h"

namespace rea {

// ---------------------------------------------------------------------------------
// Block-shared form (E = 512, bs in {16, 32, 64}): one workgroup per tpw <= 32
// consecutive tokens (32 unless the grid would be small, as when decoding a few
// tokens).  The tokens' selected block indices are sorted and deduplicated in LDS; each
// distinct block u gets a per-token multiplicity cnt(u, t) (a token lists a block at
// most once in a valid selection; -1 entries are one block whose rows are all token 0,
// counted once per entry).  The window is covered by up to three 32-row blocks with a
// per-token mask.  Every 32-row block is then attended with MFMA like a dense tile:
//   S^T = K Q^T (split over the embedding: wave w owns e in [128w, 128w + 128), the
//   four partial score tiles are summed through LDS), weights w(t, row) = multiplicity
//   or window mask, online softmax with weights (p = w * exp(s - m)), and
//   O^T += V^T P^T on the wave's embedding slice (V staged row-major in LDS, read
//   transposed with ds_read_b64_tr_b16).
// A block shared by several tokens is read once for all of them.

__global__ __launch_bounds__(256, 2) void sparse_union_kernel(SparseArgs a) {
  // LDS: partial scores 16 KiB | V slices 40 KiB (setup scratch reuses it) | counts 16 KiB
  __shared__ __attribute__((aligned(16))) float sS[4][64 * 16];
  __shared__ __attribute__((aligned(16))) __bf16 sV[4][32 * kUPITCH];
  __shared__ uint32_t ucnt[kUMaxEnt][kUQ / 4];
  __shared__ int ublk[kUMaxEnt];
  __shared__ int s_nu;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 31, lh = lane >> 5;
  const int nqb = (a.S + a.tpw - 1) / a.tpw;
  const int wg = wg_index(a.rev_order), split = wg % a.ksplit;
  // token groups of one sequence per XCD (see xcd_unit), longest first, when the split
  // is off
  const int grp_id = a.ksplit == 1 ? longest_first(xcd_unit(wg, nqb, a.xcd_seq), nqb) : wg / a.ksplit;
  const int b = grp_id / nqb, t0 = (grp_id % nqb) * a.tpw;
  const int tend = min(t0 + a.tpw, a.S);                      // this workgroup's tokens: [t0, tend)
  const int n = a.top_n, bs = a.sel_block, W = a.window;

  // ---- setup: sort (block, token) pairs, deduplicate, count per token
  const int nu = build_union(a.sel, a.S, tend, n, b, t0, (int*)&sV[0][0], ucnt, ublk, &s_nu);

  // ---- main loop over 32-row blocks: window blocks, then union blocks
  const int nwin = (W + a.tpw - 1 + 31) / 32;
  // 32-row steps per selected block: bs is 16, 32 or 64 (checked by the host), so a
  // step's entry and sub-block come from a shift and a mask rather than a division
  const int nsub_sh = bs > 32 ? 1 : 0, nsub = 1 << nsub_sh;
  const int nsteps = nwin + nu * nsub;
  // this workgroup's share of the steps (all of them unless split)
  const int sps = (nsteps + a.ksplit - 1) / a.ksplit;
  const int s_begin = min(nsteps, split * sps), s_end = min(nsteps, s_begin + sps);
  // Query row r sits at position q_pos0 + r of the key / value sequence (Skv rows): the
  // whole sequence when q_pos0 = 0 and Skv = S, or a few new tokens against a cache.
  const int wstart = a.q_pos0 + t0 - W + 1;
  const uint32_t row_b = (uint32_t)kSpE * 2;
  const size_t bbase = (size_t)b * a.S * kSpE;                 // query / output rows
  const size_t kvbase = (size_t)b * a.Skv * kSpE;              // key / value rows
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const __bf16*)a.k + kvbase, (uint32_t)a.Skv * row_b);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)a.v + kvbase, (uint32_t)a.Skv * row_b);
  const int e0 = kUDW * wave;                                  // this wave's embedding slice
  const int tok = t0 + li;                                     // this lane's token (B / C column)
  const bool tok_ok = tok < tend;
  const int tpos = a.q_pos0 + tok;                             // its position

  bf16x8 qreg[kUDW / 16];
#pragma unroll
  for (int kk = 0; kk < kUDW / 16; ++kk) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (tok_ok) u = *(const u32x4*)((const __bf16*)a.q + bbase + (size_t)tok * kSpE + e0 + 16 * kk + 8 * lh);
    qreg[kk] = as_bf16x8(u);
  }

  auto row_pos = [&](int step, int r, bool& valid) -> int {   // position of row r of a step
    valid = true;
    if (step < nwin) return wstart + 32 * step + r;
    const int u = (step - nwin) >> nsub_sh, h = (step - nwin) & (nsub - 1);
    const int c = ublk[u];
    valid = 32 * h + r < bs;
    return c < 0 ? 0 : c * bs + 32 * h + r;
  };
  u32x4 kbuf[kUDW / 16];
  // Both loaders are issued unconditionally (a step past the end, and the padding slots,
  // get an out-of-range offset and read zero without a memory access), so the loop body
  // is straight-line and the compiler's waits count exactly the loads in flight.
  auto load_k = [&](int step) {
    bool ok;
    const int pk = step < s_end ? row_pos(step, li, ok) : -1;  // K operand row of this lane
#pragma unroll
    for (int kk = 0; kk < kUDW / 16; ++kk)
      kbuf[kk] = buf_load16(rk, (uint32_t)pk * row_b + 2u * (e0 + 16 * kk + 8 * lh), 0);
  };
  // The V slice goes straight into this wave's LDS rows (buffer loads with an LDS
  // destination): instruction n fills bytes [1024 n, 1024 n + 1024) of the slice, lane l
  // the 16 bytes of slot j = 64 n + l, i.e. row j / 20, chunk j % 20 of the 320-byte
  // pitch (chunks 16..19 are padding and load nothing).  Only this wave reads the slice,
  // so it needs no barrier, only this wave's wait before the P V MFMAs.
  constexpr int kVSlots = kUPITCH / 8;                         // 16-byte slots per row
  auto dma_v = [&](int step) {
    const bool live = step < s_end;
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
    for (int n = 0; n < 32 * kVSlots / 64; ++n) {
      const int j = 64 * n + lane, r = j / kVSlots, ch = j - kVSlots * r;
      const int pv = all0 ? 0 : base + r;
      const uint32_t off = live && ch < 16 ? (uint32_t)pv * row_b + 2u * (e0 + 8 * ch) : 0xffffffffu;
      dma16(rv, &sV[wave][512 * n], off);
    }
  };

  f32x16 acc[kUDW / 32];
#pragma unroll
  for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_used = -INFINITY, m_true = -INFINITY, l_part = 0.f;
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_off = (4 * (tg >> 1) + (tj >> 2)) * kUPITCH + 16 * (tg & 1) + 4 * (tj & 3);

  if (s_begin < s_end) {
    load_k(s_begin);
    dma_v(s_begin);
  }
  for (int step = s_begin; step < s_end; ++step) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < kUDW / 16; ++kk) s = mfma32(as_bf16x8(kbuf[kk]), qreg[kk], s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v4 = {s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
      *(f32x4*)&sS[wave][part_off(lane, g)] = v4;
    }
    lds_barrier();                                             // partial tiles written
    load_k(step + 1);                                          // registers are free again

    // full scores (sum of the four embedding slices), identical in every wave
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v4 = *(const f32x4*)&sS[w2][part_off(lane, g)];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * g + e] += v4[e];
      }
    // weights of (token li, row 8(r>>2) + 4lh + (r&3))
    float wt[16];
    if (step < nwin) {
      const int p0 = wstart + 32 * step + 4 * lh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = p0 + 8 * (r >> 2) + (r & 3);
        wt[r] = (tok_ok && p >= tpos - W + 1 && p <= tpos) ? 1.f : 0.f;
      }
    } else {
      const int u = (step - nwin) >> nsub_sh, h = (step - nwin) & (nsub - 1);
      const float cnt = (float)((ucnt[u][li >> 2] >> (8 * (li & 3))) & 0xffu);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * h + 8 * (r >> 2) + 4 * lh + (r & 3);
        wt[r] = row < bs ? cnt : 0.f;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = wt[r] > 0.f ? s[r] : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, other_half(mx));
    const float mt = mx * a.scale_log2;
    m_true = fmaxf(m_true, mt);
    if (__ballot(mt > m_used + 8.0f)) {
      cold_path();
      const float m_new = fmaxf(m_used, mt);
      const float alpha = fast_exp2(m_used - (m_new == -INFINITY ? 0.f : m_new));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_used = m_new;
    }
    const float m_ref = (m_used == -INFINITY) ? 0.f : m_used;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = wt[r] * fast_exp2(fmaf(s[r], a.scale_log2, -m_ref));
      s[r] = p;
      l_part += p;
    }
    // this step's V slice has landed: it was issued before the next step's 8 K loads
    // (the memory clobber keeps the compiler from moving LDS reads above the wait)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 pb;
#pragma unroll
      for (int w = 0; w < 4; ++w) pb[w] = pack_bf16x2(s[8 * ks + 2 * w], s[8 * ks + 2 * w + 1]);
      const bf16x8 pbf = as_bf16x8(pb);
#pragma unroll
      for (int db = 0; db < kUDW / 32; ++db) {
        const __bf16* vp0 = &sV[wave][tr_off + 16 * ks * kUPITCH + 32 * db];
        const bf16x8 va = join_bf16x8(lds_read_tr16(vp0), lds_read_tr16(vp0 + 8 * kUPITCH));
        acc[db] = mfma32(va, pbf, acc[db]);
      }
    }
    // the P V MFMAs have consumed this wave's transposed reads of its slice, which the
    // next step's rows may now overwrite (the wait and clobber keep the copies after them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_v(step + 1);
    lds_barrier();                                             // sS is rewritten next step
  }

  const float l_used = l_part + other_half(l_part);
  const float corr = (m_true == -INFINITY) ? 0.f : fast_exp2(m_used - m_true);
  if (a.ksplit > 1) {
    // partial result of this share, relative to its exact max: numerator, max, sum
    if (tok_ok) {
      float* pp = a.part + (((size_t)b * a.S + tok) * a.ksplit + split) * (kSpE + 4);
#pragma unroll
      for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * g + e] * corr;
          *(f32x4*)(pp + e0 + 32 * db + 8 * g + 4 * lh) = w;
        }
      if (wave == 0 && lh == 0) {
        pp[kSpE] = m_true;
        pp[kSpE + 1] = l_used * corr;
      }
    }
    return;
  }
  if (tok_ok) {
    const float inv = l_used > 0.f ? 1.f / l_used : 0.f;
    __bf16* op = (__bf16*)a.o + bbase + (size_t)tok * kSpE + e0;
#pragma unroll
    for (int db = 0; db < kUDW / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        *(u32x2*)(op + 32 * db + 8 * g + 4 * lh) = w;
      }
    if (wave == 0 && lh == 0) {
      const size_t st = (size_t)b * a.S + tok;
      a.m[st] = (m_true == -INFINITY) ? -INFINITY : m_true * kLn2;
      a.l[st] = l_used * corr;
    }
  }
}

// Combines the ksplit partial results of each token (one workgroup per token, two
// embedding columns per thread): O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s; a token whose shares saw nothing keeps O = 0, m = -inf, l = 0.
__global__ __launch_bounds__(256) void sparse_combine_kernel(SparseArgs a) {
  const size_t tok = wg_index(a.rev_order);                    // b * S + token
  const float* pp = a.part + tok * a.ksplit * (kSpE + 4);
  float M = -INFINITY;
  for (int s = 0; s < a.ksplit; ++s) M = fmaxf(M, pp[s * (kSpE + 4) + kSpE]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  const int e = 2 * threadIdx.x;
  for (int s = 0; s < a.ksplit; ++s) {
    const float* ps = pp + s * (kSpE + 4);
    const float w = ps[kSpE] == -INFINITY ? 0.f : fast_exp2(ps[kSpE] - M);
    L = fmaf(w, ps[kSpE + 1], L);
    o0 = fmaf(w, ps[e], o0);
    o1 = fmaf(w, ps[e + 1], o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *(uint32_t*)((__bf16*)a.o + tok * kSpE + e) = pack_bf16x2(o0 * inv, o1 * inv);
  if (threadIdx.x == 0) {
    a.m[tok] = M == -INFINITY ? -INFINITY : M * kLn2;
    a.l[tok] = L;
  }
}

hipError_t launch_sparse(const SparseArgs& args, hipStream_t stream) {
  SparseArgs a = args;
  sparse_plan(a.B, a.S, a.window, a.sel_block, a.top_n, a.part != nullptr, a.tpw, a.ksplit);
  const long long nqb = (a.S + a.tpw - 1) / a.tpw;
  a.xcd_seq = a.ksplit == 1 ? xcd_per_seq(a.B, nqb) : 0;
  hipLaunchKernelGGL(sparse_union_kernel, dim3((unsigned)(a.B * nqb * a.ksplit)), dim3(256), 0, stream, a);
  if (a.ksplit > 1)
    hipLaunchKernelGGL(sparse_combine_kernel, dim3((unsigned)((long long)a.B * a.S)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rea
