// Drives every C-ABI entry point of api.cpp through its argument checks, on the host only
// (the launchers are the stand-ins of stub_launch.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Older-version structs are heap blocks of exactly their
// published size, so reading past them is caught.  Device pointers are fake addresses that
// the host never dereferences.  Prints "abi_checks: N checks passed" and exits 0, or
// names the first failed expectation and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "attn.h"

namespace rea {
extern int launches;
}

static int checks = 0;
static void expect_status(int got, int want, const char* what) {
  ++checks;
  if (got != want) {
    fprintf(stderr, "abi_checks: %s: status %d, expected %d (%s)\n", what, got, want, attn_last_error());
    exit(1);
  }
}
static void expect(bool ok, const char* what) {
  ++checks;
  if (!ok) {
    fprintf(stderr, "abi_checks: %s\n", what);
    exit(1);
  }
}

static void* fake(uintptr_t i) { return (void*)(uintptr_t)(0x100000 + 256 * i); }

static attn_params dense(int B, int S, int Hq, int Hkv, int D) {
  attn_params p;
  memset(&p, 0, sizeof p);
  p.struct_size = sizeof(attn_params);
  p.dtype = ATTN_BF16;
  p.batch = B;
  p.seqlen_q = p.seqlen_kv = S;
  p.num_q_heads = Hq;
  p.num_kv_heads = Hkv;
  p.head_dim = D;
  p.causal = 1;
  p.window_left = p.window_right = -1;
  return p;
}

static int fwd(const attn_params* p, float* acc = nullptr) {
  return attn_fwd(p, fake(1), fake(2), fake(3), fake(4), (float*)fake(5), (float*)fake(6), acc, nullptr);
}
static int bwd(const attn_params* p, void* ws, size_t bytes) {
  return attn_bwd(p, fake(1), fake(2), fake(3), fake(4), fake(5), (const float*)fake(6), (const float*)fake(7),
                  fake(8), fake(9), fake(10), ws, bytes, nullptr);
}

int main() {
  // ---- forward: valid calls launch, invalid ones do not
  attn_params p = dense(2, 300, 8, 2, 128);
  int before = rea::launches;
  expect_status(fwd(&p), ATTN_OK, "valid forward");
  expect(rea::launches == before + 1, "a valid forward launches once");
  expect_status(fwd(nullptr), ATTN_ERR_INVALID_ARG, "NULL params");
  attn_params bad = p;
  bad.num_q_heads = 6;
  bad.num_kv_heads = 4;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "Hq not a multiple of Hkv");
  bad = p;
  bad.head_dim = 96;
  expect_status(fwd(&bad), ATTN_ERR_UNSUPPORTED, "head_dim 96");
  bad = p;
  bad.window_right = 3;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "causal with a right window");
  bad = p;
  bad.kv_block = 7;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "kv_block not dividing Skv");
  bad = p;
  bad.flags = ATTN_BWD_SKIP_DQ;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "backward flag on the forward");
  bad = p;
  bad.flags = ATTN_NO_FINALIZE;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "NO_FINALIZE without acc");
  expect_status(fwd(&bad, (float*)fake(11)), ATTN_OK, "NO_FINALIZE with acc");
  bad = p;
  bad.scale = std::numeric_limits<float>::infinity();
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "infinite scale");
  bad = p;
  bad.q_pos0 = (int64_t)1 << 40;
  expect_status(fwd(&bad), ATTN_ERR_UNSUPPORTED, "huge q_pos0");
  bad = p;
  bad.seqlen_q = bad.seqlen_kv = 1 << 27;     // one batch slice past 4 GiB
  bad.num_q_heads = 128;
  bad.num_kv_heads = 8;
  expect_status(fwd(&bad), ATTN_ERR_UNSUPPORTED, "slice past 4 GiB");
  bad = p;
  bad.batch = 0;
  before = rea::launches;
  expect_status(fwd(&bad), ATTN_OK, "batch 0 is a no-op");
  expect(rea::launches == before, "batch 0 launches nothing");
  expect_status(attn_fwd(&p, nullptr, fake(2), fake(3), fake(4), (float*)fake(5), (float*)fake(6), nullptr, nullptr),
                ATTN_ERR_INVALID_ARG, "NULL q");
  expect_status(attn_fwd(&p, (char*)fake(1) + 8, fake(2), fake(3), fake(4), (float*)fake(5), (float*)fake(6),
                         nullptr, nullptr),
                ATTN_ERR_INVALID_ARG, "misaligned q");
  bad = p;
  bad.bias = (const float*)fake(12);
  bad.bias_stride[3] = -1;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "negative bias stride");
  bad = p;
  bad.drop_mask = (const uint32_t*)fake(13);
  bad.drop_stride[2] = (int64_t)1 << 50;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "huge dropout stride");
  bad = p;
  bad.o_lo = (char*)fake(14) + 2;
  expect_status(fwd(&bad), ATTN_ERR_INVALID_ARG, "misaligned o_lo");

  // ---- older struct versions as heap blocks of exactly their size
  const unsigned sizes[4] = {ATTN_PARAMS_V1_SIZE, ATTN_PARAMS_V2_SIZE, ATTN_PARAMS_V3_SIZE, ATTN_PARAMS_V4_SIZE};
  for (unsigned sz : sizes) {
    unsigned char* blk = (unsigned char*)malloc(sz);
    memcpy(blk, &p, sz);
    memcpy(blk, &sz, sizeof sz);
    expect_status(fwd((const attn_params*)blk), ATTN_OK, "older struct version, forward");
    const size_t need = attn_bwd_workspace_bytes((const attn_params*)blk);
    expect(need > 0, "older struct version, workspace size");
    expect_status(bwd((const attn_params*)blk, fake(20), need), ATTN_OK, "older struct version, backward");
    free(blk);
  }
  {
    unsigned char* tiny = (unsigned char*)malloc(16);     // nothing past 16 bytes may be read
    memcpy(tiny, &p, 16);
    const uint32_t tsz = 16;
    memcpy(tiny, &tsz, sizeof tsz);
    expect_status(fwd((const attn_params*)tiny), ATTN_ERR_INVALID_ARG, "16-byte struct, forward");
    expect_status(bwd((const attn_params*)tiny, fake(20), 1 << 20), ATTN_ERR_INVALID_ARG, "16-byte struct, backward");
    expect(attn_bwd_workspace_bytes((const attn_params*)tiny) == 0, "16-byte struct, workspace 0");
    expect(attn_fwd_workspace_bytes((const attn_params*)tiny) == 0, "16-byte struct, fwd workspace 0");
    free(tiny);
  }
  {
    unsigned char* blk = (unsigned char*)malloc(100);
    memcpy(blk, &p, 100);
    const uint32_t sz = 100;
    memcpy(blk, &sz, sizeof sz);
    expect_status(fwd((const attn_params*)blk), ATTN_ERR_INVALID_ARG, "unknown struct size");
    expect(attn_bwd_workspace_bytes((const attn_params*)blk) == 0, "unknown struct size, workspace 0");
    free(blk);
  }

  // ---- backward: workspace checks, splits, flags
  const size_t need = attn_bwd_workspace_bytes(&p);
  expect(need >= 2 * 256, "backward workspace size");
  expect_status(bwd(&p, fake(20), need), ATTN_OK, "valid backward");
  expect_status(bwd(&p, fake(20), need - 1), ATTN_ERR_WORKSPACE, "workspace one byte short");
  expect_status(bwd(&p, nullptr, need), ATTN_ERR_WORKSPACE, "NULL workspace");
  expect_status(bwd(&p, (char*)fake(20) + 16, need), ATTN_ERR_INVALID_ARG, "misaligned workspace");
  bad = p;
  bad.flags = ATTN_CARRY_IN;
  expect_status(bwd(&bad, fake(20), need), ATTN_ERR_INVALID_ARG, "forward flag on the backward");
  bad = p;
  bad.flags = ATTN_BWD_SKIP_DQ | ATTN_BWD_REUSE_STATS;
  expect_status(attn_bwd(&bad, fake(1), fake(2), fake(3), nullptr, fake(5), nullptr, nullptr, nullptr, fake(9),
                         fake(10), fake(20), need, nullptr),
                ATTN_OK, "dk/dv only from kept statistics: o, m, l, dq may be NULL");
  attn_params big = dense(8, 65536, 32, 8, 128);      // workspace size without overflow
  const size_t nbig = attn_bwd_workspace_bytes(&big);
  expect(nbig >= (size_t)2 * 8 * 32 * 65536 * 4, "large workspace size");
  attn_params mla = dense(1, 4096, 128, 8, 128);
  mla.head_dim_v = 64;
  expect(attn_bwd_workspace_bytes(&mla) > (size_t)2 * 128 * 4096 * 4, "split dk/dv partials in the workspace");
  expect_status(bwd(&mla, fake(20), attn_bwd_workspace_bytes(&mla)), ATTN_OK, "MLA backward with splits");

  // ---- sparse mode
  attn_params sp;
  memset(&sp, 0, sizeof sp);
  sp.struct_size = sizeof sp;
  sp.dtype = ATTN_BF16;
  sp.batch = 2;
  sp.seqlen_q = sp.seqlen_kv = 1024;
  sp.num_q_heads = sp.num_kv_heads = 1;
  sp.head_dim = 512;
  sp.sel_idx = (const int32_t*)fake(30);
  sp.top_n = 8;
  sp.sel_block = 32;
  sp.sparse_window = 32;
  expect_status(fwd(&sp), ATTN_OK, "sparse forward");
  const size_t sneed = attn_bwd_workspace_bytes(&sp);
  expect(sneed > 0, "sparse backward workspace");
  expect_status(bwd(&sp, fake(20), sneed), ATTN_OK, "sparse backward");
  attn_params sbad = sp;
  sbad.top_n = 17;
  expect_status(fwd(&sbad), ATTN_ERR_INVALID_ARG, "top_n 17");
  sbad = sp;
  sbad.seqlen_q = 1;
  sbad.q_pos0 = 1023;
  expect(attn_fwd_workspace_bytes(&sbad) > 0, "decode split workspace");
  expect_status(fwd(&sbad, (float*)fake(31)), ATTN_OK, "decode forward with workspace");
  sbad.q_pos0 = 1024;
  expect_status(fwd(&sbad), ATTN_ERR_INVALID_ARG, "decode row past the cache");

  // ---- block selection, including the 32-byte version-1 struct
  select_params s;
  memset(&s, 0, sizeof s);
  s.struct_size = sizeof s;
  s.dtype = ATTN_BF16;
  s.batch = 4;
  s.seqlen = 8192;
  s.embed = 512;
  s.block_size = 32;
  s.top_n = 8;
  const size_t selw = block_select_workspace_bytes(&s);
  expect(selw >= (size_t)4 * 256 * 512 * 8, "select workspace holds the means");
  expect_status(block_select(&s, fake(1), fake(2), (int32_t*)fake(3), fake(20), selw, nullptr), ATTN_OK, "select");
  expect_status(block_select(&s, fake(1), fake(2), (int32_t*)fake(3), fake(20), selw - 1, nullptr),
                ATTN_ERR_WORKSPACE, "select workspace short");
  select_params sd = s;
  sd.seqlen = 3;
  sd.seqlen_kv = 8192;
  sd.q_pos0 = 8000;
  const size_t sdw = block_select_workspace_bytes(&sd);
  expect(sdw > selw / 4, "decode select workspace with partial lists");
  expect_status(block_select(&sd, fake(1), fake(2), (int32_t*)fake(3), fake(20), sdw, nullptr), ATTN_OK,
                "decode select");
  unsigned char* v1 = (unsigned char*)malloc(SELECT_PARAMS_V1_SIZE);
  memcpy(v1, &s, SELECT_PARAMS_V1_SIZE);
  const uint32_t v1size = SELECT_PARAMS_V1_SIZE;
  memcpy(v1, &v1size, sizeof v1size);
  expect(block_select_workspace_bytes((const select_params*)v1) == selw, "select v1 workspace");
  expect_status(block_select((const select_params*)v1, fake(1), fake(2), (int32_t*)fake(3), fake(20), selw, nullptr),
                ATTN_OK, "select v1 struct");
  free(v1);
  select_params sb = s;
  sb.embed = 100;
  expect_status(block_select(&sb, fake(1), fake(2), (int32_t*)fake(3), fake(20), selw, nullptr), ATTN_ERR_UNSUPPORTED,
                "embed 100");

  expect(attn_abi_version() == ATTN_PARAMS_VERSION, "abi version");
  expect_status(fwd(&p), ATTN_OK, "success after failures");
  expect(attn_last_error()[0] == '\0', "a success clears the message");
  printf("abi_checks: %d checks passed, %d launches\n", checks, rea::launches);
  return 0;
}
