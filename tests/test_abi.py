"""The C ABI without a GPU: libattn.so loads, exports every function include/attn.h
declares, the ctypes structs match the C layout, and every argument check returns its
status before anything touches the device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import ring_exact_attention_amd as rea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rea.LIB_PATH):
        from ring_exact_attention_amd import build
        build.build()
    return rea.lib()


def declared_functions():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?(?:int|size_t|uint32_t|char\s*\*|void)\s*\*?\s*(\w+)\s*\(",
                            text, flags=re.M)
    return names


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "block_select",
            "block_select_workspace_bytes", "attn_last_error", "attn_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.attn_abi_version() == 6


def params(**kw):
    p = rea.AttnParams()
    p.struct_size = ctypes.sizeof(rea.AttnParams)
    base = dict(dtype=rea.ATTN_BF16, batch=1, seqlen_q=128, seqlen_kv=128, num_q_heads=4,
                num_kv_heads=2, head_dim=128, causal=1, window_left=-1, window_right=-1)
    base.update(kw)
    for k_, v_ in base.items():
        setattr(p, k_, v_)
    return p


def fwd_status(lib, p, ptr=None):
    dummy = ctypes.c_void_p(ptr)
    return lib.attn_fwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, None, None)


def test_struct_layout(lib):
    assert ctypes.sizeof(rea.AttnParams) == 208
    assert rea.AttnParams.softmax_type.offset == 104          # ATTN_PARAMS_V1_SIZE
    assert rea.AttnParams.bias.offset == 128                  # ATTN_PARAMS_V2_SIZE
    assert rea.AttnParams.drop_mask.offset == 168             # ATTN_PARAMS_V3_SIZE
    assert rea.AttnParams.o_lo.offset == 200                  # ATTN_PARAMS_V4_SIZE
    assert ctypes.sizeof(rea.SelectParams) == 40
    assert rea.SelectParams.seqlen_kv.offset == 32          # SELECT_PARAMS_V1_SIZE
    # a zero batch is a successful no-op only when the struct size matches
    assert fwd_status(lib, params(batch=0)) == rea.ATTN_OK
    p = params(batch=0)
    p.struct_size = 100
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG
    assert b"struct_size" in lib.attn_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(num_q_heads=6, num_kv_heads=4), rea.ATTN_ERR_INVALID_ARG, b"multiple"),
    (dict(num_q_heads=0), rea.ATTN_ERR_INVALID_ARG, b"> 0"),
    (dict(head_dim=48), rea.ATTN_ERR_UNSUPPORTED, b"head_dim"),
    (dict(dtype=rea.ATTN_F32, head_dim=128), rea.ATTN_ERR_UNSUPPORTED, b"head_dim"),
    (dict(dtype=7), rea.ATTN_ERR_UNSUPPORTED, b"dtype"),
    (dict(seqlen_q=-1), rea.ATTN_ERR_INVALID_ARG, b">= 0"),
    (dict(causal=1, window_right=3), rea.ATTN_ERR_INVALID_ARG, b"window_right"),
    (dict(window_left=-2), rea.ATTN_ERR_INVALID_ARG, b"-1"),
    (dict(query_chunk=48), rea.ATTN_ERR_INVALID_ARG, b"query_chunk"),
    (dict(key_chunk=96), rea.ATTN_ERR_INVALID_ARG, b"key_chunk"),
    (dict(kv_block=100), rea.ATTN_ERR_INVALID_ARG, b"kv_block"),
    (dict(flags=8), rea.ATTN_ERR_INVALID_ARG, b"flags"),
    (dict(causal=2), rea.ATTN_ERR_INVALID_ARG, b"causal"),
    (dict(q_pos0=1 << 40), rea.ATTN_ERR_UNSUPPORTED, b"q_pos0"),
    (dict(scale=float("inf")), rea.ATTN_ERR_INVALID_ARG, b"scale"),
    (dict(head_dim_v=-1), rea.ATTN_ERR_INVALID_ARG, b"head_dim_v"),
    (dict(softmax_type=3), rea.ATTN_ERR_INVALID_ARG, b"softmax_type"),
    (dict(bias=0x1002), rea.ATTN_ERR_INVALID_ARG, b"bias"),
    (dict(softmax_type=2), rea.ATTN_ERR_INVALID_ARG, b"sink"),
    (dict(softmax_type=2, sink=0x1002), rea.ATTN_ERR_INVALID_ARG, b"sink"),
    (dict(head_dim_v=32), rea.ATTN_ERR_UNSUPPORTED, b"head_dim_v"),
    (dict(head_dim=64, head_dim_v=128), rea.ATTN_ERR_UNSUPPORTED, b"head_dim_v"),
    (dict(dtype=1, head_dim=64, head_dim_v=48), rea.ATTN_ERR_UNSUPPORTED, b"head_dim_v"),
])
def test_forward_argument_checks(lib, kw, status, msg):
    assert fwd_status(lib, params(**kw)) == status
    assert msg in lib.attn_last_error()


@pytest.mark.parametrize("dtype,d,dv", [(rea.ATTN_BF16, 128, 64), (rea.ATTN_BF16, 128, 128),
                                         (rea.ATTN_BF16, 64, 0), (rea.ATTN_F32, 64, 32)])
def test_head_dim_pairs_accepted(lib, dtype, d, dv):
    """Every built (head_dim, head_dim_v) pair passes the argument checks (and then stops at
    the NULL q pointer, so nothing is launched)."""
    assert fwd_status(lib, params(dtype=dtype, head_dim=d, head_dim_v=dv)) == rea.ATTN_ERR_INVALID_ARG
    assert b"q is NULL" in lib.attn_last_error()


def test_bias_stride_checks(lib):
    p = params(bias=0x1000)
    p.bias_stride[2] = -1
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"bias_stride" in lib.attn_last_error()
    p.bias_stride[2] = 0
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"q is NULL" in lib.attn_last_error()


def test_version3_struct_is_accepted(lib):
    """A 168-byte struct (before the dropout fields) reads as having no dropout."""
    p = params(batch=1)
    p.drop_mask = 0x1002                              # misaligned, past the v3 size: ignored
    p.struct_size = 168
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"q is NULL" in lib.attn_last_error()
    p.struct_size = 208
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"drop_mask" in lib.attn_last_error()
    p.drop_mask = 0x1000
    p.drop_stride[1] = -4
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"drop_stride" in lib.attn_last_error()


def test_version4_struct_is_accepted(lib):
    """A 200-byte struct (versions 4 and 5, before o_lo) reads as having no o_lo."""
    p = params(batch=1)
    p.o_lo = 0x1002                                   # misaligned, past the v4 size: ignored
    p.struct_size = 200
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"q is NULL" in lib.attn_last_error()
    p.struct_size = 208
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"o_lo" in lib.attn_last_error()


def test_o_lo_checks(lib):
    """o_lo: bf16 dense only, 16-byte aligned; rejected in sparse mode."""
    d = ctypes.c_void_p(0x1000)
    p = params(dtype=rea.ATTN_F32, head_dim=64, o_lo=0x1000)
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"o_lo" in lib.attn_last_error()
    p = params(o_lo=0x1000)
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"q is NULL" in lib.attn_last_error()
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p))
    assert need == lib.attn_bwd_workspace_bytes(ctypes.byref(params()))
    p.o_lo = 0x1008
    st = lib.attn_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, need, None)
    assert st == rea.ATTN_ERR_INVALID_ARG and b"o_lo" in lib.attn_last_error()
    s = params(num_q_heads=1, num_kv_heads=1, head_dim=512, seqlen_q=64, seqlen_kv=64, causal=0, o_lo=0x1000)
    s.sel_idx = 0x1000
    s.top_n, s.sel_block, s.sparse_window = 8, 32, 32
    assert lib.attn_fwd(ctypes.byref(s), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_UNSUPPORTED
    assert b"o_lo" in lib.attn_last_error()


def test_version2_struct_is_accepted(lib):
    """A 128-byte struct (before the bias fields) reads as having no bias."""
    p = params(batch=1, bias=0x1002)                 # misaligned bias past the v2 size: ignored
    p.struct_size = 128
    assert fwd_status(lib, p) == rea.ATTN_ERR_INVALID_ARG and b"q is NULL" in lib.attn_last_error()


def test_version1_struct_is_accepted(lib):
    """A caller built against the 104-byte struct (no softmax fields) is read as a plain
    softmax; the bytes after it are not looked at."""
    class Big(ctypes.Structure):
        _fields_ = [("p", rea.AttnParams), ("junk", ctypes.c_char * 64)]
    big = Big()
    big.p = params(batch=0)
    big.p.struct_size = 104
    big.p.softmax_type = 77                      # beyond a version-1 struct: ignored
    assert lib.attn_fwd(ctypes.byref(big.p), None, None, None, None, None, None, None, None) == rea.ATTN_OK
    big.p.batch = 1
    assert fwd_status(lib, big.p) == rea.ATTN_ERR_INVALID_ARG
    assert b"q is NULL" in lib.attn_last_error()


def test_select_decode_checks(lib):
    """block_select with query rows at q_pos0 of a longer key sequence, and the 32-byte
    version-1 select struct (no decode fields)."""
    def sp(**kw):
        p = rea.SelectParams()
        p.struct_size = ctypes.sizeof(rea.SelectParams)
        for k_, v_ in dict(dtype=rea.ATTN_BF16, batch=1, seqlen=4, embed=512, block_size=32, top_n=8,
                           seqlen_kv=256, q_pos0=252).items():
            setattr(p, k_, v_)
        for k_, v_ in kw.items():
            setattr(p, k_, v_)
        return p
    d = ctypes.c_void_p(0x1000)
    call = lambda p: lib.block_select(ctypes.byref(p), d, d, None, d, 1 << 30, None)
    assert call(sp()) == rea.ATTN_ERR_INVALID_ARG and b"idx is NULL" in lib.attn_last_error()
    assert call(sp(q_pos0=253)) == rea.ATTN_ERR_INVALID_ARG and b"q_pos0" in lib.attn_last_error()
    assert call(sp(q_pos0=-1)) == rea.ATTN_ERR_INVALID_ARG
    # means_cached: 0 .. seqlen_kv / block_size (8 blocks here)
    assert call(sp(means_cached=-1)) == rea.ATTN_ERR_INVALID_ARG and b"means_cached" in lib.attn_last_error()
    assert call(sp(means_cached=9)) == rea.ATTN_ERR_INVALID_ARG and b"means_cached" in lib.attn_last_error()
    assert call(sp(means_cached=8)) == rea.ATTN_ERR_INVALID_ARG and b"idx is NULL" in lib.attn_last_error()
    # workspace: the means of the key sequence's full blocks (fp64), their two bf16
    # parts and their norms (fp32), each part 256-byte aligned
    means = lambda nb, e: nb * e * 8 + 2 * nb * e * 2 + (nb * 4 + 255) // 256 * 256
    assert lib.block_select_workspace_bytes(ctypes.byref(sp())) == means(8, 512)
    v1 = sp(seqlen=256, seqlen_kv=77, q_pos0=99)
    v1.struct_size = 32                                      # fields past 32 bytes ignored
    assert lib.block_select_workspace_bytes(ctypes.byref(v1)) == means(8, 512)
    assert call(v1) == rea.ATTN_ERR_INVALID_ARG and b"idx is NULL" in lib.attn_last_error()
    # few query blocks (decoding): the candidates of a block are shared out over
    # workgroups (here 4: 256 blocks = 4 chunks of 64), whose partial top-n lists
    # (fp64 score + int32 index per entry) follow the means
    dec = sp(seqlen=4, seqlen_kv=8192, q_pos0=8188)
    parts = 1 * 4 * 4 * 8
    assert lib.block_select_workspace_bytes(ctypes.byref(dec)) == means(256, 512) + parts * 8 + parts * 4


def test_sparse_forward_workspace(lib):
    """attn_fwd_workspace_bytes: 0 for dense params and for sparse calls with a full grid;
    the per-token partial results (512 + 4 floats per share) when decoding."""
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(params())) == 0
    p = params(num_q_heads=1, num_kv_heads=1, head_dim=512, seqlen_q=16, seqlen_kv=8192, causal=0, q_pos0=8176,
               batch=4)
    p.sel_idx = 0x1000
    p.top_n, p.sel_block, p.sparse_window = 8, 32, 32
    # one token per workgroup (64 groups), 4 shares of at most 1 + 8 steps
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(p)) == 4 * 16 * 4 * 516 * 4
    full = params(num_q_heads=1, num_kv_heads=1, head_dim=512, seqlen_q=8192, seqlen_kv=8192, causal=0, batch=4)
    full.sel_idx = 0x1000
    full.top_n, full.sel_block, full.sparse_window = 8, 32, 32
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(full)) == 0
    p.top_n = 0                                              # invalid: 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(p)) == 0


def test_sparse_decode_checks(lib):
    d = ctypes.c_void_p(0x1000)
    p = params(num_q_heads=1, num_kv_heads=1, head_dim=512, seqlen_q=2, seqlen_kv=64, causal=0, q_pos0=62)
    p.sel_idx = 0x1000
    p.top_n, p.sel_block, p.sparse_window = 8, 32, 32
    assert lib.attn_fwd(ctypes.byref(p), None, d, d, d, d, d, None, None) == rea.ATTN_ERR_INVALID_ARG
    assert b"q is NULL" in lib.attn_last_error()               # decoding shape accepted
    p.q_pos0 = 63
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_INVALID_ARG
    assert b"q_pos0" in lib.attn_last_error()
    p.q_pos0 = 62                                              # the gradient needs the whole sequence
    assert lib.attn_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, 1 << 30, None) == rea.ATTN_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers(lib):
    assert fwd_status(lib, params()) == rea.ATTN_ERR_INVALID_ARG
    assert b"q is NULL" in lib.attn_last_error()
    assert fwd_status(lib, params(), ptr=0x1008) == rea.ATTN_ERR_INVALID_ARG
    assert b"aligned" in lib.attn_last_error()


def test_no_finalize_needs_acc(lib):
    p = params(flags=rea.ATTN_NO_FINALIZE)
    d = ctypes.c_void_p(0x1000)
    st = lib.attn_fwd(ctypes.byref(p), d, d, d, None, d, d, None, None)
    assert st == rea.ATTN_ERR_INVALID_ARG and b"acc" in lib.attn_last_error()


def test_backward_checks(lib):
    p = params()
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p))
    # D and LSE (4*128 floats each, 256-aligned), then fp32 partial dk, dv of the two dk/dv
    # workgroups that share the GQA group's 2 q heads (causal without a left window)
    assert need == 2 * 2048 + 2 * 128 * 2 * (128 + 128) * 4
    # a left window (or a single q head per kv head) keeps one dk/dv workgroup per key tile
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(params(window_left=16))) == 2 * 2048
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(params(num_kv_heads=4))) == 2 * 2048
    d = ctypes.c_void_p(0x1000)
    st = lib.attn_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, need - 1, None)
    assert st == rea.ATTN_ERR_WORKSPACE
    st = lib.attn_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, None, need, None)
    assert st == rea.ATTN_ERR_WORKSPACE
    p2 = params(flags=rea.ATTN_CARRY_IN)
    st = lib.attn_bwd(ctypes.byref(p2), d, d, d, d, d, d, d, d, d, d, d, need, None)
    assert st == rea.ATTN_ERR_INVALID_ARG and b"flags" in lib.attn_last_error()
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(params(head_dim=48))) == 0
    # partial backward: dq may be NULL when skipped, not otherwise
    p3 = params(flags=rea.ATTN_BWD_SKIP_DQ | rea.ATTN_BWD_SKIP_DKDV | rea.ATTN_BWD_REUSE_STATS, batch=0)
    assert lib.attn_bwd(ctypes.byref(p3), d, d, d, d, d, d, d, None, None, None, d, need, None) == rea.ATTN_OK
    p4 = params(flags=rea.ATTN_BWD_SKIP_DKDV)
    st = lib.attn_bwd(ctypes.byref(p4), d, d, d, d, d, d, d, None, d, d, d, need, None)
    assert st == rea.ATTN_ERR_INVALID_ARG and b"dq is NULL" in lib.attn_last_error()
    p5 = params(flags=rea.ATTN_BWD_SKIP_DQ)
    assert lib.attn_fwd(ctypes.byref(p5), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_INVALID_ARG


def test_sparse_mode_checks(lib):
    d = ctypes.c_void_p(0x1000)
    p = params(num_q_heads=1, num_kv_heads=1, head_dim=512, seqlen_q=64, seqlen_kv=64, causal=0)
    p.sel_idx = 0x1000
    p.top_n, p.sel_block, p.sparse_window = 8, 32, 32
    p.num_q_heads = 8
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_INVALID_ARG
    p.num_q_heads = 1
    p.top_n = 17
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_INVALID_ARG
    p.top_n = 8
    p.head_dim_v = 64
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_UNSUPPORTED
    p.head_dim_v = 0
    p.softmax_type = rea.ATTN_SOFTMAX_OFF_BY_ONE
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_ERR_UNSUPPORTED
    p.softmax_type = 0
    p.batch = 0
    assert lib.attn_fwd(ctypes.byref(p), d, d, d, d, d, d, None, None) == rea.ATTN_OK


def test_select_checks(lib):
    p = rea.SelectParams()
    p.struct_size = ctypes.sizeof(rea.SelectParams)
    p.dtype, p.batch, p.seqlen, p.embed, p.block_size, p.top_n = rea.ATTN_BF16, 2, 256, 512, 32, 8
    need = lib.block_select_workspace_bytes(ctypes.byref(p))
    assert need == 16 * 512 * 8 + 2 * 16 * 512 * 2 + 256   # means, their bf16 parts, norms
    d = ctypes.c_void_p(0x1000)
    assert lib.block_select(ctypes.byref(p), d, d, d, d, need - 8, None) == rea.ATTN_ERR_WORKSPACE
    p.block_size = 24
    assert lib.block_select(ctypes.byref(p), d, d, d, d, need, None) == rea.ATTN_ERR_UNSUPPORTED
    p.block_size, p.embed = 32, 100
    assert lib.block_select(ctypes.byref(p), d, d, d, d, need, None) == rea.ATTN_ERR_UNSUPPORTED
    p.embed, p.batch = 512, 0
    assert lib.block_select(ctypes.byref(p), d, d, d, d, need, None) == rea.ATTN_OK


def test_success_clears_error(lib):
    fwd_status(lib, params(head_dim=48))
    assert lib.attn_last_error() != b""
    assert fwd_status(lib, params(batch=0)) == rea.ATTN_OK
    assert lib.attn_last_error() == b""


def test_noalloc_rejects_params_beyond_the_static_scratch(lib):
    """attn_bwd_noalloc checks the scratch its params need against the static array before
    it touches the device (so this runs without a GPU)."""
    p = params(batch=8, seqlen_q=65536, seqlen_kv=65536, num_q_heads=32, num_kv_heads=8)
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p))
    assert need > rea.NOALLOC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)
    st = lib.attn_bwd_noalloc(ctypes.byref(p), *([dummy] * 10), None)
    assert st == rea.ATTN_ERR_WORKSPACE
    assert b"static" in lib.attn_last_error()
    bad = params(num_q_heads=6, num_kv_heads=4)                 # invalid params: attn_bwd's message
    assert lib.attn_bwd_noalloc(ctypes.byref(bad), *([dummy] * 10), None) == rea.ATTN_ERR_INVALID_ARG
    assert b"multiple" in lib.attn_last_error()
    sp = params()
    sp.sel_idx = 256
    assert lib.attn_bwd_noalloc(ctypes.byref(sp), *([dummy] * 10), None) == rea.ATTN_ERR_UNSUPPORTED
