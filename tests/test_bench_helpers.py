"""Host logic of bench.py that its reported figures rest on (CPU only).

* kernel_source_sha, the key under which profiles/ records measured HBM traffic: a
  change to a comment or to blank space keeps it, any change to the code (an operator,
  a literal, a string) changes it, and comment markers inside string literals are code;
* visible_pairs, the pair count every algorithmic flop figure is built on, against a
  count over an explicit mask.
"""
import os
import shutil

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources with bench.py's hash pointed at it."""
    shutil.copytree(os.path.join(ROOT, "ring_exact_attention_amd", "csrc"),
                    tmp_path / "ring_exact_attention_amd" / "csrc")
    (tmp_path / "include").mkdir()
    shutil.copy(os.path.join(ROOT, "include", "attn.h"), tmp_path / "include" / "attn.h")
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    return tmp_path


def edit(path, old, new):
    text = path.read_text()
    assert old in text
    path.write_text(text.replace(old, new, 1))


def test_source_hash_ignores_comments_only(tree):
    base = bench.kernel_source_sha()
    hdr = tree / "include" / "attn.h"
    edit(hdr, "#define ATTN_PARAMS_VERSION", "/* a new block comment */\n//  and a line comment\n#define ATTN_PARAMS_VERSION")
    api = tree / "ring_exact_attention_amd" / "csrc" / "api.cpp"
    edit(api, "int reverse_order() {", "int   reverse_order()   {  // spacing and a comment")
    assert bench.kernel_source_sha() == base
    edit(api, '"ATTN_REVERSE_WORKGROUPS"', '"ATTN_REVERSE_WORKGROUPZ"')     # a string literal
    changed = bench.kernel_source_sha()
    assert changed != base
    fwd = tree / "ring_exact_attention_amd" / "csrc" / "fwd.hip"
    edit(fwd, "a.Sq", "a.Skv")                                             # code
    assert bench.kernel_source_sha() not in (base, changed)


def test_comment_markers_in_strings_are_code(tree):
    api = tree / "ring_exact_attention_amd" / "csrc" / "api.cpp"
    edit(api, "int reverse_order() {", 'static const char* kUrl = "a//b /* c */";\nint reverse_order() {')
    one = bench.kernel_source_sha()
    edit(api, '"a//b /* c */"', '"a//b /* d */"')
    assert bench.kernel_source_sha() != one


@pytest.mark.parametrize("Sq,Skv,causal,window,q0,k0", [
    (37, 53, True, (-1, -1), 16, 0), (64, 64, False, (5, 3), 0, 0), (40, 90, False, (-1, 7), 0, 25),
    (33, 33, True, (4, 0), 0, 0), (20, 70, False, (-1, -1), 0, 0)])
def test_visible_pairs_counts_the_mask(Sq, Skv, causal, window, q0, k0):
    i = np.arange(Sq)[:, None] + q0
    j = np.arange(Skv)[None, :] + k0
    vis = np.ones((Sq, Skv), dtype=bool)
    if causal:
        vis &= j <= i
    if window[0] >= 0:
        vis &= j >= i - window[0]
    if window[1] >= 0:
        vis &= j <= i + window[1]
    assert bench.visible_pairs(Sq, Skv, causal, window, q0, k0) == int(vis.sum())
