"""The C-ABI library loads and exports every entry point include/rd.h declares (CPU only).

Only calls that return before touching the HIP runtime are made here:
status strings, the version, and host-side argument validation.
"""
import ctypes
import os
import re

import pytest

import tree_attention_verification_rd_amd as rd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rd_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("rd_pack_beams", "rd_tree_mask", "rd_tree_attention", "rd_lm_head_argmax", "rd_unpack_accept",
              "rd_commit_accepted"):
        assert n in names
    assert set(names) == set(rd.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    assert os.path.exists(rd.lib_path()), "build librd.so first (python __graft_entry__.py)"
    lib = ctypes.CDLL(rd.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = rd.load_library()
    for code, word in ((0, b"RD_OK"), (-1, b"RD_E_ARG"), (-2, b"RD_E_UNSUPPORTED"), (-3, b"RD_E_WORKSPACE"),
                       (-4, b"RD_E_HIP"), (-5, b"RD_E_CONTENT")):
        assert lib.rd_status_string(code).startswith(word)
    assert lib.rd_version() >= 100


def test_host_side_validation_without_device():
    lib = rd.load_library()
    null = None
    # negative sizes -> RD_E_ARG before any launch
    assert lib.rd_pack_beams(null, -1, 4, 4, null, null, null, null, null, null) == -1
    assert lib.rd_tree_mask(null, null, 2, -3, 4, null, null) == -1
    # empty batches are no-ops, even with null pointers
    assert lib.rd_pack_beams(null, 0, 4, 4, null, null, null, null, null, null) == 0
    assert lib.rd_pack_beams(null, 3, 0, 4, null, null, null, null, null, null) == 0
    assert lib.rd_unpack_accept(null, null, null, null, null, 1, 8, 2, 4, 0, null, null, null, null, null) == 0
    # missing required pointers
    assert lib.rd_pack_beams(null, 2, 4, 4, null, null, null, null, null, null) == -1
    # limits: W > 64, L > 16 (pointers are not dereferenced on the host)
    fake = ctypes.c_void_p(0x1000)
    assert lib.rd_pack_beams(fake, 2, 65, 4, fake, fake, fake, null, null, null) == -2
    assert lib.rd_pack_beams(fake, 2, 4, 17, fake, fake, fake, null, null, null) == -2
    assert lib.rd_pack_beams_mask(fake, 2, 4, 17, fake, fake, fake, null, null, fake, null) == -2
    assert lib.rd_pack_beams_mask(fake, 2, 4, 4, fake, fake, fake, null, null, null, null) == -1
    assert lib.rd_pack_beams_mask(null, 0, 4, 4, null, null, null, null, null, null, null) == 0
    # attention: unsupported dtype / head dim, bad head grouping, negative scale
    args = [fake] * 8
    assert lib.rd_tree_attention(7, *args, 2, 8, 4, 4, 128, 64, 0.0, fake, fake, 0, null) == -2
    assert lib.rd_tree_attention(1, *args, 2, 8, 4, 4, 96, 64, 0.0, fake, fake, 0, null) == -2
    assert lib.rd_tree_attention(1, *args, 2, 8, 6, 4, 128, 64, 0.0, fake, fake, 0, null) == -1
    assert lib.rd_tree_attention(1, *args, 2, 8, 4, 4, 128, 64, -1.0, fake, fake, 0, null) == -1
    assert lib.rd_tree_attention(1, *args, 0, 8, 4, 4, 128, 64, 0.0, fake, fake, 0, null) == 0
    # paged attention: bf16 pages must hold whole 64-key tiles; bad page size; empty batch
    pa = [fake] * 5  # q, k_new, v_new, k_pages, v_pages
    assert lib.rd_tree_attention_paged(1, *pa, 8, 32, fake, 4, fake, fake, fake, 2, 8, 4, 4, 128, 0.0, fake, fake,
                                       1 << 20, null) == -2
    assert lib.rd_tree_attention_paged(1, *pa, 8, 0, fake, 4, fake, fake, fake, 2, 8, 4, 4, 128, 0.0, fake, fake,
                                       1 << 20, null) == -1
    assert lib.rd_tree_attention_paged(1, *pa, 8, 64, null, 4, fake, fake, fake, 2, 8, 4, 4, 128, 0.0, fake, fake,
                                       1 << 20, null) == -1
    assert lib.rd_tree_attention_paged(1, *pa, 8, 64, fake, 4, fake, fake, fake, 0, 8, 4, 4, 128, 0.0, fake, fake,
                                       0, null) == 0
    # stochastic accept: unknown dtype, null q, small workspace, empty batch
    st = [fake] * 7  # unpacker, packed_len, packed_tokens, logits, q, u_accept, u_bonus
    assert lib.rd_stochastic_accept(5, *st, 2, 8, 5, 1000, fake, fake, fake, null, fake, 1 << 20, null) == -2
    st_noq = [fake, fake, fake, fake, null, fake, fake]
    assert lib.rd_stochastic_accept(1, *st_noq, 2, 8, 5, 1000, fake, fake, fake, null, fake, 1 << 20, null) == -1
    assert lib.rd_stochastic_accept(1, *st, 2, 8, 5, 1000, fake, fake, fake, null, fake, 16, null) == -3
    assert lib.rd_stochastic_accept(1, *st, 0, 8, 5, 1000, fake, fake, fake, null, null, 0, null) == 0
    assert lib.rd_stochastic_accept_workspace_size(2, 8, 5) == 2 * 40 * (8 + 4)   # per slot: test pair, bonus
    # projection: K not a multiple of 8 in bf16, unknown dtype, empty
    assert lib.rd_lm_head_argmax(1, fake, fake, fake, 2, 8, 100, 50, fake, fake, fake, 1 << 20, null) == -2
    assert lib.rd_lm_head_argmax(5, fake, fake, fake, 2, 8, 128, 50, fake, fake, fake, 1 << 20, null) == -2
    assert lib.rd_lm_head_argmax(1, fake, fake, fake, 0, 8, 128, 50, fake, fake, fake, 0, null) == 0
    # unpack/accept: unknown dtype
    assert lib.rd_unpack_accept(fake, fake, fake, fake, fake, 9, 8, 2, 4, 3, fake, fake, fake, fake, null) == -2
    # commit: empty batch, null cache, hidden without hidden_next, zero heads, unknown dtype, L > 16
    c = [fake] * 6      # unpacker, best_beam, accept_len, k_new, v_new, hidden
    o = [fake] * 4      # k_cache, v_cache, kv_len, hidden_next
    assert lib.rd_commit_accepted(1, *c, 0, 8, 5, 32, 128, 4096, 1024, *o, null) == 0
    assert lib.rd_commit_accepted(1, *c, 2, 8, 5, 32, 128, 4096, 1024, null, fake, fake, fake, null) == -1
    assert lib.rd_commit_accepted(1, *c, 2, 8, 5, 32, 128, 4096, 1024, fake, fake, fake, null, null) == -1
    assert lib.rd_commit_accepted(1, *c, 2, 8, 5, 0, 128, 4096, 1024, *o, null) == -1
    assert lib.rd_commit_accepted(1, *c, 2, 8, 5, 32, 128, 4096, -1, *o, null) == -1
    assert lib.rd_commit_accepted(3, *c, 2, 8, 5, 32, 128, 4096, 1024, *o, null) == -2
    assert lib.rd_commit_accepted(1, *c, 2, 8, 17, 32, 128, 4096, 1024, *o, null) == -2
    # paged commit: page size 0, null table, unknown dtype
    assert lib.rd_commit_accepted_paged(1, *c, 2, 8, 5, 32, 128, 4096, fake, fake, 16, 0, fake, 4, fake, fake,
                                        null) == -1
    assert lib.rd_commit_accepted_paged(1, *c, 2, 8, 5, 32, 128, 4096, fake, fake, 16, 64, null, 4, fake, fake,
                                        null) == -1
    assert lib.rd_commit_accepted_paged(4, *c, 2, 8, 5, 32, 128, 4096, fake, fake, 16, 64, fake, 4, fake, fake,
                                        null) == -2


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(rd, "_lib", None)
    monkeypatch.setattr(rd, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        rd.load_library()


def test_knobs_and_debug_switch():
    """Knobs take non-negative values for the three known knobs and return the previous value;
    the debug switch returns its previous setting.  Neither touches the device."""
    lib = rd.load_library()
    for knob in (rd.RD_KNOB_ATTN_SPLITS, rd.RD_KNOB_ATTN_FEWROW, rd.RD_KNOB_LM_SHAPE):
        assert lib.rd_set_knob(knob, 3) == 0
        assert lib.rd_set_knob(knob, 0) == 3
    assert lib.rd_set_knob(0, 1) == -1
    assert lib.rd_set_knob(4, 1) == -1
    assert lib.rd_set_knob(rd.RD_KNOB_ATTN_SPLITS, -2) == -1
    prev = lib.rd_set_debug(1)
    assert lib.rd_set_debug(0) == 1
    lib.rd_set_debug(prev)
    # debug mode only adds device-side checks: host validation still comes first, without a device
    lib.rd_set_debug(1)
    try:
        fake = ctypes.c_void_p(0x1000)
        assert lib.rd_tree_mask(None, None, 2, -3, 4, None, None) == -1
        assert lib.rd_pack_beams(fake, 2, 65, 4, fake, fake, fake, None, None, None) == -2
    finally:
        lib.rd_set_debug(prev)
