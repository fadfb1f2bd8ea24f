"""Debug mode (rd_set_debug): device-side contents are checked before any kernel of the call runs.

With valid contents a call gives exactly what it gives without debug mode.
A length past its capacity, an unpacker slot past the packed width or a
block-table entry naming no page makes the call return RD_E_CONTENT and
leave its outputs untouched (the checked kernels never run on bad values).
"""
import sys

import numpy as np
import pytest
import torch

import tree_attention_verification_rd_amd as rd
from synthetic import get_config, base_seed
from harness import Problem

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    rd.load_library()


@pytest.fixture
def debug_on():
    prev = rd.rd_set_debug(True)
    yield
    rd.rd_set_debug(prev)


def expect_content_error(fn):
    with pytest.raises(rd.RdError) as ei:
        fn()
    assert ei.value.code == rd.RD_E_CONTENT


def test_valid_contents_give_the_plain_results(debug_on):
    cfg = get_config("llama_mha").with_(B=3, W=4, L=4, Hq=4, Hkv=4, S=200, V=512)
    prob = Problem(cfg, 31, plant=True)
    say("[debug] valid step with debug mode on and off")
    on = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                        prob.hidden, prob.weight)
    torch.cuda.synchronize()
    rd.rd_set_debug(False)
    off = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight)
    torch.cuda.synchronize()
    rd.rd_set_debug(True)
    for key in ("attn", "argmax", "unpacked", "best_beam", "accept_len", "accepted_tokens"):
        assert torch.equal(on[key], off[key]), key
    # logits rows past a request's packed length are never written
    for b, n in enumerate(prob.pack["length"]):
        assert torch.equal(on["logits"][b, :n], off["logits"][b, :n])


def test_bad_contents_are_reported_before_launching(debug_on):
    cfg = get_config("llama_mha").with_(B=3, W=4, L=4, Hq=4, Hkv=4, S=200, V=512)
    prob = Problem(cfg, 32)
    pk, mask = rd.rd_pack_beams_mask(prob.beams_t)
    out = torch.full_like(prob.q, 7.0)
    bad_kv = prob.kv_len_t.clone()
    bad_kv[1] = cfg.S + 1
    say("[debug] kv_len past the cache")
    expect_content_error(lambda: rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache,
                                                      bad_kv, mask, pk["length"], out=out))
    bad_len = pk["length"].clone()
    bad_len[0] = cfg.P_max + 1
    say("[debug] packed_len past the packed width")
    expect_content_error(lambda: rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache,
                                                      prob.kv_len_t, mask, bad_len, out=out))
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a rejected call must not write its output"
    bad_un = pk["unpacker"].clone()
    bad_un[2, 1, 3] = cfg.P_max
    argmax = torch.zeros((cfg.B, cfg.P_max), dtype=torch.int32, device="cuda")
    say("[debug] unpacker slot past the packed width")
    expect_content_error(lambda: rd.rd_unpack_accept(prob.beams_t, bad_un, argmax))
    expect_content_error(lambda: rd.rd_tree_mask(bad_un, pk["length"]))
    # commit: kv_len past the cache
    best = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    nacc = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    kc0 = prob.k_cache.clone()
    say("[debug] commit with kv_len past the cache")
    expect_content_error(lambda: rd.rd_commit_accepted(pk["unpacker"], best, nacc, prob.k_new, prob.v_new,
                                                       prob.k_cache, prob.v_cache, bad_kv))
    torch.cuda.synchronize()
    assert torch.equal(prob.k_cache, kc0)
    assert int(bad_kv[1]) == cfg.S + 1


def test_paged_table_entry_naming_no_page(debug_on):
    cfg = get_config("llama_mha").with_(B=2, W=4, L=4, Hq=4, Hkv=4, S=256, V=512)
    prob = Problem(cfg, 33, kv_len=np.array([256, 100], np.int32))
    pk, mask = rd.rd_pack_beams_mask(prob.beams_t)
    ps = 64
    npg = cfg.S // ps
    pool_k = prob.k_cache.reshape(cfg.B, cfg.Hkv, npg, ps, cfg.D).permute(0, 2, 1, 3, 4).reshape(
        cfg.B * npg, cfg.Hkv, ps, cfg.D).contiguous()
    pool_v = prob.v_cache.reshape(cfg.B, cfg.Hkv, npg, ps, cfg.D).permute(0, 2, 1, 3, 4).reshape(
        cfg.B * npg, cfg.Hkv, ps, cfg.D).contiguous()
    table = torch.arange(cfg.B * npg, dtype=torch.int32, device="cuda").reshape(cfg.B, npg)
    table[1, 2:] = -1            # past request 1's 100 cached tokens: never read, allowed
    ok = rd.rd_tree_attention_paged(prob.q, prob.k_new, prob.v_new, pool_k, pool_v, table, prob.kv_len_t, mask,
                                    pk["length"])
    ref = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t, mask,
                               pk["length"])
    torch.cuda.synchronize()
    assert torch.equal(ok, ref)
    table[1, 1] = -1             # position 64..99 of request 1 would read it
    say("[debug] paged table entry below kv_len naming no page")
    expect_content_error(lambda: rd.rd_tree_attention_paged(prob.q, prob.k_new, prob.v_new, pool_k, pool_v, table,
                                                            prob.kv_len_t, mask, pk["length"]))
