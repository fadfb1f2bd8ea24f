"""GPU parity of ragged batches (per-request beam count and length).

rd_pack_beams_mask_ragged and rd_unpack_accept_ragged against the oracle's
ragged pack, mask, unpack and greedy accept, bit-exactly; full widths must
reproduce the plain calls; and a whole ragged verification step must match
the oracle alone: its pack and mask on every request, and on the checked
requests its attention (per-beam definition), its greedy targets (fp64
logits with enforced margins) and the accept that follows from them.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, base_seed, draw_beams
from harness import Problem, TOL, mask_words_np, normwise_rows, to_np, fmt_err

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    rd.load_library()


def dev_int(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def ragged_widths(rng, B, W, L):
    bw = rng.integers(1, W + 1, size=B).astype(np.int32)
    bl = rng.integers(1, L + 1, size=B).astype(np.int32)
    bw[0], bl[0] = W, L         # one full request
    if B > 2:
        bw[1] = 0               # no beam
        bl[2] = 0               # no position
    if B > 3:
        bw[3], bl[3] = W + 5, -2   # clamped to W and 0
    return bw, bl


@pytest.mark.parametrize("W,L,V", [(8, 5, 3), (64, 8, 2), (64, 16, 3), (16, 16, 2), (1, 1, 2), (37, 11, 2)])
def test_ragged_pack_mask_unpack_accept(W, L, V):
    rng = np.random.default_rng(W * 100 + L + V)
    B = 24
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    bw, bl = ragged_widths(rng, B, W, L)
    ref = oracle.pack_beams(beams, bw, bl)
    got, mask = rd.rd_pack_beams_mask_ragged(dev_int(beams), dev_int(bw), dev_int(bl))
    torch.cuda.synchronize()
    for key in ("tokens", "length", "unpacker", "depth", "src"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(mask_words_np(mask),
                                  oracle.mask_to_bits(oracle.tree_mask(ref["unpacker"], ref["length"])),
                                  err_msg="mask")
    # accept on target choices from a small vocabulary (many matches), and the unpack of a packed array
    pargmax = rng.integers(0, V, size=(B, W * L)).astype(np.int32)
    pargmax[np.arange(W * L)[None, :] >= ref["length"][:, None]] = -1
    un = ref["unpacker"].reshape(B, -1)
    target = np.take_along_axis(pargmax, np.maximum(un, 0), axis=1).reshape(B, W, L)
    acc = oracle.greedy_accept(beams, target, bw, bl)
    packed = rng.standard_normal((B, W * L, 3)).astype(np.float32)
    res = rd.rd_unpack_accept_ragged(dev_int(beams), dev_int(bw), dev_int(bl), got["unpacker"], dev_int(pargmax),
                                     torch.from_numpy(packed).cuda())
    torch.cuda.synchronize()
    for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), acc[key], err_msg=key)
    np.testing.assert_array_equal(res["unpacked"].cpu().numpy(), oracle.unpack(packed, ref["unpacker"]))
    if L > 1 and W > 1:
        assert acc["accept_len"].max() > 0
    say(f"[ragged] W={W} L={L}: {int((ref['length'] == 0).sum())} empty requests, exact")


def test_full_widths_reproduce_the_plain_calls():
    cfg = get_config("dedup_p0.5")
    beams = draw_beams(cfg, base_seed(cfg, 3))
    B, W, L = beams.shape
    full = np.full(B, W, np.int32), np.full(B, L, np.int32)
    a, ma = rd.rd_pack_beams_mask(dev_int(beams))
    b, mb = rd.rd_pack_beams_mask_ragged(dev_int(beams), dev_int(full[0]), dev_int(full[1]))
    torch.cuda.synchronize()
    for key in ("tokens", "length", "unpacker", "depth", "src"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(ma, mb)


def test_ragged_verify_step_end_to_end():
    """A ragged llama_mha-shaped step against the oracle alone: pack and mask on every request;
    attention, greedy targets and the accept on checked requests with planted acceptance."""
    cfg = get_config("llama_mha")
    rng = np.random.default_rng(7)
    B, W, L, P = cfg.B, cfg.W, cfg.L, cfg.P_max
    bw, bl = ragged_widths(rng, B, W, L)
    checked = [0, 1, 2, 3, 5, B - 1]
    prob = Problem(cfg, base_seed(cfg, 5), checked=checked, plant=True, beam_width=bw, beam_len=bl)
    say(f"[ragged] step: widths {bw.tolist()} lengths {bl.tolist()}")
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache,
                         prob.kv_len_t, prob.hidden, prob.weight, want_logits=True,
                         beam_width=dev_int(bw), beam_len=dev_int(bl))
    torch.cuda.synchronize()
    prob.assert_pack_matches(res["pack"], res["mask"])
    ref = prob.pack
    am = res["argmax"].cpu().numpy()
    assert (am[np.arange(P)[None, :] >= ref["length"][:, None]] == -1).all()
    # the oracle's own greedy targets, attention and accept on the checked requests
    logits_ref = prob.oracle_logits()
    target = oracle.argmax_first(logits_ref)
    acc = prob.oracle_accept(target)
    attn_ref = prob.oracle_attention()
    attn = to_np(res["attn"])
    logits = to_np(res["logits"])
    bw_c = np.clip(bw, 0, W)
    bl_c = np.clip(bl, 0, L)
    errs, lerrs = [], []
    for i, b in enumerate(checked):
        for w in range(int(bw_c[b])):
            for l in range(int(bl_c[b])):
                slot = int(ref["unpacker"][b, w, l])
                assert am[b, slot] == target[i, w, l], f"argmax b={b} w={w} l={l}"
                errs.append(normwise_rows(attn[b, slot], attn_ref[i, w, l]))
                lerrs.append(normwise_rows(logits[b, slot], logits_ref[i, w, l]))
    errs, lerrs = np.asarray(errs), np.asarray(lerrs)
    say(f"[ragged] step: attention normwise {fmt_err(errs)}, logits {fmt_err(lerrs)}")
    assert errs.max() <= TOL[cfg.dtype] and lerrs.max() <= TOL[cfg.dtype]
    for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(res[key].cpu().numpy()[checked], acc[key], err_msg=key)
    assert acc["accept_len"].max() > 0
    # padding candidates unpack to zero rows, valid ones carry their slot's logits
    unp = res["unpacked"]
    pad = torch.from_numpy(ref["unpacker"] < 0).to(unp.device)
    assert (unp[pad] == 0).all()
    for b in range(B):
        for w in range(int(bw_c[b])):
            for l in range(int(bl_c[b])):
                assert torch.equal(unp[b, w, l], res["logits"][b, ref["unpacker"][b, w, l]])
