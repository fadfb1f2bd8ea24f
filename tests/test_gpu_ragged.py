"""GPU parity of ragged batches (per-request beam count and length).

rd_pack_beams_mask_ragged and rd_unpack_accept_ragged against the oracle's
ragged pack, mask, unpack and greedy accept, bit-exactly; full widths must
reproduce the plain calls; and a whole ragged verification step must accept
what the oracle accepts from the step's own target choices.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, base_seed, draw_beams
from harness import mask_words_np

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
    """A ragged llama_mha-shaped step: the accept equals the oracle's on the step's own target choices."""
    cfg = get_config("llama_mha")
    rng = np.random.default_rng(7)
    beams_np = draw_beams(cfg, base_seed(cfg, 5))
    B, W, L, P = cfg.B, cfg.W, cfg.L, cfg.P_max
    bw, bl = ragged_widths(rng, B, W, L)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(11)

    def rn(shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev) * scale).to(torch.bfloat16)

    q, kn, vn = rn((B, P, cfg.Hq, cfg.D)), rn((B, P, cfg.Hkv, cfg.D)), rn((B, P, cfg.Hkv, cfg.D))
    kc, vc = rn((B, cfg.Hkv, cfg.S, cfg.D)), rn((B, cfg.Hkv, cfg.S, cfg.D))
    hidden = rn((B, P, cfg.hidden))
    weight = rn((cfg.V, cfg.hidden), 0.02)
    kv_len = torch.full((B,), cfg.S, dtype=torch.int32, device=dev)
    res = rd.verify_step(dev_int(beams_np), q, kn, vn, kc, vc, kv_len, hidden, weight, want_logits=True,
                         beam_width=dev_int(bw), beam_len=dev_int(bl))
    torch.cuda.synchronize()
    ref = oracle.pack_beams(beams_np, bw, bl)
    for key in ("tokens", "length", "unpacker"):
        np.testing.assert_array_equal(res["pack"][key].cpu().numpy(), ref[key], err_msg=key)
    am = res["argmax"].cpu().numpy()
    assert (am[np.arange(P)[None, :] >= ref["length"][:, None]] == -1).all()
    un = ref["unpacker"].reshape(B, -1)
    target = np.take_along_axis(am, np.maximum(un, 0), axis=1).reshape(B, W, L)
    acc = oracle.greedy_accept(beams_np, target, bw, bl)
    for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), acc[key], err_msg=key)
    unp = res["unpacked"]
    pad = torch.from_numpy(ref["unpacker"] < 0).to(dev)
    assert (unp[pad] == 0).all()
    # valid candidates carry their slot's logits
    for b in range(B):
        for w in range(int(min(max(bw[b], 0), W))):
            for l in range(int(min(max(bl[b], 0), L))):
                assert torch.equal(unp[b, w, l], res["logits"][b, ref["unpacker"][b, w, l]])
