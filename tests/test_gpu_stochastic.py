"""GPU parity of stochastic verification (rd_stochastic_accept).

Every decision of the walk compares floats (u*q(x) < p(x), and the running
sum of p against u_bonus*total), computed in fp32 on the GPU and in fp64 by
the oracle.  So a request is compared only when its outcome is robust: the
oracle must give the same result with every uniform nudged by a relative
1e-4 and the bonus uniform by 3e-5; otherwise the request's uniforms are
redrawn (seeded).  Compared outputs (accept length, best beam, accepted
tokens, walk path) must then match bit-exactly.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, draw_beams, base_seed, round_to_bf16

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


def softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def robust_uniforms(beams_b, pk_b, logits_b, q_b, rng, W, L, tries=40):
    """Uniforms for one request whose oracle outcome survives small nudges."""
    keys = ("accept_len", "best_beam", "accepted_tokens", "path")
    for _ in range(tries):
        ua = rng.random((1, L, W))
        ub = rng.random(1)
        outs = []
        for fa, db in ((1.0, 0.0), (1 + 1e-4, 0.0), (1 - 1e-4, 0.0), (1.0, 3e-5), (1.0, -3e-5)):
            r = oracle.stochastic_accept(beams_b, pk_b["unpacker"], pk_b["length"], pk_b["tokens"], logits_b, q_b,
                                         ua * fa, np.clip(ub + db, 0, 1 - 1e-12))
            outs.append(tuple(r[k].tobytes() for k in keys))
        if all(o == outs[0] for o in outs):
            return ua, ub, oracle.stochastic_accept(beams_b, pk_b["unpacker"], pk_b["length"], pk_b["tokens"],
                                                    logits_b, q_b, ua, ub)
    raise RuntimeError("no robust uniforms found")


CASES = {
    # name: (B, W, L, V, dtype, logit scale, q mix with p)
    "small_v": (6, 4, 4, 64, "bf16", 2.0, 0.7),
    "f32": (5, 3, 5, 300, "f32", 1.5, 0.5),
    "llama_vocab": (8, 8, 5, 32000, "bf16", 3.0, 0.9),
    "wide": (3, 64, 8, 1000, "bf16", 2.5, 0.8),
    "odd_vocab": (4, 4, 4, 1003, "bf16", 2.0, 0.8),      # register-resident rows loaded entry by entry
    "big_vocab": (2, 3, 4, 40000, "bf16", 2.5, 0.8),   # beyond the register-resident row size: streamed passes
    "big_vocab_f32": (2, 3, 4, 36000, "f32", 2.5, 0.8),  # streamed 16-byte groups of f32 logits
    "big_vocab_odd": (2, 3, 4, 40003, "bf16", 2.5, 0.8),  # not a multiple of 8: streamed entry by entry
    "vocab_128k": (1, 4, 3, 128256, "bf16", 3.0, 0.9),    # the 128256-entry vocabulary of the GQA workloads
    "vocab_32768": (2, 4, 4, 32768, "bf16", 2.5, 0.8),    # the largest register-resident row: no group past the row
    "vocab_32776": (2, 4, 4, 32776, "bf16", 2.5, 0.8),    # one 8-entry group more: streamed passes
}


@pytest.mark.parametrize("name", list(CASES))
def test_stochastic_against_oracle(name):
    B, W, L, V, dtype, scale, mix = CASES[name]
    cfg = get_config("llama_mha").with_(B=B, W=W, L=L, V=V)
    beams = draw_beams(cfg, base_seed(cfg, 6))
    beams[:, :, 0] = beams[:, :1, 0]                      # one shared initial token per request
    beams = beams % V
    P = W * L
    rng = np.random.default_rng(101 + list(CASES).index(name))
    logits = (rng.standard_normal((B, P, V)) * scale).astype(np.float32)
    if dtype == "bf16":
        logits = round_to_bf16(logits)
    noise = softmax(rng.standard_normal((B, P, V)) * scale)
    q = (mix * softmax(logits.astype(np.float64)) + (1 - mix) * noise).astype(np.float32)
    pk = oracle.pack_beams(beams)
    ua = np.zeros((B, L, W), np.float32)
    ub = np.zeros(B, np.float32)
    for b in range(B):
        sl = slice(b, b + 1)
        pk_b = {k: v[sl] for k, v in pk.items()}
        a_, b_, _ = robust_uniforms(beams[sl], pk_b, logits[sl].astype(np.float64), q[sl].astype(np.float64),
                                     rng, W, L)
        ua[b], ub[b] = a_[0], b_[0]
    # the oracle saw the float32 values the device gets
    ua = ua.astype(np.float32)
    ub = ub.astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gpk = rd.rd_pack_beams(dev_int(beams))
    got = rd.rd_stochastic_accept(gpk["unpacker"], gpk["length"], gpk["tokens"], torch.from_numpy(logits).cuda().to(tdt),
                                  torch.from_numpy(q).cuda(), torch.from_numpy(ua).cuda(), torch.from_numpy(ub).cuda())
    torch.cuda.synchronize()
    for key in ("tokens", "length", "unpacker"):
        np.testing.assert_array_equal(gpk[key].cpu().numpy(), pk[key], err_msg=key)
    nacc = []
    for b in range(B):
        # the oracle ran on float64 copies of the float32 uniforms drawn above: rerun on exactly those
        pk_b = {k: v[b:b + 1] for k, v in pk.items()}
        ref = oracle.stochastic_accept(beams[b:b + 1], pk_b["unpacker"], pk_b["length"], pk_b["tokens"],
                                       logits[b:b + 1].astype(np.float64), q[b:b + 1].astype(np.float64),
                                       ua[b:b + 1].astype(np.float64), ub[b:b + 1].astype(np.float64))
        for key in ("accept_len", "best_beam", "accepted_tokens", "path"):
            np.testing.assert_array_equal(got[key][b].cpu().numpy(), ref[key][0], err_msg=f"b={b} {key}")
        nacc.append(int(ref["accept_len"][0]))
    say(f"[stochastic] {name}: accept lengths {nacc}")


def test_peaked_targets_match_the_greedy_accept():
    """Targets one logit 40 above the rest: the walk equals the greedy accept on their argmax."""
    B, W, L, V = 8, 8, 5, 32000
    cfg = get_config("llama_mha").with_(B=B, W=W, L=L, V=V)
    rng = np.random.default_rng(21)
    beams = draw_beams(cfg, base_seed(cfg, 7))
    beams[:, :, 0] = beams[:, :1, 0]
    pk = oracle.pack_beams(beams)
    P = W * L
    # aim the targets at the next beam token for part of the slots, so paths get accepted
    tgt = rng.integers(0, V, size=(B, P))
    for b in range(B):
        for w in range(W):
            for l in range(L - 1):
                if rng.random() < 0.7:
                    tgt[b, pk["unpacker"][b, w, l]] = beams[b, w, l + 1]
    logits = rng.standard_normal((B, P, V)).astype(np.float32)
    np.put_along_axis(logits, tgt[..., None], 40.0, axis=2)
    logits = round_to_bf16(logits)
    q = softmax(rng.standard_normal((B, P, V))).astype(np.float32)
    gpk = rd.rd_pack_beams(dev_int(beams))
    lt = torch.from_numpy(logits).cuda().to(torch.bfloat16)
    got = rd.rd_stochastic_accept(gpk["unpacker"], gpk["length"], gpk["tokens"], lt, torch.from_numpy(q).cuda(),
                                  torch.from_numpy(rng.random((B, L, W)).astype(np.float32)).cuda(),
                                  torch.from_numpy(rng.random(B).astype(np.float32)).cuda())
    argmax = torch.from_numpy(tgt.astype(np.int32)).cuda()
    argmax[torch.arange(P, device="cuda")[None, :] >= gpk["length"][:, None]] = -1
    greedy = rd.rd_unpack_accept(dev_int(beams), gpk["unpacker"], argmax)
    torch.cuda.synchronize()
    for key in ("accept_len", "best_beam", "accepted_tokens"):
        assert torch.equal(got[key], greedy[key]), key
    assert int(greedy["accept_len"].max()) > 0
    say(f"[stochastic] peaked: accept lengths {greedy['accept_len'].tolist()}")


def test_stochastic_empty_requests_between_full_ones():
    """Requests with no packed slots (the first, the last and two adjacent ones) between full ones.

    With bf16 logits and V a multiple of 8 the slots are split into contiguous
    ranges of the valid ones, one range per workgroup, each range spanning
    several slots here: a range that reaches an empty request must skip it.
    Empty requests give -1 everywhere, as in the oracle.
    """
    B, W, L, V = 7, 64, 8, 4096
    empty = [0, 2, 3, 6]
    cfg = get_config("llama_mha").with_(B=B, W=W, L=L, V=V)
    beams = draw_beams(cfg, base_seed(cfg, 8))
    beams[:, :, 0] = beams[:, :1, 0]
    beams = beams % V
    P = W * L
    rng = np.random.default_rng(131)
    logits = round_to_bf16((rng.standard_normal((B, P, V)) * 2.5).astype(np.float32))
    q = (0.8 * softmax(logits.astype(np.float64)) + 0.2 * softmax(rng.standard_normal((B, P, V)) * 2.5)).astype(
        np.float32)
    pk = oracle.pack_beams(beams)
    for b in empty:
        pk["length"][b] = 0
        pk["unpacker"][b] = -1
        pk["tokens"][b] = -1
    ua = np.zeros((B, L, W), np.float32)
    ub = np.zeros(B, np.float32)
    for b in range(B):
        if b in empty:
            ua[b], ub[b] = rng.random((L, W)), rng.random()
            continue
        sl = slice(b, b + 1)
        pk_b = {k: v[sl] for k, v in pk.items()}
        a_, b_, _ = robust_uniforms(beams[sl], pk_b, logits[sl].astype(np.float64), q[sl].astype(np.float64),
                                     rng, W, L)
        ua[b], ub[b] = a_[0], b_[0]
    ua = ua.astype(np.float32)
    ub = ub.astype(np.float32)
    say(f"[stochastic] empty requests {empty}: packed lengths {pk['length'].tolist()}")
    got = rd.rd_stochastic_accept(dev_int(pk["unpacker"]), dev_int(pk["length"]), dev_int(pk["tokens"]),
                                  torch.from_numpy(logits).cuda().to(torch.bfloat16), torch.from_numpy(q).cuda(),
                                  torch.from_numpy(ua).cuda(), torch.from_numpy(ub).cuda())
    torch.cuda.synchronize()
    ref = oracle.stochastic_accept(beams, pk["unpacker"], pk["length"], pk["tokens"], logits.astype(np.float64),
                                   q.astype(np.float64), ua.astype(np.float64), ub.astype(np.float64))
    for key in ("accept_len", "best_beam", "accepted_tokens", "path"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    assert (ref["accept_len"][empty] == -1).all()
    say(f"[stochastic] accept lengths {ref['accept_len'].tolist()}")
