"""GPU parity of the commit of the accepted path (rd_commit_accepted).

After a verification step, the best beam's accepted keys/values are appended
to the cache and kv_len advances.  Every compared value is a copy, so every
comparison is bit-exact: against the oracle on the requests it checks, and on
every request against the expected cache built with torch indexing from the
packed inputs (rows outside the accepted path must be untouched).  The
step's pack and, on the checked requests, its accept are first asserted
equal to the oracle's (fp64 targets), and the oracle's commit is fed the
oracle's own accept.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, base_seed
from harness import Problem, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    rd.load_library()


def expected_commit(unpacker, best, nacc, k_new, k_cache, kv_len):
    """Device-side expectation built with torch indexing: (cache, kv_len) after the commit."""
    exp = k_cache.clone()
    new_len = kv_len.clone()
    B, W, L = unpacker.shape
    S = k_cache.shape[2]
    un, bb, na, kl = (t.cpu().numpy() for t in (unpacker, best, nacc, kv_len))
    for b in range(B):
        w, n, c = int(bb[b]), int(na[b]), int(kl[b])
        if not (0 <= w < W and 0 <= n < L and 0 <= c and c + n + 1 <= S):
            continue
        slots = torch.from_numpy(un[b, w, :n + 1].astype(np.int64)).to(k_new.device)
        exp[b, :, c:c + n + 1] = k_new[b, slots].transpose(0, 1)
        new_len[b] = c + n + 1
    return exp, new_len


def ragged_lengths(cfg, seed):
    """Mostly room for a full beam; one request with an empty cache, one full (always overflows)."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(0, cfg.S - cfg.L + 1, size=cfg.B).astype(np.int32)
    kv[0] = 0
    if cfg.B > 1:
        kv[-1] = cfg.S
    if cfg.B > 2:
        kv[1] = cfg.S - 1      # commits only when nothing but the initial token is accepted
    return kv


STEP = {
    "tiny_f32": None,
    "llama_mha": None,
    "gqa": [0, 13, 31],
    "dedup_p0.5": [0, 63],
}


@pytest.mark.parametrize("name", list(STEP))
def test_commit_after_verify_step(name):
    cfg = get_config(name)
    seed = base_seed(cfg, 1)
    kv_len = ragged_lengths(cfg, seed)
    say(f"[commit] {name}: building inputs, kv_len head {kv_len[:4].tolist()}")
    prob = Problem(cfg, seed, checked=STEP[name], plant=True, kv_len=kv_len)
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight, want_logits=False)
    un, best, nacc = res["pack"]["unpacker"], res["best_beam"], res["accept_len"]
    # the step's pack on every request and its accept on the checked requests are the oracle's
    # before anything below builds on them
    prob.assert_pack_matches(res["pack"])
    sub = prob.checked
    acc = prob.oracle_accept(prob.oracle_target())
    for key in ("best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(res[key].cpu().numpy()[sub], acc[key], err_msg=key)
    exp_k, exp_len = expected_commit(un, best, nacc, prob.k_new, prob.k_cache, prob.kv_len_t)
    exp_v, _ = expected_commit(un, best, nacc, prob.v_new, prob.v_cache, prob.kv_len_t)
    say(f"[commit] {name}: step done, accept_len {nacc.cpu().numpy()[:8].tolist()}; committing")
    kv_dev = prob.kv_len_t.clone()
    hnext = rd.rd_commit_accepted(un, best, nacc, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, kv_dev,
                                  prob.hidden)
    torch.cuda.synchronize()
    # every request: exact cache, length and hidden row
    assert torch.equal(kv_dev, exp_len)
    assert torch.equal(prob.k_cache, exp_k)
    assert torch.equal(prob.v_cache, exp_v)
    moved = (kv_dev != prob.kv_len_t).cpu().numpy()
    assert moved[0]
    if cfg.B > 1:
        assert not moved[-1]
    bb, na = best.cpu().numpy(), nacc.cpu().numpy()
    unp = un.cpu().numpy()
    for b in np.nonzero(moved)[0]:
        assert torch.equal(hnext[b], prob.hidden[b, int(unp[b, bb[b], na[b]])])
    # checked requests: against the oracle's commit of the oracle's own accept, which reads the
    # unpacked per-candidate tensors
    ref = oracle.commit_accepted(prob.k_unp, prob.v_unp, prob.h_unp, acc["best_beam"], acc["accept_len"],
                                 prob.kc_np, prob.vc_np, prob.kv_len[sub])
    np.testing.assert_array_equal(kv_dev.cpu().numpy()[sub], ref["kv_len"])
    np.testing.assert_array_equal(moved[sub], ref["committed"])
    for i, b in enumerate(sub):
        np.testing.assert_array_equal(to_np(prob.k_cache[b]), ref["k_cache"][i], err_msg=f"k_cache b={b}")
        np.testing.assert_array_equal(to_np(prob.v_cache[b]), ref["v_cache"][i], err_msg=f"v_cache b={b}")
        if ref["committed"][i]:
            np.testing.assert_array_equal(to_np(hnext[b]), ref["hidden_next"][i], err_msg=f"hidden b={b}")
    say(f"[commit] {name}: {int(moved.sum())}/{cfg.B} requests committed, exact")


@pytest.mark.parametrize("dtype,Hkv,D,K", [(torch.bfloat16, 3, 24, 12), (torch.float32, 2, 64, 7),
                                           (torch.bfloat16, 8, 128, 4096), (torch.float32, 1, 5, 0)])
def test_commit_direct_with_invalid_entries(dtype, Hkv, D, K):
    """Arbitrary best/accept values, out-of-range ones included; narrow and wide copy units."""
    B, W, L, S = 9, 6, 7, 40
    P = W * L
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + D)
    dev = "cuda"
    unpacker = torch.randint(0, P, (B, W, L), generator=g, device=dev, dtype=torch.int32)
    best = torch.tensor([0, 5, 2, -1, 6, 3, 1, 4, 2], dtype=torch.int32, device=dev)
    nacc = torch.tensor([0, 6, 3, 1, 2, 7, -1, 6, 0], dtype=torch.int32, device=dev)
    kv_len = torch.tensor([0, 33, 10, 0, 0, 0, 0, 34, 40], dtype=torch.int32, device=dev)
    k_new = torch.randn((B, P, Hkv, D), generator=g, device=dev).to(dtype)
    v_new = torch.randn((B, P, Hkv, D), generator=g, device=dev).to(dtype)
    k_cache = torch.randn((B, Hkv, S, D), generator=g, device=dev).to(dtype)
    v_cache = torch.randn((B, Hkv, S, D), generator=g, device=dev).to(dtype)
    hidden = torch.randn((B, P, K), generator=g, device=dev).to(dtype) if K else None
    exp_k, exp_len = expected_commit(unpacker, best, nacc, k_new, k_cache, kv_len)
    exp_v, _ = expected_commit(unpacker, best, nacc, v_new, v_cache, kv_len)
    sentinel = torch.full((B, K), -3.0, dtype=dtype, device=dev) if K else None
    kv = kv_len.clone()
    hn = rd.rd_commit_accepted(unpacker, best, nacc, k_new, v_new, k_cache, v_cache, kv, hidden,
                               hidden_next=sentinel)
    torch.cuda.synchronize()
    assert torch.equal(kv, exp_len)
    # rows 0, 1, 2 commit (1 ends exactly at S); 3, 4, 5, 6 carry out-of-range values; 7, 8 overflow
    np.testing.assert_array_equal((kv != kv_len).cpu().numpy(), [1, 1, 1, 0, 0, 0, 0, 0, 0])
    assert torch.equal(k_cache, exp_k) and torch.equal(v_cache, exp_v)
    if K:
        un, bb, na = unpacker.cpu().numpy(), best.cpu().numpy(), nacc.cpu().numpy()
        for b in range(B):
            want = hidden[b, int(un[b, bb[b], na[b]])] if b < 3 else torch.full((K,), -3.0, dtype=dtype, device=dev)
            assert torch.equal(hn[b], want), b
    else:
        assert hn is None


def test_commit_then_next_step_attends_over_committed_rows():
    """Two-step loop: after the commit, a one-beam step attends over the longer cache as the oracle says."""
    cfg = get_config("tiny_f32").with_(B=2, S=32)
    seed = 77
    prob = Problem(cfg, seed, plant=True, kv_len=np.array([3, 11], np.int32))
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight, want_logits=False)
    kv = prob.kv_len_t.clone()
    rd.rd_commit_accepted(res["pack"]["unpacker"], res["best_beam"], res["accept_len"], prob.k_new, prob.v_new,
                          prob.k_cache, prob.v_cache, kv)
    torch.cuda.synchronize()
    bb, na = res["best_beam"].cpu().numpy(), res["accept_len"].cpu().numpy()
    ref = oracle.commit_accepted(prob.k_unp, prob.v_unp, prob.h_unp, bb, na, prob.kc_np, prob.vc_np, prob.kv_len)
    assert ref["committed"].all()
    # next step: a single beam of length 1 with fresh q/k/v per request
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q = torch.randn((cfg.B, 1, cfg.Hq, cfg.D), generator=g, device="cuda")
    k1 = torch.randn((cfg.B, 1, cfg.Hkv, cfg.D), generator=g, device="cuda")
    v1 = torch.randn((cfg.B, 1, cfg.Hkv, cfg.D), generator=g, device="cuda")
    beams1 = torch.zeros((cfg.B, 1, 1), dtype=torch.int32, device="cuda")
    pk = rd.rd_pack_beams(beams1)
    mask = rd.rd_tree_mask(pk["unpacker"], pk["length"])
    out = rd.rd_tree_attention(q, k1, v1, prob.k_cache, prob.v_cache, kv, mask, pk["length"])
    torch.cuda.synchronize()
    want = oracle.attention_per_beam(to_np(q)[:, None], to_np(k1)[:, None], to_np(v1)[:, None], ref["k_cache"],
                                     ref["v_cache"], ref["kv_len"])
    err = np.abs(to_np(out) - want[:, 0]).max() / np.abs(want).max()
    assert err <= 1e-5, err
