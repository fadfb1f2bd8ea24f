"""Pins for the oracle's commit of the accepted path (CPU only).

The commit is pinned by what it must preserve, not by its own formula:
decoding over the committed cache reproduces what verification computed
for the accepted candidates (checked with torch's scaled-dot-product
attention), the committed rows spell the accepted text that the greedy
accept reports, the chosen hidden state re-derives the bonus token, and
requests that cannot be committed stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import get_config, draw_beams, unpacked_node_tensors, kv_cache


def problem(seed=5, B=3, W=4, L=5, S=24, Hq=4, Hkv=2, D=16, V=64, kv_len=(9, 0, 17)):
    cfg = get_config("tiny_f32").with_(B=B, W=W, L=L, S=S, Hq=Hq, Hkv=Hkv, D=D, V=V)
    beams = draw_beams(cfg, seed)
    nodes = unpacked_node_tensors(cfg, seed, beams)
    kc = np.zeros((B, Hkv, S, D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(B):
        kc[b], vc[b] = kv_cache(cfg, seed, b)
    return cfg, beams, nodes, kc, vc, np.array(kv_len, np.int32)


def sdpa_over_cache(q_heads, kc_b, vc_b, n):
    """torch attention of q [Hq,D] over the first n cached keys of every KV head."""
    Hq, D = q_heads.shape
    Hkv = kc_b.shape[0]
    G = Hq // Hkv
    q = torch.from_numpy(q_heads.astype(np.float64)).reshape(Hq, 1, D)
    k = torch.from_numpy(np.repeat(kc_b[:, :n], G, axis=0).astype(np.float64))
    v = torch.from_numpy(np.repeat(vc_b[:, :n], G, axis=0).astype(np.float64))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v).reshape(Hq, D).numpy()


def test_decoding_over_committed_cache_reproduces_verification():
    """Accepted candidate j attends over cache[:c+j+1] exactly as it did in tree verification."""
    cfg, beams, nodes, kc, vc, kv_len = problem()
    best = np.array([2, 0, 3], np.int32)
    n_acc = np.array([4, 0, 2], np.int32)
    ver = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    res = oracle.commit_accepted(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kc, vc, kv_len)
    assert res["committed"].all()
    np.testing.assert_array_equal(res["kv_len"], kv_len + n_acc + 1)
    for b in range(cfg.B):
        c, w = int(kv_len[b]), int(best[b])
        for j in range(int(n_acc[b]) + 1):
            dec = sdpa_over_cache(nodes["q"][b, w, j], res["k_cache"][b], res["v_cache"][b], c + j + 1)
            np.testing.assert_allclose(dec, ver[b, w, j], rtol=0, atol=1e-12)


def planted_step(seed=11, B=4, W=5, L=5, V=48, K=32):
    """Beams whose drafts follow the target's argmax for a chosen number of positions."""
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((B, W, L, K))
    weight = rng.standard_normal((V, K)) * 0.02
    target = oracle.argmax_first(oracle.lm_head_logits(hidden, weight))
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    beams[:, :, 0] = beams[:, :1, 0]        # every beam opens with the target's initial token
    follow = rng.integers(0, L, size=(B, W))
    for b in range(B):
        for w in range(W):
            for j in range(L - 1):
                if j < follow[b, w]:
                    beams[b, w, j + 1] = target[b, w, j]
                elif beams[b, w, j + 1] == target[b, w, j]:
                    beams[b, w, j + 1] = (target[b, w, j] + 1) % V
    return beams, hidden, weight, target, follow


def test_committed_rows_spell_the_accepted_text_and_hidden_gives_the_bonus():
    beams, hidden, weight, target, follow = planted_step()
    B, W, L = beams.shape
    acc = oracle.greedy_accept(beams, target)
    assert (acc["accept_len"] == follow.max(axis=1)).all()
    Hkv, D, S = 3, 4, 20
    # tag each candidate's key with its own token, its beam and its head
    k = np.zeros((B, W, L, Hkv, D))
    k[..., 0] = beams[..., None]
    k[..., 1] = np.arange(W)[None, :, None, None]
    k[..., 2] = np.arange(Hkv)
    v = -k
    kc = np.full((B, Hkv, S, D), -7.0)
    vc = np.full((B, Hkv, S, D), 7.0)
    kv_len = np.array([0, 3, 9, 14], np.int32)[:B]
    res = oracle.commit_accepted(k, v, hidden, acc["best_beam"], acc["accept_len"], kc, vc, kv_len)
    for b in range(B):
        n, c = int(acc["accept_len"][b]), int(kv_len[b])
        rows = res["k_cache"][b, :, c:c + n + 1]                         # [Hkv, n+1, D]
        # position c holds the initial token; the drafts follow in accepted order
        assert (rows[:, 0, 0] == beams[b, 0, 0]).all()
        np.testing.assert_array_equal(rows[0, 1:, 0], acc["accepted_tokens"][b, :n])
        assert (rows[..., 1] == acc["best_beam"][b]).all()
        np.testing.assert_array_equal(rows[..., 2], np.repeat(np.arange(Hkv)[:, None], n + 1, axis=1))
        np.testing.assert_array_equal(res["v_cache"][b, :, c:c + n + 1], -rows)
        bonus = oracle.argmax_first(oracle.lm_head_logits(res["hidden_next"][b][None], weight))[0]
        assert bonus == acc["accepted_tokens"][b, n]


def test_rows_outside_the_path_are_untouched_and_requests_independent():
    cfg, beams, nodes, kc, vc, kv_len = problem(seed=8)
    best = np.array([1, 3, 0], np.int32)
    n_acc = np.array([3, 4, 1], np.int32)
    res = oracle.commit_accepted(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kc, vc, kv_len)
    for b in range(cfg.B):
        c, n = int(kv_len[b]), int(n_acc[b])
        keep = np.ones(cfg.S, bool)
        keep[c:c + n + 1] = False
        np.testing.assert_array_equal(res["k_cache"][b][:, keep], kc[b][:, keep])
        np.testing.assert_array_equal(res["v_cache"][b][:, keep], vc[b][:, keep])
        one = oracle.commit_accepted(nodes["k"][b:b + 1], nodes["v"][b:b + 1], nodes["hidden"][b:b + 1],
                                     best[b:b + 1], n_acc[b:b + 1], kc[b:b + 1], vc[b:b + 1], kv_len[b:b + 1])
        np.testing.assert_array_equal(one["k_cache"][0], res["k_cache"][b])
        np.testing.assert_array_equal(one["hidden_next"][0], res["hidden_next"][b])


@pytest.mark.parametrize("best,n_acc,c,ok", [
    (1, 2, 21, True),     # ends exactly at the capacity S = 24
    (1, 2, 22, False),    # one row past the capacity
    (0, 4, 19, True),
    (0, 4, 20, False),
    (4, 0, 0, False),     # beam index == W
    (-1, 0, 0, False),
    (0, 5, 0, False),     # accept length == L
    (0, -1, 0, False),
    (0, 0, -1, False),    # negative cache length
])
def test_capacity_and_range_edges(best, n_acc, c, ok):
    cfg, beams, nodes, kc, vc, _ = problem(seed=9, B=1, kv_len=(0,))
    res = oracle.commit_accepted(nodes["k"], nodes["v"], nodes["hidden"], np.array([best]), np.array([n_acc]),
                                 kc, vc, np.array([c], np.int32))
    assert bool(res["committed"][0]) == ok
    if ok:
        assert res["kv_len"][0] == c + n_acc + 1 <= cfg.S
        assert not np.isnan(res["hidden_next"][0]).any()
    else:
        assert res["kv_len"][0] == c
        np.testing.assert_array_equal(res["k_cache"], kc)
        np.testing.assert_array_equal(res["v_cache"], vc)
        assert np.isnan(res["hidden_next"][0]).all()
