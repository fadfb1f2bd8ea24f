"""Pins for the oracle's tree attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import get_config, draw_beams, unpacked_node_tensors, kv_cache, base_seed


def small_problem(name="tiny_f32", seed=3, **over):
    cfg = get_config(name).with_(**over)
    beams = draw_beams(cfg, seed)
    nodes = unpacked_node_tensors(cfg, seed, beams, with_hidden=False)
    kc = np.zeros((cfg.B, cfg.Hkv, cfg.S, cfg.D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(cfg.B):
        kc[b], vc[b] = kv_cache(cfg, seed, b)
    kv_len = np.full(cfg.B, cfg.S, np.int32)
    return cfg, beams, nodes, kc, vc, kv_len


def packed_from_unpacked(x_unp, pk):
    """Lay out per-candidate tensors in packed order via each node's first occurrence."""
    B, W, L = x_unp.shape[:3]
    P = W * L
    out = np.zeros((B, P) + x_unp.shape[3:], x_unp.dtype)
    for b in range(B):
        for p in range(pk["length"][b]):
            w, l = divmod(int(pk["src"][b, p]), L)
            out[b, p] = x_unp[b, w, l]
    return out


@pytest.mark.parametrize("over", [dict(), dict(Hkv=2), dict(W=6, L=5, B=2, S=37),
                                  dict(name="dedup_p0.5", B=1, W=6, L=4, Hq=2, Hkv=1, D=16, S=9)])
def test_packed_tree_attention_equals_per_beam(over):
    """The method's claim: deduplicated tree attention changes no candidate's output."""
    over = dict(over)
    name = over.pop("name", "tiny_f32")
    cfg, beams, nodes, kc, vc, kv_len = small_problem(name, **over)
    pk = oracle.pack_beams(beams)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    ref = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    got = oracle.attention_packed(packed_from_unpacked(nodes["q"], pk), packed_from_unpacked(nodes["k"], pk),
                                  packed_from_unpacked(nodes["v"], pk), kc, vc, kv_len, mask, pk["length"])
    for b in range(cfg.B):
        np.testing.assert_allclose(got[b][pk["unpacker"][b]], ref[b], rtol=0, atol=1e-12)
        assert (got[b, pk["length"][b]:] == 0).all()


def test_single_beam_matches_torch_sdpa():
    """W=1: plain causal attention behind a fully visible KV prefix."""
    cfg, beams, nodes, kc, vc, kv_len = small_problem(W=1, L=7, B=2, S=20, Hq=4, Hkv=2)
    kv_len = np.array([20, 13], np.int32)
    ref = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    G = cfg.Hq // cfg.Hkv
    for b in range(cfg.B):
        n = int(kv_len[b])
        q = torch.from_numpy(nodes["q"][b, 0].astype(np.float64)).permute(1, 0, 2)      # [Hq, L, D]
        k = np.concatenate([kc[b, :, :n], nodes["k"][b, 0].transpose(1, 0, 2)], axis=1)  # [Hkv, n+L, D]
        v = np.concatenate([vc[b, :, :n], nodes["v"][b, 0].transpose(1, 0, 2)], axis=1)
        k = torch.from_numpy(np.repeat(k, G, axis=0).astype(np.float64))
        v = torch.from_numpy(np.repeat(v, G, axis=0).astype(np.float64))
        allowed = torch.ones(cfg.L, n + cfg.L, dtype=torch.bool)
        allowed[:, n:] = torch.tril(torch.ones(cfg.L, cfg.L, dtype=torch.bool))
        sdpa = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=allowed)
        np.testing.assert_allclose(ref[b, 0], sdpa.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_empty_cache_first_token_returns_its_value():
    cfg, beams, nodes, kc, vc, _ = small_problem(B=1)
    out = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, np.zeros(1, np.int32))
    G = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        np.testing.assert_array_equal(out[0, :, 0, h], nodes["v"][0, :, 0, h // G].astype(np.float64))


def test_uniform_scores_give_mean_of_visible_values():
    cfg, beams, nodes, kc, vc, kv_len = small_problem(B=1, S=10)
    q = np.zeros_like(nodes["q"])
    out = oracle.attention_per_beam(q, nodes["k"], nodes["v"], kc, vc, kv_len)
    for w in range(cfg.W):
        for l in range(cfg.L):
            vis = np.concatenate([vc[0, :, :10], nodes["v"][0, w, :l + 1].transpose(1, 0, 2)], axis=1)
            expect = vis.astype(np.float64).mean(axis=1)              # [Hkv, D]
            np.testing.assert_allclose(out[0, w, l], expect, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    cfg, beams, nodes, kc, vc, kv_len = small_problem(Hq=4, Hkv=2, B=1)
    G = 2
    gqa = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    mha = oracle.attention_per_beam(nodes["q"], np.repeat(nodes["k"], G, axis=3), np.repeat(nodes["v"], G, axis=3),
                                    np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1), kv_len)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)


def test_cache_order_does_not_matter():
    cfg, beams, nodes, kc, vc, kv_len = small_problem(B=1, S=16)
    perm = np.random.default_rng(0).permutation(16)
    a = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    b = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc[:, :, perm], vc[:, :, perm], kv_len)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_default_scale_is_inverse_sqrt_head_dim():
    cfg, beams, nodes, kc, vc, kv_len = small_problem(B=1)
    a = oracle.attention_per_beam(nodes["q"], nodes["k"], nodes["v"], kc, vc, kv_len)
    b = oracle.attention_per_beam(nodes["q"] * 2.0, nodes["k"], nodes["v"], kc, vc, kv_len,
                                  scale=0.5 / math.sqrt(cfg.D))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_two_key_closed_form():
    """One cached key and the token itself: weights are a logistic of the score gap."""
    q = np.array([[[[[1.0, 2.0]]]]])          # [B=1,W=1,L=1,H=1,D=2]
    k = np.array([[[[[0.5, -1.0]]]]])
    v = np.array([[[[[3.0, 4.0]]]]])
    kc = np.array([[[[2.0, 1.0]]]])          # [B,Hkv,S=1,D]
    vc = np.array([[[[-1.0, 7.0]]]])
    out = oracle.attention_per_beam(q, k, v, kc, vc, np.array([1]))
    s_c, s_n = (2.0 + 2.0) / math.sqrt(2), (0.5 - 2.0) / math.sqrt(2)
    wc = 1.0 / (1.0 + math.exp(s_n - s_c))
    expect = wc * np.array([-1.0, 7.0]) + (1 - wc) * np.array([3.0, 4.0])
    np.testing.assert_allclose(out[0, 0, 0, 0], expect, rtol=0, atol=1e-14)
