"""Pins for the oracle's paged-cache attention (CPU only).

Pools are cut from a contiguous cache with numpy reshapes (not the oracle's
gather), so an identity page table must reproduce contiguous attention
exactly; permuting the pool's pages (and the table with them) and sharing
pages between requests must change nothing; table entries past a request's
cache length must never be read.
"""
import numpy as np
import pytest

import oracle
from synthetic import get_config, draw_beams, unpacked_node_tensors, kv_cache


def packed_problem(seed=4, B=3, W=3, L=4, S=40, Hq=4, Hkv=2, D=16):
    cfg = get_config("tiny_f32").with_(B=B, W=W, L=L, S=S, Hq=Hq, Hkv=Hkv, D=D)
    beams = draw_beams(cfg, seed)
    nodes = unpacked_node_tensors(cfg, seed, beams, with_hidden=False)
    pk = oracle.pack_beams(beams)
    P = W * L
    packed = {}
    for name in ("q", "k", "v"):
        x = nodes[name]
        out = np.zeros((B, P) + x.shape[3:], x.dtype)
        for b in range(B):
            for p in range(pk["length"][b]):
                w, l = divmod(int(pk["src"][b, p]), L)
                out[b, p] = x[b, w, l]
        packed[name] = out
    kc = np.zeros((B, Hkv, S, D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(B):
        kc[b], vc[b] = kv_cache(cfg, seed, b)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    return cfg, packed, kc, vc, mask, pk["length"]


def pool_from_cache(cache, ps):
    """[B,Hkv,S,D] -> pool [B*S/ps, Hkv, ps, D] and the identity table, by reshapes."""
    B, Hkv, S, D = cache.shape
    n = S // ps
    pool = cache.reshape(B, Hkv, n, ps, D).transpose(0, 2, 1, 3, 4).reshape(B * n, Hkv, ps, D)
    table = np.arange(B * n, dtype=np.int32).reshape(B, n)
    return pool, table


@pytest.mark.parametrize("ps", [1, 4, 8, 40])
def test_identity_table_reproduces_contiguous_attention(ps):
    cfg, pq, kc, vc, mask, plen = packed_problem()
    kv_len = np.array([40, 17, 0], np.int32)
    ref = oracle.attention_packed(pq["q"], pq["k"], pq["v"], kc, vc, kv_len, mask, plen)
    kp, table = pool_from_cache(kc, ps)
    vp, _ = pool_from_cache(vc, ps)
    got = oracle.attention_paged(pq["q"], pq["k"], pq["v"], kp, vp, table, kv_len, mask, plen)
    np.testing.assert_array_equal(got, ref)


def test_permuted_pool_and_unread_entries():
    cfg, pq, kc, vc, mask, plen = packed_problem(seed=6)
    ps = 8
    kv_len = np.array([33, 8, 25], np.int32)
    kp, table = pool_from_cache(kc, ps)
    vp, _ = pool_from_cache(vc, ps)
    base = oracle.attention_paged(pq["q"], pq["k"], pq["v"], kp, vp, table, kv_len, mask, plen)
    rng = np.random.default_rng(0)
    perm = rng.permutation(kp.shape[0])          # new slot of old page i is perm[i]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = perm[table].astype(np.int32)
    for b in range(cfg.B):                        # entries past the cache length: never read
        table2[b, (int(kv_len[b]) + ps - 1) // ps:] = -1
    got = oracle.attention_paged(pq["q"], pq["k"], pq["v"], kp2, vp2, table2, kv_len, mask, plen)
    np.testing.assert_array_equal(got, base)


def test_shared_prefix_pages():
    """Two requests whose tables share their first pages see the same cached prefix."""
    cfg, pq, kc, vc, mask, plen = packed_problem(seed=7)
    ps = 8
    kc[1, :, :16] = kc[0, :, :16]
    vc[1, :, :16] = vc[0, :, :16]
    kv_len = np.array([30, 21, 9], np.int32)
    ref = oracle.attention_packed(pq["q"], pq["k"], pq["v"], kc, vc, kv_len, mask, plen)
    kp, table = pool_from_cache(kc, ps)
    vp, _ = pool_from_cache(vc, ps)
    own = table[1, :2].copy()
    table[1, :2] = table[0, :2]                   # request 1 reuses request 0's first two pages
    kp[own], vp[own] = 1e3, -1e3                  # its own first pages, no longer referenced
    got = oracle.attention_paged(pq["q"], pq["k"], pq["v"], kp, vp, table, kv_len, mask, plen)
    np.testing.assert_array_equal(got, ref)


def test_paged_commit_equals_contiguous_commit_through_the_gather():
    """Committing into pages, then gathering, equals committing into the gathered cache."""
    cfg = get_config("tiny_f32").with_(B=3, W=4, L=5, S=40, Hq=4, Hkv=2, D=8)
    beams = draw_beams(cfg, 12)
    nodes = unpacked_node_tensors(cfg, 12, beams)
    kc = np.zeros((cfg.B, cfg.Hkv, cfg.S, cfg.D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(cfg.B):
        kc[b], vc[b] = kv_cache(cfg, 12, b)
    ps = 8
    kp, table = pool_from_cache(kc, ps)
    vp, _ = pool_from_cache(vc, ps)
    rng = np.random.default_rng(3)
    perm = rng.permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table = perm[table].astype(np.int32)
    kv_len = np.array([13, 0, 36], np.int32)          # request 2 overflows with more than 3 rows
    best = np.array([1, 3, 2], np.int32)
    n_acc = np.array([4, 2, 4], np.int32)
    got = oracle.commit_accepted_paged(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kp2, vp2, table, kv_len)
    ref = oracle.commit_accepted(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kc, vc, kv_len)
    np.testing.assert_array_equal(got["kv_len"], ref["kv_len"])
    np.testing.assert_array_equal(got["committed"], [True, True, False])
    np.testing.assert_array_equal(got["hidden_next"], ref["hidden_next"])
    full = np.full(cfg.B, cfg.S, np.int32)
    np.testing.assert_array_equal(oracle.gather_pages(got["k_pages"], table, full), ref["k_cache"])
    np.testing.assert_array_equal(oracle.gather_pages(got["v_pages"], table, full), ref["v_cache"])


@pytest.mark.parametrize("bad", [-1, 10_000])
def test_paged_commit_with_a_table_entry_outside_the_pool_changes_nothing(bad):
    """A request whose committed positions hit a table entry naming no page is left as it was;
    the other requests commit as usual and no page of the pool changes for it."""
    cfg = get_config("tiny_f32").with_(B=3, W=4, L=5, S=40, Hq=4, Hkv=2, D=8)
    beams = draw_beams(cfg, 12)
    nodes = unpacked_node_tensors(cfg, 12, beams)
    kc = np.zeros((cfg.B, cfg.Hkv, cfg.S, cfg.D), np.float32)
    vc = np.zeros_like(kc)
    for b in range(cfg.B):
        kc[b], vc[b] = kv_cache(cfg, 12, b)
    ps = 8
    kp, table = pool_from_cache(kc, ps)
    vp, _ = pool_from_cache(vc, ps)
    kv_len = np.array([13, 6, 20], np.int32)
    best = np.array([1, 3, 2], np.int32)
    n_acc = np.array([4, 2, 4], np.int32)
    t2 = table.copy()
    t2[0, (13 + 4) // ps] = bad          # request 0's last committed position has no page
    t2[1, 4] = bad                       # an entry request 1 never reaches (positions 6..8)
    got = oracle.commit_accepted_paged(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kp, vp, t2, kv_len)
    ref = oracle.commit_accepted_paged(nodes["k"], nodes["v"], nodes["hidden"], best, n_acc, kp, vp, table, kv_len)
    np.testing.assert_array_equal(got["committed"], [False, True, True])
    np.testing.assert_array_equal(got["kv_len"], [13, 9, 25])
    assert np.isnan(got["hidden_next"][0]).all()
    own0 = table[0]
    np.testing.assert_array_equal(got["k_pages"][own0], kp[own0])
    np.testing.assert_array_equal(got["v_pages"][own0], vp[own0])
    others = np.setdiff1d(np.arange(kp.shape[0]), own0)
    np.testing.assert_array_equal(got["k_pages"][others], ref["k_pages"][others])
    np.testing.assert_array_equal(got["v_pages"][others], ref["v_pages"][others])
