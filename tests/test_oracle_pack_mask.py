"""Pins for the oracle's pack and tree-mask steps (CPU only).

Every check is derived from the definition of a trie node as a distinct
token prefix, evaluated by brute force on token tuples, never by reusing
the oracle's own trie or ancestor walk.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synthetic import get_config, draw_beams, base_seed

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def prefixes(beams_b):
    W, L = beams_b.shape
    return {(w, l): tuple(int(t) for t in beams_b[w, :l + 1]) for w in range(W) for l in range(L)}


def check_pack_against_brute_force(beams):
    B, W, L = beams.shape
    pk = oracle.pack_beams(beams)
    for b in range(B):
        pre = prefixes(beams[b])
        distinct = set(pre.values())
        assert pk["length"][b] == len(distinct)
        u = pk["unpacker"][b]
        for (w, l), (w2, l2) in itertools.product(pre, pre):
            assert (u[w, l] == u[w2, l2]) == (pre[(w, l)] == pre[(w2, l2)])
        # first-occurrence numbering in a beam-major scan
        seen = []
        for w in range(W):
            for l in range(L):
                if u[w, l] not in seen:
                    assert u[w, l] == len(seen)
                    seen.append(u[w, l])
        n = pk["length"][b]
        for w in range(W):
            for l in range(L):
                p = u[w, l]
                assert pk["tokens"][b, p] == beams[b, w, l]
                assert pk["depth"][b, p] == l
                sw, sl = divmod(int(pk["src"][b, p]), L)
                assert pre[(sw, sl)] == pre[(w, l)] and (sw, sl) <= (w, l)
        assert (pk["tokens"][b, n:] == -1).all() and (pk["depth"][b, n:] == -1).all()
        assert (pk["src"][b, n:] == -1).all()
    return pk


def brute_force_mask(beams_b, unpacker_b, P):
    """mask[p,q] iff the prefix of q is a prefix of (or equal to) the prefix of p."""
    W, L = beams_b.shape
    m = np.zeros((P, P), bool)
    pre = prefixes(beams_b)
    for (w, l), pp in pre.items():
        for (w2, l2), qq in pre.items():
            if l2 <= l and pp[:l2 + 1] == qq:
                m[unpacker_b[w, l], unpacker_b[w2, l2]] = True
    return m


def test_exhaustive_tiny_beam_sets():
    # every beam set with W=3, L=2, V=2: 2**6 = 64 sets
    W, L, V = 3, 2, 2
    sets = np.array(list(itertools.product(range(V), repeat=W * L)), np.int32).reshape(-1, W, L)
    pk = check_pack_against_brute_force(sets)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    for b in range(sets.shape[0]):
        np.testing.assert_array_equal(mask[b], brute_force_mask(sets[b], pk["unpacker"][b], W * L))


def test_exhaustive_single_beam_l3():
    W, L, V = 2, 3, 2
    sets = np.array(list(itertools.product(range(V), repeat=W * L)), np.int32).reshape(-1, W, L)
    check_pack_against_brute_force(sets)


@pytest.mark.parametrize("name", ["tiny_f32", "llama_mha", "gqa"])
def test_workload_beams_brute_force(name):
    cfg = get_config(name)
    cfg = cfg.with_(B=min(cfg.B, 4))
    beams = draw_beams(cfg, base_seed(cfg))
    pk = check_pack_against_brute_force(beams)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    for b in range(cfg.B):
        np.testing.assert_array_equal(mask[b], brute_force_mask(beams[b], pk["unpacker"][b], cfg.P_max))


def test_no_sharing_gives_w_times_l():
    cfg = get_config("llama_mha")
    beams = draw_beams(cfg, 7, mode="distinct")
    pk = oracle.pack_beams(beams)
    assert (pk["length"] == cfg.W * cfg.L).all()
    # no sharing: slot of (w, l) is w*L + l
    np.testing.assert_array_equal(pk["unpacker"].reshape(cfg.B, -1),
                                  np.tile(np.arange(cfg.W * cfg.L), (cfg.B, 1)))


def test_identical_beams_give_l():
    cfg = get_config("llama_mha")
    beams = draw_beams(cfg, 7, mode="identical")
    pk = oracle.pack_beams(beams)
    assert (pk["length"] == cfg.L).all()
    for w in range(cfg.W):
        np.testing.assert_array_equal(pk["unpacker"][:, w], np.tile(np.arange(cfg.L), (cfg.B, 1)))


def test_unpack_round_trip_with_torch_gather():
    """The pages' unpack, restated with torch.gather, recovers the beams from the packed tokens."""
    cfg = get_config("gqa").with_(B=6)
    beams = draw_beams(cfg, 11)
    pk = oracle.pack_beams(beams)
    packed = torch.from_numpy(pk["tokens"].astype(np.int64))[:, :, None]     # [B,P,1]
    idx = torch.from_numpy(pk["unpacker"].astype(np.int64)).reshape(cfg.B, cfg.W * cfg.L, 1)
    idx = idx.expand(-1, -1, packed.shape[2])
    got = torch.gather(packed, 1, idx).reshape(cfg.B, cfg.W, cfg.L, -1)[..., 0]
    np.testing.assert_array_equal(got.numpy(), beams)


def test_mask_single_beam_is_causal():
    cfg = get_config("tiny_f32").with_(W=1, L=6, B=3)
    beams = draw_beams(cfg, 3)
    pk = oracle.pack_beams(beams)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    for b in range(cfg.B):
        np.testing.assert_array_equal(mask[b], np.tril(np.ones((6, 6), bool)))


@pytest.mark.parametrize("name", ["llama_mha", "dedup_p0.5"])
def test_mask_row_popcount_and_triangle(name):
    cfg = get_config(name).with_(B=3)
    beams = draw_beams(cfg, base_seed(cfg))
    pk = oracle.pack_beams(beams)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    for b in range(cfg.B):
        n = pk["length"][b]
        assert (mask[b].sum(axis=1)[:n] == pk["depth"][b, :n] + 1).all()
        assert not np.triu(mask[b], 1).any()          # parents precede children
        assert not mask[b, n:].any() and not mask[b, :, n:].any()


def test_mask_bits_layout():
    m = np.zeros((1, 40, 40), bool)
    m[0, 3, 0] = m[0, 3, 31] = m[0, 3, 32] = m[0, 39, 39] = True
    bits = oracle.mask_to_bits(m)
    assert bits.shape == (1, 40, 2) and bits.dtype == np.uint32
    assert bits[0, 3, 0] == (1 | (1 << 31)) and bits[0, 3, 1] == 1
    assert bits[0, 39, 1] == (1 << 7) and bits[0, 0].sum() == 0


def test_golden_pack_examples():
    with open(os.path.join(GOLDEN, "pack_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        beams = np.array(c["beams"], np.int32)
        pk = oracle.pack_beams(beams)
        for key in ("length", "unpacker", "tokens", "depth", "src"):
            np.testing.assert_array_equal(pk[key], np.array(c[key]), err_msg=f"{c['name']}: {key}")
        bits = oracle.mask_to_bits(oracle.tree_mask(pk["unpacker"], pk["length"]))
        np.testing.assert_array_equal(bits, np.array(c["mask_words"], np.uint32), err_msg=c["name"])


def test_uniform_share_rule_mean_packed_length():
    """Share length U{0..L-1} against the previous beam: E[P] = L + (W-1)(L+1)/2.

    Each later beam adds L - s nodes beyond its copied prefix unless a fresh
    token collides with an earlier beam (probability ~1/V), so the expected
    count follows from E[s] = (L-1)/2.
    """
    cfg = get_config("llama_mha").with_(B=400, V=32000)
    beams = draw_beams(cfg, 5)
    P = oracle.pack_beams(beams)["length"]
    expect = cfg.L + (cfg.W - 1) * (cfg.L + 1) / 2
    sd = np.sqrt((cfg.W - 1) * (cfg.L ** 2 - 1) / 12.0)  # variance of U{0..L-1} per beam
    assert abs(P.mean() - expect) < 5 * sd / np.sqrt(cfg.B)
    # 30-60 % fewer tokens than unpacked is the range the pages quote for real beams;
    # this synthetic rule sits near its low end
    assert 0.25 < 1 - P.mean() / (cfg.W * cfg.L) < 0.45
