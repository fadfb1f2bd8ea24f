"""Pins for the oracle's projection/argmax, unpack and greedy accept (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import torch

import oracle
from synthetic import get_config, draw_beams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_one_hot_projection_selects_hidden_entries():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 5, 8))
    cols = np.array([7, 0, 3, 3, 5, 1])
    w = np.zeros((6, 8))
    w[np.arange(6), cols] = 1.0
    logits = oracle.lm_head_logits(h, w)
    np.testing.assert_array_equal(logits, h[..., cols])


def test_projection_against_exact_sums():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((2, 3, 16)).astype(np.float32)
    w = (rng.standard_normal((11, 16)) * 0.02).astype(np.float32)
    logits = oracle.lm_head_logits(h, w)
    for i, j in itertools.product(range(2), range(3)):
        for v in range(11):
            exact = math.fsum(float(h[i, j, k]) * float(w[v, k]) for k in range(16))
            assert abs(logits[i, j, v] - exact) <= 1e-15 * max(1.0, abs(exact)) + 1e-16


def test_argmax_ties_take_the_lowest_index():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]])
    np.testing.assert_array_equal(oracle.argmax_first(x), [1, 0, 0])


def test_unpack_matches_torch_gather_restatement():
    rng = np.random.default_rng(4)
    B, W, L, P, X = 3, 4, 5, 20, 7
    packed = rng.standard_normal((B, P, X))
    unpacker = rng.integers(0, P, size=(B, W, L))
    ours = oracle.unpack(packed, unpacker)
    idx = torch.from_numpy(unpacker).reshape(B, W * L, 1).expand(-1, -1, X)
    ref = torch.gather(torch.from_numpy(packed), 1, idx).reshape(B, W, L, -1).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_golden_accept_cases():
    with open(os.path.join(GOLDEN, "accept_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = oracle.greedy_accept(np.array(c["beams"]), np.array(c["target"]))
        for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
            np.testing.assert_array_equal(got[key], np.array(c[key]), err_msg=f"{c['name']}: {key}")


def brute_force_accept(beams_b, target_b):
    """Enumerate every (beam, n) and keep the admissible ones, straight from the rule."""
    W, L = beams_b.shape
    ok = [(w, n) for w in range(W) for n in range(L)
          if all(beams_b[w, j + 1] == target_b[w, j] for j in range(n))]
    n_best = max(n for _, n in ok)
    w_best = min(w for w, n in ok if n == n_best)
    per_beam = [max(n for w2, n in ok if w2 == w) for w in range(W)]
    return per_beam, w_best, n_best


def test_accept_brute_force_random_small_vocab():
    rng = np.random.default_rng(5)
    for trial in range(300):
        W, L, V = rng.integers(1, 6), rng.integers(1, 6), rng.integers(2, 4)
        beams = rng.integers(0, V, size=(1, W, L))
        target = rng.integers(0, V, size=(1, W, L))
        got = oracle.greedy_accept(beams, target)
        per_beam, wb, nb = brute_force_accept(beams[0], target[0])
        np.testing.assert_array_equal(got["match_len"][0], per_beam)
        assert got["best_beam"][0] == wb and got["accept_len"][0] == nb
        expect = list(beams[0, wb, 1:nb + 1]) + [target[0, wb, nb]] + [-1] * (L - nb - 1)
        np.testing.assert_array_equal(got["accepted_tokens"][0], expect)


def test_accept_all_drafts_match():
    cfg = get_config("llama_mha")
    beams = draw_beams(cfg, 9)
    target = np.roll(beams, -1, axis=2)           # target at j predicts the draft at j+1
    got = oracle.greedy_accept(beams, target)
    assert (got["accept_len"] == cfg.L - 1).all() and (got["best_beam"] == 0).all()
    np.testing.assert_array_equal(got["accepted_tokens"][:, :cfg.L - 1], beams[:, 0, 1:])
    np.testing.assert_array_equal(got["accepted_tokens"][:, -1], target[:, 0, -1])
