"""Pins for the oracle's stochastic verification (CPU only).

Pinned by what the pages state and what follows from it, not by retyping
the rule: (1) the emitted token is distributed as the target p when the
draft is a sample of q (Monte Carlo, one and two levels); (2) with one-hot
targets the walk reduces to the greedy accept; (3) a hand-worked case where
the residual update decides the second child; (4) leaves and empty requests.
"""
import numpy as np
import pytest

import oracle


def chain_tree(tokens):
    """One beam: slots 0..len-1 in a chain (W = 1)."""
    beams = np.array([[tokens]], np.int32)
    pk = oracle.pack_beams(beams)
    return beams, pk


def run(beams, pk, logits, q, ua, ub):
    return oracle.stochastic_accept(beams, pk["unpacker"], pk["length"], pk["tokens"], logits, q, ua, ub)


def test_hand_worked_residual_case():
    """Root with children tokens 0 and 2; p = (.2,.5,.3), q = (.6,.1,.3), uniforms .5 and .9.

    Child 0: .5*.6 = .3 >= p(0) = .2 -> rejected; p becomes max(p-q,0) normalised = (0,1,0).
    Child 2: .9*.3 = .27 >= p(2) = 0 -> rejected (it would pass against the original p(2) = .3);
    p becomes max((0,1,0)-q,0) normalised = (0,1,0); bonus = 1 for any u_bonus.
    """
    beams = np.array([[[7, 0], [7, 2]]], np.int32)        # two beams sharing the root token 7
    pk = oracle.pack_beams(beams)
    P, V = 4, 8
    logits = np.full((1, P, V), -1e4)
    q = np.zeros((1, P, V))
    logits[0, 0, :3] = np.log([0.2, 0.5, 0.3])
    q[0, 0, :3] = [0.6, 0.1, 0.3]
    ua = np.zeros((1, 2, 2))
    ua[0, 0] = [0.5, 0.9]
    res = run(beams, pk, logits, q, ua, np.array([0.123]))
    assert res["accept_len"][0] == 0 and res["best_beam"][0] == 0
    np.testing.assert_array_equal(res["accepted_tokens"][0], [1, -1])
    # a first uniform below 1/3 accepts child 0 (.3*.6 = .18 < .2)
    ua[0, 0] = [0.3, 0.9]
    res = run(beams, pk, logits, q, ua, np.array([0.5]))
    assert res["accept_len"][0] == 1 and res["best_beam"][0] == 0
    assert res["accepted_tokens"][0, 0] == 0


def test_one_hot_targets_reduce_to_greedy():
    rng = np.random.default_rng(4)
    B, W, L, V = 30, 6, 5, 4
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    beams[:, :, 0] = beams[:, :1, 0]                        # shared initial token
    pk = oracle.pack_beams(beams)
    P = W * L
    tgt_slot = rng.integers(0, V, size=(B, P))
    logits = np.full((B, P, V), -1e4)
    np.put_along_axis(logits, tgt_slot[..., None], 0.0, axis=2)
    q = rng.dirichlet(np.ones(V), size=(B, P))
    ua = rng.random((B, L, W))
    ub = rng.random(B)
    res = oracle.stochastic_accept(beams, pk["unpacker"], pk["length"], pk["tokens"], logits, q, ua, ub)
    target = np.take_along_axis(tgt_slot, pk["unpacker"].reshape(B, -1), axis=1).reshape(B, W, L)
    ref = oracle.greedy_accept(beams, target)
    for key in ("accept_len", "best_beam", "accepted_tokens"):
        np.testing.assert_array_equal(res[key], ref[key], err_msg=key)
    assert ref["accept_len"].max() > 0


def test_emitted_token_follows_the_target_one_level():
    """Draft x ~ q, accept with u < p(x)/q(x), else sample the residual: the emitted token is ~ p."""
    rng = np.random.default_rng(0)
    p = np.array([0.5, 0.3, 0.15, 0.05])
    qd = np.array([0.1, 0.2, 0.3, 0.4])
    N, V = 40000, 4
    draft = rng.choice(V, size=N, p=qd)
    beams = np.stack([np.full(N, 9), draft], axis=1).astype(np.int32)[:, None, :]   # [N,1,2]
    pk = oracle.pack_beams(beams)
    logits = np.full((N, 2, V), -1e4)
    logits[:, 0] = np.log(p)
    q = np.zeros((N, 2, V))
    q[:, 0] = qd
    q[:, 1] = 1.0 / V
    res = oracle.stochastic_accept(beams, pk["unpacker"], pk["length"], pk["tokens"], logits, q,
                                   rng.random((N, 2, 1)), rng.random(N))
    first = res["accepted_tokens"][:, 0]
    freq = np.bincount(first, minlength=V) / N
    sigma = np.sqrt(p * (1 - p) / N)
    assert (np.abs(freq - p) < 5 * sigma).all(), (freq, p)


def test_emitted_tokens_follow_the_target_two_levels():
    """Chain root -> x1 -> x2 with x1 ~ q_root, x2 ~ q_x1: first token ~ p_root, second | first accepted ~ p_child."""
    rng = np.random.default_rng(1)
    V, N = 3, 40000
    p0, q0 = np.array([0.2, 0.5, 0.3]), np.array([0.5, 0.25, 0.25])
    p1, q1 = np.array([0.6, 0.1, 0.3]), np.array([0.2, 0.2, 0.6])
    x1 = rng.choice(V, size=N, p=q0)
    x2 = rng.choice(V, size=N, p=q1)
    beams = np.stack([np.full(N, 5), x1, x2], axis=1).astype(np.int32)[:, None, :]
    pk = oracle.pack_beams(beams)
    logits = np.full((N, 3, V), -1e4)
    logits[:, 0], logits[:, 1] = np.log(p0), np.log(p1)
    logits[:, 2] = 0.0
    q = np.zeros((N, 3, V))
    q[:, 0], q[:, 1], q[:, 2] = q0, q1, 1.0 / V
    res = oracle.stochastic_accept(beams, pk["unpacker"], pk["length"], pk["tokens"], logits, q,
                                   rng.random((N, 3, 1)), rng.random(N))
    first = res["accepted_tokens"][:, 0]
    f0 = np.bincount(first, minlength=V) / N
    assert (np.abs(f0 - p0) < 5 * np.sqrt(p0 * (1 - p0) / N)).all(), (f0, p0)
    acc1 = res["accept_len"] >= 1
    second = res["accepted_tokens"][acc1, 1]
    f1 = np.bincount(second, minlength=V) / acc1.sum()
    assert (np.abs(f1 - p1) < 5 * np.sqrt(p1 * (1 - p1) / acc1.sum())).all(), (f1, p1)


def test_leaf_and_empty_requests():
    beams, pk = chain_tree([3, 1, 2])
    V = 4
    logits = np.full((1, 3, V), -1e4)
    logits[0, 0, 1] = 0.0                     # p_root one-hot on 1: child 1 accepted
    logits[0, 1, 2] = 0.0                     # p at slot 1 one-hot on 2: child 2 accepted
    logits[0, 2, 3] = 0.0                     # the leaf's p: one-hot on 3 -> bonus 3
    q = np.full((1, 3, V), 0.25)
    res = run(beams, pk, logits, q, np.full((1, 3, 1), 0.99), np.array([0.0]))
    assert res["accept_len"][0] == 2
    np.testing.assert_array_equal(res["accepted_tokens"][0], [1, 2, 3])
    np.testing.assert_array_equal(res["path"][0], [0, 1, 2])
    empty = oracle.stochastic_accept(beams, pk["unpacker"], np.array([0]), pk["tokens"], logits, q,
                                     np.zeros((1, 3, 1)), np.zeros(1))
    assert empty["accept_len"][0] == -1 and (empty["accepted_tokens"][0] == -1).all()
