"""Pins for the oracle's ragged batches (CPU only).

A ragged request (beam_width[b] beams of beam_len[b] tokens inside a padded
[W, L] slab) must give exactly what the full-shape oracle gives on its
sliced [beam_width[b], beam_len[b]] sub-array -- pack, mask, unpack and
greedy accept -- with padding candidates at unpacker -1, zero unpacked rows
and no acceptance for requests with no beam or no position.
"""
import numpy as np
import pytest

import oracle


def ragged_case(seed, B=6, W=7, L=6, V=3):
    rng = np.random.default_rng(seed)
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    beams[:, 1::2, :2] = beams[:, 0:W - 1:2, :2]          # shared prefixes
    bw = rng.integers(1, W + 1, size=B)
    bl = rng.integers(1, L + 1, size=B)
    bw[0], bl[0] = W, L                                    # one full request
    bw[1] = 0                                              # no beam
    bl[2] = 0                                              # no position
    target = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    return beams, bw, bl, target


@pytest.mark.parametrize("seed", range(6))
def test_ragged_pack_mask_unpack_accept_equal_the_sliced_requests(seed):
    beams, bw, bl, target = ragged_case(seed)
    B, W, L = beams.shape
    pk = oracle.pack_beams(beams, bw, bl)
    mask = oracle.tree_mask(pk["unpacker"], pk["length"])
    acc = oracle.greedy_accept(beams, target, bw, bl)
    packed = np.random.default_rng(seed + 100).standard_normal((B, W * L, 5))
    unp = oracle.unpack(packed, pk["unpacker"])
    for b in range(B):
        w_, l_ = int(bw[b]), int(bl[b])
        n = int(pk["length"][b])
        if w_ == 0 or l_ == 0:
            assert n == 0 and (pk["unpacker"][b] == -1).all() and (pk["tokens"][b] == -1).all()
            assert acc["best_beam"][b] == -1 and acc["accept_len"][b] == -1
            assert (acc["accepted_tokens"][b] == -1).all() and (acc["match_len"][b] == -1).all()
            assert not mask[b].any() and (unp[b] == 0).all()
            continue
        sub = np.ascontiguousarray(beams[b:b + 1, :w_, :l_])
        ref = oracle.pack_beams(sub)
        assert n == ref["length"][0]
        np.testing.assert_array_equal(pk["tokens"][b, :n], ref["tokens"][0, :n])
        np.testing.assert_array_equal(pk["depth"][b, :n], ref["depth"][0, :n])
        w_src, l_src = np.divmod(ref["src"][0, :n], l_)
        np.testing.assert_array_equal(pk["src"][b, :n], w_src * L + l_src)
        assert (pk["tokens"][b, n:] == -1).all() and (pk["src"][b, n:] == -1).all()
        np.testing.assert_array_equal(pk["unpacker"][b, :w_, :l_], ref["unpacker"][0])
        assert (pk["unpacker"][b, w_:] == -1).all() and (pk["unpacker"][b, :, l_:] == -1).all()
        ref_mask = oracle.tree_mask(ref["unpacker"], ref["length"])[0]
        np.testing.assert_array_equal(mask[b, :n, :n], ref_mask[:n, :n])
        assert not mask[b, n:].any() and not mask[b, :, n:].any()
        ref_unp = oracle.unpack(packed[b:b + 1, :w_ * l_][:, :, :], ref["unpacker"])  # node slots agree
        np.testing.assert_array_equal(unp[b, :w_, :l_], ref_unp[0])
        assert (unp[b, w_:] == 0).all() and (unp[b, :, l_:] == 0).all()
        ref_acc = oracle.greedy_accept(sub, np.ascontiguousarray(target[b:b + 1, :w_, :l_]))
        np.testing.assert_array_equal(acc["match_len"][b, :w_], ref_acc["match_len"][0])
        assert (acc["match_len"][b, w_:] == -1).all()
        assert acc["best_beam"][b] == ref_acc["best_beam"][0]
        assert acc["accept_len"][b] == ref_acc["accept_len"][0]
        np.testing.assert_array_equal(acc["accepted_tokens"][b, :l_], ref_acc["accepted_tokens"][0])
        assert (acc["accepted_tokens"][b, l_:] == -1).all()


def test_full_widths_change_nothing():
    beams, _, _, target = ragged_case(9)
    B, W, L = beams.shape
    full = oracle.pack_beams(beams)
    rag = oracle.pack_beams(beams, [W] * B, [L] * B)
    for k in full:
        np.testing.assert_array_equal(rag[k], full[k])
    a = oracle.greedy_accept(beams, target)
    r = oracle.greedy_accept(beams, target, [W] * B, [L] * B)
    for k in a:
        np.testing.assert_array_equal(r[k], a[k])
