"""GPU parity of the tree attention over a wide dynamic range of scores.

The bf16 kernel computes probabilities as exp2 of scores taken relative to a
per-row reference maximum, which is set on a row's first tile with a visible
key and moved only when a later tile's maximum exceeds it by more than a
threshold (a lazy rescale of O and the row sum).  These cases drive that
logic away from the unit-variance scores of the workloads, against the fp64
oracle (per-beam attention over the same bf16-rounded inputs):

- growing keys: cached key t scaled by 1 + 3t/S, so the row maxima climb
  across the tiles and the reference moves several times;
- common offsets: every score of a row shifted by about -200 or +200 (log2
  units) through a shared direction in q and k -- exp2 of such scores
  underflows or overflows fp32 unless the reference tracks them; the shift
  is the same for every key of a row, so the softmax is that of the
  unshifted scores.

Each runs on a few rows (8 wavefronts, two key groups), on many rows (8
wavefronts), on a GQA group of 160 rows and at D = 64, with and without a
forced split of the cache.
"""
import sys

import numpy as np
import pytest
import torch

import tree_attention_verification_rd_amd as rd
from synthetic import get_config, round_to_bf16
from harness import Problem, TOL, normwise_rows, to_np, fmt_err

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    rd.load_library()


SHAPES = {
    "few_rows": get_config("llama_mha").with_(B=2, W=4, L=5, Hq=4, Hkv=4, S=300, V=512),
    "many_rows": get_config("dedup_p0.5").with_(B=2, Hq=2, Hkv=2, S=200, V=512),
    "gqa_d64": get_config("gqa").with_(B=2, W=16, L=5, Hq=8, Hkv=2, D=64, S=260, V=512),
    "mid_rows": get_config("gqa").with_(B=2, W=8, L=5, Hq=8, Hkv=2, D=128, S=330, V=512),
}


def rewrite_inputs(prob: Problem, q_fn, k_fn, kc_fn):
    """Apply the transforms to the oracle's copies (rounded to bf16) and rebuild the device tensors from them."""
    cfg = prob.cfg
    prob.q_unp = round_to_bf16(q_fn(prob.q_unp.astype(np.float64)).astype(np.float32))
    prob.k_unp = round_to_bf16(k_fn(prob.k_unp.astype(np.float64)).astype(np.float32))
    prob.kc_np = round_to_bf16(kc_fn(prob.kc_np.astype(np.float64)).astype(np.float32))
    for i, b in enumerate(prob.checked):
        n = int(prob.pack["length"][b])
        w_idx, l_idx = np.divmod(prob.pack["src"][b, :n], cfg.L)
        prob.q[b].zero_()
        prob.k_new[b].zero_()
        prob.q[b, :n].copy_(torch.from_numpy(np.ascontiguousarray(prob.q_unp[i][w_idx, l_idx])).to(prob.q.dtype))
        prob.k_new[b, :n].copy_(torch.from_numpy(np.ascontiguousarray(prob.k_unp[i][w_idx, l_idx])).to(prob.q.dtype))
        prob.k_cache[b].copy_(torch.from_numpy(prob.kc_np[i]).to(prob.q.dtype))


def unit_dirs(cfg, seed):
    u = np.random.default_rng(seed).standard_normal((cfg.Hkv, cfg.D))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def make_case(cfg, kind, seed):
    prob = Problem(cfg, seed)
    G = cfg.Hq // cfg.Hkv
    if kind == "growing_keys":
        g = 1.0 + 3.0 * np.arange(cfg.S) / max(cfg.S, 1)
        rewrite_inputs(prob, lambda q: 2.0 * q, lambda k: k, lambda kc: kc * g[None, None, :, None])
    else:
        # (q + a u)(k - sign*a u)/sqrt(D) holds the offset -sign*a^2/sqrt(D) (nats) in every score of a row
        sign = 1.0 if kind == "offset_down" else -1.0
        a = np.sqrt(200.0 / np.log2(np.e) * np.sqrt(cfg.D))
        u = unit_dirs(cfg, seed + 1)
        uq = u[np.arange(cfg.Hq) // G]
        rewrite_inputs(prob, lambda q: q + a * uq, lambda k: k - sign * a * u,
                       lambda kc: kc - sign * a * u[None, :, None, :])
    return prob


def run(prob, splits):
    cfg = prob.cfg
    old = rd.rd_set_knob(rd.RD_KNOB_ATTN_SPLITS, splits or 0)
    try:
        pk, mask = rd.rd_pack_beams_mask(prob.beams_t)
        torch.cuda.synchronize()
        prob.assert_pack_matches(pk, mask)
        out = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                                   mask, pk["length"])
        torch.cuda.synchronize()
    finally:
        rd.rd_set_knob(rd.RD_KNOB_ATTN_SPLITS, old)
    return to_np(out)


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("kind", ["growing_keys", "offset_down", "offset_up"])
@pytest.mark.parametrize("splits", [None, 3])
def test_attention_dynamic_range(shape, kind, splits):
    cfg = SHAPES[shape]
    seed = 4200 + 10 * list(SHAPES).index(shape) + ["growing_keys", "offset_down", "offset_up"].index(kind)
    prob = make_case(cfg, kind, seed)
    say(f"[attn range] {shape} {kind} splits={splits} B={cfg.B} W={cfg.W} L={cfg.L} Hq={cfg.Hq} D={cfg.D} S={cfg.S}")
    out = run(prob, splits)
    ref = prob.oracle_attention()
    assert np.isfinite(ref).all()
    errs = []
    for i, b in enumerate(prob.checked):
        got = out[b][prob.pack["unpacker"][b]]
        assert np.isfinite(got).all(), "non-finite attention output"
        errs.append(normwise_rows(got, ref[i]).ravel())
        assert (out[b, prob.pack["length"][b]:] == 0).all(), "padding rows must be zero"
    errs = np.concatenate(errs)
    say(f"    attention normwise error {fmt_err(errs)} (tol {TOL[cfg.dtype]})")
    assert errs.max() <= TOL[cfg.dtype]
