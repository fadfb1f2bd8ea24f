"""GPU parity: every entry point of librd against the CPU oracle on seeded inputs.

Integers (packed tokens, lengths, unpacker, depth, src, mask words, argmax,
match lengths, best beam, accept length, accepted tokens) must match
bit-exactly.  Floats are compared per row with the normwise error
max|x - r| / max|r| <= 1e-5 (fp32) or 2e-2 (bf16).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, draw_beams, base_seed, Config, round_to_bf16
from harness import Problem, TOL, MARGIN, normwise_rows, to_np, mask_words_np, fmt_err

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


def check_pack(beams: np.ndarray):
    """Separate pack and mask calls, and the fused call, against the oracle."""
    ref = oracle.pack_beams(beams)
    got = rd.rd_pack_beams(dev_int(beams))
    mask = rd.rd_tree_mask(got["unpacker"], got["length"])
    fused, fmask = rd.rd_pack_beams_mask(dev_int(beams))
    torch.cuda.synchronize()
    ref_bits = oracle.mask_to_bits(oracle.tree_mask(ref["unpacker"], ref["length"]))
    for tag, g, m in (("separate", got, mask), ("fused", fused, fmask)):
        for key in ("tokens", "length", "unpacker", "depth", "src"):
            np.testing.assert_array_equal(g[key].cpu().numpy(), ref[key], err_msg=f"{tag} {key}")
        np.testing.assert_array_equal(mask_words_np(m), ref_bits, err_msg=f"{tag} mask")
    return ref


# ------------------------------------------------------------------ pack + mask
@pytest.mark.parametrize("name", ["tiny_f32", "llama_mha", "gqa", "dedup_p0.1", "dedup_p0.5", "dedup_p0.9",
                                  "long_ctx"])
def test_pack_mask_workloads(name):
    cfg = get_config(name)
    say(f"[pack] {name} B={cfg.B} W={cfg.W} L={cfg.L}")
    for trial in range(2):
        check_pack(draw_beams(cfg, base_seed(cfg, trial)))


@pytest.mark.parametrize("mode,expect", [("distinct", "WL"), ("identical", "L")])
def test_pack_no_sharing_and_all_identical(mode, expect):
    cfg = get_config("dedup_p0.5")
    ref = check_pack(draw_beams(cfg, 5, mode))
    assert (ref["length"] == (cfg.W * cfg.L if expect == "WL" else cfg.L)).all()


@pytest.mark.parametrize("W,L,V", [(64, 16, 3), (64, 16, 2), (1, 16, 5), (64, 1, 7), (1, 1, 9), (37, 11, 2),
                                   (5, 3, 1)])
def test_pack_limits_and_degenerate(W, L, V):
    rng = np.random.default_rng(W * 100 + L * 10 + V)
    beams = rng.integers(0, V, size=(9, W, L)).astype(np.int32)
    say(f"[pack] limits W={W} L={L} V={V}")
    check_pack(beams)


def test_pack_large_token_ids():
    rng = np.random.default_rng(3)
    beams = rng.integers(-2**31, 2**31 - 1, size=(4, 8, 5), dtype=np.int64).astype(np.int32)
    beams[:, 1::2, :2] = beams[:, 0::2, :2]
    check_pack(beams)


def test_empty_inputs_are_noops():
    e = torch.empty((0, 4, 3), dtype=torch.int32, device="cuda")
    out = rd.rd_pack_beams(e)
    assert out["tokens"].shape == (0, 12)
    m = rd.rd_tree_mask(out["unpacker"], out["length"])
    assert m.shape == (0, 12, 1)
    fo, fm = rd.rd_pack_beams_mask(e)
    assert fo["tokens"].shape == (0, 12) and fm.shape == (0, 12, 1)
    for shape in ((3, 0, 4), (3, 4, 0)):
        t = torch.empty(shape, dtype=torch.int32, device="cuda")
        rd.rd_pack_beams(t)
    acc = rd.rd_unpack_accept(e, out["unpacker"], torch.empty((0, 12), dtype=torch.int32, device="cuda"))
    assert acc["accept_len"].shape == (0,)


def test_invalid_arguments_raise():
    beams = torch.zeros((2, 65, 3), dtype=torch.int32, device="cuda")
    with pytest.raises(rd.RdError) as ei:
        rd.rd_pack_beams(beams)
    assert ei.value.code == -2
    beams = torch.zeros((2, 4, 17), dtype=torch.int32, device="cuda")
    with pytest.raises(rd.RdError):
        rd.rd_pack_beams(beams)


# ----------------------------------------------------------------------- accept
@pytest.mark.parametrize("W,L,V", [(8, 5, 3), (64, 8, 2), (16, 16, 2), (1, 4, 2), (4, 1, 3), (64, 16, 3)])
def test_accept_against_oracle(W, L, V):
    rng = np.random.default_rng(W + 7 * L + 31 * V)
    B = 40
    beams = rng.integers(0, V, size=(B, W, L)).astype(np.int32)
    pk = oracle.pack_beams(beams)
    # a target choice per packed slot from the same small vocabulary: many matches
    pargmax = rng.integers(0, V, size=(B, W * L)).astype(np.int32)
    pargmax[np.arange(W * L)[None, :] >= pk["length"][:, None]] = -1
    target = np.take_along_axis(pargmax, pk["unpacker"].reshape(B, -1), axis=1).reshape(B, W, L)
    ref = oracle.greedy_accept(beams, target)
    got = rd.rd_unpack_accept(dev_int(beams), dev_int(pk["unpacker"]), dev_int(pargmax))
    for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    if L > 1:
        assert ref["accept_len"].max() > 0


# ----------------------------------------------------------------------- unpack
@pytest.mark.parametrize("dtype,X", [(torch.bfloat16, 1000), (torch.float32, 7), (torch.bfloat16, 3),
                                     (torch.bfloat16, 32000), (torch.float32, 4096)])
def test_unpack_gather(dtype, X):
    rng = np.random.default_rng(X)
    B, W, L = 3, 8, 5
    beams = rng.integers(0, 4, size=(B, W, L)).astype(np.int32)
    pk = oracle.pack_beams(beams)
    packed = rng.standard_normal((B, W * L, X)).astype(np.float32)
    packed_t = torch.from_numpy(packed).to("cuda", dtype)
    pargmax = np.zeros((B, W * L), np.int32)
    got = rd.rd_unpack_accept(dev_int(beams), dev_int(pk["unpacker"]), dev_int(pargmax), packed_t)
    ref = oracle.unpack(to_np(packed_t), pk["unpacker"])
    np.testing.assert_array_equal(to_np(got["unpacked"]), ref)


# -------------------------------------------------------------------- attention
def run_attention(prob: Problem, splits=None):
    old = rd.rd_set_knob(rd.RD_KNOB_ATTN_SPLITS, splits or 0)
    try:
        pk = rd.rd_pack_beams(prob.beams_t)
        mask = rd.rd_tree_mask(pk["unpacker"], pk["length"])
        torch.cuda.synchronize()
        prob.assert_pack_matches(pk, mask)
        out = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                                   mask, pk["length"])
        torch.cuda.synchronize()
    finally:
        rd.rd_set_knob(rd.RD_KNOB_ATTN_SPLITS, old)
    return to_np(out)


def check_attention(prob: Problem, out_np: np.ndarray):
    cfg = prob.cfg
    ref = prob.oracle_attention()
    errs = []
    for i, b in enumerate(prob.checked):
        got = out_np[b][prob.pack["unpacker"][b]]               # [W,L,Hq,D]
        errs.append(normwise_rows(got, ref[i]).ravel())
        n = prob.pack["length"][b]
        assert (out_np[b, n:] == 0).all(), "padding rows must be zero"
    errs = np.concatenate(errs)
    say(f"    attention normwise error {fmt_err(errs)} (tol {TOL[cfg.dtype]})")
    assert errs.max() <= TOL[cfg.dtype]


SMALL_ATTN = {
    "tiny_f32": get_config("tiny_f32"),
    "f32_gqa_ragged": get_config("tiny_f32").with_(name="f32_gqa", B=3, W=5, L=4, Hq=8, Hkv=2, D=128, S=75),
    "bf16_mha_ragged": get_config("llama_mha").with_(B=3, W=6, L=5, Hq=4, Hkv=4, S=200, V=512),
    "bf16_gqa_d64": get_config("gqa").with_(B=2, W=16, L=5, Hq=8, Hkv=2, D=64, S=130, V=512),
    "bf16_big_tree": get_config("dedup_p0.5").with_(B=2, Hq=2, Hkv=2, S=70, V=512),
    "bf16_no_cache": get_config("llama_mha").with_(B=2, W=4, L=6, Hq=4, Hkv=4, S=0, V=512),
    # GQA groups of 160 and 192 rows per (request, KV head)
    "bf16_gqa_mid_rows": get_config("gqa").with_(B=3, W=8, L=5, Hq=8, Hkv=2, D=128, S=300, V=512),
    "bf16_gqa_mid_rows_d64": get_config("gqa").with_(B=2, W=12, L=4, Hq=8, Hkv=2, D=64, S=190, V=512),
}


@pytest.mark.parametrize("name", list(SMALL_ATTN))
@pytest.mark.parametrize("splits", [None, 3])
def test_attention_small(name, splits):
    cfg = SMALL_ATTN[name]
    if splits is not None and cfg.dtype == "f32":
        pytest.skip("the fp32 kernel has no split path")
    prob = Problem(cfg, 1000 + len(name))
    say(f"[attn] {name} splits={splits} B={cfg.B} W={cfg.W} L={cfg.L} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} S={cfg.S}")
    check_attention(prob, run_attention(prob, splits))


def test_attention_ragged_kv_len():
    cfg = get_config("gqa").with_(B=4, W=6, L=5, Hq=8, Hkv=2, S=300, V=512)
    prob = Problem(cfg, 77, kv_len=[300, 0, 129, 64])
    for splits in (None, 4):
        say(f"[attn] ragged kv_len splits={splits}")
        check_attention(prob, run_attention(prob, splits))


# ---------------------------------------------------------------------- lm_head
SMALL_LM = {
    "tiny_f32": get_config("tiny_f32"),
    "bf16_tail": get_config("llama_mha").with_(B=3, W=4, L=5, Hq=4, Hkv=4, D=128, S=16, V=1000),
    "bf16_many_rows": get_config("dedup_p0.5").with_(B=2, Hq=4, Hkv=4, S=16, V=777),
}


@pytest.mark.parametrize("name", list(SMALL_LM))
def test_lm_head_small(name):
    cfg = SMALL_LM[name]
    prob = Problem(cfg, 4242)
    say(f"[lm] {name} rows~{prob.pack['length'].sum()} K={cfg.hidden} V={cfg.V}")
    pk = rd.rd_pack_beams(prob.beams_t)
    logits, am = rd.rd_lm_head_argmax(prob.hidden, pk["length"], prob.weight)
    torch.cuda.synchronize()
    ref = prob.oracle_logits()
    am_np = am.cpu().numpy()
    lg_np = to_np(logits)
    errs = []
    for i, b in enumerate(prob.checked):
        u = prob.pack["unpacker"][b]
        np.testing.assert_array_equal(am_np[b][u], oracle.argmax_first(ref[i]))
        assert (am_np[b, prob.pack["length"][b]:] == -1).all()
        errs.append(normwise_rows(lg_np[b][u], ref[i]).ravel())
    errs = np.concatenate(errs)
    say(f"    logits normwise error {fmt_err(errs)}")
    assert errs.max() <= TOL[cfg.dtype]


# Inner sizes that are not multiples of the k-step: a partial last k-step
# (K % 64 != 0) and an odd k-step count (the kernel pads with one all-zero
# step) in both tile shapes -- up to 512 padded rows (the wave-specialized
# shape) and above.  Packed lengths include 0 and P_max.
LM_K = {
    "few_rows_odd_ksteps": (3, 40, 576, 1000),
    "few_rows_partial_kstep": (3, 40, 584, 1000),
    "many_rows_odd_ksteps": (4, 160, 520, 777),
    "many_rows_partial_kstep": (4, 160, 584, 777),
}


@pytest.mark.parametrize("name", list(LM_K))
def test_lm_head_inner_sizes(name):
    B, P, K, V = LM_K[name]
    rng = np.random.default_rng(7100 + list(LM_K).index(name))
    plen = np.array([P, 0] + list(rng.integers(1, P, size=B - 2)), dtype=np.int32)
    hidden = round_to_bf16(rng.standard_normal((B, P, K)).astype(np.float32))
    weight = round_to_bf16((rng.standard_normal((V, K)) * 0.02).astype(np.float32))
    # redraw valid rows whose fp64 top-1 / top-2 gap is below the margin
    for _ in range(50):
        bad = []
        for b in range(B):
            lg = oracle.lm_head_logits(hidden[b, :plen[b]], weight)
            part = np.partition(lg, -2, axis=-1)
            bad += [(b, p) for p in np.nonzero(part[:, -1] - part[:, -2] < MARGIN)[0]]
        if not bad:
            break
        for b, p in bad:
            hidden[b, p] = round_to_bf16(rng.standard_normal(K).astype(np.float32))
    assert not bad
    say(f"[lm] {name}: B={B} P_max={P} K={K} V={V} rows={int(plen.sum())}")
    logits, am = rd.rd_lm_head_argmax(torch.from_numpy(hidden).cuda().to(torch.bfloat16),
                                      torch.from_numpy(plen).cuda(),
                                      torch.from_numpy(weight).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    am_np = am.cpu().numpy()
    lg_np = to_np(logits)
    errs = []
    for b in range(B):
        n = int(plen[b])
        ref = oracle.lm_head_logits(hidden[b, :n], weight)
        np.testing.assert_array_equal(am_np[b, :n], oracle.argmax_first(ref), err_msg=f"b={b}")
        assert (am_np[b, n:] == -1).all()
        if n:
            errs.append(normwise_rows(lg_np[b, :n], ref).ravel())
    errs = np.concatenate(errs)
    say(f"    logits normwise error {fmt_err(errs)}")
    assert errs.max() <= TOL["bf16"]


# ------------------------------------------------------------- whole step
FULL = {
    "tiny_f32": (None, True),
    "llama_mha": (None, True),
    "gqa": ([0, 13, 31], True),
    "dedup_p0.1": ([63], False),
    "dedup_p0.5": ([5], True),
    "dedup_p0.9": ([40], True),
    "long_ctx": ([0, 15], True),
}


@pytest.mark.parametrize("name", list(FULL))
def test_verify_step_full_size(name):
    cfg = get_config(name)
    checked, plant = FULL[name]
    say(f"[step] {name}: building inputs (checked requests {checked})")
    prob = Problem(cfg, base_seed(cfg), checked=checked, plant=plant)
    say(f"[step] {name}: inputs ready in {prob.setup_s:.1f}s, margin redraws {prob.margin_redraws}")
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight, want_logits=True)
    torch.cuda.synchronize()
    say(f"[step] {name}: GPU step done; comparing integers")
    # pack + mask for every request
    for key in ("tokens", "length", "unpacker", "depth", "src"):
        np.testing.assert_array_equal(res["pack"][key].cpu().numpy(), prob.pack[key], err_msg=key)
    np.testing.assert_array_equal(
        mask_words_np(res["mask"]),
        oracle.mask_to_bits(oracle.tree_mask(prob.pack["unpacker"], prob.pack["length"])), err_msg="mask")
    # floats and acceptance on the checked requests
    ref_logits = prob.oracle_logits()
    target = oracle.argmax_first(ref_logits)
    am = res["argmax"].cpu().numpy()
    for i, b in enumerate(prob.checked):
        np.testing.assert_array_equal(am[b][prob.pack["unpacker"][b]], target[i], err_msg=f"argmax b={b}")
    acc = prob.oracle_accept(target)
    for key in ("match_len", "best_beam", "accept_len", "accepted_tokens"):
        np.testing.assert_array_equal(res[key].cpu().numpy()[prob.checked], acc[key], err_msg=key)
    if plant:
        assert acc["accept_len"].max() > 0
    un = res["unpacked"]
    lerr = []
    for i, b in enumerate(prob.checked):
        lerr.append(normwise_rows(to_np(un[b]), ref_logits[i]).ravel())
    lerr = np.concatenate(lerr)
    say(f"[step] {name}: unpacked-logits normwise error {fmt_err(lerr)}; accept_len {acc['accept_len'].tolist()}")
    assert lerr.max() <= TOL[cfg.dtype]
    say(f"[step] {name}: oracle attention on {len(prob.checked)} requests")
    check_attention(prob, to_np(res["attn"]))


@pytest.mark.parametrize("fuse", [False, True])
def test_step_is_deterministic(fuse):
    """Two runs give bit-identical outputs (logit rows past packed_len are unspecified and skipped),
    with the logits gathered by rd_unpack_accept or in the projection."""
    cfg = get_config("gqa").with_(B=4)
    prob = Problem(cfg, 99, checked=[0])
    outs = []
    for _ in range(2):
        r = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache,
                           prob.kv_len_t, prob.hidden, prob.weight, fuse_unpack=fuse)
        torch.cuda.synchronize()
        o = {k: v.clone() for k, v in r.items() if isinstance(v, torch.Tensor)}
        n = prob.pack["length"]
        assert (o.get("logits") is None) == fuse
        if not fuse:
            o["logits"] = torch.cat([o["logits"][b, :n[b]].reshape(-1) for b in range(cfg.B)])
        outs.append(o)
    for k in outs[0]:
        a, b = outs[0][k], outs[1][k]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), k
