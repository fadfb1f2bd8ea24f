"""GPU parity of rd_lm_head_argmax_unpack: the projection with the unpack gather folded in.

Against the oracle: every candidate row of the checked requests (the fp64
projection of the candidate's hidden row, normwise 2e-2 / 1e-5), the greedy
target of every candidate, and zeros for the padding candidates of ragged
requests.  Against the separate calls: the unpacked logits and the argmax
equal rd_lm_head_argmax followed by rd_unpack_accept's gather bit for bit,
in the fp32 path and both bf16 tile shapes, at full workload sizes, with
ragged batches, and when the prefix sharing makes most rows stand for many
candidates.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config
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


CASES = {
    # name: (config, checked requests (None: all), ragged)
    "tiny_f32": (get_config("tiny_f32"), None, False),
    "few_rows_bf16": (get_config("llama_mha").with_(B=3, W=4, L=5, Hq=4, Hkv=4, D=128, S=16, V=1000), None, False),
    "many_rows_bf16": (get_config("dedup_p0.5").with_(B=2, Hq=4, Hkv=4, S=16, V=777), None, False),
    "shared_prefixes": (get_config("dedup_p0.9").with_(B=2, Hq=4, Hkv=4, S=16, V=777), None, False),
    "ragged_few_rows": (get_config("llama_mha").with_(B=6, Hq=4, Hkv=4, S=16, V=1000), None, True),
    "ragged_many_rows": (get_config("dedup_p0.5").with_(B=3, Hq=4, Hkv=4, S=16, V=777), None, True),
    "llama_mha": (get_config("llama_mha"), [0, 7], False),
    "dedup_p0.1": (get_config("dedup_p0.1"), [63], False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_lm_head_unpack(name):
    cfg, checked, ragged = CASES[name]
    B, W, L = cfg.B, cfg.W, cfg.L
    kw = {}
    if ragged:
        rng = np.random.default_rng(8801 + list(CASES).index(name))
        bw = rng.integers(0, W + 1, size=B).astype(np.int32)
        bl = rng.integers(0, L + 1, size=B).astype(np.int32)
        bw[0], bl[0] = W, L
        kw = {"beam_width": bw, "beam_len": bl}
    prob = Problem(cfg, 8800 + list(CASES).index(name), checked=checked, **kw)
    say(f"[fused unpack] {name}: B={B} W={W} L={L} V={cfg.V} rows={int(prob.pack['length'].sum())}")
    if ragged:
        pk, _ = rd.rd_pack_beams_mask(prob.beams_t, beam_width=torch.from_numpy(kw["beam_width"]).cuda(),
                                      beam_len=torch.from_numpy(kw["beam_len"]).cuda())
    else:
        pk, _ = rd.rd_pack_beams_mask(prob.beams_t)
    prob.assert_pack_matches(pk)
    unp, am = rd.rd_lm_head_argmax_unpack(prob.hidden, pk["length"], prob.weight, pk["unpacker"])
    logits, am2 = rd.rd_lm_head_argmax(prob.hidden, pk["length"], prob.weight)
    sep = rd.rd_unpack_accept(prob.beams_t, pk["unpacker"], am2, logits)["unpacked"]
    torch.cuda.synchronize()
    # the separate calls, bit for bit
    assert torch.equal(am, am2)
    assert torch.equal(unp.view(torch.int16) if unp.dtype == torch.bfloat16 else unp.view(torch.int32),
                       sep.view(torch.int16) if sep.dtype == torch.bfloat16 else sep.view(torch.int32))
    # the oracle, on the checked requests
    ref = prob.oracle_logits()          # [n, W, L, V]; padding candidates have zero hidden rows
    target = prob.oracle_target()       # [n, W, L]
    am_np = am.cpu().numpy()
    un_np = to_np(unp)
    errs = []
    for i, b in enumerate(prob.checked):
        u = prob.pack["unpacker"][b]
        real = u >= 0
        got = un_np[b][real]
        errs.append(normwise_rows(got, ref[i][real]).ravel())
        np.testing.assert_array_equal(am_np[b][u[real]], target[i][real], err_msg=f"b={b}")
        assert (un_np[b][~real] == 0).all(), "padding candidates unpack to zeros"
    errs = np.concatenate(errs)
    say(f"    unpacked logits normwise error {fmt_err(errs)}")
    assert errs.max() <= TOL[cfg.dtype]


def test_lm_head_unpack_empty_and_errors():
    cfg = get_config("llama_mha").with_(B=2, W=4, L=3, Hq=4, Hkv=4, S=16, V=300)
    prob = Problem(cfg, 8850)
    pk, _ = rd.rd_pack_beams_mask(prob.beams_t)
    # B = 0 is a no-op
    lib = rd.load_library()
    assert lib.rd_lm_head_argmax_unpack(rd.RD_BF16, None, None, None, None, 0, 4, 3, 128, 300, None, None, None, 0,
                                        None) == rd.RD_OK
    # a workspace smaller than the size query
    need = rd.rd_lm_head_argmax_unpack_workspace_size(rd.RD_BF16, cfg.B, cfg.W, cfg.L, cfg.hidden, cfg.V)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(rd.RdError) as ei:
        rd.rd_lm_head_argmax_unpack(prob.hidden, pk["length"], prob.weight, pk["unpacker"], workspace=small)
    assert ei.value.code == rd.RD_E_WORKSPACE
