"""A whole verification step captured once in a HIP graph and replayed.

Every call of the step takes torch's current stream, allocates nothing when
given buffers and records no memset, so the step (pack+mask, attention,
projection, unpack+accept) can be captured in a torch.cuda.CUDAGraph.  Each
replay must give bit for bit what the same step gives run eagerly on the same
inputs.  The replays alternate between two input sets copied into the
captured tensors, with eager steps and synchronisations in between.
"""
import sys

import pytest
import torch

import tree_attention_verification_rd_amd as rd
from synthetic import get_config
from harness import Problem

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
    # name: (config, fuse the gather into the projection)
    "few_rows_separate_gather": (get_config("llama_mha").with_(B=4, S=512, V=4096), False),
    "gqa_folded_gather": (get_config("gqa").with_(B=3, S=1024, V=8192), True),
}
INPUTS = ("beams_t", "q", "k_new", "v_new", "k_cache", "v_cache", "kv_len_t", "hidden", "weight")


def buffers(cfg, dt):
    return rd.VerifyBuffers(cfg.B, cfg.W, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.S, cfg.hidden, cfg.V, dt, "cuda")


def step(t, bufs, fuse):
    return rd.verify_step(t["beams_t"], t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["kv_len_t"],
                          t["hidden"], t["weight"], buffers=bufs, fuse_unpack=fuse)


def snapshot(res, plen, fuse):
    """The step's outputs, cloned; logits rows past a request's packed length are unspecified and dropped."""
    out = {}
    for k, v in res.items():
        if isinstance(v, dict):
            out.update({f"{k}.{kk}": vv.clone() for kk, vv in v.items()})
        elif isinstance(v, torch.Tensor):
            out[k] = v.clone()
    if not fuse:
        out["logits"] = torch.cat([out["logits"][b, :int(plen[b])].reshape(-1) for b in range(len(plen))])
    return out


def same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return torch.equal(a, b)


@pytest.mark.parametrize("name", list(CASES))
def test_step_in_a_graph_replays_like_eager(name):
    cfg, fuse = CASES[name]
    probs = [Problem(cfg, 7100 + 10 * list(CASES).index(name) + i, checked=[0]) for i in range(2)]
    dt = probs[0].q.dtype
    say(f"[graph] {name}: B={cfg.B} W={cfg.W} L={cfg.L} V={cfg.V} fuse={fuse}")
    # eager references, one buffer set each
    refs = []
    for p in probs:
        t = {k: getattr(p, k) for k in INPUTS}
        res = step(t, buffers(cfg, dt), fuse)
        torch.cuda.synchronize()
        refs.append(snapshot(res, p.pack["length"], fuse))
    # static inputs and buffers captured by the graph
    static = {k: getattr(probs[0], k).clone() for k in INPUTS}
    bufs = buffers(cfg, dt)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static, bufs, fuse)  # first calls (library load, plans) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(static, bufs, fuse)
    torch.cuda.synchronize()
    other = buffers(cfg, dt)
    for rep, i in enumerate((0, 1, 0, 1, 1, 0)):
        for k in INPUTS:
            static[k].copy_(getattr(probs[i], k))
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(out, probs[i].pack["length"], fuse)
        bad = [k for k in refs[i] if not same(got[k], refs[i][k])]
        assert not bad, f"replay {rep} (input set {i}) differs from the eager step in {bad}"
        # eager work between replays
        step({k: getattr(probs[1 - i], k) for k in INPUTS}, other, fuse)
        torch.cuda.synchronize()
    say(f"[graph] {name}: 6 replays equal to the eager steps; accept_len {refs[0]['accept_len'].tolist()}")
