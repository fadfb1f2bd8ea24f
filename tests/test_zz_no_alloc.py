"""rd_lm_head_argmax_noalloc (no workspace, fixed device scratch) against rd_lm_head_argmax.

Two calls in a row through the C ABI, the second with a smaller input, each
compared with the workspace entry point on the same inputs: argmax bit-exact
and the logits of every valid row identical (the same kernels run on both
paths, only the partials' home differs).  Sizes whose partials do not fit
the fixed array are refused before anything is launched.
"""
import sys

import numpy as np
import pytest
import torch

import tree_attention_verification_rd_amd as rd

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    rd.load_library()


def inputs(B, P, K, V, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hidden = torch.randn((B, P, K), generator=g, device="cuda").to(dtype)
    weight = (torch.randn((V, K), generator=g, device="cuda") * 0.02).to(dtype)
    plen = torch.from_numpy(np.random.default_rng(seed).integers(0, P + 1, size=B).astype(np.int32)).cuda()
    plen[0] = P
    return hidden, plen, weight


# (B, P, K, V): the many-row tile shape at the dedup sweep's width, then the few-row shape (smaller)
CASES = [(8, 512, 4096, 32000, torch.bfloat16), (3, 20, 512, 1000, torch.bfloat16), (2, 16, 256, 1000, torch.float32)]


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    for i, (B, P, K, V, dt) in enumerate(CASES):
        hidden, plen, weight = inputs(B, P, K, V, 100 + i, dt)
        need = rd.rd_lm_head_workspace_size(rd.RD_F32 if dt == torch.float32 else rd.RD_BF16, B, P, K, V)
        assert need <= rd.RD_NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] call {i}: B={B} P={P} K={K} V={V} {dt}, partials {need} bytes")
        ref_logits, ref_arg = rd.rd_lm_head_argmax(hidden, plen, weight)
        logits = torch.full((B, P, V), 3.0, dtype=dt, device="cuda")
        argmax = torch.full((B, P), -7, dtype=torch.int32, device="cuda")
        rd.rd_lm_head_argmax_noalloc(hidden, plen, weight, logits=logits, argmax=argmax)
        torch.cuda.synchronize()
        assert torch.equal(argmax, ref_arg), f"call {i}: argmax differs"
        for b, n in enumerate(plen.cpu().numpy()):
            assert torch.equal(logits[b, :n], ref_logits[b, :n]), f"call {i}: logits of request {b} differ"
            assert (logits[b, n:] == 3.0).all(), f"call {i}: rows past the packed length were written"
        # argmax-only form: no logits pointer
        argmax2 = torch.full((B, P), -7, dtype=torch.int32, device="cuda")
        rd.rd_lm_head_argmax_noalloc(hidden, plen, weight, logits=None, argmax=argmax2)
        torch.cuda.synchronize()
        assert torch.equal(argmax2, ref_arg)


def test_sizes_beyond_the_fixed_scratch_are_refused():
    # 64 x 1024 rows at V = 128256: the partials need about 260 MB
    B, P, K, V = 64, 1024, 8, 128256
    need = rd.rd_lm_head_workspace_size(rd.RD_BF16, B, P, K, V)
    assert need > rd.RD_NOALLOC_SCRATCH_BYTES
    hidden = torch.zeros((B, P, K), dtype=torch.bfloat16, device="cuda")
    weight = torch.zeros((V, K), dtype=torch.bfloat16, device="cuda")
    argmax = torch.full((B, P), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(rd.RdError) as ei:
        rd.rd_lm_head_argmax_noalloc(hidden, None, weight, logits=None, argmax=argmax)
    assert ei.value.code == rd.RD_E_SCRATCH
    torch.cuda.synchronize()
    assert (argmax == -7).all()
