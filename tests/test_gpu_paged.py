"""GPU parity of tree attention over a paged KV cache (rd_tree_attention_paged).

Pools are cut from a contiguous cache (torch reshapes) and their pages
permuted at random, with extra unreferenced pages and table entries past
each cache length set to -1 (never read).  Where the contiguous kernel
walks the same key order (one split), the paged result must equal
rd_tree_attention's bit for bit; everywhere it must match the oracle's
paged attention (with the oracle's own mask) and the per-beam definition to
the usual normwise tolerance.  The paged commit is compared with the
oracle's paged commit of the oracle's own accept, and a table entry naming
no page must leave its request and the pool untouched.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_rd_amd as rd
from synthetic import get_config, base_seed
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


def make_pool(k_cache, v_cache, kv_len, ps, seed, extra=3, unread_to_minus_one=True):
    """Permuted page pools holding the contiguous caches, and their block table."""
    B, Hkv, S, D = k_cache.shape
    n = (S + ps - 1) // ps
    Sp = n * ps
    if Sp != S:
        pad = (0, 0, 0, Sp - S)
        k_cache = torch.nn.functional.pad(k_cache, pad)
        v_cache = torch.nn.functional.pad(v_cache, pad)

    def cut(c):
        return c.reshape(B, Hkv, n, ps, D).permute(0, 2, 1, 3, 4).reshape(B * n, Hkv, ps, D)

    kp, vp = cut(k_cache), cut(v_cache)
    g = torch.Generator()
    g.manual_seed(seed)
    total = B * n + extra
    perm = torch.randperm(total, generator=g)[: B * n]     # new slot of page i
    k_pool = torch.randn((total, Hkv, ps, D), device=k_cache.device).to(k_cache.dtype) * 100
    v_pool = torch.randn((total, Hkv, ps, D), device=k_cache.device).to(k_cache.dtype) * 100
    k_pool[perm.to(k_cache.device)] = kp
    v_pool[perm.to(k_cache.device)] = vp
    table = perm.reshape(B, n).to(torch.int32).clone()
    kl = kv_len.cpu().numpy()
    if unread_to_minus_one:
        for b in range(B):
            table[b, (int(kl[b]) + ps - 1) // ps:] = -1
    return k_pool.contiguous(), v_pool.contiguous(), table.to(k_cache.device)


def logical_from_pool(pool, table, S):
    """[B, Hkv, S, D] view of the pool through the table (torch indexing)."""
    B, n = table.shape
    ps = pool.shape[2]
    rows = pool[table.long().reshape(-1)]                         # [B*n, Hkv, ps, D]
    rows = rows.reshape(B, n, pool.shape[1], ps, pool.shape[3]).permute(0, 2, 1, 3, 4)
    return rows.reshape(B, pool.shape[1], n * ps, pool.shape[3])[:, :, :S]


def oracle_paged(prob, k_pool, v_pool, table):
    """The oracle's paged attention with the oracle's own mask and packed lengths, on the
    packed inputs of `prob` and the pools (fp64 copies)."""
    mask = oracle.tree_mask(prob.pack["unpacker"], prob.pack["length"])
    return oracle.attention_paged(to_np(prob.q), to_np(prob.k_new), to_np(prob.v_new), to_np(k_pool),
                                  to_np(v_pool), table.cpu().numpy(), prob.kv_len, mask, prob.pack["length"])


SMALL = {
    # name: (config overrides, page sizes, kv lengths)
    "mha_d128": (dict(name="llama_mha", B=3, W=4, L=4, Hq=4, Hkv=4, S=256), (64, 128), [256, 100, 0]),
    "gqa_d128": (dict(name="gqa", B=2, W=5, L=3, Hq=8, Hkv=2, S=320), (64,), [320, 129]),
    "mha_d64": (dict(name="llama_mha", B=2, W=3, L=5, Hq=2, Hkv=2, D=64, S=192), (64, 192), [191, 64]),
    "f32": (dict(name="tiny_f32", B=3, W=4, L=4, S=60), (1, 7, 16, 60), [60, 23, 1]),
    "split": (dict(name="gqa", B=1, W=4, L=4, Hq=4, Hkv=1, S=4096), (64, 256), [4096]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_paged_small(name):
    over, page_sizes, kvl = SMALL[name]
    over = dict(over)
    base = get_config(over.pop("name")).with_(**over)
    prob = Problem(base, base_seed(base, 4), kv_len=np.array(kvl, np.int32))
    pk = rd.rd_pack_beams(prob.beams_t)
    mask = rd.rd_tree_mask(pk["unpacker"], pk["length"])
    torch.cuda.synchronize()
    prob.assert_pack_matches(pk, mask)   # the mask the kernels read is the oracle's
    ref = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t, mask,
                               pk["length"])
    per_beam = prob.oracle_attention()   # the plain definition: each candidate over its own beam
    for ps in page_sizes:
        k_pool, v_pool, table = make_pool(prob.k_cache, prob.v_cache, prob.kv_len_t, ps, seed=ps)
        got = rd.rd_tree_attention_paged(prob.q, prob.k_new, prob.v_new, k_pool, v_pool, table, prob.kv_len_t,
                                         mask, pk["length"])
        torch.cuda.synchronize()
        plan_split = name == "split"
        if not plan_split:
            assert torch.equal(got, ref), f"{name} ps={ps}: paged differs from contiguous"
        want = oracle_paged(prob, k_pool, v_pool, table)
        plen = prob.pack["length"]
        errs = np.concatenate([normwise_rows(to_np(got[b, :plen[b]]), want[b, :plen[b]]).ravel()
                               for b in range(base.B)])
        un = prob.pack["unpacker"]
        errs_pb = np.concatenate([normwise_rows(to_np(got[b])[un[b]], per_beam[b]).ravel() for b in range(base.B)])
        say(f"[paged] {name} ps={ps}: oracle paged normwise {fmt_err(errs)}, per-beam {fmt_err(errs_pb)}")
        assert errs.max() <= TOL[base.dtype] and errs_pb.max() <= TOL[base.dtype]
        for b in range(base.B):
            assert (got[b, plen[b]:] == 0).all()


@pytest.mark.parametrize("name,split_exact", [("llama_mha", True), ("long_ctx", False)])
def test_paged_full_size(name, split_exact):
    """The bench's workloads: paged (64-token pages, permuted pool) against the contiguous call."""
    cfg = get_config(name)
    prob = Problem(cfg, base_seed(cfg), checked=[0])
    pk = rd.rd_pack_beams(prob.beams_t)
    mask = rd.rd_tree_mask(pk["unpacker"], pk["length"])
    torch.cuda.synchronize()
    prob.assert_pack_matches(pk, mask)
    ref = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t, mask,
                               pk["length"])
    k_pool, v_pool, table = make_pool(prob.k_cache, prob.v_cache, prob.kv_len_t, 64, seed=1)
    got = rd.rd_tree_attention_paged(prob.q, prob.k_new, prob.v_new, k_pool, v_pool, table, prob.kv_len_t, mask,
                                     pk["length"])
    torch.cuda.synchronize()
    if split_exact:
        assert torch.equal(got, ref)
    else:
        # several splits: the contiguous kernel strides its cache tiles, the paged one does not, so the
        # summation order differs; both are compared per row
        plen = pk["length"].cpu().numpy()
        errs = np.concatenate([normwise_rows(to_np(got[b, :plen[b]]), to_np(ref[b, :plen[b]])).ravel()
                               for b in range(cfg.B)])
        say(f"[paged] {name}: paged vs contiguous normwise {fmt_err(errs)}")
        assert errs.max() <= TOL[cfg.dtype]
    # request 0 against the oracle, through the paged definition
    ref0 = prob.oracle_attention()[0]
    un = pk["unpacker"].cpu().numpy()[0]
    err = normwise_rows(to_np(got[0])[un], ref0).max()
    say(f"[paged] {name}: request 0 vs oracle normwise {err:.3e}")
    assert err <= TOL[cfg.dtype]


def test_paged_invalid_arguments():
    q = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((2, 2, 32, 128), dtype=torch.bfloat16, device="cuda")   # 32-token pages: not for bf16
    table = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    kvl = torch.zeros((1,), dtype=torch.int32, device="cuda")
    mask = torch.zeros((1, 4, 1), dtype=torch.int32, device="cuda")
    plen = torch.ones((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(rd.RdError) as ei:
        rd.rd_tree_attention_paged(q, kv, kv, pool, pool, table, kvl, mask, plen)
    assert ei.value.code == -2


@pytest.mark.parametrize("name,ps", [("llama_mha", 64), ("gqa", 128), ("tiny_f32", 7)])
def test_paged_commit_then_attention(name, ps):
    """Paged commit equals the contiguous commit; the next step's paged attention sees the same cache."""
    # S is a multiple of the page size, so both caches hold the same number of positions
    over = {"llama_mha": dict(B=4, S=256), "gqa": dict(B=3, S=384), "tiny_f32": dict(B=3, S=42)}[name]
    cfg = get_config(name).with_(**over)
    kv = np.array([0, cfg.S - cfg.L] + [37] * (cfg.B - 3) + [cfg.S], np.int32)   # the last one overflows
    prob = Problem(cfg, base_seed(cfg, 2), plant=True, kv_len=kv)
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight, want_logits=False)
    un, best, nacc = res["pack"]["unpacker"], res["best_beam"], res["accept_len"]
    prob.assert_pack_matches(res["pack"], res["mask"])
    acc = prob.oracle_accept(prob.oracle_target())
    for key in ("best_beam", "accept_len"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), acc[key], err_msg=key)
    k_pool, v_pool, table = make_pool(prob.k_cache, prob.v_cache, prob.kv_len_t, ps, seed=5,
                                      unread_to_minus_one=False)
    # the oracle's paged commit of its own accept, on the pools as they are before the commit
    want = oracle.commit_accepted_paged(prob.k_unp, prob.v_unp, prob.h_unp, acc["best_beam"], acc["accept_len"],
                                        to_np(k_pool), to_np(v_pool), table.cpu().numpy(), prob.kv_len)
    untouched = [i for i in range(k_pool.shape[0]) if i not in set(table.cpu().numpy().ravel().tolist())]
    spare_k, spare_v = k_pool[untouched].clone(), v_pool[untouched].clone()
    kv_c, kv_p = prob.kv_len_t.clone(), prob.kv_len_t.clone()
    h_c = rd.rd_commit_accepted(un, best, nacc, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, kv_c,
                                prob.hidden)
    h_p = rd.rd_commit_accepted_paged(un, best, nacc, prob.k_new, prob.v_new, k_pool, v_pool, table, kv_p,
                                      prob.hidden)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv_p.cpu().numpy(), want["kv_len"])
    np.testing.assert_array_equal(to_np(k_pool), want["k_pages"])
    np.testing.assert_array_equal(to_np(v_pool), want["v_pages"])
    for b in np.nonzero(want["committed"])[0]:
        np.testing.assert_array_equal(to_np(h_p[b]), want["hidden_next"][b])
    assert torch.equal(kv_p, kv_c)
    moved = (kv_c != prob.kv_len_t).cpu().numpy()
    np.testing.assert_array_equal(moved, want["committed"])
    assert moved[0] and not moved[-1]
    for b in np.nonzero(moved)[0]:
        assert torch.equal(h_p[b], h_c[b])
    assert torch.equal(logical_from_pool(k_pool, table, cfg.S), prob.k_cache)
    assert torch.equal(logical_from_pool(v_pool, table, cfg.S), prob.v_cache)
    assert torch.equal(k_pool[untouched], spare_k) and torch.equal(v_pool[untouched], spare_v)
    # next step over the grown caches: paged and contiguous attention agree bit for bit
    pk = rd.rd_pack_beams(prob.beams_t)
    mask = rd.rd_tree_mask(pk["unpacker"], pk["length"])
    a_c = rd.rd_tree_attention(prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, kv_c, mask, pk["length"])
    a_p = rd.rd_tree_attention_paged(prob.q, prob.k_new, prob.v_new, k_pool, v_pool, table, kv_p, mask,
                                     pk["length"])
    torch.cuda.synchronize()
    assert torch.equal(a_p, a_c)
    say(f"[paged] commit {name} ps={ps}: {int(moved.sum())}/{cfg.B} committed, exact")


@pytest.mark.parametrize("bad", [-1, 1 << 20])
def test_paged_commit_with_a_table_entry_outside_the_pool(bad):
    """A request whose committed positions reach an entry naming no page stays unchanged (no page written,
    kv_len kept); the other requests commit as the oracle says."""
    cfg = get_config("llama_mha").with_(B=4, S=256)
    kv = np.array([60, 100, 0, 130], np.int32)
    prob = Problem(cfg, base_seed(cfg, 6), plant=True, kv_len=kv)
    res = rd.verify_step(prob.beams_t, prob.q, prob.k_new, prob.v_new, prob.k_cache, prob.v_cache, prob.kv_len_t,
                         prob.hidden, prob.weight, want_logits=False)
    acc = prob.oracle_accept(prob.oracle_target())
    for key in ("best_beam", "accept_len"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), acc[key], err_msg=key)
    k_pool, v_pool, table = make_pool(prob.k_cache, prob.v_cache, prob.kv_len_t, 64, seed=9,
                                      unread_to_minus_one=False)
    tbl = table.cpu().numpy()
    tbl[0, 1] = bad      # request 0 commits positions 60..60+n: position 64 onwards has no page when n >= 4
    tbl[1, 2] = bad      # request 1 commits 100..100+n (page 1): this entry is never reached
    tbl[3, 2] = bad      # request 3 commits 130..130+n (page 2): always rejected
    table = torch.from_numpy(tbl).to(k_pool.device)
    want = oracle.commit_accepted_paged(prob.k_unp, prob.v_unp, prob.h_unp, acc["best_beam"], acc["accept_len"],
                                        to_np(k_pool), to_np(v_pool), tbl, prob.kv_len)
    kv_p = prob.kv_len_t.clone()
    h_p = rd.rd_commit_accepted_paged(res["pack"]["unpacker"], res["best_beam"], res["accept_len"], prob.k_new,
                                      prob.v_new, k_pool, v_pool, table, kv_p, prob.hidden)
    torch.cuda.synchronize()
    assert not want["committed"][3] and want["committed"][1] and want["committed"][2]
    np.testing.assert_array_equal(kv_p.cpu().numpy(), want["kv_len"])
    np.testing.assert_array_equal(to_np(k_pool), want["k_pages"])
    np.testing.assert_array_equal(to_np(v_pool), want["v_pages"])
    for b in np.nonzero(want["committed"])[0]:
        np.testing.assert_array_equal(to_np(h_p[b]), want["hidden_next"][b])
    say(f"[paged] commit with entry {bad}: committed {want['committed'].tolist()}, exact")
