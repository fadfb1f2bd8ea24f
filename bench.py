"""Throughput of one ReDrafter verification step on one MI355X.

A step is the whole path: pack -> tree mask -> tree attention -> projection
+ argmax -> unpack + greedy accept, enqueued through the C ABI on one
stream.  Inputs are resident in HBM before timing starts.  The workload
defaults to the largest single-GPU setting, the dedup sweep at p = 0.1
(B=64 requests, W=64 beams of L=8 tokens, 32x128 heads, 2048 cached tokens,
vocabulary 32000, bf16); the other settings are selectable.

Prints one JSON line with the step throughput (candidate tokens/s), the
roofline position of the dominant call, of tree attention and of the
unpack gather (HIP events on the launch stream between the calls of the
timed steps), and the CPU oracle timed on a bounded sample of requests on
this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="dedup_p0.1")
    ap.add_argument("--variant", choices=["full", "argmax-only"], default="full")
    ap.add_argument("--unpack", choices=["auto", "separate", "fused"], default="auto",
                    help="full variant: gather the logits in rd_unpack_accept (separate) or in the projection "
                         "(rd_lm_head_argmax_unpack); auto chooses by size as verify_step does")
    ap.add_argument("--rotate-mb", type=float, default=1024.0,
                    help="rotate input sets until they exceed this many MB (defeats cache residency)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="requests in the oracle sample (0 = auto)")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0,
                    help="also run a plain device copy of this size (a known-traffic reference for HBM counters)")
    ap.add_argument("--graph", choices=["on", "off"], default="off",
                    help="'on' times the steps as replays of HIP graphs captured once per input set (the per-call "
                         "durations, and so the rooflines, then come from as many eager steps after the timed "
                         "region); 'off' (default) times eager calls with the per-call events inside the timed "
                         "steps. A failed capture falls back to 'off' and says so in the JSON line")
    ap.add_argument("--legs", choices=["all", "step"], default="all",
                    help="'step' times the verification step only (no commit/paged/ragged/stochastic legs)")
    ap.add_argument("--peaks", action="store_true",
                    help="also measure this box's streaming-copy rate and a vendor GEMM (torch.matmul) "
                         "of the projection's shape, for comparison")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "tree_attention_verification_rd_amd", "csrc")
CALL_SOURCES = {"lm_head": ("rd_lm_head.hip",), "lm_head_unpack": ("rd_lm_head.hip", "rd_unpack_accept.hip"),
                "attention": ("rd_attention.hip",), "unpack": ("rd_unpack_accept.hip",)}


def counted_traffic(workload: str, call: str):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record for this workload (scaled by a copy of known size), or None when
    there is no record or the kernel's sources changed since it was taken.
    The counters cannot be read inside an ordinary run, so this value is the
    record's, not a measurement of this run."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for ln in open(path):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in (*CALL_SOURCES[call], "rd_common.h", "rd_internal.h"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    if rec.get(f"{call}.sources_sha256") != h.hexdigest()[:16] or f"{call}.traffic_bytes" not in rec:
        return None
    return int(rec[f"{call}.traffic_bytes"])


def traffic_source(workload: str) -> str:
    return f"profiles/{workload}_hbm_traffic.txt (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"


def step_bytes_and_flops(cfg, plen: np.ndarray, kv_len: np.ndarray, want_logits: bool, depth=None, fused=False):
    """Algorithmic traffic and work of each call (valid packed rows only; caches read once).

    Attention flops count 4*D per (query head, visible key): every cached key
    plus the token's ancestors and itself (depth + 1 packed keys).  With the
    gather folded into the projection (fused) the projection writes every
    candidate's row once and the unpack call moves no rows."""
    R = int(plen.sum())
    e = 2 if cfg.dtype == "bf16" else 4
    D, Hq, Hkv, K, V = cfg.D, cfg.Hq, cfg.Hkv, cfg.hidden, cfg.V
    cache = int(kv_len.sum()) * Hkv * D * 2 * e
    attn_bytes = cache + R * Hkv * D * 2 * e + R * Hq * D * 2 * e
    tree_keys = 0
    if depth is not None:
        for b in range(len(plen)):
            tree_keys += int((depth[b, :plen[b]] + 1).sum())
    attn_flops = 4 * D * Hq * (int((plen.astype(np.int64) * kv_len).sum()) + tree_keys)
    cand = cfg.B * cfg.W * cfg.L
    lm_bytes = V * K * e + R * K * e + ((cand if fused else R) * V * e if want_logits else 0)
    lm_flops = 2 * R * V * K
    unpack_bytes = (R * V * e + cand * V * e) if want_logits and not fused else 0
    return {"attention": (attn_bytes, attn_flops), "lm_head": (lm_bytes, lm_flops), "unpack": (unpack_bytes, 0)}


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def baseline_requests(cfg, seed: int, sample: int):
    """Requests the oracle runs: all of them for the small workloads, else
    {0, B-1} plus seeded random ones up to `sample`."""
    if cfg.candidates <= 400 or sample >= cfg.B:
        return list(range(cfg.B))
    req = [0, cfg.B - 1]
    rng = np.random.default_rng(seed + 5)
    while len(req) < max(sample, 2):
        r = int(rng.integers(1, cfg.B - 1))
        if r not in req:
            req.append(r)
    return sorted(req)


def cpu_baseline(cfg, seed: int, sample: int):
    """The oracle as it stands (fp64 numpy, the unpacked per-candidate
    definition) on a subset of the workload's requests, with numpy's BLAS
    threads set to the host cores this process may use."""
    import oracle
    from synthetic import draw_beams, unpacked_node_tensors, kv_cache, lm_weight
    cores = len(os.sched_getaffinity(0))
    req = baseline_requests(cfg, seed, sample)
    all_beams = draw_beams(cfg, seed)
    beams = all_beams[req]
    nodes = unpacked_node_tensors(cfg, seed, all_beams, requests=req)
    kc = np.stack([kv_cache(cfg, seed, b)[0] for b in req])
    vc = np.stack([kv_cache(cfg, seed, b)[1] for b in req])
    w = lm_weight(cfg, seed)
    kv = np.full(len(req), cfg.S, np.int32)
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    # the oracle's definition is per candidate: its logits are already in
    # the unpacked [W, L, V] layout, so the step has no separate gather
    if threadpool_limits is not None:
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            oracle.verify_requests(beams, nodes["q"], nodes["k"], nodes["v"], kc, vc, kv, nodes["hidden"], w)
            dt = time.perf_counter() - t0
    else:  # pragma: no cover
        t0 = time.perf_counter()
        oracle.verify_requests(beams, nodes["q"], nodes["k"], nodes["v"], kc, vc, kv, nodes["hidden"], w)
        dt = time.perf_counter() - t0
    per_req = dt / len(req)
    full = len(req) == cfg.B
    value = cfg.W * cfg.L / per_req
    how = "full batch" if full else (f"requests {req} of {cfg.B}; per-request time x B "
                                      f"(extrapolated: requests are independent)")
    return {"value": round(value, 2), "unit": "candidate tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{cfg.name}, {how}: full step per request (pack, mask, per-beam attention, fp64 "
                      f"projection of every candidate, argmax, accept), {dt:.1f} s for {len(req)} requests"}


def measure_peaks(cfg, s, torch, dev, plen_rows: int):
    """This box's reference rates: a plain device copy (torch copy_ of 2 GB,
    source pushed out of the last-level cache by a 1 GB fill between
    copies) and the vendor GEMM (torch.matmul, hipBLASLt) of the
    projection's shape, [R, K] x [K, V] for R valid packed rows."""
    def timed(fn, reps, prep=None):
        ts = []
        for _ in range(reps):
            if prep is not None:
                prep()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    n = 2_000_000_000 // 4
    src_t = torch.ones(n, dtype=torch.float32, device=dev)
    dst_t = torch.empty_like(src_t)
    flush = torch.empty(250_000_000, dtype=torch.float32, device=dev)
    t_copy = timed(lambda: dst_t.copy_(src_t), 5, lambda: flush.fill_(1.0))
    del src_t, dst_t, flush
    K, V = cfg.hidden, cfg.V
    x = s["hidden"].reshape(-1, K)[:plen_rows].contiguous()
    wt = s["weight"].t().contiguous()  # [K, V]: a plain (non-batched) product
    for _ in range(2):
        torch.matmul(x, wt)
    torch.cuda.synchronize()
    t_mm = timed(lambda: torch.matmul(x, wt), 10)
    del x, wt
    torch.cuda.synchronize()
    return {"copy_GBs": round(2 * n * 4 / t_copy / 1e9, 1),
            "vendor_gemm": {"call": "torch.matmul (hipBLASLt), projection shape", "M": plen_rows, "N": V, "K": K,
                            "us": round(t_mm * 1e6, 1),
                            "TFLOPs": round(2 * plen_rows * V * K / t_mm / 1e12, 1)}}


def make_sets(cfg, n_sets, seed, dev, dt):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    B, P = cfg.B, cfg.P_max

    def rn(shape, scale=1.0):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * scale).to(dt)

    sets = []
    for _ in range(n_sets):
        sets.append({
            "q": rn((B, P, cfg.Hq, cfg.D)), "k_new": rn((B, P, cfg.Hkv, cfg.D)), "v_new": rn((B, P, cfg.Hkv, cfg.D)),
            "k_cache": rn((B, cfg.Hkv, cfg.S, cfg.D)), "v_cache": rn((B, cfg.Hkv, cfg.S, cfg.D)),
            "hidden": rn((B, P, cfg.hidden)), "weight": rn((cfg.V, cfg.hidden), 0.02),
        })
    return sets


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the verification path shards by "
              f"request with no exchange, and this build runs on a single device", file=sys.stderr)
        sys.exit(2)

    import torch
    import tree_attention_verification_rd_amd as rd
    from synthetic import get_config, base_seed, draw_beams, kv_lengths

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = get_config(args.config)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    esz = 2 if cfg.dtype == "bf16" else 4
    seed = base_seed(cfg)
    full = args.variant == "full"
    fused = full and (args.unpack == "fused" or
                      (args.unpack == "auto" and rd.fuse_unpack_pays(cfg.B, cfg.W, cfg.L, cfg.V, esz)))

    beams = torch.from_numpy(draw_beams(cfg, seed)).to(dev)
    kv_len_np = kv_lengths(cfg)
    kv_len = torch.from_numpy(kv_len_np).to(dev)
    B, P = cfg.B, cfg.P_max
    set_bytes = esz * (B * P * (2 * cfg.Hq + 2 * cfg.Hkv) * cfg.D + 2 * B * cfg.Hkv * cfg.S * cfg.D
                       + B * P * cfg.hidden + cfg.V * cfg.hidden)
    n_sets = int(min(8, max(2, np.ceil(args.rotate_mb * 1e6 / set_bytes))))
    sets = make_sets(cfg, n_sets, seed, dev, dt)
    bufs = rd.VerifyBuffers(B, cfg.W, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.S, cfg.hidden, cfg.V, dt, dev,
                            want_logits=full)
    pk = bufs.pack

    def step(s, ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        rd.rd_pack_beams_mask(beams, packed_tokens=pk["tokens"], packed_len=pk["length"], unpacker=pk["unpacker"],
                              packed_depth=pk["depth"], packed_src=pk["src"], mask=bufs.mask)
        rec(2)
        rd.rd_tree_attention(s["q"], s["k_new"], s["v_new"], s["k_cache"], s["v_cache"], kv_len, bufs.mask,
                             pk["length"], out=bufs.attn, workspace=bufs.attn_ws)
        rec(3)
        if fused:
            rd.rd_lm_head_argmax_unpack(s["hidden"], pk["length"], s["weight"], pk["unpacker"],
                                        unpacked=bufs.unpacked, argmax=bufs.argmax, workspace=bufs.lm_ws)
            rec(4)
            rd.rd_unpack_accept(beams, pk["unpacker"], bufs.argmax, None, **bufs.accept)
        else:
            rd.rd_lm_head_argmax(s["hidden"], pk["length"], s["weight"], want_logits=full, logits=bufs.logits,
                                 argmax=bufs.argmax, workspace=bufs.lm_ws)
            rec(4)
            rd.rd_unpack_accept(beams, pk["unpacker"], bufs.argmax, bufs.logits if full else None,
                                unpacked=bufs.unpacked, **bufs.accept)
        rec(5)

    if args.copy_calibration_mb > 0:
        # a device-to-device copy of known size; a 1 GB fill in between keeps
        # the source out of the 256 MB last-level cache, so every byte is
        # fetched from HBM
        n = int(args.copy_calibration_mb * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        flush = torch.empty(250_000_000, dtype=torch.float32, device=dev)
        for _ in range(3):
            flush.fill_(1.0)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush

    peaks = None
    if args.peaks:
        step(sets[0])
        torch.cuda.synchronize()
        peaks = measure_peaks(cfg, sets[0], torch, dev, int(pk["length"].sum().item()))

    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    K = args.steps
    # The step captured once per input set in a HIP graph (every call takes
    # torch's current stream and the preallocated buffers, and records no
    # memset): a replay launches the same kernels without the host's
    # per-call work and the gaps between launches.
    graphs, graph_note = None, None
    if args.graph == "on":
        try:
            graphs = []
            for s_ in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(s_)
                graphs.append(g)
            torch.cuda.synchronize()
            graph_note = f"timed steps are replays of {len(graphs)} HIP graphs (one per input set)"
        except Exception as exc:  # noqa: BLE001 -- any capture failure falls back to eager timing
            graphs = None
            graph_note = f"graph capture failed, eager steps timed: {type(exc).__name__}: {exc}"[:240]
            torch.cuda.synchronize()
    # Timed region: K whole steps, bracketed by synchronisation.  Eager: a HIP
    # event on the launch stream (torch's current stream, which the binding
    # passes to every call) sits between consecutive calls, so the per-call
    # durations come from the timed steps themselves; at this size each event
    # costs the GPU a few microseconds of a step of milliseconds.  Graphs: the
    # K replays are timed, and the per-call durations come from K eager steps
    # with the events run after them.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    torch.cuda.synchronize()
    if graphs:
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        w0 = time.perf_counter()
        ge[0].record()
        for i in range(K):
            graphs[i % n_sets].replay()
        ge[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_gpu = ge[0].elapsed_time(ge[1]) / K
        for i in range(K):
            step(sets[i % n_sets], evs[i])
        torch.cuda.synchronize()
    else:
        w0 = time.perf_counter()
        for i in range(K):
            step(sets[i % n_sets], evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_gpu = evs[0][0].elapsed_time(evs[K - 1][5]) / K
    ms_per_step = max(wall * 1e3 / K, ms_gpu)
    marks = {"pack_mask": (0, 2), "attention": (2, 3), "lm_head": (3, 4), "unpack_accept": (4, 5)}
    per_call_us = {n: float(np.mean([e[j0].elapsed_time(e[j1]) for e in evs]) * 1e3) for n, (j0, j1) in marks.items()}

    def queued_call_us(call, prepare):
        """Mean GPU time of call(i), i < K, run back to back.  A call can be
        shorter than its host-side enqueue, so a busy-wait kernel sized to the
        measured enqueue time goes first: the calls then queue up behind it
        and the events time the GPU, not the host.  prepare() restores any
        state the calls consume and runs before each pass, outside the events."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]

        def run():
            for i in range(K):
                evs[i][0].record()
                call(i)
                evs[i][1].record()

        prepare()
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        run()
        enqueue_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        cal = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        cal[0].record()
        torch.cuda._sleep(1_000_000)
        cal[1].record()
        torch.cuda.synchronize()
        cycles_per_ms = 1_000_000 / max(cal[0].elapsed_time(cal[1]), 1e-3)
        prepare()
        torch.cuda._sleep(int(cycles_per_ms * (2 * enqueue_s * 1e3 + 1.0)))
        run()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)

    extras = {}
    if args.legs == "all":
        # The commit of the accepted path, the call after the step (not part of
        # the timed step): at full acceptance (n = L-1 on beam 0) every request
        # appends L rows per KV head; call i advances its own kv_len row.
        c_best = torch.zeros(B, dtype=torch.int32, device=dev)
        c_nacc = torch.full((B,), cfg.L - 1, dtype=torch.int32, device=dev)
        c_kv = torch.empty((K, B), dtype=torch.int32, device=dev)
        c_hid = torch.empty((B, cfg.hidden), dtype=dt, device=dev)

        def commit_call(i):
            s = sets[i % n_sets]
            rd.rd_commit_accepted(pk["unpacker"], c_best, c_nacc, s["k_new"], s["v_new"], s["k_cache"], s["v_cache"],
                                  c_kv[i], s["hidden"], hidden_next=c_hid)

        commit_us = queued_call_us(commit_call, lambda: c_kv.fill_(cfg.S - cfg.L))

        # Tree attention over a paged cache (the same keys, cut into 64-token
        # pages of a pool in random order, one pool per input set).
        ps = 64
        npg = (cfg.S + ps - 1) // ps
        pools = []
        for si, s in enumerate(sets):
            gperm = torch.Generator()
            gperm.manual_seed(1000 + si)
            perm = torch.randperm(B * npg, generator=gperm).to(dev)
            pool = []
            for c in (s["k_cache"], s["v_cache"]):
                cp = torch.nn.functional.pad(c, (0, 0, 0, npg * ps - cfg.S)) if npg * ps != cfg.S else c
                cut = cp.reshape(B, cfg.Hkv, npg, ps, cfg.D).permute(0, 2, 1, 3, 4).reshape(B * npg, cfg.Hkv, ps, cfg.D)
                p_ = torch.empty_like(cut)
                p_[perm] = cut
                pool.append(p_)
            pools.append((pool[0], pool[1], perm.reshape(B, npg).to(torch.int32).contiguous()))
        paged_ws = torch.empty(max(rd.rd_tree_attention_workspace_size(1 if cfg.dtype == "bf16" else 0, B, P, cfg.Hq,
                                                                      cfg.Hkv, cfg.D, npg * ps), 1),
                               dtype=torch.uint8, device=dev)
        paged_out = torch.empty_like(bufs.attn)

        def paged_call(i):
            s = sets[i % n_sets]
            kp, vp, tbl = pools[i % n_sets]
            rd.rd_tree_attention_paged(s["q"], s["k_new"], s["v_new"], kp, vp, tbl, kv_len, bufs.mask, pk["length"],
                                       out=paged_out, workspace=paged_ws)

        paged_us = queued_call_us(paged_call, lambda: None)

        def commit_paged_call(i):
            s = sets[i % n_sets]
            kp, vp, tbl = pools[i % n_sets]
            rd.rd_commit_accepted_paged(pk["unpacker"], c_best, c_nacc, s["k_new"], s["v_new"], kp, vp, tbl, c_kv[i],
                                        s["hidden"], hidden_next=c_hid)

        commit_paged_us = queued_call_us(commit_paged_call, lambda: c_kv.fill_(cfg.S - cfg.L))

        # Ragged batch: the same beams with seeded per-request beam counts and
        # lengths (1..W, 1..L), through the two calls whose work depends on them.
        rng_r = np.random.default_rng(seed + 17)
        r_bw = torch.from_numpy(rng_r.integers(1, cfg.W + 1, size=B).astype(np.int32)).to(dev)
        r_bl = torch.from_numpy(rng_r.integers(1, cfg.L + 1, size=B).astype(np.int32)).to(dev)
        r_pk = {k: torch.empty_like(v) for k, v in pk.items()}
        r_mask = torch.empty_like(bufs.mask)
        r_acc = {k: torch.empty_like(v) for k, v in bufs.accept.items()}

        def ragged_pack_call(i):
            rd.rd_pack_beams_mask(beams, packed_tokens=r_pk["tokens"], packed_len=r_pk["length"],
                                  unpacker=r_pk["unpacker"], packed_depth=r_pk["depth"], packed_src=r_pk["src"],
                                  mask=r_mask, beam_width=r_bw, beam_len=r_bl)

        def ragged_accept_call(i):
            rd.rd_unpack_accept(beams, r_pk["unpacker"], bufs.argmax, bufs.logits if full else None,
                                unpacked=bufs.unpacked, beam_width=r_bw, beam_len=r_bl, **r_acc)

        # With the gather folded into the projection the step leaves no packed
        # logits: one plain projection call provides them to the legs below
        # (the separate gather, the ragged gather, stochastic verification).
        gather_us = None
        if fused:
            rd.rd_lm_head_argmax(sets[0]["hidden"], pk["length"], sets[0]["weight"], logits=bufs.logits,
                                 argmax=bufs.argmax, workspace=bufs.lm_ws)
            gather_us = queued_call_us(lambda i: rd.rd_unpack_accept(
                beams, pk["unpacker"], bufs.argmax, bufs.logits, unpacked=bufs.unpacked, **bufs.accept), lambda: None)

        # Stochastic step 4 on the step's own logits (full variant), with a
        # seeded draft distribution and uniforms.
        stoch_us = None
        if full:
            gq = torch.Generator(device=dev)
            gq.manual_seed(seed + 23)
            s_q = torch.softmax(torch.randn((B, P, cfg.V), generator=gq, device=dev), dim=-1)
            s_ua = torch.rand((B, cfg.L, cfg.W), generator=gq, device=dev)
            s_ub = torch.rand((B,), generator=gq, device=dev)
            s_ws = torch.empty(max(rd.rd_stochastic_accept_workspace_size(B, cfg.W, cfg.L), 1), dtype=torch.uint8,
                               device=dev)
            s_out = {k: torch.empty_like(v) for k, v in bufs.accept.items() if k != "match_len"}
            s_path = torch.empty_like(bufs.accept["accepted_tokens"])

            def stoch_call(i):
                rd.rd_stochastic_accept(pk["unpacker"], pk["length"], pk["tokens"], bufs.logits, s_q, s_ua, s_ub,
                                        path=s_path, workspace=s_ws, **s_out)

            stoch_us = queued_call_us(stoch_call, lambda: None)
        # bytes the call must read: the logits and q rows of every valid slot
        # (the tree structure, uniforms and outputs are a few hundred KB)
        stoch_entry = {"call": "rd_stochastic_accept", "avg_us": None if stoch_us is None else round(stoch_us, 2)}
        if stoch_us is not None:
            sbytes = int(pk["length"].sum().item()) * cfg.V * (esz + 4)
            stoch_entry.update({"hbm_bytes": sbytes, "tb_per_s": round(sbytes / stoch_us / 1e6, 3),
                                "frac_of_8tbps": round(sbytes / stoch_us / 1e6 / 8.0, 3)})

        ragged_pack_us = queued_call_us(ragged_pack_call, lambda: None)
        ragged_accept_us = queued_call_us(ragged_accept_call, lambda: None)
        ragged_packed = int(r_pk["length"].sum().item())
        contig_us = queued_call_us(lambda i: rd.rd_tree_attention(
            sets[i % n_sets]["q"], sets[i % n_sets]["k_new"], sets[i % n_sets]["v_new"], sets[i % n_sets]["k_cache"],
            sets[i % n_sets]["v_cache"], kv_len, bufs.mask, pk["length"], out=paged_out, workspace=bufs.attn_ws),
            lambda: None)
        commit_bytes = 2 * (2 * B * cfg.Hkv * cfg.L * cfg.D + B * cfg.hidden) * esz   # read + write
        extras = {
            "separate_gather_us": None if gather_us is None else round(gather_us, 2),
            "after_step": {"call": "rd_commit_accepted", "accept_len": cfg.L - 1, "avg_us": round(commit_us, 2),
                           "paged_avg_us": round(commit_paged_us, 2), "bytes_moved": int(commit_bytes)},
            "stochastic": stoch_entry,
            "ragged": {"calls": "rd_pack_beams_mask_ragged + rd_unpack_accept_ragged",
                       "candidates": int((r_bw * r_bl).sum().item()), "packed_tokens": ragged_packed,
                       "pack_mask_us": round(ragged_pack_us, 2), "unpack_accept_us": round(ragged_accept_us, 2)},
            "attention_paged": {"call": "rd_tree_attention_paged", "page_size": ps, "avg_us": round(paged_us, 2),
                                "contiguous_avg_us": round(contig_us, 2)},
        }

    plen = pk["length"].cpu().numpy()
    work = step_bytes_and_flops(cfg, plen, kv_len_np, full, pk["depth"].cpu().numpy(), fused)
    sep_work = step_bytes_and_flops(cfg, plen, kv_len_np, full, pk["depth"].cpu().numpy(), False)
    lm_call = "rd_lm_head_argmax_unpack" if fused else "rd_lm_head_argmax"
    cand = B * cfg.W * cfg.L

    def roof(call, bound):
        nbytes, flops = work[call]
        t = per_call_us[call] * 1e-6
        traffic = counted_traffic(cfg.name, "lm_head_unpack" if (fused and call == "lm_head") else call) if full else None
        if bound == "hbm":
            ach = nbytes / t / 1e9
            return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": int(nbytes), "avg_us": round(per_call_us[call], 2)}
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        ach = flops / t / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic, "algorithmic_flops": int(flops),
                "avg_us": round(per_call_us[call], 2)}

    def bound_of(call):
        nbytes, flops = work[call]
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        return "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (peak * 1e12) else "mfma"

    def binding_frac(call):
        """max(bytes at peak HBM, flops at peak MFMA) / measured: the fraction of the call's own roof."""
        nbytes, flops = work[call]
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        return max(nbytes / (PEAK_HBM_GBS * 1e9), flops / (peak * 1e12)) / (per_call_us[call] * 1e-6)

    dominant = max(("attention", "lm_head"), key=lambda c: per_call_us[c])
    line = {
        "metric": "verified candidate tokens/sec per verify step; attention HBM GB/s % peak",
        "value": round(cand / (ms_per_step * 1e-3), 1),
        "unit": "candidate tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded beams from the workload's share rule; N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": cfg.name, "B": B, "W": cfg.W, "L": cfg.L, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "S": cfg.S, "V": cfg.V, "hidden": cfg.hidden, "variant": args.variant,
                   "logits_gather": ("folded into the projection" if fused else "rd_unpack_accept") if full else None,
                   "packed_tokens": int(plen.sum()), "candidates": cand, "input_sets_rotated": n_sets},
        "roofline": {"kernel": lm_call if dominant == "lm_head" else "rd_tree_attention",
                     **roof(dominant, bound_of(dominant))},
        "attention_hbm": {"kernel": "rd_tree_attention", **roof("attention", "hbm"),
                          "algorithmic_flops": int(work["attention"][1]),
                          "binding_roof_frac": round(binding_frac("attention"), 4)},
        "per_call_us": {k: round(v, 2) for k, v in per_call_us.items()},
        "gpu_ms_per_step": round(ms_gpu, 4),
        "graph": bool(graphs), "timing": graph_note or "eager calls timed",
    }
    # The gather's roofline: the step's rd_unpack_accept, or, when the step
    # folds the gather into the projection, the separate call timed beside it
    # (--legs all).
    gather_t = per_call_us["unpack_accept"] if not fused else extras.get("separate_gather_us")
    if full and gather_t:
        nb = sep_work["unpack"][0]
        ach = nb / (gather_t * 1e-6) / 1e9
        line["gather_hbm"] = {"kernel": "rd_unpack_accept", "bound": "hbm", "achieved": round(ach, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                              "traffic": counted_traffic(cfg.name, "unpack"), "algorithmic_bytes": int(nb),
                              "avg_us": round(gather_t, 2), "in_step": not fused}
    if "attention_paged" in extras:
        ap_ = extras["attention_paged"]
        ach = work["attention"][0] / (ap_["avg_us"] * 1e-6) / 1e9
        ap_.update({"achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4)})
    line.update(extras)
    if any(line[k].get("traffic") is not None for k in ("roofline", "attention_hbm", "gather_hbm") if k in line):
        line["traffic_source"] = traffic_source(cfg.name)
    if peaks is not None:
        line["peaks_on_box"] = peaks
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, seed, args.cpu_sample or 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
