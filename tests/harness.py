"""Shared helpers for the GPU parity tests and the smoke check.

Builds one verification-step problem from the seeded generator: beams for
every request; prefix-keyed per-token tensors, KV caches and the output
projection exactly as the generator draws them for the requests the oracle
checks; seeded device noise of the same shape for the others (their values
are never compared).  Hidden states of the checked requests are redrawn
until every candidate's fp64 top-1/top-2 logit gap is at least MARGIN, so
the greedy target is unambiguous; optional "plants" add a multiple of a
vocabulary row to a prefix's hidden state to force a chosen target token.
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle
from synthetic import (Config, draw_beams, node_qkv, node_hidden, kv_cache, lm_weight, round_to_bf16,
                       kv_lengths)

MARGIN = 1e-2
TOL = {"f32": 1e-5, "bf16": 2e-2}


def torch_dtype(cfg: Config):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def prefix_table(beams_b: np.ndarray):
    """Unique prefixes of one request in first-occurrence order, and each candidate's prefix."""
    W, L = beams_b.shape
    order, where = [], {}
    for w in range(W):
        for l in range(L):
            pre = tuple(int(t) for t in beams_b[w, :l + 1])
            if pre not in where:
                where[pre] = []
                order.append(pre)
            where[pre].append((w, l))
    return order, where


def top2_gap(logits: np.ndarray) -> np.ndarray:
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]


def build_hidden(cfg: Config, seed: int, b: int, prefixes, weight: np.ndarray, plants=None, log=None):
    """Hidden state per prefix with enforced argmax margins; returns dict prefix -> vector, logits."""
    plants = plants or {}
    retry = {pre: 0 for pre in prefixes}
    hid, logit = {}, {}
    todo = list(prefixes)
    rounds = 0
    while todo:
        rows = []
        for pre in todo:
            h = node_hidden(cfg, seed, b, pre, retry[pre])
            if pre in plants:
                h = h.astype(np.float32) + np.float32(plants[pre][1]) * weight[plants[pre][0]].astype(np.float32)
                h = round_to_bf16(h) if cfg.dtype == "bf16" else h.astype(np.float32)
            hid[pre] = h
            rows.append(h)
        lg = oracle.lm_head_logits(np.stack(rows), weight)
        gaps = top2_gap(lg)
        nxt = []
        for pre, row, gap in zip(todo, lg, gaps):
            logit[pre] = row
            if gap < MARGIN:
                retry[pre] += 1
                nxt.append(pre)
        todo = nxt
        rounds += 1
        if rounds > 50:
            raise RuntimeError("could not enforce argmax margins")
    if log is not None:
        log.append(sum(1 for r in retry.values() if r))
    return hid, logit


class Problem:
    """One verification-step problem on the device plus the oracle's view of the checked requests."""

    def __init__(self, cfg: Config, seed: int, checked=None, beams_mode="workload", plant=False,
                 device="cuda", kv_len=None, beams=None, beam_width=None, beam_len=None):
        t0 = time.time()
        self.cfg, self.seed = cfg, seed
        B, W, L, P = cfg.B, cfg.W, cfg.L, cfg.P_max
        self.checked = list(range(B)) if checked is None else sorted(set(checked))
        self.beams = draw_beams(cfg, seed, beams_mode) if beams is None else np.asarray(beams, np.int32)
        self.kv_len = kv_lengths(cfg) if kv_len is None else np.asarray(kv_len, np.int32)
        # ragged batches: per-request beam count and length (None: every request is full)
        self.beam_width = None if beam_width is None else np.asarray(beam_width, np.int32)
        self.beam_len = None if beam_len is None else np.asarray(beam_len, np.int32)
        self.pack = oracle.pack_beams(self.beams, self.beam_width, self.beam_len)
        dt = torch_dtype(cfg)
        dev = torch.device(device)
        self.weight_np = lm_weight(cfg, seed)
        self.weight64 = self.weight_np.astype(np.float64)  # converted once for the oracle
        self.weight = torch.from_numpy(self.weight_np).to(dev, dt)

        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 7919 + 17)

        def noise(shape):
            return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(dt)

        self.q = noise((B, P, cfg.Hq, cfg.D))
        self.k_new = noise((B, P, cfg.Hkv, cfg.D))
        self.v_new = noise((B, P, cfg.Hkv, cfg.D))
        self.hidden = noise((B, P, cfg.hidden))
        self.k_cache = torch.empty((B, cfg.Hkv, cfg.S, cfg.D), dtype=dt, device=dev)
        self.v_cache = torch.empty_like(self.k_cache)
        n = len(self.checked)
        self.q_unp = np.zeros((n, W, L, cfg.Hq, cfg.D), np.float32)
        self.k_unp = np.zeros((n, W, L, cfg.Hkv, cfg.D), np.float32)
        self.v_unp = np.zeros_like(self.k_unp)
        self.h_unp = np.zeros((n, W, L, cfg.hidden), np.float32)
        self.kc_np = np.zeros((n, cfg.Hkv, cfg.S, cfg.D), np.float32)
        self.vc_np = np.zeros_like(self.kc_np)
        self.plants = {}
        margin_fix = []
        checked_set = set(self.checked)
        for b in range(B):
            if b not in checked_set:
                self.k_cache[b].copy_(noise((cfg.Hkv, cfg.S, cfg.D)))
                self.v_cache[b].copy_(noise((cfg.Hkv, cfg.S, cfg.D)))
        for i, b in enumerate(self.checked):
            order, where = prefix_table(self.beams[b])
            plants = self._plants(b, where) if plant else {}
            self.plants[b] = plants
            hid, _ = build_hidden(cfg, seed, b, order, self.weight64, plants, margin_fix)
            for pre in order:
                qv, kv, vv = node_qkv(cfg, seed, b, pre)
                for (w, l) in where[pre]:
                    self.q_unp[i, w, l], self.k_unp[i, w, l], self.v_unp[i, w, l] = qv, kv, vv
                    self.h_unp[i, w, l] = hid[pre]
            kc, vc = kv_cache(cfg, seed, b)
            self.kc_np[i], self.vc_np[i] = kc, vc
            self.k_cache[b].copy_(torch.from_numpy(kc).to(dev, dt))
            self.v_cache[b].copy_(torch.from_numpy(vc).to(dev, dt))
            # packed layout: slot p holds the tensors of its first occurrence
            src = self.pack["src"][b, :self.pack["length"][b]]
            w_idx, l_idx = np.divmod(src, L)
            npk = len(src)
            for name, arr in (("q", self.q_unp), ("k_new", self.k_unp), ("v_new", self.v_unp),
                              ("hidden", self.h_unp)):
                dst = getattr(self, name)
                dst[b].zero_()
                dst[b, :npk].copy_(torch.from_numpy(np.ascontiguousarray(arr[i][w_idx, l_idx])).to(dev, dt))
        self.margin_redraws = sum(margin_fix)
        self.kv_len_t = torch.from_numpy(self.kv_len).to(dev)
        self.beams_t = torch.from_numpy(self.beams).to(dev)
        self.setup_s = time.time() - t0

    def _plants(self, b, where):
        """Force the target along a prefix of one beam: target(w*, j) = beams[w*, j+1] for j < n*."""
        cfg = self.cfg
        rng = np.random.default_rng(self.seed * 131 + b)
        W, L = cfg.W, cfg.L
        if self.beam_width is not None:     # plant inside the request's own beams
            W = int(min(max(self.beam_width[b], 1), cfg.W))
            L = int(min(max(self.beam_len[b], 1), cfg.L))
        w_star = int(rng.integers(0, W))
        n_star = int(rng.integers(1, L)) if L > 1 else 0
        # raises the target logit by about 12, far above the ~4 sigma maximum of the random logits
        scale = 12.0 / (cfg.hidden * 0.02 ** 2)
        plants = {}
        for j in range(n_star):
            pre = tuple(int(t) for t in self.beams[b, w_star, :j + 1])
            plants[pre] = (int(self.beams[b, w_star, j + 1]), scale)
        return plants

    # ---------------------------------------------------------- oracle side
    def oracle_attention(self):
        sub = self.checked
        return oracle.attention_per_beam(self.q_unp, self.k_unp, self.v_unp, self.kc_np, self.vc_np,
                                         self.kv_len[sub])

    def oracle_logits(self):
        return oracle.lm_head_logits(self.h_unp, self.weight64)

    def oracle_accept(self, target_unp):
        sub = self.checked
        if self.beam_width is None:
            return oracle.greedy_accept(self.beams[sub], target_unp)
        return oracle.greedy_accept(self.beams[sub], target_unp, self.beam_width[sub], self.beam_len[sub])

    def oracle_target(self):
        """Greedy target token of every candidate of the checked requests (fp64 oracle logits)."""
        return oracle.argmax_first(self.oracle_logits())

    def oracle_mask_bits(self):
        """The oracle's tree-mask words of every request."""
        return oracle.mask_to_bits(oracle.tree_mask(self.pack["unpacker"], self.pack["length"]))

    def assert_pack_matches(self, pk, mask=None):
        """GPU pack (and mask) bit-exact against the oracle's on every request."""
        for key in ("tokens", "length", "unpacker"):
            np.testing.assert_array_equal(pk[key].cpu().numpy(), self.pack[key], err_msg=f"pack {key}")
        if mask is not None:
            np.testing.assert_array_equal(mask_words_np(mask), self.oracle_mask_bits(), err_msg="mask")


def normwise_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row error max|x - r| / max|r| over the last axis."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def mask_words_np(mask_t: torch.Tensor) -> np.ndarray:
    return mask_t.detach().cpu().numpy().view(np.uint32)


def gather_unpacked(packed_np: np.ndarray, unpacker_b: np.ndarray) -> np.ndarray:
    """Rows of one request's packed array at each candidate's slot (comparison indexing)."""
    return packed_np[unpacker_b]


def fmt_err(x: np.ndarray) -> str:
    return f"max {x.max():.3e}, mean {x.mean():.3e}" if x.size else "empty"


def sqrt_d(cfg: Config) -> float:
    return math.sqrt(cfg.D)
