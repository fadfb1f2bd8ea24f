"""Seeded input generator for the verification-step workloads.

Every array is a pure function of (workload, seed, request, ...), drawn with
numpy's PCG64 behind a SeedSequence keyed by integer words, so a single
request's inputs can be regenerated without drawing the whole batch.

Workload shapes follow the five synthetic settings the build targets:
beam-search candidates [B, W, L] whose beams copy a prefix of the previous
beam (uniform share length, or a per-position continue-with-probability-p
rule), N(0,1) queries / keys / values / hidden states and an N(0, 0.02^2)
output projection.  The per-token tensors are a function of the token
prefix (the tokens from depth 0 to the token itself), because a real target
model produces identical states for identical prefixes; that is what makes
removing duplicated prefixes lossless.

bf16 workloads: values are drawn in fp32 and rounded to the nearest bf16
(ties to even), then kept as float32 arrays holding exactly representable
values, so both sides consume identical numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "base_seed", "rng_for", "round_to_bf16",
    "draw_beams", "node_qkv", "node_hidden", "unpacked_node_tensors",
    "kv_cache", "lm_weight", "kv_lengths",
]

# integer tags that key the independent random streams
TAG_BEAMS = 1
TAG_QKV = 2
TAG_HIDDEN = 3
TAG_KCACHE = 4
TAG_VCACHE = 5
TAG_WEIGHT = 6


@dataclass(frozen=True)
class Config:
    name: str
    index: int          # workload number, keys the seed
    B: int              # requests
    W: int              # beams per request
    L: int              # tokens per beam
    V: int              # vocabulary
    Hq: int             # query heads
    Hkv: int            # key/value heads
    D: int              # head dim
    S: int              # KV-cache tokens per request
    dtype: str          # "f32" or "bf16"
    share: str          # "uniform" (U{0..L-1}) or "geometric" (continue w.p. p, cap L)
    p: float = 0.0

    @property
    def hidden(self) -> int:
        return self.Hq * self.D

    @property
    def P_max(self) -> int:
        return self.W * self.L

    @property
    def candidates(self) -> int:
        return self.B * self.W * self.L

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny_f32": Config("tiny_f32", 0, B=1, W=4, L=4, V=1000, Hq=4, Hkv=4, D=64, S=64,
                       dtype="f32", share="uniform"),
    "llama_mha": Config("llama_mha", 1, B=8, W=8, L=5, V=32000, Hq=32, Hkv=32, D=128, S=1024,
                        dtype="bf16", share="uniform"),
    "gqa": Config("gqa", 2, B=32, W=16, L=5, V=128256, Hq=32, Hkv=8, D=128, S=4096,
                  dtype="bf16", share="uniform"),
    "dedup_p0.1": Config("dedup_p0.1", 31, B=64, W=64, L=8, V=32000, Hq=32, Hkv=32, D=128,
                         S=2048, dtype="bf16", share="geometric", p=0.1),
    "dedup_p0.5": Config("dedup_p0.5", 35, B=64, W=64, L=8, V=32000, Hq=32, Hkv=32, D=128,
                         S=2048, dtype="bf16", share="geometric", p=0.5),
    "dedup_p0.9": Config("dedup_p0.9", 39, B=64, W=64, L=8, V=32000, Hq=32, Hkv=32, D=128,
                         S=2048, dtype="bf16", share="geometric", p=0.9),
    "long_ctx": Config("long_ctx", 4, B=16, W=8, L=5, V=128256, Hq=32, Hkv=8, D=128, S=32768,
                       dtype="bf16", share="uniform"),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def base_seed(cfg: Config, trial: int = 0) -> int:
    return 1000 * cfg.index + trial


def rng_for(seed: int, *words: int) -> np.random.Generator:
    """Independent PCG64 stream keyed by non-negative integer words."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, words)])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def _finish(cfg: Config, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if cfg.dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _share_length(cfg: Config, rng: np.random.Generator) -> int:
    if cfg.share == "uniform":
        return int(rng.integers(0, cfg.L))          # U{0..L-1}
    if cfg.share == "geometric":
        s = 0
        while s < cfg.L and rng.random() < cfg.p:  # keep sharing while U < p; cap L
            s += 1
        return s
    raise ValueError(cfg.share)


def draw_beams(cfg: Config, seed: int, mode: str = "workload") -> np.ndarray:
    """Candidate beams int32 [B, W, L].

    mode "workload": each beam copies a prefix of the previous beam (length
    from the workload's share rule) and draws the rest uniformly from the
    vocabulary.  "distinct": first tokens pairwise distinct (no shared
    prefix anywhere).  "identical": every beam equals beam 0.
    """
    B, W, L, V = cfg.B, cfg.W, cfg.L, cfg.V
    out = np.zeros((B, W, L), dtype=np.int32)
    for b in range(B):
        rng = rng_for(seed, TAG_BEAMS, b)
        if mode == "distinct":
            if W > V:
                raise ValueError("distinct first tokens need W <= V")
            out[b, :, 0] = rng.choice(V, size=W, replace=False)
            out[b, :, 1:] = rng.integers(0, V, size=(W, L - 1))
            continue
        out[b, 0] = rng.integers(0, V, size=L)
        for w in range(1, W):
            if mode == "identical":
                out[b, w] = out[b, 0]
                continue
            s = _share_length(cfg, rng)
            out[b, w, :s] = out[b, w - 1, :s]
            out[b, w, s:] = rng.integers(0, V, size=L - s)
    return out


def _prefix_words(prefix) -> list:
    return [len(prefix), *(int(t) for t in prefix)]


def node_qkv(cfg: Config, seed: int, b: int, prefix):
    """(q [Hq,D], k [Hkv,D], v [Hkv,D]) of the token whose prefix is `prefix`."""
    rng = rng_for(seed, TAG_QKV, b, *_prefix_words(prefix))
    q = rng.standard_normal((cfg.Hq, cfg.D), dtype=np.float32)
    k = rng.standard_normal((cfg.Hkv, cfg.D), dtype=np.float32)
    v = rng.standard_normal((cfg.Hkv, cfg.D), dtype=np.float32)
    return _finish(cfg, q), _finish(cfg, k), _finish(cfg, v)


def node_hidden(cfg: Config, seed: int, b: int, prefix, retry: int = 0) -> np.ndarray:
    """Hidden state [hidden] fed to the output projection for `prefix`.

    `retry` > 0 gives an independent redraw (used to move a row away from an
    argmax near-tie)."""
    rng = rng_for(seed, TAG_HIDDEN, b, retry, *_prefix_words(prefix))
    return _finish(cfg, rng.standard_normal(cfg.hidden, dtype=np.float32))


def unpacked_node_tensors(cfg: Config, seed: int, beams: np.ndarray, requests=None,
                          hidden_retry=None, with_qkv: bool = True, with_hidden: bool = True):
    """Per-candidate tensors in unpacked layout for the listed requests.

    Returns a dict with q [R,W,L,Hq,D], k/v [R,W,L,Hkv,D], hidden [R,W,L,hidden]
    (R = len(requests)).  hidden_retry maps (b, prefix tuple) -> retry count.
    """
    requests = list(range(cfg.B)) if requests is None else list(requests)
    R, W, L = len(requests), cfg.W, cfg.L
    out = {}
    if with_qkv:
        out["q"] = np.zeros((R, W, L, cfg.Hq, cfg.D), np.float32)
        out["k"] = np.zeros((R, W, L, cfg.Hkv, cfg.D), np.float32)
        out["v"] = np.zeros((R, W, L, cfg.Hkv, cfg.D), np.float32)
    if with_hidden:
        out["hidden"] = np.zeros((R, W, L, cfg.hidden), np.float32)
    hidden_retry = hidden_retry or {}
    for i, b in enumerate(requests):
        seen_qkv, seen_h = {}, {}
        for w in range(W):
            for l in range(L):
                pre = tuple(int(t) for t in beams[b, w, :l + 1])
                if with_qkv:
                    if pre not in seen_qkv:
                        seen_qkv[pre] = node_qkv(cfg, seed, b, pre)
                    out["q"][i, w, l], out["k"][i, w, l], out["v"][i, w, l] = seen_qkv[pre]
                if with_hidden:
                    if pre not in seen_h:
                        seen_h[pre] = node_hidden(cfg, seed, b, pre, hidden_retry.get((b, pre), 0))
                    out["hidden"][i, w, l] = seen_h[pre]
    return out


def kv_cache(cfg: Config, seed: int, b: int):
    """(k_cache [Hkv,S,D], v_cache [Hkv,S,D]) of request b."""
    k = rng_for(seed, TAG_KCACHE, b).standard_normal((cfg.Hkv, cfg.S, cfg.D), dtype=np.float32)
    v = rng_for(seed, TAG_VCACHE, b).standard_normal((cfg.Hkv, cfg.S, cfg.D), dtype=np.float32)
    return _finish(cfg, k), _finish(cfg, v)


def lm_weight(cfg: Config, seed: int) -> np.ndarray:
    """Output projection [V, hidden] (nn.Linear layout), N(0, 0.02^2)."""
    w = rng_for(seed, TAG_WEIGHT).standard_normal((cfg.V, cfg.hidden), dtype=np.float32)
    return _finish(cfg, w * np.float32(0.02))


def kv_lengths(cfg: Config) -> np.ndarray:
    """Cached tokens per request: the full cache in every workload."""
    return np.full(cfg.B, cfg.S, dtype=np.int32)
