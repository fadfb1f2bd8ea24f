"""Python binding of librd, the gfx950 library behind include/rd.h.

Argument marshalling only: every function checks tensor dtypes, shapes,
devices and contiguity, allocates outputs with torch when the caller gives
none, and passes raw device pointers plus torch's current HIP stream to the
C entry point of the same name.  Every step runs in the library's kernels;
there is no fallback: if librd.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RD_OK", "RD_F32", "RD_BF16", "RdError", "lib_path", "load_library", "EXPORTED_SYMBOLS",
    "rd_pack_beams", "rd_tree_mask", "rd_pack_beams_mask", "rd_pack_beams_mask_ragged", "rd_tree_attention",
    "rd_tree_attention_paged", "rd_unpack_accept_ragged", "rd_tree_attention_workspace_size",
    "rd_lm_head_argmax", "rd_lm_head_workspace_size", "rd_unpack_accept", "rd_commit_accepted", "rd_commit_accepted_paged", "rd_stochastic_accept",
    "rd_stochastic_accept_workspace_size", "verify_step", "rd_set_knob", "rd_set_debug", "rd_lm_head_argmax_noalloc",
    "rd_lm_head_argmax_unpack", "rd_lm_head_argmax_unpack_workspace_size", "fuse_unpack_pays",
    "RD_KNOB_ATTN_SPLITS", "RD_KNOB_ATTN_FEWROW", "RD_KNOB_LM_SHAPE",
    "VerifyBuffers",
]

RD_OK, RD_E_ARG, RD_E_UNSUPPORTED, RD_E_WORKSPACE, RD_E_HIP, RD_E_CONTENT, RD_E_SCRATCH = 0, -1, -2, -3, -4, -5, -6
RD_NOALLOC_SCRATCH_BYTES = 32 << 20
RD_KNOB_ATTN_SPLITS, RD_KNOB_ATTN_FEWROW, RD_KNOB_LM_SHAPE = 1, 2, 3
RD_F32, RD_BF16 = 0, 1
MAX_BEAMS, MAX_BEAM_LEN = 64, 16

EXPORTED_SYMBOLS = (
    "rd_status_string", "rd_version", "rd_pack_beams", "rd_tree_mask", "rd_pack_beams_mask",
    "rd_pack_beams_mask_ragged", "rd_unpack_accept_ragged",
    "rd_tree_attention_workspace_size", "rd_tree_attention", "rd_tree_attention_paged", "rd_lm_head_workspace_size",
    "rd_lm_head_argmax", "rd_unpack_accept", "rd_commit_accepted", "rd_commit_accepted_paged",
    "rd_stochastic_accept_workspace_size", "rd_stochastic_accept", "rd_set_knob", "rd_set_debug",
    "rd_lm_head_argmax_noalloc", "rd_lm_head_argmax_unpack_workspace_size", "rd_lm_head_argmax_unpack",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class RdError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load_library().rd_status_string(code).decode()
        super().__init__(f"{where}: {msg} (status {code})")
        self.code = code


def lib_path() -> str:
    return os.path.join(_HERE, "librd.so")


def load_library():
    """Load librd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with tree_attention_verification_rd_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sigs = {
        "rd_status_string": ([i32], ctypes.c_char_p),
        "rd_version": ([], i32),
        "rd_set_knob": ([i32, i32], i32),
        "rd_set_debug": ([i32], i32),
        "rd_pack_beams": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "rd_tree_mask": ([vp, vp, i32, i32, i32, vp, vp], i32),
        "rd_pack_beams_mask": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "rd_pack_beams_mask_ragged": ([vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "rd_unpack_accept_ragged": ([vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp], i32),
        "rd_tree_attention_workspace_size": ([i32, i32, i32, i32, i32, i32, i32], sz),
        "rd_tree_attention": ([i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                               vp, vp, sz, vp], i32),
        "rd_tree_attention_paged": ([i32, vp, vp, vp, vp, vp, i64, i32, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                     f32, vp, vp, sz, vp], i32),
        "rd_lm_head_workspace_size": ([i32, i32, i32, i32, i32], sz),
        "rd_lm_head_argmax": ([i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp], i32),
        "rd_lm_head_argmax_noalloc": ([i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp], i32),
        "rd_lm_head_argmax_unpack_workspace_size": ([i32, i32, i32, i32, i32, i32], sz),
        "rd_lm_head_argmax_unpack": ([i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp], i32),
        "rd_unpack_accept": ([vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp], i32),
        "rd_commit_accepted": ([i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                vp], i32),
        "rd_stochastic_accept_workspace_size": ([i32, i32, i32], sz),
        "rd_stochastic_accept": ([i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp], i32),
        "rd_commit_accepted_paged": ([i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i64, i32,
                                      vp, i32, vp, vp, vp], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


# ------------------------------------------------------------------ helpers
def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(code: int, where: str):
    if code != RD_OK:
        raise RdError(code, where)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RD_F32
    if t.dtype == torch.bfloat16:
        return RD_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _out(t, name, shape, dtype, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, name, dtype, shape, device)


# -------------------------------------------------------------- entry points
def rd_set_knob(knob: int, value: int) -> int:
    """Force a tuning choice (RD_KNOB_*; 0 = automatic).  Returns the previous value."""
    code = load_library().rd_set_knob(int(knob), int(value))
    _check(min(code, 0), "rd_set_knob")
    return code


def rd_set_debug(on: bool) -> bool:
    """Switch the library's debug-mode content checks on or off.  Returns the previous setting."""
    return bool(load_library().rd_set_debug(1 if on else 0))


def rd_pack_beams(beams: torch.Tensor, *, packed_tokens=None, packed_len=None, unpacker=None,
                  packed_depth=None, packed_src=None, with_depth_src: bool = True) -> dict:
    """Step 1: pack beams [B,W,L] int32 into the deduplicated token tree."""
    lib = load_library()
    _need(beams, "beams", torch.int32)
    if beams.dim() != 3:
        raise ValueError("beams must be [B, W, L]")
    B, W, L = beams.shape
    dev = beams.device
    P = W * L
    out = {
        "tokens": _out(packed_tokens, "packed_tokens", (B, P), torch.int32, dev),
        "length": _out(packed_len, "packed_len", (B,), torch.int32, dev),
        "unpacker": _out(unpacker, "unpacker", (B, W, L), torch.int32, dev),
        "depth": _out(packed_depth, "packed_depth", (B, P), torch.int32, dev) if with_depth_src else None,
        "src": _out(packed_src, "packed_src", (B, P), torch.int32, dev) if with_depth_src else None,
    }
    _check(lib.rd_pack_beams(_p(beams), B, W, L, _p(out["tokens"]), _p(out["length"]), _p(out["unpacker"]),
                             _p(out["depth"]), _p(out["src"]), _stream(beams)), "rd_pack_beams")
    return out


def rd_tree_mask(unpacker: torch.Tensor, packed_len: torch.Tensor, *, mask=None) -> torch.Tensor:
    """Step 1b: bit-packed tree-causal mask uint32 words, returned as int32 [B,P,ceil(P/32)]."""
    lib = load_library()
    _need(unpacker, "unpacker", torch.int32)
    B, W, L = unpacker.shape
    _need(packed_len, "packed_len", torch.int32, (B,), unpacker.device)
    P = W * L
    mask = _out(mask, "mask", (B, P, (P + 31) // 32), torch.int32, unpacker.device)
    _check(lib.rd_tree_mask(_p(unpacker), _p(packed_len), B, W, L, _p(mask), _stream(unpacker)), "rd_tree_mask")
    return mask


def rd_pack_beams_mask(beams: torch.Tensor, *, packed_tokens=None, packed_len=None, unpacker=None,
                       packed_depth=None, packed_src=None, mask=None, with_depth_src: bool = True,
                       beam_width=None, beam_len=None):
    """Steps 1 + 1b in one launch: returns (pack dict as rd_pack_beams, mask as rd_tree_mask).

    With beam_width and beam_len (int32 [B]) the batch is ragged (rd_pack_beams_mask_ragged).
    """
    lib = load_library()
    _need(beams, "beams", torch.int32)
    if beams.dim() != 3:
        raise ValueError("beams must be [B, W, L]")
    B, W, L = beams.shape
    dev = beams.device
    ragged = beam_width is not None or beam_len is not None
    if ragged:
        if beam_width is None or beam_len is None:
            raise ValueError("give both beam_width and beam_len")
        _need(beam_width, "beam_width", torch.int32, (B,), dev)
        _need(beam_len, "beam_len", torch.int32, (B,), dev)
    P = W * L
    out = {
        "tokens": _out(packed_tokens, "packed_tokens", (B, P), torch.int32, dev),
        "length": _out(packed_len, "packed_len", (B,), torch.int32, dev),
        "unpacker": _out(unpacker, "unpacker", (B, W, L), torch.int32, dev),
        "depth": _out(packed_depth, "packed_depth", (B, P), torch.int32, dev) if with_depth_src else None,
        "src": _out(packed_src, "packed_src", (B, P), torch.int32, dev) if with_depth_src else None,
    }
    mask = _out(mask, "mask", (B, P, (P + 31) // 32), torch.int32, dev)
    if ragged:
        _check(lib.rd_pack_beams_mask_ragged(_p(beams), _p(beam_width), _p(beam_len), B, W, L, _p(out["tokens"]),
                                             _p(out["length"]), _p(out["unpacker"]), _p(out["depth"]),
                                             _p(out["src"]), _p(mask), _stream(beams)), "rd_pack_beams_mask_ragged")
    else:
        _check(lib.rd_pack_beams_mask(_p(beams), B, W, L, _p(out["tokens"]), _p(out["length"]), _p(out["unpacker"]),
                                      _p(out["depth"]), _p(out["src"]), _p(mask), _stream(beams)),
               "rd_pack_beams_mask")
    return out, mask


def rd_pack_beams_mask_ragged(beams, beam_width, beam_len, **kw):
    """Steps 1 + 1b for a ragged batch (see rd_pack_beams_mask)."""
    return rd_pack_beams_mask(beams, beam_width=beam_width, beam_len=beam_len, **kw)


def rd_tree_attention_workspace_size(dtype_code: int, B, P_max, Hq, Hkv, D, S_max) -> int:
    return int(load_library().rd_tree_attention_workspace_size(dtype_code, B, P_max, Hq, Hkv, D, S_max))


def rd_tree_attention(q, k_new, v_new, k_cache, v_cache, kv_len, mask, packed_len, *, scale: float = 0.0,
                      out=None, workspace=None) -> torch.Tensor:
    """Step 2: tree attention; returns out [B,P_max,Hq,D] in q's dtype."""
    lib = load_library()
    dt = _dtype_code(q)
    _need(q, "q", q.dtype)
    B, P, Hq, D = q.shape
    dev = q.device
    Hkv = k_new.shape[2]
    S = k_cache.shape[2]
    _need(k_new, "k_new", q.dtype, (B, P, Hkv, D), dev)
    _need(v_new, "v_new", q.dtype, (B, P, Hkv, D), dev)
    _need(k_cache, "k_cache", q.dtype, (B, Hkv, S, D), dev)
    _need(v_cache, "v_cache", q.dtype, (B, Hkv, S, D), dev)
    _need(kv_len, "kv_len", torch.int32, (B,), dev)
    _need(mask, "mask", torch.int32, (B, P, (P + 31) // 32), dev)
    _need(packed_len, "packed_len", torch.int32, (B,), dev)
    out = _out(out, "out", (B, P, Hq, D), q.dtype, dev)
    need = rd_tree_attention_workspace_size(dt, B, P, Hq, Hkv, D, S)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.rd_tree_attention(dt, _p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(kv_len), _p(mask),
                                 _p(packed_len), B, P, Hq, Hkv, D, S, float(scale), _p(out), _p(workspace),
                                 workspace.numel(), _stream(q)), "rd_tree_attention")
    return out


def rd_tree_attention_paged(q, k_new, v_new, k_pages, v_pages, block_table, kv_len, mask, packed_len, *,
                            scale: float = 0.0, out=None, workspace=None) -> torch.Tensor:
    """Step 2 over a paged cache: pools [num_pages, Hkv, page_size, D], block_table [B, max_pages] int32."""
    lib = load_library()
    dt = _dtype_code(q)
    _need(q, "q", q.dtype)
    B, P, Hq, D = q.shape
    dev = q.device
    Hkv = k_new.shape[2]
    _need(k_new, "k_new", q.dtype, (B, P, Hkv, D), dev)
    _need(v_new, "v_new", q.dtype, (B, P, Hkv, D), dev)
    _need(k_pages, "k_pages", q.dtype, None, dev)
    if k_pages.dim() != 4 or k_pages.shape[1] != Hkv or k_pages.shape[3] != D:
        raise ValueError("k_pages must be [num_pages, Hkv, page_size, D]")
    num_pages, page_size = k_pages.shape[0], k_pages.shape[2]
    _need(v_pages, "v_pages", q.dtype, tuple(k_pages.shape), dev)
    _need(block_table, "block_table", torch.int32, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    max_pages = block_table.shape[1]
    _need(kv_len, "kv_len", torch.int32, (B,), dev)
    _need(mask, "mask", torch.int32, (B, P, (P + 31) // 32), dev)
    _need(packed_len, "packed_len", torch.int32, (B,), dev)
    out = _out(out, "out", (B, P, Hq, D), q.dtype, dev)
    need = rd_tree_attention_workspace_size(dt, B, P, Hq, Hkv, D, max_pages * page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.rd_tree_attention_paged(dt, _p(q), _p(k_new), _p(v_new), _p(k_pages), _p(v_pages), num_pages,
                                       page_size, _p(block_table), max_pages, _p(kv_len), _p(mask), _p(packed_len),
                                       B, P, Hq, Hkv, D, float(scale), _p(out), _p(workspace), workspace.numel(),
                                       _stream(q)), "rd_tree_attention_paged")
    return out


def rd_lm_head_workspace_size(dtype_code: int, B, P_max, K, V) -> int:
    return int(load_library().rd_lm_head_workspace_size(dtype_code, B, P_max, K, V))


def rd_lm_head_argmax(hidden, packed_len, weight, *, want_logits: bool = True, logits=None, argmax=None,
                      workspace=None):
    """Step 3: projection + greedy target.  Returns (logits [B,P,V] or None, argmax [B,P])."""
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", hidden.dtype)
    B, P, K = hidden.shape
    dev = hidden.device
    V = weight.shape[0]
    _need(weight, "weight", hidden.dtype, (V, K), dev)
    if packed_len is not None:
        _need(packed_len, "packed_len", torch.int32, (B,), dev)
    if want_logits:
        logits = _out(logits, "logits", (B, P, V), hidden.dtype, dev)
    else:
        logits = None
    argmax = _out(argmax, "argmax", (B, P), torch.int32, dev)
    need = rd_lm_head_workspace_size(dt, B, P, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.rd_lm_head_argmax(dt, _p(hidden), _p(packed_len), _p(weight), B, P, K, V, _p(logits), _p(argmax),
                                 _p(workspace), workspace.numel(), _stream(hidden)), "rd_lm_head_argmax")
    return logits, argmax


FUSE_UNPACK_MIN_BYTES = 64 << 20


def fuse_unpack_pays(B: int, W: int, L: int, V: int, elem_bytes: int) -> bool:
    """Whether to fold the logits gather into the projection (rd_lm_head_argmax_unpack).

    The folded gather saves writing and re-reading the packed logits but adds two small launches (the
    first-candidate table and the duplicate-row copy), a few microseconds: it pays once the unpacked logits
    reach tens of MB (measured on MI355X: 7% of the step at 2.1 GB, 5% slower at 20 MB)."""
    return B * W * L * V * elem_bytes >= FUSE_UNPACK_MIN_BYTES


def rd_lm_head_argmax_unpack_workspace_size(dtype_code: int, B: int, W: int, L: int, K: int, V: int) -> int:
    return load_library().rd_lm_head_argmax_unpack_workspace_size(dtype_code, B, W, L, K, V)


def rd_lm_head_argmax_unpack(hidden, packed_len, weight, unpacker, *, unpacked=None, argmax=None, workspace=None):
    """Steps 3 + 3b in one pass: projection and greedy target, with the logits written unpacked.

    Returns (unpacked [B,W,L,V], argmax [B,W*L]); the values equal rd_lm_head_argmax followed by the gather of
    rd_unpack_accept.  Run rd_unpack_accept with packed=None afterwards for the accept."""
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", hidden.dtype)
    B, P, K = hidden.shape
    dev = hidden.device
    _need(unpacker, "unpacker", torch.int32, None, dev)
    if unpacker.dim() != 3 or unpacker.shape[0] != B or unpacker.shape[1] * unpacker.shape[2] != P:
        raise ValueError("unpacker must be [B, W, L] with W*L equal to hidden's packed width")
    W, L = unpacker.shape[1], unpacker.shape[2]
    V = weight.shape[0]
    _need(weight, "weight", hidden.dtype, (V, K), dev)
    if packed_len is not None:
        _need(packed_len, "packed_len", torch.int32, (B,), dev)
    unpacked = _out(unpacked, "unpacked", (B, W, L, V), hidden.dtype, dev)
    argmax = _out(argmax, "argmax", (B, P), torch.int32, dev)
    need = rd_lm_head_argmax_unpack_workspace_size(dt, B, W, L, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.rd_lm_head_argmax_unpack(dt, _p(hidden), _p(packed_len), _p(weight), _p(unpacker), B, W, L, K, V,
                                        _p(unpacked), _p(argmax), _p(workspace), workspace.numel(), _stream(hidden)),
           "rd_lm_head_argmax_unpack")
    return unpacked, argmax


def rd_lm_head_argmax_noalloc(hidden, packed_len, weight, *, logits, argmax):
    """rd_lm_head_argmax without a workspace: the library's fixed device scratch holds the argmax
    partials.  The caller supplies every output (logits may be None); nothing is allocated here or in
    the library.  Raises RdError(RD_E_SCRATCH) when the sizes need more than RD_NOALLOC_SCRATCH_BYTES."""
    lib = load_library()
    dt = _dtype_code(hidden)
    _need(hidden, "hidden", hidden.dtype)
    B, P, K = hidden.shape
    dev = hidden.device
    V = weight.shape[0]
    _need(weight, "weight", hidden.dtype, (V, K), dev)
    if packed_len is not None:
        _need(packed_len, "packed_len", torch.int32, (B,), dev)
    if logits is not None:
        _need(logits, "logits", hidden.dtype, (B, P, V), dev)
    _need(argmax, "argmax", torch.int32, (B, P), dev)
    _check(lib.rd_lm_head_argmax_noalloc(dt, _p(hidden), _p(packed_len), _p(weight), B, P, K, V, _p(logits),
                                         _p(argmax), _stream(hidden)), "rd_lm_head_argmax_noalloc")
    return logits, argmax


def rd_unpack_accept(beams, unpacker, packed_argmax, packed=None, *, unpacked=None, match_len=None,
                     best_beam=None, accept_len=None, accepted_tokens=None, beam_width=None, beam_len=None) -> dict:
    """Steps 3b + 4: optional gather of packed rows to [B,W,L,X] and greedy accept.

    With beam_width and beam_len (int32 [B]) the batch is ragged (rd_unpack_accept_ragged).
    """
    lib = load_library()
    _need(beams, "beams", torch.int32)
    B, W, L = beams.shape
    dev = beams.device
    ragged = beam_width is not None or beam_len is not None
    if ragged:
        if beam_width is None or beam_len is None:
            raise ValueError("give both beam_width and beam_len")
        _need(beam_width, "beam_width", torch.int32, (B,), dev)
        _need(beam_len, "beam_len", torch.int32, (B,), dev)
    _need(unpacker, "unpacker", torch.int32, (B, W, L), dev)
    _need(packed_argmax, "packed_argmax", torch.int32, (B, W * L), dev)
    dt, row_len = RD_BF16, 0
    if packed is not None:
        dt = _dtype_code(packed)
        _need(packed, "packed", packed.dtype, None, dev)
        if packed.dim() != 3 or packed.shape[0] != B or packed.shape[1] != W * L:
            raise ValueError("packed must be [B, W*L, X]")
        row_len = packed.shape[2]
        unpacked = _out(unpacked, "unpacked", (B, W, L, row_len), packed.dtype, dev)
    else:
        unpacked = None
    res = {
        "unpacked": unpacked,
        "match_len": _out(match_len, "match_len", (B, W), torch.int32, dev),
        "best_beam": _out(best_beam, "best_beam", (B,), torch.int32, dev),
        "accept_len": _out(accept_len, "accept_len", (B,), torch.int32, dev),
        "accepted_tokens": _out(accepted_tokens, "accepted_tokens", (B, L), torch.int32, dev),
    }
    if ragged:
        _check(lib.rd_unpack_accept_ragged(_p(beams), _p(beam_width), _p(beam_len), _p(unpacker), _p(packed_argmax),
                                           _p(packed), _p(unpacked), dt, row_len, B, W, L, _p(res["match_len"]),
                                           _p(res["best_beam"]), _p(res["accept_len"]), _p(res["accepted_tokens"]),
                                           _stream(beams)), "rd_unpack_accept_ragged")
    else:
        _check(lib.rd_unpack_accept(_p(beams), _p(unpacker), _p(packed_argmax), _p(packed), _p(unpacked), dt,
                                    row_len, B, W, L, _p(res["match_len"]), _p(res["best_beam"]),
                                    _p(res["accept_len"]), _p(res["accepted_tokens"]), _stream(beams)),
               "rd_unpack_accept")
    return res


def rd_unpack_accept_ragged(beams, beam_width, beam_len, unpacker, packed_argmax, packed=None, **kw) -> dict:
    """Steps 3b + 4 for a ragged batch (see rd_unpack_accept)."""
    return rd_unpack_accept(beams, unpacker, packed_argmax, packed, beam_width=beam_width, beam_len=beam_len, **kw)


def rd_commit_accepted(unpacker, best_beam, accept_len, k_new, v_new, k_cache, v_cache, kv_len, hidden=None, *,
                       hidden_next=None):
    """After step 4: append the accepted path's keys/values to the cache and advance kv_len, in place.

    k_new/v_new are packed [B, W*L, Hkv, D]; k_cache/v_cache [B, Hkv, S, D]; hidden (optional) [B, W*L, K].
    Returns hidden_next [B, K] (the drafter's hidden state) or None when hidden is None.  Requests
    that would overflow the cache are left unchanged (their kv_len does not move).
    """
    lib = load_library()
    _need(unpacker, "unpacker", torch.int32)
    B, W, L = unpacker.shape
    dev = unpacker.device
    dt = _dtype_code(k_new)
    _need(k_new, "k_new", k_new.dtype, None, dev)
    if k_new.dim() != 4 or k_new.shape[0] != B or k_new.shape[1] != W * L:
        raise ValueError("k_new must be [B, W*L, Hkv, D]")
    Hkv, D = k_new.shape[2], k_new.shape[3]
    _need(v_new, "v_new", k_new.dtype, (B, W * L, Hkv, D), dev)
    _need(k_cache, "k_cache", k_new.dtype, None, dev)
    if k_cache.dim() != 4 or tuple(k_cache.shape[:2]) != (B, Hkv) or k_cache.shape[3] != D:
        raise ValueError("k_cache must be [B, Hkv, S, D]")
    S = k_cache.shape[2]
    _need(v_cache, "v_cache", k_new.dtype, (B, Hkv, S, D), dev)
    for t, name in ((best_beam, "best_beam"), (accept_len, "accept_len"), (kv_len, "kv_len")):
        _need(t, name, torch.int32, (B,), dev)
    K = 0
    if hidden is not None:
        _need(hidden, "hidden", k_new.dtype, None, dev)
        if hidden.dim() != 3 or tuple(hidden.shape[:2]) != (B, W * L):
            raise ValueError("hidden must be [B, W*L, K]")
        K = hidden.shape[2]
        hidden_next = _out(hidden_next, "hidden_next", (B, K), k_new.dtype, dev)
    else:
        hidden_next = None
    _check(lib.rd_commit_accepted(dt, _p(unpacker), _p(best_beam), _p(accept_len), _p(k_new), _p(v_new), _p(hidden),
                                  B, W, L, Hkv, D, K, S, _p(k_cache), _p(v_cache), _p(kv_len), _p(hidden_next),
                                  _stream(unpacker)), "rd_commit_accepted")
    return hidden_next


def rd_commit_accepted_paged(unpacker, best_beam, accept_len, k_new, v_new, k_pages, v_pages, block_table, kv_len,
                             hidden=None, *, hidden_next=None):
    """rd_commit_accepted into paged pools [num_pages, Hkv, page_size, D] through block_table [B, max_pages]."""
    lib = load_library()
    _need(unpacker, "unpacker", torch.int32)
    B, W, L = unpacker.shape
    dev = unpacker.device
    dt = _dtype_code(k_new)
    _need(k_new, "k_new", k_new.dtype, None, dev)
    if k_new.dim() != 4 or k_new.shape[0] != B or k_new.shape[1] != W * L:
        raise ValueError("k_new must be [B, W*L, Hkv, D]")
    Hkv, D = k_new.shape[2], k_new.shape[3]
    _need(v_new, "v_new", k_new.dtype, (B, W * L, Hkv, D), dev)
    _need(k_pages, "k_pages", k_new.dtype, None, dev)
    if k_pages.dim() != 4 or k_pages.shape[1] != Hkv or k_pages.shape[3] != D:
        raise ValueError("k_pages must be [num_pages, Hkv, page_size, D]")
    _need(v_pages, "v_pages", k_new.dtype, tuple(k_pages.shape), dev)
    _need(block_table, "block_table", torch.int32, None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    for t, name in ((best_beam, "best_beam"), (accept_len, "accept_len"), (kv_len, "kv_len")):
        _need(t, name, torch.int32, (B,), dev)
    K = 0
    if hidden is not None:
        _need(hidden, "hidden", k_new.dtype, None, dev)
        if hidden.dim() != 3 or tuple(hidden.shape[:2]) != (B, W * L):
            raise ValueError("hidden must be [B, W*L, K]")
        K = hidden.shape[2]
        hidden_next = _out(hidden_next, "hidden_next", (B, K), k_new.dtype, dev)
    else:
        hidden_next = None
    _check(lib.rd_commit_accepted_paged(dt, _p(unpacker), _p(best_beam), _p(accept_len), _p(k_new), _p(v_new),
                                        _p(hidden), B, W, L, Hkv, D, K, _p(k_pages), _p(v_pages), k_pages.shape[0],
                                        k_pages.shape[2], _p(block_table), block_table.shape[1], _p(kv_len),
                                        _p(hidden_next), _stream(unpacker)), "rd_commit_accepted_paged")
    return hidden_next


def rd_stochastic_accept_workspace_size(B, W, L) -> int:
    return int(load_library().rd_stochastic_accept_workspace_size(B, W, L))


def rd_stochastic_accept(unpacker, packed_len, packed_tokens, logits, q, u_accept, u_bonus, *, best_beam=None,
                         accept_len=None, accepted_tokens=None, path=None, workspace=None) -> dict:
    """Stochastic step 4 (multi-step speculative sampling over the tree); see include/rd.h."""
    lib = load_library()
    _need(unpacker, "unpacker", torch.int32)
    B, W, L = unpacker.shape
    dev = unpacker.device
    P = W * L
    dt = _dtype_code(logits)
    _need(logits, "logits", logits.dtype, None, dev)
    if logits.dim() != 3 or tuple(logits.shape[:2]) != (B, P):
        raise ValueError("logits must be [B, W*L, V]")
    V = logits.shape[2]
    _need(packed_len, "packed_len", torch.int32, (B,), dev)
    _need(packed_tokens, "packed_tokens", torch.int32, (B, P), dev)
    _need(q, "q", torch.float32, (B, P, V), dev)
    _need(u_accept, "u_accept", torch.float32, (B, L, W), dev)
    _need(u_bonus, "u_bonus", torch.float32, (B,), dev)
    res = {
        "best_beam": _out(best_beam, "best_beam", (B,), torch.int32, dev),
        "accept_len": _out(accept_len, "accept_len", (B,), torch.int32, dev),
        "accepted_tokens": _out(accepted_tokens, "accepted_tokens", (B, L), torch.int32, dev),
        "path": _out(path, "path", (B, L), torch.int32, dev),
    }
    need = rd_stochastic_accept_workspace_size(B, W, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.rd_stochastic_accept(dt, _p(unpacker), _p(packed_len), _p(packed_tokens), _p(logits), _p(q),
                                    _p(u_accept), _p(u_bonus), B, W, L, V, _p(res["best_beam"]),
                                    _p(res["accept_len"]), _p(res["accepted_tokens"]), _p(res["path"]),
                                    _p(workspace), workspace.numel(), _stream(unpacker)), "rd_stochastic_accept")
    return res


class VerifyBuffers:
    """Preallocated outputs and workspaces for repeated verify_step calls of one shape."""

    def __init__(self, B, W, L, Hq, Hkv, D, S, K, V, dtype, device, want_logits=True):
        P = W * L
        i32 = torch.int32
        dt = RD_F32 if dtype == torch.float32 else RD_BF16
        e = lambda shape, d=i32: torch.empty(shape, dtype=d, device=device)  # noqa: E731
        self.pack = {"tokens": e((B, P)), "length": e((B,)), "unpacker": e((B, W, L)), "depth": e((B, P)),
                     "src": e((B, P))}
        self.mask = e((B, P, (P + 31) // 32))
        self.attn = e((B, P, Hq, D), dtype)
        self.attn_ws = e((max(rd_tree_attention_workspace_size(dt, B, P, Hq, Hkv, D, S), 1),), torch.uint8)
        self.logits = e((B, P, V), dtype) if want_logits else None
        self.argmax = e((B, P))
        self.lm_ws = e((max(rd_lm_head_workspace_size(dt, B, P, K, V),
                            rd_lm_head_argmax_unpack_workspace_size(dt, B, W, L, K, V), 1),), torch.uint8)
        self.unpacked = e((B, W, L, V), dtype) if want_logits else None
        self.accept = {"match_len": e((B, W)), "best_beam": e((B,)), "accept_len": e((B,)),
                       "accepted_tokens": e((B, L))}


def verify_step(beams, q, k_new, v_new, k_cache, v_cache, kv_len, hidden, weight, *, want_logits=True,
                buffers: VerifyBuffers | None = None, scale: float = 0.0, beam_width=None, beam_len=None,
                fuse_unpack: bool | None = None) -> dict:
    """One verification step: pack+mask, attention, projection, unpack+accept, enqueued in order on the current stream.

    q/k_new/v_new/hidden are in packed layout [B, W*L, ...] (rows past the packed length are ignored).
    With fuse_unpack (and want_logits) the projection writes the logits unpacked (rd_lm_head_argmax_unpack):
    "unpacked" holds them and "logits" is None; None chooses by size (fuse_unpack_pays).
    """
    B, W, L = beams.shape
    bufs = buffers
    pk, mask = rd_pack_beams_mask(beams, **({} if bufs is None else {
        "packed_tokens": bufs.pack["tokens"], "packed_len": bufs.pack["length"], "unpacker": bufs.pack["unpacker"],
        "packed_depth": bufs.pack["depth"], "packed_src": bufs.pack["src"], "mask": bufs.mask}),
        beam_width=beam_width, beam_len=beam_len)
    attn = rd_tree_attention(q, k_new, v_new, k_cache, v_cache, kv_len, mask, pk["length"], scale=scale,
                             out=None if bufs is None else bufs.attn,
                             workspace=None if bufs is None else bufs.attn_ws)
    if fuse_unpack is None:
        fuse_unpack = fuse_unpack_pays(B, W, L, weight.shape[0], hidden.element_size())
    if fuse_unpack and want_logits:
        unpacked, argmax = rd_lm_head_argmax_unpack(hidden, pk["length"], weight, pk["unpacker"],
                                                    unpacked=None if bufs is None else bufs.unpacked,
                                                    argmax=None if bufs is None else bufs.argmax,
                                                    workspace=None if bufs is None else bufs.lm_ws)
        acc = rd_unpack_accept(beams, pk["unpacker"], argmax, None, **({} if bufs is None else bufs.accept),
                               beam_width=beam_width, beam_len=beam_len)
        acc["unpacked"] = unpacked
        return {"pack": pk, "mask": mask, "attn": attn, "logits": None, "argmax": argmax, **acc}
    logits, argmax = rd_lm_head_argmax(hidden, pk["length"], weight, want_logits=want_logits,
                                       logits=None if bufs is None else bufs.logits,
                                       argmax=None if bufs is None else bufs.argmax,
                                       workspace=None if bufs is None else bufs.lm_ws)
    acc = rd_unpack_accept(beams, pk["unpacker"], argmax, logits,
                           **({} if bufs is None else {"unpacked": bufs.unpacked, **bufs.accept}),
                           beam_width=beam_width, beam_len=beam_len)
    return {"pack": pk, "mask": mask, "attn": attn, "logits": logits, "argmax": argmax, **acc}
