"""Thin ctypes binding to libh3attn.so (argument marshalling only).

Every function here has the name of the C entry point it calls
(``include/h3attn.h``).  Tensor arguments are torch tensors on the GPU; their
device pointers and the current HIP stream are passed straight through.  No
step of the computation runs in Python: a missing library raises, it never
falls back to anything else.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh3attn.so")
_lib = None

H3ATTN_OK = 0
H3ATTN_ERR_INVALID_ARG = 1
H3ATTN_ERR_UNSUPPORTED = 2
H3ATTN_ERR_WORKSPACE = 3
H3ATTN_ERR_HIP = 4

ITEM_VISUAL = 0
ITEM_AUDIO = 1
ITEM_CLOCK = 2
ITEM_TEXT = 3
AUDIO_LINEAR = 0
AUDIO_ROUND_HALF_EVEN = 1

DEFAULT_THETA = 10000.0
DEFAULT_DIMS = (32, 48, 48)


class RopeCfg(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("dim_t", ctypes.c_int32), ("dim_h", ctypes.c_int32),
                ("dim_w", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Item(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("n_audio", ctypes.c_int32), ("attached", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("span", ctypes.c_double)]


class H3AttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {h3attn_status_string(status)}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libh3attn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m joint_sequence_attention_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    c_i32, c_i64, c_sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    rp = ctypes.POINTER(RopeCfg)
    L.h3attn_status_string.restype = ctypes.c_char_p
    L.h3attn_status_string.argtypes = [ctypes.c_int]
    L.h3attn_last_error.restype = ctypes.c_char_p
    L.h3attn_last_error.argtypes = []
    L.h3attn_abi_version.restype = c_i32
    L.h3attn_abi_version.argtypes = []
    L.h3attn_build_layout.restype = ctypes.c_int
    L.h3attn_build_layout.argtypes = [ctypes.POINTER(Item), ctypes.POINTER(c_i32), c_i32, ctypes.POINTER(c_i32),
                                      ctypes.POINTER(ctypes.c_float), c_i64, ctypes.POINTER(c_i64)]
    L.h3attn_rope_apply.restype = ctypes.c_int
    L.h3attn_rope_apply.argtypes = [vp, vp, vp, c_i64, c_i32, c_i32, rp, vp]
    L.h3attn_varlen_fwd_workspace_size.restype = c_sz
    L.h3attn_varlen_fwd_workspace_size.argtypes = [c_i64, c_i32, c_i32, c_i32]
    L.h3attn_varlen_fwd.restype = ctypes.c_int
    L.h3attn_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.c_float, rp,
                                    vp, c_sz, vp]
    L.h3attn_varlen_kv_prologue.restype = ctypes.c_int
    L.h3attn_varlen_kv_prologue.argtypes = [vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32, rp, vp, c_sz, vp]
    L.h3attn_varlen_attention.restype = ctypes.c_int
    L.h3attn_varlen_attention.argtypes = [vp, vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.c_float, rp,
                                          vp, c_sz, vp]
    L.h3attn_varlen_fwd_fp8_workspace_size.restype = c_sz
    L.h3attn_varlen_fwd_fp8_workspace_size.argtypes = [c_i64, c_i32, c_i32, c_i32]
    L.h3attn_varlen_fwd_fp8.restype = ctypes.c_int
    L.h3attn_varlen_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.c_float,
                                        ctypes.c_float, rp, vp, c_sz, vp, vp]
    L.h3attn_varlen_kv_prologue_fp8.restype = ctypes.c_int
    L.h3attn_varlen_kv_prologue_fp8.argtypes = list(L.h3attn_varlen_kv_prologue.argtypes)
    L.h3attn_varlen_attention_fp8.restype = ctypes.c_int
    L.h3attn_varlen_attention_fp8.argtypes = [vp, vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.c_float,
                                              ctypes.c_float, rp, vp, c_sz, vp, vp]
    L.h3attn_varlen_fwd_noalloc.restype = ctypes.c_int
    L.h3attn_varlen_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, c_i64, c_i32, c_i32, c_i32, c_i32,
                                            ctypes.c_float, rp, vp]
    L.h3attn_skip_gate.restype = ctypes.c_int
    L.h3attn_skip_gate.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_float)]
    _lib = L
    return L


# Every symbol include/h3attn.h declares.
EXPORTED = (
    "h3attn_build_layout",
    "h3attn_rope_apply",
    "h3attn_varlen_fwd_workspace_size",
    "h3attn_varlen_fwd",
    "h3attn_varlen_kv_prologue",
    "h3attn_varlen_attention",
    "h3attn_varlen_fwd_noalloc",
    "h3attn_varlen_fwd_fp8_workspace_size",
    "h3attn_varlen_fwd_fp8",
    "h3attn_varlen_kv_prologue_fp8",
    "h3attn_varlen_attention_fp8",
    "h3attn_skip_gate",
    "h3attn_status_string",
    "h3attn_last_error",
    "h3attn_abi_version",
)


def h3attn_status_string(status: int) -> str:
    return lib().h3attn_status_string(int(status)).decode()


def h3attn_last_error() -> str:
    return lib().h3attn_last_error().decode()


def h3attn_abi_version() -> int:
    return int(lib().h3attn_abi_version())


def _check(status: int, where: str):
    if status != H3ATTN_OK:
        raise H3AttnError(status, where, h3attn_last_error())


def rope_cfg(theta: float = DEFAULT_THETA, dims=DEFAULT_DIMS) -> RopeCfg:
    return RopeCfg(float(theta), int(dims[0]), int(dims[1]), int(dims[2]), 0)


def _items(segments):
    flat, counts = [], []
    for seg in segments:
        counts.append(len(seg))
        for it in seg:
            if it["kind"] == "visual":
                flat.append(Item(ITEM_VISUAL, it["T"], it["H"], it["W"], 0, 0, 0, 0, 0.0))
            elif it["kind"] == "audio":
                rule = AUDIO_ROUND_HALF_EVEN if it["rule"] == "round" else AUDIO_LINEAR
                flat.append(Item(ITEM_AUDIO, 0, 0, 0, it["n"], 1 if it["attached"] else 0, rule, 0, it["span"]))
            elif it["kind"] == "clock":
                flat.append(Item(ITEM_CLOCK, 0, 0, 0, 0, 0, 0, 0, it["span"]))
            elif it["kind"] == "text":
                flat.append(Item(ITEM_TEXT, 0, 0, 0, it["n"], 0, 0, 0, 0.0))
            else:
                raise ValueError(f"unknown item kind {it['kind']!r}")
    items = (Item * max(1, len(flat)))(*flat)
    cnt = (ctypes.c_int32 * max(1, len(counts)))(*counts)
    return items, cnt, len(counts)


def h3attn_build_layout(segments):
    """Segments of item dicts (see workloads.py) -> (cu_seqlens int32 [B+1], pos_thw float32 [N, 3])."""
    L = lib()
    items, cnt, n_seqs = _items(segments)
    n = ctypes.c_int64(0)
    _check(L.h3attn_build_layout(items, cnt, n_seqs, None, None, 0, ctypes.byref(n)), "h3attn_build_layout")
    cu = np.zeros(n_seqs + 1, dtype=np.int32)
    pos = np.zeros((max(1, n.value), 3), dtype=np.float32)
    _check(L.h3attn_build_layout(items, cnt, n_seqs, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 pos.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n.value, ctypes.byref(n)),
           "h3attn_build_layout")
    return cu, pos[:n.value]


# ---------------------------------------------------------------- GPU entry points

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def h3attn_rope_apply(x, pos_thw, out=None, theta=DEFAULT_THETA, dims=DEFAULT_DIMS, stream=None):
    """y = rope(x) on the GPU; x bf16 [N, H, 128], pos_thw fp32 [N, 3].  out may be x (in place)."""
    torch = _torch()
    _need(x, torch.bfloat16, None, "x")
    N, H, Dh = x.shape
    _need(pos_thw, torch.float32, (N, 3), "pos_thw")
    if out is None:
        out = torch.empty_like(x)
    _need(out, torch.bfloat16, x.shape, "out")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_rope_apply(x.data_ptr(), out.data_ptr(), pos_thw.data_ptr(), N, H, Dh, ctypes.byref(cfg),
                                   _stream_ptr(stream)), "h3attn_rope_apply")
    return out


def h3attn_varlen_fwd_workspace_size(n_tokens: int, n_heads: int, head_dim: int, n_seqs: int) -> int:
    return int(lib().h3attn_varlen_fwd_workspace_size(n_tokens, n_heads, head_dim, n_seqs))


def h3attn_skip_gate(skip_threshold: float, disabled_until_timestep: float, sigma: float) -> float:
    """The skip_threshold for a denoising step at noise level sigma: 0 (dense) above the cutoff."""
    out = ctypes.c_float()
    _check(lib().h3attn_skip_gate(float(skip_threshold), float(disabled_until_timestep), float(sigma),
                                  ctypes.byref(out)), "h3attn_skip_gate")
    return float(out.value)


def h3attn_varlen_fwd_fp8_workspace_size(n_tokens: int, n_heads: int, head_dim: int, n_seqs: int) -> int:
    return int(lib().h3attn_varlen_fwd_fp8_workspace_size(n_tokens, n_heads, head_dim, n_seqs))


def alloc_workspace(n_tokens: int, n_heads: int, n_seqs: int, device=None, fp8: bool = False):
    """Workspace for the exact path, or for the FP8 path with fp8=True (torch's allocation is 256-byte aligned)."""
    torch = _torch()
    size = h3attn_varlen_fwd_fp8_workspace_size if fp8 else h3attn_varlen_fwd_workspace_size
    nbytes = size(n_tokens, n_heads, 128, n_seqs)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device or "cuda")


def _varlen_common(q, cu_seqlens, pos_thw, max_seqlen):
    torch = _torch()
    _need(q, torch.bfloat16, None, "q")
    N, H, Dh = q.shape
    _need(cu_seqlens, torch.int32, None, "cu_seqlens")
    if cu_seqlens.ndim != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
    _need(pos_thw, torch.float32, (N, 3), "pos_thw")
    if max_seqlen is None:
        raise ValueError("max_seqlen is required (the library does not read device memory on the host)")
    return N, H, Dh, cu_seqlens.numel() - 1


def h3attn_varlen_fwd(q, k, v, cu_seqlens, pos_thw, max_seqlen, out=None, lse=None, softmax_scale=0.0,
                      theta=DEFAULT_THETA, dims=DEFAULT_DIMS, workspace=None, stream=None):
    """Packed varlen attention with fused multi-axis RoPE.  Returns (out bf16 [N,H,128], lse fp32 [H,N])."""
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(q, cu_seqlens, pos_thw, max_seqlen)
    _need(k, torch.bfloat16, q.shape, "k")
    _need(v, torch.bfloat16, q.shape, "v")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(out, torch.bfloat16, q.shape, "out")
    _need(lse, torch.float32, (H, N), "lse")
    if workspace is None:
        workspace = alloc_workspace(N, H, n_seqs, q.device)
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                   pos_thw.data_ptr(), out.data_ptr(), lse.data_ptr(), N, H, Dh, n_seqs,
                                   int(max_seqlen), float(softmax_scale), ctypes.byref(cfg), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "h3attn_varlen_fwd")
    return out, lse


def h3attn_varlen_fwd_noalloc(q, k, v, cu_seqlens, pos_thw, max_seqlen, out=None, lse=None, softmax_scale=0.0,
                              theta=DEFAULT_THETA, dims=DEFAULT_DIMS, stream=None):
    """h3attn_varlen_fwd on the library's own scratch array (no workspace argument, no allocation by the
    library); out and lse are allocated here when not given.  Returns (out, lse)."""
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(q, cu_seqlens, pos_thw, max_seqlen)
    _need(k, torch.bfloat16, q.shape, "k")
    _need(v, torch.bfloat16, q.shape, "v")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(out, torch.bfloat16, q.shape, "out")
    _need(lse, torch.float32, (H, N), "lse")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                           pos_thw.data_ptr(), out.data_ptr(), lse.data_ptr(), N, H, Dh, n_seqs,
                                           int(max_seqlen), float(softmax_scale), ctypes.byref(cfg),
                                           _stream_ptr(stream)),
           "h3attn_varlen_fwd_noalloc")
    return out, lse


def h3attn_varlen_kv_prologue(k, v, cu_seqlens, pos_thw, max_seqlen, workspace, theta=DEFAULT_THETA,
                              dims=DEFAULT_DIMS, stream=None):
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(k, cu_seqlens, pos_thw, max_seqlen)
    _need(v, torch.bfloat16, k.shape, "v")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_kv_prologue(k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), pos_thw.data_ptr(), N,
                                           H, Dh, n_seqs, int(max_seqlen), ctypes.byref(cfg), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "h3attn_varlen_kv_prologue")
    return workspace


def h3attn_varlen_attention(q, cu_seqlens, pos_thw, max_seqlen, workspace, out=None, lse=None, softmax_scale=0.0,
                            theta=DEFAULT_THETA, dims=DEFAULT_DIMS, stream=None):
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(q, cu_seqlens, pos_thw, max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(out, torch.bfloat16, q.shape, "out")
    _need(lse, torch.float32, (H, N), "lse")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_attention(q.data_ptr(), cu_seqlens.data_ptr(), pos_thw.data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), N, H, Dh, n_seqs, int(max_seqlen), float(softmax_scale),
                                         ctypes.byref(cfg), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "h3attn_varlen_attention")
    return out, lse


def _skip_stats_ptr(skip_stats):
    if skip_stats is None:
        return None
    torch = _torch()
    _need(skip_stats, torch.int64, (2,), "skip_stats")
    return skip_stats.data_ptr()


def h3attn_varlen_fwd_fp8(q, k, v, cu_seqlens, pos_thw, max_seqlen, out=None, lse=None, softmax_scale=0.0,
                          skip_threshold=0.0, theta=DEFAULT_THETA, dims=DEFAULT_DIMS, workspace=None, skip_stats=None,
                          stream=None):
    """Lossy FP8 (SAGE-style) mode of h3attn_varlen_fwd, optionally with Skip-Softmax; same results' layout.

    skip_stats: None or an int64 tensor [2] on the GPU that the call adds (tiles seen, tiles skipped) to.
    """
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(q, cu_seqlens, pos_thw, max_seqlen)
    _need(k, torch.bfloat16, q.shape, "k")
    _need(v, torch.bfloat16, q.shape, "v")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(out, torch.bfloat16, q.shape, "out")
    _need(lse, torch.float32, (H, N), "lse")
    if workspace is None:
        workspace = alloc_workspace(N, H, n_seqs, q.device, fp8=True)
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                       pos_thw.data_ptr(), out.data_ptr(), lse.data_ptr(), N, H, Dh, n_seqs,
                                       int(max_seqlen), float(softmax_scale), float(skip_threshold),
                                       ctypes.byref(cfg), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _skip_stats_ptr(skip_stats),
                                       _stream_ptr(stream)),
           "h3attn_varlen_fwd_fp8")
    return out, lse


def h3attn_varlen_kv_prologue_fp8(k, v, cu_seqlens, pos_thw, max_seqlen, workspace, theta=DEFAULT_THETA,
                                  dims=DEFAULT_DIMS, stream=None):
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(k, cu_seqlens, pos_thw, max_seqlen)
    _need(v, torch.bfloat16, k.shape, "v")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_kv_prologue_fp8(k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                               pos_thw.data_ptr(), N, H, Dh, n_seqs, int(max_seqlen),
                                               ctypes.byref(cfg), workspace.data_ptr(),
                                               workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "h3attn_varlen_kv_prologue_fp8")
    return workspace


def h3attn_varlen_attention_fp8(q, cu_seqlens, pos_thw, max_seqlen, workspace, out=None, lse=None,
                                softmax_scale=0.0, skip_threshold=0.0, theta=DEFAULT_THETA, dims=DEFAULT_DIMS,
                                skip_stats=None, stream=None):
    torch = _torch()
    N, H, Dh, n_seqs = _varlen_common(q, cu_seqlens, pos_thw, max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    _need(out, torch.bfloat16, q.shape, "out")
    _need(lse, torch.float32, (H, N), "lse")
    cfg = rope_cfg(theta, dims)
    _check(lib().h3attn_varlen_attention_fp8(q.data_ptr(), cu_seqlens.data_ptr(), pos_thw.data_ptr(),
                                             out.data_ptr(), lse.data_ptr(), N, H, Dh, n_seqs, int(max_seqlen),
                                             float(softmax_scale), float(skip_threshold), ctypes.byref(cfg),
                                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                             _skip_stats_ptr(skip_stats), _stream_ptr(stream)),
           "h3attn_varlen_attention_fp8")
    return out, lse


def attention_flops(cu_seqlens, n_heads: int, head_dim: int = 128) -> float:
    """Algorithmic FLOP of one call: 4 * S^2 * d per segment and head (in-segment pairs only)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    return float(4.0 * head_dim * n_heads * float(np.sum(lens.astype(np.float64) ** 2)))


def default_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)
