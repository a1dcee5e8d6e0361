"""Host-side tests of the C ABI (no GPU needed): exports, layout builder, argument checks.

The layout builder is compared bit for bit with the oracle's layout; the
argument checks are exercised through ctypes with raw pointers and must return
their status before anything is launched.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(H.library_path()):
        from joint_sequence_attention_amd import build
        build.build()
    return H.lib()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "h3attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3attn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    declared = _header_functions()
    assert declared == sorted(H.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name
    assert H.h3attn_abi_version() == 1


def test_status_strings(L):
    assert H.h3attn_status_string(0) == "H3ATTN_OK"
    assert H.h3attn_status_string(3) == "H3ATTN_ERR_WORKSPACE"
    assert H.h3attn_status_string(99) == "H3ATTN_UNKNOWN_STATUS"


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_layout_bit_exact_vs_oracle(L, name):
    segs = wl.config(name)["segments"]
    cu, pos = H.h3attn_build_layout(segs)
    cu_o, pos_o = oracle.layout(segs)
    assert cu.dtype == np.int32 and pos.dtype == np.float32
    assert np.array_equal(cu, cu_o)
    assert pos.shape == pos_o.shape
    assert np.array_equal(pos.view(np.uint32), pos_o.view(np.uint32))


def test_layout_edge_cases_bit_exact(L):
    segs = [
        [wl.visual(1, 1, 1)],
        [],
        [wl.visual(2, 3, 5), wl.audio(7, 2, attached=True), wl.audio(5, 1.5, attached=False, rule="round"),
         wl.audio(0, 3, attached=False), wl.visual(1, 2, 2), wl.audio(3, 1, attached=True, rule="round")],
        [wl.audio(9, 2.25, attached=False)],
        [wl.text(4), wl.clock(2.5), wl.visual(1, 2, 2), wl.clock(0.0), wl.audio(3, 1, attached=True),
         wl.clock(1e6 + 0.25), wl.visual(2, 1, 1), wl.text(0), wl.audio(2, 0.5, attached=False)],
        [wl.clock(3.0)],
    ]
    cu, pos = H.h3attn_build_layout(segs)
    cu_o, pos_o = oracle.layout(segs)
    assert np.array_equal(cu, cu_o)
    assert np.array_equal(pos.view(np.uint32), pos_o.view(np.uint32))


def _item(kind, T=1, Hh=1, W=1, n=0, attached=0, rule=0, span=0.0):
    return H.Item(kind, T, Hh, W, n, attached, rule, 0, span)


def _layout_status(L, items, counts):
    arr = (H.Item * max(1, len(items)))(*items)
    cnt = (ctypes.c_int32 * max(1, len(counts)))(*counts)
    n = ctypes.c_int64(-1)
    return L.h3attn_build_layout(arr, cnt, len(counts), None, None, 0, ctypes.byref(n)), n.value


@pytest.mark.parametrize(
    "items,counts",
    [
        ([_item(0, T=0)], [1]),                                  # empty grid
        ([_item(0, W=-2)], [1]),
        ([_item(1, n=-1, span=1.0)], [1]),                       # negative audio rows
        ([_item(1, n=4, span=float("nan"))], [1]),
        ([_item(1, n=4, span=-1.0)], [1]),
        ([_item(1, n=4, span=1.0, attached=1)], [1]),            # attached audio without a video
        ([_item(1, n=4, span=1.0, rule=7)], [1]),
        ([_item(2, span=float("nan"))], [1]),                    # clock advance not finite
        ([_item(2, span=float("inf"))], [1]),
        ([_item(2, span=-0.5)], [1]),                            # clock going back
        ([_item(3, n=-1)], [1]),                                 # negative text rows
        ([_item(5)], [1]),                                       # unknown kind
        ([_item(0)], [-1]),
        ([_item(0, T=2048, Hh=2048, W=1024)], [1]),              # more than INT32_MAX tokens
    ],
)
def test_layout_rejects_malformed_items(L, items, counts):
    st, _ = _layout_status(L, items, counts)
    assert st == H.H3ATTN_ERR_INVALID_ARG
    assert H.h3attn_last_error() != ""


def test_layout_capacity_checked(L):
    arr = (H.Item * 1)(_item(0, T=2, Hh=2, W=2))
    cnt = (ctypes.c_int32 * 1)(1)
    n = ctypes.c_int64(0)
    buf = (ctypes.c_float * 3)()
    st = L.h3attn_build_layout(arr, cnt, 1, None, buf, 1, ctypes.byref(n))
    assert st == H.H3ATTN_ERR_INVALID_ARG and n.value == 8
    assert L.h3attn_build_layout(arr, cnt, 0, None, None, 0, ctypes.byref(n)) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_build_layout(arr, cnt, 1, None, None, 0, None) == H.H3ATTN_ERR_INVALID_ARG


FAKE = 0x10000  # host-side stand-in address; the checks below fail before any launch


def _cfg(theta=10000.0, dims=(32, 48, 48)):
    return ctypes.byref(H.rope_cfg(theta, dims))


def _fwd(L, q=FAKE, k=FAKE * 2, v=FAKE * 3, cu=FAKE * 4, pos=FAKE * 5, out=1 << 40, lse=1 << 41, N=64, Hh=2,
         Dh=128, ns=1, ms=64, scale=0.0, cfg=None, ws=1 << 42, wsb=None, fp8=False, skip=0.0):
    size = L.h3attn_varlen_fwd_fp8_workspace_size if fp8 else L.h3attn_varlen_fwd_workspace_size
    if wsb is None:
        wsb = size(N, Hh, 128, ns)
    if fp8:
        return L.h3attn_varlen_fwd_fp8(q, k, v, cu, pos, out, lse, N, Hh, Dh, ns, ms, scale, skip, cfg or _cfg(), ws,
                                       wsb, None, None)
    return L.h3attn_varlen_fwd(q, k, v, cu, pos, out, lse, N, Hh, Dh, ns, ms, scale, cfg or _cfg(), ws, wsb, None)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(Dh=64), H.H3ATTN_ERR_UNSUPPORTED),
        (dict(Dh=256), H.H3ATTN_ERR_UNSUPPORTED),
        (dict(Hh=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(N=-1), H.H3ATTN_ERR_INVALID_ARG),
        (dict(ns=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(ms=-1), H.H3ATTN_ERR_INVALID_ARG),
        (dict(ms=65), H.H3ATTN_ERR_INVALID_ARG),
        (dict(q=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(k=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(cu=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(pos=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(out=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(lse=0), H.H3ATTN_ERR_INVALID_ARG),
        (dict(scale=float("nan")), H.H3ATTN_ERR_INVALID_ARG),
        (dict(ws=0), H.H3ATTN_ERR_WORKSPACE),
        (dict(ws=(1 << 42) + 8), H.H3ATTN_ERR_WORKSPACE),
        (dict(wsb=1024), H.H3ATTN_ERR_WORKSPACE),
        (dict(out=FAKE), H.H3ATTN_ERR_INVALID_ARG),          # out overlaps q
        (dict(lse=(1 << 40) + 64), H.H3ATTN_ERR_INVALID_ARG),  # lse overlaps out
    ],
)
@pytest.mark.parametrize("fp8", [False, True])
def test_varlen_fwd_argument_checks(L, kw, status, fp8):
    assert _fwd(L, fp8=fp8, **kw) == status
    assert H.h3attn_last_error() != ""


@pytest.mark.parametrize(
    "dims,theta,status",
    [
        ((32, 48, 40), 10000.0, H.H3ATTN_ERR_UNSUPPORTED),   # does not add up to 128
        ((33, 47, 48), 10000.0, H.H3ATTN_ERR_UNSUPPORTED),   # odd widths
        ((32, 48, 48), 0.0, H.H3ATTN_ERR_INVALID_ARG),
        ((32, 48, 48), float("inf"), H.H3ATTN_ERR_INVALID_ARG),
    ],
)
def test_rope_config_checks(L, dims, theta, status):
    assert _fwd(L, cfg=_cfg(theta, dims)) == status
    assert _fwd(L, cfg=_cfg(theta, dims), fp8=True) == status
    assert L.h3attn_rope_apply(FAKE, FAKE, FAKE * 2, 8, 1, 128, _cfg(theta, dims), None) == status


def test_null_rope_config(L):
    assert L.h3attn_varlen_fwd(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1 << 40, 1 << 41, 8, 1, 128, 1, 8, 0.0,
                               None, 1 << 42, 1 << 30, None) == H.H3ATTN_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(L):
    # N = 0 returns OK without touching any pointer or launching anything
    assert _fwd(L, q=0, k=0, v=0, cu=0, pos=0, out=0, lse=0, N=0, ms=0, ws=0, wsb=0) == H.H3ATTN_OK
    assert _fwd(L, q=0, k=0, v=0, cu=0, pos=0, out=0, lse=0, N=0, ms=0, ws=0, wsb=0, fp8=True) == H.H3ATTN_OK
    assert L.h3attn_rope_apply(None, None, None, 0, 1, 128, _cfg(), None) == H.H3ATTN_OK


def test_rope_apply_argument_checks(L):
    assert L.h3attn_rope_apply(FAKE, FAKE, FAKE * 8, 8, 1, 64, _cfg(), None) == H.H3ATTN_ERR_UNSUPPORTED
    assert L.h3attn_rope_apply(0, FAKE, FAKE * 8, 8, 1, 128, _cfg(), None) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_apply(FAKE, FAKE + 16, FAKE * 8, 8, 1, 128, _cfg(), None) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_rope_apply(FAKE, FAKE, FAKE * 8, -1, 1, 128, _cfg(), None) == H.H3ATTN_ERR_INVALID_ARG


def test_workspace_size_formula(L):
    # per head: 64 * (ceil(N / 64) + n_seqs) rows of 128 16-bit values, for keys and for
    # values, plus one fp32 key scale per 64-row tile; then, from the next 256-byte boundary,
    # one int32 per segment (the segments' order by length)
    for N, Hh, ns in [(1, 1, 1), (64, 2, 1), (65, 3, 4), (130048, 5, 1), (45760, 16, 4), (2542, 56, 8)]:
        rows = 64 * ((N + 63) // 64 + ns)
        order_at = (2 * Hh * rows * 128 * 2 + Hh * (rows // 64) * 4 + 255) // 256 * 256
        assert L.h3attn_varlen_fwd_workspace_size(N, Hh, 128, ns) == order_at + 4 * ns
    assert L.h3attn_varlen_fwd_workspace_size(10, 1, 64, 1) == 0


def test_fp8_workspace_size_formula(L):
    # per head: 64 * (ceil(N / 64) + n_seqs) rows of 128 bytes for keys and for values, then one
    # 32-bit word per 64-row tile (key scales) and one per (head, segment, value channel) (the
    # channels' largest magnitudes), each padded to 256 bytes, then one int32 per segment (the
    # segments' order by length)
    for N, Hh, ns in [(1, 1, 1), (64, 2, 1), (65, 3, 4), (130048, 5, 1), (45760, 16, 4), (2542, 56, 8)]:
        rows = 64 * ((N + 63) // 64 + ns)
        kscales = (Hh * (rows // 64) * 4 + 255) // 256 * 256
        vamax = (Hh * ns * 128 * 4 + 255) // 256 * 256
        assert L.h3attn_varlen_fwd_fp8_workspace_size(N, Hh, 128, ns) == \
            2 * Hh * rows * 128 + kscales + vamax + 4 * ns
    assert L.h3attn_varlen_fwd_fp8_workspace_size(10, 1, 64, 1) == 0


def test_fp8_stage_argument_checks(L):
    wsb = L.h3attn_varlen_fwd_fp8_workspace_size(64, 2, 128, 1)
    assert L.h3attn_varlen_kv_prologue_fp8(FAKE, FAKE * 2, FAKE * 4, FAKE * 5, 64, 2, 128, 1, 64, _cfg(), 1 << 42,
                                           wsb - 1, None) == H.H3ATTN_ERR_WORKSPACE
    assert L.h3attn_varlen_attention_fp8(FAKE, FAKE * 4, FAKE * 5, 1 << 40, 1 << 41, 64, 2, 128, 1, 64, 0.0, 0.0,
                                         _cfg(), 1 << 42, wsb - 1, None, None) == H.H3ATTN_ERR_WORKSPACE
    assert L.h3attn_varlen_attention_fp8(FAKE, FAKE * 4, FAKE * 5, FAKE, 1 << 41, 64, 2, 128, 1, 64, 0.0, 0.0,
                                         _cfg(), 1 << 42, wsb, None, None) == H.H3ATTN_ERR_INVALID_ARG   # out overlaps q
    for bad in (-0.1, 1.0, float("nan"), float("inf")):
        assert _fwd(L, fp8=True, skip=bad) == H.H3ATTN_ERR_INVALID_ARG
        assert L.h3attn_varlen_attention_fp8(FAKE, FAKE * 4, FAKE * 5, 1 << 40, 1 << 41, 64, 2, 128, 1, 64, 0.0, bad,
                                             _cfg(), 1 << 42, wsb, None, None) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_varlen_kv_prologue_fp8(FAKE, FAKE * 2, FAKE * 4, FAKE * 5, 64, 2, 64, 1, 64, _cfg(), 1 << 42,
                                           wsb, None) == H.H3ATTN_ERR_UNSUPPORTED


def test_max_seqlen_limit(L):
    # A segment's keys are addressed through 32-bit buffer offsets, 256 bytes per key: max_seqlen
    # above 2^22 is refused in both modes and by every stage, before anything is launched.
    N = (1 << 22) + 1
    big = 1 << 44
    for fp8 in (False, True):
        wsb = (L.h3attn_varlen_fwd_fp8_workspace_size if fp8 else L.h3attn_varlen_fwd_workspace_size)(N, 1, 128, 1)
        assert _fwd(L, N=N, Hh=1, ms=N, out=big, lse=2 * big, ws=4 * big, wsb=wsb, fp8=fp8) == \
            H.H3ATTN_ERR_UNSUPPORTED
        assert "2^22" in H.h3attn_last_error()
        # 2^22 itself passes the size check and fails only later, on a NULL pointer
        assert _fwd(L, N=N, Hh=1, ms=1 << 22, q=0, out=big, lse=2 * big, ws=4 * big, wsb=wsb, fp8=fp8) == \
            H.H3ATTN_ERR_INVALID_ARG
    wsb = L.h3attn_varlen_fwd_workspace_size(N, 1, 128, 1)
    assert L.h3attn_varlen_kv_prologue(FAKE, FAKE * 2, FAKE * 4, FAKE * 5, N, 1, 128, 1, N, _cfg(), 4 * big, wsb,
                                       None) == H.H3ATTN_ERR_UNSUPPORTED
    assert L.h3attn_varlen_attention(FAKE, FAKE * 4, FAKE * 5, big, 2 * big, N, 1, 128, 1, N, 0.0, _cfg(), 4 * big,
                                     wsb, None) == H.H3ATTN_ERR_UNSUPPORTED
    wsb8 = L.h3attn_varlen_fwd_fp8_workspace_size(N, 1, 128, 1)
    assert L.h3attn_varlen_kv_prologue_fp8(FAKE, FAKE * 2, FAKE * 4, FAKE * 5, N, 1, 128, 1, N, _cfg(), 4 * big,
                                           wsb8, None) == H.H3ATTN_ERR_UNSUPPORTED
    assert L.h3attn_varlen_attention_fp8(FAKE, FAKE * 4, FAKE * 5, big, 2 * big, N, 1, 128, 1, N, 0.0, 0.0, _cfg(),
                                         4 * big, wsb8, None, None) == H.H3ATTN_ERR_UNSUPPORTED


def test_noalloc_checks_before_any_launch(L):
    # the no-allocation entry point refuses a call beyond its 128 MiB array, and bad arguments,
    # before it touches the GPU; N = 0 is a no-op
    cfg = _cfg()
    big = 1 << 44
    st = L.h3attn_varlen_fwd_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, big, 2 * big, 130048, 5, 128, 1,
                                     130048, 0.0, cfg, None)
    assert st == H.H3ATTN_ERR_UNSUPPORTED and "128 MiB" in H.h3attn_last_error()
    assert L.h3attn_varlen_fwd_workspace_size(130048, 5, 128, 1) > 128 << 20
    assert L.h3attn_varlen_fwd_workspace_size(7936, 24, 128, 1) <= 128 << 20
    assert L.h3attn_varlen_fwd_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, big, 2 * big, 64, 2, 64, 1, 64,
                                       0.0, cfg, None) == H.H3ATTN_ERR_UNSUPPORTED
    assert L.h3attn_varlen_fwd_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, big, 2 * big, 64, 2, 128, 1, 65,
                                       0.0, cfg, None) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_varlen_fwd_noalloc(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, big, 2 * big, 64, 2, 128, 1, 64,
                                       float("nan"), cfg, None) == H.H3ATTN_ERR_INVALID_ARG
    assert L.h3attn_varlen_fwd_noalloc(None, None, None, None, None, None, None, 0, 2, 128, 1, 0, 0.0, cfg,
                                       None) == H.H3ATTN_OK
