"""The C ABI under HIP graph capture and on concurrent streams (GPU).

Every call takes device pointers, enqueues its kernels on the caller's stream
and allocates, frees, synchronizes and clears nothing, so a caller may capture
it in a graph and replay it, or run independent calls on several streams.
Each graph is replayed several times, with the program's own eager work and
synchronizations between replays, and every replay is compared bitwise with
the eager result.
"""

import numpy as np
import pytest

from helpers import Case, bf16_bits, ragged_segments, say
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _eager_and_graph(c, fp8, replays=3):
    import torch
    ws = H.alloc_workspace(c.N, c.heads, len(c.lens), fp8=fp8)
    fwd = H.h3attn_varlen_fwd_fp8 if fp8 else H.h3attn_varlen_fwd
    out_e, lse_e = fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, workspace=ws)   # also the first-use set-up
    torch.cuda.synchronize()
    ref = (bf16_bits(out_e).copy(), lse_e.cpu().numpy().copy())
    out = torch.empty_like(c.q)
    lse = torch.empty((c.heads, c.N), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, out=out, lse=lse, workspace=ws,
                stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(replays):
        out.fill_(0)
        lse.fill_(0)
        ws.fill_(255)                          # the replay must rebuild the workspace itself
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = np.array_equal(bf16_bits(out), ref[0]) and np.array_equal(lse.cpu().numpy(), ref[1])
        say(f"  replay {r}: bitwise equal to eager: {same}")
        assert same
        # eager work of the program between replays
        fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_replays_equal_eager_calls(gpu, fp8):
    c = Case(ragged_segments(), 3, 200)
    say(f"graph capture, {'fp8' if fp8 else 'exact'}: lens={c.lens.tolist()}")
    _eager_and_graph(c, fp8)


def test_graph_replays_on_the_refiner_workload(gpu):
    cfg = wl.config("refiner")
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    say(f"graph capture, refiner: N={c.N} H={c.heads}")
    _eager_and_graph(c, False)


def test_concurrent_streams_equal_serial_calls(gpu):
    import torch
    cases = [Case(ragged_segments(), 2, 201), Case(wl.config("480p")["segments"], 24, 202)]
    serial = []
    for c in cases:
        o, l = c.run()
        serial.append((bf16_bits(o).copy(), l.cpu().numpy().copy()))
    streams = [torch.cuda.Stream() for _ in cases]
    results = []
    torch.cuda.synchronize()
    for _ in range(3):
        outs = []
        for c, s in zip(cases, streams):
            ws = H.alloc_workspace(c.N, c.heads, len(c.lens))
            out = torch.empty_like(c.q)
            lse = torch.empty((c.heads, c.N), dtype=torch.float32, device="cuda")
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                H.h3attn_varlen_fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, out=out, lse=lse, workspace=ws,
                                    stream=s)
            outs.append((out, lse, ws))
        torch.cuda.synchronize()
        for (out, lse, _), (o_ref, l_ref) in zip(outs, serial):
            assert np.array_equal(bf16_bits(out), o_ref) and np.array_equal(lse.cpu().numpy(), l_ref)
        results.append(True)
    say(f"concurrent streams: {len(results)} rounds equal to the serial calls")
