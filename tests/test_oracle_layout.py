"""Pins for the oracle's layout: closed forms, golden row maps, invariants.

None of these expected values comes from the oracle: token counts, prefix sums
and row maps are hand-computed from the workload statements (fixtures under
tests/golden/ carry their sources), and the per-row positions are re-derived
here by index arithmetic (division and remainder) rather than the oracle's
nested walk.
"""

import json
import os

import numpy as np
import pytest

import oracle
from joint_sequence_attention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_cu_seqlens_closed_form(name):
    g = _golden("layout_closed_forms.json")[name]
    cu, pos = oracle.layout(wl.config(name)["segments"])
    assert cu.dtype == np.int32 and pos.dtype == np.float32
    assert cu.tolist() == g["cu_seqlens"]
    assert pos.shape == (g["cu_seqlens"][-1], 3)


def _grid_positions(T, H, W, t0):
    r = np.arange(T * H * W)
    return np.stack([t0 + r // (H * W), (r // W) % H, r % W], axis=1).astype(np.float64)


def test_tiny_layout_exact():
    g = _golden("tiny_audio_t.json")
    cu, pos = oracle.layout(wl.config("tiny")["segments"])
    np.testing.assert_array_equal(pos[:192].astype(np.float64), _grid_positions(3, 8, 8, 0))
    np.testing.assert_array_equal(pos[192:, 0], np.array(g["audio_t"], dtype=np.float32))
    assert np.all(pos[192:, 1:] == 0)


@pytest.mark.parametrize("name,T,H,W,na", [("480p", 8, 24, 40, 256), ("1344x768", 32, 48, 84, 1024)])
def test_single_video_layout_exact(name, T, H, W, na):
    cu, pos = oracle.layout(wl.config(name)["segments"])
    nv = T * H * W
    np.testing.assert_array_equal(pos[:nv].astype(np.float64), _grid_positions(T, H, W, 0))
    # linearly spaced over [0, T): i * T / na, here exactly i / 32
    np.testing.assert_array_equal(pos[nv:, 0], (np.arange(na) / 32.0).astype(np.float32))
    assert np.all(pos[nv:, 1:] == 0)
    assert pos[nv:, 0].max() < T


def test_packed_segments_restart_clock():
    g = _golden("layout_closed_forms.json")["packed"]
    cu, pos = oracle.layout(wl.config("packed")["segments"])
    for s, (T, nv, na) in enumerate(g["segments"]):
        a = cu[s]
        np.testing.assert_array_equal(pos[a:a + nv].astype(np.float64), _grid_positions(T, 24, 42, 0))
        np.testing.assert_array_equal(pos[a + nv:a + nv + na, 0], (np.arange(na) / 32.0).astype(np.float32))
        assert a + nv + na == cu[s + 1]


def test_ref2va_row_map():
    g = _golden("ref2va_row_map.json")
    cu, pos = oracle.layout(wl.config("ref2va")["segments"])
    assert cu.tolist() == [0, g["n_tokens"]]
    for first, last, what, t0, t1, hmax, wmax in g["rows"]:
        blk = pos[first:last + 1]
        assert blk[0, 0] == t0 and blk[-1, 0] == t1, what
        assert blk[:, 1].max() == hmax and blk[:, 2].max() == wmax, what
        assert np.all(np.diff(blk[:, 0]) >= 0), what
    # each image j sits at t = j on a full 24x42 grid
    for j in range(9):
        np.testing.assert_array_equal(pos[1008 * j:1008 * (j + 1)].astype(np.float64), _grid_positions(1, 24, 42, j))
    np.testing.assert_array_equal(pos[9072:17136].astype(np.float64), _grid_positions(8, 24, 42, 9))
    np.testing.assert_array_equal(pos[17648:34784].astype(np.float64), _grid_positions(17, 24, 42, 25))


def test_reference_order_changes_positions():
    # A different reference order is a different request: the shared clock is
    # advanced in reference order.
    seg = wl.config("ref2va")["segments"][0]
    swapped = [seg[9], seg[10], seg[11]] + seg[:9] + seg[12:]   # video(+audio), audio, then images
    _, p1 = oracle.layout([seg])
    _, p2 = oracle.layout([swapped])
    assert p1.shape == p2.shape
    assert not np.array_equal(p1, p2)
    # The video reference now starts the clock at 0 and the images follow it.
    np.testing.assert_array_equal(p2[:8064].astype(np.float64), _grid_positions(8, 24, 42, 0))
    assert p2[8064 + 256 + 256, 0] == 16.0   # first image after video (8) + standalone audio (8)


def test_positions_exact_in_float32():
    # every position the workloads produce is exactly representable: the
    # float64 -> float32 cast loses nothing
    for name in wl.CONFIG_ORDER:
        segs = wl.config(name)["segments"]
        _, pos = oracle.layout(segs)
        assert np.all(np.isfinite(pos))
        assert np.all(pos.astype(np.float64) * 32 == np.round(pos.astype(np.float64) * 32))


def test_round_half_even_matches_python_round():
    xs = [i / 8 for i in range(-40, 41)] + [0.5, 1.5, 2.5, -0.5, -1.5, 3.4999, 3.5001]
    for x in xs:
        assert oracle.round_half_even(x) == float(round(x)), x


def test_empty_and_degenerate_segments():
    segs = [[wl.visual(1, 1, 1)], [], [wl.visual(2, 1, 3), wl.audio(1, 2, attached=True)]]
    cu, pos = oracle.layout(segs)
    assert cu.tolist() == [0, 1, 1, 8]
    np.testing.assert_array_equal(pos[0], [0, 0, 0])
    np.testing.assert_array_equal(pos[1:7].astype(np.float64), _grid_positions(2, 1, 3, 0))
    np.testing.assert_array_equal(pos[7], [0, 0, 0])


def test_attached_audio_needs_visual():
    with pytest.raises(ValueError):
        oracle.layout([[wl.audio(4, 1, attached=True)]])


def test_native_frame_grid_matches_recipe_example():
    # vLLM-Omni "MiniMax-H3" recipe, "Long video and driving audio": a 75-second request becomes
    # 1,807 frames (75.292 s at 24 FPS) on the 17n+5 grid
    assert wl.native_frames(75) == 1807 and abs(1807 / 24 - 75.292) < 5e-4
    assert wl.latent_frames(1807) == 5 * 106 + 2
    assert wl.native_frames(300) == 7213 and wl.latent_frames(7213) == 2122


def test_long_video_chunk_keeps_global_time():
    g = _golden("layout_closed_forms.json")["long300"]
    cu, pos = oracle.layout(wl.config("long300")["segments"])
    assert cu.tolist() == g["cu_seqlens"]
    a, b = g["image_rows"], g["image_rows"] + g["chunk_rows"]
    np.testing.assert_array_equal(pos[:a].astype(np.float64), _grid_positions(1, 24, 42, 0))
    np.testing.assert_array_equal(pos[a:b].astype(np.float64), _grid_positions(17, 24, 42, g["chunk_t_first"]))
    assert pos[b - 1, 0] == g["chunk_t_last"]
    np.testing.assert_array_equal(pos[b:, 0], (g["chunk_t_first"] + np.arange(g["audio_rows"]) / 32.0).astype(np.float32))
    assert np.all(pos[b:, 1:] == 0)


def test_clock_item_moves_only_what_follows():
    base = [wl.visual(2, 2, 3), wl.audio(4, 2, attached=True), wl.visual(1, 2, 2)]
    moved = [wl.visual(2, 2, 3), wl.clock(7.5), wl.audio(4, 2, attached=True), wl.visual(1, 2, 2)]
    _, p0 = oracle.layout([base])
    _, p1 = oracle.layout([moved])
    np.testing.assert_array_equal(p0[:16], p1[:16])           # the video and its soundtrack stay
    np.testing.assert_array_equal(p1[16:, 0], p0[16:, 0] + 7.5)  # the next item starts 7.5 later
    np.testing.assert_array_equal(p1[16:, 1:], p0[16:, 1:])
    # a zero advance changes nothing, and advances add up
    _, pz = oracle.layout([[wl.clock(0.0)] + base])
    np.testing.assert_array_equal(pz, p0)
    _, pa = oracle.layout([[wl.clock(3.0), wl.clock(4.5)] + base])
    _, pb = oracle.layout([[wl.clock(7.5)] + base])
    np.testing.assert_array_equal(pa, pb)


def test_text_rows_sit_at_origin():
    g = _golden("layout_closed_forms.json")["refiner"]
    cu, pos = oracle.layout(wl.config("refiner")["segments"])
    assert cu.tolist() == g["cu_seqlens"]
    assert np.all(pos == 0)
    # text rows leave the clock alone
    _, p = oracle.layout([[wl.text(5), wl.visual(1, 1, 2), wl.text(3), wl.visual(1, 1, 1)]])
    assert p[5:7, 0].tolist() == [0.0, 0.0] and p[10, 0] == 1.0 and np.all(p[7:10] == 0)
