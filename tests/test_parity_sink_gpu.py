"""GPU parity of the read-time positional path (VideoMLA §3.2: the cache keeps k^R
unrotated; App. D.4-D.5: a sink frame plus the most recent local frames, re-indexed
to window-local temporal coordinates when the window is assembled), through the C
ABI, against the fp64 oracle on the same seeded inputs.  Same tolerances as the
other parity tests; cache rows within one bf16 ulp, slot map exact."""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W
from latent_kv_attention_down_amd.layer import DeviceLayer, to_host
from parity_helpers import TOL, Run, assert_cache_rows, assert_close, say
from test_parity_gpu import full_step, sampled_full, small_wan

pytestmark = pytest.mark.gpu


def test_read_rotation_without_sink():
    """Unrotated keys, rotated on assembly at window-local t: the cache holds raw k^R
    and the step matches the oracle (and so, by the oracle's pin, write rotation)."""
    full_step(Run(small_wan(rope_at_read=True, t0=9), random_gains=True))


def test_sink_and_local_window():
    """Sink frame 0 plus local frames 11..13 in 1 + 3 slots (frame 13 has evicted
    frame 10 from slot 1); the chunk is frames 12-13."""
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=3, chunk_frames=2, t0=12,
                  n_valid_frames=3)
    assert O.window_frames(s.t0, s.chunk_frames, s.n_valid_frames, s.sink_frames) == [0, 11, 12, 13]
    full_step(Run(s, random_gains=True))


def test_sink_fp32_tiny():
    s = W.shape_by_name("tiny-f32").with_(rope_at_read=True, sink_frames=1, t0=6)
    assert O.window_frames(s.t0, s.chunk_frames, s.n_valid_frames, s.sink_frames) == [0, 3, 4, 5, 6]
    full_step(Run(s, random_gains=True))


def test_sink_frame_attends_only_itself():
    """The first chunk of a rollout is the sink frame alone: no local frames."""
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=3, chunk_frames=1, t0=0,
                  n_valid_frames=0)
    assert O.window_frames(s.t0, s.chunk_frames, s.n_valid_frames, s.sink_frames) == [0]
    full_step(Run(s))


def test_rollout_through_eviction():
    """Write frames 0..13 two at a time from an empty cache, then attend from the
    last chunk: the ring is exactly what FIFO over 3 local slots plus one sink slot
    leaves (App. D.4), and the output is the oracle's over the re-indexed context."""
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=3, chunk_frames=2, t0=12,
                  n_valid_frames=3)
    say(f"case rollout S=1 W=3 C=2 frames 0..13 grid {s.grid_h}x{s.grid_w}")
    stored, w = W.draw_weights(s, random_gains=True)
    frames = list(range(14))
    xs, xe = W.draw_frames(s, frames)
    L = DeviceLayer(s, stored)
    tpf = s.tokens_per_frame
    for t0 in range(0, 14, 2):
        L.cache_write(L.chunk(2, t0, 0), L.tokens(xs[:, t0 * tpf:(t0 + 2) * tpf]))
    ch = L.chunk(2, 12, 3)
    out = L.chunk_attention(ch, L.tokens(xs[:, 12 * tpf:14 * tpf]))
    torch.cuda.synchronize()
    ring = to_host(L.ring())[0]
    ref_ring = O.expected_ring(s, w, xe[0], frames)
    assert_cache_rows(ring, ref_ring, "bf16", "ring after the rollout")
    ref = O.step(s, w, {f: xe[0][f * tpf:(f + 1) * tpf] for f in frames})
    assert_close(to_host(out)[0], ref["out"], TOL["bf16"], "out_heads")


@pytest.mark.parametrize("name", ["wan1.3b-w21-read", "wan1.3b-sink1-w6-t240"])
def test_read_rotation_full_size_sampled(name):
    """Full Wan-1.3B layer: the 21-frame window with read-time rotation, and the
    long-rollout cache of one sink frame plus six local frames at frames 238-240."""
    sampled_full(W.shape_by_name(name))
