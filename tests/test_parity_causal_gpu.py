"""GPU parity of the chunk-causal forward (the training-time pass of VideoMLA §3.3
with the block masks of App. D.4): the query chunk spans several blocks of
causal_frames frames and each block attends the context before the chunk plus
its own and earlier blocks.  Through the C ABI against the fp64 oracle, same
tolerances as the other parity tests."""
import pytest

import oracle as O
import workload as W
from parity_helpers import Run
from test_parity_gpu import full_step, sampled_full, small_wan

pytestmark = pytest.mark.gpu


def test_clip_in_blocks_of_two():
    """Six frames written and attended in one call, blocks of two: 1440 rows per
    block (5.6 row tiles of 256) and 120, 240, 360 keys (ragged key tiles)."""
    s = small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6, causal_frames=2)
    full_step(Run(s, random_gains=True))


def test_blocks_after_cached_frames():
    """Frames 0-3 cached, chunk 4-7 in blocks [4,5] and [6,7]."""
    s = small_wan(window_frames=8, chunk_frames=4, t0=4, n_valid_frames=8, causal_frames=2)
    full_step(Run(s))


def test_blocks_over_a_wrapped_ring():
    """Window frames 8-12 in a 5-slot ring (slots 3,4,0,1,2), chunk 9-12 in blocks
    of two: the block prefixes cross the ring's wrap point."""
    s = small_wan(window_frames=5, chunk_frames=4, t0=9, n_valid_frames=5, causal_frames=2)
    full_step(Run(s))


def test_single_frame_blocks_batch_of_two():
    s = small_wan(window_frames=4, chunk_frames=4, t0=0, n_valid_frames=4, causal_frames=1)
    full_step(Run(s, batch=2))


def test_blocks_with_sink_and_read_rotation():
    """Sink frame 0 plus local frames 8-11, the chunk being 8-11 in two blocks: the
    keys before the chunk are the sink's."""
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=4, chunk_frames=4, t0=8,
                  n_valid_frames=4, causal_frames=2)
    assert O.window_frames(s.t0, s.chunk_frames, s.n_valid_frames, s.sink_frames) == [0, 8, 9, 10, 11]
    full_step(Run(s, random_gains=True))


def test_blocks_fp32():
    s = W.shape_by_name("tiny-f32").with_(chunk_frames=4, t0=0, n_valid_frames=4, causal_frames=2)
    full_step(Run(s, random_gains=True))


def test_blocks_sharp_softmax():
    """RMSNorm gain of c^Q x8 (a scale on W^Q_down would be cancelled by the
    normalisation): logits of standard deviation ~8 nats, inside the fast kernel's
    range, so nothing is flagged."""
    run = Run(small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6,
                        causal_frames=3), scale={"g_q": 8.0})
    full_step(run, check_cache=False)
    flags = run.L.overflow_flags(run.chunk())
    assert len(flags) > 0 and not flags.any(), flags


def test_blocks_exact_path(monkeypatch):
    """The fast kernel's bound forced down to 2 (MLA_ATTN_OVERFLOW_LIMIT): every piece
    of every block's row tiles is recomputed against its exact maximum, each over its
    own block's key count."""
    monkeypatch.setenv("MLA_ATTN_OVERFLOW_LIMIT", "2")
    run = Run(small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6,
                        causal_frames=2), random_gains=True)
    full_step(run, check_cache=False)
    flags = run.L.overflow_flags(run.chunk())
    assert flags.all(), f"{int((flags == 0).sum())} of {len(flags)} row tiles not flagged"


def test_clip21_full_size_sampled():
    """The Wan-1.3B 21-frame clip in 3-frame blocks, written and attended in one
    call: sampled tokens of every block (all heads) and sampled cache rows."""
    sampled_full(W.shape_by_name("wan1.3b-clip21-causal3"))
