"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on
the same seeded inputs.  Tolerances: relative 2e-2 (Frobenius and max-abs over
max) for bf16 outputs, 1e-5 in fp32 mode; cache contents within one bf16 ulp;
slot map and window bookkeeping exact."""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W
from latent_kv_attention_down_amd.layer import to_host
from parity_helpers import TOL, Run, assert_cache_rows, assert_close, rel_errors, say

pytestmark = pytest.mark.gpu


def small_wan(**kw):
    """Wan-1.3B head geometry on a 6x10 grid: 60 tokens per frame, so windows span
    several 64-key tiles with a ragged tail and query rows several row tiles."""
    base = W.shape_by_name("wan1.3b-w21").with_(grid_h=6, grid_w=10, window_frames=5,
                                                 chunk_frames=2, t0=3, n_valid_frames=5)
    return base.with_(**kw)


def full_step(run, check_cache=True, sample=None):
    say(f"case {run.s.name} dtype={run.s.dtype} W={run.s.window_frames} C={run.s.chunk_frames} "
        f"t0={run.s.t0} n_valid={run.s.n_valid_frames} grid={run.s.grid_h}x{run.s.grid_w} "
        f"d_c={run.s.d_c} d_rope={run.s.d_rope} batch={run.batch}")
    run.prefill()
    ch = run.chunk()
    y = run.L.step(ch, run.chunk_tokens())
    torch.cuda.synchronize()
    tol = TOL[run.s.dtype]
    ring = to_host(run.L.ring())
    y_h = to_host(y)
    for b in range(run.batch):
        ref = run.oracle(b, query_rows=sample)
        got_y = y_h[b] if sample is None else y_h[b][sample]
        assert_close(got_y, ref["y"], tol, f"y[b={b}]")
        if check_cache:
            assert_cache_rows(ring[b], run.oracle_ring(b), run.s.dtype, f"cache[b={b}]")
    return y


def test_tiny_fp32_step():
    """Tiny fp32 layer: hidden 64, 2 heads, d_c 16, 4x4 grid, 3 cached + 1 query frame."""
    run = Run(W.shape_by_name("tiny-f32"), random_gains=True)
    full_step(run)


def test_tiny_fp32_chunk_attention_out_heads():
    run = Run(W.shape_by_name("tiny-f32"))
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    run.L.cache_write(ch, x)
    out = run.L.chunk_attention(ch, x)
    torch.cuda.synchronize()
    assert_close(to_host(out)[0], run.oracle()["out"], TOL["f32"], "out_heads")


def test_small_bf16_step():
    full_step(Run(small_wan(), random_gains=True))


def test_small_bf16_out_heads():
    run = Run(small_wan())
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    run.L.cache_write(ch, x)
    out = run.L.chunk_attention(ch, x)
    torch.cuda.synchronize()
    assert_close(to_host(out)[0], run.oracle()["out"], TOL["bf16"], "out_heads")


@pytest.mark.parametrize("d_nope", [32, 128, 224])
def test_head_widths(d_nope):
    """d_head = 64, 160 and 256 (32 RoPE columns each): the per-head value
    up-projection's 128-wide column tiles come out short, ragged (128 + 32) and
    doubled, with the split row tiles combined as they load; out_heads and y."""
    run = Run(small_wan(d_nope=d_nope, d_head=d_nope + 32), random_gains=True)
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    run.L.cache_write(ch, x)
    out = run.L.chunk_attention(ch, x)
    torch.cuda.synchronize()
    assert_close(to_host(out)[0], run.oracle()["out"], TOL["bf16"], "out_heads")
    full_step(run, check_cache=False)


def test_ring_wraps_around():
    """Window frames 6..10 in a 5-slot ring: slots 1,2,3,4,0 (FIFO, App. D.4)."""
    full_step(Run(small_wan(t0=9)))


def test_partial_window_leaves_other_slots_untouched():
    """3 valid frames of a 5-slot ring: the unwritten slots stay exactly zero and
    only the valid frames are attended."""
    run = Run(small_wan(t0=5, n_valid_frames=3))
    full_step(run)
    ring = to_host(run.L.ring())[0]
    written = {O.ring_slot(f, 5) for f in run.window_ids}
    for slot in range(5):
        rows = ring[slot * run.tpf:(slot + 1) * run.tpf]
        if slot not in written:
            assert np.all(rows == 0), f"slot {slot} was written"
        else:
            assert np.any(rows != 0)


def test_window_is_the_chunk_only():
    full_step(Run(small_wan(t0=0, n_valid_frames=2)))


@pytest.mark.parametrize("dc,dr", [(128, 32), (256, 32), (192, 64)])
def test_latent_and_rope_widths(dc, dr):
    pairs = (6, 5, 5) if dr == 32 else (12, 10, 10)
    full_step(Run(small_wan(d_c=dc, d_rope=dr, d_nope=128 - dr, rope_pairs=pairs)))


def test_sharp_softmax():
    """RMSNorm gain of c^Q x8 (the scale must come after the normalisation, which
    would cancel one on W^Q_down): logits of standard deviation ~8 nats, still
    inside the fast kernel's range, so no row tile is flagged."""
    for s in (small_wan(), long_window()):
        run = Run(s, scale={"g_q": 8.0})
        full_step(run, check_cache=False)
        flags = run.L.overflow_flags(run.chunk())
        assert len(flags) > 0 and not flags.any(), flags


def long_window(**kw):
    """One Wan frame of queries over three frames of keys: 74 row tiles x 74 key
    tiles, so each workgroup's piece spans about 21 key tiles (in a small problem
    every piece is one key tile, whose own max is its reference and nothing can
    overflow)."""
    return W.shape_by_name("wan1.3b-w21").with_(window_frames=3, chunk_frames=1, t0=2,
                                                 n_valid_frames=3, **kw)


@pytest.mark.parametrize("case", ["small", "long", "batch-causal", "sink-read", "dc256"])
def test_exact_path_recomputes_flagged_pieces(case, monkeypatch):
    """The bound of the fast kernel forced down to 2 (MLA_ATTN_OVERFLOW_LIMIT): every
    row sum exceeds it, so every piece of every row tile is recomputed inside the
    attention kernel (a pass for the exact maximum, then the softmax against it) and
    every row tile is flagged, on ordinary data and at the usual
    tolerance, with causal blocks, two requests, a sink with read-time rotation and
    the 32-rows-per-wave d_c = 256 build."""
    monkeypatch.setenv("MLA_ATTN_OVERFLOW_LIMIT", "2")
    shape, batch = {
        "small": (small_wan(), 1),
        "long": (long_window(), 1),
        "batch-causal": (small_wan(t0=6, window_frames=6, chunk_frames=4, n_valid_frames=6,
                                   causal_frames=2), 2),
        "sink-read": (small_wan(rope_at_read=True, sink_frames=1, window_frames=3,
                                chunk_frames=2, t0=12, n_valid_frames=3), 1),
        "dc256": (small_wan(d_c=256), 1),
    }[case]
    run = Run(shape, batch=batch, random_gains=True)
    full_step(run, check_cache=False)
    flags = run.L.overflow_flags(run.chunk())
    assert flags.all(), f"{int((flags == 0).sum())} of {len(flags)} row tiles not flagged"


def test_needle_key_overflows_the_fast_kernel():
    """A needle: one token of the middle frame with x scaled by 64 (exact in bf16),
    so its positional key k^R = W^K_R x, which RMSNorm does not touch, is 64 times
    larger and its scores reach far above the rest.  Pieces that start before its
    key tile see scores more than 64 (base 2) above their reference, so the fast
    kernel recomputes those pieces and flags their row tiles by itself.
    Parity here is the Frobenius relative error alone: with scores this sharp
    (tens of units, base 2), the bf16 rounding of the absorbed query and the keys
    by itself moves single rows by about 1.4e-2 of max|y| in fp64 (computed on the
    CPU for this case), so the max-abs criterion measures the inputs' precision,
    not the path; the exact path itself is held to both criteria on ordinary data
    by the forced-bound test above."""
    run = Run(long_window())
    tpf = run.s.tokens_per_frame
    run.x[:, tpf + 700] *= 64.0
    run.x_store = W.round_to_bf16_bits(run.x)
    run.prefill()
    ch = run.chunk()
    y = run.L.step(ch, run.chunk_tokens())
    torch.cuda.synchronize()
    flags = run.L.overflow_flags(ch)
    assert flags.any(), "no row tile was flagged: the fast kernel did not detect the overflow"
    fro, _ = rel_errors(to_host(y)[0], run.oracle()["y"])
    assert fro <= TOL["bf16"], fro


def test_cache_write_register_staged_path():
    """d_model = 96 (not a multiple of 64) takes the register-staged bf16 cache-write
    kernel instead of the direct-load one; ring and y against the oracle."""
    full_step(Run(small_wan(d_model=96), random_gains=True))


SCORE_FORM_CASES = {
    "small": lambda: small_wan(),
    "causal-blocks": lambda: small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6,
                                       causal_frames=2),
    "sink-read": lambda: small_wan(rope_at_read=True, sink_frames=1, window_frames=3,
                                   chunk_frames=2, t0=12, n_valid_frames=3),
    "dc128": lambda: small_wan(d_c=128, d_rope=32, d_nope=96, rope_pairs=(6, 5, 5)),
    "dc256": lambda: small_wan(d_c=256, d_rope=32, d_nope=96, rope_pairs=(6, 5, 5)),
    "wan1.3b-w21": lambda: W.shape_by_name("wan1.3b-w21"),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", list(SCORE_FORM_CASES))
def test_score_mfma_forms_agree_bitwise(case, monkeypatch):
    """The fast attention kernel issues its score MFMAs as inline asm, and the waits
    before their results are read were counted by hand.  The same kernel with the
    compiler's own MFMA form (MLA_ATTN_SCORE_MFMA=builtin), on the same device inputs
    and in the launch the benchmark times, must give the same bits of y.  A missing
    wait would let a read of S see a stale value, and y would differ.  The cases cover
    the first and the masked last key tile, causal blocks, a gathered window and
    every latent width that uses the asm form.  Both runs are also checked against
    the oracle (sampled query tokens at full size)."""
    s = SCORE_FORM_CASES[case]()
    run = Run(s)
    say(f"case score MFMA forms {case}")
    run.prefill()
    ch, x = run.chunk(), run.chunk_tokens()
    run.L.absorb_query()
    y_asm = run.L.step(ch, x).clone()
    monkeypatch.setenv("MLA_ATTN_SCORE_MFMA", "builtin")
    y_builtin = run.L.step(ch, x).clone()
    monkeypatch.delenv("MLA_ATTN_SCORE_MFMA")
    y_again = run.L.step(ch, x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_asm, y_again)
    assert torch.equal(y_asm, y_builtin), "asm and builtin score MFMAs disagree"
    rows = sample_rows(s) if s.tokens_per_frame > 1000 else None
    ref = run.oracle(query_rows=rows)
    y_h = to_host(y_asm)[0]
    assert_close(y_h if rows is None else y_h[rows], ref["y"], TOL["bf16"], "y")


@pytest.mark.parametrize("t0,read", [(1_000_003, False), (3_000_000_001, False),
                                     (3_000_000_001, True)])
def test_large_absolute_positions(t0, read):
    """A long rollout without the read-time re-indexing: write-time rotation at frame
    indices far beyond what fp32 resolves (at t0 = 10^6 an fp32 product pos * omega is
    off by up to ~0.03 rad, several bf16 steps of the rotated key).  The angle is
    formed and reduced modulo 2 pi in fp64, so every ring element stays within one
    bf16 ulp of the oracle's exact rotation and y within tolerance.  Past 2^31 the
    frame index also exercises the 64-bit position and slot arithmetic; read-time
    rotation there re-indexes to window-local positions."""
    full_step(Run(small_wan(t0=t0, rope_at_read=read), random_gains=True))


def test_batch_of_two_requests():
    full_step(Run(small_wan(t0=6), batch=2))


def test_single_token_frames_single_key():
    """One token per frame and one valid frame: the only key gets weight 1."""
    full_step(Run(small_wan(grid_h=1, grid_w=1, chunk_frames=1, t0=4, n_valid_frames=1)))


def test_single_token_frames_fp32():
    s = W.shape_by_name("tiny-f32").with_(grid_h=1, grid_w=1)
    full_step(Run(s))


@pytest.mark.parametrize("layout", ["split", "split-padded"])
def test_two_tensor_cache(layout):
    """The cache as App. D.4 writes it, two tensors c^KV (B x T x d_c) and k^R
    (B x T x d_rope), here with their own row and request strides: the cache write
    stores into both parts and the attention reads them through the gathered
    window.  Ring contents and y against the oracle."""
    full_step(Run(small_wan(t0=9), random_gains=True, cache_layout=layout))


def test_two_tensor_cache_batch_sink_fp32():
    """Strided two-tensor caches with two requests (batch strides), with a sink frame
    and read-time rotation, and in fp32."""
    full_step(Run(small_wan(t0=6), batch=2, cache_layout="split-padded"))
    full_step(Run(small_wan(rope_at_read=True, sink_frames=1, window_frames=3, chunk_frames=2,
                            t0=12, n_valid_frames=3), cache_layout="split-padded"))
    full_step(Run(W.shape_by_name("tiny-f32"), random_gains=True, cache_layout="split-padded"))


def test_two_tensor_cache_matches_interleaved_bitwise():
    """Gathering a two-tensor ring into the workspace changes nothing but where the
    keys come from: y is bit-identical to the interleaved ring's."""
    ys = []
    for layout in ("interleaved", "split-padded"):
        run = Run(small_wan(t0=8), cache_layout=layout)
        run.prefill()
        y = run.L.step(run.chunk(), run.chunk_tokens())
        torch.cuda.synchronize()
        ys.append(y.clone())
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("read", [False, True])
def test_explicit_rope_frequency_table(read):
    """An explicit per-pair frequency table (drawn at random, an input to both sides
    like the weights), so the comparison does not rest on the derived bands."""
    s = small_wan(t0=9, rope_at_read=read)
    s = s.with_(rope_freq=W.draw_rope_freq(s, seed=4))
    full_step(Run(s, random_gains=True))
    t = W.shape_by_name("tiny-f32")
    full_step(Run(t.with_(rope_freq=W.draw_rope_freq(t, seed=5), rope_at_read=read)))


def test_run_to_run_bitwise_deterministic():
    run = Run(small_wan())
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    y1 = run.L.step(ch, x).clone()
    y2 = run.L.step(ch, x).clone()  # same t0: overwrites the same slots
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_attention_on_oracle_cache():
    """Isolate the attention path: the ring is filled with the oracle's cache
    (rounded to bf16), not with the GPU's cache write."""
    run = Run(small_wan(t0=7))
    ring = run.oracle_ring()
    run.L.cache.copy_(torch.from_numpy(ring[None]).to(torch.bfloat16).cuda())
    ch = run.chunk()
    out = run.L.chunk_attention(ch, run.chunk_tokens())
    torch.cuda.synchronize()
    assert_close(to_host(out)[0], run.oracle()["out"], TOL["bf16"], "out_heads")


# ---------------------------------------------------------------- full-size shapes
def sample_rows(shape, n=48, seed=1):
    rng = np.random.default_rng(seed)
    t = shape.chunk_tokens
    edges = [0, 1, t - 2, t - 1]
    if shape.causal_frames:  # both sides of every block boundary
        step = shape.causal_frames * shape.tokens_per_frame
        edges += [e for k in range(step, t, step) for e in (k - 1, k)]
    rows = np.unique(np.concatenate([rng.choice(t, n, replace=False), edges]))
    return rows


def sampled_full(shape, batch=1):
    run = Run(shape, batch=batch)
    y = full_step(run, check_cache=False, sample=sample_rows(shape))
    # cache: sampled ring rows of every request against the oracle's entries
    rng = np.random.default_rng(2)
    ring = to_host(run.L.ring())
    for b in range(batch):
        ref = run.oracle_ring(b)
        rows = rng.choice(ring.shape[1], 600, replace=False)
        assert_cache_rows(ring[b][rows], ref[rows], "bf16", f"cache sample[b={b}]")
    return run, y


@pytest.mark.timeout(600)
def test_wan13b_layer_full_tensors():
    """Wan-1.3B layer, 3-frame chunk over the 21-frame window, compared in full against
    the oracle -- no sampling: every element of out_heads from mla_chunk_attention
    (4680 x 1536, the unabsorbed query route and per-head W^V_up), of y from mla_step in
    the launch the benchmark times (absorbed query, W^V_up then W_O) and of y with the
    value-absorbed epilogue as well (4680 x 1536 each), and every element of the ring
    (21 slots x 1560 tokens x 224, one bf16 ulp)."""
    s = W.shape_by_name("wan1.3b-w21")
    run = Run(s)
    say(f"case {s.name} full tensors: prefill {len(run.window_ids) - s.chunk_frames} frames")
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    run.L.cache_write(ch, x)
    out = run.L.chunk_attention(ch, x)
    torch.cuda.synchronize()
    out_h = to_host(out)[0]
    run.L.absorb_query()
    y_two = to_host(run.L.step(ch, x))[0]  # writes the chunk's frames again (same values)
    run.L.absorb_value()
    y_abs = to_host(run.L.step(ch, x))[0]
    torch.cuda.synchronize()
    ring = to_host(run.L.ring())[0]
    say("  device done; oracle over all 4680 query tokens ...")
    ref = run.oracle()
    assert out_h.shape == ref["out"].shape == (4680, 1536)
    fro, mx = assert_close(out_h, ref["out"], TOL["bf16"], "out_heads (all elements)")
    say(f"  out_heads: frobenius {fro:.3e}, max {mx:.3e}")
    for name, y_h in (("y, W^V_up then W_O", y_two), ("y, value-absorbed", y_abs)):
        fro, mx = assert_close(y_h, ref["y"], TOL["bf16"], f"{name} (all elements)")
        say(f"  {name}: frobenius {fro:.3e}, max {mx:.3e}")
    ref_ring = run.oracle_ring()
    assert ring.shape == ref_ring.shape == (21 * 1560, 224)
    assert_cache_rows(ring, ref_ring, "bf16", "ring (all 32760 rows)")


def test_wan13b_two_tensor_cache_sampled():
    """Full Wan-1.3B size with the ring held as two tensors (App. D.4's c^KV and k^R):
    sampled query tokens (all heads) and ring rows against the oracle."""
    run = Run(W.shape_by_name("wan1.3b-w21"), cache_layout="split")
    full_step(run, check_cache=False, sample=sample_rows(run.s))
    ring = to_host(run.L.ring())[0]
    rows = np.random.default_rng(2).choice(ring.shape[0], 600, replace=False)
    assert_cache_rows(ring[rows], run.oracle_ring()[rows], "bf16", "two-tensor ring sample")


@pytest.mark.parametrize("name,batch", [("wan1.3b-w21", 3), ("wan1.3b-sink1-w6-t240", 4)])
def test_batched_requests_full_size_sampled(name, batch):
    """Several independent requests in one call, each with its own ring and its own
    tokens, at full Wan-1.3B size: every request is checked on sampled query rows
    and sampled ring rows."""
    sampled_full(W.shape_by_name(name), batch=batch)


@pytest.mark.parametrize("name", ["wan1.3b-w6-t240", "wan1.3b-w42-t240", "wan1.3b-w21-t240-q1"])
def test_window_sweep_sampled(name):
    sampled_full(W.shape_by_name(name))


@pytest.mark.parametrize("name", ["wan1.3b-w21-dc128-dr32", "wan1.3b-w21-dc256-dr32",
                                  "wan1.3b-w21-dc192-dr64"])
def test_latent_width_variants_full_size_sampled(name):
    """The (d_c, d_rope) variants at full Wan-1.3B size, in the launch the sweep times
    (d_c = 256 runs the attention kernel with 32 query rows per wave)."""
    sampled_full(W.shape_by_name(name))

