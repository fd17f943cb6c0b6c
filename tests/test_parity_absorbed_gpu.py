"""GPU parity of the absorbed weight forms of VideoMLA App. E: B_h = W_O,h W^V_up,h
(Eq. 10-11), with which mla_step maps the latent attention output to the model width
in one GEMM, and W_qk,h = (W^K_up,h)^T W^Q_up,h (Eq. 8-9), stacked with W^Q_R,h so
that each absorbed query row is one GEMM from c^Q.  Each prepared weight against the oracle's, and the
steps' y against the oracle's unabsorbed step, at the usual tolerances, through the
C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W
from latent_kv_attention_down_amd.layer import to_host
from parity_helpers import TOL, Run, assert_close
from test_parity_gpu import full_step, sample_rows, small_wan

pytestmark = pytest.mark.gpu


def oracle_b(run):
    s = run.s
    return np.concatenate([O.value_absorbed_output(s, run.w, h) for h in range(s.n_heads)], axis=1)


@pytest.mark.parametrize("name", ["tiny-f32", "wan1.3b-w21"])
def test_absorbed_weights(name):
    run = Run(W.shape_by_name(name))
    w_b = run.L.absorb_value()
    torch.cuda.synchronize()
    s = run.s
    assert tuple(w_b.shape) == (s.d_model, s.n_heads * s.d_c)
    assert_close(to_host(w_b), oracle_b(run), TOL[s.dtype], "B")


def oracle_wqlat(run):
    """Per head: A_h^T (the oracle's A_h of App. E Eq. 8-9, transposed), then W^Q_R,h."""
    s = run.s
    parts = []
    for h in range(s.n_heads):
        parts.append(O.query_absorbed(s, run.w, h).T)
        parts.append(run.w["w_qr"][h * s.d_rope:(h + 1) * s.d_rope])
    return np.concatenate(parts, axis=0)


@pytest.mark.parametrize("name", ["tiny-f32", "wan1.3b-w21"])
def test_query_absorbed_weights(name):
    run = Run(W.shape_by_name(name))
    w_qlat = run.L.absorb_query()
    torch.cuda.synchronize()
    s = run.s
    assert tuple(w_qlat.shape) == (s.n_heads * (s.d_c + s.d_rope), s.d_q)
    assert_close(to_host(w_qlat), oracle_wqlat(run), TOL[s.dtype], "W_qlat")


def absorbed(run, query=False):
    run.L.absorb_value()
    if query:
        run.L.absorb_query()
    return run


def query_absorbed(run):
    run.L.absorb_query()
    return run


def test_query_absorbed_step_small_bf16():
    full_step(query_absorbed(Run(small_wan(), random_gains=True)))


def test_both_absorbed_step_fp32():
    full_step(absorbed(Run(W.shape_by_name("tiny-f32"), random_gains=True), query=True))


def test_both_absorbed_step_causal_sink():
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=4, chunk_frames=4, t0=8,
                  n_valid_frames=4, causal_frames=2)
    full_step(absorbed(Run(s, batch=2), query=True))


def test_both_absorbed_step_full_size_sampled():
    s = W.shape_by_name("wan1.3b-w21")
    full_step(absorbed(Run(s), query=True), check_cache=False, sample=sample_rows(s))


def test_absorbed_step_small_bf16():
    full_step(absorbed(Run(small_wan(), random_gains=True)))


def test_absorbed_step_fp32():
    full_step(absorbed(Run(W.shape_by_name("tiny-f32"), random_gains=True)))


def test_absorbed_step_causal_blocks():
    s = small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6, causal_frames=2)
    full_step(absorbed(Run(s)))


def test_absorbed_step_sink_read_rotation():
    s = small_wan(rope_at_read=True, sink_frames=1, window_frames=3, chunk_frames=2, t0=12,
                  n_valid_frames=3)
    full_step(absorbed(Run(s, batch=2)))


def test_absorbed_step_full_size_sampled():
    """The Wan-1.3B C1 step with the absorbed output, on sampled tokens."""
    s = W.shape_by_name("wan1.3b-w21")
    full_step(absorbed(Run(s)), check_cache=False, sample=sample_rows(s))


def test_absorbed_and_two_stage_steps_agree():
    """Both epilogues on the same device inputs give the same y within the bf16
    tolerance (they differ only in where the bf16 roundings fall)."""
    run = Run(small_wan(t0=7))
    run.prefill()
    ch = run.chunk()
    x = run.chunk_tokens()
    y2 = run.L.step(ch, x).clone()
    run.L.absorb_value()
    y1 = run.L.step(ch, x)
    torch.cuda.synchronize()
    assert_close(to_host(y1)[0], to_host(y2)[0], TOL["bf16"], "absorbed vs two-stage")


@pytest.mark.parametrize("grid,t0", [((30, 52), None), ((1, 1560), None),
                                     ((30, 52), 3_000_000_018)])
def test_absorbed_query_full_size_sampled(grid, t0):
    """Full Wan-1.3B size with the absorbed query (App. E Eq. 8-9): y of mla_step (the
    query GEMM rotates its RoPE columns in its tiles and shares its launch with the
    cache write) and out_heads of mla_chunk_attention (the query GEMM alone), sampled
    query tokens against the oracle.  On the 30 x 52 grid the tiles take the RoPE cos/sin
    from a per-tile table; on a 1 x 1560 grid a pair spans more positions than that table
    holds, so the tiles rotate position by position.  At frame 3e9 the table's angles
    (frame index times frequency, reduced in fp64) are checked far past fp32 and 2^31."""
    s = W.shape_by_name("wan1.3b-w21").with_(grid_h=grid[0], grid_w=grid[1])
    if t0 is not None:
        s = s.with_(t0=t0)
    run = query_absorbed(Run(s))
    rows = sample_rows(s)
    full_step(run, check_cache=False, sample=rows)
    out = run.L.chunk_attention(run.chunk(), run.chunk_tokens())
    torch.cuda.synchronize()
    ref = run.oracle(query_rows=rows)
    assert_close(to_host(out)[0][rows], ref["out"], TOL["bf16"], "out_heads")


def test_absorbed_query_two_requests_full_size_sampled():
    """Two requests at full Wan-1.3B size with the absorbed query: the query GEMM (407
    tiles) runs alone, rotating its RoPE columns in its tiles, before the cache write."""
    s = W.shape_by_name("wan1.3b-w21")
    full_step(query_absorbed(Run(s, batch=2)), check_cache=False, sample=sample_rows(s))
