"""GPU parity of the value-absorbed output (VideoMLA App. E Eq. 10-11): the device
computes B_h = W_O,h W^V_up,h once per weight set, and mla_step then maps the
latent attention output to the model width with one GEMM.  B against the oracle's
B_h, and the step's y against the oracle's unabsorbed step, at the usual
tolerances, through the C ABI."""
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


def absorbed(run):
    run.L.absorb_value()
    return run


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
