"""mla_step_static, the entry point that allocates nothing (its scratch is a
static device array of the library), against mla_step with a caller workspace:
through the C ABI, two calls in a row -- the full Wan-1.3B chunk (3 frames over the
21-frame window), then a smaller layer -- each bit-identical to mla_step on the
same inputs and within the bf16 tolerance of the oracle.  The second call reuses
the array the first one left behind."""
import numpy as np
import pytest
import torch

import workload as W
import latent_kv_attention_down_amd as mla
from latent_kv_attention_down_amd.layer import to_host
from parity_helpers import TOL, Run, assert_close, say

pytestmark = pytest.mark.gpu


def _small():
    return W.shape_by_name("wan1.3b-w21").with_(grid_h=6, grid_w=10, window_frames=5,
                                                 chunk_frames=2, t0=9, n_valid_frames=5)


@pytest.mark.timeout(600)
def test_static_scratch_step_matches_workspace_step():
    big = W.shape_by_name("wan1.3b-w21")
    for i, (shape, absorbed) in enumerate(((big, True), (_small(), False))):
        say(f"call {i + 1}: {shape.name} {shape.grid_h}x{shape.grid_w} C={shape.chunk_frames} "
            f"W={shape.window_frames} absorbed={absorbed}")
        run = Run(shape, random_gains=True, seed=3 + i)
        if absorbed:
            run.L.absorb_value()
            run.L.absorb_query()
        run.prefill()
        ch = run.chunk()
        x = run.chunk_tokens()
        y_ws = run.L.step(ch, x)  # caller workspace
        y_st = torch.empty_like(y_ws)
        mla.step_static(run.L.cfg, run.L.weights, ch, x, run.L.cache_desc, y_st)
        torch.cuda.synchronize()
        assert torch.equal(y_st, y_ws), "static-scratch step differs from the workspace step"
        rows = None if shape is not big else np.unique(np.concatenate(
            [np.random.default_rng(i).choice(shape.chunk_tokens, 48, replace=False),
             [0, shape.chunk_tokens - 1]]))
        ref = run.oracle(query_rows=rows)
        got = to_host(y_st)[0]
        fro, mx = assert_close(got if rows is None else got[rows], ref["y"], TOL["bf16"], "y")
        say(f"  equal to mla_step; oracle frobenius {fro:.3e}, max {mx:.3e}")
