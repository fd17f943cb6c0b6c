"""mla_step and mla_step_static captured in a HIP graph.  A step makes no device
allocation, memset or host synchronisation (every buffer it clears is cleared by a
kernel), so a caller can capture it.  Each replay of the captured step, with eager
steps run between the replays, must give the same bits of y as the eager call on
the same inputs; the eager call is itself checked against the oracle."""
import numpy as np
import pytest
import torch

import workload as W
import latent_kv_attention_down_amd as mla
from latent_kv_attention_down_amd.layer import to_host
from parity_helpers import TOL, Run, assert_close, say

pytestmark = pytest.mark.gpu

CASES = {
    "small": lambda: W.shape_by_name("wan1.3b-w21").with_(grid_h=6, grid_w=10, window_frames=5,
                                                            chunk_frames=2, t0=9, n_valid_frames=5),
    "wan1.3b-w21": lambda: W.shape_by_name("wan1.3b-w21"),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("entry", ["mla_step", "mla_step_static"])
@pytest.mark.parametrize("case", list(CASES))
def test_step_replays_from_a_graph(case, entry):
    s = CASES[case]()
    run = Run(s, random_gains=True, seed=5)
    run.L.absorb_query()
    run.prefill()
    L = run.L
    ch, x = run.chunk(), run.chunk_tokens()
    y = L.new_out(ch, s.d_model)
    ws = L.workspace(ch)
    say(f"case {case} through {entry}: eager step, capture, replays")

    def step():
        if entry == "mla_step":
            mla.step(L.cfg, L.weights, ch, x, L.cache_desc, y, ws)
        else:
            mla.step_static(L.cfg, L.weights, ch, x, L.cache_desc, y)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    rows = None if s.tokens_per_frame < 1000 else np.arange(0, s.chunk_tokens, 97)
    ref = run.oracle(query_rows=rows)
    got = to_host(y_eager)[0]
    assert_close(got if rows is None else got[rows], ref["y"], TOL["bf16"], "eager y")

    # one step on a side stream first, as stream capture expects, then the capture
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r} differs from the eager step"
        step()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"eager step after replay {r} differs"
    say("  3 replays and the eager steps between them all equal")
