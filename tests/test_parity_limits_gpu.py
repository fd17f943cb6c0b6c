"""GPU checks at the size limit of the bf16 path, by properties that hold at any size
(no oracle pass over millions of keys): one request's ring just under 2 GiB (the
32-bit byte offsets of the key-tile loads), attended by one query row through
mla_latent_attention.  Every key is the same latent except one "needle" whose score
is 30 (base 2) above the rest, placed at the first or the last ring row; the softmax
weights are then 1 for the n - 1 plain keys and 2^30 for the needle, so the output is
(n - 1) c + 2^30 c' over n - 1 + 2^30, in closed form.  With a single query row the
persistent grid cuts that row tile into one piece per workgroup, which also
exercises the merge of hundreds of split records."""
import numpy as np
import pytest
import torch

import workload as W
from latent_kv_attention_down_amd.layer import DeviceLayer, to_host

pytestmark = pytest.mark.gpu

DK = 224
ROWS = (1 << 31) // (DK * 2) - 1  # ring rows: the largest bf16 ring under 2 GiB


def tiny_layer():
    base = W.shape_by_name("wan1.3b-w21")
    return base.with_(d_model=32, n_heads=1, d_q=32, grid_h=1, grid_w=1, window_frames=ROWS,
                      chunk_frames=1, t0=ROWS - 1, n_valid_frames=ROWS)


@pytest.fixture(scope="module")
def layer():
    s = tiny_layer()
    stored, _ = W.draw_weights(s)
    L = DeviceLayer(s, stored)
    assert L.cache.numel() * 2 < (1 << 31) and L.cache.numel() * 2 > (1 << 31) - 1024
    yield s, L
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("needle_row", [0, ROWS - 1])
def test_needle_at_the_ends_of_a_2gib_ring(layer, needle_row):
    s, L = layer
    plain = torch.zeros(DK, dtype=torch.bfloat16, device="cuda")
    plain[0] = 1.0                      # c = e_0, score 0
    needle = torch.zeros(DK, dtype=torch.bfloat16, device="cuda")
    needle[1] = 1.0                     # c' = e_1, score 30
    L.cache[0].copy_(plain.expand(ROWS, DK))
    L.cache[0, needle_row].copy_(needle)
    q = torch.zeros((1, 1, DK), dtype=torch.bfloat16, device="cuda")
    q[0, 0, 1] = 30.0
    ch = L.chunk(1, ROWS - 1, ROWS)
    o = L.latent_attention(ch, q)
    torch.cuda.synchronize()
    got = to_host(o)[0, 0]
    n = ROWS - 1
    w_needle = 2.0 ** 30
    expect0 = n / (n + w_needle)
    expect1 = w_needle / (n + w_needle)
    assert abs(got[0] - expect0) <= 2e-2 * expect0 + 1e-6, (got[0], expect0)
    assert abs(got[1] - expect1) <= 2e-2 * expect1, (got[1], expect1)
    assert np.all(got[2:] == 0)


def test_uniform_keys_over_a_2gib_ring(layer):
    """Identical keys: uniform weights, so the output is the common latent itself."""
    s, L = layer
    row = torch.zeros(DK, dtype=torch.bfloat16, device="cuda")
    row[:192] = torch.linspace(-1, 1, 192, device="cuda").to(torch.bfloat16)
    row[192:] = 0.5
    L.cache[0].copy_(row.expand(ROWS, DK))
    q = torch.full((1, 1, DK), 0.01, dtype=torch.bfloat16, device="cuda")
    o = L.latent_attention(L.chunk(1, ROWS - 1, ROWS), q)
    torch.cuda.synchronize()
    got = to_host(o)[0, 0]
    ref = to_host(row[:192])
    assert np.abs(got - ref).max() <= 2e-2 * np.abs(ref).max(), np.abs(got - ref).max()
