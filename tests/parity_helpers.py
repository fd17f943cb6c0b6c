"""Shared helpers of the GPU parity tests: run a layer through the C ABI on seeded
inputs and compute the oracle's answer on the same inputs."""
import sys

import numpy as np

import oracle as O
import workload as W

TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = np.abs(d).max() / np.abs(ref).max()
    return fro, mx


def assert_close(got, ref, tol, what):
    fro, mx = rel_errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert fro <= tol and mx <= tol, f"{what}: frobenius rel {fro:.3e}, max rel {mx:.3e} > {tol}"
    return fro, mx


def bf16_ulp(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.maximum(a, 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def assert_cache_rows(got, ref, dtype, what):
    """Every element within one bf16 ulp of the exact value (plus a tiny absolute
    allowance for fp32 summation order on near-zero results); fp32 mode: 1e-5."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    if dtype == "bf16":
        bound = bf16_ulp(ref) + 1e-5 * scale
    else:
        bound = 1e-5 * scale
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements outside bound, worst " \
                          f"{np.max(np.abs(got - ref) - bound):.3e}"


class Run:
    """A layer on the GPU plus the exact inputs the oracle uses."""

    def __init__(self, shape, seed=0, random_gains=False, scale=None, batch=1, layer=0,
                 pool=None, cache_layout="interleaved"):
        from latent_kv_attention_down_amd.layer import DeviceLayer
        self.s = shape
        self.batch = batch
        self.stored, self.w = W.draw_weights(shape, layer=layer, seed=seed,
                                             random_gains=random_gains, scale=scale)
        self.L = DeviceLayer(shape, self.stored, batch=batch, pool=pool, cache_layout=cache_layout)
        self.seed = seed
        self.layer = layer
        # the frames to draw and prefill are the ones the oracle says are attended
        self.window_ids = O.window_frames(shape.t0, shape.chunk_frames, shape.n_valid_frames,
                                          shape.sink_frames)
        self.chunk_ids = O.chunk_frame_ids(shape)
        xs, xe = W.draw_frames(shape, self.window_ids, layer=layer, seed=seed, batch=batch)
        self.x_store, self.x = xs, xe
        tpf = shape.tokens_per_frame
        self.tpf = tpf
        first = self.window_ids.index(self.chunk_ids[0])
        self.chunk_slice = slice(first * tpf, (first + shape.chunk_frames) * tpf)

    def prefill(self):
        """Write the window's frames that precede the chunk, one frame per call."""
        for i, f in enumerate(self.window_ids):
            if f >= self.chunk_ids[0]:
                break
            ch = self.L.chunk(1, f, 1)
            xt = self.L.tokens(self.x_store[:, i * self.tpf:(i + 1) * self.tpf])
            self.L.cache_write(ch, xt)

    def chunk(self):
        return self.L.chunk(self.s.chunk_frames, self.s.t0, self.s.n_valid_frames,
                            self.s.causal_frames)

    def chunk_tokens(self):
        return self.L.tokens(self.x_store[:, self.chunk_slice])

    def frame_tokens(self, b=0):
        """Exact tokens of request b by absolute frame, as written to the GPU."""
        return {f: self.x[b][i * self.tpf:(i + 1) * self.tpf]
                for i, f in enumerate(self.window_ids)}

    def oracle(self, b=0, query_rows=None):
        return O.step(self.s, self.w, self.frame_tokens(b), query_rows=query_rows)

    def oracle_ring(self, b=0):
        return O.expected_ring(self.s, self.w, self.x[b], self.window_ids)
