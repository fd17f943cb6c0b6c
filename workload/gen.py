"""Seeded draws of weights and per-frame inputs.

Recipe: NumPy PCG64; weight tensor k of layer l comes from SeedSequence([seed, l, k])
as N(0, 1/fan_in) with fan_in the number of input columns; the input of absolute
latent frame f of layer l comes from SeedSequence([seed, l, 10000 + f]) as N(0, 1),
so a frame has the same tokens in every window and every call.  RMSNorm gains are
ones unless ``random_gains`` is set (then N(1, 0.1^2)).  Values are drawn in fp64
and rounded once to the storage type; the rounded values are what both sides use.
"""
import numpy as np

# (name, rows, cols, fan_in) for each weight, in draw order k = 0, 1, ...
WEIGHT_NAMES = ("w_kv_down", "w_kr", "w_q_down", "w_q_up", "w_qr", "w_k_up",
                "w_v_up", "w_o", "g_kv", "g_q")


def _weight_dims(s):
    nh = s.n_heads
    return {
        "w_kv_down": (s.d_c, s.d_model),
        "w_kr": (s.d_rope, s.d_model),
        "w_q_down": (s.d_q, s.d_model),
        "w_q_up": (nh * s.d_nope, s.d_q),
        "w_qr": (nh * s.d_rope, s.d_q),
        "w_k_up": (nh * s.d_nope, s.d_c),
        "w_v_up": (nh * s.d_head, s.d_c),
        "w_o": (s.d_model, nh * s.d_head),
    }


def round_to_bf16_bits(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) and return the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _store(a, dtype):
    """Round fp64 draws to the storage type; returns (storage array, exact fp64 view)."""
    if dtype == "bf16":
        bits = round_to_bf16_bits(a)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    f = np.asarray(a, dtype=np.float32)
    return f, f.astype(np.float64)


def draw_weights(s, layer=0, seed=0, random_gains=False, scale=None):
    """Return (stored, exact): dicts of storage arrays (uint16 bf16 bits or float32)
    and their exact fp64 values.  ``scale`` optionally multiplies named weights
    before rounding (e.g. {"w_q_down": 8.0} gives sharp softmax logits)."""
    dims = _weight_dims(s)
    stored, exact = {}, {}
    for k, name in enumerate(WEIGHT_NAMES):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, k])))
        if name in ("g_kv", "g_q"):
            n = s.d_c if name == "g_kv" else s.d_q
            a = rng.normal(1.0, 0.1, size=n) if random_gains else np.ones(n)
        else:
            rows, cols = dims[name]
            a = rng.normal(0.0, 1.0, size=(rows, cols)) / np.sqrt(cols)
        if scale and name in scale:
            a = a * scale[name]
        stored[name], exact[name] = _store(a, s.dtype)
    return stored, exact


def draw_frames(s, frames, layer=0, seed=0, batch=None):
    """Inputs for the given absolute latent frames: shape (B, len(frames)*tpf, d).
    Batch element b uses seed + 7919*b so requests differ.  Every (request, frame)
    has its own seed, so the frames are drawn and rounded on a few threads (NumPy
    releases the GIL for both); the values do not depend on the thread count."""
    B = s.batch if batch is None else batch
    tpf = s.tokens_per_frame
    n = len(frames)
    stored = np.empty((B, n * tpf, s.d_model), dtype=np.uint16 if s.dtype == "bf16"
                      else np.float32)
    exact = np.empty((B, n * tpf, s.d_model), dtype=np.float64)

    def one(job):
        b, i = divmod(job, n)
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([seed + 7919 * b, layer, 10000 + frames[i]])))
        st, ex = _store(rng.normal(0.0, 1.0, size=(tpf, s.d_model)), s.dtype)
        stored[b, i * tpf:(i + 1) * tpf] = st
        exact[b, i * tpf:(i + 1) * tpf] = ex

    jobs = B * n
    if jobs * tpf * s.d_model < (1 << 20):
        for j in range(jobs):
            one(j)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(8, jobs)) as ex:
            list(ex.map(one, range(jobs)))
    return stored, exact


def draw_rope_freq(s, seed=0, low=0.02, high=1.5):
    """A random explicit RoPE frequency table (one fp32 value per pair, uniform in
    [low, high) radians per position), drawn from SeedSequence([seed, 20000]) and
    rounded to fp32 -- an input given to both sides like the weights."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 20000])))
    v = rng.uniform(low, high, size=s.d_rope // 2).astype(np.float32)
    return tuple(float(t) for t in v)


class FrameTokens:
    """Tokens of any absolute latent frame on demand, drawn with the per-frame seed
    of draw_frames and cached: frames(f) -> (stored (tpf, d), exact fp64 (tpf, d))
    for request b.  Calling the object returns the exact values, so it can be
    handed to anything that asks for a frame's tokens."""

    def __init__(self, s, layer=0, seed=0, b=0):
        self.s, self.layer, self.seed, self.b = s, layer, seed, b
        self._cache = {}

    def frames(self, f):
        if f not in self._cache:
            st, ex = draw_frames(self.s, [f], layer=self.layer, seed=self.seed + 7919 * self.b,
                                 batch=1)
            self._cache[f] = (st[0], ex[0])
        return self._cache[f]

    def __call__(self, f):
        return self.frames(f)[1]
