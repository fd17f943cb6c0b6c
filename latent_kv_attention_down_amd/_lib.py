"""ctypes binding of libmla.so (include/mla.h): argument marshalling only.

Every entry point of the C ABI has a Python function of the same name (without
the ``mla_`` prefix).  Tensors are torch device tensors; their data pointers and
torch's current HIP stream are handed to the library, which does all the work.
Loading fails loudly when the library has not been built.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED = 0, -1, -2
MLA_ERR_ALIGNMENT, MLA_ERR_WORKSPACE, MLA_ERR_HIP = -3, -4, -5
MLA_BF16, MLA_F32 = 0, 1
MLA_ROPE_AT_WRITE, MLA_ROPE_AT_READ = 0, 1

# Every function include/mla.h declares, with (restype, argtypes).
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class Config(ctypes.Structure):
    _fields_ = [("d_model", _i32), ("n_heads", _i32), ("d_head", _i32), ("d_nope", _i32),
                ("d_rope", _i32), ("d_c", _i32), ("d_q", _i32), ("rope_pairs", _i32 * 3),
                ("rope_theta", ctypes.c_float), ("rope_freq", ctypes.c_float * 64),
                ("grid_h", _i32), ("grid_w", _i32),
                ("window_frames", _i32), ("dtype", _i32), ("rms_eps", ctypes.c_float),
                ("rope_mode", _i32), ("sink_frames", _i32)]


class Cache(ctypes.Structure):
    _fields_ = [("c_kv", _vp), ("k_r", _vp), ("c_kv_row_stride", _i64), ("k_r_row_stride", _i64),
                ("c_kv_batch_stride", _i64), ("k_r_batch_stride", _i64)]


class Weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_kv_down", "w_kr", "g_kv", "w_q_down", "g_q", "w_q_up",
                                   "w_qr", "w_k_up", "w_v_up", "w_o", "w_b", "w_qlat")]


class Chunk(ctypes.Structure):
    _fields_ = [("batch", _i32), ("chunk_frames", _i32), ("t0", _i64), ("n_valid_frames", _i32),
                ("causal_frames", _i32)]


_P = ctypes.POINTER
SIGNATURES = {
    "mla_validate": (ctypes.c_int, [_P(Config), _P(Chunk)]),
    "mla_workspace_bytes": (_sz, [_P(Config), _P(Chunk)]),
    "mla_cache_bytes": (_sz, [_P(Config), _i32]),
    "mla_cache_interleaved": (ctypes.c_int, [_P(Config), _i32, _vp, _P(Cache)]),
    "mla_cache_write": (ctypes.c_int, [_P(Config), _P(Weights), _P(Chunk), _vp, _P(Cache), _vp]),
    "mla_chunk_attention": (ctypes.c_int, [_P(Config), _P(Weights), _P(Chunk), _vp, _P(Cache), _vp,
                                           _vp, _sz, _vp]),
    "mla_step": (ctypes.c_int, [_P(Config), _P(Weights), _P(Chunk), _vp, _P(Cache), _vp, _vp, _sz,
                                _vp]),
    "mla_latent_attention": (ctypes.c_int, [_P(Config), _P(Chunk), _vp, _P(Cache), _vp, _vp, _sz,
                                            _vp]),
    "mla_step_static": (ctypes.c_int, [_P(Config), _P(Weights), _P(Chunk), _vp, _P(Cache), _vp,
                                       _vp]),
    "mla_value_absorbed_weights": (ctypes.c_int, [_P(Config), _P(Weights), _vp, _vp]),
    "mla_query_absorbed_weights": (ctypes.c_int, [_P(Config), _P(Weights), _vp, _vp]),
    "mla_set_timing_events": (None, [_vp, _vp]),
    "mla_attention_grid": (ctypes.c_int, [_P(Config), _P(Chunk)]),
    "mla_overflow_flags": (ctypes.c_int, [_P(Config), _P(Chunk), _P(_sz), _P(_i64)]),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load(path=None):
    """Load libmla.so once; raise if it is missing (there is no fallback path).
    MLA_LIBRARY names another build of the same library (for instance the host-
    sanitized one the ABI tests run against)."""
    global _lib
    if path is None:
        path = os.environ.get("MLA_LIBRARY") or LIB_PATH
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m latent_kv_attention_down_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MLAError(RuntimeError):
    def __init__(self, status, where):
        lib = load()
        super().__init__(f"{where}: {lib.mla_status_string(status).decode()} "
                         f"({lib.mla_last_error().decode()})")
        self.status = status


def _check(status, where):
    if status != MLA_OK:
        raise MLAError(status, where)


def make_config(shape, dtype=None):
    """Build an mla_config from any object with the shape fields (d_model, n_heads,
    d_head, d_nope, d_rope, d_c, d_q, rope_pairs, rope_theta, grid_h, grid_w,
    window_frames, dtype ('bf16'/'f32'), rms_eps)."""
    dt = shape.dtype if dtype is None else dtype
    c = Config()
    for f in ("d_model", "n_heads", "d_head", "d_nope", "d_rope", "d_c", "d_q", "grid_h",
              "grid_w", "window_frames"):
        setattr(c, f, int(getattr(shape, f)))
    for i, v in enumerate(shape.rope_pairs):
        c.rope_pairs[i] = int(v)
    c.rope_theta = float(shape.rope_theta)
    for i, v in enumerate(getattr(shape, "rope_freq", None) or ()):
        c.rope_freq[i] = float(v)
    c.rms_eps = float(shape.rms_eps)
    c.dtype = MLA_BF16 if dt == "bf16" else MLA_F32
    c.rope_mode = MLA_ROPE_AT_READ if getattr(shape, "rope_at_read", False) else MLA_ROPE_AT_WRITE
    c.sink_frames = int(getattr(shape, "sink_frames", 0))
    return c


def make_chunk(batch, chunk_frames, t0, n_valid_frames, causal_frames=0):
    return Chunk(int(batch), int(chunk_frames), int(t0), int(n_valid_frames), int(causal_frames))


def make_weights(tensors):
    """tensors: dict name -> device tensor (or None) for the mla_weights fields."""
    w = Weights()
    for name, _ in Weights._fields_:
        t = tensors.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    return w


def _ptr(t):
    return None if t is None else t.data_ptr()


def interleaved_cache(cfg, batch, base):
    """The mla_cache descriptor of the interleaved layout over one buffer (a device
    tensor of mla_cache_bytes(cfg, batch) bytes, or a device address)."""
    c = Cache()
    addr = base if isinstance(base, int) or base is None else base.data_ptr()
    _check(load().mla_cache_interleaved(ctypes.byref(cfg), int(batch), addr, ctypes.byref(c)),
           "mla_cache_interleaved")
    return c


def split_cache(c_kv, k_r):
    """The mla_cache descriptor of two separate device tensors, c_kv (B, rows, >= d_c)
    and k_r (B, rows, >= d_rope) with unit column stride (any row and batch stride)."""
    c = Cache()
    c.c_kv, c.k_r = c_kv.data_ptr(), k_r.data_ptr()
    c.c_kv_row_stride, c.k_r_row_stride = c_kv.stride(1), k_r.stride(1)
    c.c_kv_batch_stride, c.k_r_batch_stride = c_kv.stride(0), k_r.stride(0)
    return c


def _cache(cfg, cache):
    """A Cache struct as given, or the interleaved descriptor of a (B, rows, d_c +
    d_rope) device tensor."""
    if isinstance(cache, Cache):
        return ctypes.byref(cache)
    if cache is None:
        return None
    return ctypes.byref(interleaved_cache(cfg, cache.shape[0], cache))


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def validate(cfg, chunk):
    return load().mla_validate(ctypes.byref(cfg), ctypes.byref(chunk))


def workspace_bytes(cfg, chunk):
    return load().mla_workspace_bytes(ctypes.byref(cfg), ctypes.byref(chunk))


def cache_bytes(cfg, batch):
    return load().mla_cache_bytes(ctypes.byref(cfg), int(batch))


def cache_write(cfg, weights, chunk, x, cache, stream=None):
    _check(load().mla_cache_write(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(chunk),
                                  _ptr(x), _cache(cfg, cache), _stream(stream)), "mla_cache_write")


def chunk_attention(cfg, weights, chunk, x, cache, out_heads, workspace, stream=None):
    _check(load().mla_chunk_attention(ctypes.byref(cfg), ctypes.byref(weights),
                                      ctypes.byref(chunk), _ptr(x), _cache(cfg, cache),
                                      _ptr(out_heads),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "mla_chunk_attention")


def step(cfg, weights, chunk, x, cache, y, workspace, stream=None):
    _check(load().mla_step(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(chunk), _ptr(x),
                           _cache(cfg, cache), _ptr(y), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_step")


def step_static(cfg, weights, chunk, x, cache, y, stream=None):
    _check(load().mla_step_static(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(chunk),
                                  _ptr(x), _cache(cfg, cache), _ptr(y), _stream(stream)),
           "mla_step_static")


MLA_STATIC_SCRATCH_BYTES = 256 << 20


def value_absorbed_weights(cfg, weights, w_b, stream=None):
    _check(load().mla_value_absorbed_weights(ctypes.byref(cfg), ctypes.byref(weights), _ptr(w_b),
                                             _stream(stream)), "mla_value_absorbed_weights")


def query_absorbed_weights(cfg, weights, w_qlat, stream=None):
    _check(load().mla_query_absorbed_weights(ctypes.byref(cfg), ctypes.byref(weights),
                                             _ptr(w_qlat), _stream(stream)),
           "mla_query_absorbed_weights")


def latent_attention(cfg, chunk, q_lat, cache, o_lat, workspace, stream=None):
    _check(load().mla_latent_attention(ctypes.byref(cfg), ctypes.byref(chunk), _ptr(q_lat),
                                       _cache(cfg, cache), _ptr(o_lat), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "mla_latent_attention")


def set_timing_events(ev_start, ev_stop):
    load().mla_set_timing_events(ev_start, ev_stop)


def attention_grid(cfg, chunk):
    return load().mla_attention_grid(ctypes.byref(cfg), ctypes.byref(chunk))


def overflow_flags(cfg, chunk):
    """(byte offset, count) of the int32 overflow flags in the workspace."""
    off, n = _sz(), _i64()
    _check(load().mla_overflow_flags(ctypes.byref(cfg), ctypes.byref(chunk), ctypes.byref(off),
                                     ctypes.byref(n)), "mla_overflow_flags")
    return off.value, n.value


def status_string(status):
    return load().mla_status_string(int(status)).decode()


def last_error():
    return load().mla_last_error().decode()
