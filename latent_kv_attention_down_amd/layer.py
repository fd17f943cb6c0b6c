"""Device memory for one MLA layer: weights, ring cache and workspace as torch
tensors, with the ctypes structs the C ABI takes.  PyTorch is used only to own
device memory and to name the stream."""
import numpy as np
import torch

from . import _lib

WEIGHT_FIELDS = ("w_kv_down", "w_kr", "g_kv", "w_q_down", "g_q", "w_q_up", "w_qr", "w_k_up",
                 "w_v_up", "w_o")


def to_device(arr, dtype, device="cuda"):
    """Host array -> device tensor.  bf16 arrays are given as uint16 bit patterns."""
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 arrays are passed as uint16 bit patterns")
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.astype(np.float32)).to(device)


def to_host(t):
    """Device tensor -> float64 numpy (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


class WorkspacePool:
    """One device workspace for several layers that are stepped in turn on one
    stream (a backbone's attention layers): each call takes the same buffer,
    grown to the largest size asked for."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        return self.buf


class DeviceLayer:
    """One layer's weights and ring cache on the device.  cache_layout picks how the
    ring is held: "interleaved" (one tensor, rows [c^KV | k], read in place by the
    attention kernels), "split" (the two tensors c^KV and k^R) or "split-padded"
    (the two tensors inside larger allocations, so rows and requests have strides
    of their own); the library is handed the matching mla_cache descriptor."""

    def __init__(self, shape, stored_weights, batch=1, device="cuda", pool=None,
                 cache_layout="interleaved"):
        self.shape = shape
        self.dtype = shape.dtype
        self.tdtype = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        self.device = device
        self.cfg = _lib.make_config(shape)
        self.tensors = {k: to_device(stored_weights[k], self.dtype, device)
                        for k in WEIGHT_FIELDS if stored_weights.get(k) is not None}
        self.weights = _lib.make_weights(self.tensors)
        self.batch = batch
        tpf = shape.grid_h * shape.grid_w
        frames = getattr(shape, "sink_frames", 0) + shape.window_frames
        rows = frames * tpf
        self.cache_layout = cache_layout
        if cache_layout == "interleaved":
            self.cache = torch.zeros((batch, rows, shape.d_c + shape.d_rope),
                                     dtype=self.tdtype, device=device)
            assert self.cache.numel() * self.cache.element_size() == _lib.cache_bytes(self.cfg,
                                                                                     batch)
            self.cache_desc = _lib.interleaved_cache(self.cfg, batch, self.cache)
        elif cache_layout in ("split", "split-padded"):
            pad = 8 if cache_layout == "split-padded" else 0
            cbuf = torch.zeros((batch, rows + pad, shape.d_c + pad), dtype=self.tdtype,
                               device=device)
            kbuf = torch.zeros((batch, rows + 2 * pad, shape.d_rope + 2 * pad), dtype=self.tdtype,
                               device=device)
            self._bufs = (cbuf, kbuf)
            self.c_kv = cbuf[:, :rows, :shape.d_c]
            self.k_r = kbuf[:, :rows, :shape.d_rope]
            self.cache = None
            self.cache_desc = _lib.split_cache(self.c_kv, self.k_r)
        else:
            raise ValueError(f"unknown cache layout {cache_layout!r}")
        self.pool = pool if pool is not None else WorkspacePool(device)

    def absorb_value(self):
        """Compute B = [B_1 .. B_nh] (B_h = W_O,h W^V_up,h) on the device and make
        step() project the latent attention output with it."""
        s = self.shape
        w_b = torch.empty((s.d_model, s.n_heads * s.d_c), dtype=self.tdtype, device=self.device)
        _lib.value_absorbed_weights(self.cfg, self.weights, w_b)
        self.tensors["w_b"] = w_b
        self.weights = _lib.make_weights(self.tensors)
        return w_b

    def absorb_query(self):
        """Compute the latent query projection (per head (W^K_up,h)^T W^Q_up,h, then
        W^Q_R,h) on the device and make the step build the absorbed query with it."""
        s = self.shape
        w_qlat = torch.empty((s.n_heads * (s.d_c + s.d_rope), s.d_q), dtype=self.tdtype,
                             device=self.device)
        _lib.query_absorbed_weights(self.cfg, self.weights, w_qlat)
        self.tensors["w_qlat"] = w_qlat
        self.weights = _lib.make_weights(self.tensors)
        return w_qlat

    def ring(self):
        """The ring as one (B, rows, d_c + d_rope) device tensor (a copy for the
        split layouts)."""
        if self.cache is not None:
            return self.cache
        return torch.cat([self.c_kv, self.k_r], dim=-1)

    def chunk(self, chunk_frames, t0, n_valid_frames, causal_frames=0):
        return _lib.make_chunk(self.batch, chunk_frames, t0, n_valid_frames, causal_frames)

    def workspace(self, chunk):
        n = _lib.workspace_bytes(self.cfg, chunk)
        if n == 0:
            raise _lib.MLAError(_lib.validate(self.cfg, chunk), "mla_workspace_bytes")
        return self.pool.get(n)

    def overflow_flags(self, chunk):
        """The attention's overflow flags left in the workspace by the last call
        (one per row tile; nonzero: recomputed against the exact maximum), as a host array."""
        off, n = _lib.overflow_flags(self.cfg, chunk)
        ws = self.workspace(chunk)
        return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()

    def tokens(self, x_host):
        return to_device(x_host, self.dtype, self.device)

    def new_out(self, chunk, width):
        tpf = self.shape.grid_h * self.shape.grid_w
        return torch.empty((self.batch, chunk.chunk_frames * tpf, width), dtype=self.tdtype,
                           device=self.device)

    def cache_write(self, chunk, x):
        _lib.cache_write(self.cfg, self.weights, chunk, x, self.cache_desc)

    def chunk_attention(self, chunk, x):
        s = self.shape
        out = self.new_out(chunk, s.n_heads * s.d_head)
        _lib.chunk_attention(self.cfg, self.weights, chunk, x, self.cache_desc, out,
                             self.workspace(chunk))
        return out

    def step(self, chunk, x):
        y = self.new_out(chunk, self.shape.d_model)
        _lib.step(self.cfg, self.weights, chunk, x, self.cache_desc, y, self.workspace(chunk))
        return y

    def latent_attention(self, chunk, q_lat):
        s = self.shape
        o = torch.empty((q_lat.shape[0], q_lat.shape[1], s.d_c), dtype=self.tdtype,
                        device=self.device)
        _lib.latent_attention(self.cfg, chunk, q_lat, self.cache_desc, o, self.workspace(chunk))
        return o
