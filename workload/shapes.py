"""Layer shapes and chunk/window geometry of the workloads.

Shapes follow the VideoMLA paper (Low-Rank Latent KV Cache for Minute-Scale
Autoregressive Video Diffusion): Table 4 and App. D.1-D.2 give the Wan-1.3B
layer (d=1536, 12 heads, d_h=128 split 96 NoPE + 32 RoPE, d_c=192, d_q=768,
30x52 tokens per latent frame, 3-frame chunks, 21-frame clips).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MLAShape:
    name: str
    d_model: int
    n_heads: int
    d_head: int
    d_nope: int
    d_rope: int
    d_c: int
    d_q: int
    rope_pairs: tuple          # complex pairs on the (t, y, x) axes
    grid_h: int
    grid_w: int
    window_frames: int         # W: ring capacity in latent frames
    chunk_frames: int          # C: latent frames per query chunk
    t0: int                    # absolute index of the chunk's first frame
    n_valid_frames: int        # frames attended after the chunk is written
    dtype: str                 # "bf16" or "f32"
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    batch: int = 1
    rope_at_read: bool = False # cache keeps k^R unrotated; rotation on window assembly
    sink_frames: int = 0       # leading frames kept for good (read-time rotation only)
    causal_frames: int = 0     # chunk-causal blocks of this many chunk frames (0: no mask)
    rope_freq: tuple = None    # explicit radians per position for each RoPE pair (t, y, x
                               # order), fp32 values; None: the bands derived from rope_theta

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def window_tokens(self) -> int:
        return len(self.window_frame_ids) * self.tokens_per_frame

    @property
    def cache_frames(self) -> int:
        """Frame slots of the ring: the sink slots plus the W local slots."""
        return self.sink_frames + self.window_frames

    @property
    def chunk_frame_ids(self):
        return list(range(self.t0, self.t0 + self.chunk_frames))

    @property
    def window_frame_ids(self):
        """Attended frames in context order: the sink frames generated so far,
        then the n_valid most recent frames (the chunk's own among them)."""
        last = self.t0 + self.chunk_frames - 1
        sinks = list(range(min(self.sink_frames, last + 1)))
        return sinks + list(range(last - self.n_valid_frames + 1, last + 1))

    def with_(self, **kw) -> "MLAShape":
        return replace(self, **kw)


def _wan(name, d_c=192, d_rope=32, window=21, chunk=3, t0=18, n_valid=None,
         pairs=None, dtype="bf16", rope_at_read=False, sink=0, causal=0):
    if pairs is None:
        pairs = (6, 5, 5) if d_rope == 32 else (12, 10, 10)
    return MLAShape(name=name, d_model=1536, n_heads=12, d_head=128,
                    d_nope=128 - d_rope, d_rope=d_rope, d_c=d_c, d_q=768,
                    rope_pairs=pairs, grid_h=30, grid_w=52, window_frames=window,
                    chunk_frames=chunk, t0=t0,
                    n_valid_frames=window if n_valid is None else n_valid,
                    dtype=dtype, rope_at_read=rope_at_read, sink_frames=sink,
                    causal_frames=causal)


SHAPES = {
    # Tiny fp32 layer: hidden 64, 2 heads of 32 (24 NoPE + 8 RoPE), d_c 16,
    # 4x4 tokens per frame, 3 cached frames plus 1 query frame.
    "tiny-f32": MLAShape(name="tiny-f32", d_model=64, n_heads=2, d_head=32,
                         d_nope=24, d_rope=8, d_c=16, d_q=32, rope_pairs=(2, 1, 1),
                         grid_h=4, grid_w=4, window_frames=4, chunk_frames=1, t0=3,
                         n_valid_frames=4, dtype="f32"),
    # Wan-1.3B-shaped layer, 3-frame chunk over a 21-frame window (chunk included).
    "wan1.3b-w21": _wan("wan1.3b-w21"),
}
for _w in (6, 12, 21, 42):
    # window sweep with the newest frame at absolute index 240
    SHAPES[f"wan1.3b-w{_w}-t240"] = _wan(f"wan1.3b-w{_w}-t240", window=_w, t0=238)
SHAPES["wan1.3b-w21-t240-q1"] = _wan("wan1.3b-w21-t240-q1", window=21, chunk=1, t0=240)
for _dc, _dr in ((128, 32), (256, 32), (192, 64)):
    SHAPES[f"wan1.3b-w21-dc{_dc}-dr{_dr}"] = _wan(f"wan1.3b-w21-dc{_dc}-dr{_dr}", d_c=_dc,
                                                  d_rope=_dr)


# Keys kept unrotated and rotated at window-local positions on assembly (§3.2,
# App. D.5): the 21-frame window, and the long-rollout cache of one sink frame plus
# the six most recent frames with the chunk at frames 238-240 (App. D.4).
SHAPES["wan1.3b-w21-read"] = _wan("wan1.3b-w21-read", rope_at_read=True)
SHAPES["wan1.3b-sink1-w6-t240"] = _wan("wan1.3b-sink1-w6-t240", window=6, t0=238,
                                       rope_at_read=True, sink=1)

# Training-time forward (§3.3, App. D.4): the whole 21-frame clip is the query
# chunk, written to the cache in one call, with chunk-causal blocks of 3 frames.
SHAPES["wan1.3b-clip21-causal3"] = _wan("wan1.3b-clip21-causal3", chunk=21, t0=0, causal=3)


def attended_pairs(s: MLAShape) -> int:
    """(query token, key token) pairs one request attends, per head: every chunk
    token sees the whole window, or with causal blocks the context up to the end
    of its block."""
    tpf = s.tokens_per_frame
    nk = s.window_tokens
    if not s.causal_frames:
        return s.chunk_tokens * nk
    before = nk - s.chunk_tokens
    blocks = -(-s.chunk_frames // s.causal_frames)
    total = 0
    for k in range(blocks):
        frames = min(s.causal_frames, s.chunk_frames - k * s.causal_frames)
        total += frames * tpf * min(before + (k + 1) * s.causal_frames * tpf, nk)
    return total


def shape_by_name(name: str) -> MLAShape:
    return SHAPES[name]
