"""CPU oracle for the VideoMLA latent-KV chunk step.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path: no kernels, headers, helpers,
tables or constants.  Everything is plain NumPy in float64 with no intermediate
rounding; inputs are the exact values of what the GPU receives.

Source: the VideoMLA paper ("VideoMLA: Low-Rank Latent KV Cache for Minute-Scale
Autoregressive Video Diffusion").  Each function names the section and equation
it writes out.  The oracle is the *unabsorbed* training-time definition (§3,
App. D.2-D.4): per-head keys and values are reconstructed explicitly and a
dense softmax is taken over the whole active window.  The absorbed form of
App. E is kept here too, as an independent route used to pin the oracle.

Readings taken where the paper is silent (same numbering as the design notes):
  * RMSNorm: u / sqrt(mean(u^2) + eps) * g, applied to c^KV and c^Q (App. D.2);
    the cache holds the normalised latent.
  * RoPE pair split for d_rope/2 = P pairs: y and x get floor(P/3) pairs each,
    t gets the rest -> (6,5,5) at P=16 (App. D.3).
  * RoPE frequencies: axis group widths of a full-d_head split, D_y = D_x =
    2*floor(d_head/6), D_t = d_head - 2*D_y; pair k of axis a rotates by
    theta^(-2k/D_a) per unit position, k from 0 (the highest-frequency bands,
    §3.2 and App. D.3); theta = 10000.  A layer may instead carry an explicit
    per-pair table (an input, shared with the GPU like the weights), so that
    parity does not rest on this reading.
  * Pair m is channels (2m, 2m+1) = (re, im), axis order t, y, x; the same
    rotation e^{+i*angle} for queries and keys.
  * Position of token n of latent frame f: (t, y, x) = (f, n // grid_w,
    n % grid_w), tokens flattened frame-major then row-major (App. C.1, S=FHW).
  * Keys are rotated at their absolute position when written; the whole valid
    window (the chunk's own frames included) is attended with no mask.
  * Ring buffer: latent frame f lives in slot f mod W (FIFO eviction of whole
    frames, App. D.4).
  * Read-time rotation with a sink (the long-rollout cache of App. D.4-D.5, and
    §3.2 where the cache keeps k^R unrotated): the first S frames keep slots
    0..S-1 for good; frame f >= S lives in slot S + (f - S) mod W.  The attended
    context is the sink frames generated so far followed by the n_valid most
    recent frames, in that order, and its frame i takes temporal coordinate i
    (keys and the query chunk alike); y and x stay as they are.
  * Chunk-causal forward (the training-time pass of §3.3 with the block masks
    of App. D.4): the query chunk is a whole clip (or any run of frames) split
    into blocks of B consecutive frames; a token of block k attends every
    context frame before the chunk, every frame of blocks 0..k, and nothing
    after its block.  B = 0 means no mask: the whole window, as at inference.
"""
import numpy as np

__all__ = [
    "rope_pair_split", "rope_omegas", "rope_frequencies", "rope3d", "rmsnorm", "token_positions",
    "ring_slot", "window_frames", "ring_rows_for_window", "context_times", "visible_keys",
    "cache_entries", "expected_ring", "query_parts", "reconstruct_kv",
    "attention_unabsorbed", "attention_absorbed", "query_absorbed", "value_absorbed_output",
    "output_projection", "step", "chunk_frame_ids", "cache_scalars_per_token",
    "dense_scalars_per_token",
]


# ----------------------------------------------------------------- accounting
def cache_scalars_per_token(d_c, d_rope):
    """Scalars cached per token per layer: the latent plus the shared RoPE key
    (§3.1 and App. E, Eq. 13)."""
    return d_c + d_rope


def dense_scalars_per_token(n_heads, d_head):
    """Scalars a dense per-head KV cache holds per token per layer (App. E, Eq. 14)."""
    return 2 * n_heads * d_head


# ----------------------------------------------------------------- 3D-RoPE
def rope_pair_split(d_rope):
    """(t, y, x) complex pairs for a RoPE subspace of d_rope channels (App. D.3)."""
    p = d_rope // 2
    n_sp = p // 3
    return (p - 2 * n_sp, n_sp, n_sp)


def rope_omegas(d_head, pairs, theta=10000.0):
    """Per-pair angular frequency and axis index.  For axis a the pairs take the
    first (highest-frequency) bands of that axis's group (§3.2, App. D.3)."""
    d_sp = 2 * (d_head // 6)
    widths = (d_head - 2 * d_sp, d_sp, d_sp)
    omegas, axes = [], []
    for axis in range(3):
        for k in range(pairs[axis]):
            omegas.append(float(theta) ** (-2.0 * k / widths[axis]))
            axes.append(axis)
    return np.array(omegas, dtype=np.float64), np.array(axes, dtype=np.int64)


def rope_frequencies(s):
    """Angular frequency and axis of every RoPE pair of a layer.  A layer may carry
    an explicit table (rope_freq, one value per pair in t, y, x order, an input
    like the weights); a missing or all-zero table means the bands derived from
    theta by rope_omegas."""
    om, ax = rope_omegas(s.d_head, s.rope_pairs, s.rope_theta)
    table = getattr(s, "rope_freq", None)
    if table is not None and any(float(v) != 0.0 for v in table):
        if len(table) != len(om):
            raise ValueError(f"rope_freq has {len(table)} entries for {len(om)} pairs")
        om = np.asarray(table, dtype=np.float64)
    return om, ax


def rope3d(v, pos, omegas, axes):
    """Rotate the RoPE subspace (§3.2 Eq. 5-6).  v: (..., 2P); pos: (..., 3)
    integer (t, y, x) broadcastable against v's leading dims."""
    v = np.asarray(v, dtype=np.float64)
    z = v[..., 0::2] + 1j * v[..., 1::2]
    angle = np.asarray(pos, dtype=np.float64)[..., axes] * omegas
    z = z * np.exp(1j * angle)
    out = np.empty_like(v)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def rmsnorm(u, g, eps):
    """RMSNorm applied to c^KV and c^Q before their up-projections (App. D.2)."""
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps) * g


def token_positions(frames, grid_h, grid_w, times=None):
    """(t, y, x) for every token of the given latent frames, frame-major then
    row-major (App. C.1: S = F*H*W).  t is the frame's absolute index, or
    times[frame] when a temporal coordinate per frame is given (App. D.5)."""
    pos = []
    for f in frames:
        t = f if times is None else times[f]
        for n in range(grid_h * grid_w):
            pos.append((t, n // grid_w, n % grid_w))
    return np.array(pos, dtype=np.int64).reshape(-1, 3)


# ----------------------------------------------------------------- ring bookkeeping
def ring_slot(frame, window_frames, sink_frames=0):
    """Ring slot of an absolute latent frame (App. D.4): FIFO over whole frames;
    the first sink_frames frames keep their own slots and are never evicted."""
    if frame < sink_frames:
        return frame
    return sink_frames + (frame - sink_frames) % window_frames


def window_frames(t0, chunk_frames, n_valid_frames, sink_frames=0):
    """Frames attended once the chunk [t0, t0+C) is written, in context order:
    the sink frames generated so far, then the n_valid most recent frames
    (App. D.4).  Without a sink this is the chronological window."""
    last = t0 + chunk_frames - 1
    local = list(range(last - n_valid_frames + 1, last + 1))
    if sink_frames and local and local[0] < sink_frames:
        raise ValueError("local frames overlap the sink")
    return list(range(min(sink_frames, last + 1))) + local


def ring_rows_for_window(t0, chunk_frames, n_valid_frames, window_frames_, tpf, sink_frames=0):
    """Ring rows holding the attended frames, in context order."""
    rows = []
    for f in window_frames(t0, chunk_frames, n_valid_frames, sink_frames):
        base = ring_slot(f, window_frames_, sink_frames) * tpf
        rows.extend(range(base, base + tpf))
    return np.array(rows, dtype=np.int64)


def context_times(frames, rope_at_read):
    """Temporal RoPE coordinate of each attended frame: its absolute index when
    keys are rotated as they are written; its index in the attended context when
    the cache keeps k^R unrotated and the window is re-indexed on assembly
    (§3.2 Eq. 5, App. D.5)."""
    return {f: (i if rope_at_read else f) for i, f in enumerate(frames)}


def visible_keys(s, window_ids, chunk_ids):
    """How many context keys each chunk token may attend, as a prefix of the
    context (keys are in context order, the chunk's frames last).  With causal
    blocks of B frames (App. D.4: tokens see their own 3-frame chunk and earlier
    ones, never a later one; §3.3 trains with these block masks), token i of the
    chunk lies in block (i // tpf) // B and sees the context up to that block's
    last frame.  Without blocks every token sees the whole window."""
    tpf = s.tokens_per_frame
    n = len(chunk_ids) * tpf
    total = len(window_ids) * tpf
    bf = getattr(s, "causal_frames", 0)
    if not bf:
        return np.full(n, total, dtype=np.int64)
    first = window_ids.index(chunk_ids[0])
    block = (np.arange(n) // tpf) // bf
    return np.minimum((first + (block + 1) * bf) * tpf, total)


# ----------------------------------------------------------------- the layer
def _head_rows(w, h, width):
    return w[h * width:(h + 1) * width]


def cache_entries(s, w, x, frames, times=None):
    """Per-token cache state (c^KV, k^R) for tokens x of the given frames.
    c = RMSNorm(W_down^KV x) (§3.1 Eq. 1, App. D.2); k^R = W_R^K x (§3.2 Eq. 5);
    the rotated key k^rope = RoPE3D(k^R) at the token's position (absolute t, or
    times[frame]).  x: (N, d).
    Returns (c (N, d_c), k_r_raw (N, d_rope), k_rope (N, d_rope))."""
    x = np.asarray(x, dtype=np.float64)
    c = rmsnorm(x @ w["w_kv_down"].T, w["g_kv"], s.rms_eps)
    k_r = x @ w["w_kr"].T
    om, ax = rope_frequencies(s)
    pos = token_positions(frames, s.grid_h, s.grid_w, times)
    return c, k_r, rope3d(k_r, pos, om, ax)


def expected_ring(s, w, x, frames, ring=None):
    """Ring contents after writing the tokens x of the given frames.  Row
    slot(f)*tpf + n holds [c^KV | RoPE3D(k^R)] when keys are rotated at write,
    [c^KV | k^R] when they are rotated on window assembly (§3.2, App. D.4-D.5)."""
    tpf = s.tokens_per_frame
    sink = getattr(s, "sink_frames", 0)
    at_read = getattr(s, "rope_at_read", False)
    if ring is None:
        ring = np.zeros(((sink + s.window_frames) * tpf, s.d_c + s.d_rope))
    c, k_r, k_rope = cache_entries(s, w, x, frames)
    for i, f in enumerate(frames):
        base = ring_slot(f, s.window_frames, sink) * tpf
        ring[base:base + tpf, :s.d_c] = c[i * tpf:(i + 1) * tpf]
        ring[base:base + tpf, s.d_c:] = (k_r if at_read else k_rope)[i * tpf:(i + 1) * tpf]
    return ring


def query_parts(s, w, x, frames, times=None):
    """Per-head queries (§3.1 Eq. 3-4, §3.2 Eq. 6): c^Q = RMSNorm(W_down^Q x),
    q^nope_h = W_up,h^Q c^Q, q^rope_h = RoPE3D(W_R,h^Q c^Q) at the token's
    position (absolute t, or times[frame] in the re-indexed context, App. D.5).
    Returns (c_q (N, d_q), q_nope (N, H, d_nope), q_rope (N, H, d_rope))."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    c_q = rmsnorm(x @ w["w_q_down"].T, w["g_q"], s.rms_eps)
    q_nope = (c_q @ w["w_q_up"].T).reshape(n, s.n_heads, s.d_nope)
    q_r = (c_q @ w["w_qr"].T).reshape(n, s.n_heads, s.d_rope)
    om, ax = rope_frequencies(s)
    pos = token_positions(frames, s.grid_h, s.grid_w, times)[:, None, :]
    return c_q, q_nope, rope3d(q_r, pos, om, ax)


def reconstruct_kv(s, w, c):
    """Per-head content keys and values from the cached latent (§3.1 Eq. 2):
    k^nope_{j,h} = W_up,h^K c_j, v_{j,h} = W_up,h^V c_j."""
    n = c.shape[0]
    k_nope = (c @ w["w_k_up"].T).reshape(n, s.n_heads, s.d_nope)
    v = (c @ w["w_v_up"].T).reshape(n, s.n_heads, s.d_head)
    return k_nope, v


def attention_unabsorbed(s, w, q_nope, q_rope, c, k_rope, block=1024, visible=None):
    """Chunk attention as defined in §3.3 Eq. 7: per head, score =
    (q^nope.k^nope + q^rope.k^rope) / sqrt(d_nope + d_rope) over every window
    token, softmax over the window, weighted sum of v_{j,h}; heads concatenated.
    q_nope (N, H, d_nope), q_rope (N, H, d_rope), c (M, d_c), k_rope (M, d_rope).
    visible (N,) optionally limits query i to keys 0..visible[i]-1 (the block
    mask of the chunk-causal forward).  Returns out (N, H*d_head)."""
    k_nope, v = reconstruct_kv(s, w, c)
    n = q_nope.shape[0]
    m = c.shape[0]
    scale = 1.0 / np.sqrt(s.d_nope + s.d_rope)
    out = np.empty((n, s.n_heads, s.d_head))
    for h in range(s.n_heads):
        kn = k_nope[:, h, :]
        vh = v[:, h, :]
        for i0 in range(0, n, block):
            i1 = min(n, i0 + block)
            sc = (q_nope[i0:i1, h, :] @ kn.T + q_rope[i0:i1, h, :] @ k_rope.T) * scale
            if visible is not None:
                sc[np.arange(m)[None, :] >= np.asarray(visible[i0:i1])[:, None]] = -np.inf
            sc = sc - sc.max(axis=1, keepdims=True)
            a = np.exp(sc)
            a /= a.sum(axis=1, keepdims=True)
            out[i0:i1, h, :] = a @ vh
    return out.reshape(n, s.n_heads * s.d_head)


def output_projection(w, out):
    """Heads mixed by the output projection W_O (§3.3)."""
    return out @ w["w_o"].T


def value_absorbed_output(s, w, h):
    """B_h = W_O,h W_up,h^V (App. E Eq. 10-11): the columns of W_O that mix head h,
    times that head's value up-projection; (d, d_c)."""
    return w["w_o"][:, h * s.d_head:(h + 1) * s.d_head] @ _head_rows(w["w_v_up"], h, s.d_head)


def query_absorbed(s, w, h):
    """A_h = (W_up,h^Q)^T W_up,h^K (App. E Eq. 8-9): the query-side absorption, so
    that the content score is (c^Q)^T A_h c^KV; (d_q, d_c)."""
    return _head_rows(w["w_q_up"], h, s.d_nope).T @ _head_rows(w["w_k_up"], h, s.d_nope)


def attention_absorbed(s, w, c_q, q_rope, c, k_rope):
    """The inference reparameterisation of App. E, written as the paper states it:
    content score (c^Q)^T A_h c^KV with A_h = (W_up,h^Q)^T W_up,h^K (Eq. 8-9), the
    RoPE term kept separate (Eq. 12), and the output sum_h B_h sum_j a_j c_j with
    B_h = W_O,h W_up,h^V (Eq. 10-11).  Returns y (N, d)."""
    n = c_q.shape[0]
    scale = 1.0 / np.sqrt(s.d_nope + s.d_rope)
    y = np.zeros((n, s.d_model))
    for h in range(s.n_heads):
        a_h = query_absorbed(s, w, h)
        b_h = value_absorbed_output(s, w, h)
        sc = (c_q @ a_h @ c.T + q_rope[:, h, :] @ k_rope.T) * scale
        sc = sc - sc.max(axis=1, keepdims=True)
        a = np.exp(sc)
        a /= a.sum(axis=1, keepdims=True)
        y += (a @ c) @ b_h.T
    return y


def chunk_frame_ids(s):
    """Absolute indices of the chunk's latent frames: t0 .. t0 + C - 1."""
    return list(range(s.t0, s.t0 + s.chunk_frames))


def _frame_tokens(tokens, f):
    x = tokens(f) if callable(tokens) else tokens[f]
    return np.asarray(x, dtype=np.float64)


def step(s, w, tokens, query_rows=None):
    """One chunk step for one batch element.  The attended frames are derived
    here from the chunk (t0, C), the window length n_valid and the sink
    (window_frames, App. D.4): the sink frames generated so far, then the local
    window chronologically, the chunk's frames last.  tokens maps an absolute
    frame index to that frame's (tpf, d) tokens (a dict, or a callable).  Cache
    entries are formed for every attended frame, queries for the chunk, then
    attention and W_O.  Keys and queries are rotated at absolute t, or at their
    frame's index in the context when the shape rotates on window assembly
    (App. D.5).  query_rows optionally restricts the queries to a subset of chunk
    tokens (indices into the chunk).  With causal blocks (the training-time
    forward over a clip) each query sees the context only up to the end of its
    block.  Returns dict(out=(Nq, H*d_h), y=(Nq, d), c, k_rope, window_ids)."""
    window_ids = window_frames(s.t0, s.chunk_frames, s.n_valid_frames,
                               getattr(s, "sink_frames", 0))
    chunk_ids = chunk_frame_ids(s)
    x_window = np.concatenate([_frame_tokens(tokens, f) for f in window_ids])
    times = context_times(window_ids, getattr(s, "rope_at_read", False))
    c, _, k_rope = cache_entries(s, w, x_window, window_ids, times)
    x_chunk = np.concatenate([_frame_tokens(tokens, f) for f in chunk_ids])
    _, q_nope, q_rope = query_parts(s, w, x_chunk, chunk_ids, times)
    visible = visible_keys(s, window_ids, chunk_ids)
    if query_rows is not None:
        q_nope, q_rope = q_nope[query_rows], q_rope[query_rows]
        visible = visible[query_rows]
    masked = bool(getattr(s, "causal_frames", 0))
    out = attention_unabsorbed(s, w, q_nope, q_rope, c, k_rope,
                               visible=visible if masked else None)
    return {"out": out, "y": output_projection(w, out), "c": c, "k_rope": k_rope,
            "window_ids": window_ids}
