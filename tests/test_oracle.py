"""Pins for the CPU oracle (no GPU).  Each pin ties the oracle to something other
than itself: numbers the VideoMLA paper prints, identities the paper states,
library routines, closed forms, and brute force on tiny inputs.  The mutation
tests at the end plant plausible mistakes in the oracle and check that at least
one pin catches each of them."""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting.json")


def small_wan(**kw):
    """Wan-1.3B head geometry on a small grid so the fp64 oracle runs in seconds."""
    base = W.shape_by_name("wan1.3b-w21").with_(grid_h=3, grid_w=5, window_frames=4,
                                                 chunk_frames=1, t0=3, n_valid_frames=4,
                                                 dtype="f32")
    return base.with_(**kw)


def window_ids(s):
    """The attended frames as the oracle derives them (sink frames, then the local
    window), from the chunk, the window length and the sink."""
    return O.window_frames(s.t0, s.chunk_frames, s.n_valid_frames, s.sink_frames)


def layer_inputs(s, seed=0, random_gains=True):
    _, w = W.draw_weights(s, seed=seed, random_gains=random_gains)
    ids = window_ids(s)
    _, x = W.draw_frames(s, ids, seed=seed)
    return w, ids, x[0]


def by_frame(s, ids, x):
    """Frame index -> its tokens, for tokens x laid out frame after frame in ids."""
    tpf = s.tokens_per_frame
    return {f: x[i * tpf:(i + 1) * tpf] for i, f in enumerate(ids)}


# ---------------------------------------------------------------- pin bodies
# Written as functions of the oracle module so the mutation tests can re-run
# them against a deliberately broken copy.

def pin_accounting(o):
    """P-1: closed-form cache accounting against the numbers the paper prints."""
    g = json.load(open(GOLDEN))
    c = o.cache_scalars_per_token(192, 32)
    d = o.dense_scalars_per_token(12, 128)
    assert c == g["cache_scalars_per_token"]["value"]
    assert d == g["dense_scalars_per_token"]["value"]
    assert round(100 * (1 - c / d), 1) == g["reduction_percent"]["value"]
    assert round(d / c, 1) == g["reduction_factor"]["value"]
    dw = g["dense_window_scalars_billion"]
    n = dw["frames"] * dw["tokens_per_frame"] * dw["layers"] * d
    assert round(n / 1e9, 2) == dw["value"]
    assert round(n * 2 / 1e9, 1) == g["dense_window_gb_bf16"]["value"]
    scd = g["scd_reduction_percent"]
    assert round(100 * (1 - scd["cached_layers"] / scd["layers"]), 1) == scd["value"]
    ratio = scd["cached_layers"] * d / (scd["layers"] * c)
    assert round(ratio, 1) == g["videomla_vs_scd_factor"]["value"]
    t5 = g["table5a_memory_ratio"]
    for dc, v in zip(t5["d_c"], t5["value"]):
        assert round(d / o.cache_scalars_per_token(dc, t5["d_rope"]), 2) == v
    assert tuple(o.rope_pair_split(32)) == tuple(g["rope_pairs_default"]["value"])
    assert g["tokens_per_frame"]["value"] == 30 * 52
    assert g["clip_tokens"]["value"] == 21 * 30 * 52


def pin_absorbed(o, s=None):
    """P-2: App. E states the absorbed form computes the same attention; the
    oracle's unabsorbed step must equal Eq. 8-12 evaluated through A_h and B_h."""
    s = s or small_wan()
    w, ids, x = layer_inputs(s)
    r = o.step(s, w, by_frame(s, ids, x))
    tpf = s.tokens_per_frame
    c_q, _, q_rope = o.query_parts(s, w, x[-s.chunk_frames * tpf:], s.chunk_frame_ids)
    y2 = o.attention_absorbed(s, w, c_q, q_rope, r["c"], r["k_rope"])
    err = np.abs(y2 - r["y"]).max() / np.abs(r["y"]).max()
    assert err < 1e-12, err


def pin_sdpa(o, s=None):
    """P-5: the score/softmax/value sum equals torch's fp64 scaled-dot-product
    attention over explicitly concatenated per-head [nope; rope] queries and keys
    (§3.3 Eq. 7 written as a dense attention layer, App. D.3)."""
    s = s or small_wan()
    w, ids, x = layer_inputs(s)
    r = o.step(s, w, by_frame(s, ids, x))
    tpf = s.tokens_per_frame
    _, q_nope, q_rope = o.query_parts(s, w, x[-s.chunk_frames * tpf:], s.chunk_frame_ids)
    k_nope, v = o.reconstruct_kv(s, w, r["c"])
    m = k_nope.shape[0]
    q = np.concatenate([q_nope, q_rope], axis=-1).transpose(1, 0, 2)[None]
    k_rope_h = np.broadcast_to(r["k_rope"][:, None, :], (m, s.n_heads, s.d_rope))
    k = np.concatenate([k_nope, k_rope_h], axis=-1).transpose(1, 0, 2)[None]
    vv = v.transpose(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q)), torch.from_numpy(np.ascontiguousarray(k)),
        torch.from_numpy(np.ascontiguousarray(vv))).numpy()
    ref = ref[0].transpose(1, 0, 2).reshape(-1, s.n_heads * s.d_head)
    err = np.abs(ref - r["out"]).max() / np.abs(ref).max()
    assert err < 1e-12, err


def brute_force_y(s, w, x, ids, chunk_ids, token, times=None):
    """One output row of the layer with explicit scalar loops only, for tiny
    shapes (§3.1 Eq. 1-4, §3.2 Eq. 5-6, §3.3 Eq. 7, App. D.2-D.3).  times maps a
    frame to its temporal RoPE coordinate (default: the absolute index)."""
    tpf = s.grid_h * s.grid_w
    d = s.d_model

    def mv(mat, vec, r0, nrows):
        return [sum(mat[r0 + r][k] * vec[k] for k in range(len(vec))) for r in range(nrows)]

    def norm(u, g):
        ms = sum(t * t for t in u) / len(u)
        return [u[k] / math.sqrt(ms + s.rms_eps) * g[k] for k in range(len(u))]

    # frequency bands: group widths 2*floor(d_h/6) for y and x, the rest for t
    dsp = 2 * (s.d_head // 6)
    width = [s.d_head - 2 * dsp, dsp, dsp]
    pair_axis, pair_k = [], []
    for a in range(3):
        for k in range(s.rope_pairs[a]):
            pair_axis.append(a)
            pair_k.append(k)

    def rot(vec, f, n):
        p = (f if times is None else times[f], n // s.grid_w, n % s.grid_w)
        out = list(vec)
        for m in range(len(vec) // 2):
            ang = p[pair_axis[m]] * s.rope_theta ** (-2.0 * pair_k[m] / width[pair_axis[m]])
            re, im = vec[2 * m], vec[2 * m + 1]
            out[2 * m] = re * math.cos(ang) - im * math.sin(ang)
            out[2 * m + 1] = re * math.sin(ang) + im * math.cos(ang)
        return out

    keys = []
    for fi, f in enumerate(ids):
        for n in range(tpf):
            xj = [x[fi * tpf + n][k] for k in range(d)]
            c = norm(mv(w["w_kv_down"], xj, 0, s.d_c), w["g_kv"])
            kr = rot(mv(w["w_kr"], xj, 0, s.d_rope), f, n)
            keys.append((c, kr))
    fq = chunk_ids[token // tpf]
    nq = token % tpf
    row = ids.index(fq) * tpf + nq
    xi = [x[row][k] for k in range(d)]
    cq = norm(mv(w["w_q_down"], xi, 0, s.d_q), w["g_q"])
    out = []
    for h in range(s.n_heads):
        qn = mv(w["w_q_up"], cq, h * s.d_nope, s.d_nope)
        qr = rot(mv(w["w_qr"], cq, h * s.d_rope, s.d_rope), fq, nq)
        scores, vals = [], []
        for c, kr in keys:
            kn = mv(w["w_k_up"], c, h * s.d_nope, s.d_nope)
            sc = sum(qn[t] * kn[t] for t in range(s.d_nope)) + sum(qr[t] * kr[t] for t in range(s.d_rope))
            scores.append(sc / math.sqrt(s.d_nope + s.d_rope))
            vals.append(mv(w["w_v_up"], c, h * s.d_head, s.d_head))
        mx = max(scores)
        e = [math.exp(t - mx) for t in scores]
        z = sum(e)
        out.extend(sum(e[j] * vals[j][t] for j in range(len(keys))) / z for t in range(s.d_head))
    return [sum(w["w_o"][r][k] * out[k] for k in range(len(out))) for r in range(s.d_model)]


def tiny_brute_shape():
    return W.MLAShape(name="brute", d_model=12, n_heads=2, d_head=14, d_nope=2, d_rope=12,
                      d_c=3, d_q=5, rope_pairs=(2, 2, 2), grid_h=2, grid_w=3, window_frames=3,
                      chunk_frames=2, t0=5, n_valid_frames=3, dtype="f32")


def pin_bruteforce(o):
    """Brute force: the vectorised oracle equals scalar loops on a tiny layer
    whose RoPE pairs cover all three axes and two frequency bands each."""
    s = tiny_brute_shape()
    w, ids, x = layer_inputs(s, seed=3)
    r = o.step(s, w, by_frame(s, ids, x))
    for token in (0, 4, 7, 11):
        yb = np.array(brute_force_y(s, w, x, ids, s.chunk_frame_ids, token))
        err = np.abs(yb - r["y"][token]).max() / np.abs(yb).max()
        assert err < 1e-12, (token, err)


def pin_rope(o):
    """P-3: RoPE3D preserves norms, is the identity at position 0, and depends
    only on relative positions: q(p+D).k(p'+D) = q(p).k(p') for any integer
    shift D per axis (§3.2; App. D.5 relies on this for re-indexing)."""
    rng = np.random.default_rng(7)
    for d_head, d_rope in ((128, 32), (128, 64), (32, 8), (14, 12)):
        pairs = o.rope_pair_split(d_rope)
        assert sum(pairs) == d_rope // 2
        om, ax = o.rope_omegas(d_head, pairs)
        assert len(om) == d_rope // 2
        for a in range(3):  # highest band of every axis rotates one radian per step
            sel = om[ax == a]
            if len(sel):
                assert sel[0] == 1.0 and np.all(np.diff(sel) < 0)
        v = rng.normal(size=(50, d_rope))
        k = rng.normal(size=(50, d_rope))
        p = rng.integers(0, 300, size=(50, 3))
        p2 = rng.integers(0, 300, size=(50, 3))
        rv = o.rope3d(v, p, om, ax)
        assert np.allclose(np.linalg.norm(rv, axis=1), np.linalg.norm(v, axis=1), rtol=1e-14)
        assert np.array_equal(o.rope3d(v, np.zeros((50, 3), dtype=int), om, ax), v)
        shift = rng.integers(-100, 100, size=(1, 3))
        d1 = np.sum(o.rope3d(v, p, om, ax) * o.rope3d(k, p2, om, ax), axis=1)
        d2 = np.sum(o.rope3d(v, p + shift, om, ax) * o.rope3d(k, p2 + shift, om, ax), axis=1)
        assert np.allclose(d1, d2, rtol=1e-10, atol=1e-10)
        # and it is not trivially position-free: moving one side changes the score
        d3 = np.sum(o.rope3d(v, p + shift, om, ax) * o.rope3d(k, p2, om, ax), axis=1)
        assert not np.allclose(d1, d3)
    # complex-pair rotation equals an explicit 2x2 rotation of channels (2m, 2m+1)
    om, ax = o.rope_omegas(128, (6, 5, 5))
    v = rng.normal(size=32)
    pos = np.array([17, 4, 29])
    out = o.rope3d(v, pos, om, ax)
    for m in range(16):
        th = pos[ax[m]] * om[m]
        rmat = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
        assert np.allclose(out[2 * m:2 * m + 2], rmat @ v[2 * m:2 * m + 2], rtol=1e-13, atol=1e-13)


def pin_positions(o):
    """Token order S = F*H*W (App. C.1): token n of frame f sits at
    (f, n // grid_w, n % grid_w); 30x52 = 1560 tokens per latent frame (App. D.1)."""
    pos = o.token_positions([5, 6], 30, 52)
    assert pos.shape == (3120, 3)
    assert tuple(pos[0]) == (5, 0, 0) and tuple(pos[51]) == (5, 0, 51)
    assert tuple(pos[52]) == (5, 1, 0) and tuple(pos[1559]) == (5, 29, 51)
    assert tuple(pos[1560]) == (6, 0, 0)


def pin_sink_context(o):
    """Long-rollout cache of App. D.4: one sink latent frame kept for good plus the
    six most recent frames, FIFO over whole frames.  Explicit cases, and a deque
    simulation of a 100-frame rollout written one 3-frame chunk at a time."""
    assert o.window_frames(238, 3, 6, sink_frames=1) == [0, 235, 236, 237, 238, 239, 240]
    assert o.window_frames(0, 3, 2, sink_frames=1) == [0, 1, 2]
    assert o.window_frames(18, 3, 21) == list(range(0, 21))
    assert [o.ring_slot(f, 6, 1) for f in (0, 1, 6, 7, 12, 13)] == [0, 1, 6, 1, 6, 1]
    assert o.ring_slot(240, 6, 1) == 6 and o.ring_slot(240, 21) == 240 % 21
    sink, W, tpf = 1, 6, 4
    local = collections.deque(maxlen=W)
    slots = {}
    for t0 in range(0, 99, 3):
        for f in range(t0, t0 + 3):
            slots[o.ring_slot(f, W, sink)] = f
            if f >= sink:
                local.append(f)
        present = sorted(slots.values())
        assert present == list(range(sink)) + list(local)
        ctx = o.window_frames(t0, 3, len(local), sink_frames=sink)
        assert ctx == list(range(sink)) + list(local)
        rows = o.ring_rows_for_window(t0, 3, len(local), W, tpf, sink_frames=sink)
        assert [slots[int(r) // tpf] for r in rows[::tpf]] == ctx


def pin_read_rotation(o):
    """Read-time rotation (§3.2: the cache keeps k^R unrotated; App. D.5: the
    window is re-indexed to local temporal coordinates on assembly).
    (a) Without a sink it equals rotation at write: RoPE depends on relative
    positions only, and the re-indexing is a uniform shift.  (b) With a sink the
    result does not depend on absolute rollout time: the same tokens at frames
    (0 | 235..240) and (0 | 35..40) give the same outputs, while rotating at the
    absolute positions does not.  (c) It equals scalar loops that rotate every
    key and query at its frame's index in the context."""
    s = small_wan(window_frames=4, n_valid_frames=4, chunk_frames=2, t0=8)
    w, ids, x = layer_inputs(s)
    a = o.step(s, w, by_frame(s, ids, x))
    b = o.step(s.with_(rope_at_read=True), w, by_frame(s, ids, x))
    assert np.abs(a["y"] - b["y"]).max() < 1e-12 * np.abs(a["y"]).max()
    sr = small_wan(window_frames=3, n_valid_frames=3, chunk_frames=2, t0=38, rope_at_read=True,
                   sink_frames=1)
    w, ids, x = layer_inputs(sr)
    assert ids == [0, 37, 38, 39]
    early = sr.with_(t0=8)
    ids_e = window_ids(early)
    assert ids_e == [0, 7, 8, 9]
    r1 = o.step(sr, w, by_frame(sr, ids, x))
    r2 = o.step(early, w, by_frame(early, ids_e, x))
    assert np.abs(r1["y"] - r2["y"]).max() < 1e-12 * np.abs(r1["y"]).max()
    a1 = o.step(sr.with_(rope_at_read=False), w, by_frame(sr, ids, x))
    a2 = o.step(early.with_(rope_at_read=False), w, by_frame(early, ids_e, x))
    assert not np.allclose(a1["y"], a2["y"])
    sb = tiny_brute_shape().with_(rope_at_read=True, sink_frames=1)
    w, ids, x = layer_inputs(sb, seed=5)
    assert ids == [0, 4, 5, 6]
    times = {f: i for i, f in enumerate(ids)}
    r = o.step(sb, w, by_frame(sb, ids, x))
    for token in (0, 5, 9, 11):
        yb = np.array(brute_force_y(sb, w, x, ids, sb.chunk_frame_ids, token, times=times))
        err = np.abs(yb - r["y"][token]).max() / np.abs(yb).max()
        assert err < 1e-12, (token, err)


def pin_chunk_causal(o):
    """Chunk-causal forward over a clip (§3.3 trains with block masks; App. D.4:
    tokens see their own chunk and earlier ones, never a later one).
    (a) Block k of the clip pass equals the inference step whose chunk is block
    k over a window of the frames before it and the block itself (no mask).
    (b) Scalar loops over the truncated context give the same rows.
    (c) Blocks as long as the chunk reduce to the unmasked step.
    (d) Changing a later frame's tokens leaves every earlier block bit-identical
    and changes the later block."""
    s = small_wan(window_frames=6, chunk_frames=6, t0=0, n_valid_frames=6, causal_frames=2)
    w, ids, x = layer_inputs(s)
    assert ids == list(range(6))
    tpf = s.tokens_per_frame
    r = o.step(s, w, by_frame(s, ids, x))
    for k in range(3):
        dk = s.with_(chunk_frames=2, t0=2 * k, n_valid_frames=2 * k + 2, causal_frames=0)
        ids_k = window_ids(dk)
        assert ids_k == list(range(2 * k + 2))
        rk = o.step(dk, w, by_frame(s, ids, x))
        got = r["y"][2 * k * tpf:(2 * k + 2) * tpf]
        assert np.abs(got - rk["y"]).max() < 1e-12 * np.abs(rk["y"]).max(), k
    sb = tiny_brute_shape().with_(window_frames=4, chunk_frames=4, t0=0, n_valid_frames=4,
                                  causal_frames=2)
    wb, idb, xb = layer_inputs(sb, seed=4)
    rb = o.step(sb, wb, by_frame(sb, idb, xb))
    tb = sb.tokens_per_frame
    for token in (0, 7, 12, 23):
        vis = (token // tb) // 2 * 2 + 2
        yb = np.array(brute_force_y(sb, wb, xb[:vis * tb], idb[:vis], sb.chunk_frame_ids, token))
        err = np.abs(yb - rb["y"][token]).max() / np.abs(yb).max()
        assert err < 1e-12, (token, err)
    full = o.step(s.with_(causal_frames=6), w, by_frame(s, ids, x))
    plain = o.step(s.with_(causal_frames=0), w, by_frame(s, ids, x))
    assert np.array_equal(full["y"], plain["y"])
    x2 = x.copy()
    x2[5 * tpf:] += 1.0
    r2 = o.step(s, w, by_frame(s, ids, x2))
    assert np.array_equal(r2["y"][:4 * tpf], r["y"][:4 * tpf])
    assert not np.allclose(r2["y"][4 * tpf:], r["y"][4 * tpf:])


def pin_rmsnorm(o):
    """RMSNorm (App. D.2 normalises c^KV and c^Q) against what the mathematics
    fixes, not against a restatement of its formula:
    (a) with unit gain and eps = 0 every output row has root-mean-square 1;
    (b) it is invariant to positive scaling of the row at eps = 0, and eps
        scales with the square of the row: RMSNorm(a u; a^2 eps) = RMSNorm(u; eps);
    (c) the gain multiplies the normalised row elementwise;
    (d) with unit gain the output's mean square is ms / (ms + eps), ms the
        input's: eps sits inside the root, added to the mean square;
    (e) a library routine: torch.nn.functional.rms_norm in fp64;
    (f) a worked case: (3, 4) has mean square 12.5, so it maps to (3, 4) / sqrt(12.5);
    (g) rows are normalised independently of each other."""
    rng = np.random.default_rng(11)
    n = 24
    u = rng.normal(size=(40, n)) * rng.uniform(0.01, 10.0, size=(40, 1))
    ones = np.ones(n)
    r0 = o.rmsnorm(u, ones, 0.0)
    assert np.allclose(np.sqrt(np.mean(r0 * r0, axis=-1)), 1.0, rtol=1e-14, atol=0)
    for a in (1e-3, 0.5, 7.0, 1e4):
        assert np.allclose(o.rmsnorm(a * u, ones, 0.0), r0, rtol=1e-13, atol=0)
        assert np.allclose(o.rmsnorm(a * u, ones, 0.3 * a * a), o.rmsnorm(u, ones, 0.3),
                           rtol=1e-13, atol=0)
    g = rng.normal(1.0, 0.5, size=n)
    assert np.allclose(o.rmsnorm(u, g, 1e-6), o.rmsnorm(u, ones, 1e-6) * g, rtol=1e-14, atol=0)
    eps = 0.25
    ms = np.mean(u * u, axis=-1)
    r = o.rmsnorm(u, ones, eps)
    assert np.allclose(np.mean(r * r, axis=-1), ms / (ms + eps), rtol=1e-13, atol=0)
    for e in (1e-6, eps):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(u), (n,), weight=torch.from_numpy(g),
                                           eps=e).numpy()
        assert np.allclose(o.rmsnorm(u, g, e), ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(o.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0),
                       np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=1e-15, atol=0)
    one = np.stack([o.rmsnorm(u[i], g, eps) for i in range(u.shape[0])])
    assert np.allclose(one, o.rmsnorm(u, g, eps), rtol=1e-15, atol=0)


def pin_rope_table(o):
    """An explicit per-pair frequency table is used as given: rotating unit vectors
    e_2m through the layer's key path gives (cos, sin) of the table's angle for
    pair m at the token's coordinate on that pair's axis (§3.2 Eq. 5 with the
    frequencies as an input), and an all-zero table means the derived bands."""
    s = tiny_brute_shape()
    om_derived, ax = o.rope_omegas(s.d_head, s.rope_pairs, s.rope_theta)
    table = tuple(0.05 + 0.11 * m for m in range(s.d_rope // 2))
    st = s.with_(rope_freq=table)
    om, ax2 = o.rope_frequencies(st)
    assert np.array_equal(ax, ax2) and np.array_equal(om, np.array(table))
    om0, _ = o.rope_frequencies(s.with_(rope_freq=(0.0,) * (s.d_rope // 2)))
    assert np.array_equal(om0, om_derived)
    # the key path: W^K_R = identity on the first d_rope input channels, so k^R = x
    w = {"w_kv_down": np.ones((s.d_c, s.d_model)), "g_kv": np.ones(s.d_c),
         "w_kr": np.eye(s.d_rope, s.d_model)}
    frames = [3, 11]
    tpf = s.tokens_per_frame
    for m in range(s.d_rope // 2):
        x = np.zeros((len(frames) * tpf, s.d_model))
        x[:, 2 * m] = 1.0
        _, _, k_rope = o.cache_entries(st, w, x, frames)
        for i, f in enumerate(frames):
            for nn in range(tpf):
                p = (f, nn // s.grid_w, nn % s.grid_w)[ax[m]]
                row = k_rope[i * tpf + nn]
                assert abs(row[2 * m] - math.cos(p * table[m])) < 1e-14
                assert abs(row[2 * m + 1] - math.sin(p * table[m])) < 1e-14
                others = np.delete(row, [2 * m, 2 * m + 1])
                assert np.all(others == 0)


def pin_window_derivation(o):
    """The step derives its attended frames from (t0, C, n_valid, S) itself: frames
    it does not attend are never read (a token source that refuses them), and the
    returned window matches explicit cases of App. D.4 (sink first, then the
    chronological window, the chunk last)."""
    cases = [(small_wan(), [0, 1, 2, 3]),
             (small_wan(window_frames=4, t0=9, n_valid_frames=3), [7, 8, 9]),
             (small_wan(window_frames=3, n_valid_frames=3, chunk_frames=2, t0=38,
                        rope_at_read=True, sink_frames=1), [0, 37, 38, 39])]
    for s, expect in cases:
        w, ids, x = layer_inputs(s)
        assert ids == expect
        tok = by_frame(s, ids, x)

        def source(f, tok=tok):
            if f not in tok:
                raise AssertionError(f"frame {f} read but not attended")
            return tok[f]
        r = o.step(s, w, source)
        assert r["window_ids"] == expect


ALL_PINS = [pin_accounting, pin_absorbed, pin_sdpa, pin_bruteforce, pin_rope, pin_positions,
            pin_sink_context, pin_read_rotation, pin_chunk_causal, pin_rmsnorm, pin_rope_table,
            pin_window_derivation]


# ---------------------------------------------------------------- the pins as tests
def test_accounting_matches_paper():
    pin_accounting(O)


def test_absorbed_equals_unabsorbed_small_wan():
    pin_absorbed(O)


def test_absorbed_equals_unabsorbed_tiny_and_c4_dims():
    pin_absorbed(O, W.shape_by_name("tiny-f32"))
    pin_absorbed(O, small_wan(d_c=128, d_rope=64, d_nope=64, rope_pairs=(12, 10, 10)))


def test_sdpa_brute_force_small_wan():
    pin_sdpa(O)


def test_sdpa_tiny():
    pin_sdpa(O, W.shape_by_name("tiny-f32"))


def test_scalar_loop_brute_force():
    pin_bruteforce(O)


def test_rope_invariants():
    pin_rope(O)


def test_token_positions():
    pin_positions(O)


def test_rmsnorm_properties():
    pin_rmsnorm(O)


def test_explicit_rope_table():
    pin_rope_table(O)


def test_step_derives_its_window():
    pin_window_derivation(O)


def test_generator_window_matches_oracle():
    """The seeded-input module lists a shape's attended frames too (it decides which
    frames to draw and prefill); that list must be the oracle's window_frames for
    every named workload and for random chunk/window/sink draws, so no expected
    value rests on the generator's copy of the ring bookkeeping."""
    for name, s in W.SHAPES.items():
        assert s.window_frame_ids == window_ids(s), name
    rng = np.random.default_rng(5)
    base = W.shape_by_name("tiny-f32")
    checked = 0
    while checked < 500:
        sink = int(rng.integers(0, 3))
        wf = int(rng.integers(1, 9))
        c = int(rng.integers(1, wf + 1))
        t0 = int(rng.integers(0, 300))
        nv = int(rng.integers(c, wf + 1))
        s = base.with_(window_frames=wf, chunk_frames=c, t0=t0, n_valid_frames=nv,
                       sink_frames=sink, rope_at_read=bool(sink))
        if t0 + c - nv < sink:  # the local window would reach into the sink
            continue
        assert s.window_frame_ids == window_ids(s), s
        checked += 1


def test_rank_bound():
    """P-4: the composed operator [W_up^K W_down^KV; W_up^V W_down^KV] has rank at
    most d_c (§4 spectral analysis of the MLA projection)."""
    for s in (W.shape_by_name("tiny-f32"), W.shape_by_name("wan1.3b-w21").with_(dtype="f32")):
        _, w = W.draw_weights(s)
        m = np.concatenate([w["w_k_up"] @ w["w_kv_down"], w["w_v_up"] @ w["w_kv_down"]])
        assert m.shape == (s.n_heads * (s.d_nope + s.d_head), s.d_model)
        assert np.linalg.matrix_rank(m) <= s.d_c
        assert np.linalg.matrix_rank(m) == s.d_c  # generic draws reach the bound


def test_single_key_returns_its_value():
    """P-6: with one valid key the softmax weight is 1, so out_h = W_up,h^V c_j."""
    s = small_wan(grid_h=1, grid_w=1, n_valid_frames=1)
    w, ids, x = layer_inputs(s)
    r = O.step(s, w, by_frame(s, ids, x))
    c = r["c"][0]
    for h in range(s.n_heads):
        v = w["w_v_up"][h * s.d_head:(h + 1) * s.d_head] @ c
        assert np.allclose(r["out"][0, h * s.d_head:(h + 1) * s.d_head], v, rtol=1e-13, atol=1e-13)


def test_zero_query_averages_values():
    """P-6: q = 0 gives equal scores, so the output is the mean of the values."""
    s = small_wan()
    w, ids, x = layer_inputs(s)
    w = dict(w, w_q_up=np.zeros_like(w["w_q_up"]), w_qr=np.zeros_like(w["w_qr"]))
    r = O.step(s, w, by_frame(s, ids, x))
    _, v = O.reconstruct_kv(s, w, r["c"])
    mean = v.mean(axis=0).reshape(-1)
    assert np.allclose(r["out"], mean[None, :], rtol=1e-12, atol=1e-12)


def test_identical_keys_give_uniform_weights():
    """P-6: identical window tokens and no positional key -> every weight is 1/M,
    whatever the query."""
    s = small_wan()
    w, ids, x = layer_inputs(s)
    x = np.broadcast_to(x[:1], x.shape).copy()
    w = dict(w, w_kr=np.zeros_like(w["w_kr"]))
    r = O.step(s, w, by_frame(s, ids, x))
    _, v = O.reconstruct_kv(s, w, r["c"][:1])
    assert np.allclose(r["out"], v.reshape(1, -1), rtol=1e-12, atol=1e-12)


def test_ring_traversal_order_is_irrelevant():
    """P-7: softmax over the window is permutation-invariant, so attending the
    ring in slot order equals attending it chronologically."""
    s = small_wan(window_frames=4, t0=5, n_valid_frames=4)  # frames 2..5 wrap the ring
    w, ids, x = layer_inputs(s)
    tpf = s.tokens_per_frame
    ring = O.expected_ring(s, w, x, ids)
    rows = O.ring_rows_for_window(s.t0, s.chunk_frames, s.n_valid_frames, s.window_frames, tpf)
    assert sorted(rows.tolist()) == list(range(s.window_frames * tpf))
    assert rows[0] != 0  # chronological order really differs from slot order
    _, qn, qr = O.query_parts(s, w, x[-tpf:], s.chunk_frame_ids)
    chrono = O.attention_unabsorbed(s, w, qn, qr, ring[rows, :s.d_c], ring[rows, s.d_c:])
    slot = O.attention_unabsorbed(s, w, qn, qr, ring[:, :s.d_c], ring[:, s.d_c:])
    assert np.abs(chrono - slot).max() <= 1e-13 * np.abs(chrono).max()


@pytest.mark.parametrize("wf,cf", [(4, 1), (21, 3), (6, 3), (42, 3), (21, 1)])
def test_ring_fifo_matches_deque(wf, cf):
    """P-8: slot(f) = f mod W is FIFO eviction of whole frames (App. D.4): after
    every chunk write, the ring holds exactly the last W frames a deque keeps."""
    dq = collections.deque(maxlen=wf)
    slots = [None] * wf
    for step_i in range(100):
        t0 = step_i * cf
        for f in range(t0, t0 + cf):
            dq.append(f)
            slots[O.ring_slot(f, wf)] = f
        assert sorted(f for f in slots if f is not None) == list(dq)
        n_valid = min(len(dq), wf)
        assert O.window_frames(t0, cf, n_valid) == list(dq)[-n_valid:]
        rows = O.ring_rows_for_window(t0, cf, n_valid, wf, 2)
        assert [slots[r // 2] for r in rows[::2]] == list(dq)[-n_valid:]


def test_write_rotate_equals_read_rotate_without_sink():
    """P-9: rotating keys at their absolute frame index when written gives the same
    scores as keeping them unrotated and rotating at window-local positions when
    the window is assembled (§3.2, App. D.5) -- as long as queries use the same
    frame of reference and the window is contiguous.  With a re-indexed sink frame
    the two differ, which is why the sink path needs read-time rotation."""
    s = small_wan(window_frames=6, t0=40, n_valid_frames=6, chunk_frames=1)
    w, ids, x = layer_inputs(s)
    tpf = s.tokens_per_frame
    om, ax = O.rope_omegas(s.d_head, s.rope_pairs)
    _, k_r, k_abs = O.cache_entries(s, w, x, ids)
    c_q = O.rmsnorm(x[-tpf:] @ w["w_q_down"].T, w["g_q"], s.rms_eps)
    q_r = (c_q @ w["w_qr"].T).reshape(tpf, s.n_heads, s.d_rope)
    pos_abs = O.token_positions(ids, s.grid_h, s.grid_w)
    pos_loc = pos_abs - np.array([ids[0], 0, 0])
    qpa = O.token_positions(s.chunk_frame_ids, s.grid_h, s.grid_w)
    qpl = qpa - np.array([ids[0], 0, 0])
    k_loc = O.rope3d(k_r, pos_loc, om, ax)
    for h in range(s.n_heads):
        sa = O.rope3d(q_r[:, h], qpa, om, ax) @ k_abs.T
        sl = O.rope3d(q_r[:, h], qpl, om, ax) @ k_loc.T
        assert np.allclose(sa, sl, rtol=1e-10, atol=1e-10)
    # sink frame 0 re-indexed to local t=0 next to local frames 1..5: not a uniform shift
    sink_ids = [0] + ids[1:]
    pos_sink = O.token_positions(sink_ids, s.grid_h, s.grid_w)
    pos_sink_loc = pos_sink.copy()
    pos_sink_loc[:tpf, 0] = 0
    pos_sink_loc[tpf:, 0] = pos_sink[tpf:, 0] - ids[0]
    sa = O.rope3d(q_r[:, 0], qpa, om, ax) @ O.rope3d(k_r, pos_sink, om, ax).T
    sl = O.rope3d(q_r[:, 0], qpl, om, ax) @ O.rope3d(k_r, pos_sink_loc, om, ax).T
    assert not np.allclose(sa, sl)


def test_expected_ring_layout():
    """O12: row (f mod W)*tpf + n holds [c^KV | RoPE3D(k^R)] of token n of frame f."""
    s = W.shape_by_name("tiny-f32")
    w, ids, x = layer_inputs(s)
    ring = O.expected_ring(s, w, x, ids)
    c, _, kr = O.cache_entries(s, w, x, ids)
    tpf = s.tokens_per_frame
    for i, f in enumerate(ids):
        r0 = (f % s.window_frames) * tpf
        assert np.array_equal(ring[r0:r0 + tpf, :s.d_c], c[i * tpf:(i + 1) * tpf])
        assert np.array_equal(ring[r0:r0 + tpf, s.d_c:], kr[i * tpf:(i + 1) * tpf])
    assert ring.shape[1] == O.cache_scalars_per_token(s.d_c, s.d_rope)


def test_sink_context_and_slots():
    pin_sink_context(O)


def test_read_time_rotation():
    pin_read_rotation(O)


def test_chunk_causal_forward():
    pin_chunk_causal(O)


def test_chunk_causal_visible_keys():
    """Prefix lengths of the block mask: a 21-frame clip in 3-frame blocks, and a
    chunk that follows cached frames (the blocks start after them)."""
    s = W.shape_by_name("wan1.3b-clip21-causal3")
    v = O.visible_keys(s, window_ids(s), s.chunk_frame_ids)
    tpf = s.tokens_per_frame
    assert v.shape == (21 * tpf,)
    assert v[0] == v[3 * tpf - 1] == 3 * tpf and v[3 * tpf] == 6 * tpf and v[-1] == 21 * tpf
    assert int(v.sum()) == W.attended_pairs(s) == tpf * tpf * 3 * 3 * (1 + 2 + 3 + 4 + 5 + 6 + 7)
    t = small_wan(window_frames=6, chunk_frames=4, t0=2, n_valid_frames=6, causal_frames=2)
    v = O.visible_keys(t, window_ids(t), t.chunk_frame_ids)
    tp = t.tokens_per_frame
    assert list(v[::tp]) == [4 * tp, 4 * tp, 6 * tp, 6 * tp]
    assert int(v.sum()) == W.attended_pairs(t)


def test_expected_ring_with_sink_keeps_raw_keys():
    """With read-time rotation the ring keeps [c^KV | k^R] unrotated (§3.2); the sink
    frame sits in slot 0 for good and later frames go FIFO over slots 1..W."""
    s = small_wan(window_frames=3, n_valid_frames=3, chunk_frames=1, t0=8, rope_at_read=True,
                  sink_frames=1)
    w, ids, x = layer_inputs(s)
    assert ids == [0, 6, 7, 8]
    ring = O.expected_ring(s, w, x, ids)
    c, kr_raw, _ = O.cache_entries(s, w, x, ids)
    tpf = s.tokens_per_frame
    assert ring.shape[0] == (1 + 3) * tpf
    for i, f in enumerate(ids):
        r0 = (0 if f == 0 else 1 + (f - 1) % 3) * tpf
        assert np.array_equal(ring[r0:r0 + tpf, :s.d_c], c[i * tpf:(i + 1) * tpf])
        assert np.array_equal(ring[r0:r0 + tpf, s.d_c:], kr_raw[i * tpf:(i + 1) * tpf])


# ---------------------------------------------------------------- planted mistakes
# Each mutant replaces one oracle function (module attribute, so every caller
# inside the oracle sees it) with a plausible mistake.
from oracle import mla_oracle as _M  # noqa: E402

_ORIG = {k: getattr(_M, k) for k in ("rope3d", "rmsnorm", "reconstruct_kv",
                                     "attention_unabsorbed", "rope_omegas", "visible_keys",
                                     "value_absorbed_output", "query_absorbed",
                                     "window_frames")}


def _mut_rope_sign(v, pos, omegas, axes):
    return _ORIG["rope3d"](v, -np.asarray(pos), omegas, axes)


def _mut_rope_axes(v, pos, omegas, axes):
    return _ORIG["rope3d"](v, np.asarray(pos)[..., ::-1], omegas, axes)


def _mut_rmsnorm_sum(u, g, eps):
    u = np.asarray(u, dtype=np.float64)
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + eps) * g


def _mut_kv_head_order(s, w, c):
    n = c.shape[0]
    k_nope = (c @ w["w_k_up"].T).reshape(n, s.d_nope, s.n_heads).transpose(0, 2, 1)
    v = (c @ w["w_v_up"].T).reshape(n, s.n_heads, s.d_head)
    return k_nope, v


def _mut_drop_rope_term(s, w, q_nope, q_rope, c, k_rope, block=1024, visible=None):
    return _ORIG["attention_unabsorbed"](s, w, q_nope, np.zeros_like(q_rope), c, k_rope, block,
                                         visible)


def _mut_scale_nope_only(s, w, q_nope, q_rope, c, k_rope, block=1024, visible=None):
    f = math.sqrt((s.d_nope + s.d_rope) / s.d_nope)
    return _ORIG["attention_unabsorbed"](s, w, q_nope * f, q_rope * f, c, k_rope, block, visible)


def _mut_mask_ignored(s, w, q_nope, q_rope, c, k_rope, block=1024, visible=None):
    return _ORIG["attention_unabsorbed"](s, w, q_nope, q_rope, c, k_rope, block, None)


def _mut_mask_per_frame(s, window_ids, chunk_ids):
    v = _ORIG["visible_keys"](s, window_ids, chunk_ids)
    if not getattr(s, "causal_frames", 0):
        return v
    tpf = s.tokens_per_frame
    first = window_ids.index(chunk_ids[0])
    return (first + np.arange(len(v)) // tpf + 1) * tpf


def _mut_mask_one_block_late(s, window_ids, chunk_ids):
    v = _ORIG["visible_keys"](s, window_ids, chunk_ids)
    if not getattr(s, "causal_frames", 0):
        return v
    return np.minimum(v + s.causal_frames * s.tokens_per_frame, len(window_ids) * s.tokens_per_frame)


def _mut_omega_lowband(d_head, pairs, theta=10000.0):
    om, ax = _ORIG["rope_omegas"](d_head, pairs, theta)
    out = om.copy()
    for a in range(3):
        out[ax == a] = om[ax == a][::-1]
    return out, ax


def _mut_times_absolute(frames, rope_at_read):
    return {f: f for f in frames}


def _mut_sink_evicted(frame, window_frames, sink_frames=0):
    return frame % window_frames


def _mut_sink_last(t0, chunk_frames, n_valid_frames, sink_frames=0):
    last = t0 + chunk_frames - 1
    return list(range(last - n_valid_frames + 1, last + 1)) + list(range(min(sink_frames, last + 1)))


def _mut_b_transposed_head(s, w, h):
    wo = w["w_o"][:, h * s.d_head:(h + 1) * s.d_head]
    wv = w["w_v_up"][h * s.d_head:(h + 1) * s.d_head]
    return wo[:, ::-1] @ wv


def _mut_b_next_head(s, w, h):
    return _ORIG["value_absorbed_output"](s, w, (h + 1) % s.n_heads)


def _mut_a_transposed_query(s, w, h):
    return _ORIG["query_absorbed"](s, w, h)[::-1]


def _mut_a_other_head_keys(s, w, h):
    wq = w["w_q_up"][h * s.d_nope:(h + 1) * s.d_nope]
    g = (h + 1) % s.n_heads
    return wq.T @ w["w_k_up"][g * s.d_nope:(g + 1) * s.d_nope]


def _mut_rmsnorm_eps_outside(u, g, eps):
    u = np.asarray(u, dtype=np.float64)
    return u / (np.sqrt(np.mean(u * u, axis=-1, keepdims=True)) + eps) * g


def _mut_rmsnorm_gain_inside(u, g, eps):
    u = np.asarray(u, dtype=np.float64) * g
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)


def _mut_rmsnorm_unbiased(u, g, eps):
    u = np.asarray(u, dtype=np.float64)
    n = u.shape[-1]
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) / max(n - 1, 1) + eps) * g


def _mut_rmsnorm_no_eps(u, g, eps):
    return _ORIG["rmsnorm"](u, g, 0.0)


def _mut_rope_table_ignored(s):
    return _M.rope_omegas(s.d_head, s.rope_pairs, s.rope_theta)


def _mut_window_short(t0, chunk_frames, n_valid_frames, sink_frames=0):
    return _ORIG["window_frames"](t0, chunk_frames, n_valid_frames, sink_frames)[1:]


MUTANTS = {
    "rope rotation sign": dict(rope3d=_mut_rope_sign),
    "rope axis order": dict(rope3d=_mut_rope_axes),
    "rmsnorm sum instead of mean": dict(rmsnorm=_mut_rmsnorm_sum),
    "rmsnorm eps outside the root": dict(rmsnorm=_mut_rmsnorm_eps_outside),
    "rmsnorm gain before the norm": dict(rmsnorm=_mut_rmsnorm_gain_inside),
    "rmsnorm over n - 1": dict(rmsnorm=_mut_rmsnorm_unbiased),
    "rmsnorm without eps": dict(rmsnorm=_mut_rmsnorm_no_eps),
    "explicit rope table ignored": dict(rope_frequencies=_mut_rope_table_ignored),
    "window one frame short": dict(window_frames=_mut_window_short),
    "head/channel order in W_up^K": dict(reconstruct_kv=_mut_kv_head_order),
    "dropped RoPE score term": dict(attention_unabsorbed=_mut_drop_rope_term),
    "scale 1/sqrt(d_nope)": dict(attention_unabsorbed=_mut_scale_nope_only),
    "lowest instead of highest bands": dict(rope_omegas=_mut_omega_lowband),
    "absolute times at read": dict(context_times=_mut_times_absolute),
    "sink frame evicted": dict(ring_slot=_mut_sink_evicted),
    "sink after the local frames": dict(window_frames=_mut_sink_last),
    "causal mask ignored": dict(attention_unabsorbed=_mut_mask_ignored),
    "causal mask per frame, not per block": dict(visible_keys=_mut_mask_per_frame),
    "causal mask one block late": dict(visible_keys=_mut_mask_one_block_late),
    "B_h with W_O columns reversed": dict(value_absorbed_output=_mut_b_transposed_head),
    "B_h of the next head": dict(value_absorbed_output=_mut_b_next_head),
    "A_h with the query latent reversed": dict(query_absorbed=_mut_a_transposed_query),
    "A_h with another head's keys": dict(query_absorbed=_mut_a_other_head_keys),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for k, fn in MUTANTS[name].items():
        monkeypatch.setattr(_M, k, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(_M)
        except Exception:  # an assertion, or the pin cannot even run on the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
