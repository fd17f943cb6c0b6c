"""C-ABI checks that need no GPU: the library loads, exports every function
include/mla.h declares, and its host-only calls (validation, workspace and cache
sizing, status strings) behave as documented.  No compute entry point is called
with valid arguments here."""
import ctypes
import os
import re

import pytest

import latent_kv_attention_down_amd as mla
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def test_header_declares_the_three_entry_points():
    fns = header_functions()
    for name in ("mla_cache_write", "mla_chunk_attention", "mla_step"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    fns = header_functions()
    assert fns, "no declarations parsed"
    for name in fns:
        assert hasattr(lib, name), name
    assert set(fns) == set(mla.SIGNATURES), "binding and header disagree"


def test_probe_library_exports_its_header():
    """The ceiling probe (a library of its own, not the MLA path) exports what
    include/mla_probe.h declares, and libmla.so does not carry it."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mla_probe.h")).read(),
                  flags=re.S)
    fns = sorted(set(re.findall(r"\b(mla_probe_[a-z0-9_]+)\s*\(", text)))
    assert fns == ["mla_probe_mfma_bf16", "mla_probe_mfma_bf16_flop"]
    probe = ctypes.CDLL(os.path.join(ROOT, "latent_kv_attention_down_amd", "libmla_probe.so"))
    for name in fns:
        assert hasattr(probe, name), name
    assert not hasattr(mla.load(), "mla_probe_mfma_bf16")
    probe.mla_probe_mfma_bf16_flop.restype = ctypes.c_double
    assert probe.mla_probe_mfma_bf16_flop(2, 3) == 2 * 8 * 3 * 4 * 2 * 32 * 32 * 16


def cfg_of(name, **kw):
    return mla.make_config(W.shape_by_name(name).with_(**kw))


def chunk_of(s, **kw):
    d = dict(batch=1, chunk_frames=s.chunk_frames, t0=s.t0, n_valid_frames=s.n_valid_frames,
             causal_frames=s.causal_frames)
    d.update(kw)
    return mla.make_chunk(**d)


@pytest.mark.parametrize("name", ["tiny-f32", "wan1.3b-w21", "wan1.3b-w42-t240",
                                  "wan1.3b-w21-t240-q1", "wan1.3b-w21-dc128-dr32",
                                  "wan1.3b-w21-dc256-dr32", "wan1.3b-w21-dc192-dr64",
                                  "wan1.3b-w21-read", "wan1.3b-sink1-w6-t240",
                                  "wan1.3b-clip21-causal3"])
def test_workload_shapes_validate(name):
    s = W.shape_by_name(name)
    assert mla.validate(mla.make_config(s), chunk_of(s)) == mla.MLA_OK, mla.last_error()


def test_cache_bytes_is_224_scalars_per_token():
    """Only d_c + d_rope scalars per token are cached (VideoMLA App. E, Eq. 13)."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    assert mla.cache_bytes(cfg, 1) == 21 * 1560 * 224 * 2
    assert mla.cache_bytes(cfg, 3) == 3 * 21 * 1560 * 224 * 2
    assert mla.cache_bytes(mla.make_config(s, dtype="f32"), 1) == 21 * 1560 * 224 * 4
    assert mla.cache_bytes(cfg, 0) == 0


def test_workspace_bytes_positive_and_monotone():
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    w1 = mla.workspace_bytes(cfg, chunk_of(s))
    w2 = mla.workspace_bytes(cfg, chunk_of(s, batch=2))
    assert 0 < w1 < w2
    assert w1 % 256 == 0


@pytest.mark.parametrize("field,value,code", [
    ("d_model", 0, mla.MLA_ERR_INVALID_ARG),
    ("d_nope", 95, mla.MLA_ERR_INVALID_ARG),          # d_nope + d_rope != d_head
    ("d_rope", 31, mla.MLA_ERR_INVALID_ARG),
    ("window_frames", 0, mla.MLA_ERR_INVALID_ARG),
    ("grid_w", -1, mla.MLA_ERR_INVALID_ARG),
    ("dtype", 7, mla.MLA_ERR_INVALID_ARG),
    ("rope_theta", 0.0, mla.MLA_ERR_INVALID_ARG),
    ("d_c", 160, mla.MLA_ERR_UNSUPPORTED),            # bf16 kernel not built for 160
    ("d_q", 100, mla.MLA_ERR_UNSUPPORTED),            # bf16 needs multiples of 32
])
def test_validate_rejects(field, value, code):
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    setattr(cfg, field, value)
    if field == "d_rope":
        cfg.d_nope = cfg.d_head - value
    assert mla.validate(cfg, chunk_of(s)) == code
    assert mla.last_error() != ""


def test_validate_rope_pairs_sum():
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    cfg.rope_pairs[0] = 7
    assert mla.validate(cfg, chunk_of(s)) == mla.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(batch=0), dict(chunk_frames=0), dict(chunk_frames=22),
                                dict(n_valid_frames=2), dict(n_valid_frames=22), dict(t0=-1),
                                dict(t0=0, n_valid_frames=21)])
def test_validate_rejects_bad_chunk(kw):
    s = W.shape_by_name("wan1.3b-w21")
    assert mla.validate(mla.make_config(s), chunk_of(s, **kw)) == mla.MLA_ERR_INVALID_ARG


def test_sink_needs_read_rotation():
    """A sink frame only makes sense with window-local re-indexing (App. D.5), which
    needs k^R kept unrotated; other rope_mode values and negative sinks are refused."""
    s = W.shape_by_name("wan1.3b-sink1-w6-t240")
    for field, value in (("rope_mode", mla.MLA_ROPE_AT_WRITE), ("rope_mode", 5),
                         ("sink_frames", -1)):
        cfg = mla.make_config(s)
        setattr(cfg, field, value)
        assert mla.validate(cfg, chunk_of(s)) == mla.MLA_ERR_INVALID_ARG, (field, value)


@pytest.mark.parametrize("kw,ok", [
    (dict(), True),                                       # sink 0 + frames 235..240
    (dict(n_valid_frames=7), False),                      # more than W local frames
    (dict(n_valid_frames=2), False),                      # misses a chunk frame
    (dict(t0=0, n_valid_frames=2), True),                 # sink 0 + frames 1, 2
    (dict(t0=0, n_valid_frames=3), False),                # local window reaches the sink
    (dict(t0=1, n_valid_frames=3), True),                 # sink 0 + frames 1..3
    (dict(t0=0, chunk_frames=1, n_valid_frames=0), True),  # the sink frame on its own
])
def test_sink_window_geometry(kw, ok):
    s = W.shape_by_name("wan1.3b-sink1-w6-t240")
    st = mla.validate(mla.make_config(s), chunk_of(s, **kw))
    assert (st == mla.MLA_OK) == ok, (kw, st, mla.last_error())


def test_cache_and_workspace_bytes_with_sink():
    """The ring holds S sink slots plus W local slots; the workspace always has room
    for the gathered window (attended keys x (d_c + d_rope)), used by read-time
    rotation and by rings not in the interleaved layout, so its size does not depend
    on either."""
    s = W.shape_by_name("wan1.3b-sink1-w6-t240")
    cfg = mla.make_config(s)
    assert mla.cache_bytes(cfg, 1) == (1 + 6) * 1560 * 224 * 2
    w21 = W.shape_by_name("wan1.3b-w21")
    a = mla.workspace_bytes(mla.make_config(w21), chunk_of(w21))
    b = mla.workspace_bytes(mla.make_config(w21.with_(rope_at_read=True)), chunk_of(w21))
    assert a == b
    one = mla.workspace_bytes(mla.make_config(w21.with_(window_frames=22)),
                              chunk_of(w21, t0=19, n_valid_frames=22))
    assert one - a >= 1560 * 224 * 2  # one more attended frame: one more frame of window room


@pytest.mark.parametrize("causal,ok", [(0, True), (1, True), (3, True), (7, True), (21, True),
                                       (2, False), (4, False), (-1, False)])
def test_causal_blocks_must_divide_the_chunk(causal, ok):
    """Chunk-causal blocks tile the 21-frame clip exactly or are refused."""
    s = W.shape_by_name("wan1.3b-clip21-causal3")
    st = mla.validate(mla.make_config(s), chunk_of(s, causal_frames=causal))
    assert (st == mla.MLA_OK) == ok, (causal, st, mla.last_error())


def test_causal_blocks_add_split_records():
    """Each causal block starts a new row tile, so the clip pass needs a few more
    row tiles (split records and flags) than the unmasked pass over the same rows."""
    s = W.shape_by_name("wan1.3b-clip21-causal3")
    cfg = mla.make_config(s)
    a = mla.workspace_bytes(cfg, chunk_of(s, causal_frames=0))
    b = mla.workspace_bytes(cfg, chunk_of(s))
    assert 0 < a < b


def test_bf16_ring_over_2gib_is_refused():
    """The attention kernel addresses one request's ring with 32-bit byte offsets, so
    the bf16 path refuses rings of 2 GiB or more per request; fp32 has no such limit."""
    s = W.shape_by_name("wan1.3b-w21")
    frames = (1 << 31) // (1560 * 224 * 2)  # 3072 frames of 1560 tokens: just over 2 GiB
    big = mla.make_config(s.with_(window_frames=frames + 1))
    assert mla.validate(big, chunk_of(s)) == mla.MLA_ERR_UNSUPPORTED
    ok = mla.make_config(s.with_(window_frames=frames - 1))
    assert mla.validate(ok, chunk_of(s)) == mla.MLA_OK, mla.last_error()
    assert mla.validate(mla.make_config(s.with_(window_frames=frames + 1, dtype="f32")),
                        chunk_of(s)) == mla.MLA_OK


def fake_cache(cfg, batch=1, base=1 << 20):
    """An interleaved descriptor over a made-up device address (never dereferenced:
    the calls below fail or are refused before any launch)."""
    return mla.interleaved_cache(cfg, batch, base)


def test_latent_attention_refuses_read_rotation(lib):
    s = W.shape_by_name("wan1.3b-w21-read")
    cfg = mla.make_config(s)
    ch = chunk_of(s)
    n = mla.workspace_bytes(cfg, ch)
    cache = fake_cache(cfg)
    assert lib.mla_latent_attention(ctypes.byref(cfg), ctypes.byref(ch), 4096, ctypes.byref(cache),
                                    4096, 4096, n, None) == mla.MLA_ERR_UNSUPPORTED


def test_fp32_path_accepts_odd_dims():
    s = W.shape_by_name("tiny-f32").with_(d_c=17, d_q=33)
    assert mla.validate(mla.make_config(s), chunk_of(s)) == mla.MLA_OK


def test_null_arguments_fail_before_any_launch(lib):
    """Invalid calls return a status on the host; nothing is launched (no GPU here)."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    ch = chunk_of(s)
    w = mla.Weights()
    assert lib.mla_cache_write(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), None, None,
                               None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_step(None, None, None, None, None, None, None, 0, None) == mla.MLA_ERR_INVALID_ARG
    # misaligned pointers are refused before any HIP call
    fake = {n: 4096 for n, _ in mla.Weights._fields_}
    wt = mla.Weights(**fake)
    cache = fake_cache(cfg)
    assert lib.mla_cache_write(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4097,
                               ctypes.byref(cache), None) == mla.MLA_ERR_ALIGNMENT
    # a NULL cache descriptor is refused
    assert lib.mla_cache_write(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4096, None,
                               None) == mla.MLA_ERR_INVALID_ARG
    # a workspace that is too small is refused before any HIP call
    assert lib.mla_latent_attention(ctypes.byref(cfg), ctypes.byref(ch), 4096, ctypes.byref(cache),
                                    4096, 4096, 16, None) == mla.MLA_ERR_WORKSPACE


def test_value_absorbed_weights_checks_before_launch(lib):
    """mla_value_absorbed_weights needs W^V_up, W_O and an aligned output; it refuses
    anything else on the host.  mla_step accepts w_b in place of W^V_up and W_O."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    fake = {n: 4096 for n, _ in mla.Weights._fields_}
    assert lib.mla_value_absorbed_weights(ctypes.byref(cfg), ctypes.byref(mla.Weights(**fake)),
                                          None, None) == mla.MLA_ERR_INVALID_ARG
    no_o = mla.Weights(**dict(fake, w_o=None))
    assert lib.mla_value_absorbed_weights(ctypes.byref(cfg), ctypes.byref(no_o), 4096,
                                          None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_value_absorbed_weights(ctypes.byref(cfg), ctypes.byref(mla.Weights(**fake)),
                                          4100, None) == mla.MLA_ERR_ALIGNMENT
    ch = chunk_of(s)
    n = mla.workspace_bytes(cfg, ch)
    # no w_b and no w_o: refused; a misaligned w_b: refused (both before any launch)
    cache = fake_cache(cfg)
    wt = mla.Weights(**dict(fake, w_o=None, w_b=None))
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, n, None) == mla.MLA_ERR_INVALID_ARG
    wt = mla.Weights(**dict(fake, w_o=None, w_v_up=None, w_b=4100))
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, n, None) == mla.MLA_ERR_ALIGNMENT


def test_query_absorbed_weights_checks_before_launch(lib):
    """mla_query_absorbed_weights needs W^K_up, W^Q_up, W^Q_R and an aligned output; a
    step accepts w_qlat in place of all three."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    fake = {n: 4096 for n, _ in mla.Weights._fields_}
    assert lib.mla_query_absorbed_weights(ctypes.byref(cfg), ctypes.byref(mla.Weights(**fake)),
                                          None, None) == mla.MLA_ERR_INVALID_ARG
    for missing in ("w_k_up", "w_q_up", "w_qr"):
        w = mla.Weights(**dict(fake, **{missing: None}))
        assert lib.mla_query_absorbed_weights(ctypes.byref(cfg), ctypes.byref(w), 4096,
                                              None) == mla.MLA_ERR_INVALID_ARG, missing
    ch = chunk_of(s)
    n = mla.workspace_bytes(cfg, ch)
    cache = fake_cache(cfg)
    wt = mla.Weights(**dict(fake, w_qr=None, w_qlat=None))
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, n, None) == mla.MLA_ERR_INVALID_ARG
    wt = mla.Weights(**dict(fake, w_q_up=None, w_k_up=None, w_qr=None, w_qlat=4100))
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(wt), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, n, None) == mla.MLA_ERR_ALIGNMENT


def test_status_strings(lib):
    for code, name in ((0, "MLA_OK"), (-1, "MLA_ERR_INVALID_ARG"), (-2, "MLA_ERR_UNSUPPORTED"),
                       (-3, "MLA_ERR_ALIGNMENT"), (-4, "MLA_ERR_WORKSPACE"), (-5, "MLA_ERR_HIP")):
        assert mla.status_string(code) == name
    assert mla.status_string(42) == "MLA_UNKNOWN_STATUS"


# ---------------------------------------------------------------- cache descriptor
def test_interleaved_descriptor():
    """mla_cache_interleaved: k_r right after the d_c latent elements of the same row,
    rows of d_c + d_rope, requests one ring apart (the layout mla_cache_bytes sizes)."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    c = mla.interleaved_cache(cfg, 3, 1 << 20)
    assert c.c_kv == 1 << 20 and c.k_r == (1 << 20) + 192 * 2
    assert c.c_kv_row_stride == c.k_r_row_stride == 224
    assert c.c_kv_batch_stride == c.k_r_batch_stride == 21 * 1560 * 224
    assert 3 * c.c_kv_batch_stride * 2 == mla.cache_bytes(cfg, 3)
    f = mla.interleaved_cache(mla.make_config(s, dtype="f32"), 1, 1 << 20)
    assert f.k_r == (1 << 20) + 192 * 4
    lib = mla.load()
    out = mla.Cache()
    assert lib.mla_cache_interleaved(ctypes.byref(cfg), 1, 4100, ctypes.byref(out)) == \
        mla.MLA_ERR_ALIGNMENT
    assert lib.mla_cache_interleaved(ctypes.byref(cfg), 0, 4096, ctypes.byref(out)) == \
        mla.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_interleaved(ctypes.byref(cfg), 1, None, ctypes.byref(out)) == \
        mla.MLA_ERR_INVALID_ARG


def _split(c_kv=1 << 20, k_r=1 << 24, cr=192, kr=32, cb=21 * 1560 * 192, kb=21 * 1560 * 32):
    c = mla.Cache()
    c.c_kv, c.k_r, c.c_kv_row_stride, c.k_r_row_stride = c_kv, k_r, cr, kr
    c.c_kv_batch_stride, c.k_r_batch_stride = cb, kb
    return c


@pytest.mark.parametrize("kw,batch,code", [
    (dict(), 2, mla.MLA_ERR_HIP),                           # valid: refused only by injection
    (dict(cr=200, kr=40, cb=21 * 1560 * 200, kb=21 * 1560 * 40), 2, mla.MLA_ERR_HIP),
    (dict(c_kv=None), 1, mla.MLA_ERR_INVALID_ARG),
    (dict(k_r=None), 1, mla.MLA_ERR_INVALID_ARG),
    (dict(k_r=1 << 20), 1, mla.MLA_ERR_INVALID_ARG),          # both parts at one address
    (dict(c_kv=(1 << 20) + 8), 1, mla.MLA_ERR_ALIGNMENT),
    (dict(k_r=(1 << 24) + 4), 1, mla.MLA_ERR_ALIGNMENT),
    (dict(cr=191), 1, mla.MLA_ERR_INVALID_ARG),             # row narrower than d_c
    (dict(kr=16), 1, mla.MLA_ERR_INVALID_ARG),              # row narrower than d_rope
    (dict(cr=196), 1, mla.MLA_ERR_ALIGNMENT),               # 392-byte rows: not 16-byte steps
    (dict(kb=21 * 1560 * 32 + 4), 2, mla.MLA_ERR_ALIGNMENT),
    (dict(cb=21 * 1560 * 192 - 192), 2, mla.MLA_ERR_INVALID_ARG),  # requests would overlap
    (dict(cb=21 * 1560 * 192 - 192), 1, mla.MLA_ERR_HIP),   # one request: no batch stride used
])
def test_cache_descriptor_rules(kw, batch, code, monkeypatch):
    """Every rule of mla_cache is checked on the host before anything is launched;
    a valid descriptor gets as far as the launch (refused here by the injection)."""
    monkeypatch.setenv("MLA_FAULT_INJECT", "launch")
    lib = mla.load()
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    ch = chunk_of(s, batch=batch)
    cache = _split(**kw)
    w = mla.Weights(**{n: 4096 for n, _ in mla.Weights._fields_})
    st = lib.mla_cache_write(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), 4096,
                             ctypes.byref(cache), None)
    assert st == code, (kw, mla.status_string(st), mla.last_error())
    n = mla.workspace_bytes(cfg, ch)
    st = lib.mla_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), 4096,
                      ctypes.byref(cache), 4096, 4096, n, None)
    assert st == code, (kw, mla.status_string(st), mla.last_error())


@pytest.mark.parametrize("freq,code", [
    ((0.0,) * 16, mla.MLA_OK),                      # all zero: derived from theta
    (tuple(0.1 * (i + 1) for i in range(16)), mla.MLA_OK),
    ((0.0,) * 15 + (2.5,), mla.MLA_OK),              # one set entry makes the table explicit
    ((float("nan"),) + (0.1,) * 15, mla.MLA_ERR_INVALID_ARG),
    ((0.1,) * 15 + (float("inf"),), mla.MLA_ERR_INVALID_ARG),
])
def test_rope_freq_table_rules(freq, code):
    s = W.shape_by_name("wan1.3b-w21").with_(rope_freq=freq)
    assert mla.validate(mla.make_config(s), chunk_of(s)) == code, mla.last_error()


def test_explicit_table_makes_theta_unused():
    """rope_theta is only needed when the table is derived from it."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s.with_(rope_freq=(0.3,) * 16))
    cfg.rope_theta = 0.0
    assert mla.validate(cfg, chunk_of(s)) == mla.MLA_OK
    cfg = mla.make_config(s)
    cfg.rope_theta = 0.0
    assert mla.validate(cfg, chunk_of(s)) == mla.MLA_ERR_INVALID_ARG


# ---------------------------------------------------------------- failure injection
def test_fault_injection_reaches_every_launching_entry_point(monkeypatch):
    """MLA_FAULT_INJECT=launch: every entry point that would launch returns
    MLA_ERR_HIP after its argument checks, with the injection named in
    mla_last_error(); invalid arguments still give their own codes first; unset,
    the hook is inert (host-only calls are unaffected either way)."""
    lib = mla.load()
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    ch = chunk_of(s)
    n = mla.workspace_bytes(cfg, ch)
    cache = fake_cache(cfg)
    w = mla.Weights(**{k: 4096 for k, _ in mla.Weights._fields_})
    monkeypatch.setenv("MLA_FAULT_INJECT", "launch")
    calls = {
        "mla_cache_write": lambda: lib.mla_cache_write(ctypes.byref(cfg), ctypes.byref(w),
                                                       ctypes.byref(ch), 4096,
                                                       ctypes.byref(cache), None),
        "mla_chunk_attention": lambda: lib.mla_chunk_attention(
            ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), 4096, ctypes.byref(cache), 4096,
            4096, n, None),
        "mla_step": lambda: lib.mla_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch),
                                         4096, ctypes.byref(cache), 4096, 4096, n, None),
        "mla_latent_attention": lambda: lib.mla_latent_attention(
            ctypes.byref(cfg), ctypes.byref(ch), 4096, ctypes.byref(cache), 4096, 4096, n, None),
        "mla_value_absorbed_weights": lambda: lib.mla_value_absorbed_weights(
            ctypes.byref(cfg), ctypes.byref(w), 4096, None),
        "mla_query_absorbed_weights": lambda: lib.mla_query_absorbed_weights(
            ctypes.byref(cfg), ctypes.byref(w), 4096, None),
    }
    for name, call in calls.items():
        assert call() == mla.MLA_ERR_HIP, name
        assert "MLA_FAULT_INJECT" in mla.last_error(), name
    # argument errors come first
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, 16, None) == mla.MLA_ERR_WORKSPACE
    # host-only calls never launch, so they are unaffected
    assert mla.validate(cfg, ch) == mla.MLA_OK and mla.workspace_bytes(cfg, ch) == n
    assert mla.last_error() == ""
    monkeypatch.setenv("MLA_FAULT_INJECT", "something-else")
    assert lib.mla_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ch), 4096,
                        ctypes.byref(cache), 4096, 4096, 16, None) == mla.MLA_ERR_WORKSPACE


def test_binding_raises_on_injected_launch_failure(monkeypatch):
    """The Python binding turns MLA_ERR_HIP into MLAError carrying the status and the
    library's message."""
    monkeypatch.setenv("MLA_FAULT_INJECT", "launch")
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    w = mla.Weights(**{k: 4096 for k, _ in mla.Weights._fields_})

    class FakeTensor:
        def data_ptr(self):
            return 4096
    with pytest.raises(mla.MLAError) as e:
        mla.cache_write(cfg, w, chunk_of(s), FakeTensor(), fake_cache(cfg), stream=0)
    assert e.value.status == mla.MLA_ERR_HIP and "MLA_FAULT_INJECT" in str(e.value)


def test_static_step_refuses_problems_beyond_its_scratch(monkeypatch):
    """mla_step_static's scratch holds MLA_STATIC_SCRATCH_BYTES: a problem whose
    workspace would be larger (three Wan-1.3B requests in one call) is refused on the
    host with MLA_ERR_WORKSPACE and a message naming both sizes; one request fits
    and gets as far as the launch (refused here by the injection)."""
    monkeypatch.setenv("MLA_FAULT_INJECT", "launch")
    lib = mla.load()
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    w = mla.Weights(**{k: 4096 for k, _ in mla.Weights._fields_})
    one, three = chunk_of(s), chunk_of(s, batch=3)
    assert mla.workspace_bytes(cfg, one) <= mla.MLA_STATIC_SCRATCH_BYTES
    assert mla.workspace_bytes(cfg, three) > mla.MLA_STATIC_SCRATCH_BYTES
    c1, c3 = fake_cache(cfg, 1), fake_cache(cfg, 3)
    st = lib.mla_step_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(three), 4096,
                             ctypes.byref(c3), 4096, None)
    assert st == mla.MLA_ERR_WORKSPACE
    assert str(mla.MLA_STATIC_SCRATCH_BYTES) in mla.last_error()
    st = lib.mla_step_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(one), 4096,
                             ctypes.byref(c1), 4096, None)
    assert st == mla.MLA_ERR_HIP and "MLA_FAULT_INJECT" in mla.last_error()
    # argument checks as mla_step's
    assert lib.mla_step_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(one), 4097,
                               ctypes.byref(c1), 4096, None) == mla.MLA_ERR_ALIGNMENT
    assert lib.mla_step_static(None, None, None, None, None, None, None) == mla.MLA_ERR_INVALID_ARG


def test_overflow_flag_location():
    """The overflow flags lie inside the workspace, one per row tile of the fast
    kernel (256 query rows: 56160 rows at the Wan-1.3B chunk -> 220 tiles); none on
    the fp32 path."""
    s = W.shape_by_name("wan1.3b-w21")
    cfg = mla.make_config(s)
    off, n = mla.overflow_flags(cfg, chunk_of(s))
    assert n == (4680 * 12 + 255) // 256 and off % 256 == 0
    assert off + 4 * n <= mla.workspace_bytes(cfg, chunk_of(s))
    t = W.shape_by_name("tiny-f32")
    assert mla.overflow_flags(mla.make_config(t), chunk_of(t))[1] == 0
