"""Benchmark of the VideoMLA latent-KV chunk step on one MI355X.

A step is one mla_step call per layer: cache write of the 3-frame chunk into the
21-frame ring, query preparation, latent chunk attention over the whole window,
value up-projection and W_O, on the Wan-1.3B layer shape (bf16 storage, fp32
accumulation), inputs resident in HBM.  By default one layer; --layers 30 steps a
30-layer stack (independent seeded weights, inputs and rings per layer, one
stream, one shared workspace).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers L]
                  [--no-cpu-baseline]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def step_flops(s):
    """Algorithmic FLOP of one chunk step over the s.batch requests (each projection
    counted once, attention as one (d_c+d_rope)-wide score plus one d_c-wide latent
    value per (query, key, head))."""
    tq, nh = s.batch * s.chunk_tokens, s.n_heads
    write = 2 * tq * s.d_model * (s.d_c + s.d_rope)
    qprep = (2 * tq * s.d_model * s.d_q + 2 * tq * s.d_q * nh * (s.d_nope + s.d_rope)
             + 2 * tq * nh * s.d_nope * s.d_c)
    attn = attention_flops(s)
    vup = 2 * tq * nh * s.d_c * s.d_head
    out = 2 * tq * nh * s.d_head * s.d_model
    return {"write": write, "qprep": qprep, "attention": attn, "vup": vup, "out": out,
            "total": write + qprep + attn + vup + out}


def attention_flops(s):
    """Attended (query, key) pairs per head (the whole window, or with chunk-causal
    blocks the context up to each block's end) x heads x the two contractions."""
    from workload import attended_pairs
    return 2 * s.batch * attended_pairs(s) * s.n_heads * (2 * s.d_c + s.d_rope)


def cache_write_bytes(s):
    """Algorithmic HBM bytes of one cache write: read x and the two weights once,
    write the new ring rows (all s.batch requests)."""
    tq = s.batch * s.chunk_tokens
    return 2 * (tq * s.d_model + (s.d_c + s.d_rope) * s.d_model + tq * (s.d_c + s.d_rope))


class Hip:
    """hipEvent helpers from the HIP runtime (the library records into them)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        t = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return t.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(kernel_src, summary):
    """HBM bytes per launch from a committed PMC summary, if it was taken on the
    current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha256_16") != source_hash(kernel_src):
        return None
    return d.get("hbm_bytes_per_launch")


def spread(v):
    """mean, median, 10th and 90th percentile of a list of timings."""
    v = sorted(v)
    n = len(v)

    def q(p):
        return v[min(n - 1, max(0, int(round(p * (n - 1)))))]
    return {"mean": round(sum(v) / n, 4), "median": round(q(0.5), 4), "p10": round(q(0.1), 4),
            "p90": round(q(0.9), 4)}


def ceilings(hip, stream):
    """What this device sustains, next to the rated peaks the roofline uses: a loop of
    independent bf16 MFMAs (libmla_probe.so, not the MLA path) and a 1 GiB device
    copy (read + write bytes)."""
    import torch
    out = {}
    path = os.path.join(ROOT, "latent_kv_attention_down_amd", "libmla_probe.so")
    if os.path.exists(path):
        probe = ctypes.CDLL(path)
        probe.mla_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
        probe.mla_probe_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
        probe.mla_probe_mfma_bf16_flop.restype = ctypes.c_double
        blocks = torch.cuda.get_device_properties(0).multi_processor_count
        iters = 4096
        buf = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
        a, b = hip.event(), hip.event()
        best = None
        for _ in range(3):
            hip.record(a, stream)
            assert probe.mla_probe_mfma_bf16(blocks, iters, buf.data_ptr(), stream) == 0
            hip.record(b, stream)
            torch.cuda.synchronize()
            t = hip.ms(a, b)
            best = t if best is None else min(best, t)
        out["mfma_bf16_tflops"] = round(probe.mla_probe_mfma_bf16_flop(blocks, iters) / (best * 1e-3)
                                        / 1e12, 1)
        hip.destroy(a)
        hip.destroy(b)
    else:
        print(f"[bench] {path} missing: no MFMA ceiling", file=sys.stderr)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_gbs"] = round(2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    out["note"] = "measured here; roofline fractions use the rated 2.5 PF bf16 and 8 TB/s"
    return out


def cpu_baseline(s, w_exact, x_window, n_tokens):
    """The oracle (fp64 NumPy, unabsorbed) on a bounded sample: n_tokens evenly
    spaced query tokens of the chunk, all heads, the full window (cache entries and
    K/V reconstruction for every window token)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    rows = np.linspace(0, s.chunk_tokens - 1, n_tokens).round().astype(int)
    tpf = s.tokens_per_frame
    tokens = {f: x_window[i * tpf:(i + 1) * tpf] for i, f in enumerate(s.window_frame_ids)}
    t0 = time.perf_counter()
    r = O.step(s, w_exact, tokens, query_rows=rows)
    dt = time.perf_counter() - t0
    f1 = step_flops(s.with_(batch=1))
    vis = O.visible_keys(s, r["window_ids"], O.chunk_frame_ids(s))[rows]
    flops = ((f1["total"] - f1["attention"]) * n_tokens / s.chunk_tokens
             + 2 * float(vis.sum()) * s.n_heads * (2 * s.d_c + s.d_rope))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tokens} of {s.chunk_tokens} query tokens (all {s.n_heads} heads) over "
                      f"the full {s.window_tokens}-token window, fp64 NumPy; "
                      f"{dt:.1f} s wall; credited {flops / 1e12:.4f} TFLOP pro rata"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan1.3b-w21")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers per step, each with its own seeded weights, tokens and ring "
                         "(30: the Wan-1.3B backbone's attention layers)")
    ap.add_argument("--batch", type=int, default=1,
                    help="independent requests per step, each with its own cache")
    ap.add_argument("--epilogue", choices=("two-stage", "absorbed"), default="two-stage",
                    help="two-stage: per-head W^V_up then W_O; absorbed: y = sum_h B_h O_lat,h "
                         "with B_h = W_O,h W^V_up,h prepared once (FLOPs are counted as "
                         "two-stage either way)")
    ap.add_argument("--query", choices=("direct", "absorbed"), default="absorbed",
                    help="direct: W^Q_up, then (W^K_up,h)^T per head, and W^Q_R apart; "
                         "absorbed: each query row from c^Q in one GEMM with [(W^K_up,h)^T "
                         "W^Q_up,h ; W^Q_R,h] prepared once (FLOPs are counted as direct "
                         "either way)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4680)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB first (a known-size kernel "
                         "for scaling FETCH_SIZE/WRITE_SIZE counters); the run then makes no "
                         "other copies (no ceilings, no cold cache write)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA and copy ceilings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured run.", file=sys.stderr)
        sys.exit(2)
    if args.layers < 1:
        print("--layers must be >= 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import workload as W
    import latent_kv_attention_down_amd as mla
    from latent_kv_attention_down_amd.layer import DeviceLayer, WorkspacePool

    s = W.shape_by_name(args.workload).with_(batch=args.batch)
    NL = args.layers
    print(f"[bench] workload {s.name} x {NL} layer(s): {s.batch} x {s.chunk_tokens} query "
          f"tokens x {s.n_heads} heads over {s.window_tokens} keys", file=sys.stderr, flush=True)
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ids = s.window_frame_ids
    tpf = s.tokens_per_frame
    pool = WorkspacePool()
    layers = []  # (DeviceLayer, chunk tokens, y) per layer
    w_exact0 = xe0 = None
    for l in range(NL):
        stored, w_exact = W.draw_weights(s, layer=l)
        xs, xe = W.draw_frames(s, ids, layer=l)
        if l == 0:
            w_exact0, xe0 = w_exact, xe[0]
        L = DeviceLayer(s, stored, batch=s.batch, pool=pool)
        if args.epilogue == "absorbed":
            L.absorb_value()  # weight preparation, once, outside the timed region
        if args.query == "absorbed":
            L.absorb_query()  # likewise
        for i, f in enumerate(ids):
            if f >= s.t0:
                break
            L.cache_write(L.chunk(1, f, 1), L.tokens(xs[:, i * tpf:(i + 1) * tpf]))
        x = L.tokens(xs[:, -s.chunk_frames * tpf:])
        chunk = L.chunk(s.chunk_frames, s.t0, s.n_valid_frames, s.causal_frames)
        layers.append((L, x, L.new_out(chunk, s.d_model)))
        del xs, xe
        if NL > 1 and (l + 1) % 10 == 0:
            print(f"[bench] {l + 1} of {NL} layers prefilled", file=sys.stderr, flush=True)
    L0, x0, _ = layers[0]
    chunk = L0.chunk(s.chunk_frames, s.t0, s.n_valid_frames, s.causal_frames)
    ws = L0.workspace(chunk)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()

    def one_step(evs=None):
        for j, (L, x, y) in enumerate(layers):
            if evs is not None:
                mla.set_timing_events(evs[j][0], evs[j][1])
            mla.step(L.cfg, L.weights, chunk, x, L.cache_desc, y, ws, stream)

    K = args.steps
    # The chunk attention on its own (a2-a4: query preparation, latent attention,
    # per-head value up-projection with the merge of split row tiles), layer 0, back to
    # back, after the chunk's own frames are in the ring (a1).  It runs first, with ten
    # untimed calls of its own, so that neither it nor the step loop that follows at once
    # is timed while the GPU's clocks are still settling from idle (the first ~10 ms of
    # heavy work after an idle stretch run up to ~25% slower).
    mla.cache_write(L0.cfg, L0.weights, L0.chunk(s.chunk_frames, s.t0, s.n_valid_frames), x0,
                    L0.cache_desc, stream)
    out_heads = L0.new_out(chunk, s.n_heads * s.d_head)
    ca_ev = [(hip.event(), hip.event()) for _ in range(K)]
    ev = [[(hip.event(), hip.event()) for _ in range(NL)] for _ in range(K)]
    t_start, t_stop = hip.event(), hip.event()
    for _ in range(10):
        mla.chunk_attention(L0.cfg, L0.weights, chunk, x0, L0.cache_desc, out_heads, ws, stream)
    for a, b in ca_ev:
        hip.record(a, stream)
        mla.chunk_attention(L0.cfg, L0.weights, chunk, x0, L0.cache_desc, out_heads, ws, stream)
        hip.record(b, stream)

    # the step: W untimed warm-up steps, then K timed ones
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    hip.record(t_start, stream)
    for i in range(K):
        one_step(ev[i])
    hip.record(t_stop, stream)
    mla.set_timing_events(None, None)
    torch.cuda.synchronize()
    ms_total = hip.ms(t_start, t_stop)
    ms_step = ms_total / K
    ca_ms = [hip.ms(a, b) for a, b in ca_ev]
    ca_avg = sum(ca_ms) / K
    attn_ms = [hip.ms(a, b) for row in ev for a, b in row]
    attn_by_layer = [sum(hip.ms(*ev[i][j]) for i in range(K)) / K for j in range(NL)]
    attn_avg = sum(attn_ms) / len(attn_ms)
    for L, x, y in layers:
        assert torch.isfinite(y.float()).all(), "non-finite output"

    # cache write on its own: back-to-back launches between one pair of events
    wr_ch = L0.chunk(s.chunk_frames, s.t0, s.n_valid_frames)
    for _ in range(3):
        mla.cache_write(L0.cfg, L0.weights, wr_ch, x0, L0.cache_desc, stream)
    torch.cuda.synchronize()
    nw = max(K, 20)
    hip.record(t_start, stream)
    for _ in range(nw):
        mla.cache_write(L0.cfg, L0.weights, wr_ch, x0, L0.cache_desc, stream)
    hip.record(t_stop, stream)
    torch.cuda.synchronize()
    write_ms = hip.ms(t_start, t_stop) / nw
    device_bytes = {"cache_per_request_per_layer": L0.cache[0].numel() * L0.cache.element_size(),
                    "workspace": int(ws.numel()),
                    "peak_allocated": int(torch.cuda.max_memory_allocated())}

    # cold cache write: 1 GiB written before each launch evicts the 256 MB last-level
    # cache, so x and the weights come from HBM (skipped in counter-calibration runs,
    # whose only large copy must be the calibration one)
    cold_us = None
    if args.copy_calibration <= 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold_ev = [(hip.event(), hip.event()) for _ in range(10)]
        for a, b in cold_ev:
            flush.fill_(1)
            hip.record(a, stream)
            mla.cache_write(L0.cfg, L0.weights, wr_ch, x0, L0.cache_desc, stream)
            hip.record(b, stream)
        torch.cuda.synchronize()
        cold_us = [1e3 * hip.ms(a, b) for a, b in cold_ev]
        for a, b in cold_ev:
            hip.destroy(a)
            hip.destroy(b)
        del flush

    fl = step_flops(s)
    tflops = NL * fl["total"] / (ms_step * 1e-3) / 1e12
    kernel_tflops = fl["attention"] / (attn_avg * 1e-3) / 1e12
    ca_tflops = fl["attention"] / (ca_avg * 1e-3) / 1e12
    wbytes = cache_write_bytes(s)
    write_gbs = wbytes / (write_ms * 1e-3) / 1e9
    csrc = os.path.join(ROOT, "latent_kv_attention_down_amd", "csrc")
    traffic = traffic_from_profiles(os.path.join(csrc, "attention.hip"),
                                    "latent_attention_wan1.3b_w21_traffic.json")
    cw_traffic = traffic_from_profiles(os.path.join(csrc, "cache_write.hip"),
                                       "cache_write_wan1.3b_w21_traffic.json")

    line = {
        "metric": "MLA chunk-attention TFLOP/s + cache GB/s, Wan-1.3B shape, 21-frame window",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights; no trained model)",
        "config": {"workload": s.name if NL == 1 else f"{s.name}-{NL}layers", "layers": NL,
                   "batch": s.batch, "epilogue": args.epilogue, "query": args.query,
                   "query_tokens": s.chunk_tokens,
                   "window_tokens": s.window_tokens, "chunk_frames": s.chunk_frames,
                   "window_frames": s.window_frames, "heads": s.n_heads, "d_c": s.d_c,
                   "d_rope": s.d_rope, "d_model": s.d_model, "grid": [s.grid_h, s.grid_w],
                   "step_tflop": round(NL * fl["total"] / 1e12, 4)},
        "chunk_attention_tflops": round(ca_tflops, 2),
        "chunk_attention_ms": spread(ca_ms),
        "chunk_attention_note": "mla_chunk_attention timed whole (query preparation, latent "
                                "attention, per-head W^V_up with the merge of split row "
                                "tiles), attention FLOPs only",
        "fast_kernel_tflops": round(kernel_tflops, 2),
        "cache_write_gbs": round(write_gbs, 1),
        "cache_write_us": round(write_ms * 1e3, 2),
        "attention_ms": spread(attn_ms),
        "window_read_gbs": round(s.batch * s.window_tokens * (s.d_c + s.d_rope) * 2
                                 / (attn_avg * 1e-3) / 1e9, 1),
        "cache_write_cold_us": spread(cold_us) if cold_us else None,
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kernel_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "k_latent_attn_w1 (the dominant kernel: latent attention, "
                               "without the merge of split row tiles)",
                     "kernel_ms": round(attn_avg, 4)},
        "cache_write_roofline": {"bound": "hbm", "achieved": round(write_gbs, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(write_gbs / HBM_PEAK_GBS, 4),
                                 "traffic": cw_traffic,
                                 "kernel": "mla_cache_write",
                                 "bytes_per_launch": wbytes},
        "device_bytes": device_bytes,
        "ceilings": (None if args.no_ceilings or args.copy_calibration > 0
                     else ceilings(hip, stream)),
    }
    if NL > 1:
        line["attention_ms_by_layer"] = [round(v, 4) for v in attn_by_layer]
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(s, w_exact0, xe0, args.cpu_tokens)
    for row in ev:
        for a, b in row:
            hip.destroy(a)
            hip.destroy(b)
    for a, b in ca_ev:
        hip.destroy(a)
        hip.destroy(b)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
