"""Benchmark: sliding-window attention prefill (and ring-buffer decode) on one MI355X.

One step = one swa_prefill over the Mistral-7B-shaped layer (B=1, H_q=32, H_kv=8, N=32768,
d=128, w=4096, softmax, RoPE theta 1e6, bf16 in / fp32 accumulate, float32 output), the
largest single-GPU prefill workload, with inputs already in HBM. The value is in-window
TFLOP/s: 4 * B * H_q * d * sum_i |K(i)| per step, counting only the two contractions inside
the band (SWAT: Sliding Window Attention Training, linear O(N w) cost), divided by the timed
wall clock of K steps. After the W warm-up steps the step keeps running untimed for 0.2 s
(settle_steps in the line): the GPU's clocks ramp up over the first milliseconds of
sustained load, and the timed steps should see the steady state.

The JSON line also carries:
  roofline      the headline prefill call against the bf16 matrix-core peak, with its
                average launch duration timed by HIP events on the launch stream;
  prefill_legs  the other prefill workloads (the Gemma-3-style 128K local layer, the
                SWAT-340M layer) and bf16-output variants, each timed the same way with
                its own roofline;
  decode        the SWA(64, 4) decode workload (64 sequences, 256 steps of ring append +
                decode) in tokens/s and algorithmic GB/s against HBM peak, with the cache
                resident in the last-level cache (as specified) and, as decode_cold, with 18
                cache copies in rotation so that the rings come from HBM; decode_long adds
                two long-window decode workloads and decode_global a global layer over a
                131,072-token cache, whose caches live in HBM;
  chunk_prefill chunked prefill over the ring cache (8 prompts x 2048 rows per step at the
                Mistral-7B layer shape, histories past the 4,096-token window), in-window
                TFLOP/s of whole swa_prefill_chunk calls;
  backward      the training backward (swa_prefill_backward) of the SWAT-340M and
                Mistral-7B-shaped layers, in TFLOP/s of its five band contractions;
  elementwise   the standalone rotation (swa_rope_apply on the SWAT layer's q) and ring
                append (a 2,048-token chunk into 4,096-slot rings), GB/s against HBM;
  cpu_baseline  the float64 CPU oracle timed on the host cores on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "SWA prefill in-window TFLOP/s (% MFMA peak); decode tok/s (% HBM BW)"
KERNEL_SRC = os.path.join(ROOT, "sliding_window_attention_prefill_amd", "csrc", "prefill_mfma.hip")
SETTLE_S = 0.2   # untimed steady load before the timed prefill steps (clock ramp-up)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.json")
DECODE_SRC = os.path.join(ROOT, "sliding_window_attention_prefill_amd", "csrc", "decode.hip")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def in_window_keys(N: int, w: int, s: int) -> int:
    """sum_i |K(i)| with |K(i)| = min(i+1, w+s)."""
    c = w + s
    if N <= c:
        return N * (N + 1) // 2
    return c * (c + 1) // 2 + (N - c) * c


def prefill_flops(cfg) -> float:
    return 4.0 * cfg.B * cfg.H_q * cfg.d * in_window_keys(cfg.N, cfg.w, cfg.s)


def prefill_bytes(cfg, out_bytes: int) -> float:
    el = 2 if cfg.dtype == "bf16" else 4
    q = cfg.B * cfg.N * cfg.H_q * cfg.d
    kv = cfg.B * cfg.N * cfg.H_kv * cfg.d
    return float(q * el + 2 * kv * el + q * out_bytes)


def kernel_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(workload: str, out_dtype: str, path: str = TRAFFIC_FILE,
                   src: str = KERNEL_SRC):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from a committed
    counter profile, if it was taken on the current kernel source: one prefill call
    (pre-pass + main kernel), or one fused append + decode launch."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash(src):
        return None
    e = t.get("workloads", {}).get("%s/%s" % (workload, out_dtype))
    return None if e is None else e.get("hbm_bytes_per_launch")


def bench_prefill(cfg, steps: int, warmup: int, out_dtype):
    import torch
    import sliding_window_attention_prefill_amd as swa
    import swa_workloads as wl

    q, k, v = wl.prefill_inputs(cfg, device="cuda")
    slopes = wl.slopes_tensor(cfg.slopes, device="cuda")
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta) if cfg.rope_theta > 0 else None
    out = torch.empty((cfg.B, cfg.N, cfg.H_q, cfg.d), dtype=out_dtype, device="cuda")
    ws_bytes = swa.swa_prefill_workspace_bytes(q, k, w=cfg.w, s=cfg.s, mode=cfg.mode,
                                               out_dtype=out_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        swa.swa_prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, alibi_slopes=slopes,
                        rope_table=table, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the GPU's clocks ramp up over the first few milliseconds of sustained load: keep
    # stepping (untimed) until SETTLE_S of it has passed, so the timed steps see the
    # steady state (reported as settle_steps)
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        settle += 10
        torch.cuda.synchronize()
    # per-launch HIP events on the launch stream give the kernel's average duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    return wall, kernel_ms, settle


def bench_decode(cfg, out_dtype, copies=1):
    """cfg.steps steps of ring append + decode (one fused launch per step), captured once
    in a HIP graph so the launches replay without host overhead; timed over the whole
    replay. With copies > 1, step t works on cache copy t % copies, so that the copies
    together outgrow the 256 MB last-level cache and each step reads its ring from HBM (the
    step's work is the same)."""
    import torch
    import sliding_window_attention_prefill_amd as swa
    import swa_workloads as wl

    st = wl.decode_inputs(cfg, device="cuda")
    T, S = cfg.steps, cfg.num_seqs
    clone = lambda t: None if t is None else t.clone()
    caches = [swa.SwaCache(clone(st.k_ring), clone(st.v_ring), clone(st.k_sink),
                           clone(st.v_sink)) for _ in range(copies)]
    cache = caches[0]
    table = swa.swa_rope_table(cfg.len_hi + T + 1, cfg.d, cfg.rope_theta)
    pos = torch.stack([(st.lengths + t).to(torch.int32) for t in range(T)]).contiguous()
    out = torch.empty((T, S, cfg.H_q, cfg.d), dtype=out_dtype, device="cuda")
    ws_bytes = swa.swa_decode_workspace_bytes(cache, cfg.H_q, mode=cfg.mode, out_dtype=out_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()

    k_steps = st.k_steps[:, :, 0].contiguous()   # [T, S, H_kv, d]
    v_steps = st.v_steps[:, :, 0].contiguous()

    def run_all():
        # one launch per step: append the step's token and answer its query
        for t in range(T):
            swa.swa_decode_append(st.q_steps[t], k_steps[t], v_steps[t], pos[t],
                                  caches[t % copies], mode=cfg.mode, rope_table=table,
                                  out=out[t], workspace=ws, stream=stream)

    with torch.cuda.stream(stream):
        run_all()                     # warm-up, eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run_all()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(reps):
        graph.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    el = 2
    cache_bytes = sum(t.numel() * t.element_size() for t in
                      (cache.k_ring, cache.v_ring, cache.k_sink, cache.v_sink) if t is not None)
    ob = 4 if out_dtype == torch.float32 else 2
    # keys read per step: |K(p)| = min(p + 1, w + s) for each sequence's query position p
    # (w + s once a sequence is past its window; the whole history for a global layer)
    lens = st.lengths.to(torch.int64).cpu()
    keys_all = sum(int(torch.clamp(lens + t + 1, max=cfg.w + cfg.s).sum()) for t in range(T))
    per_step = (cfg.H_kv * keys_all / T * cfg.d * el * 2    # ring + sink K and V read
                + S * cfg.H_q * cfg.d * el                  # q read
                + S * cfg.H_q * cfg.d * ob                  # o written
                + 2 * S * cfg.H_kv * cfg.d * el * 2)        # append: new k, v read + written
    per_step = int(round(per_step))
    secs = ms / 1e3
    gbs = per_step * T / secs / 1e9
    return {
        "workload": cfg.name, "steps": T, "sequences": S,
        "ms_total": round(ms, 4), "us_per_step": round(ms * 1e3 / T, 3),
        "tok_per_s": round(S * T / secs, 1),
        "algorithmic_bytes_per_step": per_step,
        "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "cache_copies": copies,
        "cache_mb": round(copies * cache_bytes / 1e6, 1),
        # counters see the eager launches of the same rotation (graph replays are not
        # counted), so the bytes stand for the HBM-resident case only
        "traffic": (stored_traffic(cfg.name, "f32" if out_dtype == torch.float32 else "bf16",
                                   DECODE_TRAFFIC_FILE, DECODE_SRC) if copies > 1 else None),
        "note": ("cache (%.0f MB) %s the 256 MB last-level cache" % (
                     cache_bytes / 1e6, "fits in" if cache_bytes < 200e6 else "outgrows")
                 if copies == 1 else "%d cache copies in rotation: rings are read from HBM"
                 % copies),
    }


def _event_ms(fn, reps: int = 20) -> float:
    """Average duration of fn() over reps calls, from HIP events on the current stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_elementwise():
    """The standalone rotation and ring append, HBM-bound: swa_rope_apply in place on the
    SWAT-340M layer's q [8, 4096, 16, 64] bf16, and swa_kv_append of a 2,048-token chunk per
    sequence (8 sequences, 8 kv heads, d 128, bf16) into 4,096-slot rings. Algorithmic
    bytes: every element read and written once, plus the rotation angles of each position
    (float32 cos, sin per pair) once."""
    import torch
    import sliding_window_attention_prefill_amd as swa
    import swa_workloads as wl

    out = []
    cfg = wl.C2
    q, _, _ = wl.prefill_inputs(cfg, device="cuda")
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta)
    pos0 = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    ms = _event_ms(lambda: swa.swa_rope_apply(q, pos0, table))
    nbytes = 2 * q.numel() * 2 + cfg.B * cfg.N * (cfg.d // 2) * 8
    out.append({"op": "swa_rope_apply", "workload": "q_bf16_B8_N4096_H16_d64", "us_per_call": round(ms * 1e3, 2),
                "algorithmic_bytes": nbytes, "GB_per_s": round(nbytes / ms / 1e6, 1),
                "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)})
    S, n_new, Hkv, d, w = 8, 2048, 8, 128, 4096
    g = torch.Generator(device="cuda").manual_seed(7)
    k = torch.randn((S, n_new, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((S, n_new, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    cache = swa.SwaCache.empty(S, Hkv, w, 0, d, torch.bfloat16, device="cuda")
    table = swa.swa_rope_table(w + n_new, d, 1e6)
    pos = torch.full((S,), 1000, dtype=torch.int32, device="cuda")
    ms = _event_ms(lambda: swa.swa_kv_append(cache, k, v, pos, rope_table=table))
    nbytes = 2 * (2 * k.numel() * 2) + S * n_new * (d // 2) * 8
    out.append({"op": "swa_kv_append", "workload": "chunk2048_bf16_S8_Hkv8_d128_w4096", "us_per_call": round(ms * 1e3, 2),
                "algorithmic_bytes": nbytes, "GB_per_s": round(nbytes / ms / 1e6, 1),
                "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)})
    return out


def bench_chunk(cfg, out_dtype):
    """Chunked prefill over the ring cache: step t prefills rows [hist + t * chunk, hist +
    (t + 1) * chunk) of every sequence (gather, attention, append in one swa_prefill_chunk
    call), so each step reads the history the previous step appended. HIP events around
    each call on its stream; one untimed call on a separate copy of the cache first."""
    import torch
    import sliding_window_attention_prefill_amd as swa
    import swa_workloads as wl

    st = wl.chunk_inputs(cfg, device="cuda")
    S, C, T = cfg.num_seqs, cfg.chunk, cfg.num_seqs * cfg.chunk
    clone = lambda t: None if t is None else t.clone()
    make = lambda: swa.SwaCache(clone(st.k_ring), clone(st.v_ring), clone(st.k_sink),
                                clone(st.v_sink))
    table = swa.swa_rope_table(cfg.hist_hi + (cfg.steps + 1) * C + 1, cfg.d, cfg.rope_theta)
    cu = (torch.arange(S + 1, dtype=torch.int32, device="cuda") * C).contiguous()
    pos = [(st.hist + t * C).to(torch.int32).to("cuda") for t in range(cfg.steps)]
    out = torch.empty((T, cfg.H_q, cfg.d), dtype=out_dtype, device="cuda")
    warm = make()
    need = swa.swa_prefill_chunk_workspace_bytes(warm, cfg.H_q, T, C, mode=cfg.mode,
                                                 rope_table=table)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()

    def call(cache, p):
        swa.swa_prefill_chunk(st.q, st.k, st.v, cu, p, cache, max_seqlen=C, mode=cfg.mode,
                              rope_table=table, out=out, workspace=ws, stream=stream)

    call(warm, pos[0])
    cache = make()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(cfg.steps)]
    for t in range(cfg.steps):
        ev[t][0].record(stream)
        call(cache, pos[t])
        ev[t][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / cfg.steps
    # every row's key set is the whole window (histories start past w + s)
    flops = 4.0 * cfg.H_q * cfg.d * T * (cfg.w + cfg.s)
    tf = flops / (ms / 1e3) / 1e12
    return {
        "workload": cfg.name, "sequences": S, "rows_per_sequence": C, "steps": cfg.steps,
        "ms_per_step": round(ms, 4), "rows_per_s": round(T / (ms / 1e3), 1),
        "in_window_flops_per_step": flops, "TFLOP_s": round(tf, 2),
        "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "one call per step: gather pre-pass, matrix-core attention, append",
    }


def bench_backward(cfg, steps: int = 5):
    """The backward of one prefill layer (swa_prefill_backward: pre-passes, dk/dv and dq
    kernels) given the forward's o and lse, bf16 gradients; HIP events around each call on
    its stream. Algorithmic FLOPs: the score recompute and the four gradient products,
    5 x 2d per in-window (query, key) pair = 2.5 x the forward's."""
    import torch
    import sliding_window_attention_prefill_amd as swa
    import swa_workloads as wl

    q, k, v = wl.prefill_inputs(cfg, device="cuda")
    sl = wl.slopes_tensor(cfg.slopes, device="cuda")
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta)
    o, lse = swa.swa_prefill_train(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, alibi_slopes=sl,
                                   rope_table=table, out_dtype=torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 100)
    dout = torch.randn(o.shape, generator=g, device="cuda").to(torch.bfloat16)
    grads = tuple(torch.empty(t.shape, dtype=torch.bfloat16, device="cuda") for t in (q, k, v))
    need = swa.swa_prefill_backward_workspace_bytes(q, k, w=cfg.w, s=cfg.s, mode=cfg.mode)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()

    def call():
        swa.swa_prefill_backward(q, k, v, o, lse, dout, w=cfg.w, s=cfg.s, mode=cfg.mode,
                                 alibi_slopes=sl, rope_table=table, grads=grads, workspace=ws,
                                 stream=stream)

    call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = 2.5 * prefill_flops(cfg)
    tf = flops / (ms / 1e3) / 1e12
    return {"workload": cfg.name, "ms_per_call": round(ms, 4), "algorithmic_flops": flops,
            "TFLOP_s": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "note": "bf16 gradients; pre-passes, dk/dv and dq kernels"}


def cpu_baseline(cfg, sample_rows: int):
    """The float64 oracle on a bounded sample of the workload: the last `sample_rows` query
    rows of the first sequence, every head (rows past the window edge, each with a full key
    set), timed on the host; reported in the metric's unit (in-window FLOPs of the sample
    per second)."""
    import oracle
    import swa_workloads as wl

    sub = cfg.with_(B=1)
    q, k, v = wl.prefill_inputs(sub, device="cpu")
    n = min(sample_rows, cfg.N)
    rows = list(range(cfg.N - n, cfg.N))
    oracle.build()
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, w=sub.w, s=sub.s, mode=sub.mode, slopes=sub.slopes,
                   rope_theta=sub.rope_theta, rows=rows)
    secs = time.perf_counter() - t0
    keys = sum(min(i + 1, cfg.w + cfg.s) for i in rows)
    flops = 4.0 * cfg.H_q * cfg.d * keys
    return {
        "value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s",
        "cores": oracle.threads(), "cpu": oracle.cpu_model(), "kind": "oracle",
        "sample": "rows %d..%d of %d of sequence 0 (all %d heads, %.3g in-window FLOPs): "
                  "%.1f s" % (rows[0], rows[-1], cfg.N, cfg.H_q, flops, secs),
    }


def prefill_line(cfg, steps: int, warmup: int, out_name: str):
    """One prefill workload timed as the headline step is: (wall, kernel_ms, settle) plus
    its roofline object."""
    import torch
    out_dtype = torch.float32 if out_name == "f32" else torch.bfloat16
    wall, kernel_ms, settle = bench_prefill(cfg, steps, warmup, out_dtype)
    flops = prefill_flops(cfg)
    achieved = flops / (kernel_ms / 1e3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": stored_traffic(cfg.name, out_name), "kernel_ms": round(kernel_ms, 5),
            "algorithmic_bytes": prefill_bytes(cfg, 4 if out_name == "f32" else 2)}
    return wall, kernel_ms, settle, roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c5"])
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-elementwise", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192,
                    help="query rows of sequence 0 the CPU baseline computes")
    ap.add_argument("--profile-decode-cold", type=int, default=0, metavar="STEPS",
                    help="only run STEPS fused append + decode launches of the SWA(64, 4) "
                         "workload eagerly over 18 cache copies in rotation (for byte "
                         "counters, which see eager launches), then exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes three times (the "
                         "known-size kernel that scales the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the workloads "
              "fit one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import swa_workloads as wl

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)
        return

    if args.profile_decode_cold:
        import sliding_window_attention_prefill_amd as swa
        c = wl.C4
        st = wl.decode_inputs(c, device="cuda", steps=1)
        copies = 18
        caches = [swa.SwaCache(st.k_ring.clone(), st.v_ring.clone(), st.k_sink.clone(),
                               st.v_sink.clone()) for _ in range(copies)]
        table = swa.swa_rope_table(c.len_hi + args.profile_decode_cold + 1, c.d, c.rope_theta)
        out = torch.empty((c.num_seqs, c.H_q, c.d), dtype=torch.float32, device="cuda")
        kn, vn = st.k_steps[0, :, 0].contiguous(), st.v_steps[0, :, 0].contiguous()
        for t in range(args.profile_decode_cold):
            pos = (st.lengths + t).to(torch.int32)
            swa.swa_decode_append(st.q_steps[0], kn, vn, pos, caches[t % copies], mode=c.mode,
                                  rope_table=table, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"decode_cold_eager_steps": args.profile_decode_cold,
                          "cache_copies": copies}), flush=True)
        return

    cfgs = {"c2": wl.C2, "c3": wl.C3, "c5": wl.C5}
    cfg = cfgs[args.workload]
    wall, kernel_ms, settle, roof = prefill_line(cfg, args.steps, args.warmup, args.out_dtype)
    flops = prefill_flops(cfg)
    value = flops * args.steps / wall / 1e12
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settle,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H_q": cfg.H_q, "H_kv": cfg.H_kv,
                   "N": cfg.N, "d": cfg.d, "w": cfg.w, "s": cfg.s,
                   "mode": "sigmoid" if cfg.mode == wl.SIGMOID else "softmax",
                   "out_dtype": args.out_dtype, "in_window_flops": flops},
        "roofline": roof,
    }
    if not args.no_legs:
        legs = []
        order = [("c5", "f32"), ("c2", "f32"), ("c3", "bf16"), ("c5", "bf16"), ("c2", "bf16")]
        for name, od in order:
            if name == args.workload and od == args.out_dtype:
                continue
            c = cfgs[name]
            lw, lk, _, lroof = prefill_line(c, args.steps, args.warmup, od)
            legs.append({"workload": c.name, "out_dtype": od,
                         "ms_per_step": round(lw * 1e3 / args.steps, 4),
                         "TFLOP_s": round(prefill_flops(c) * args.steps / lw / 1e12, 2),
                         "roofline": lroof})
        result["prefill_legs"] = legs
    if not args.no_decode:
        result["decode"] = bench_decode(wl.C4, torch.float32)
        result["decode_cold"] = bench_decode(wl.C4, torch.float32, copies=18)
        result["decode_long"] = [bench_decode(c, torch.float32)
                                 for c in (wl.DECODE_W4096, wl.DECODE_W32K)]
        result["decode_global"] = bench_decode(wl.DECODE_GLOBAL_128K, torch.float32)
    if not args.no_chunk:
        result["chunk_prefill"] = bench_chunk(wl.CHUNK_W4096, torch.float32)
    if not args.no_elementwise:
        result["elementwise"] = bench_elementwise()
    if not args.no_backward:
        result["backward"] = [bench_backward(c) for c in (wl.C2, wl.C3)]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
