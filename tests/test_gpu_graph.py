"""HIP graph capture of the library's calls (torch.cuda.CUDAGraph around calls through the C ABI).

The library allocates nothing, waits on nothing and records no memset, so a serving or training
loop can capture a call once and replay it. Each test captures one call with its outputs and
workspace allocated beforehand, then replays it several times. Before every replay it refills
the inputs in place, runs the same call eagerly into separate outputs, and synchronises. Every
replay must give the eager call's bits: the kernels are deterministic, and a replay reads
whatever the captured buffers hold at that moment. The last test runs calls concurrently on
separate streams.
"""
import numpy as np
import pytest
import torch

import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 3


def _fill(g, *ts):
    for t in ts:
        t.copy_((torch.randn(t.shape, generator=g) * 0.5).to(t.dtype))


def _capture(fn):
    fn()                                  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _clone_cache(c):
    return swa.SwaCache(c.k_ring.clone(), c.v_ring.clone(),
                        None if c.s == 0 else c.k_sink.clone(), None if c.s == 0 else c.v_sink.clone())


def _copy_cache(dst, src):
    dst.k_ring.copy_(src.k_ring)
    dst.v_ring.copy_(src.v_ring)
    if src.s > 0:
        dst.k_sink.copy_(src.k_sink)
        dst.v_sink.copy_(src.v_sink)


def _caches_equal(a, b):
    same = torch.equal(a.k_ring, b.k_ring) and torch.equal(a.v_ring, b.v_ring)
    if a.s > 0:
        same = same and torch.equal(a.k_sink, b.k_sink) and torch.equal(a.v_sink, b.v_sink)
    return same


@pytest.mark.parametrize("d,mode,Hq,Hkv,dil", [(64, wl.SIGMOID, 4, 4, 1), (128, wl.SOFTMAX, 8, 2, 1),
                                               (64, wl.SOFTMAX, 4, 2, 3)])
def test_prefill_replays_match_eager(d, mode, Hq, Hkv, dil):
    """swa_prefill (pre-pass + main kernel; with dilation 3, six launches) in a graph."""
    B, N, w, s, theta = 2, 333, 90, 0 if dil > 1 else 3, 1e4
    g = torch.Generator().manual_seed(d + Hq + dil)
    q = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    _fill(g, q, k, v)
    sl = torch.tensor(np.linspace(-0.5, 0.5, Hq), dtype=torch.float32, device=DEV)
    table = swa.swa_rope_table(N, d, theta)
    kw = dict(w=w, s=s, mode=mode, alibi_slopes=sl, rope_table=table, dilation=dil)
    need = swa.swa_prefill_workspace_bytes(q, k, w=w, s=s, mode=mode, out_dtype=torch.float32,
                                           dilation=dil)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=DEV)
    out_g = torch.empty((B, N, Hq, d), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    graph = _capture(lambda: swa.swa_prefill(q, k, v, out=out_g, workspace=ws, **kw))
    for rep in range(REPLAYS):
        _fill(g, q, k, v)
        swa.swa_prefill(q, k, v, out=out_e, workspace=ws, **kw)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d" % rep


@pytest.mark.parametrize("d,mode", [(64, wl.SIGMOID), (128, wl.SOFTMAX)])
def test_backward_replays_match_eager(d, mode):
    """swa_prefill_backward (two pre-passes, dk/dv, sink splits, dq) in a graph."""
    B, N, Hq, Hkv, w, s, theta = 1, 1400, 4, 2, 64, 2, 1e4   # sinks past the window: split workgroups
    g = torch.Generator().manual_seed(10 + d)
    q = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    dout = torch.empty((B, N, Hq, d), dtype=torch.float32, device=DEV)
    _fill(g, q, k, v, dout)
    sl = torch.tensor(np.linspace(-0.3, 0.3, Hq), dtype=torch.float32, device=DEV)
    table = swa.swa_rope_table(N, d, theta)
    kw = dict(w=w, s=s, mode=mode, alibi_slopes=sl, rope_table=table)
    o, lse = swa.swa_prefill_train(q, k, v, out_dtype=torch.float32, **kw)
    need = swa.swa_prefill_backward_workspace_bytes(q, k, w=w, s=s, mode=mode,
                                                    grad_dtype=torch.float32)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=DEV)
    grads_g = tuple(torch.empty(t.shape, dtype=torch.float32, device=DEV) for t in (q, k, v))
    grads_e = tuple(torch.empty_like(t) for t in grads_g)
    graph = _capture(lambda: swa.swa_prefill_backward(q, k, v, o, lse, dout, grads=grads_g,
                                                      workspace=ws, **kw))
    for rep in range(REPLAYS):
        _fill(g, dout)
        swa.swa_prefill_backward(q, k, v, o, lse, dout, grads=grads_e, workspace=ws, **kw)
        torch.cuda.synchronize()
        for t in grads_g:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), grads_g, grads_e):
            assert torch.equal(a, b), "replay %d %s" % (rep, name)


def test_chunk_replays_match_eager():
    """swa_prefill_chunk (gather pre-pass, main kernel, append) in a graph: the replay reads
    the cache as it stands and appends the chunk, like the eager call."""
    S, Hq, Hkv, d, w, s, theta, chunk, hist = 2, 8, 2, 128, 200, 3, 1e4, 96, 150
    g = torch.Generator().manual_seed(3)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    table = swa.swa_rope_table(hist + chunk, d, theta)
    k_hist = torch.empty((S, hist, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v_hist = torch.empty_like(k_hist)
    _fill(g, k_hist, v_hist)
    swa.swa_kv_append(cache, k_hist, v_hist, torch.zeros(S, dtype=torch.int32, device=DEV),
                      rope_table=table)
    base = _clone_cache(cache)
    q = torch.empty((S * chunk, Hq, d), dtype=torch.bfloat16, device=DEV)
    kn = torch.empty((S * chunk, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    _fill(g, q, kn, vn)
    cu = torch.tensor([0, chunk, 2 * chunk], dtype=torch.int32, device=DEV)
    pos0 = torch.full((S,), hist, dtype=torch.int32, device=DEV)
    sl = torch.tensor(np.linspace(-0.4, 0.4, Hq), dtype=torch.float32, device=DEV)
    kw = dict(max_seqlen=chunk, mode=wl.SOFTMAX, alibi_slopes=sl, rope_table=table)
    need = swa.swa_prefill_chunk_workspace_bytes(cache, Hq, S * chunk, chunk)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=DEV)
    out_g = torch.empty((S * chunk, Hq, d), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    graph = _capture(lambda: swa.swa_prefill_chunk(q, kn, vn, cu, pos0, cache, out=out_g,
                                                   workspace=ws, **kw))
    for rep in range(REPLAYS):
        _fill(g, q, kn, vn)
        _copy_cache(cache, base)
        swa.swa_prefill_chunk(q, kn, vn, cu, pos0, cache, out=out_e, workspace=ws, **kw)
        after_eager = _clone_cache(cache)
        _copy_cache(cache, base)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d" % rep
        assert _caches_equal(cache, after_eager), "replay %d cache" % rep


@pytest.mark.parametrize("w,s", [(64, 4), (4096, 0)])
def test_decode_loop_replays_match_eager(w, s):
    """A decode loop: one fused append + decode captured once and replayed step after step,
    the positions advanced in place between steps (the replay reads them from the device),
    against the same steps run eagerly on a twin cache. w = 4096 takes the split-KV path."""
    S, Hq, Hkv, d, theta, start = 3, 8, 2, 128, 1e4, 300
    g = torch.Generator().manual_seed(w + s)
    table = swa.swa_rope_table(start + 16, d, theta)
    cache_e = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    k_hist = torch.empty((S, start, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v_hist = torch.empty_like(k_hist)
    _fill(g, k_hist, v_hist)
    swa.swa_kv_append(cache_e, k_hist, v_hist, torch.zeros(S, dtype=torch.int32, device=DEV),
                      rope_table=table)
    cache_g = _clone_cache(cache_e)
    scratch = _clone_cache(cache_e)       # warm-up target, so the graph's cache starts untouched
    q = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=DEV)
    kn = torch.empty((S, Hkv, d), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    _fill(g, q, kn, vn)
    pos = torch.full((S,), start, dtype=torch.int32, device=DEV)
    kw = dict(mode=wl.SOFTMAX, rope_table=table)
    need = swa.swa_decode_workspace_bytes(cache_e, Hq, mode=wl.SOFTMAX)
    ws_g = torch.empty(max(1, need), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws_g)
    out_g = torch.empty((S, Hq, d), dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(out_g)
    swa.swa_decode_append(q, kn, vn, pos, scratch, out=out_g, workspace=ws_g, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.swa_decode_append(q, kn, vn, pos, cache_g, out=out_g, workspace=ws_g, **kw)
    torch.cuda.synchronize()
    for step in range(4):
        _fill(g, q, kn, vn)
        swa.swa_decode_append(q, kn, vn, pos, cache_e, out=out_e, workspace=ws_e, **kw)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "step %d" % step
        assert _caches_equal(cache_g, cache_e), "step %d cache" % step
        pos += 1


def test_calls_on_separate_streams_run_concurrently():
    """The library holds no state, so calls on different streams may overlap: a prefill, a
    backward and a decode step enqueued on three streams (each with its own workspace) at
    once give the bits of the same calls run one after another."""
    g = torch.Generator().manual_seed(11)
    B, N, Hq, Hkv, d, w, theta = 1, 700, 8, 2, 128, 200, 1e4
    q = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    dout = torch.empty((B, N, Hq, d), dtype=torch.float32, device=DEV)
    _fill(g, q, k, v, dout)
    table = swa.swa_rope_table(N, d, theta)
    pkw = dict(w=w, s=2, mode=wl.SOFTMAX, rope_table=table)
    bkw = dict(w=w, s=0, mode=wl.SIGMOID, rope_table=table)
    o_sig, _ = swa.swa_prefill_train(q, k, v, out_dtype=torch.float32, **bkw)
    S = 4
    cache = swa.SwaCache.empty(S, Hkv, 64, 4, d, torch.bfloat16)
    hist = torch.empty((S, 100, Hkv, d), dtype=torch.bfloat16, device=DEV)
    hist_v = torch.empty_like(hist)
    _fill(g, hist, hist_v)
    swa.swa_kv_append(cache, hist, hist_v, torch.zeros(S, dtype=torch.int32, device=DEV),
                      rope_table=table)
    dq_ = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=DEV)
    dk_ = torch.empty((S, Hkv, d), dtype=torch.bfloat16, device=DEV)
    dv_ = torch.empty_like(dk_)
    _fill(g, dq_, dk_, dv_)
    pos = torch.full((S,), 100, dtype=torch.int32, device=DEV)
    twin = _clone_cache(cache)
    torch.cuda.synchronize()

    def run(streams, c):
        outs = {}
        with torch.cuda.stream(streams[0]):
            outs["prefill"] = swa.swa_prefill(q, k, v, out_dtype=torch.float32, **pkw)
        with torch.cuda.stream(streams[1]):
            outs["grads"] = swa.swa_prefill_backward(q, k, v, o_sig, None, dout, **bkw)
        with torch.cuda.stream(streams[2]):
            outs["decode"] = swa.swa_decode_append(dq_, dk_, dv_, pos, c, mode=wl.SOFTMAX,
                                                   rope_table=table, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return outs

    cur = torch.cuda.current_stream()
    seq = run([cur, cur, cur], twin)
    side = [torch.cuda.Stream() for _ in range(3)]
    for st in side:
        st.wait_stream(cur)
    par = run(side, cache)
    assert torch.equal(par["prefill"], seq["prefill"])
    for a, b in zip(par["grads"], seq["grads"]):
        assert torch.equal(a, b)
    assert torch.equal(par["decode"], seq["decode"])
    assert _caches_equal(cache, twin)
