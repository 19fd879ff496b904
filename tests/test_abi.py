"""The C-ABI library loads, exports every symbol include/swa.h declares, and rejects bad
arguments on the host before touching a device (no GPU needed: validation happens before
any HIP call)."""
import ctypes
import os
import re

import pytest

import sliding_window_attention_prefill_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(swa.LIB_PATH):
        from sliding_window_attention_prefill_amd import build
        build.build()
    return swa.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(swa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.swa_status_string(0) == b"ok"
    assert lib.swa_status_string(1) == b"invalid argument"
    assert lib.swa_status_string(2) == b"unsupported combination"
    assert lib.swa_status_string(3) == b"HIP runtime error"
    assert lib.swa_version() >= 100
    assert lib.swa_last_hip_error() == 0


def _params(**kw):
    base = dict(B=1, H_q=4, H_kv=2, N=16, d=64, w=4, s=0, mode=0, in_dtype=1, out_dtype=0,
                scale=0.0, alibi_slopes=None, rope_table=None, rope_rows=0)
    base.update(kw)
    return swa.PrefillParams(**base)


DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=3, H_kv=2), 1), (dict(H_kv=0), 1), (dict(B=-1), 1), (dict(N=-5), 1),
    (dict(d=63), 1), (dict(d=0), 1), (dict(w=0), 1), (dict(s=-1), 1), (dict(mode=2), 1),
    (dict(in_dtype=7), 1), (dict(out_dtype=-1), 1), (dict(scale=float("nan")), 1),
    (dict(rope_table=0x2000, rope_rows=8), 1), (dict(d=258), 2),
])
def test_prefill_rejects_bad_arguments(lib, kw, status):
    p = _params(**kw)
    assert lib.swa_prefill(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == status


def test_prefill_rejects_null_tensors(lib):
    p = _params()
    assert lib.swa_prefill(ctypes.byref(p), None, DUMMY, DUMMY, DUMMY, None, 0, None) == 1
    assert lib.swa_prefill(None, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == 1


def _tile_images(B, H_kv, N, d):
    # one float16 image of every 64-key tile of every (batch, kv head)
    return B * H_kv * ((N + 63) // 64) * 64 * d * 2


@pytest.mark.parametrize("kw,expect", [
    (dict(), "k"),                                       # sigmoid, 2 query heads per kv head
    (dict(H_q=2, H_kv=2), "k"),                          # sigmoid, one head per kv head
    (dict(mode=1), "kv"),                                # softmax packs K and V
    (dict(mode=1, N=1000, d=128), "kv"),
    (dict(in_dtype=0), 0),                               # float32 inputs: vector kernel
    (dict(d=96), 0),                                     # head size without a matrix path
    (dict(B=0), 0),
    (dict(w=0), 0),                                      # invalid parameters
])
def test_prefill_workspace_bytes(lib, kw, expect):
    p = _params(**kw)
    img = _tile_images(p.B, p.H_kv, p.N, p.d)
    want = {0: 0, "k": img, "kv": 2 * img}[expect]
    assert lib.swa_prefill_workspace_bytes(ctypes.byref(p)) == want


def test_prefill_rejects_missing_or_short_workspace(lib):
    p = _params(mode=1)
    need = lib.swa_prefill_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert lib.swa_prefill(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == 1
    assert lib.swa_prefill(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, need - 16,
                           None) == 1
    misaligned = ctypes.c_void_p(0x1008)
    assert lib.swa_prefill(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, misaligned, need,
                           None) == 1


def test_rope_table_rejects_bad_arguments(lib):
    assert lib.swa_rope_table(DUMMY, 10, 63, 1e4, None) == 1
    assert lib.swa_rope_table(DUMMY, 10, 64, 0.0, None) == 1
    assert lib.swa_rope_table(DUMMY, -1, 64, 1e4, None) == 1
    assert lib.swa_rope_table(None, 10, 64, 1e4, None) == 1


def _cache(**kw):
    base = dict(num_seqs=2, H_kv=2, w=8, s=2, d=64, dtype=1, reserved=0, k_ring=0x1000,
                v_ring=0x1000, k_sink=0x1000, v_sink=0x1000)
    base.update(kw)
    return swa.CacheDesc(**base)


@pytest.mark.parametrize("kw", [dict(w=0), dict(s=-1), dict(d=7), dict(H_kv=0), dict(dtype=5),
                                dict(k_ring=None), dict(k_sink=None)])
def test_append_rejects_bad_cache(lib, kw):
    c = _cache(**kw)
    assert lib.swa_kv_append(ctypes.byref(c), DUMMY, DUMMY, DUMMY, 1, None, 0, None) == 1


def test_decode_rejects_bad_arguments(lib):
    c = _cache()
    p = swa.DecodeParams(H_q=3, mode=1, out_dtype=0, scale=0.0, reserved=0, alibi_slopes=None,
                         rope_table=None, rope_rows=0)
    assert lib.swa_decode(ctypes.byref(p), ctypes.byref(c), DUMMY, DUMMY, DUMMY, None, 0,
                          None) == 1
    p.H_q = 4
    p.mode = 9
    assert lib.swa_decode(ctypes.byref(p), ctypes.byref(c), DUMMY, DUMMY, DUMMY, None, 0,
                          None) == 1
    p.mode = 1
    assert lib.swa_decode(ctypes.byref(p), ctypes.byref(c), None, DUMMY, DUMMY, None, 0,
                          None) == 1
    assert lib.swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(c)) == 0


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(swa, "_lib", None)
    monkeypatch.setattr(swa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        swa.load()


def test_decode_workspace_bytes_split_kv(lib):
    """Long windows with few (sequence, kv head) pairs are split over several blocks; the
    workspace holds one partial output (d values, maximum, sum) per head and range."""
    def wsb(S, H_kv, w, s, d, Hq, mode=1):
        c = _cache(num_seqs=S, H_kv=H_kv, w=w, s=s, d=d)
        p = swa.DecodeParams(Hq, mode, 0, 0.0, 0, None, None, 0)
        return lib.swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(c))
    # whole-window kernel (w + s <= 128) and plenty of blocks: no workspace
    assert wsb(64, 8, 64, 4, 128, 32) == 0
    assert wsb(64, 8, 1024, 0, 128, 32) == 0          # 512 blocks already
    # 1 sequence x 8 kv heads, 4096 keys: min(ceil(512 / 8), 4096 / 512) = 8 ranges
    assert wsb(1, 8, 4096, 0, 128, 32) == 4 * 1 * 8 * 8 * 4 * (128 + 2)
    # at most 64 ranges
    assert wsb(1, 1, 1 << 20, 0, 64, 2) == 4 * 1 * 1 * 64 * 2 * (64 + 2)
    # eight query heads per kv head on a long window: split like the others
    assert wsb(1, 2, 4096, 0, 128, 16) == 4 * 1 * 2 * 8 * 8 * (128 + 2)
    # general kernel, no workspace: eight heads per kv head on a short window, and a ring
    # slice per (sequence, kv head) of 2 GB (32-bit buffer offsets)
    assert wsb(1, 2, 64, 4, 128, 16) == 0
    assert wsb(1, 1, 1 << 23, 0, 128, 4) == 0
    assert wsb(1, 1, (1 << 23) - 1, 0, 128, 4) == 4 * 1 * 1 * 64 * 4 * (128 + 2)


def _dparams(H_q=4, mode=1, rope_table=None, rope_rows=0):
    return swa.DecodeParams(H_q, mode, 0, 0.0, 0, None, rope_table, rope_rows)


def test_prefill_chunk_workspace_bytes(lib):
    """K and V tile images per (sequence, kv head): the sink tiles, then the window tiles a
    chunk of max_seqlen rows can reach, (max_seqlen + w + 62) // 64 + 1 of them, or fewer
    when the rotation table bounds the positions."""
    def wsb(S=2, H_kv=2, w=8, s=2, d=64, T=10, max_q=5, **kw):
        c = _cache(num_seqs=S, H_kv=H_kv, w=w, s=s, d=d)
        p = _dparams(**kw)
        return lib.swa_prefill_chunk_workspace_bytes(ctypes.byref(p), ctypes.byref(c), T, max_q)
    tiles = lambda s, w, q: (s + 63) // 64 + (q + w + 62) // 64 + 1
    assert wsb() == 2 * 2 * 2 * tiles(2, 8, 5) * 64 * 64 * 2
    assert wsb(w=4096, s=0, d=128, max_q=2048, S=3, H_kv=8, H_q=32) == \
        2 * 3 * 8 * tiles(0, 4096, 2048) * 64 * 128 * 2
    # a table of 1000 positions: at most 16 window tiles
    assert wsb(w=100000, s=4, max_q=512, rope_table=0x2000, rope_rows=1000) == \
        2 * 2 * 2 * (1 + 16) * 64 * 64 * 2
    assert wsb(T=0) == 0 and wsb(max_q=0) == 0 and wsb(S=0) == 0
    assert wsb(d=96) == 0                      # unsupported head size
    c = _cache(dtype=0)                        # float32 cache: unsupported
    assert lib.swa_prefill_chunk_workspace_bytes(ctypes.byref(_dparams()), ctypes.byref(c),
                                                 10, 5) == 0


def test_prefill_chunk_rejects_bad_arguments(lib):
    c = _cache()
    p = _dparams()

    def call(c=c, p=p, q=DUMMY, cu=DUMMY, pos=DUMMY, T=10, max_q=5, ws=None, ws_bytes=0):
        return lib.swa_prefill_chunk(ctypes.byref(p), ctypes.byref(c), q, DUMMY, DUMMY, cu, pos,
                                     T, max_q, DUMMY, ws, ws_bytes, None)
    assert call(T=-1) == 1
    assert call(max_q=-1) == 1
    assert call(cu=None) == 1
    assert call(pos=None) == 1
    assert call(q=None) == 1
    assert call(p=_dparams(H_q=3)) == 1                       # H_q % H_kv != 0
    assert call(c=_cache(dtype=0)) == 2                       # float32 cache
    assert call(c=_cache(d=96)) == 2                          # head size 96
    assert call(q=ctypes.c_void_p(0x1008)) == 2               # 16-byte alignment
    assert call() == 1                                        # no workspace
    need = lib.swa_prefill_chunk_workspace_bytes(ctypes.byref(p), ctypes.byref(c), 10, 5)
    assert call(ws=DUMMY, ws_bytes=need - 16) == 1            # short workspace
    assert call(ws=ctypes.c_void_p(0x1004), ws_bytes=need) == 1  # misaligned workspace


def test_training_pair_rejections(lib):
    """Softmax needs o and lse, every tensor must be given, and the matrix-core backward
    checks its workspace (shapes it does not take run on the general kernels, which need
    none)."""
    p = _params(mode=1)
    z = ctypes.c_void_p(0)
    assert lib.swa_prefill_train(ctypes.byref(_params(d=258)), DUMMY, DUMMY, DUMMY, DUMMY,
                                 DUMMY, None, 0, None) == 2        # head size above 256
    assert lib.swa_prefill_train(ctypes.byref(_params(in_dtype=0, mode=1)), DUMMY, DUMMY, DUMMY,
                                 DUMMY, None, None, 0, None) == 1  # float32, softmax, no lse
    assert lib.swa_prefill_train(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, None, None, 0,
                                 None) == 1                        # softmax without lse
    assert lib.swa_prefill_train(ctypes.byref(p), DUMMY, z, DUMMY, DUMMY, DUMMY, None, 0,
                                 None) == 1                        # no k
    assert lib.swa_prefill_backward(ctypes.byref(p), DUMMY, DUMMY, DUMMY, None, None, DUMMY,
                                    DUMMY, DUMMY, DUMMY, None, 0, None) == 1   # no o / lse
    assert lib.swa_prefill_backward(ctypes.byref(_params(d=96, mode=1)), DUMMY, DUMMY, DUMMY,
                                    DUMMY, None, DUMMY, DUMMY, DUMMY, DUMMY, None, 0,
                                    None) == 1                     # general path, no lse
    assert lib.swa_prefill_backward(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                    z, DUMMY, DUMMY, None, 0, None) == 1       # no dq
    assert lib.swa_prefill_backward(ctypes.byref(_params(H_q=3)), DUMMY, DUMMY, DUMMY, DUMMY,
                                    DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, 0,
                                    None) == 1                     # H_q % H_kv != 0
    need = lib.swa_prefill_backward_workspace_bytes(ctypes.byref(p))
    assert lib.swa_prefill_backward(ctypes.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                    DUMMY, DUMMY, DUMMY, DUMMY, need - 16, None) == 1
    g = _params(in_dtype=0, mode=1)
    need = lib.swa_prefill_backward_workspace_bytes(ctypes.byref(g))
    assert need > 0
    assert lib.swa_prefill_backward(ctypes.byref(g), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                    DUMMY, DUMMY, DUMMY, None, 0, None) == 1   # general, no ws
    assert lib.swa_prefill_backward(ctypes.byref(g), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                    DUMMY, DUMMY, DUMMY, DUMMY, need - 4, None) == 1


def test_backward_workspace_bytes(lib):
    """k, v, q and dout images (64-row tiles, float16), softmax row statistics, and the sink
    keys' float32 partial gradients when some queries see a sink only through the sink rule."""
    def wsb(**kw):
        return lib.swa_prefill_backward_workspace_bytes(ctypes.byref(_params(**kw)))
    B, Hq, Hkv, N, d = 1, 4, 2, 16, 64
    img = lambda H: B * H * 1 * 64 * d * 2
    assert wsb(mode=0) == 2 * img(Hkv) + 2 * img(Hq)
    assert wsb(mode=1) == 2 * img(Hkv) + 2 * img(Hq) + B * Hq * 64 * 8
    # N 1000, w 100, s 4: the sink rule reaches queries past 127 + 100 -> one sink block
    big = dict(N=1000, w=100, s=4, mode=0)
    tiles = (1000 + 63) // 64
    assert wsb(**big) == 2 * B * Hkv * tiles * 64 * d * 2 + 2 * B * Hq * tiles * 64 * d * 2 + \
        2 * B * Hkv * 128 * d * 4
    assert wsb(in_dtype=0) == 0 and wsb(d=96) == 0 and wsb(B=0) == 0
    # the general path (float32, other head sizes, dilation): one float per softmax row
    assert wsb(in_dtype=0, mode=1) == B * Hq * N * 4 == wsb(d=96, mode=1)
    assert wsb(dilation=3, mode=1) == B * Hq * N * 4


def test_dilation_arguments(lib):
    """A negative dilation is rejected; a dilated window trains on the general kernels,
    whose backward needs no workspace."""
    assert lib.swa_prefill(ctypes.byref(_params(dilation=-1)), DUMMY, DUMMY, DUMMY, DUMMY, None,
                           0, None) == 1
    assert lib.swa_prefill_train(ctypes.byref(_params(dilation=-1)), DUMMY, DUMMY, DUMMY, DUMMY,
                                 DUMMY, None, 0, None) == 1
    assert lib.swa_prefill_backward_workspace_bytes(ctypes.byref(_params(dilation=2))) == 0
    # the workspace of the forward does not depend on the dilation
    assert lib.swa_prefill_workspace_bytes(ctypes.byref(_params(dilation=4))) == \
        lib.swa_prefill_workspace_bytes(ctypes.byref(_params()))


def test_static_decode_rejects_problems_past_its_scratch(lib):
    """swa_decode_append_static keeps the split partials in a 4 MiB array: a problem whose
    partials need more (511 sequences, one kv head, eight query heads, d 128, a 1100-token
    window: 511 x 2 ranges x 8 x 130 floats) is rejected before any launch; bad arguments
    are rejected as in swa_decode_append."""
    c = _cache(num_seqs=511, H_kv=1, w=1100, s=0, d=128, k_sink=None, v_sink=None)
    p = swa.DecodeParams(8, 1, 0, 0.0, 0, None, None, 0)
    need = lib.swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(c))
    assert need == 511 * 2 * 8 * 130 * 4 > 4 << 20
    assert lib.swa_decode_append_static(ctypes.byref(p), ctypes.byref(c), DUMMY, DUMMY, DUMMY,
                                        DUMMY, DUMMY, None) == 2
    ok = _cache(num_seqs=2, H_kv=1, w=1100, s=0, d=128, k_sink=None, v_sink=None)
    assert lib.swa_decode_append_static(ctypes.byref(p), ctypes.byref(ok), DUMMY, None, DUMMY,
                                        DUMMY, DUMMY, None) == 1
    p.mode = 7
    assert lib.swa_decode_append_static(ctypes.byref(p), ctypes.byref(ok), DUMMY, DUMMY, DUMMY,
                                        DUMMY, DUMMY, None) == 1
