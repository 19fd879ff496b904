"""CPU oracle for causal sliding-window attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the bench's
CPU-baseline leg. The product path never imports it, and it imports nothing of the
product (no kernels, headers, tables or helpers are shared).

Two independent implementations of the same definition, both in float64:
  * `prefill`, `backward`, `Ring.decode`, `Ring.append`, `Ring.chunk`: a plain C windowed loop
    (swa_oracle.c), one query row at a time, OpenMP across rows;
  * `dense.prefill_dense`: numpy, a full [N, N] score matrix masked with the boolean band
    mask built as in the Sliding Window Attention glossary's example.

Parity status: the selection, the weights (sigmoid and softmax), the bias sign, the
rotation and the ring are pinned by the tests in tests/test_oracle_pins.py against the
pages' printed values, closed forms and library special cases. Outputs on random inputs
beyond those are pinned only by the agreement of the two implementations.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import platform
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_lock = threading.Lock()
_lib = None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; the machine type where that is
    missing)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def _host_tag() -> str:
    """A short tag of the host CPU (model and feature flags): the library is compiled for
    the host it runs on (-march=native), so each CPU kind gets its own build."""
    flags = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("flags"):
                    flags = line
                    break
    except OSError:
        pass
    return hashlib.sha1((cpu_model() + flags).encode()).hexdigest()[:12]


_LIB = os.path.join(_HERE, "libswa_oracle_%s.so" % _host_tag())

SIGMOID = 0
SOFTMAX = 1


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O3 -march=native, OpenMP) for this host into
    oracle/libswa_oracle_<cpu tag>.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=native", "-fopenmp", "-shared", "-fPIC", "-std=c11",
               "-Wall", "-Werror", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, dbl, ip, dp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p
    lib.swa_oracle_prefill.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                       dbl, dp, dbl, dp, dp, dp, ip, i64, dp]
    lib.swa_oracle_prefill.restype = ctypes.c_int
    lib.swa_oracle_prefill_dilated.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64,
                                               ctypes.c_int, dbl, dp, dbl, dp, dp, dp, ip, i64,
                                               dp]
    lib.swa_oracle_prefill_dilated.restype = ctypes.c_int
    lib.swa_oracle_append.argtypes = [i64, i64, i64, i64, i64, dbl, dp, dp, ip, dp, dp,
                                      dp, dp, ip, i64]
    lib.swa_oracle_append.restype = ctypes.c_int
    lib.swa_oracle_decode.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, dbl, dp,
                                      dbl, dp, ip, dp, dp, ip, dp, dp, dp]
    lib.swa_oracle_decode.restype = ctypes.c_int
    lib.swa_oracle_chunk.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, dbl, dp,
                                     dbl, dp, dp, dp, ip, ip, i64, dp, dp, ip, dp, dp, ip, i64,
                                     dp]
    lib.swa_oracle_chunk.restype = ctypes.c_int
    lib.swa_oracle_backward.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int, dbl,
                                        dp, dbl, dp, dp, dp, dp, dp, dp, dp]
    lib.swa_oracle_backward.restype = ctypes.c_int
    lib.swa_oracle_backward_dilated.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64,
                                                ctypes.c_int, dbl, dp, dbl, dp, dp, dp, dp, dp,
                                                dp, dp]
    lib.swa_oracle_backward_dilated.restype = ctypes.c_int
    lib.swa_oracle_ring_fill_positions.argtypes = [i64, i64, ip]
    lib.swa_oracle_ring_fill_positions.restype = None
    lib.swa_oracle_threads.argtypes = []
    lib.swa_oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = bind(_LIB)
    return _lib


def _f64(a) -> np.ndarray:
    """Exact upcast of a float tensor/array (fp32 or bf16 values) to a C-contiguous float64
    numpy array."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i64(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return int(_load().swa_oracle_threads())


def prefill(q, k, v, *, w: int, s: int = 0, mode: int = SIGMOID, scale: float = 0.0,
            slopes=None, rope_theta: float = 0.0, rows=None, dilation: int = 1) -> np.ndarray:
    """float64 attention output. q [B,N,H_q,d], k/v [B,N,H_kv,d]. rows: optional list of
    query rows; then the result is [B, len(rows), H_q, d]. dilation r > 1: window keys
    i, i - r, ..., i - r (w - 1) (swa_oracle_prefill_dilated)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, N, Hkv, d) and v.shape == k.shape
    sl = None if slopes is None else _f64(slopes)
    if sl is not None:
        assert sl.shape == (Hq,)
    if rows is None:
        r, nr = None, N
    else:
        r = _i64(rows)
        nr = r.shape[0]
    out = np.zeros((B, nr, Hq, d), dtype=np.float64)
    if dilation == 1:
        rc = _load().swa_oracle_prefill(B, Hq, Hkv, N, d, w, s, mode, float(scale), _ptr(sl),
                                        float(rope_theta), _ptr(q), _ptr(k), _ptr(v), _ptr(r),
                                        nr if r is not None else 0, _ptr(out))
    else:
        rc = _load().swa_oracle_prefill_dilated(B, Hq, Hkv, N, d, w, s, int(dilation), mode,
                                                float(scale), _ptr(sl), float(rope_theta),
                                                _ptr(q), _ptr(k), _ptr(v), _ptr(r),
                                                nr if r is not None else 0, _ptr(out))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return out


def backward(q, k, v, dout, *, w: int, s: int = 0, mode: int = SIGMOID, scale: float = 0.0,
             slopes=None, rope_theta: float = 0.0, dilation: int = 1):
    """float64 gradients (dq, dk, dv) of prefill for the output gradient dout [B,N,H_q,d]
    (swa_oracle_backward; with dilation r > 1 the dilated window's,
    swa_oracle_backward_dilated)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, N, Hkv, d) and v.shape == k.shape and g.shape == q.shape
    sl = None if slopes is None else _f64(slopes)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    if dilation == 1:
        rc = _load().swa_oracle_backward(B, Hq, Hkv, N, d, w, s, mode, float(scale), _ptr(sl),
                                         float(rope_theta), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(dq), _ptr(dk), _ptr(dv))
    else:
        rc = _load().swa_oracle_backward_dilated(B, Hq, Hkv, N, d, w, s, int(dilation), mode,
                                                 float(scale), _ptr(sl), float(rope_theta),
                                                 _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq),
                                                 _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return dq, dk, dv


class Ring:
    """The oracle's ring-buffer cache for S sequences: w slots of (position, rotated key,
    value) per (sequence, kv head), plus s sink entries."""

    def __init__(self, S: int, H_kv: int, w: int, s: int, d: int):
        self.S, self.H_kv, self.w, self.s, self.d = S, H_kv, w, s, d
        self.k = np.zeros((S, H_kv, w, d))
        self.v = np.zeros((S, H_kv, w, d))
        self.pos = np.full((S, w), -1, dtype=np.int64)
        self.k_sink = np.zeros((S, H_kv, max(s, 1), d))
        self.v_sink = np.zeros((S, H_kv, max(s, 1), d))

    @classmethod
    def from_state(cls, k_ring, v_ring, k_sink, v_sink, last_pos):
        """A ring whose slots hold the given rotated keys/values, as left by appending
        positions 0..last_pos[q] in order (positions found by simulating those writes)."""
        k_ring, v_ring = _f64(k_ring), _f64(v_ring)
        S, H_kv, w, d = k_ring.shape
        s = 0 if k_sink is None else k_sink.shape[2]
        r = cls(S, H_kv, w, s, d)
        r.k[...] = k_ring
        r.v[...] = v_ring
        if s > 0:
            r.k_sink[...] = _f64(k_sink)
            r.v_sink[...] = _f64(v_sink)
        lp = _i64(last_pos)
        for qi in range(S):
            r.pos[qi] = ring_fill_positions(int(lp[qi]), w)
        return r

    def append(self, k_new, v_new, pos0, rope_theta: float = 0.0):
        """k_new/v_new [S, n_new, H_kv, d] (keys not yet rotated); pos0 [S]."""
        kn, vn, p0 = _f64(k_new), _f64(v_new), _i64(pos0)
        n_new = kn.shape[1]
        assert kn.shape == (self.S, n_new, self.H_kv, self.d) and vn.shape == kn.shape
        rc = _load().swa_oracle_append(self.S, self.H_kv, self.w, self.s, self.d,
                                       float(rope_theta), _ptr(self.k), _ptr(self.v),
                                       _ptr(self.pos), _ptr(self.k_sink), _ptr(self.v_sink),
                                       _ptr(kn), _ptr(vn), _ptr(p0), n_new)
        if rc != 0:
            raise ValueError("oracle append rejected its arguments")

    def decode(self, q, q_pos, *, H_q: int, mode: int, scale: float = 0.0, slopes=None,
               rope_theta: float = 0.0) -> np.ndarray:
        """q [S, H_q, d] (not rotated), q_pos [S] -> float64 [S, H_q, d]."""
        qq, qp = _f64(q), _i64(q_pos)
        assert qq.shape == (self.S, H_q, self.d)
        sl = None if slopes is None else _f64(slopes)
        out = np.zeros((self.S, H_q, self.d))
        rc = _load().swa_oracle_decode(self.S, H_q, self.H_kv, self.d, self.w, self.s, mode,
                                       float(scale), _ptr(sl), float(rope_theta), _ptr(qq),
                                       _ptr(qp), _ptr(self.k), _ptr(self.v), _ptr(self.pos),
                                       _ptr(self.k_sink), _ptr(self.v_sink), _ptr(out))
        if rc != 0:
            raise ValueError("oracle decode rejected its arguments")
        return out

    def chunk(self, q, k_new, v_new, cu_seqlens, pos0, *, H_q: int, mode: int,
              scale: float = 0.0, slopes=None, rope_theta: float = 0.0,
              append: bool = True, rows=None) -> np.ndarray:
        """Chunked prefill over this ring (swa_oracle_chunk): packed rows, sequence q owns
        rows cu_seqlens[q] .. cu_seqlens[q+1]-1 at positions pos0[q], pos0[q]+1, ...
        q [T, H_q, d], k_new/v_new [T, H_kv, d] (keys not rotated) -> float64 [T, H_q, d].
        With append, the chunk is then appended, one sequence at a time, as append does.
        rows: optional list of packed rows; then the result is [len(rows), H_q, d]."""
        qq, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
        cu, p0 = _i64(cu_seqlens), _i64(pos0)
        T = qq.shape[0]
        assert qq.shape == (T, H_q, self.d) and kn.shape == (T, self.H_kv, self.d)
        assert vn.shape == kn.shape and cu.shape == (self.S + 1,) and p0.shape == (self.S,)
        sl = None if slopes is None else _f64(slopes)
        r = None if rows is None else _i64(rows)
        out = np.zeros((T if r is None else r.shape[0], H_q, self.d))
        rc = _load().swa_oracle_chunk(self.S, H_q, self.H_kv, self.d, self.w, self.s, mode,
                                      float(scale), _ptr(sl), float(rope_theta), _ptr(qq),
                                      _ptr(kn), _ptr(vn), _ptr(cu), _ptr(p0), T,
                                      _ptr(self.k), _ptr(self.v), _ptr(self.pos),
                                      _ptr(self.k_sink), _ptr(self.v_sink), _ptr(r),
                                      0 if r is None else r.shape[0], _ptr(out))
        if rc == -2:
            raise ValueError("oracle chunk: the ring does not hold a key the chunk needs")
        if rc != 0:
            raise ValueError("oracle chunk rejected its arguments")
        if append:
            for sq in range(self.S):
                a, b = int(cu[sq]), int(cu[sq + 1])
                if b == a:
                    continue
                kpad = np.zeros((self.S, b - a, self.H_kv, self.d))
                vpad = np.zeros_like(kpad)
                kpad[sq], vpad[sq] = kn[a:b], vn[a:b]
                only = np.full(self.S, -1, dtype=np.int64)
                only[sq] = p0[sq]
                self.append(kpad, vpad, only, rope_theta=rope_theta)
        return out


def ring_fill_positions(p_last: int, w: int) -> np.ndarray:
    out = np.empty(w, dtype=np.int64)
    _load().swa_oracle_ring_fill_positions(int(p_last), int(w), _ptr(out))
    return out
