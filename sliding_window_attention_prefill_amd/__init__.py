"""Python binding for libswa: causal sliding-window attention on MI355X (gfx950).

A thin ctypes layer over the C ABI declared in include/swa.h, with the same entry-point
names. It only marshals arguments: torch tensors supply device pointers (data_ptr) and the
current HIP stream; every step of the computation runs in the library's HIP kernels. If
libswa.so is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswa.so")

SWA_SIGMOID = 0
SWA_SOFTMAX = 1
SWA_F32 = 0
SWA_BF16 = 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported combination", 3: "HIP runtime error"}

c_i64, c_i32, c_f32, c_ptr = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class SwaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        msg = "%s failed: %s" % (fn, _STATUS.get(status, "status %d" % status))
        if status == 3:
            msg += " (hipError %d)" % hip_error
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


class PrefillParams(ctypes.Structure):
    _fields_ = [("B", c_i64), ("H_q", c_i64), ("H_kv", c_i64), ("N", c_i64), ("d", c_i64),
                ("w", c_i64), ("s", c_i64), ("mode", c_i32), ("in_dtype", c_i32),
                ("out_dtype", c_i32), ("scale", c_f32), ("alibi_slopes", c_ptr),
                ("rope_table", c_ptr), ("rope_rows", c_i64), ("dilation", c_i64)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_seqs", c_i64), ("H_kv", c_i64), ("w", c_i64), ("s", c_i64), ("d", c_i64),
                ("dtype", c_i32), ("reserved", c_i32), ("k_ring", c_ptr), ("v_ring", c_ptr),
                ("k_sink", c_ptr), ("v_sink", c_ptr)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("H_q", c_i64), ("mode", c_i32), ("out_dtype", c_i32), ("scale", c_f32),
                ("reserved", c_i32), ("alibi_slopes", c_ptr), ("rope_table", c_ptr),
                ("rope_rows", c_i64)]


EXPORTS = ["swa_prefill", "swa_prefill_workspace_bytes", "swa_rope_table", "swa_rope_apply", "swa_kv_append", "swa_decode",
           "swa_decode_append", "swa_decode_append_static", "swa_decode_workspace_bytes",
           "swa_prefill_chunk",
           "swa_prefill_chunk_workspace_bytes", "swa_prefill_train", "swa_prefill_backward",
           "swa_prefill_backward_workspace_bytes", "swa_status_string",
           "swa_last_hip_error", "swa_version"]

_lib = None


def load():
    """Load libswa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libswa.so is not built (python -m "
                              "sliding_window_attention_prefill_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        lib.swa_prefill.argtypes = [P(PrefillParams), c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                    ctypes.c_size_t, c_ptr]
        lib.swa_prefill.restype = ctypes.c_int
        lib.swa_prefill_workspace_bytes.argtypes = [P(PrefillParams)]
        lib.swa_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.swa_rope_table.argtypes = [c_ptr, c_i64, c_i64, ctypes.c_double, c_ptr]
        lib.swa_rope_table.restype = ctypes.c_int
        lib.swa_rope_apply.argtypes = [c_ptr, c_i64, c_i64, c_i64, c_i64, c_ptr, c_ptr, c_i64,
                                       c_i32, c_ptr]
        lib.swa_rope_apply.restype = ctypes.c_int
        lib.swa_kv_append.argtypes = [P(CacheDesc), c_ptr, c_ptr, c_ptr, c_i64, c_ptr, c_i64,
                                      c_ptr]
        lib.swa_kv_append.restype = ctypes.c_int
        lib.swa_decode.argtypes = [P(DecodeParams), P(CacheDesc), c_ptr, c_ptr, c_ptr, c_ptr,
                                   ctypes.c_size_t, c_ptr]
        lib.swa_decode.restype = ctypes.c_int
        lib.swa_decode_append.argtypes = [P(DecodeParams), P(CacheDesc), c_ptr, c_ptr, c_ptr, c_ptr,
                                          c_ptr, c_ptr, ctypes.c_size_t, c_ptr]
        lib.swa_decode_append.restype = ctypes.c_int
        lib.swa_decode_append_static.argtypes = [P(DecodeParams), P(CacheDesc), c_ptr, c_ptr,
                                                 c_ptr, c_ptr, c_ptr, c_ptr]
        lib.swa_decode_append_static.restype = ctypes.c_int
        lib.swa_decode_workspace_bytes.argtypes = [P(DecodeParams), P(CacheDesc)]
        lib.swa_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.swa_prefill_chunk.argtypes = [P(DecodeParams), P(CacheDesc), c_ptr, c_ptr, c_ptr,
                                          c_ptr, c_ptr, c_i64, c_i64, c_ptr, c_ptr,
                                          ctypes.c_size_t, c_ptr]
        lib.swa_prefill_chunk.restype = ctypes.c_int
        lib.swa_prefill_chunk_workspace_bytes.argtypes = [P(DecodeParams), P(CacheDesc), c_i64,
                                                          c_i64]
        lib.swa_prefill_chunk_workspace_bytes.restype = ctypes.c_size_t
        lib.swa_prefill_train.argtypes = [P(PrefillParams), c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                          c_ptr, ctypes.c_size_t, c_ptr]
        lib.swa_prefill_train.restype = ctypes.c_int
        lib.swa_prefill_backward.argtypes = [P(PrefillParams), c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                             c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, ctypes.c_size_t,
                                             c_ptr]
        lib.swa_prefill_backward.restype = ctypes.c_int
        lib.swa_prefill_backward_workspace_bytes.argtypes = [P(PrefillParams)]
        lib.swa_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.swa_status_string.argtypes = [ctypes.c_int]
        lib.swa_status_string.restype = ctypes.c_char_p
        lib.swa_last_hip_error.argtypes = []
        lib.swa_last_hip_error.restype = ctypes.c_int
        lib.swa_version.argtypes = []
        lib.swa_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise SwaError(fn, status, load().swa_last_hip_error() if status == 3 else 0)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SWA_F32
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    raise ValueError("libswa takes float32 or bfloat16 tensors, got %s" % t.dtype)


def _torch_dt(dt: int) -> torch.dtype:
    return torch.float32 if dt == SWA_F32 else torch.bfloat16


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _mode(mode) -> int:
    if isinstance(mode, str):
        return {"sigmoid": SWA_SIGMOID, "softmax": SWA_SOFTMAX}[mode]
    return int(mode)


def swa_rope_table(n_pos: int, d: int, theta: float, device=None, stream=None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """float32 [n_pos, d/2, 2] table of (cos, sin) of pos * theta^(-2t/d)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty((n_pos, d // 2, 2), dtype=torch.float32, device=device)
    _dev(out, "out")
    if out.numel() < n_pos * (d // 2) * 2 or out.dtype != torch.float32:
        raise ValueError("table buffer too small or not float32")
    _check("swa_rope_table", load().swa_rope_table(_ptr(out), n_pos, d, float(theta),
                                                   _stream(out.device, stream)))
    return out


def swa_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, w: int, s: int = 0,
                mode=SWA_SIGMOID, scale: float = 0.0,
                alibi_slopes: Optional[torch.Tensor] = None,
                rope_table: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                stream=None, dilation: int = 1) -> torch.Tensor:
    """Sliding-window attention over whole sequences. q [B,N,H_q,d], k/v [B,N,H_kv,d].
    dilation r > 1: the window keys are i, i - r, ..., i - r (w - 1) (plus the sinks).

    workspace: a device uint8 tensor of at least swa_prefill_workspace_bytes(...) bytes;
    allocated here when it is not given and the call needs one."""
    if q.dim() != 4:
        raise ValueError("q must be [B,N,H_q,d] and k, v [B,N,H_kv,d]")
    if out is None:
        B, N, Hq, d = q.shape
        out = torch.empty((B, N, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    p = _prefill_params(q, k, v, out, w, s, mode, scale, alibi_slopes, rope_table, dilation)
    lib = load()
    workspace, ws_bytes = _workspace(int(lib.swa_prefill_workspace_bytes(ctypes.byref(p))),
                                     workspace, q.device)
    _check("swa_prefill", lib.swa_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                          _ptr(workspace), ws_bytes, _stream(q.device, stream)))
    return out


def _prefill_params(q, k, v, out, w, s, mode, scale, alibi_slopes, rope_table, dilation=1):
    """Shape checks shared by the prefill entry points; returns PrefillParams."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4:
        raise ValueError("q must be [B,N,H_q,d] and k, v [B,N,H_kv,d]")
    B, N, Hq, d = q.shape
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError("q, k, v shapes disagree")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if tuple(out.shape) != (B, N, Hq, d):
        raise ValueError("out must be [B,N,H_q,d]")
    if alibi_slopes is not None:
        _dev(alibi_slopes, "alibi_slopes")
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != Hq:
            raise ValueError("alibi_slopes must be float32[H_q]")
    rows = 0
    if rope_table is not None:
        _dev(rope_table, "rope_table")
        if rope_table.dtype != torch.float32 or rope_table.dim() != 3 or \
                rope_table.shape[1] != d // 2 or rope_table.shape[2] != 2:
            raise ValueError("rope_table must be float32 [rows, d/2, 2]")
        rows = rope_table.shape[0]
    return PrefillParams(B, Hq, k.shape[2], N, d, w, s, _mode(mode), _dt(q), _dt(out), scale,
                         _ptr(alibi_slopes), _ptr(rope_table), rows, dilation)


def _workspace(need: int, workspace, device):
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return workspace, ws_bytes


def swa_prefill_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, w: int, s: int = 0,
                      mode=SWA_SIGMOID, scale: float = 0.0,
                      alibi_slopes: Optional[torch.Tensor] = None,
                      rope_table: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None, dilation: int = 1):
    """Forward for training: returns (o, lse), lse float32 [B, H_q, N] the natural-log row
    normalisers (softmax; None for sigmoid)."""
    B, N, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, N, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    p = _prefill_params(q, k, v, out, w, s, mode, scale, alibi_slopes, rope_table, dilation)
    if p.mode == SWA_SOFTMAX:
        if lse is None:
            lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        _dev(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
            raise ValueError("lse must be float32 [B, H_q, N]")
    else:
        lse = None
    lib = load()
    workspace, ws_bytes = _workspace(int(lib.swa_prefill_workspace_bytes(ctypes.byref(p))),
                                     workspace, q.device)
    _check("swa_prefill_train",
           lib.swa_prefill_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(workspace), ws_bytes, _stream(q.device, stream)))
    return out, lse


def swa_prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         o: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                         dout: torch.Tensor, *, w: int, s: int = 0, mode=SWA_SIGMOID,
                         scale: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None,
                         rope_table: Optional[torch.Tensor] = None,
                         grads=None, workspace: Optional[torch.Tensor] = None, stream=None,
                         dilation: int = 1):
    """Gradients (dq, dk, dv) in dout's dtype for the output gradient dout [B,N,H_q,d];
    o and lse (from swa_prefill_train) are needed for softmax only."""
    p = _prefill_params(q, k, v, dout, w, s, mode, scale, alibi_slopes, rope_table, dilation)
    if p.mode == SWA_SOFTMAX:
        if o is None or lse is None:
            raise ValueError("softmax needs the forward's o and lse")
        _dev(o, "o")
        _dev(lse, "lse")
        if o.shape != dout.shape or o.dtype != dout.dtype:
            raise ValueError("o must match dout")
    if grads is None:
        grads = (torch.empty(q.shape, dtype=dout.dtype, device=q.device),
                 torch.empty(k.shape, dtype=dout.dtype, device=q.device),
                 torch.empty(v.shape, dtype=dout.dtype, device=q.device))
    dq, dk, dv = grads
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _dev(t, n)
        if t.shape != ref.shape or t.dtype != dout.dtype:
            raise ValueError("%s must have the shape of its input and dout's dtype" % n)
    lib = load()
    workspace, ws_bytes = _workspace(
        int(lib.swa_prefill_backward_workspace_bytes(ctypes.byref(p))), workspace, q.device)
    _check("swa_prefill_backward",
           lib.swa_prefill_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), ws_bytes, _stream(q.device, stream)))
    return dq, dk, dv


def swa_prefill_workspace_bytes(q: torch.Tensor, k: torch.Tensor, *, w: int, s: int = 0,
                                mode=SWA_SIGMOID, out_dtype: Optional[torch.dtype] = None,
                                dilation: int = 1) -> int:
    """Workspace bytes swa_prefill needs for q [B,N,H_q,d], k [B,N,H_kv,d] and these options
    (ALiBi and RoPE do not change it)."""
    B, N, Hq, d = q.shape
    out_dt = SWA_F32 if (out_dtype or q.dtype) == torch.float32 else SWA_BF16
    p = PrefillParams(B, Hq, k.shape[2], N, d, w, s, _mode(mode), _dt(q), out_dt, 0.0,
                      None, None, 0, dilation)
    return int(load().swa_prefill_workspace_bytes(ctypes.byref(p)))


def swa_prefill_backward_workspace_bytes(q: torch.Tensor, k: torch.Tensor, *, w: int, s: int = 0,
                                         mode=SWA_SIGMOID,
                                         grad_dtype: Optional[torch.dtype] = None,
                                         dilation: int = 1) -> int:
    """Workspace bytes swa_prefill_backward needs for q [B,N,H_q,d], k [B,N,H_kv,d]."""
    B, N, Hq, d = q.shape
    out_dt = SWA_F32 if (grad_dtype or q.dtype) == torch.float32 else SWA_BF16
    p = PrefillParams(B, Hq, k.shape[2], N, d, w, s, _mode(mode), _dt(q), out_dt, 0.0,
                      None, None, 0, dilation)
    return int(load().swa_prefill_backward_workspace_bytes(ctypes.byref(p)))


def swa_rope_apply(x: torch.Tensor, pos0: torch.Tensor, rope_table: torch.Tensor,
                   stream=None) -> torch.Tensor:
    """Rotate x [B,N,H,d] in place; row n of batch b at position pos0[b] + n."""
    _dev(x, "x")
    _dev(pos0, "pos0")
    _dev(rope_table, "rope_table")
    if pos0.dtype != torch.int32 or pos0.numel() != x.shape[0]:
        raise ValueError("pos0 must be int32[B]")
    B, N, H, d = x.shape
    _check("swa_rope_apply", load().swa_rope_apply(_ptr(x), B, N, H, d, _ptr(pos0),
                                                   _ptr(rope_table), rope_table.shape[0], _dt(x),
                                                   _stream(x.device, stream)))
    return x


class SwaCache:
    """Ring-buffer KV cache tensors: k_ring/v_ring [S, H_kv, w, d], k_sink/v_sink
    [S, H_kv, s, d] (None when s == 0)."""

    def __init__(self, k_ring, v_ring, k_sink=None, v_sink=None):
        self.k_ring, self.v_ring, self.k_sink, self.v_sink = k_ring, v_ring, k_sink, v_sink
        for t, n in ((k_ring, "k_ring"), (v_ring, "v_ring")):
            _dev(t, n)
        S, Hkv, w, d = k_ring.shape
        if v_ring.shape != k_ring.shape or v_ring.dtype != k_ring.dtype:
            raise ValueError("k_ring and v_ring must match")
        s = 0
        if k_sink is not None:
            _dev(k_sink, "k_sink")
            _dev(v_sink, "v_sink")
            s = k_sink.shape[2]
            if k_sink.shape != (S, Hkv, s, d) or v_sink.shape != k_sink.shape:
                raise ValueError("sink stores must be [S, H_kv, s, d]")
        self.S, self.H_kv, self.w, self.s, self.d = S, Hkv, w, s, d
        self.dtype = k_ring.dtype
        self.desc = CacheDesc(S, Hkv, w, s, d, _dt(k_ring), 0, _ptr(k_ring), _ptr(v_ring),
                              _ptr(k_sink), _ptr(v_sink))

    @classmethod
    def empty(cls, S, H_kv, w, s, d, dtype=torch.bfloat16, device=None):
        device = device or torch.device("cuda", torch.cuda.current_device())
        z = lambda n: torch.zeros((S, H_kv, n, d), dtype=dtype, device=device)
        return cls(z(w), z(w), z(s) if s > 0 else None, z(s) if s > 0 else None)


def swa_kv_append(cache: SwaCache, k_new: torch.Tensor, v_new: torch.Tensor,
                  pos0: torch.Tensor, rope_table: Optional[torch.Tensor] = None, stream=None):
    """Append k_new/v_new [S, n_new, H_kv, d] at positions pos0[q] + n."""
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    _dev(pos0, "pos0")
    if k_new.dim() != 4 or k_new.shape != v_new.shape or k_new.shape[0] != cache.S or \
            k_new.shape[2] != cache.H_kv or k_new.shape[3] != cache.d:
        raise ValueError("k_new/v_new must be [S, n_new, H_kv, d]")
    if k_new.dtype != cache.dtype or v_new.dtype != cache.dtype:
        raise ValueError("new tokens must have the cache dtype")
    if pos0.dtype != torch.int32 or pos0.numel() != cache.S:
        raise ValueError("pos0 must be int32[S]")
    rows = 0
    if rope_table is not None:
        _dev(rope_table, "rope_table")
        rows = rope_table.shape[0]
    _check("swa_kv_append", load().swa_kv_append(ctypes.byref(cache.desc), _ptr(k_new),
                                                 _ptr(v_new), _ptr(pos0), k_new.shape[1],
                                                 _ptr(rope_table), rows,
                                                 _stream(k_new.device, stream)))


def _decode_params(H_q, mode, scale, alibi_slopes, rope_table, out_dt):
    rows = 0 if rope_table is None else rope_table.shape[0]
    return DecodeParams(H_q, _mode(mode), out_dt, scale, 0, _ptr(alibi_slopes),
                        _ptr(rope_table), rows)


def swa_decode_workspace_bytes(cache: SwaCache, H_q: int, *, mode=SWA_SOFTMAX,
                               out_dtype=torch.float32) -> int:
    p = _decode_params(H_q, mode, 0.0, None, None, _dt(torch.empty(0, dtype=out_dtype)))
    return int(load().swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(cache.desc)))


def swa_decode(q: torch.Tensor, q_pos: torch.Tensor, cache: SwaCache, *, mode=SWA_SOFTMAX,
               scale: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None,
               rope_table: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """One query token per sequence: q [S, H_q, d] (not rotated) at positions q_pos[S]."""
    _dev(q, "q")
    _dev(q_pos, "q_pos")
    if q.dim() != 3 or q.shape[0] != cache.S or q.shape[2] != cache.d:
        raise ValueError("q must be [S, H_q, d]")
    if q.dtype != cache.dtype:
        raise ValueError("q must have the cache dtype")
    if q_pos.dtype != torch.int32 or q_pos.numel() != cache.S:
        raise ValueError("q_pos must be int32[S]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    if alibi_slopes is not None:
        _dev(alibi_slopes, "alibi_slopes")
    if rope_table is not None:
        _dev(rope_table, "rope_table")
    p = _decode_params(q.shape[1], mode, scale, alibi_slopes, rope_table, _dt(out))
    need = int(load().swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(cache.desc)))
    ws_bytes = 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("swa_decode", load().swa_decode(ctypes.byref(p), ctypes.byref(cache.desc), _ptr(q),
                                           _ptr(q_pos), _ptr(out), _ptr(workspace), ws_bytes,
                                           _stream(q.device, stream)))
    return out


def swa_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      q_pos: torch.Tensor, cache: SwaCache, *, mode=SWA_SOFTMAX,
                      scale: float = 0.0, alibi_slopes: Optional[torch.Tensor] = None,
                      rope_table: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append one token per sequence (k_new, v_new [S, H_kv, d], key not rotated) at q_pos
    and answer q [S, H_q, d] there, in one launch."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (q_pos, "q_pos")):
        _dev(t, n)
    if q.dim() != 3 or q.shape[0] != cache.S or q.shape[2] != cache.d:
        raise ValueError("q must be [S, H_q, d]")
    if tuple(k_new.shape) != (cache.S, cache.H_kv, cache.d) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [S, H_kv, d]")
    if q.dtype != cache.dtype or k_new.dtype != cache.dtype or v_new.dtype != cache.dtype:
        raise ValueError("q, k_new, v_new must have the cache dtype")
    if q_pos.dtype != torch.int32 or q_pos.numel() != cache.S:
        raise ValueError("q_pos must be int32[S]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    if alibi_slopes is not None:
        _dev(alibi_slopes, "alibi_slopes")
    if rope_table is not None:
        _dev(rope_table, "rope_table")
    p = _decode_params(q.shape[1], mode, scale, alibi_slopes, rope_table, _dt(out))
    need = int(load().swa_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(cache.desc)))
    ws_bytes = 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("swa_decode_append",
           load().swa_decode_append(ctypes.byref(p), ctypes.byref(cache.desc), _ptr(q),
                                    _ptr(k_new), _ptr(v_new), _ptr(q_pos), _ptr(out),
                                    _ptr(workspace), ws_bytes, _stream(q.device, stream)))
    return out


def swa_decode_append_static(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             q_pos: torch.Tensor, cache: SwaCache, out: torch.Tensor, *,
                             mode=SWA_SOFTMAX, scale: float = 0.0,
                             alibi_slopes: Optional[torch.Tensor] = None,
                             rope_table: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """swa_decode_append without a workspace: the split partials live in the library's own
    device scratch array (for callers that cannot allocate). out [S, H_q, d] must be given;
    nothing is allocated here or in the library."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (q_pos, "q_pos"), (out, "out")):
        _dev(t, n)
    if q.dim() != 3 or q.shape[0] != cache.S or q.shape[2] != cache.d:
        raise ValueError("q must be [S, H_q, d]")
    if tuple(k_new.shape) != (cache.S, cache.H_kv, cache.d) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [S, H_kv, d]")
    if q.dtype != cache.dtype or k_new.dtype != cache.dtype or v_new.dtype != cache.dtype:
        raise ValueError("q, k_new, v_new must have the cache dtype")
    if q_pos.dtype != torch.int32 or q_pos.numel() != cache.S:
        raise ValueError("q_pos must be int32[S]")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be [S, H_q, d]")
    if alibi_slopes is not None:
        _dev(alibi_slopes, "alibi_slopes")
    if rope_table is not None:
        _dev(rope_table, "rope_table")
    p = _decode_params(q.shape[1], mode, scale, alibi_slopes, rope_table, _dt(out))
    _check("swa_decode_append_static",
           load().swa_decode_append_static(ctypes.byref(p), ctypes.byref(cache.desc), _ptr(q),
                                           _ptr(k_new), _ptr(v_new), _ptr(q_pos), _ptr(out),
                                           _stream(q.device, stream)))
    return out


def swa_prefill_chunk_workspace_bytes(cache: SwaCache, H_q: int, total_rows: int,
                                      max_seqlen: int, *, mode=SWA_SOFTMAX,
                                      rope_table: Optional[torch.Tensor] = None) -> int:
    """Workspace bytes swa_prefill_chunk needs (the rotation table, when given, bounds the
    positions and can shrink it)."""
    p = _decode_params(H_q, mode, 0.0, None, rope_table, SWA_F32)
    return int(load().swa_prefill_chunk_workspace_bytes(ctypes.byref(p), ctypes.byref(cache.desc),
                                                        int(total_rows), int(max_seqlen)))


def swa_prefill_chunk(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      cu_seqlens: torch.Tensor, pos0: torch.Tensor, cache: SwaCache, *,
                      max_seqlen: int, mode=SWA_SOFTMAX, scale: float = 0.0,
                      alibi_slopes: Optional[torch.Tensor] = None,
                      rope_table: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunked prefill over the ring cache. Packed rows: sequence s owns rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1 of q [T, H_q, d] and k_new/v_new [T, H_kv, d] (keys
    not rotated), at positions pos0[s], pos0[s]+1, ...; the cache holds each sequence's
    positions below pos0[s]. Returns o [T, H_q, d]; the chunk is appended to the cache."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (cu_seqlens, "cu_seqlens"),
                 (pos0, "pos0")):
        _dev(t, n)
    T = q.shape[0]
    if q.dim() != 3 or q.shape[2] != cache.d:
        raise ValueError("q must be [T, H_q, d]")
    if tuple(k_new.shape) != (T, cache.H_kv, cache.d) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [T, H_kv, d]")
    if q.dtype != cache.dtype or k_new.dtype != cache.dtype or v_new.dtype != cache.dtype:
        raise ValueError("q, k_new, v_new must have the cache dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.numel() != cache.S + 1:
        raise ValueError("cu_seqlens must be int32[S + 1]")
    if pos0.dtype != torch.int32 or pos0.numel() != cache.S:
        raise ValueError("pos0 must be int32[S]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    if alibi_slopes is not None:
        _dev(alibi_slopes, "alibi_slopes")
    if rope_table is not None:
        _dev(rope_table, "rope_table")
    p = _decode_params(q.shape[1], mode, scale, alibi_slopes, rope_table, _dt(out))
    need = int(load().swa_prefill_chunk_workspace_bytes(ctypes.byref(p), ctypes.byref(cache.desc),
                                                        T, int(max_seqlen)))
    ws_bytes = 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("swa_prefill_chunk",
           load().swa_prefill_chunk(ctypes.byref(p), ctypes.byref(cache.desc), _ptr(q),
                                    _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens), _ptr(pos0), T,
                                    int(max_seqlen), _ptr(out), _ptr(workspace), ws_bytes,
                                    _stream(q.device, stream)))
    return out
