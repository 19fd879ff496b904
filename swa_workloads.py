"""Seeded synthetic workloads shared by the tests, the bench and the smoke run.

This module only draws random numbers and lays out shapes. It holds none of the
attention arithmetic: no rotation, no scores, no weights. Both the HIP path and
the CPU oracle receive exactly the tensors produced here (the oracle gets them
upcast to float64), so neither side depends on the other.

Workload shapes follow the pages' settings:
  * SWAT-340M-shaped layer (SWAT: Sliding Window Attention Training, "The number" and
    "Balanced ALiBi"): d=64, sigmoid weights, balanced ALiBi, RoPE.
  * Mistral-7B-shaped window (Sliding Window Attention glossary, first paragraph):
    w=4096, grouped-query heads 32/8, d=128, softmax.
  * SWA(64, 4) with sinks (Sliding-window beats linear attention, "technical approach").
  * Gemma-3-style local layer (Sliding Window Attention glossary, "interleaving local and
    global layers"): w=1024 at 128K context.

ALiBi slope lists are inputs to the library (it takes a signed per-head float array).
The balanced lists use the same geometric magnitudes in both halves, negative for the
first half of the heads and positive for the second half (SWAT page, "Balanced ALiBi":
slopes follow a geometric sequence in both directions).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

SIGMOID = 0
SOFTMAX = 1


def balanced_alibi_slopes(h_q: int) -> list:
    """Signed slopes for h_q heads: heads [0, h_q/2) get -2^(-8k/h_q), heads [h_q/2, h_q)
    get +2^(-8k/h_q), with k = 1..h_q/2 inside each half."""
    assert h_q % 2 == 0
    half = h_q // 2
    mags = [2.0 ** (-8.0 * k / h_q) for k in range(1, half + 1)]
    return [-m for m in mags] + [m for m in mags]


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str            # "f32" or "bf16": the input element type
    B: int
    H_q: int
    H_kv: int
    N: int
    d: int
    w: int
    s: int
    mode: int             # SIGMOID or SOFTMAX
    rope_theta: float     # <= 0: no rotation
    slopes: Optional[tuple]   # signed per-query-head ALiBi slopes, or None
    input_scale: float = 1.0  # inputs ~ N(0, 1) * input_scale
    heavy_k_frac: float = 0.0  # fraction of (position, kv head) K rows multiplied by heavy_k_mult
    heavy_k_mult: float = 8.0
    seed: int = 0

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: str
    num_seqs: int
    H_q: int
    H_kv: int
    d: int
    w: int
    s: int
    mode: int
    rope_theta: float
    slopes: Optional[tuple]
    len_lo: int
    len_hi: int
    steps: int
    seed: int = 0

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


# The five workloads, smallest first.
C1 = PrefillConfig("tiny_swat_f32_N256_w16", "f32", B=1, H_q=4, H_kv=4, N=256, d=64, w=16, s=0,
                   mode=SIGMOID, rope_theta=1e4,
                   slopes=(-2.0 ** -1, -2.0 ** -2, 2.0 ** -1, 2.0 ** -2), seed=1)
C2 = PrefillConfig("swat340m_layer_bf16_B8_H16_N4096_d64_w512", "bf16", B=8, H_q=16, H_kv=16,
                   N=4096, d=64, w=512, s=0, mode=SIGMOID, rope_theta=1e4,
                   slopes=tuple(balanced_alibi_slopes(16)), seed=2)
C3 = PrefillConfig("mistral7b_prefill_bf16_Hq32_Hkv8_N32768_d128_w4096", "bf16", B=1, H_q=32,
                   H_kv=8, N=32768, d=128, w=4096, s=0, mode=SOFTMAX, rope_theta=1e6,
                   slopes=None, input_scale=1.0 / math.sqrt(2.0), seed=3)
C4 = DecodeConfig("swa64_4_decode_bf16_S64_Hq32_Hkv8_d128", "bf16", num_seqs=64, H_q=32, H_kv=8,
                  d=128, w=64, s=4, mode=SOFTMAX, rope_theta=1e6, slopes=None,
                  len_lo=2048, len_hi=16384, steps=256, seed=4)
C5 = PrefillConfig("gemma3_local_bf16_Hq16_Hkv8_N131072_d128_w1024", "bf16", B=1, H_q=16, H_kv=8,
                   N=131072, d=128, w=1024, s=0, mode=SIGMOID, rope_theta=1e4,
                   slopes=tuple(balanced_alibi_slopes(16)), heavy_k_frac=0.01, seed=5)

# Decode at long windows (measurement only): the C3 layer shape with its 4,096-token window
# over 64 sequences, and a 32K sliding window over 8 sequences (positions past the window),
# which runs split over several blocks per (sequence, kv head). Both caches outgrow the
# last-level cache.
DECODE_W4096 = DecodeConfig("mistral7b_window_decode_bf16_S64_Hq32_Hkv8_d128_w4096", "bf16",
                            num_seqs=64, H_q=32, H_kv=8, d=128, w=4096, s=0, mode=SOFTMAX,
                            rope_theta=1e6, slopes=None, len_lo=8192, len_hi=32768, steps=32,
                            seed=6)
DECODE_W32K = DecodeConfig("sliding_w32k_decode_bf16_S8_Hq32_Hkv8_d128_w32768", "bf16",
                           num_seqs=8, H_q=32, H_kv=8, d=128, w=32768, s=0, mode=SOFTMAX,
                           rope_theta=1e6, slopes=None, len_lo=40000, len_hi=60000, steps=32,
                           seed=7)
# A global layer of a Gemma-3-style local/global stack (Sliding Window Attention glossary,
# "interleaving local and global layers": the global layers see the whole 128K context):
# a cache of the full 131,072-token context, every query position below it (so each key set
# is the whole history), at the local layer's head shape (H_q 16, H_kv 8, d 128), softmax.
DECODE_GLOBAL_128K = DecodeConfig("gemma3_global_decode_bf16_S2_Hq16_Hkv8_d128_ctx131072",
                                  "bf16", num_seqs=2, H_q=16, H_kv=8, d=128, w=131072, s=0,
                                  mode=SOFTMAX, rope_theta=1e6, slopes=None, len_lo=98304,
                                  len_hi=131000, steps=32, seed=9)


@dataclass(frozen=True)
class ChunkConfig:
    """Chunked prefill over the ring cache: every step gives each of num_seqs sequences its
    next `chunk` prompt rows; the cache already holds a history of hist_lo..hist_hi tokens
    (synthetic rotated keys and values, as for decode)."""
    name: str
    dtype: str
    num_seqs: int
    H_q: int
    H_kv: int
    d: int
    w: int
    s: int
    mode: int
    rope_theta: float
    slopes: Optional[tuple]
    hist_lo: int
    hist_hi: int
    chunk: int
    steps: int
    seed: int = 0


# Serving-style chunked prefill at the C3 layer shape: 8 prompts, 2048 rows each per step,
# histories past the 4,096-token window (measurement only).
CHUNK_W4096 = ChunkConfig("mistral7b_chunked_prefill_bf16_S8_chunk2048_Hq32_Hkv8_d128_w4096",
                          "bf16", num_seqs=8, H_q=32, H_kv=8, d=128, w=4096, s=0, mode=SOFTMAX,
                          rope_theta=1e6, slopes=None, hist_lo=4096, hist_hi=32768, chunk=2048,
                          steps=8, seed=8)

PREFILL_CONFIGS = {c.name: c for c in (C1, C2, C3, C5)}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(cfg: PrefillConfig, device="cpu"):
    """Q [B,N,H_q,d], K/V [B,N,H_kv,d] drawn N(0,1)*input_scale in float32, then rounded
    to the input dtype. When heavy_k_frac > 0, exactly round(frac*B*N*H_kv) (position,
    kv head) K rows, chosen without replacement by a seeded permutation, are multiplied by
    heavy_k_mult before rounding."""
    g = _gen(cfg.seed, device)
    dt = torch_dtype(cfg.dtype)
    shape_q = (cfg.B, cfg.N, cfg.H_q, cfg.d)
    shape_k = (cfg.B, cfg.N, cfg.H_kv, cfg.d)
    q = torch.randn(shape_q, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shape_k, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape_k, generator=g, device=device, dtype=torch.float32)
    if cfg.input_scale != 1.0:
        q.mul_(cfg.input_scale)
        k.mul_(cfg.input_scale)
        v.mul_(cfg.input_scale)
    if cfg.heavy_k_frac > 0.0:
        rows = cfg.B * cfg.N * cfg.H_kv
        n_heavy = int(round(cfg.heavy_k_frac * rows))
        perm = torch.randperm(rows, generator=g, device=device)[:n_heavy]
        kf = k.view(rows, cfg.d)
        kf[perm] *= cfg.heavy_k_mult
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def slopes_tensor(slopes, device="cpu") -> Optional[torch.Tensor]:
    if slopes is None:
        return None
    return torch.tensor(list(slopes), dtype=torch.float32, device=device)


@dataclass
class DecodeState:
    """Initial cache contents and per-step new tokens for a decode workload.

    k_ring/v_ring [S, H_kv, w, d] and k_sink/v_sink [S, H_kv, s, d] are synthetic
    already-rotated keys and values: the ring is taken to hold the w most recent
    positions before each sequence's start length, the sink store positions 0..s-1.
    lengths [S] int32: the position of each sequence's first decode token.
    q_steps [steps, S, H_q, d], k_steps/v_steps [steps, S, 1, H_kv, d]: the new tokens
    (queries and keys before rotation)."""
    lengths: torch.Tensor
    k_ring: torch.Tensor
    v_ring: torch.Tensor
    k_sink: Optional[torch.Tensor]
    v_sink: Optional[torch.Tensor]
    q_steps: torch.Tensor
    k_steps: torch.Tensor
    v_steps: torch.Tensor


def decode_inputs(cfg: DecodeConfig, device="cpu", steps: Optional[int] = None) -> DecodeState:
    g = _gen(cfg.seed, device)
    dt = torch_dtype(cfg.dtype)
    T = cfg.steps if steps is None else steps
    S = cfg.num_seqs
    lengths = torch.randint(cfg.len_lo, cfg.len_hi + 1, (S,), generator=g, device=device,
                            dtype=torch.int64).to(torch.int32)
    rn = lambda *shape: torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt)
    k_ring = rn(S, cfg.H_kv, cfg.w, cfg.d)
    v_ring = rn(S, cfg.H_kv, cfg.w, cfg.d)
    k_sink = rn(S, cfg.H_kv, cfg.s, cfg.d) if cfg.s > 0 else None
    v_sink = rn(S, cfg.H_kv, cfg.s, cfg.d) if cfg.s > 0 else None
    q_steps = rn(T, S, cfg.H_q, cfg.d)
    k_steps = rn(T, S, 1, cfg.H_kv, cfg.d)
    v_steps = rn(T, S, 1, cfg.H_kv, cfg.d)
    return DecodeState(lengths, k_ring.contiguous(), v_ring.contiguous(), k_sink, v_sink,
                       q_steps.contiguous(), k_steps.contiguous(), v_steps.contiguous())


def sample_rows(n: int, count: int, seed: int, must=(0,)) -> list:
    """A sorted list of distinct row indices in [0, n): the given must-have rows, the last
    row, rows just around the window edges are added by callers; the rest uniform."""
    g = torch.Generator()
    g.manual_seed(seed)
    picked = set(int(m) for m in must if 0 <= m < n)
    picked.add(n - 1)
    if count > len(picked):
        extra = torch.randperm(n, generator=g)[: count].tolist()
        for e in extra:
            if len(picked) >= count:
                break
            picked.add(int(e))
    return sorted(picked)


@dataclass
class ChunkState:
    """hist [S] int32: tokens already in each sequence's cache; k_ring/v_ring [S, H_kv, w, d]
    and k_sink/v_sink [S, H_kv, s, d]: synthetic already-rotated cache contents; q [S*chunk,
    H_q, d], k/v [S*chunk, H_kv, d]: one packed chunk (keys not rotated), reused by every
    step at that step's positions."""
    hist: torch.Tensor
    k_ring: torch.Tensor
    v_ring: torch.Tensor
    k_sink: Optional[torch.Tensor]
    v_sink: Optional[torch.Tensor]
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor


def chunk_inputs(cfg: ChunkConfig, device="cpu") -> ChunkState:
    g = _gen(cfg.seed, device)
    dt = torch_dtype(cfg.dtype)
    S, T = cfg.num_seqs, cfg.num_seqs * cfg.chunk
    hist = torch.randint(cfg.hist_lo, cfg.hist_hi + 1, (S,), generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)
    rn = lambda *shape: torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt)
    k_ring, v_ring = rn(S, cfg.H_kv, cfg.w, cfg.d), rn(S, cfg.H_kv, cfg.w, cfg.d)
    k_sink = rn(S, cfg.H_kv, cfg.s, cfg.d) if cfg.s > 0 else None
    v_sink = rn(S, cfg.H_kv, cfg.s, cfg.d) if cfg.s > 0 else None
    q = rn(T, cfg.H_q, cfg.d)
    k, v = rn(T, cfg.H_kv, cfg.d), rn(T, cfg.H_kv, cfg.d)
    return ChunkState(hist, k_ring, v_ring, k_sink, v_sink, q, k, v)
