"""Seeded synthetic inputs for loop-aware attention (CPU and GPU, bit-identical).

This module generates inputs only: keys, values, queries, quantised codes and
their fp16 scale/zero metadata, the per-(layer, loop) cell plan, and the
workload shapes.  It holds none of the attention arithmetic; the fp64 oracle
under ``oracle/`` and the HIP library under ``verify_attention_loop_amd/``
both consume what it produces.

Definitions (identical in ``synth.h`` for the GPU fill kernels):

* stream key of a (tensor, seq, layer, plane, head) row: the SplitMix64 output
  function (Steele, Lea, Flood, OOPSLA 2014) applied in five stages;
* element counter ``pos * d + ch``; each element draws four 64-bit words;
* normal: Irwin-Hall sum of twelve 20-bit uniforms minus 6, on a 2^-20 grid,
  so the value is exact in fp32; bf16/fp16 by explicit round-to-nearest-even;
* ripening planes (the Huginn-shaped workload): plane r < R-1 equals the
  deepest plane plus ``0.88^(R-1-r)`` times an independent normal, summed in
  fp64 (the product is exact) and rounded once to bf16 (``MODE_RIPEN``, the
  workload's literal recipe); ``MODE_RIPEN_PAPER`` takes ``0.88^(r+1)`` instead,
  the direction of the RIPE page's ripening fit (the difference to the deepest
  plane shrinks geometrically as the loop index grows, Sec. 3.2);
* codes: Binomial(2^b - 1, 1/2) via the popcount of 2^b - 1 hashed bits;
  scales ``base * (1 + u/2^21)`` and zeros ``-mid * scale + n/8`` in fp16.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
MASK20 = (1 << 20) - 1

T_K, T_V, T_Q, T_KNOISE, T_VNOISE = 1, 2, 3, 4, 5
T_KCODE, T_VCODE, T_KSCALE, T_KZERO, T_VSCALE, T_VZERO = 6, 7, 8, 9, 10, 11
T_DRAFTK, T_DRAFTV, T_PLAN, T_PERM = 12, 13, 14, 15

DT_F32, DT_BF16 = 0, 1
MODE_PLAIN, MODE_RIPEN, MODE_RIPEN_PAPER = 0, 1, 2
CELL_BF16, CELL_INT4, CELL_INT2, CELL_SHARED = 0, 1, 2, 3


# ----------------------------------------------------------------------------- hash

def mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * MUL1) & _M64
    z = ((z ^ (z >> 27)) * MUL2) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor: int, seq: int, layer: int, plane: int, head: int) -> int:
    k = mix64_int(seed + GAMMA * (1 + tensor))
    for c in (seq, layer, plane, head):
        k = mix64_int(k + GAMMA * (1 + c))
    return k


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def draw(key: int, counter: np.ndarray) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(np.uint64(key) + np.uint64(GAMMA) * (c + np.uint64(1)))


def normal20(key: int, elem: np.ndarray) -> np.ndarray:
    """Integer n of the Irwin-Hall(12) normal n * 2^-20 (int64 array)."""
    e = np.asarray(elem, dtype=np.uint64)
    s = np.zeros(e.shape, dtype=np.uint64)
    m = np.uint64(MASK20)
    for i in range(4):
        x = draw(key, np.uint64(4) * e + np.uint64(i))
        s += (x & m) + ((x >> np.uint64(20)) & m) + ((x >> np.uint64(40)) & m)
    return s.astype(np.int64) - 6 * (1 << 20)


def normal_f32(key: int, elem: np.ndarray) -> np.ndarray:
    return (normal20(key, elem).astype(np.float32) * np.float32(1.0 / 1048576.0)).astype(np.float32)


def binom_code(key: int, elem: np.ndarray, bits: int) -> np.ndarray:
    x = draw(key, elem)
    mask = np.uint64((1 << ((1 << bits) - 1)) - 1)
    v = (x & mask).astype(np.uint64)
    # popcount of at most 15 bits
    cnt = np.zeros(v.shape, dtype=np.uint8)
    for b in range((1 << bits) - 1):
        cnt += ((v >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
    return cnt


# ----------------------------------------------------------------------------- rounding

def bf16_from_f32(f: np.ndarray) -> np.ndarray:
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_from_f64(d: np.ndarray) -> np.ndarray:
    u = np.asarray(d, dtype=np.float64).view(np.uint64).copy()
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    with np.errstate(over="ignore"):
        u = u + np.uint64((1 << 44) - 1) + lsb
    u &= np.uint64(~((1 << 45) - 1) & _M64)
    f = u.view(np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_from_f32(f: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bits, round to nearest even (finite inputs), integer algorithm."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.int64)
    sign = (u >> 16) & 0x8000
    u = u & 0x7FFFFFFF
    e = u >> 23
    sub = e < 113
    shift = np.clip(126 - e, 1, 31)
    m_sub = (u & 0x7FFFFF) | 0x800000
    h_sub = m_sub >> shift
    rem_sub = m_sub & ((np.int64(1) << shift) - 1)
    half_sub = np.int64(1) << (shift - 1)
    h_nrm = ((e - 112) << 10) | ((u & 0x7FFFFF) >> 13)
    rem_nrm = u & 0x1FFF
    h = np.where(sub, h_sub, h_nrm)
    rem = np.where(sub, rem_sub, rem_nrm)
    half = np.where(sub, half_sub, 0x1000)
    h = np.where(sub & (126 - e > 31), 0, h)
    rem = np.where(sub & (126 - e > 31), 0, rem)
    up = (rem > half) | ((rem == half) & ((h & 1) == 1))
    h = h + up.astype(np.int64)
    h = np.minimum(h, 0x7C00)
    return (sign | h).astype(np.uint16)


def f64_from_f16(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def ripen_coef(k: int) -> np.float32:
    c = 1.0
    for _ in range(k):
        c *= 0.88
    return np.float32(c)


# ----------------------------------------------------------------------------- CPU generators

def kv(dtype: int, seed: int, tensor: int, seq: int, layer: int, plane: int, n_heads: int, d: int,
       pos0: int, n_pos: int, mode: int = MODE_PLAIN, n_loops: int = 1, scale: float = 1.0,
       heads=None) -> np.ndarray:
    """Values of one (tensor, seq, layer, plane) for positions [pos0, pos0+n_pos).

    Returns [n_pos][len(heads)][d]: float32 values for DT_F32, uint16 bf16 bits for DT_BF16.
    """
    heads = list(range(n_heads)) if heads is None else list(heads)
    deepest = n_loops - 1
    ripen = mode in (MODE_RIPEN, MODE_RIPEN_PAPER) and plane != deepest
    pos = np.arange(pos0, pos0 + n_pos, dtype=np.uint64)
    elem = (pos[:, None] * np.uint64(d) + np.arange(d, dtype=np.uint64)[None, :])
    sc = np.float32(scale)
    out = np.empty((n_pos, len(heads), d), dtype=np.float32 if dtype == DT_F32 else np.uint16)
    for hi, h in enumerate(heads):
        base_plane = deepest if ripen else plane
        base = (normal_f32(stream_key(seed, tensor, seq, layer, base_plane, h), elem) * sc).astype(np.float32)
        if ripen:
            noise = (normal_f32(stream_key(seed, tensor + 3, seq, layer, plane, h), elem) * sc).astype(np.float32)
            coef = np.float64(ripen_coef(deepest - plane if mode == MODE_RIPEN else plane + 1))
        if dtype == DT_F32:
            if ripen:
                out[:, hi, :] = (base.astype(np.float64) + coef * noise.astype(np.float64)).astype(np.float32)
            else:
                out[:, hi, :] = base
        else:
            b16 = bf16_from_f32(base)
            if ripen:
                s = f32_from_bf16(b16).astype(np.float64) + coef * noise.astype(np.float64)
                out[:, hi, :] = bf16_from_f64(s)
            else:
                out[:, hi, :] = b16
    return out


def q(dtype: int, seed: int, seq_ids, t0s, layer: int, loop: int, q_len: int, n_heads: int, d: int,
      scale: float = 1.0) -> np.ndarray:
    """Queries of one (layer, loop) call: [n_seqs][q_len][n_heads][d] at positions t0+i."""
    seq_ids = list(seq_ids)
    out = np.empty((len(seq_ids), q_len, n_heads, d), dtype=np.float32 if dtype == DT_F32 else np.uint16)
    for b, (s, t0) in enumerate(zip(seq_ids, t0s)):
        pos = np.arange(t0, t0 + q_len, dtype=np.uint64)
        elem = pos[:, None] * np.uint64(d) + np.arange(d, dtype=np.uint64)[None, :]
        for h in range(n_heads):
            x = (normal_f32(stream_key(seed, T_Q, s, layer, loop, h), elem) * np.float32(scale)).astype(np.float32)
            out[b, :, h, :] = x if dtype == DT_F32 else bf16_from_f32(x)
    return out


def codes(seed: int, tensor: int, seq: int, layer: int, plane: int, n_heads: int, d: int,
          pos0: int, n_pos: int, bits: int, heads=None) -> np.ndarray:
    """Quantised codes [n_pos][heads][d] (uint8), Binomial(2^bits-1, 1/2)."""
    heads = list(range(n_heads)) if heads is None else list(heads)
    pos = np.arange(pos0, pos0 + n_pos, dtype=np.uint64)
    elem = pos[:, None] * np.uint64(d) + np.arange(d, dtype=np.uint64)[None, :]
    out = np.empty((n_pos, len(heads), d), dtype=np.uint8)
    for hi, h in enumerate(heads):
        out[:, hi, :] = binom_code(stream_key(seed, tensor, seq, layer, plane, h), elem, bits)
    return out


def meta(seed: int, which: int, seq: int, layer: int, plane: int, n_heads: int, n_ch: int,
         row0: int, n_rows: int, bits: int, heads=None) -> np.ndarray:
    """fp16 (scale, zero) bits [n_rows][heads][n_ch][2] (uint16).

    which=0: K metadata, one row per 32-token group, n_ch = head_dim channels.
    which=1: V metadata, one row per token, n_ch = head_dim/32 channel groups.
    """
    heads = list(range(n_heads)) if heads is None else list(heads)
    ts, tz = (T_KSCALE, T_KZERO) if which == 0 else (T_VSCALE, T_VZERO)
    base = np.float32(0.5 if bits == 4 else 1.0)
    mid = np.float32(7.5 if bits == 4 else 1.5)
    rows = np.arange(row0, row0 + n_rows, dtype=np.uint64)
    elem = rows[:, None] * np.uint64(n_ch) + np.arange(n_ch, dtype=np.uint64)[None, :]
    out = np.empty((n_rows, len(heads), n_ch, 2), dtype=np.uint16)
    for hi, h in enumerate(heads):
        u = (draw(stream_key(seed, ts, seq, layer, plane, h), elem) & np.uint64(MASK20)).astype(np.float32)
        sigma32 = (base * (np.float32(1.0) + u * np.float32(1.0 / 2097152.0))).astype(np.float32)
        s16 = f16_from_f32(sigma32)
        s_back = s16.view(np.float16).astype(np.float32)
        n = normal_f32(stream_key(seed, tz, seq, layer, plane, h), elem)
        z32 = ((-mid) * s_back + np.float32(0.125) * n).astype(np.float32)
        out[:, hi, :, 0] = s16
        out[:, hi, :, 1] = f16_from_f32(z32)
    return out


def cell_plan(seed: int, n_layers: int, n_loops: int) -> np.ndarray:
    """Per-(layer, loop) cell kinds: loops below the deepest draw INT4 / INT2 / SHARED with
    probabilities 0.5 / 0.3 / 0.2; the deepest loop, which shared cells read, stays INT4."""
    plan = np.empty((n_layers, n_loops), dtype=np.int8)
    for l in range(n_layers):
        for r in range(n_loops):
            if r == n_loops - 1:
                plan[l, r] = CELL_INT4
                continue
            u = int(draw(stream_key(seed, T_PLAN, 0, l, r, 0), np.array([0], dtype=np.uint64))[0] & MASK20)
            x = u / float(1 << 20)
            plan[l, r] = CELL_INT4 if x < 0.5 else (CELL_INT2 if x < 0.8 else CELL_SHARED)
    return plan


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""
    name: str
    batch: int
    n_layers: int
    n_loops: int
    n_heads: int
    head_dim: int
    length: int              # positions including the query (decode) or the block (verify)
    dtype: int
    policy: str              # "full" or "ripe"
    window: int = 0
    q_len: int = 1
    page: int = 16
    mode: int = MODE_PLAIN   # value recipe of the planes
    scale: float = 1.0       # value scale of K, V, Q
    split_k: int = 1
    shuffle: bool = False
    quant: bool = False
    sink: int = 0
    tail: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict)
    n_kv_heads: int = 0      # 0: multi-head (= n_heads); else grouped-query attention

    @property
    def hkv(self) -> int:
        return self.n_kv_heads or self.n_heads


WORKLOADS = {
    # Tiny fp32 full-depth decode; RIPE windows {0, 16, 128} run on the same inputs.
    "tiny": Workload("tiny", 1, 1, 4, 2, 64, 128, DT_F32, "full", 0, 1, 16, MODE_PLAIN, 0.125),
    # Huginn-shaped RIPE decode: 4 core layers x 32 planes, 55 heads x 96, W=64, batch 32.
    "huginn_ripe": Workload("huginn_ripe", 32, 4, 32, 55, 96, 1024, DT_BF16, "ripe", 64, 1, 16,
                            MODE_RIPEN, 1.0),
    # Self-speculative verify on the Huginn shape: 800 cached + block of 8, batch 16.
    "huginn_verify": Workload("huginn_verify", 16, 4, 32, 55, 96, 808, DT_BF16, "ripe", 64, 8, 16,
                              MODE_RIPEN, 1.0, extra={"draft_loops": 4}),
    # The draft passes of the same self-speculative step: 7 single-token passes (draft block growing from 1 to 7
    # tokens) through the first 4 loops of every layer, 16 seqs with 800 cached positions (length counts the
    # cached positions here) that the draft reads from the deepest plane (draft window 0); the block's own keys
    # and values come from scratch.
    "huginn_draft": Workload("huginn_draft", 16, 4, 32, 55, 96, 800, DT_BF16, "ripe", 64, 1, 16, MODE_RIPEN, 1.0,
                             extra={"draft_passes": 7, "draft_loops": 4, "draft_window": 0}),
    # Ouro-shaped paged decode: 24 layers x 4 loops, 16 heads x 128, L=8192, batch 32, 8 splits.
    "ouro_splitk": Workload("ouro_splitk", 32, 24, 4, 16, 128, 8192, DT_BF16, "full", 0, 1, 16,
                            MODE_PLAIN, 1.0, split_k=8, shuffle=True),
    # LoopKV-style cells on the Ouro shape at L=16384, batch 16; sink 4, tail 128.
    # Raven-shaped RIPE decode with grouped-query attention: 6 core layers x 32 planes, 8 KV heads x 64 shared
    # by groups of 4 query heads (32 query heads), L=1024, W=64, batch 64.
    "raven_ripe": Workload("raven_ripe", 64, 6, 32, 32, 64, 1024, DT_BF16, "ripe", 64, 1, 16, MODE_RIPEN, 1.0,
                           split_k=0, n_kv_heads=8),
    # Dory-shaped grouped-query decode in the model's trained last-loop mode: every loop reads the final
    # loop's KV for the history (the deepest-plane cache, RIPE with W = 0) and its own plane only for the
    # current token.  5 recurrent full-attention layers x 4 loops, 4 KV heads x 256 shared by groups of 4
    # query heads (16 query heads), L = 16384, batch 32.
    "dory_lastloop": Workload("dory_lastloop", 32, 5, 4, 16, 256, 16384, DT_BF16, "ripe", 0, 1, 16, MODE_PLAIN,
                              1.0, split_k=0, n_kv_heads=4),
    # split_k 0: the library chooses the number of far splits.
    "loopkv_cells": Workload("loopkv_cells", 16, 24, 4, 16, 128, 16384, DT_BF16, "full", 0, 1, 16,
                             MODE_PLAIN, 1.0, split_k=0, quant=True, sink=4, tail=128),
}


# ----------------------------------------------------------------------------- GPU fill kernels

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libsynth.so")


def _lib():
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(p)
        vp, i32, u64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float
        L.synth_fill_kv.argtypes = [vp, i32, u64, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp]
        L.synth_fill_q.argtypes = [vp, i32, u64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                   i32, i32, i32, i32, i32, i32, f32, vp]
        L.synth_fill_codes.argtypes = [vp, u64, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]
        L.synth_fill_meta.argtypes = [vp, u64, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]
        for f in (L.synth_fill_kv, L.synth_fill_q, L.synth_fill_codes, L.synth_fill_meta):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def gpu_kv(ptr: int, dtype: int, seed: int, tensor: int, seq: int, layer: int, plane: int, n_heads: int,
           d: int, pos0: int, n_pos: int, mode: int, n_loops: int, scale: float, stream: int):
    _check(_lib().synth_fill_kv(ptr, dtype, seed, tensor, seq, layer, plane, n_heads, d, pos0, n_pos, mode,
                                n_loops, scale, stream), "synth_fill_kv")


def gpu_q(ptr: int, dtype: int, seed: int, seq_ids, t0s, layer: int, loop: int, q_len: int, n_heads: int,
          d: int, scale: float, stream: int):
    n = len(seq_ids)
    a = (ctypes.c_int32 * n)(*seq_ids)
    b = (ctypes.c_int32 * n)(*t0s)
    _check(_lib().synth_fill_q(ptr, dtype, seed, a, b, n, layer, loop, q_len, n_heads, d, scale, stream),
           "synth_fill_q")


def gpu_codes(ptr: int, seed: int, tensor: int, seq: int, layer: int, plane: int, n_heads: int, d: int,
              pos0: int, n_pos: int, bits: int, stream: int):
    _check(_lib().synth_fill_codes(ptr, seed, tensor, seq, layer, plane, n_heads, d, pos0, n_pos, bits, stream),
           "synth_fill_codes")


def gpu_meta(ptr: int, seed: int, which: int, seq: int, layer: int, plane: int, n_heads: int, n_ch: int,
             row0: int, n_rows: int, bits: int, stream: int):
    _check(_lib().synth_fill_meta(ptr, seed, which, seq, layer, plane, n_heads, n_ch, row0, n_rows, bits, stream),
           "synth_fill_meta")
