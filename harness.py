"""Workload builder shared by the GPU tests, ``__graft_entry__.smoke()`` and ``bench.py``.

Builds a ``LoopCache`` for a ``synth.Workload`` by generating each plane on the
GPU with the seeded fill kernels and appending it through the C-ABI, exactly as
a serving engine would append the planes its loops produce.  It also assembles
the CPU-side inputs of sampled rows (same generator, same bits) for the oracle.
This module does no attention arithmetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

import synth
import verify_attention_loop_amd as vla


def torch_dtype(dt):
    import torch
    return torch.float32 if dt == synth.DT_F32 else torch.bfloat16


@dataclass
class Built:
    cache: vla.LoopCache
    w: synth.Workload
    seqs: list          # sequence slot per batch row
    lengths: list       # L per batch row
    rows: list          # generator sequence coordinate per batch row
    layers: list
    planes: list
    window: int


def ripe_window_start(L: int, q_len: int, W: int) -> int:
    """First position whose non-deepest planes a RIPE cache still holds for a call whose block
    starts at t0 = L - q_len (RIPE page, Alg. 1 step 7: planes of positions older than W are dropped)."""
    return max(0, L - q_len - W)


def pages_needed(w: synth.Workload, lengths, layers, planes, policy: int, W: int, q_len: int) -> int:
    R = w.n_loops
    n = 0
    for L in lengths:
        for _ in layers:
            for p in planes:
                if policy == vla.POLICY_RIPE and p < R - 1:
                    a = ripe_window_start(L, q_len, W)
                    n += (L - 1) // 16 - a // 16 + 1
                else:
                    n += (L + 15) // 16
    return n


def build_plain(w: synth.Workload, *, lengths=None, layers=(0,), planes=None, policy=None, window=None,
                q_len=None, shuffle=None, poison=False, seed=None, extra_pages=0, max_len=None,
                chunk_tokens=4096, rows=None) -> Built:
    """Cache of a plain (fp32/bf16) workload holding the given layers and planes."""
    import torch
    R = w.n_loops
    lengths = list(lengths) if lengths is not None else [w.length] * w.batch
    rows = list(rows) if rows is not None else list(range(len(lengths)))
    planes = list(planes) if planes is not None else list(range(R))
    policy = policy if policy is not None else (vla.POLICY_RIPE if w.policy == "ripe" else vla.POLICY_FULL)
    W = w.window if window is None else window
    q_len = w.q_len if q_len is None else q_len
    shuffle = w.shuffle if shuffle is None else shuffle
    seed = w.seed if seed is None else seed
    if policy == vla.POLICY_RIPE and R - 1 not in planes:
        planes = planes + [R - 1]
    n_pages = pages_needed(w, lengths, layers, planes, policy, W, q_len) + extra_pages
    cfg = vla.LoopCache.config(n_layers=w.n_layers, n_loops=R, n_heads_q=w.n_heads, n_heads_kv=w.n_heads,
                               head_dim=w.head_dim, kv_dtype=w.dtype, policy=policy, window=W,
                               max_seqs=len(lengths), max_len=max_len or max(lengths), max_block=max(1, q_len),
                               poison=1 if poison else 0, shuffle_seed=(0x5EED + seed) if shuffle else 0)
    cache = vla.LoopCache.on_device(cfg, n_pages)
    dt = torch_dtype(w.dtype)
    H, d = w.n_heads, w.head_dim
    stream = torch.cuda.current_stream().cuda_stream
    seqs = []
    chunk = min(chunk_tokens, max(lengths))
    kbuf = torch.empty((chunk, H, d), dtype=dt, device="cuda")
    vbuf = torch.empty((chunk, H, d), dtype=dt, device="cuda")
    for b, L in enumerate(lengths):
        s = cache.lkv_add_seq()
        seqs.append(s)
        for layer in layers:
            order = [R - 1] + [p for p in planes if p != R - 1] if policy == vla.POLICY_RIPE else planes
            for p in order:
                a = 0
                if policy == vla.POLICY_RIPE and p < R - 1:
                    a = ripe_window_start(L, q_len, W)
                for p0 in range(a, L, chunk):
                    n = min(chunk, L - p0)
                    synth.gpu_kv(kbuf.data_ptr(), w.dtype, seed, synth.T_K, rows[b], layer, p, H, d, p0, n,
                                 w.mode, R, w.scale, stream)
                    synth.gpu_kv(vbuf.data_ptr(), w.dtype, seed, synth.T_V, rows[b], layer, p, H, d, p0, n,
                                 w.mode, R, w.scale, stream)
                    cache.lkv_append_plane(s, layer, p, p0, kbuf[:n], vbuf[:n])
                if policy == vla.POLICY_RIPE and p == R - 1:
                    cache.lkv_commit(s, L - q_len)
        if policy != vla.POLICY_RIPE:
            cache.lkv_commit(s, L - q_len)
    torch.cuda.synchronize()
    return Built(cache, w, seqs, lengths, rows, list(layers), planes, W)


def gpu_queries(built: Built, layer: int, loop: int, q_len: int, t0s=None, seed=None):
    import torch
    w = built.w
    t0s = t0s if t0s is not None else [L - q_len for L in built.lengths]
    out = torch.empty((len(built.seqs), q_len, w.n_heads, w.head_dim), dtype=torch_dtype(w.dtype), device="cuda")
    for b0 in range(0, len(built.seqs), 64):
        b1 = min(len(built.seqs), b0 + 64)
        synth.gpu_q(out[b0:b1].data_ptr(), w.dtype, w.seed if seed is None else seed, built.rows[b0:b1],
                    t0s[b0:b1], layer, loop, q_len, w.n_heads, w.head_dim, w.scale,
                    torch.cuda.current_stream().cuda_stream)
    return out


def cpu_values(w: synth.Workload, tensor: int, b: int, layer: int, plane: int, head: int, n_pos: int, seed=None):
    """fp64 values [n_pos][d] of one (tensor, row, layer, plane, head), as the cache holds them."""
    x = synth.kv(w.dtype, w.seed if seed is None else seed, tensor, b, layer, plane, w.n_heads, w.head_dim, 0,
                 n_pos, w.mode, w.n_loops, w.scale, heads=[head])[:, 0, :]
    return to_f64(x, w.dtype)


def cpu_query(w: synth.Workload, b: int, layer: int, loop: int, head: int, pos: int, seed=None):
    x = synth.q(w.dtype, w.seed if seed is None else seed, [b], [pos], layer, loop, 1, w.n_heads, w.head_dim,
                w.scale)[0, 0, head]
    return to_f64(x, w.dtype)


def to_f64(x, dt):
    if dt == synth.DT_F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return synth.f32_from_bf16(np.asarray(x, dtype=np.uint16)).astype(np.float64)


def out_f64(t):
    """Device output tensor (fp32 or bf16) -> numpy fp64."""
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(
        np.float64)


def oracle_rows(w: synth.Workload, rows, layer: int, loop: int, lengths, q_len: int, policy: int, W: int,
                synth_rows=None):
    """Oracle outputs of sampled rows: rows is a list of (b, i, h) with query position L_b - q_len + i."""
    import oracle
    R = w.n_loops
    outs, lses = [], []
    cache = {}
    for (b, i, h) in rows:
        L = lengths[b]
        sb = synth_rows[b] if synth_rows is not None else b
        key = (sb, h, L)
        if key not in cache:
            ko = cpu_values(w, synth.T_K, sb, layer, loop, h, L)
            vo = cpu_values(w, synth.T_V, sb, layer, loop, h, L)
            if loop == R - 1 or policy == oracle.FULL:
                kd, vd = ko, vo
            else:
                kd = cpu_values(w, synth.T_K, sb, layer, R - 1, h, L)
                vd = cpu_values(w, synth.T_V, sb, layer, R - 1, h, L)
            cache = {key: (ko, vo, kd, vd)}
        ko, vo, kd, vd = cache[key]
        t0 = L - q_len
        t = t0 + i
        q = cpu_query(w, sb, layer, loop, h, t)
        o, lse = oracle.attend_row(q, ko, vo, kd, vd, t, t0, policy, loop, R, W)
        outs.append(o)
        lses.append(lse)
    return np.array(outs), np.array(lses)


def sample_rows(n_b: int, q_len: int, n_h: int, k: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    rows = set()
    # corners first
    for b in (0, n_b - 1):
        for h in (0, n_h - 1):
            rows.add((b, q_len - 1, h))
    while len(rows) < min(k, n_b * q_len * n_h):
        rows.add((int(rng.integers(n_b)), int(rng.integers(q_len)), int(rng.integers(n_h))))
    return sorted(rows, key=lambda r: (r[0], r[2], r[1]))


def algorithmic_bytes_per_call(w: synth.Workload, lengths, q_len: int = 1) -> int:
    """Distinct K/V bytes one (layer, loop) call must read: every visible position once per
    (sequence, KV head), in the cache dtype, plus Q and O."""
    es = 4 if w.dtype == synth.DT_F32 else 2
    kv = sum(2 * L * w.n_heads * w.head_dim * es for L in lengths)
    qo = 2 * len(lengths) * q_len * w.n_heads * w.head_dim * es
    return kv + qo
