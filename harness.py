"""Workload builder shared by the GPU tests, ``__graft_entry__.smoke()`` and ``bench.py``.

Builds a ``LoopCache`` for a ``synth.Workload`` by generating each plane on the
GPU with the seeded fill kernels and appending it through the C-ABI, exactly as
a serving engine would append the planes its loops produce.  It also assembles
the CPU-side inputs of sampled rows (same generator, same bits) for the oracle;
the functions that reach the oracle (``oracle_rows``, ``cell_inputs``,
``cell_oracle_row``) import it on call and serve only the tests, ``smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never a timed or product path.  This module
does no attention arithmetic.
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
    starts at t0 = L - q_len (RIPE page, Sec. 4 and Algorithm 1: once a position leaves the window its non-deepest planes are dropped)."""
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
                chunk_tokens=4096, rows=None, max_block=None) -> Built:
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
    cfg = vla.LoopCache.config(n_layers=w.n_layers, n_loops=R, n_heads_q=w.n_heads, n_heads_kv=w.hkv,
                               head_dim=w.head_dim, kv_dtype=w.dtype, policy=policy, window=W,
                               max_seqs=len(lengths), max_len=max_len or max(lengths),
                               max_block=max_block or max(1, q_len),
                               poison=1 if poison else 0, shuffle_seed=(0x5EED + seed) if shuffle else 0)
    cache = vla.LoopCache.on_device(cfg, n_pages)
    dt = torch_dtype(w.dtype)
    H, d = w.hkv, w.head_dim  # keys and values per KV head
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
        rows = getattr(built, "rows", None) or list(range(len(built.seqs)))
        synth.gpu_q(out[b0:b1].data_ptr(), w.dtype, w.seed if seed is None else seed, rows[b0:b1],
                    t0s[b0:b1], layer, loop, q_len, w.n_heads, w.head_dim, w.scale,
                    torch.cuda.current_stream().cuda_stream)
    return out


def gpu_draft_kv(w: synth.Workload, rows, layer: int, loop: int, n_cached, dl: int, seed=None):
    """Scratch keys and values of a draft block, device [n_seqs][dl][n_kv_heads][d]: positions n_cached[b] ..
    n_cached[b] + dl - 1 of the draft streams of each sequence's row."""
    import torch
    dt = torch_dtype(w.dtype)
    dk = torch.empty((len(rows), dl, w.hkv, w.head_dim), dtype=dt, device="cuda")
    dv = torch.empty_like(dk)
    st = torch.cuda.current_stream().cuda_stream
    seed = w.seed if seed is None else seed
    for b, r in enumerate(rows):
        for t, buf in ((synth.T_DRAFTK, dk), (synth.T_DRAFTV, dv)):
            synth.gpu_kv(buf[b].data_ptr(), w.dtype, seed, t, r, layer, loop, w.hkv, w.head_dim, n_cached[b], dl,
                         synth.MODE_PLAIN, w.n_loops, w.scale, st)
    return dk, dv


def cpu_draft_values(w: synth.Workload, tensor: int, b: int, layer: int, loop: int, head: int, n_cached: int, dl: int,
                     seed=None):
    """fp64 values [dl][d] of one KV head of a draft block (the host side of gpu_draft_kv)."""
    x = synth.kv(w.dtype, w.seed if seed is None else seed, tensor, b, layer, loop, w.hkv, w.head_dim, n_cached, dl,
                 synth.MODE_PLAIN, w.n_loops, w.scale, heads=[head])[:, 0, :]
    return to_f64(x, w.dtype)


def cpu_values(w: synth.Workload, tensor: int, b: int, layer: int, plane: int, head: int, n_pos: int, seed=None):
    """fp64 values [n_pos][d] of one (tensor, row, layer, plane, KV head), as the cache holds them."""
    x = synth.kv(w.dtype, w.seed if seed is None else seed, tensor, b, layer, plane, w.hkv, w.head_dim, 0,
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
    """Oracle outputs of sampled rows: rows is a list of (b, i, h) with query position L_b - q_len + i; query head
    h reads KV head h // (n_heads / n_kv_heads)."""
    import oracle
    R = w.n_loops
    group = w.n_heads // w.hkv
    outs, lses = [], []
    cache = {}
    for (b, i, h) in rows:
        L = lengths[b]
        sb = synth_rows[b] if synth_rows is not None else b
        hk = h // group
        key = (sb, hk, L)
        if key not in cache:
            ko = cpu_values(w, synth.T_K, sb, layer, loop, hk, L)
            vo = cpu_values(w, synth.T_V, sb, layer, loop, hk, L)
            if loop == R - 1 or policy == oracle.FULL:
                kd, vd = ko, vo
            else:
                kd = cpu_values(w, synth.T_K, sb, layer, R - 1, hk, L)
                vd = cpu_values(w, synth.T_V, sb, layer, R - 1, hk, L)
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
    kv = sum(2 * L * w.hkv * w.head_dim * es for L in lengths)
    qo = 2 * len(lengths) * q_len * w.n_heads * w.head_dim * es
    return kv + qo


# ----------------------------------------------------------------------------- quantised cells

@dataclass
class BuiltCells:
    cache: vla.LoopCache
    w: synth.Workload
    seqs: list
    lengths: list
    layers: list
    plan: np.ndarray


def cell_src_loop(plan, layer: int, loop: int) -> int:
    """A shared cell reads the final loop's codes (LoopKV page, Sec. 3.2)."""
    return plan.shape[1] - 1 if plan[layer, loop] == synth.CELL_SHARED else loop


def cell_bits(plan, layer: int, loop: int) -> int:
    return 2 if plan[layer, cell_src_loop(plan, layer, loop)] == synth.CELL_INT2 else 4


def build_cells(w: synth.Workload, *, lengths=None, layers=(0,), loops=None, plan=None, seed=None) -> BuiltCells:
    """LoopKV-style cache: bf16 sink and tail of every cell, and far-history code pages of every
    non-shared cell, written through lkv_append_plane / lkv_append_coded."""
    import torch
    R, H, D = w.n_loops, w.n_heads, w.head_dim
    seed = w.seed if seed is None else seed
    lengths = list(lengths) if lengths is not None else [w.length] * w.batch
    loops = list(loops) if loops is not None else list(range(R))
    plan = np.array(plan if plan is not None else synth.cell_plan(seed, w.n_layers, R), dtype=np.int8)
    needed = set()
    for layer in layers:
        for r in loops:
            needed.add((layer, r))
            needed.add((layer, cell_src_loop(plan, layer, r)))
    n_near = n4 = n2 = 0
    for L in lengths:
        n_far = L - w.sink - w.tail
        n_cp = (n_far + 31) // 32
        near_pages = len(set(range((w.sink - 1) // 16 + 1)) | set(range((L - w.tail) // 16, (L - 1) // 16 + 1)))
        for (layer, r) in needed:
            n_near += near_pages
            if plan[layer, r] == synth.CELL_INT4:
                n4 += n_cp
            elif plan[layer, r] == synth.CELL_INT2:
                n2 += n_cp
    cfg = vla.LoopCache.config(n_layers=w.n_layers, n_loops=R, n_heads_q=H, n_heads_kv=H, head_dim=D,
                               kv_dtype=synth.DT_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=len(lengths),
                               max_len=max(lengths), max_block=1, quant=1, sink=w.sink, tail=w.tail)
    cache = vla.LoopCache.on_device(cfg, n_near, n4, n2)
    cache.lkv_set_plan(plan)
    st = torch.cuda.current_stream().cuda_stream
    seqs = []
    for b, L in enumerate(lengths):
        s = cache.lkv_add_seq()
        seqs.append(s)
        n_far = L - w.sink - w.tail
        n_cp = (n_far + 31) // 32
        for (layer, r) in sorted(needed):
            for (p0, n) in ((0, w.sink), (L - w.tail, w.tail)):
                if n <= 0:
                    continue
                k = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
                v = torch.empty_like(k)
                synth.gpu_kv(k.data_ptr(), synth.DT_BF16, seed, synth.T_K, b, layer, r, H, D, p0, n, synth.MODE_PLAIN,
                             R, w.scale, st)
                synth.gpu_kv(v.data_ptr(), synth.DT_BF16, seed, synth.T_V, b, layer, r, H, D, p0, n, synth.MODE_PLAIN,
                             R, w.scale, st)
                cache.lkv_append_plane(s, layer, r, p0, k, v)
            if plan[layer, r] == synth.CELL_SHARED:
                continue
            bits = 2 if plan[layer, r] == synth.CELL_INT2 else 4
            kc = torch.empty((n_cp * 32, H, D), dtype=torch.uint8, device="cuda")
            vc = torch.empty_like(kc)
            km = torch.empty((n_cp, H, D, 2), dtype=torch.int16, device="cuda")
            vm = torch.empty((n_cp * 32, H, D // 32, 2), dtype=torch.int16, device="cuda")
            synth.gpu_codes(kc.data_ptr(), seed, synth.T_KCODE, b, layer, r, H, D, w.sink, n_cp * 32, bits, st)
            synth.gpu_codes(vc.data_ptr(), seed, synth.T_VCODE, b, layer, r, H, D, w.sink, n_cp * 32, bits, st)
            synth.gpu_meta(km.data_ptr(), seed, 0, b, layer, r, H, D, 0, n_cp, bits, st)
            synth.gpu_meta(vm.data_ptr(), seed, 1, b, layer, r, H, D // 32, 0, n_cp * 32, bits, st)
            cache.lkv_append_coded(s, layer, r, 0, n_cp, kc, km, vc, vm)
        torch.cuda.synchronize()
    return BuiltCells(cache, w, seqs, lengths, list(layers), plan)


def cell_inputs(bc: BuiltCells, b: int, layer: int, loop: int, h: int, seed=None):
    """The oracle's inputs for one cell row, regenerated on the host from the generator (same bits as the
    device cache): query, exact near keys/values, far codes and fp64 metadata, the oracle cell kind."""
    import oracle
    w = bc.w
    seed = w.seed if seed is None else seed
    L = bc.lengths[b]
    D = w.head_dim
    n_far = L - w.sink - w.tail
    n_cp = (n_far + 31) // 32
    src = cell_src_loop(bc.plan, layer, loop)
    bits = cell_bits(bc.plan, layer, loop)
    kind = {synth.CELL_INT4: oracle.CELL_INT4, synth.CELL_INT2: oracle.CELL_INT2,
            synth.CELL_SHARED: oracle.CELL_SHARED}[int(bc.plan[layer, loop])]
    kn = np.zeros((L, D))
    vn = np.zeros((L, D))
    for (p0, n) in ((0, w.sink), (L - w.tail, w.tail)):
        kn[p0:p0 + n] = to_f64(synth.kv(synth.DT_BF16, seed, synth.T_K, b, layer, loop, w.n_heads, D, p0, n,
                                        heads=[h])[:, 0], synth.DT_BF16)
        vn[p0:p0 + n] = to_f64(synth.kv(synth.DT_BF16, seed, synth.T_V, b, layer, loop, w.n_heads, D, p0, n,
                                        heads=[h])[:, 0], synth.DT_BF16)
    kc = synth.codes(seed, synth.T_KCODE, b, layer, src, w.n_heads, D, w.sink, n_far, bits, heads=[h])[:, 0]
    vc = synth.codes(seed, synth.T_VCODE, b, layer, src, w.n_heads, D, w.sink, n_far, bits, heads=[h])[:, 0]
    km = synth.f64_from_f16(synth.meta(seed, 0, b, layer, src, w.n_heads, D, 0, n_cp, bits, heads=[h])[:, 0])
    vm = synth.f64_from_f16(synth.meta(seed, 1, b, layer, src, w.n_heads, D // 32, 0, n_far, bits, heads=[h])[:, 0])
    q = cpu_query(w, b, layer, loop, h, L - 1, seed=seed)
    return dict(q=q, k_near=kn, v_near=vn, kc=kc, ks=km[..., 0], kz=km[..., 1], vc=vc, vs=vm[..., 0],
                vz=vm[..., 1], sink=w.sink, tail=w.tail, kind=kind)


def cell_oracle_row(bc: BuiltCells, b: int, layer: int, loop: int, h: int, thr_offset: float, seed=None):
    """Oracle inputs of one cell row from the generator, and the oracle's (out, lse, hot bits, scores)."""
    import oracle
    w = bc.w
    D = w.head_dim
    a = cell_inputs(bc, b, layer, loop, h, seed)
    out, lse, hot, n_cold = oracle.cell_row(a["q"], a["k_near"], a["v_near"], a["kc"], a["ks"], a["kz"], a["vc"],
                                            a["vs"], a["vz"], a["sink"], a["tail"], a["kind"], thr_offset)
    # scores of far tokens and the threshold (only to place the rounding band of the mask comparison)
    n_far = a["kc"].shape[0]
    g = np.arange(n_far) // 32
    kh = a["kz"][g] + a["ks"][g] * a["kc"]
    s_far = kh @ a["q"] / np.sqrt(D)
    m0 = (a["k_near"][:w.sink] @ a["q"] / np.sqrt(D)).max()
    return out, lse, hot, s_far, m0 - thr_offset


def cell_bytes_per_call(bc: BuiltCells, layer: int, loop: int, n_cold: int = 0) -> int:
    """Algorithmic bytes of one cell call: every far token-head's codes and metadata once (INT4 and shared
    cells: K codes 64 B + K metadata 16 B + V hi 32 B + V lo 32 B + V metadata 16 B = 160 B, the lo 32 B
    only for hot tokens; INT2: 96 B), the exact sink and tail keys and values, and Q and O."""
    w = bc.w
    H, D = w.n_heads, w.head_dim
    per_tok = (40 if cell_bits(bc.plan, layer, loop) == 4 else 24) * D // 32  # bytes per token-head
    far = sum(L - w.sink - w.tail for L in bc.lengths) * H * per_tok
    near = len(bc.lengths) * (w.sink + w.tail) * H * 2 * D * 2
    qo = 2 * len(bc.lengths) * H * D * 2
    lo_skipped = 32 * n_cold if cell_bits(bc.plan, layer, loop) == 4 else 0
    return far + near + qo - lo_skipped


# ----------------------------------------------------------------------------- multi-step self-speculative loop

class SpecLoop:
    """A synthetic run of the RIPE page's self-speculative step (Sec. 4, Algorithm 1) through the C-ABI.

    The cache holds positions [0, len) of each sequence; the next block starts with the last emitted token x at
    position len.  One step of block length gamma (drawn per step by the caller, 1 <= gamma <= max_gamma): gamma
    draft passes (q = 1 at loops 0..d-1, cached positions read plane R, the block from caller scratch), one verify
    pass over the block of gamma + 1 tokens at every loop (the block's plane r is appended before loop r
    attends), then a seeded acceptance of a in [0, gamma] drafts: the planes of x and the accepted drafts stay
    (commit to len + 1 + a, which also drops non-deepest planes that left the window) and the rest is truncated.
    Keys and values of position j are generated with a per-position version that grows every time the position
    is written again, so a truncated and rewritten position holds new values.  There are no logits: acceptance
    is drawn, and the attention outputs are what the caller checks."""

    def __init__(self, w: synth.Workload, prefix_lengths, max_gamma: int, d: int, window: int, seed: int = 0):
        import torch
        self.w, self.max_gamma, self.d, self.W = w, max_gamma, d, window
        self.max_block = max_gamma + 1
        self.rng = np.random.default_rng(seed)
        R, H, D = w.n_loops, w.hkv, w.head_dim
        max_len = max(prefix_lengths) + 64 * self.max_block
        self.max_len = max_len
        cfg = vla.LoopCache.config(n_layers=w.n_layers, n_loops=R, n_heads_q=w.n_heads, n_heads_kv=H, head_dim=D,
                                   kv_dtype=w.dtype, policy=vla.POLICY_RIPE, window=window,
                                   max_seqs=len(prefix_lengths), max_len=max_len, max_block=self.max_block, poison=1,
                                   shuffle_seed=0x5EED + seed)
        n_pages = len(prefix_lengths) * w.n_layers * ((max_len + 15) // 16 +
                                                      (R - 1) * ((window + self.max_block) // 16 + 2))
        self.cache = vla.LoopCache.on_device(cfg, n_pages)
        self.version = [np.zeros(max_len, dtype=np.int64) for _ in prefix_lengths]
        self.seqs = [self.cache.lkv_add_seq() for _ in prefix_lengths]
        self.lengths = list(prefix_lengths)
        for b, L in enumerate(prefix_lengths):
            for layer in range(w.n_layers):
                self._append(b, layer, R - 1, 0, L)
            self.cache.lkv_commit(self.seqs[b], L)  # the window is measured from the committed length
            for layer in range(w.n_layers):
                for plane in range(R - 1):
                    a = max(0, L - window)
                    self._append(b, layer, plane, a, L - a)
        torch.cuda.synchronize()

    def draw_gamma(self, lo: int = 1, hi: int = 0) -> int:
        """A block length for the next step, uniform in [lo, hi] (hi = max_gamma by default), seeded."""
        return int(self.rng.integers(lo, (hi or self.max_gamma) + 1))

    # generator coordinates of (seq b, position j): one row per (b, version)
    def _row(self, b, j):
        return b * 4096 + int(self.version[b][j])

    def _append(self, b, layer, plane, pos0, n):
        import torch
        w = self.w
        dt = torch_dtype(w.dtype)
        k = torch.empty((n, w.hkv, w.head_dim), dtype=dt, device="cuda")
        v = torch.empty_like(k)
        st = torch.cuda.current_stream().cuda_stream
        for j in range(pos0, pos0 + n):
            r = self._row(b, j)
            synth.gpu_kv(k[j - pos0].data_ptr(), w.dtype, w.seed, synth.T_K, r, layer, plane, w.hkv, w.head_dim, j, 1,
                         w.mode, w.n_loops, w.scale, st)
            synth.gpu_kv(v[j - pos0].data_ptr(), w.dtype, w.seed, synth.T_V, r, layer, plane, w.hkv, w.head_dim, j, 1,
                         w.mode, w.n_loops, w.scale, st)
        self.cache.lkv_append_plane(self.seqs[b], layer, plane, pos0, k, v)

    def host_kv(self, tensor, b, layer, plane, hk, L):
        """fp64 [L][d] keys or values of positions 0..L-1 as currently written (their versions)."""
        w = self.w
        out = np.empty((L, w.head_dim))
        for j in range(L):
            x = synth.kv(w.dtype, w.seed, tensor, self._row(b, j), layer, plane, w.hkv, w.head_dim, j, 1, w.mode,
                         w.n_loops, w.scale, heads=[hk])[0, 0]
            out[j] = to_f64(x, w.dtype)
        return out

    def query(self, b, layer, loop, h, pos, salt=0):
        return cpu_query(self.w, self._row(b, pos) + 100000 * salt, layer, loop, h, pos)

    def gpu_query(self, layer, loop, t0s, q_len, salt=0):
        import torch
        w = self.w
        out = torch.empty((len(self.seqs), q_len, w.n_heads, w.head_dim), dtype=torch_dtype(w.dtype), device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        for b, t0 in enumerate(t0s):
            for i in range(q_len):
                synth.gpu_q(out[b, i].data_ptr(), w.dtype, w.seed, [self._row(b, t0 + i) + 100000 * salt], [t0 + i],
                            layer, loop, 1, w.n_heads, w.head_dim, w.scale, st)
        return out

    def draft_pass(self, i):
        """Draft token i (1..gamma) at every draft loop; returns {(layer, loop): (out, draft scratch k, v)}."""
        import torch
        w = self.w
        dt = torch_dtype(w.dtype)
        res = {}
        st = torch.cuda.current_stream().cuda_stream
        for layer in range(w.n_layers):
            for loop in range(self.d):
                dk = torch.empty((len(self.seqs), i, w.hkv, w.head_dim), dtype=dt, device="cuda")
                dv = torch.empty_like(dk)
                for b, L in enumerate(self.lengths):
                    synth.gpu_kv(dk[b].data_ptr(), w.dtype, w.seed, synth.T_DRAFTK, self._row(b, L), layer, loop,
                                 w.hkv, w.head_dim, L, i, synth.MODE_PLAIN, w.n_loops, w.scale, st)
                    synth.gpu_kv(dv[b].data_ptr(), w.dtype, w.seed, synth.T_DRAFTV, self._row(b, L), layer, loop,
                                 w.hkv, w.head_dim, L, i, synth.MODE_PLAIN, w.n_loops, w.scale, st)
                q = self.gpu_query(layer, loop, [L + i - 1 for L in self.lengths], 1, salt=1)
                out = torch.empty_like(q)
                ws = torch.empty(max(4, self.cache.lkv_workspace_bytes(layer, loop, self.seqs, mode=vla.MODE_DRAFT,
                                                                       split_k=2)), dtype=torch.uint8, device="cuda")
                self.cache.lkv_attend(layer, loop, self.seqs, q, out, mode=vla.MODE_DRAFT, window=0, split_k=2,
                                      workspace=ws, draft_k=dk, draft_v=dv, draft_len=i)
                res[(layer, loop)] = (out, dk, dv)
        return res

    def verify_pass(self, gamma: int):
        """Append the planes of a block of gamma + 1 tokens and verify at every (layer, loop); returns
        {(layer, loop): out}."""
        import torch
        assert 1 <= gamma <= self.max_gamma
        w, k = self.w, gamma + 1
        outs = {}
        for loop in range(w.n_loops):
            for layer in range(w.n_layers):
                for b, L in enumerate(self.lengths):
                    self._append(b, layer, loop, L, k)
                q = self.gpu_query(layer, loop, self.lengths, k)
                out = torch.empty_like(q)
                ws = torch.empty(max(4, self.cache.lkv_workspace_bytes(layer, loop, self.seqs, q_len=k,
                                                                       mode=vla.MODE_VERIFY, split_k=2)),
                                 dtype=torch.uint8, device="cuda")
                self.cache.lkv_attend(layer, loop, self.seqs, q, out, q_len=k, mode=vla.MODE_VERIFY, split_k=2,
                                      workspace=ws)
                outs[(layer, loop)] = out
        self.lengths = [L + k for L in self.lengths]
        return outs

    def accept(self, gamma: int):
        """Seeded acceptance after a verified block of gamma + 1 tokens: keep x and a in [0, gamma] drafts of each
        sequence, drop the rest."""
        accepted = []
        for b, L in enumerate(self.lengths):
            a = int(self.rng.integers(0, gamma + 1))
            new_len = L - (gamma + 1) + 1 + a
            self.cache.lkv_commit(self.seqs[b], new_len)
            self.cache.lkv_truncate(self.seqs[b], new_len)
            self.version[b][new_len:] += 1  # positions past the accepted prefix get new values when rewritten
            self.lengths[b] = new_len
            accepted.append(a)
        return accepted

    def expected_pages(self):
        """Physical pages a RIPE cache must hold now: plane R of every position, and the non-deepest planes of
        positions >= len - W (the window ring), per sequence and layer."""
        w, W = self.w, self.W
        n = 0
        for L in self.lengths:
            deep = (L + 15) // 16
            lo = max(0, L - W)
            ring = ((L - 1) // 16 - lo // 16 + 1) if L > lo else 0
            n += w.n_layers * (deep + (w.n_loops - 1) * ring)
        return n
