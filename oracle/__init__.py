"""fp64 CPU oracle for loop-aware attention over a looped model's multi-plane KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never calls it; it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one row at a time, OpenMP
only across independent rows).  This module loads it, converts numpy arrays,
and adds the closed-form memory and byte models the pages print:

* ``oracle_plane``      -- RIPE page, Sec. 2 policy pi and Sec. 4 Eq. (9);
* ``attend_row(s)``     -- exact softmax attention over the plane-selected view;
* ``split_partials``/``lse_merge`` -- LoopKV page, Sec. 3.4 and App. E Alg. 1;
* ``cell_row``          -- LoopKV page, Sec. 3.1-3.4 (INT4 / INT2 / shared cells,
                           bit-plane V, fixed hot rule s >= m0 - offset);
* ``cell_row_running``  -- LoopKV page, Sec. 3.3 and App. E Algorithm 1 (the running-maximum V-precision rule);
* ``kivi_encode``       -- LoopKV page, Sec. 3.1 and 3.3 (the window-exit codec);
* ``mem_full``/``mem_deep``/``mem_ripe`` -- RIPE page, Eq. (3) and Eq. (10);
* ``loopkv_bytes_per_token_layer`` -- LoopKV page, App. C byte model.

Pins: every function is checked in ``tests/test_oracle_pins.py`` against
values the pages print (``tests/golden``), closed forms, invariants the pages
state (Prop. 1 of the RIPE page, Prop. 1 of the LoopKV page, W >= L-1 equals
the full cache, W = 0 reads the deepest plane), a textbook routine (torch's
fp64 scaled-dot-product attention on a materialised view) and brute force.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

FULL, RIPE = 0, 1
CELL_INT4, CELL_INT2, CELL_SHARED = 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, no contraction, OpenMP over rows)."""
    src = os.path.join(_HERE, "oracle.c")
    out = lib_path()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11", src, "-o",
           out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path()):
            build()
        L = ctypes.CDLL(lib_path())
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        pd = ctypes.POINTER(ctypes.c_double)
        pi = ctypes.POINTER(ctypes.c_int32)
        pu8 = ctypes.POINTER(ctypes.c_uint8)
        L.oracle_plane.argtypes = [i32, i32, i32, i64, i64, i64, i64]
        L.oracle_plane.restype = i32
        L.oracle_attend_row.argtypes = [i32, i32, i32, i32, pd, pd, pd, pd, pd, i32, i32, i32, i32, pd, pd, pi]
        L.oracle_attend_row.restype = None
        L.oracle_attend_rows.argtypes = [i32, i32, i32, pi, pi, pi, pd, pd, pd, pd, pd, i32, i32, i32, pd, pd]
        L.oracle_attend_rows.restype = None
        L.oracle_split_partials.argtypes = [i32, i32, i32, i32, pd, pd, pd, pd, pd, i32, i32, i32, i32, i32, i32,
                                            pd, pd, pd]
        L.oracle_split_partials.restype = None
        L.oracle_lse_merge.argtypes = [i32, i32, pd, pd, pd, pd, pd]
        L.oracle_lse_merge.restype = None
        L.oracle_cell_row.argtypes = [i32, i32, i32, i32, i32, pd, pd, pd, pu8, pd, pd, pu8, pd, pd, dbl, pd, pd,
                                      pu8]
        L.oracle_cell_row.restype = i32
        L.oracle_cell_row_rule.argtypes = [i32, i32, i32, i32, i32, pd, pd, pd, pu8, pd, pd, pu8, pd, pd, i32, dbl,
                                           i32, pd, pd, pu8, pd]
        L.oracle_cell_row_rule.restype = i32
        L.oracle_kivi_encode.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                          pu8, ctypes.POINTER(ctypes.c_uint16), pu8, ctypes.POINTER(ctypes.c_uint16)]
        L.oracle_kivi_encode.restype = None
        L.oracle_f16_from_f32.argtypes = [ctypes.c_float]
        L.oracle_f16_from_f32.restype = ctypes.c_uint16
        L.oracle_f32_from_f16.argtypes = [ctypes.c_uint16]
        L.oracle_f32_from_f16.restype = ctypes.c_float
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = i32
        _LIB = L
    return _LIB


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _u8(a):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def threads() -> int:
    """OpenMP threads the row-parallel oracle routines run on."""
    return int(_lib().oracle_threads())


def set_threads(n: int) -> int:
    """Run the row-parallel routines on n threads from here on; returns the previous setting."""
    return int(_lib().oracle_set_threads(n))


def oracle_plane(policy: int, loop: int, n_loops: int, t: int, t0: int, j: int, window: int) -> int:
    return int(_lib().oracle_plane(policy, loop, n_loops, t, t0, j, window))


def plane_map(policy: int, loop: int, n_loops: int, t: int, t0: int, L: int, window: int) -> np.ndarray:
    """Plane read at each position 0..L-1 by the query at t (-1 beyond t)."""
    return np.array([oracle_plane(policy, loop, n_loops, t, t0, j, window) if j <= t else -1 for j in range(L)],
                    dtype=np.int32)


def attend_row(q, k_own, v_own, k_deep, v_deep, t: int, t0: int, policy: int, loop: int, n_loops: int,
               window: int, trace: bool = False):
    """Exact attention of one row.  k_*/v_* are [L][d]; returns (out[d], lse[, plane trace[L]])."""
    q, qp = _d(q)
    ko, kop = _d(k_own)
    vo, vop = _d(v_own)
    kd, kdp = _d(k_deep)
    vd, vdp = _d(v_deep)
    L, d = ko.shape
    out, outp = _d(np.zeros(d))
    lse, lsep = _d(np.zeros(1))
    tr, trp = _i(np.zeros(L, dtype=np.int32))
    _lib().oracle_attend_row(d, L, t, t0, qp, kop, vop, kdp, vdp, policy, loop, n_loops, window, outp, lsep,
                             trp if trace else None)
    if trace:
        return out, float(lse[0]), tr
    return out, float(lse[0])


def attend_rows(q, k_own, v_own, k_deep, v_deep, t, t0, loop, policy: int, n_loops: int, window: int):
    """Rows in parallel.  q [n][d]; k_*/v_* [n][L][d]; t, t0, loop [n].  Returns (out [n][d], lse [n])."""
    q, qp = _d(q)
    ko, kop = _d(k_own)
    vo, vop = _d(v_own)
    kd, kdp = _d(k_deep)
    vd, vdp = _d(v_deep)
    n, L, d = ko.shape
    ta, tp = _i(t)
    t0a, t0p = _i(t0)
    la, lp = _i(loop)
    out, outp = _d(np.zeros((n, d)))
    lse, lsep = _d(np.zeros(n))
    _lib().oracle_attend_rows(n, d, L, tp, t0p, lp, qp, kop, vop, kdp, vdp, policy, n_loops, window, outp, lsep)
    return out, lse


def split_partials(q, k_own, v_own, k_deep, v_deep, t, t0, policy, loop, n_loops, window, page, n_splits):
    q, qp = _d(q)
    ko, kop = _d(k_own)
    vo, vop = _d(v_own)
    kd, kdp = _d(k_deep)
    vd, vdp = _d(v_deep)
    L, d = ko.shape
    o, op = _d(np.zeros((n_splits, d)))
    m, mp = _d(np.zeros(n_splits))
    lsum, lp = _d(np.zeros(n_splits))
    _lib().oracle_split_partials(d, L, t, t0, qp, kop, vop, kdp, vdp, policy, loop, n_loops, window, page,
                                 n_splits, op, mp, lp)
    return o, m, lsum


def lse_merge(o_parts, m_parts, l_parts):
    o, op = _d(o_parts)
    m, mp = _d(m_parts)
    lsum, lp = _d(l_parts)
    n, d = o.shape
    out, outp = _d(np.zeros(d))
    lse, lsep = _d(np.zeros(1))
    _lib().oracle_lse_merge(n, d, op, mp, lp, outp, lsep)
    return out, float(lse[0])


def cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink: int, tail: int, kind: int,
             thr_offset: float = 4.0):
    """One LoopKV-style cell row.  k_near/v_near [L][d]; kc/vc [n_far][d] codes; ks/kz [n_groups][d];
    vs/vz [n_far][d/32].  Returns (out[d], lse, hot_bits[n_far], n_cold)."""
    q, qp = _d(q)
    kn, knp = _d(k_near)
    vn, vnp = _d(v_near)
    L, d = kn.shape
    n_far = L - sink - tail
    kca, kcp = _u8(kc)
    vca, vcp = _u8(vc)
    ksa, ksp = _d(ks)
    kza, kzp = _d(kz)
    vsa, vsp = _d(vs)
    vza, vzp = _d(vz)
    assert kca.shape == (n_far, d) and vca.shape == (n_far, d)
    assert ksa.shape[1] == d and ksa.shape[0] * 32 >= n_far and vsa.shape == (n_far, d // 32)
    out, outp = _d(np.zeros(d))
    lse, lsep = _d(np.zeros(1))
    hot, hotp = _u8(np.zeros(n_far, dtype=np.uint8))
    n_cold = _lib().oracle_cell_row(d, L, sink, tail, kind, qp, knp, vnp, kcp, ksp, kzp, vcp, vsp, vzp,
                                    float(thr_offset), outp, lsep, hotp)
    return out, float(lse[0]), hot, int(n_cold)


def kivi_encode(k, v, bits: int):
    """Window-exit codec of one far page of one head (LoopKV page, Sec. 3.1 and 3.3).  k, v: [n_tok][d]
    exact values (float32).  Returns (k_codes [n_tok][d] u8, k_meta [d][2] fp16 bits, v_codes [n_tok][d] u8,
    v_meta [n_tok][d/32][2] fp16 bits)."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    n, d = k.shape
    assert v.shape == (n, d) and d % 32 == 0 and 1 <= n
    kc = np.zeros((n, d), dtype=np.uint8)
    vc = np.zeros((n, d), dtype=np.uint8)
    km = np.zeros((d, 2), dtype=np.uint16)
    vm = np.zeros((n, d // 32, 2), dtype=np.uint16)
    pf = ctypes.POINTER(ctypes.c_float)
    p16 = ctypes.POINTER(ctypes.c_uint16)
    _lib().oracle_kivi_encode(n, d, bits, k.ctypes.data_as(pf), v.ctypes.data_as(pf), _u8(kc)[1],
                              km.ctypes.data_as(p16), _u8(vc)[1], vm.ctypes.data_as(p16))
    return kc, km, vc, vm


def f16_from_f32(x: float) -> int:
    return int(_lib().oracle_f16_from_f32(float(x)))


def f32_from_f16(h: int) -> float:
    return float(_lib().oracle_f32_from_f16(int(h)))


def cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink: int, tail: int, kind: int, tau: float,
                     n_splits: int):
    """One cell row under the LoopKV page's own V-precision rule (Sec. 3.3, App. E Algorithm 1): far block c of
    n_splits walks its 32-token pages in order with a running maximum m of its scores so far; a token is hot
    iff s >= max(m, m0) - tau ln 2.  Returns (out[d], lse, hot_bits[n_far], n_cold, thresholds[n_far])."""
    q, qp = _d(q)
    kn, knp = _d(k_near)
    vn, vnp = _d(v_near)
    L, d = kn.shape
    n_far = L - sink - tail
    kca, kcp = _u8(kc)
    vca, vcp = _u8(vc)
    ksa, ksp = _d(ks)
    kza, kzp = _d(kz)
    vsa, vsp = _d(vs)
    vza, vzp = _d(vz)
    out, outp = _d(np.zeros(d))
    lse, lsep = _d(np.zeros(1))
    hot, hotp = _u8(np.zeros(n_far, dtype=np.uint8))
    thr, thrp = _d(np.zeros(n_far))
    n_cold = _lib().oracle_cell_row_rule(d, L, sink, tail, kind, qp, knp, vnp, kcp, ksp, kzp, vcp, vsp, vzp, 1,
                                         float(tau) * math.log(2.0), int(n_splits), outp, lsep, hotp, thrp)
    return out, float(lse[0]), hot, int(n_cold), thr


# ----------------------------------------------------------------------------- closed-form models

def kv_bytes_per_layer_token(n_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """b = 2 * Hkv * dh elements per layer per token (keys and values), in bytes (RIPE page, Sec. 2)."""
    return 2 * n_kv_heads * head_dim * elem_bytes


def mem_full(L: int, b: int, n_pre: int, n_coda: int, n_core: int, n_loops: int) -> int:
    """M_full(L) = b L (n_pre + n_coda + R n_core) (RIPE page, Eq. (3))."""
    return b * L * (n_pre + n_coda + n_loops * n_core)


def mem_deep(L: int, b: int, n_pre: int, n_coda: int, n_core: int) -> int:
    """M_deep(L) = b L (n_pre + n_coda + n_core) (RIPE page, Eq. (3))."""
    return b * L * (n_pre + n_coda + n_core)


def mem_ripe(L: int, b: int, n_pre: int, n_coda: int, n_core: int, n_loops: int, window: int) -> int:
    """M_RIPE(L) = M_deep(L) + b n_core (R - 1) min(W, L) (RIPE page, Eq. (10))."""
    return mem_deep(L, b, n_pre, n_coda, n_core) + b * n_core * (n_loops - 1) * min(window, L)


def loopkv_bytes_per_token_layer(n_kv_heads: int, head_dim: int, bits: int, group: int = 32) -> float:
    """Stored bytes of one token in one layer and loop for K and V codes with one fp16 scale and one
    fp16 zero per group of `group` elements (LoopKV page, App. C): (bits + 32/group) bits per element."""
    elems = 2 * n_kv_heads * head_dim
    return elems * (bits + 32.0 / group) / 8.0
