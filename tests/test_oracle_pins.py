"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names the passage it checks.  Page names: "RIPE page" = "Prefix Keys
and Values Matter Late: RIPE Caching for Self-Speculative Decoding in Looped
Language Models"; "LoopKV page" = "LoopKV: Loop-Aware KV Cache Compression for
Serving Looped Transformers".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth


def _planes(rng, n_loops, L, d):
    k = rng.standard_normal((n_loops, L, d))
    v = rng.standard_normal((n_loops, L, d))
    return k, v


def _sdpa(q, k, v):
    """Textbook attention (torch, fp64, CPU): softmax(q k^T / sqrt(d)) v."""
    qt = torch.tensor(q, dtype=torch.float64).view(1, 1, 1, -1)
    kt = torch.tensor(np.ascontiguousarray(k), dtype=torch.float64).view(1, 1, k.shape[0], -1)
    vt = torch.tensor(np.ascontiguousarray(v), dtype=torch.float64).view(1, 1, v.shape[0], -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(-1).numpy()


# ----------------------------------------------------------------------------- index function

def test_plane_reads_match_worked_cases(golden_dir):
    """RIPE page, Sec. 4 Eq. (9), Alg. 1 and the proof of Prop. 1 (tests/golden/ripe_block_reads.json)."""
    g = json.load(open(os.path.join(golden_dir, "ripe_block_reads.json")))
    for case in g["cases"]:
        pol = oracle.RIPE if case["policy"] == "ripe" else oracle.FULL
        if "reads" in case:
            for t, want in case["reads"].items():
                t = int(t)
                got = [oracle.oracle_plane(pol, case["loop"], case["n_loops"], t, case["t0"], j, case["window"])
                       for j in range(t + 1)]
                assert got == want, (case["what"], t)
        for t, j_own in case.get("own_from", {}).items():
            t = int(t)
            got = [oracle.oracle_plane(pol, case["loop"], case["n_loops"], t, case["t0"], j, case["window"])
                   for j in range(t + 1)]
            assert all(p == case["n_loops"] - 1 for p in got[:j_own]), case["what"]
            assert all(p == case["loop"] for p in got[j_own:]), case["what"]


@pytest.mark.parametrize("k_block", [2, 3, 5])
def test_prop1_block_independence(k_block):
    """RIPE page, Prop. 1: if W >= gamma (block of gamma + 1 tokens), verifying the block in one pass
    equals decoding its tokens one at a time, and equals any split of the block into two passes."""
    rng = np.random.default_rng(1)
    R, L, d = 5, 20, 16
    k, v = _planes(rng, R, L, d)
    t0 = L - k_block
    gamma = k_block - 1
    for W in (gamma, gamma + 1, 64):
        for r in range(R):
            for i in range(k_block):
                t = t0 + i
                q = rng.standard_normal(d)
                batched, lb = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t0, oracle.RIPE, r, R, W)
                seq, ls = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t, oracle.RIPE, r, R, W)
                np.testing.assert_allclose(batched, seq, rtol=0, atol=1e-13)
                assert abs(lb - ls) < 1e-13
                for cut in range(1, k_block):
                    s0 = t0 + cut if i >= cut else t0
                    two, _ = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, s0, oracle.RIPE, r, R, W)
                    np.testing.assert_allclose(two, seq, rtol=0, atol=1e-13)


def test_prop1_fails_for_deepest_plane_cache():
    """RIPE page, Prop. 1 discussion: W = 0 violates the premise; the block reads plane r of earlier
    block tokens where sequential decoding reads plane R, so outputs depend on where blocks start."""
    rng = np.random.default_rng(2)
    R, L, d, kb = 4, 16, 8, 4
    k, v = _planes(rng, R, L, d)
    t0 = L - kb
    q = rng.standard_normal(d)
    r = 0
    t = t0 + kb - 1
    batched, _ = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t0, oracle.RIPE, r, R, 0)
    seq, _ = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t, oracle.RIPE, r, R, 0)
    assert np.max(np.abs(batched - seq)) > 1e-3


def test_window_covering_context_equals_full_cache():
    """A RIPE window covering the whole context reads every plane r, i.e. the full cache (RIPE page,
    Eq. (9) with t - j <= W for every j)."""
    rng = np.random.default_rng(3)
    R, L, d = 4, 33, 12
    k, v = _planes(rng, R, L, d)
    for r in range(R):
        q = rng.standard_normal(d)
        full, lf = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], L - 1, L - 1, oracle.FULL, r, R, 0)
        for W in (L - 1, L, 10 * L):
            ripe, lr = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], L - 1, L - 1, oracle.RIPE, r, R, W)
            assert np.array_equal(full, ripe) and lf == lr


@pytest.mark.parametrize("W", [0, 1, 5, 17])
def test_ripe_equals_full_cache_after_direct_substitution(W):
    """RIPE page, Sec. 2: a policy is checked against direct substitution.  RIPE(W) equals the full
    cache run on planes whose positions with t - j > W (j < t0) were overwritten by plane R; W = 0 is
    the deepest-plane cache (every cached position at plane R)."""
    rng = np.random.default_rng(4)
    R, L, d, kb = 4, 24, 8, 3
    k, v = _planes(rng, R, L, d)
    t0 = L - kb
    for r in range(R):
        for i in range(kb):
            t = t0 + i
            q = rng.standard_normal(d)
            ks, vs = k[r].copy(), v[r].copy()
            for j in range(t0):
                if t - j > W:
                    ks[j], vs[j] = k[R - 1][j], v[R - 1][j]
            ripe, _ = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t0, oracle.RIPE, r, R, W)
            sub, _ = oracle.attend_row(q, ks, vs, ks, vs, t, t0, oracle.FULL, r, R, 0)
            np.testing.assert_allclose(ripe, sub, rtol=0, atol=1e-14)


def test_attention_matches_textbook_routine():
    """The exact-softmax definition vs torch's fp64 scaled_dot_product_attention on the materialised,
    causally truncated view (scale 1/sqrt(d))."""
    rng = np.random.default_rng(5)
    R, L, d = 3, 40, 24
    k, v = _planes(rng, R, L, d)
    for W in (0, 7):
        for t in (0, 5, L - 1):
            r = 1
            q = rng.standard_normal(d)
            t0 = t
            pm = oracle.plane_map(oracle.RIPE, r, R, t, t0, L, W)
            kv_k = np.stack([k[pm[j]][j] for j in range(t + 1)])
            kv_v = np.stack([v[pm[j]][j] for j in range(t + 1)])
            out, lse = oracle.attend_row(q, k[r], v[r], k[R - 1], v[R - 1], t, t0, oracle.RIPE, r, R, W)
            np.testing.assert_allclose(out, _sdpa(q, kv_k, kv_v), rtol=0, atol=1e-12)
            s = kv_k @ q / math.sqrt(d)
            assert abs(lse - (s.max() + math.log(np.exp(s - s.max()).sum()))) < 1e-12


def test_closed_forms():
    """q = 0 gives the mean of the visible values with lse = ln(t+1); one key far above the rest gives its
    value; a one-position cache gives v_0 and lse = s_0."""
    rng = np.random.default_rng(6)
    R, L, d = 2, 10, 8
    k, v = _planes(rng, R, L, d)
    out, lse = oracle.attend_row(np.zeros(d), k[0], v[0], k[1], v[1], 6, 6, oracle.FULL, 0, R, 0)
    np.testing.assert_allclose(out, v[0][:7].mean(axis=0), atol=1e-14)
    assert abs(lse - math.log(7)) < 1e-14
    q = rng.standard_normal(d)
    kd = k[0].copy()
    kd[3] = q * (80.0 * math.sqrt(d) / (q @ q))
    out, _ = oracle.attend_row(q, kd, v[0], kd, v[0], L - 1, L - 1, oracle.FULL, 0, R, 0)
    np.testing.assert_allclose(out, v[0][3], atol=1e-12)
    out, lse = oracle.attend_row(q, k[0][:1], v[0][:1], k[1][:1], v[1][:1], 0, 0, oracle.RIPE, 0, R, 0)
    np.testing.assert_allclose(out, v[0][0], atol=0)
    assert abs(lse - q @ k[0][0] / math.sqrt(d)) < 1e-14


# ----------------------------------------------------------------------------- split-K and merge

@pytest.mark.parametrize("n_splits", [1, 2, 3, 8, 13])
def test_split_partials_merge_to_unsplit(n_splits):
    """LoopKV page, Sec. 3.4 / App. E Alg. 1: partials merged by log-sum-exp give the exact softmax."""
    rng = np.random.default_rng(7)
    R, L, d, P = 4, 45, 16, 4
    k, v = _planes(rng, R, L, d)
    for W in (0, 9):
        for t in (0, 3, 21, L - 1):
            q = rng.standard_normal(d) * 2
            full, lf = oracle.attend_row(q, k[2], v[2], k[R - 1], v[R - 1], t, t, oracle.RIPE, 2, R, W)
            o, m, lsum = oracle.split_partials(q, k[2], v[2], k[R - 1], v[R - 1], t, t, oracle.RIPE, 2, R, W, P,
                                               n_splits)
            n_pages = (t + P) // P
            empty = [c for c in range(n_splits) if (c * n_pages) // n_splits == ((c + 1) * n_pages) // n_splits]
            for c in empty:
                assert m[c] == -math.inf and lsum[c] == 0 and not o[c].any()
            merged, lm = oracle.lse_merge(o, m, lsum)
            np.testing.assert_allclose(merged, full, rtol=0, atol=1e-12 * max(1.0, np.abs(v).max()))
            assert abs(lm - lf) < 1e-12


def test_merge_is_order_independent_and_single_partial_is_identity():
    rng = np.random.default_rng(8)
    d = 6
    o = rng.standard_normal((5, d))
    m = rng.standard_normal(5) * 3
    lsum = rng.uniform(0.5, 4.0, 5)
    a, la = oracle.lse_merge(o, m, lsum)
    perm = rng.permutation(5)
    b, lb = oracle.lse_merge(o[perm], m[perm], lsum[perm])
    np.testing.assert_allclose(a, b, atol=1e-14)
    assert abs(la - lb) < 1e-13
    one, l1 = oracle.lse_merge(o[:1], m[:1], lsum[:1])
    np.testing.assert_allclose(one, o[0], atol=1e-15)
    assert abs(l1 - (m[0] + math.log(lsum[0]))) < 1e-14


# ----------------------------------------------------------------------------- quantised cells

def _cell_inputs(rng, L, d, sink, tail, bits):
    n_far = L - sink - tail
    n_grp = (n_far + 31) // 32
    hi = (1 << bits) - 1
    kc = rng.integers(0, hi + 1, (n_far, d)).astype(np.uint8)
    vc = rng.integers(0, hi + 1, (n_far, d)).astype(np.uint8)
    ks = rng.uniform(0.2, 0.4, (n_grp, d))
    kz = rng.uniform(-3.0, -2.0, (n_grp, d))
    vs = rng.uniform(0.2, 0.4, (n_far, d // 32))
    vz = rng.uniform(-3.0, -2.0, (n_far, d // 32))
    k_near = rng.standard_normal((L, d))
    v_near = rng.standard_normal((L, d))
    return k_near, v_near, kc, ks, kz, vc, vs, vz


def _dequant(kc, ks, kz, vc, vs, vz, chat_v):
    n_far, d = kc.shape
    g = np.arange(n_far) // 32
    kh = kz[g] + ks[g] * kc
    grp = np.arange(d) // 32
    vh = vz[:, grp] + vs[:, grp] * chat_v
    return kh, vh


def _view(k_near, v_near, kh, vh, sink, tail):
    L = k_near.shape[0]
    kk = np.concatenate([k_near[:sink], kh, k_near[L - tail:]])
    vv = np.concatenate([v_near[:sink], vh, v_near[L - tail:]])
    return kk, vv


@pytest.mark.parametrize("kind,bits", [(oracle.CELL_INT4, 4), (oracle.CELL_SHARED, 4), (oracle.CELL_INT2, 2)])
def test_cell_all_hot_is_attention_over_dequantised_codes(kind, bits):
    """LoopKV page, Sec. 3.1 and App. E proof of Prop. 1 (a decoded value is z + sigma c): with the threshold
    at -inf every far token is hot, and the cell is exact attention over sink, dequantised far and tail."""
    rng = np.random.default_rng(9)
    L, d, sink, tail = 150, 64, 4, 16
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, bits)
    q = rng.standard_normal(d)
    out, lse, hot, n_cold = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, kind,
                                            thr_offset=math.inf)
    assert hot.all() and n_cold == 0
    kh, vh = _dequant(kc, ks, kz, vc, vs, vz, vc.astype(np.float64))
    kk, vv = _view(k_near, v_near, kh, vh, sink, tail)
    np.testing.assert_allclose(out, _sdpa(q, kk, vv), rtol=0, atol=1e-12)


def test_cell_all_cold_reads_bucket_midpoints():
    """LoopKV page, Sec. 3.3: a cold token reads only the hi plane and decodes to 4*hi + 1.5."""
    rng = np.random.default_rng(10)
    L, d, sink, tail = 140, 64, 4, 8
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, 4)
    q = rng.standard_normal(d)
    out, _, hot, n_cold = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                          oracle.CELL_INT4, thr_offset=-math.inf)
    assert not hot.any() and n_cold == L - sink - tail
    kh, vh = _dequant(kc, ks, kz, vc, vs, vz, 4.0 * (vc >> 2) + 1.5)
    kk, vv = _view(k_near, v_near, kh, vh, sink, tail)
    np.testing.assert_allclose(out, _sdpa(q, kk, vv), rtol=0, atol=1e-12)


@pytest.mark.parametrize("offset", [0.5, 2.0, 4.0])
def test_cell_hot_rule_error_bound(offset):
    """LoopKV page, Prop. 1: relative to the reader of both planes, the output moves by at most
    1.5 * sum_{j cold} a_j sigma_j <= 1.5 sigma_max |C| 2^-tau a_max (here the fixed rule's e^-offset takes
    the place of 2^-tau), since m0 never exceeds the row maximum.  Cold tokens have a_j < e^-offset a_max."""
    rng = np.random.default_rng(11)
    L, d, sink, tail = 300, 64, 4, 16
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, 4)
    q = rng.standard_normal(d) * 1.5
    k_near[:sink] += q * 0.1  # raise the sink scores so that some far tokens fall below the threshold
    out, lse, hot, n_cold = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                            oracle.CELL_INT4, thr_offset=offset)
    ref, lref, _, _ = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, oracle.CELL_INT4,
                                      thr_offset=math.inf)
    assert 0 < n_cold < L - sink - tail
    assert abs(lse - lref) < 1e-12  # scores, hence weights, are those of the full INT4 reader
    kh, _ = _dequant(kc, ks, kz, vc, vs, vz, vc.astype(np.float64))
    s = np.concatenate([k_near[:sink], kh, k_near[L - tail:]]) @ q / math.sqrt(d)
    a = np.exp(s - s.max())
    a /= a.sum()
    cold = np.where(hot == 0)[0]
    a_far = a[sink:L - tail]
    grp = np.arange(d) // 32
    bound_c = 1.5 * (a_far[cold, None] * vs[cold][:, grp]).sum(axis=0)
    assert np.all(np.abs(out - ref) <= bound_c + 1e-13)
    assert np.all(a_far[cold] < math.exp(-offset) * a.max())
    assert np.abs(out - ref).max() <= 1.5 * vs.max() * len(cold) * math.exp(-offset) * a.max() + 1e-13


def test_cell_midpoint_bound():
    """LoopKV page, App. E: |c - (4 floor(c/4) + 1.5)| <= 1.5 for every 4-bit code c."""
    c = np.arange(16)
    assert np.abs(c - (4 * (c // 4) + 1.5)).max() == 1.5


def test_cell_seed_is_a_lower_bound_of_the_row_max():
    """LoopKV page, Sec. 3.3 footnote: the seed m0 is the largest sink score and never exceeds the row
    maximum, so tokens with s_j >= max(s) - offset are always hot."""
    rng = np.random.default_rng(12)
    L, d, sink, tail = 200, 64, 4, 8
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, 4)
    q = rng.standard_normal(d)
    _, _, hot, _ = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, oracle.CELL_INT4, 1.0)
    kh, _ = _dequant(kc, ks, kz, vc, vs, vz, vc.astype(np.float64))
    s_far = kh @ q / math.sqrt(d)
    s_all = np.concatenate([k_near[:sink] @ q, kh @ q, k_near[L - tail:] @ q]) / math.sqrt(d)
    assert np.all(hot[s_far >= s_all.max() - 1.0] == 1)


# ----------------------------------------------------------------------------- closed-form models

def test_memory_model_reproduces_table2(golden_dir):
    """RIPE page, Eq. (3), Eq. (10) and Table 2 (MB = 1e6 bytes, bf16)."""
    g = json.load(open(os.path.join(golden_dir, "ripe_table2.json")))
    L = g["L"]
    for name, m in g["models"].items():
        b = oracle.kv_bytes_per_layer_token(m["n_kv_heads"], m["head_dim"])
        args = (m["n_pre"], m["n_coda"], m["n_core"])
        full = oracle.mem_full(L, b, *args, m["n_loops"])
        deep = oracle.mem_deep(L, b, *args)
        two = b * L * (m["n_pre"] + m["n_coda"] + 2 * m["n_core"])
        got = {"full": full, "deepest": deep, "two_planes": two}
        for W in (16, 64, 256):
            got[f"ripe_w{W}"] = oracle.mem_ripe(L, b, *args, m["n_loops"], W)
        for key, mb in m["MB"].items():
            assert round(got[key] / 1e6) == mb, (name, key, got[key])
            assert round(100.0 * got[key] / full, 1) == m["percent"][key], (name, key)
        kb_full = b * (m["n_pre"] + m["n_coda"] + m["n_loops"] * m["n_core"]) / 1e3
        kb_deep = b * (m["n_pre"] + m["n_coda"] + m["n_core"]) / 1e3
        assert abs(kb_full - m["KB_per_token"]["full"]) < 0.5
        assert abs(kb_deep - m["KB_per_token"]["deepest"]) < 0.5


def test_loopkv_byte_model(golden_dir):
    """LoopKV page, App. C and Sec. 3.1/3.3."""
    g = json.load(open(os.path.join(golden_dir, "loopkv_byte_model.json")))
    o = g["ouro"]
    h, d = o["n_kv_heads"], o["head_dim"]
    kib = g["KiB_per_token_layer"]
    assert oracle.loopkv_bytes_per_token_layer(h, d, 4) / 1024 == kib["int4"]
    assert oracle.loopkv_bytes_per_token_layer(h, d, 2) / 1024 == kib["int2"]
    assert oracle.kv_bytes_per_layer_token(h, d) / 1024 == kib["bf16"]
    cells = o["n_layers"] * o["n_loops"]
    assert cells * oracle.loopkv_bytes_per_token_layer(h, d, 4) / 1024 == g["KiB_per_token_all_cells"]["int4"]
    assert cells * oracle.kv_bytes_per_layer_token(h, d) / 1024 == g["KiB_per_token_all_cells"]["bf16"]
    assert h * d * 2 / 8 / 1024 == g["lo_plane_KiB_per_token_layer"]
    sw = g["sink_window_tokens"] * cells * oracle.kv_bytes_per_layer_token(h, d) / 2 ** 20
    assert sw == g["sink_window_MiB_per_request_step"]


# ----------------------------------------------------------------------------- brute force

def _brute_force_row(q, view_k, view_v):
    d = len(q)
    s = [math.fsum(q[c] * kk[c] for c in range(d)) / math.sqrt(d) for kk in view_k]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    lsum = math.fsum(e)
    return [math.fsum(e[j] * view_v[j][c] for j in range(len(e))) / lsum for c in range(d)]


def test_bruteforce_on_tiny_workload():
    """The whole Tiny workload (fp32, 1 layer, 4 loops, 2 heads x 64, L=128, q=1, seed 0) by dense
    brute force with math.fsum over the directly substituted view, for the full cache and RIPE W in
    {0, 16, 128}."""
    w = synth.WORKLOADS["tiny"]
    R, H, d, L = w.n_loops, w.n_heads, w.head_dim, w.length
    planes_k = [synth.kv(synth.DT_F32, 0, synth.T_K, 0, 0, r, H, d, 0, L, scale=w.scale).astype(np.float64)
                for r in range(R)]
    planes_v = [synth.kv(synth.DT_F32, 0, synth.T_V, 0, 0, r, H, d, 0, L, scale=w.scale).astype(np.float64)
                for r in range(R)]
    t = L - 1
    for pol, W in ((oracle.FULL, 0), (oracle.RIPE, 0), (oracle.RIPE, 16), (oracle.RIPE, 128)):
        for r in range(R):
            qv = synth.q(synth.DT_F32, 0, [0], [t], 0, r, 1, H, d, scale=w.scale).astype(np.float64)
            for h in range(H):
                # direct substitution: plane R where the policy drops plane r (full cache keeps all)
                vk = [planes_k[r][j, h] if (pol == oracle.FULL or t - j <= W) else planes_k[R - 1][j, h]
                      for j in range(L)]
                vv = [planes_v[r][j, h] if (pol == oracle.FULL or t - j <= W) else planes_v[R - 1][j, h]
                      for j in range(L)]
                bf = _brute_force_row(qv[0, 0, h], vk, vv)
                out, _ = oracle.attend_row(qv[0, 0, h], planes_k[r][:, h], planes_v[r][:, h],
                                           planes_k[R - 1][:, h], planes_v[R - 1][:, h], t, t, pol, r, R, W)
                np.testing.assert_allclose(out, bf, rtol=0, atol=1e-15)


def test_cell_hot_rule_closed_form():
    """LoopKV page, Sec. 3.3 (a token is cold when its score falls below the threshold; Alg. 1 in App. E
    tests s_j >= threshold, so a tie is hot) with the fixed seed rule s_j >= m0 - 4.0.  With q = sqrt(d) e_0
    the score is the key's channel 0; the sink's channel 0 is 3.0, so m0 = 3 and far token j is hot exactly
    when z + sigma * c_j >= -1, i.e. c_j >= 4 for z = -2, sigma = 1/4 (all values exact in binary)."""
    d, sink, tail, L = 32, 4, 4, 4 + 64 + 4
    q = np.zeros(d)
    q[0] = math.sqrt(d)
    k_near = np.zeros((L, d))
    k_near[:sink, 0] = [3.0, -5.0, 0.5, 2.75]
    v_near = np.zeros((L, d))
    n_far = L - sink - tail
    kc = np.zeros((n_far, d), dtype=np.uint8)
    kc[:, 0] = np.arange(n_far) % 16
    ks = np.full((2, d), 0.25)
    kz = np.full((2, d), -2.0)
    vc = np.zeros((n_far, d), dtype=np.uint8)
    vs = np.full((n_far, 1), 0.25)
    vz = np.zeros((n_far, 1))
    _, _, hot, n_cold = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, oracle.CELL_INT4, 4.0)
    np.testing.assert_array_equal(hot, (kc[:, 0] >= 4).astype(np.uint8))
    assert n_cold == int((kc[:, 0] < 4).sum())


# ----------------------------------------------------------------------------- the running-maximum V-precision rule

def test_running_rule_worked_case():
    """LoopKV page, Sec. 3.3 and App. E Algorithm 1: a far block's running maximum m covers its pages so far and a
    token is hot iff s >= max(m, m0) - tau ln 2.  With q = sqrt(d) e_0 a score is the key's channel 0.  One far
    token scores 20 (code 10 at scale 2), every other far token 0, the sink maximum m0 is 5, tau = 14
    (tau ln 2 = 9.70).  With two far blocks the first block's later tokens fall below 20 - 9.70 and are cold, the
    second block never sees the 20 and keeps all its tokens hot (0 >= 5 - 9.70); with one block every token after
    the 20 is cold."""
    d, sink, tail = 32, 4, 4
    n_far = 128
    L = sink + n_far + tail
    q = np.zeros(d)
    q[0] = math.sqrt(d)
    k_near = np.zeros((L, d))
    k_near[:sink, 0] = [5.0, 1.0, 1.0, 1.0]
    v_near = np.zeros((L, d))
    kc = np.zeros((n_far, d), dtype=np.uint8)
    kc[0, 0] = 10
    ks = np.full((4, d), 2.0)
    kz = np.zeros((4, d))
    vc = np.zeros((n_far, d), dtype=np.uint8)
    vs = np.full((n_far, 1), 0.25)
    vz = np.zeros((n_far, 1))
    _, _, hot2, cold2, _ = oracle.cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                                   oracle.CELL_INT4, 14.0, 2)
    want2 = np.zeros(n_far, np.uint8)
    want2[0] = 1
    want2[64:] = 1
    np.testing.assert_array_equal(hot2, want2)
    assert cold2 == 63
    _, _, hot1, cold1, _ = oracle.cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                                   oracle.CELL_INT4, 14.0, 1)
    want1 = np.zeros(n_far, np.uint8)
    want1[0] = 1
    np.testing.assert_array_equal(hot1, want1)
    assert cold1 == n_far - 1


@pytest.mark.parametrize("n_splits", [1, 3, 8])
def test_running_rule_bounds(n_splits):
    """The running maximum never exceeds the row maximum (LoopKV page, footnote 9 and Prop. 1): cold tokens lie
    below s_max - tau ln 2, tokens at or above it are hot, and the output is within
    1.5 * sum_{cold} a_j sigma_j <= 1.5 sigma_max |C| 2^-tau a_max of the reader of both planes."""
    rng = np.random.default_rng(20 + n_splits)
    L, d, sink, tail = 900, 64, 4, 16
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, 4)
    q = rng.standard_normal(d) * 3.0
    for tau in (2.0, 5.0, 14.0):
        out, lse, hot, n_cold, thr = oracle.cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                                             oracle.CELL_INT4, tau, n_splits)
        ref, lref, _, _ = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, oracle.CELL_INT4,
                                          thr_offset=math.inf)
        assert abs(lse - lref) < 1e-12
        kh, _ = _dequant(kc, ks, kz, vc, vs, vz, vc.astype(np.float64))
        s = np.concatenate([k_near[:sink], kh, k_near[L - tail:]]) @ q / math.sqrt(d)
        s_far = s[sink:L - tail]
        smax = s.max()
        cold = hot == 0
        assert np.all(s_far[cold] < smax - tau * math.log(2))
        assert np.all(hot[s_far >= smax - tau * math.log(2)] == 1)
        a = np.exp(s - smax)
        a /= a.sum()
        grp = np.arange(d) // 32
        bound_c = 1.5 * (a[sink:L - tail][cold, None] * vs[cold][:, grp]).sum(axis=0)
        assert np.all(np.abs(out - ref) <= bound_c + 1e-13)
        assert np.abs(out - ref).max() <= 1.5 * vs.max() * cold.sum() * 2.0 ** -tau * a.max() + 1e-13
        if tau == 2.0:
            assert 0 < n_cold < L - sink - tail


def test_running_rule_with_dominant_seed_is_the_fixed_rule():
    """If the sink maximum m0 is at least every far score, max(m, m0) = m0 throughout and the running rule is the
    fixed rule s >= m0 - tau ln 2; at tau = infinity every token is hot and the row is the reader of both planes."""
    rng = np.random.default_rng(31)
    L, d, sink, tail = 600, 64, 4, 16
    k_near, v_near, kc, ks, kz, vc, vs, vz = _cell_inputs(rng, L, d, sink, tail, 4)
    q = rng.standard_normal(d)
    k_near[0] = q * (60.0 * math.sqrt(d) / (q @ q))  # sink score 60, above every far score
    for tau in (3.0, 6.0):
        _, _, hot_r, _, _ = oracle.cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                                    oracle.CELL_INT4, tau, 4)
        _, _, hot_f, _ = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail, oracle.CELL_INT4,
                                         thr_offset=tau * math.log(2))
        np.testing.assert_array_equal(hot_r, hot_f)
    out, _, hot, n_cold, _ = oracle.cell_row_running(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                                     oracle.CELL_INT4, math.inf, 4)
    assert hot.all() and n_cold == 0
    kh, vh = _dequant(kc, ks, kz, vc, vs, vz, vc.astype(np.float64))
    kk, vv = _view(k_near, v_near, kh, vh, sink, tail)
    np.testing.assert_allclose(out, _sdpa(q, kk, vv), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- the row-parallel routine

@pytest.mark.parametrize("policy", [oracle.FULL, oracle.RIPE])
def test_attend_rows_equals_attend_row_bitwise(policy):
    """The OpenMP row routine (the one the CPU baseline times) is the single-row definition (RIPE page,
    Sec. 2 policy pi and Eq. (9)) applied row by row: identical bits for rows of mixed query position,
    block start, loop and window, including W = 0 (the deepest-plane cache) and W >= L (the full cache)."""
    rng = np.random.default_rng(41)
    R, L, d = 4, 70, 32
    n = 12
    q = rng.standard_normal((n, d))
    ko, vo, kd, vd = (rng.standard_normal((n, L, d)) for _ in range(4))
    t = rng.integers(L // 2, L, n).astype(np.int32)
    t0 = np.array([rng.integers(max(0, ti - 7), ti + 1) for ti in t], dtype=np.int32)
    loops = rng.integers(0, R, n).astype(np.int32)
    for W in (0, 7, L + 3):
        out, lse = oracle.attend_rows(q, ko, vo, kd, vd, t, t0, loops, policy, R, W)
        for i in range(n):
            o1, l1 = oracle.attend_row(q[i], ko[i], vo[i], kd[i], vd[i], int(t[i]), int(t0[i]), policy,
                                       int(loops[i]), R, W)
            assert np.array_equal(out[i], o1), (W, i)
            assert lse[i] == l1, (W, i)
    # and on one thread (the one-core figure) the same bits again
    prev = oracle.set_threads(1)
    try:
        out1, lse1 = oracle.attend_rows(q, ko, vo, kd, vd, t, t0, loops, policy, R, 7)
    finally:
        oracle.set_threads(prev)
    out7, lse7 = oracle.attend_rows(q, ko, vo, kd, vd, t, t0, loops, policy, R, 7)
    assert np.array_equal(out1, out7) and np.array_equal(lse1, lse7)


# ----------------------------------------------------------------------------- cell groups against exact values

def _bf16_round(x):
    """Round fp64 values to the nearest bf16 (ties to even), returned as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("bits", [4, 2])
def test_cell_over_codec_codes_stays_within_the_codec_error_of_exact_attention(bits):
    """LoopKV page, Sec. 3.1 (KIVI groups of 32: keys per channel over a page's 32 tokens, values per token
    over 32 channels) and Sec. 3.4 (a page holds 32 tokens of one cell; far pages start after the sink).
    Exact keys and values are encoded page by page from the far start with the codec, and the cell routine
    reads the codes with every far token hot.  Position j's value is the unit vector e_j, so output channel j
    is the softmax weight the routine gave position j, and each weight must lie within the codec's error of
    the exact attention weight: e^(+-2 delta) (1 +- eps_v) times it, with delta the largest score error the
    codec's key error allows.  Each far page's keys carry their own offset along q, so a grouping counted
    from another origin (e.g. position 0 instead of the far start) would dequantise the tokens at a page edge
    with a neighbour page's zero, move their scores by several units and break the bound."""
    rng = np.random.default_rng(77)
    d, sink, tail = 128, 4, 4
    n_far = 3 * 32 + 11  # three whole pages and a partial last one
    L = sink + n_far + tail
    assert L <= d
    k = rng.standard_normal((L, d)) * 0.5
    for p in range((n_far + 31) // 32):
        k[sink + 32 * p: sink + 32 * p + 32] += 1.5 * (p + 1) * (-1) ** p  # per-page offsets
    v = np.zeros((L, d))
    v[np.arange(L), np.arange(L)] = 1.0
    k = _bf16_round(k).astype(np.float64)
    q = np.full(d, 0.1)
    n_pg = (n_far + 31) // 32
    kc = np.zeros((n_far, d), np.uint8)
    vc = np.zeros((n_far, d), np.uint8)
    ks, kz = np.zeros((n_pg, d)), np.zeros((n_pg, d))
    vs, vz = np.zeros((n_far, d // 32)), np.zeros((n_far, d // 32))
    f16 = np.vectorize(oracle.f32_from_f16)
    for p in range(n_pg):
        f0, f1 = 32 * p, min(n_far, 32 * p + 32)
        a, b = sink + f0, sink + f1
        c_k, m_k, c_v, m_v = oracle.kivi_encode(k[a:b].astype(np.float32), v[a:b].astype(np.float32), bits)
        kc[f0:f1], vc[f0:f1] = c_k, c_v
        ks[p], kz[p] = f16(m_k[:, 0]), f16(m_k[:, 1])
        vs[f0:f1], vz[f0:f1] = f16(m_v[..., 0]), f16(m_v[..., 1])
    kind = oracle.CELL_INT2 if bits == 2 else oracle.CELL_INT4
    out, lse, hot, n_cold = oracle.cell_row(q, k, v, kc, ks, kz, vc, vs, vz, sink, tail, kind, thr_offset=math.inf)
    assert hot.all() and n_cold == 0
    s = k @ q / math.sqrt(d)
    w_exact = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    # codec error per element: half a step, plus the fp16 rounding of the group's zero and of its step
    # (x_hat = z16 + s16 c, c clamped to [0, 2^b - 1])
    levels = (1 << bits) - 1
    eps_k = 0.0
    for p in range(n_pg):
        grp = k[sink + 32 * p: sink + min(n_far, 32 * p + 32)]
        mn, mx = grp.min(0), grp.max(0)
        eps_k = max(eps_k, (ks[p] / 2 + np.abs(kz[p] - mn) + levels * np.abs(ks[p] - (mx - mn) / levels)).max())
    vg = v[sink:sink + n_far].reshape(n_far, d // 32, 32)
    mnv, mxv = vg.min(2), vg.max(2)
    eps_v = (vs / 2 + np.abs(vz - mnv) + levels * np.abs(vs - (mxv - mnv) / levels)).max()
    delta = np.abs(q).sum() * eps_k / math.sqrt(d)
    ratio = out[:L] / w_exact
    lo, hi = (1 - eps_v) * math.exp(-2 * delta), (1 + eps_v) * math.exp(2 * delta)
    assert ((ratio >= lo) & (ratio <= hi)).all(), (ratio.min(), ratio.max(), lo, hi)
    assert np.abs(out[L:]).max() == 0.0
    # a misplaced group moves a page-edge token's score by at least 4.5 * 12.8 / sqrt(128) = 5.1 (the offsets
    # of neighbouring pages differ by >= 4.5 along q), a weight ratio of e^(+-5.1): outside the bound
    assert math.log(hi) < 3.0 and math.log(lo) > -3.0


def test_cell_groups_start_at_the_far_start_worked_case():
    """A hand-computed cell whose two far groups have different zeros (LoopKV page, Sec. 3.1 groups of 32
    counted from the far start, Sec. 3.3 fixed hot rule and bucket midpoint).  sink 4, far 40, tail 1, d 32;
    q = sqrt(d) e_0.  Every far key code is 1 on channel 0 with scale 1: group 0 (far tokens 0..31) has zero -10
    and decodes to k_0 = -9, score -9 (cold: below m0 - 4 = -4, with m0 = 0 from zero sink keys); group 1 (far
    tokens 32..39) has zero 0, decodes to k_0 = 1, score 1 (hot).  A grouping shifted by the sink would give far
    tokens 28..31 group 1's metadata and make them hot.  Every V code is 5 (hi 1, lo 1) with scale 1 and zero
    0: hot tokens decode to 5, cold ones to 4 + 1.5 = 5.5; sink and tail values are 0 and the tail key is 0.
    So out_c = (32 e^-9 5.5 + 8 e^1 5) / (4 + 1 + 32 e^-9 + 8 e) in every channel."""
    d, sink, tail, n_far = 32, 4, 1, 40
    L = sink + n_far + tail
    q = np.zeros(d)
    q[0] = math.sqrt(d)
    k_near = np.zeros((L, d))
    v_near = np.zeros((L, d))
    kc = np.zeros((n_far, d), np.uint8)
    kc[:, 0] = 1
    ks = np.ones((2, d))
    kz = np.zeros((2, d))
    kz[0, 0] = -10.0
    vc = np.full((n_far, d), 5, np.uint8)
    vs = np.ones((n_far, 1))
    vz = np.zeros((n_far, 1))
    out, lse, hot, n_cold = oracle.cell_row(q, k_near, v_near, kc, ks, kz, vc, vs, vz, sink, tail,
                                            oracle.CELL_INT4, thr_offset=4.0)
    assert hot.tolist() == [0] * 32 + [1] * 8 and n_cold == 32
    den = 4 + 1 + 32 * math.exp(-9) + 8 * math.e
    want = (32 * math.exp(-9) * 5.5 + 8 * math.e * 5) / den
    np.testing.assert_allclose(out, np.full(d, want), rtol=0, atol=1e-13)
    assert abs(lse - (1.0 + math.log(den / math.e))) < 1e-13
