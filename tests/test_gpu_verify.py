"""GPU parity of q = k self-speculative verification (MFMA tile, causal inside the block)
and of the q = 1 draft step, through the C-ABI, against the fp64 oracle."""
import numpy as np
import pytest

import harness
import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _verify(built, layer, loop, q, split_k=0, window=-1, trace_len=0):
    n, k = q.shape[0], q.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty((n, k, built.w.n_heads), dtype=torch.float32, device="cuda")
    ws_bytes = built.cache.lkv_workspace_bytes(layer, loop, built.seqs, q_len=k, mode=vla.MODE_VERIFY,
                                               split_k=split_k)
    ws = torch.empty(max(4, ws_bytes), dtype=torch.uint8, device="cuda")
    tr = torch.empty((n, k, trace_len, 2), dtype=torch.int32, device="cuda") if trace_len else None
    built.cache.lkv_attend(layer, loop, built.seqs, q, out, q_len=k, mode=vla.MODE_VERIFY, split_k=split_k,
                           lse=lse, workspace=ws, window=window, index_trace=tr, trace_len=trace_len)
    torch.cuda.synchronize()
    return out, lse, tr


def _wl(D, dt=synth.DT_BF16, scale=1.0, R=5, H=3):
    return synth.Workload("verify", 4, 2, R, H, D, 300, dt, "ripe", 20, 8, 16, synth.MODE_RIPEN, scale)


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 0), (vla.POLICY_RIPE, 7),
                                      (vla.POLICY_RIPE, 20)])
def test_verify_bf16_every_row(D, policy, W):
    """Blocks of k = 8 at ragged lengths (block inside the first page, across a page edge, long context),
    shuffled NaN-poisoned pages; every query row of every head vs the oracle, and the exact trace."""
    w = _wl(D)
    lengths = [8, 21, 100, 300]
    k = 8
    built = harness.build_plain(w, lengths=lengths, policy=policy, window=W, q_len=k, shuffle=True, poison=True)
    rows = [(b, i, h) for b in range(len(lengths)) for i in range(k) for h in range(w.n_heads)]
    for loop in (0, w.n_loops - 1):
        q = harness.gpu_queries(built, 0, loop, k)
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, lengths, k, policy, W)
        for split_k in (1, 3):
            out, lse, tr = _verify(built, 0, loop, q, split_k, trace_len=300)
            o = harness.out_f64(out)
            got = np.array([o[b, i, h] for (b, i, h) in rows])
            assert np.isfinite(got).all()
            assert np.abs(got - want).max() <= TOL_BF16, (loop, split_k)
            gl = lse.cpu().numpy()
            assert np.abs(np.array([gl[b, i, h] for (b, i, h) in rows]) - want_lse).max() <= 1e-2
            t = tr.cpu().numpy()
            for b, L in enumerate(lengths):
                for i in range(k):
                    pm = oracle.plane_map(policy, loop, w.n_loops, L - k + i, L - k, 300, W)
                    np.testing.assert_array_equal(t[b, i, :, 0], pm)
    built.cache.close()


@pytest.mark.parametrize("W", [7, 8, 40])
def test_prop1_verify_equals_sequential_decode_fp32(W):
    """RIPE page, Prop. 1 on the GPU: with W >= gamma = k - 1, one verify pass over a block of k equals k
    sequential q = 1 decodes of the same tokens (fp32 cache, within 1e-5)."""
    w = _wl(64, synth.DT_F32, 0.25)
    k, L = 8, 150
    t0 = L - k
    ver = harness.build_plain(w, lengths=[L], policy=vla.POLICY_RIPE, window=W, q_len=k, rows=[0])
    seq = harness.build_plain(w, lengths=[t0 + 1 + i for i in range(k)], policy=vla.POLICY_RIPE, window=W,
                              q_len=1, rows=[0] * k, max_len=L)
    for loop in (0, 2, 4):
        qv = harness.gpu_queries(ver, 0, loop, k)
        ov = harness.out_f64(_verify(ver, 0, loop, qv)[0])[0]
        qs = harness.gpu_queries(seq, 0, loop, 1)
        out = torch.empty_like(qs)
        seq.cache.lkv_attend(0, loop, seq.seqs, qs, out, split_k=1)
        torch.cuda.synchronize()
        os_ = harness.out_f64(out)[:, 0]
        assert np.abs(ov - os_).max() <= TOL_F32, loop
    ver.cache.close()
    seq.cache.close()


def test_deepest_plane_cache_makes_verify_block_dependent_fp32():
    """With W = 0 the premise of Prop. 1 fails: block tokens read plane r of earlier block tokens, which
    sequential decoding reads at plane R, so the two differ (here by far more than rounding)."""
    w = _wl(64, synth.DT_F32, 1.0)
    k, L = 8, 60
    t0 = L - k
    ver = harness.build_plain(w, lengths=[L], policy=vla.POLICY_RIPE, window=0, q_len=k, rows=[0])
    seq = harness.build_plain(w, lengths=[t0 + 1 + i for i in range(k)], policy=vla.POLICY_RIPE, window=0,
                              q_len=1, rows=[0] * k, max_len=L)
    qv = harness.gpu_queries(ver, 0, 0, k)
    ov = harness.out_f64(_verify(ver, 0, 0, qv)[0])[0]
    qs = harness.gpu_queries(seq, 0, 0, 1)
    out = torch.empty_like(qs)
    seq.cache.lkv_attend(0, 0, seq.seqs, qs, out, split_k=1)
    torch.cuda.synchronize()
    diff = np.abs(ov - harness.out_f64(out)[:, 0]).max(axis=(1, 2))
    assert diff[0] <= TOL_F32 and diff[1:].max() > 1e-3
    ver.cache.close()
    seq.cache.close()


def test_verify_fp32_every_row():
    w = _wl(64, synth.DT_F32, 0.25)
    lengths = [9, 47, 130]
    k = 5
    built = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_RIPE, window=10, q_len=k, shuffle=True,
                                poison=True)
    rows = [(b, i, h) for b in range(3) for i in range(k) for h in range(w.n_heads)]
    for loop in (1, 4):
        q = harness.gpu_queries(built, 0, loop, k)
        want, _ = harness.oracle_rows(w, rows, 0, loop, lengths, k, vla.POLICY_RIPE, 10)
        o = harness.out_f64(_verify(built, 0, loop, q, 2)[0])
        got = np.array([o[b, i, h] for (b, i, h) in rows])
        assert np.abs(got - want).max() <= TOL_F32
    built.cache.close()


def _draft_inputs(w, n_seqs, layer, loop, n_cached, dl, rows):
    """Scratch keys/values of the draft block, device [n_seqs][dl][H][D], plus fp64 copies."""
    dt = harness.torch_dtype(w.dtype)
    dk = torch.empty((n_seqs, dl, w.n_heads, w.head_dim), dtype=dt, device="cuda")
    dv = torch.empty_like(dk)
    st = torch.cuda.current_stream().cuda_stream
    for b in range(n_seqs):
        synth.gpu_kv(dk[b].data_ptr(), w.dtype, w.seed, synth.T_DRAFTK, rows[b], layer, loop, w.n_heads, w.head_dim,
                     n_cached[b], dl, synth.MODE_PLAIN, w.n_loops, w.scale, st)
        synth.gpu_kv(dv[b].data_ptr(), w.dtype, w.seed, synth.T_DRAFTV, rows[b], layer, loop, w.n_heads, w.head_dim,
                     n_cached[b], dl, synth.MODE_PLAIN, w.n_loops, w.scale, st)
    return dk, dv


@pytest.mark.parametrize("policy,W", [(vla.POLICY_RIPE, 0), (vla.POLICY_RIPE, 12), (vla.POLICY_FULL, 0)])
@pytest.mark.parametrize("D", [96, 128, 256])
def test_draft_step(policy, W, D):
    """RIPE page, Alg. 1 draft: the query (last draft token) reads cached positions through the policy
    (W = 0: the deepest plane) and the draft block's own keys/values from scratch."""
    w = _wl(D)
    n_cached = [30, 64, 200]
    dl = 4
    built = harness.build_plain(w, lengths=n_cached, policy=policy, window=W, q_len=1, shuffle=True, poison=True,
                                max_block=8)
    for loop in (0, 3):
        dk, dv = _draft_inputs(w, 3, 0, loop, n_cached, dl, built.rows)
        q = harness.gpu_queries(built, 0, loop, 1, t0s=[n + dl - 1 for n in n_cached])
        out = torch.empty_like(q)
        for split_k in (1, 3):
            ws = torch.empty(max(4, 3 * w.n_heads * split_k * (D + 1) * 4), dtype=torch.uint8, device="cuda")
            built.cache.lkv_attend(0, loop, built.seqs, q, out, mode=vla.MODE_DRAFT, window=W, split_k=split_k,
                                   workspace=ws, draft_k=dk, draft_v=dv, draft_len=dl)
            torch.cuda.synchronize()
            o = harness.out_f64(out)
            R = w.n_loops
            for b, n in enumerate(n_cached):
                for h in range(w.n_heads):
                    L = n + dl
                    ko = harness.cpu_values(w, synth.T_K, b, 0, loop, h, L)
                    vo = harness.cpu_values(w, synth.T_V, b, 0, loop, h, L)
                    kd = harness.cpu_values(w, synth.T_K, b, 0, R - 1, h, L)
                    vd = harness.cpu_values(w, synth.T_V, b, 0, R - 1, h, L)
                    sk = synth.kv(w.dtype, w.seed, synth.T_DRAFTK, b, 0, loop, w.n_heads, D, n, dl, heads=[h])[:, 0]
                    sv = synth.kv(w.dtype, w.seed, synth.T_DRAFTV, b, 0, loop, w.n_heads, D, n, dl, heads=[h])[:, 0]
                    ko[n:], vo[n:] = harness.to_f64(sk, w.dtype), harness.to_f64(sv, w.dtype)
                    qq = harness.cpu_query(w, b, 0, loop, h, L - 1)
                    want, _ = oracle.attend_row(qq, ko, vo, kd, vd, L - 1, n, policy, loop, R, W)
                    assert np.abs(o[b, 0, h] - want).max() <= TOL_BF16, (loop, b, h)
    built.cache.close()


@pytest.mark.slow
@pytest.mark.parametrize("policy", [vla.POLICY_FULL, vla.POLICY_RIPE])
def test_huginn_verify_full_size_sampled(policy):
    """Self-speculative verify at the Huginn shape: 16 sequences, L = 808 (800 cached + block of 8),
    55 heads x 96, full cache vs RIPE W = 64; layer 0, loops 0 and 31; sampled rows against the oracle in the
    launch configuration the benchmark times (one split, the untraced two-wave verify kernel, no merge) and with
    the library's own split choice (splits and the merge)."""
    w = synth.WORKLOADS["huginn_verify"]
    assert w.split_k == 1  # the benchmark's launch configuration
    built = harness.build_plain(w, layers=(0,), policy=policy, planes=[0, 31])
    rows = harness.sample_rows(w.batch, w.q_len, w.n_heads, 40, seed=3)
    for loop in (0, 31):
        q = harness.gpu_queries(built, 0, loop, w.q_len)
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, built.lengths, w.q_len, policy, w.window)
        for split_k in (1, 0):
            out, lse, _ = _verify(built, 0, loop, q, split_k=split_k)
            o = harness.out_f64(out)
            assert np.isfinite(o).all()
            got = np.array([o[b, i, h] for (b, i, h) in rows])
            assert np.abs(got - want).max() <= TOL_BF16, (loop, split_k)
            got_lse = lse.cpu().numpy()
            assert np.abs(np.array([got_lse[b, i, h] for (b, i, h) in rows]) - want_lse).max() <= 1e-3
    built.cache.close()


@pytest.mark.slow
def test_huginn_draft_full_size_sampled():
    """The draft passes at the Huginn shape, in the launch configuration the benchmark times: 16 sequences with
    800 cached positions, 55 heads x 96, draft window 0 (cached positions from the deepest plane), draft blocks of
    1, 4 and 7 tokens from scratch; layer 0, loops 0 and 3; sampled heads of every sequence against the oracle."""
    w = synth.WORKLOADS["huginn_draft"]
    R = w.n_loops
    built = harness.build_plain(w, layers=(0,), planes=[0, 3], max_block=w.extra["draft_passes"] + 1)
    rng = np.random.default_rng(5)
    for loop in (0, 3):
        for g in (1, 4, 7):
            dk, dv = harness.gpu_draft_kv(w, built.rows, 0, loop, built.lengths, g)
            q = harness.gpu_queries(built, 0, loop, 1, t0s=[L + g - 1 for L in built.lengths])
            out = torch.empty_like(q)
            built.cache.lkv_attend(0, loop, built.seqs, q, out, mode=vla.MODE_DRAFT, window=0, split_k=1,
                                   draft_k=dk, draft_v=dv, draft_len=g)
            torch.cuda.synchronize()
            o = harness.out_f64(out)
            assert np.isfinite(o).all()
            for b, n in enumerate(built.lengths):
                h = int(rng.integers(w.n_heads))
                L = n + g
                kd = harness.cpu_values(w, synth.T_K, b, 0, R - 1, h, L)
                vd = harness.cpu_values(w, synth.T_V, b, 0, R - 1, h, L)
                ko, vo = kd.copy(), vd.copy()  # cached positions come from the deepest plane at window 0
                ko[n:] = harness.cpu_draft_values(w, synth.T_DRAFTK, b, 0, loop, h, n, g)
                vo[n:] = harness.cpu_draft_values(w, synth.T_DRAFTV, b, 0, loop, h, n, g)
                qq = harness.cpu_query(w, b, 0, loop, h, L - 1)
                want, _ = oracle.attend_row(qq, ko, vo, kd, vd, L - 1, n, vla.POLICY_RIPE, loop, R, 0)
                assert np.abs(o[b, 0, h] - want).max() <= TOL_BF16, (loop, g, b, h)
    built.cache.close()


@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 7)])
def test_verify_traced_physical_slots_hold_the_oracle_planes_keys(policy, W):
    """The physical half of the verify trace, checked by content: for every (block row, key) the pool bytes at the
    traced physical page and slot (head 0's K row) equal the generator's key of that position in the plane the
    oracle names (RIPE page, Eq. (9); block positions read the own plane, proof of Prop. 1)."""
    w = _wl(96)
    lengths = [8, 21, 100, 300]
    k = 8
    built = harness.build_plain(w, lengths=lengths, policy=policy, window=W, q_len=k, shuffle=True, poison=True)
    pool = built.cache._keep[0].cpu().numpy()
    page_bytes = vla.LoopCache.sizes(built.cache.cfg).page_bytes
    D, R = w.head_dim, w.n_loops
    for loop in (0, R - 1):
        q = harness.gpu_queries(built, 0, loop, k)
        _, _, tr = _verify(built, 0, loop, q, 2, trace_len=300)
        t = tr.cpu().numpy()
        for b, L in enumerate(lengths):
            keys = {p: synth.kv(w.dtype, w.seed, synth.T_K, built.rows[b], 0, p, w.hkv, D, 0, L, w.mode, R, w.scale,
                                heads=[0])[:, 0, :] for p in (loop, R - 1)}
            for i in range(k):
                pm = oracle.plane_map(policy, loop, R, L - k + i, L - k, 300, W)
                np.testing.assert_array_equal(t[b, i, :, 0], pm)
                for j in range(L - k + i + 1):
                    phys, slot = divmod(int(t[b, i, j, 1]), 16)
                    off = phys * page_bytes + slot * D * 2
                    assert np.array_equal(pool[off:off + D * 2].view(np.uint16), keys[int(pm[j])][j]), (loop, b, i, j)
    built.cache.close()
