"""Grouped-query attention through the C-ABI against the fp64 oracle: a workgroup serves the G query heads of a
KV head from one stream of its pages (G = 2, 4, 8); query head h reads KV head h // G.  Decode runs on the MFMA
tile kernel (G columns) and, with the kernel choice LKV_KERNEL_VALU, on the VALU decode kernel; verify blocks whose k G fits the
tile's 16 columns share the tile too.  Draft runs on the same caches.  Tolerances as for multi-head caches:
1e-5 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest

import harness
import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _wl(D, G, dt=synth.DT_BF16, hkv=2, q_len=1, scale=1.0):
    return synth.Workload("gqa", 4, 2, 5, hkv * G, D, 300, dt, "ripe", 20, q_len, 16, synth.MODE_RIPEN, scale,
                          n_kv_heads=hkv)


def _attend(built, layer, loop, q, split_k, mode=vla.MODE_DECODE, trace_len=0, **kw):
    n, k = q.shape[0], q.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty((n, k, built.w.n_heads), dtype=torch.float32, device="cuda")
    wsb = built.cache.lkv_workspace_bytes(layer, loop, built.seqs, q_len=k, mode=mode, split_k=split_k)
    ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
    tr = torch.empty((n, k, trace_len, 2), dtype=torch.int32, device="cuda") if trace_len else None
    built.cache.lkv_attend(layer, loop, built.seqs, q, out, q_len=k, mode=mode, split_k=split_k, lse=lse, workspace=ws,
                           index_trace=tr, trace_len=trace_len, **kw)
    torch.cuda.synchronize()
    return harness.out_f64(out), lse.cpu().numpy(), tr


@pytest.mark.parametrize("kernel", ["tile", "valu"])
@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("D,dt,tol", [(64, synth.DT_F32, 1e-5), (128, synth.DT_BF16, 2e-2), (96, synth.DT_BF16, 2e-2),
                                      (256, synth.DT_BF16, 2e-2)])
@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 20)])
def test_gqa_decode_every_row(G, D, dt, tol, policy, W, kernel):
    kern = vla.KERNEL_VALU if kernel == "valu" else vla.KERNEL_AUTO
    w = _wl(D, G, dt, scale=0.25 if dt == synth.DT_F32 else 1.0)
    lengths = [1, 17, 100, 300]
    built = harness.build_plain(w, lengths=lengths, policy=policy, window=W, shuffle=True, poison=True)
    rows = [(b, 0, h) for b in range(len(lengths)) for h in range(w.n_heads)]
    for loop in (0, w.n_loops - 1):
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, lengths, 1, policy, W)
        q = harness.gpu_queries(built, 0, loop, 1)
        for split_k in (1, 3):
            o, lse, tr = _attend(built, 0, loop, q, split_k, trace_len=300, kernel=kern)
            got = o[:, 0].reshape(-1, D)
            assert np.isfinite(got).all()
            assert np.abs(got - want).max() <= tol, (loop, split_k)
            assert np.abs(lse[:, 0].reshape(-1) - want_lse).max() <= max(tol, 1e-3)
            t = tr.cpu().numpy()
            for b, L in enumerate(lengths):
                pm = oracle.plane_map(policy, loop, w.n_loops, L - 1, L - 1, 300, W)
                np.testing.assert_array_equal(t[b, 0, :, 0], pm)
    built.cache.close()


@pytest.mark.parametrize("G,k,D", [(2, 8, 64), (4, 4, 64), (8, 2, 64), (8, 1, 64), (2, 5, 64),
                                   (4, 8, 64), (8, 4, 64), (4, 5, 96), (2, 16, 128), (8, 3, 128),
                                   (4, 4, 256), (4, 8, 256)])
def test_gqa_verify_every_row(G, k, D):
    """Verify tiles on a GQA cache (each query head reads its group's KV head): k G <= 16 puts the block's rows
    of all G heads in one tile; 16 < k G <= 32 takes two tiles sharing the page's K/V registers (head dim <= 128);
    larger blocks, and k G > 16 at head dim 256, take one query head per tile.  RIPE window 20 >= k - 1."""
    w = _wl(D, G, q_len=k)
    lengths = [k, 40, 300]
    assert k <= 16
    built = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_RIPE, window=20, q_len=k, shuffle=True,
                                poison=True)
    rows = [(b, i, h) for b in range(3) for i in range(k) for h in range(w.n_heads)]
    for loop in (1, 4):
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, lengths, k, vla.POLICY_RIPE, 20)
        q = harness.gpu_queries(built, 0, loop, k)
        for split_k in (1, 2):
            o, lse, tr = _attend(built, 0, loop, q, split_k, mode=vla.MODE_VERIFY, trace_len=300)
            got = np.array([o[b, i, h] for (b, i, h) in rows])
            assert np.abs(got - want).max() <= 2e-2, (loop, split_k)
            got_lse = np.array([lse[b, i, h] for (b, i, h) in rows])
            assert np.abs(got_lse - want_lse).max() <= 2e-2
            t = tr.cpu().numpy()
            for b, L in enumerate(lengths):
                for i in range(k):
                    pm = oracle.plane_map(vla.POLICY_RIPE, loop, w.n_loops, L - k + i, L - k, 300, 20)
                    np.testing.assert_array_equal(t[b, i, :, 0], pm)
    built.cache.close()


@pytest.mark.parametrize("G,D", [(2, 128), (8, 128), (4, 256)])
def test_gqa_draft_step(G, D):
    """Draft step on a GQA cache: cached positions through the policy, the block from scratch keys/values of the
    KV heads."""
    w = _wl(D, G)
    n_cached = [30, 200]
    dl = 3
    built = harness.build_plain(w, lengths=n_cached, policy=vla.POLICY_RIPE, window=12, q_len=1, shuffle=True,
                                poison=True, max_block=8)
    st = torch.cuda.current_stream().cuda_stream
    R, H, HK, D = w.n_loops, w.n_heads, w.hkv, w.head_dim
    for loop in (0, 3):
        dk = torch.empty((2, dl, HK, D), dtype=torch.bfloat16, device="cuda")
        dv = torch.empty_like(dk)
        for b in range(2):
            synth.gpu_kv(dk[b].data_ptr(), w.dtype, 0, synth.T_DRAFTK, b, 0, loop, HK, D, n_cached[b], dl,
                         synth.MODE_PLAIN, R, 1.0, st)
            synth.gpu_kv(dv[b].data_ptr(), w.dtype, 0, synth.T_DRAFTV, b, 0, loop, HK, D, n_cached[b], dl,
                         synth.MODE_PLAIN, R, 1.0, st)
        q = harness.gpu_queries(built, 0, loop, 1, t0s=[n + dl - 1 for n in n_cached])
        o, _, _ = _attend(built, 0, loop, q, 2, mode=vla.MODE_DRAFT, window=0, draft_k=dk, draft_v=dv, draft_len=dl)
        for b, n in enumerate(n_cached):
            L = n + dl
            for h in range(H):
                hk = h // G
                ko = harness.cpu_values(w, synth.T_K, b, 0, loop, hk, L)
                vo = harness.cpu_values(w, synth.T_V, b, 0, loop, hk, L)
                kd = harness.cpu_values(w, synth.T_K, b, 0, R - 1, hk, L)
                vd = harness.cpu_values(w, synth.T_V, b, 0, R - 1, hk, L)
                sk = synth.kv(w.dtype, 0, synth.T_DRAFTK, b, 0, loop, HK, D, n, dl, heads=[hk])[:, 0]
                sv = synth.kv(w.dtype, 0, synth.T_DRAFTV, b, 0, loop, HK, D, n, dl, heads=[hk])[:, 0]
                ko[n:], vo[n:] = harness.to_f64(sk, w.dtype), harness.to_f64(sv, w.dtype)
                qq = harness.cpu_query(w, b, 0, loop, h, L - 1)
                want, _ = oracle.attend_row(qq, ko, vo, kd, vd, L - 1, n, oracle.RIPE, loop, R, 0)
                assert np.abs(o[b, 0, h] - want).max() <= 2e-2, (loop, b, h)
    built.cache.close()


@pytest.mark.slow
def test_raven_ripe_full_size_sampled():
    """Raven-shaped RIPE decode at full size for one layer (64 sequences, 32 query heads over 8 KV heads x 64,
    L = 1024, W = 64): sampled rows vs the oracle, the launch configuration the benchmark times."""
    w = synth.WORKLOADS["raven_ripe"]
    built = harness.build_plain(w, layers=(0,))
    rows = harness.sample_rows(w.batch, 1, w.n_heads, 24, seed=5)
    for loop in (0, 31):
        q = harness.gpu_queries(built, 0, loop, 1)
        o, _, _ = _attend(built, 0, loop, q, 0)
        assert np.isfinite(o).all()
        want, _ = harness.oracle_rows(w, rows, 0, loop, built.lengths, 1, vla.POLICY_RIPE, w.window)
        got = np.array([o[b, i, h] for (b, i, h) in rows])
        assert np.abs(got - want).max() <= 2e-2
    built.cache.close()


@pytest.mark.slow
def test_dory_lastloop_full_size_sampled():
    """Dory-shaped decode in the last-loop mode at full size for one layer (32 sequences, 16 query heads over
    4 KV heads x 256, L = 16384, W = 0: the history from the final loop's plane, the current token from the
    loop's own): sampled rows vs the oracle, in the launch configuration the benchmark times."""
    w = synth.WORKLOADS["dory_lastloop"]
    built = harness.build_plain(w, layers=(0,))
    rows = harness.sample_rows(w.batch, 1, w.n_heads, 16, seed=6)
    for loop in (0, 3):
        q = harness.gpu_queries(built, 0, loop, 1)
        o, _, _ = _attend(built, 0, loop, q, 0)
        assert np.isfinite(o).all()
        want, _ = harness.oracle_rows(w, rows, 0, loop, built.lengths, 1, vla.POLICY_RIPE, w.window)
        got = np.array([o[b, i, h] for (b, i, h) in rows])
        assert np.abs(got - want).max() <= 2e-2
    built.cache.close()
