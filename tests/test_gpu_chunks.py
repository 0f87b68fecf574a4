"""Calls with more sequences than one launch takes (64 per launch): the library issues such a call as several
launches over consecutive groups of 64 sequences, each with its own offsets into the queries, outputs, lse,
split workspace, draft scratch and traces.  Decode (unsplit and with split partials), verify (q = k, causal
inside the block; RIPE page, Algorithm 1 and Eq. (9)), the draft step, grouped-query decode and quantised cells
(LoopKV page, Sec. 3.1-3.4) over
70 / 66 ragged sequences, against the fp64 oracle on every row of every launch; the index and mask traces of the
later launch land on their own rows; the entry point that allocates nothing gives the same bits."""
import numpy as np
import pytest

import harness
import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
BAND = 1e-4
N_SEQS = 70  # two launches: 64 + 6 sequences


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _lengths(n, lo, span):
    return [lo + (b * 7) % span for b in range(n)]


def _call(built, loop, q, mode, split_k, trace_len=0, noalloc=False):
    w = built.w
    n, k = q.shape[0], q.shape[1]
    out = torch.full_like(q, float("nan"))
    lse = torch.full((n, k, w.n_heads), float("nan"), dtype=torch.float32, device="cuda")
    tr = torch.full((n, k, trace_len, 2), -7, dtype=torch.int32, device="cuda") if trace_len else None
    if noalloc:
        built.cache.lkv_attend_noalloc(0, loop, built.seqs, q, out, q_len=k, mode=mode, split_k=split_k, lse=lse,
                                       index_trace=tr, trace_len=trace_len)
    else:
        wsb = built.cache.lkv_workspace_bytes(0, loop, built.seqs, q_len=k, mode=mode, split_k=split_k)
        ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
        built.cache.lkv_attend(0, loop, built.seqs, q, out, q_len=k, mode=mode, split_k=split_k, lse=lse,
                               workspace=ws, index_trace=tr, trace_len=trace_len)
    torch.cuda.synchronize()
    return harness.out_f64(out), lse.cpu().numpy(), (tr.cpu().numpy() if trace_len else None)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2)])
def test_decode_and_verify_past_one_launch(hq, hkv):
    """70 ragged sequences (lengths 20-48), RIPE W = 8, loops 0 and deepest: decode unsplit and with 3 splits
    (multi-head: the VALU kernel; 8 / 2 heads: the grouped-query kernel), verify with a 4-token block; every row
    within 2e-2 of the oracle, lse within 1e-3 (1e-2 on the MFMA tiles, whose weights go in as bf16); the plane
    trace of every row (both launches) equals the oracle's plane map; no-alloc decode bitwise equal."""
    W, k = 8, 4
    w = synth.Workload("chunks", N_SEQS, 1, 3, hq, 64, 48, synth.DT_BF16, "ripe", W, k, 16, synth.MODE_RIPEN, 1.0,
                       n_kv_heads=hkv)
    lengths = _lengths(N_SEQS, 20, 29)
    built = harness.build_plain(w, lengths=lengths, layers=(0,), policy=vla.POLICY_RIPE, window=W, q_len=k,
                                shuffle=True, poison=True)
    R = w.n_loops
    lse_tol_decode = 1e-3 if hq == hkv else 1e-2  # grouped-query decode runs on the MFMA tile
    for loop in (0, R - 1):
        q1 = harness.gpu_queries(built, 0, loop, 1)
        rows = [(b, 0, h) for b in range(N_SEQS) for h in range(hq)]
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, lengths, 1, oracle.RIPE, W)
        for split_k in (1, 3):
            got, lse, tr = _call(built, loop, q1, vla.MODE_DECODE, split_k, trace_len=max(lengths))
            assert np.abs(got[:, 0].reshape(-1, w.head_dim) - want).max() <= TOL, (loop, split_k)
            assert np.abs(lse[:, 0].reshape(-1) - want_lse).max() <= lse_tol_decode, (loop, split_k)
            for b, L in enumerate(lengths):
                pm = oracle.plane_map(oracle.RIPE, loop, R, L - 1, L - 1, L, W)
                np.testing.assert_array_equal(tr[b, 0, :L, 0], pm)
                assert np.all(tr[b, 0, L:, 0] == -1), b  # cleared past the row's keys, not left as the fill
        a, _, _ = _call(built, loop, q1, vla.MODE_DECODE, 3)
        b_, _, _ = _call(built, loop, q1, vla.MODE_DECODE, 3, noalloc=True)
        assert np.array_equal(a, b_), loop
        qk = harness.gpu_queries(built, 0, loop, k)
        rows = [(b, i, h) for b in range(N_SEQS) for i in range(k) for h in range(hq)]
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, lengths, k, oracle.RIPE, W)
        for split_k in (1, 2):
            got, lse, _ = _call(built, loop, qk, vla.MODE_VERIFY, split_k)
            assert np.abs(got.reshape(-1, w.head_dim) - want).max() <= TOL, (loop, split_k)
            assert np.abs(lse.reshape(-1) - want_lse).max() <= 1e-2, (loop, split_k)
    built.cache.close()


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_draft_step_past_one_launch(hq, hkv):
    """The draft step (RIPE page, Algorithm 1: cached positions through the policy at W = 0, the block's own keys
    and values from caller scratch, whose rows take the same per-launch offsets) over 70 ragged sequences with a
    3-token draft block, unsplit and with 2 splits: every row within 2e-2 of the oracle."""
    dl = 3
    w = synth.Workload("chunks", N_SEQS, 1, 3, hq, 64, 48, synth.DT_BF16, "ripe", 0, 1, 16, synth.MODE_RIPEN, 1.0,
                       n_kv_heads=hkv)
    n_cached = _lengths(N_SEQS, 17, 29)
    built = harness.build_plain(w, lengths=n_cached, layers=(0,), policy=vla.POLICY_RIPE, window=0, q_len=1,
                                shuffle=True, poison=True, max_block=8)
    R, D, group = w.n_loops, w.head_dim, hq // hkv
    for loop in (0, 1):
        dk, dv = harness.gpu_draft_kv(w, built.rows, 0, loop, n_cached, dl)
        q = harness.gpu_queries(built, 0, loop, 1, t0s=[n + dl - 1 for n in n_cached])
        want = []
        for b, n in enumerate(n_cached):
            L = n + dl
            for h in range(hq):
                hk = h // group
                ko = harness.cpu_values(w, synth.T_K, b, 0, loop, hk, L)
                vo = harness.cpu_values(w, synth.T_V, b, 0, loop, hk, L)
                kd = harness.cpu_values(w, synth.T_K, b, 0, R - 1, hk, L)
                vd = harness.cpu_values(w, synth.T_V, b, 0, R - 1, hk, L)
                ko[n:] = harness.cpu_draft_values(w, synth.T_DRAFTK, b, 0, loop, hk, n, dl)
                vo[n:] = harness.cpu_draft_values(w, synth.T_DRAFTV, b, 0, loop, hk, n, dl)
                qq = harness.cpu_query(w, b, 0, loop, h, L - 1)
                want.append(oracle.attend_row(qq, ko, vo, kd, vd, L - 1, n, oracle.RIPE, loop, R, 0)[0])
        want = np.array(want)
        for split_k in (1, 2):
            out = torch.full_like(q, float("nan"))
            wsb = built.cache.lkv_workspace_bytes(0, loop, built.seqs, mode=vla.MODE_DRAFT, split_k=split_k)
            ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
            built.cache.lkv_attend(0, loop, built.seqs, q, out, mode=vla.MODE_DRAFT, window=0, split_k=split_k,
                                   workspace=ws, draft_k=dk, draft_v=dv, draft_len=dl)
            torch.cuda.synchronize()
            got = harness.out_f64(out)[:, 0].reshape(-1, D)
            assert np.abs(got - want).max() <= TOL, (loop, split_k)
    built.cache.close()


def test_cells_past_one_launch():
    """66 quantised-cell sequences (lengths 133-332: one far token up to six code pages), INT4 / INT2 / shared /
    INT4 loops, fixed rule at offset 1 (many cold tokens): every row of both launches within 2e-2 of the
    oracle, hot masks bit-exact outside a 1e-4 band and on the rows of the later launch; no-alloc bitwise."""
    n = 66
    w = synth.Workload("cells", n, 1, 4, 2, 128, 400, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN, 1.0,
                       quant=True, sink=4, tail=128)
    lengths = _lengths(n, 133, 200)
    plan = np.array([[synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED, synth.CELL_INT4]], dtype=np.int8)
    bc = harness.build_cells(w, lengths=lengths, layers=(0,), plan=plan)
    max_far = max(lengths) - w.sink - w.tail
    words = (max_far + 31) // 32
    band_hits = 0
    for loop in range(4):
        q = harness.gpu_queries(bc, 0, loop, 1)
        res = []
        for noalloc in (False, True):
            out = torch.full_like(q, float("nan"))
            lse = torch.full((n, 1, w.n_heads), float("nan"), dtype=torch.float32, device="cuda")
            mask = torch.full((n, w.n_heads, words), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
            if noalloc:
                bc.cache.lkv_attend_noalloc(0, loop, bc.seqs, q, out, v_thresh_offset=1.0, lse=lse, mask_trace=mask)
            else:
                ws = torch.empty(bc.cache.lkv_workspace_bytes(0, loop, bc.seqs) + 4, dtype=torch.uint8, device="cuda")
                bc.cache.lkv_attend(0, loop, bc.seqs, q, out, v_thresh_offset=1.0, lse=lse, workspace=ws,
                                    mask_trace=mask)
            torch.cuda.synchronize()
            res.append((harness.out_f64(out), lse.cpu().numpy(), mask.cpu().numpy().view(np.uint32)))
        (out, lse, mask), (out2, lse2, mask2) = res
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2) and np.array_equal(mask, mask2), loop
        for b, L in enumerate(lengths):
            n_far = L - w.sink - w.tail
            for h in range(w.n_heads):
                want, want_lse, hot, s_far, thr = harness.cell_oracle_row(bc, b, 0, loop, h, 1.0)
                assert np.abs(out[b, 0, h] - want).max() <= TOL, (loop, b, h)
                assert abs(lse[b, 0, h] - want_lse) <= 1e-2, (loop, b, h)
                got = np.unpackbits(mask[b, h].view(np.uint8), bitorder="little")[:n_far]
                near = np.abs(s_far - thr) <= BAND
                if plan[0, loop] != synth.CELL_INT2:
                    assert np.array_equal(got[~near], hot[~near]), (loop, b, h)
                    band_hits += int(near.sum())
    assert band_hits < 5
    bc.cache.close()
