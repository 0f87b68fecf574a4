"""GPU parity of q = 1 decode through the C-ABI against the fp64 oracle.

Tolerances (max-abs on outputs): 1e-5 for fp32 caches, 2e-2 for bf16 caches
(bf16 inputs, fp32 accumulation, bf16 output rounding).  Page indexing is
compared exactly: the kernel's per-position trace of (plane, physical slot)
against the oracle's plane map and the host block tables.
"""
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


def _attend(built, layer, loop, q, split_k, window=-1, trace_len=0):
    w = built.w
    n = len(built.seqs)
    out = torch.empty_like(q)
    lse = torch.empty((n, q.shape[1], w.n_heads), dtype=torch.float32, device="cuda")
    ws_bytes = built.cache.lkv_workspace_bytes(layer, loop, built.seqs, q_len=q.shape[1], split_k=split_k)
    ws = torch.empty(max(4, ws_bytes), dtype=torch.uint8, device="cuda")
    tr = torch.empty((n, q.shape[1], trace_len, 2), dtype=torch.int32, device="cuda") if trace_len else None
    built.cache.lkv_attend(layer, loop, built.seqs, q, out, q_len=q.shape[1], split_k=split_k, lse=lse,
                           workspace=ws, window=window, index_trace=tr, trace_len=trace_len)
    torch.cuda.synchronize()
    return out, lse, tr


@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 0), (vla.POLICY_RIPE, 16),
                                      (vla.POLICY_RIPE, 128)])
@pytest.mark.parametrize("split_k", [1, 3])
def test_tiny_fp32_every_row_and_trace(policy, W, split_k):
    """Tiny workload: fp32, 1 layer, 4 loops, 2 heads x 64, L = 128, seed 0: every output, lse and the
    exact page-index trace, for the full cache and RIPE W in {0, 16, 128} on the same inputs."""
    w = synth.WORKLOADS["tiny"]
    built = harness.build_plain(w, policy=policy, window=W, poison=True)
    L = w.length
    for loop in range(w.n_loops):
        q = harness.gpu_queries(built, 0, loop, 1)
        out, lse, tr = _attend(built, 0, loop, q, split_k, trace_len=L)
        rows = [(0, 0, h) for h in range(w.n_heads)]
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, built.lengths, 1, policy, W)
        got = harness.out_f64(out)[0, 0]
        assert np.abs(got - want).max() <= TOL_F32
        assert np.abs(lse.cpu().numpy()[0, 0] - want_lse).max() <= TOL_F32
        trace = tr.cpu().numpy()[0, 0]
        pm = oracle.plane_map(policy, loop, w.n_loops, L - 1, L - 1, L, W)
        np.testing.assert_array_equal(trace[:, 0], pm)
        for j in range(L):
            plane, phys, slot = built.cache.lkv_debug_resolve(built.seqs[0], 0, loop, L - 1, L - 1, j, W)
            assert plane == pm[j] and trace[j, 1] == phys * 16 + slot
    built.cache.close()


def _ragged(D, mode=synth.MODE_RIPEN):
    return synth.Workload("ragged", 6, 2, 5, 3, D, 257, synth.DT_BF16, "ripe", 20, 1, 16, mode, 1.0)


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("policy", [vla.POLICY_FULL, vla.POLICY_RIPE])
def test_ragged_lengths_bf16(D, policy):
    """Ragged batch (lengths 1, 15, 16, 17, 100, 257: empty window, page edges, partial pages), shuffled
    pages poisoned with NaN, loops 0 / 2 / deepest, splits 1 / 2 / 5."""
    w = _ragged(D)
    lengths = [1, 15, 16, 17, 100, 257]
    built = harness.build_plain(w, lengths=lengths, layers=(1,), policy=policy, window=20, shuffle=True,
                                poison=True)
    rows = [(b, 0, h) for b in range(len(lengths)) for h in range(w.n_heads)]
    for loop in (0, 2, w.n_loops - 1):
        want, want_lse = harness.oracle_rows(w, rows, 1, loop, lengths, 1, policy, 20)
        q = harness.gpu_queries(built, 1, loop, 1)
        for split_k in (1, 2, 5):
            out, lse, _ = _attend(built, 1, loop, q, split_k)
            got = harness.out_f64(out)[:, 0]
            assert np.isfinite(got).all()
            err = np.abs(got.reshape(-1, D) - want).max()
            assert err <= TOL_BF16, (loop, split_k, err)
            assert np.abs(lse.cpu().numpy()[:, 0].reshape(-1) - want_lse).max() <= 1e-3
    built.cache.close()


@pytest.mark.parametrize("D", [96, 128])
@pytest.mark.parametrize("waves", [2, 4, 8])
def test_waves_per_workgroup(D, waves):
    """The multi-head decode kernel at 2, 4 and 8 waves per workgroup (the library picks 2 for grids of 768-1024
    workgroups, else 8): ragged lengths 1-257, RIPE W = 20, loops 0 / 2 / deepest, splits 1 and 3, every row
    against the oracle."""
    w = _ragged(D)
    lengths = [1, 15, 16, 17, 100, 257]
    built = harness.build_plain(w, lengths=lengths, layers=(1,), policy=vla.POLICY_RIPE, window=20, shuffle=True,
                                poison=True)
    rows = [(b, 0, h) for b in range(len(lengths)) for h in range(w.n_heads)]
    for loop in (0, 2, w.n_loops - 1):
        want, want_lse = harness.oracle_rows(w, rows, 1, loop, lengths, 1, vla.POLICY_RIPE, 20)
        q = harness.gpu_queries(built, 1, loop, 1)
        for split_k in (1, 3):
            out = torch.empty_like(q)
            lse = torch.empty((len(lengths), 1, w.n_heads), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(4, built.cache.lkv_workspace_bytes(1, loop, built.seqs, split_k=split_k)),
                             dtype=torch.uint8, device="cuda")
            built.cache.lkv_attend(1, loop, built.seqs, q, out, split_k=split_k, lse=lse, workspace=ws, waves=waves)
            torch.cuda.synchronize()
            got = harness.out_f64(out)[:, 0].reshape(-1, D)
            assert np.abs(got - want).max() <= TOL_BF16, (loop, split_k)
            assert np.abs(lse.cpu().numpy()[:, 0].reshape(-1) - want_lse).max() <= 1e-3, (loop, split_k)
    built.cache.close()


@pytest.mark.parametrize("policy", [vla.POLICY_FULL, vla.POLICY_RIPE])
def test_ripening_planes_in_the_page_direction(policy):
    """Planes ripening in the RIPE page's direction (MODE_RIPEN_PAPER: plane r = plane R + 0.88^(r+1) noise,
    shrinking with r, Sec. 3.2): the GPU fill kernel writes the planes the numpy generator gives the oracle, and
    the path matches the oracle as under the workload's recipe (ragged lengths, loops 0 / 2 / deepest, splits 1
    and 2)."""
    w = _ragged(96, synth.MODE_RIPEN_PAPER)
    lengths = [1, 17, 100, 257]
    built = harness.build_plain(w, lengths=lengths, layers=(1,), policy=policy, window=20, shuffle=True,
                                poison=True)
    rows = [(b, 0, h) for b in range(len(lengths)) for h in range(w.n_heads)]
    for loop in (0, 2, w.n_loops - 1):
        want, want_lse = harness.oracle_rows(w, rows, 1, loop, lengths, 1, policy, 20)
        q = harness.gpu_queries(built, 1, loop, 1)
        for split_k in (1, 2):
            out, lse, _ = _attend(built, 1, loop, q, split_k)
            got = harness.out_f64(out)[:, 0]
            assert np.abs(got.reshape(-1, w.head_dim) - want).max() <= TOL_BF16, (loop, split_k)
            assert np.abs(lse.cpu().numpy()[:, 0].reshape(-1) - want_lse).max() <= 1e-3
    built.cache.close()


def test_shuffled_tables_are_bitwise_identical_to_identity_tables():
    """Paging changes addresses, not values: identical outputs for shuffled and in-order page tables."""
    w = _ragged(96)
    lengths = [33, 100, 257]
    outs = []
    for shuffle in (False, True):
        built = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_RIPE, window=20, shuffle=shuffle)
        q = harness.gpu_queries(built, 0, 1, 1)
        outs.append([_attend(built, 0, 1, q, s)[0].cpu() for s in (1, 4)])
        built.cache.close()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_window_covering_context_is_bitwise_the_full_cache():
    """RIPE with W >= L - 1 reads plane r everywhere, i.e. exactly the full cache."""
    w = _ragged(128)
    lengths = [40, 64, 90]
    full = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_FULL)
    ripe = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_RIPE, window=200, max_len=256)
    for loop in (0, 3):
        q = harness.gpu_queries(full, 0, loop, 1)
        for s in (1, 3):
            a = _attend(full, 0, loop, q, s)[0]
            b = _attend(ripe, 0, loop, q, s)[0]
            assert torch.equal(a, b)
    full.cache.close()
    ripe.cache.close()


def test_window_zero_reads_the_deepest_plane():
    """W = 0 is the deepest-plane cache: every cached position reads plane R (RIPE page, Sec. 2)."""
    w = _ragged(64)
    lengths = [50, 77]
    built = harness.build_plain(w, lengths=lengths, policy=vla.POLICY_RIPE, window=0)
    rows = [(b, 0, h) for b in range(2) for h in range(w.n_heads)]
    for loop in (0, 1):
        q = harness.gpu_queries(built, 0, loop, 1)
        out, _, tr = _attend(built, 0, loop, q, 2, trace_len=80)
        t = tr.cpu().numpy()
        for b, L in enumerate(lengths):
            assert (t[b, 0, :L - 1, 0] == w.n_loops - 1).all() and t[b, 0, L - 1, 0] == loop
            assert (t[b, 0, L:, 0] == -1).all()
        want, _ = harness.oracle_rows(w, rows, 0, loop, lengths, 1, vla.POLICY_RIPE, 0)
        assert np.abs(harness.out_f64(out)[:, 0].reshape(-1, 64) - want).max() <= TOL_BF16
    built.cache.close()


def test_split_k_merge_matches_unsplit_fp32():
    """LSE merge of split partials equals the unsplit softmax (fp32 cache: within 1e-6)."""
    w = synth.Workload("f32", 3, 1, 3, 4, 128, 700, synth.DT_F32, "ripe", 33, 1, 16, synth.MODE_RIPEN, 0.25)
    built = harness.build_plain(w, lengths=[700, 129, 16], policy=vla.POLICY_RIPE, window=33, shuffle=True)
    q = harness.gpu_queries(built, 0, 1, 1)
    base = harness.out_f64(_attend(built, 0, 1, q, 1)[0])
    for s in (2, 7, 16, 64):
        got = harness.out_f64(_attend(built, 0, 1, q, s)[0])
        assert np.abs(got - base).max() <= 1e-6
    built.cache.close()


@pytest.mark.slow
def test_huginn_ripe_full_size_sampled():
    """Huginn-shaped RIPE decode at full size (32 sequences, 55 heads x 96, L = 1024, W = 64, page 16),
    layer 0, loops 0 / 17 / 31, in two launch configurations:
      * the one the benchmark times: one split, the untraced 8-wave decode kernel, no merge;
      * the library's own split choice with the index trace on (the traced kernel instance and the merge).
    Sampled rows of both against the oracle element by element, and the whole index trace of head 0 against the
    oracle's plane map."""
    w = synth.WORKLOADS["huginn_ripe"]
    assert w.split_k == 1  # the benchmark's launch configuration
    built = harness.build_plain(w, layers=(0,))
    L = w.length
    rows = harness.sample_rows(w.batch, 1, w.n_heads, 40, seed=1)
    for loop in (0, 17, 31):
        q = harness.gpu_queries(built, 0, loop, 1)
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, built.lengths, 1, vla.POLICY_RIPE, w.window)
        # the timed configuration
        out, lse, _ = _attend(built, 0, loop, q, 1)
        o = harness.out_f64(out)
        assert np.isfinite(o).all()
        got = np.array([o[b, i, h] for (b, i, h) in rows])
        assert np.abs(got - want).max() <= TOL_BF16, loop
        got_lse = lse.cpu().numpy()
        assert np.abs(np.array([got_lse[b, i, h] for (b, i, h) in rows]) - want_lse).max() <= 1e-3
        # library-chosen splits with the trace
        out_t, _, tr = _attend(built, 0, loop, q, 0, trace_len=L)
        o_t = harness.out_f64(out_t)
        assert np.isfinite(o_t).all()
        assert np.abs(np.array([o_t[b, i, h] for (b, i, h) in rows]) - want).max() <= TOL_BF16, loop
        pm = oracle.plane_map(vla.POLICY_RIPE, loop, w.n_loops, L - 1, L - 1, L, w.window)
        t = tr.cpu().numpy()
        for b in range(w.batch):
            np.testing.assert_array_equal(t[b, 0, :, 0], pm)
    built.cache.close()


@pytest.mark.slow
def test_ouro_full_size_sampled():
    """Ouro-shaped paged decode at full size for one layer (32 sequences, 16 heads x 128, L = 8192,
    shuffled page tables, 8 splits merged by LSE): sampled rows vs the oracle."""
    w = synth.WORKLOADS["ouro_splitk"]
    built = harness.build_plain(w, layers=(0,), planes=[0, 3])
    rows = harness.sample_rows(w.batch, 1, w.n_heads, 12, seed=2)
    for loop in (0, 3):
        q = harness.gpu_queries(built, 0, loop, 1)
        out, lse, _ = _attend(built, 0, loop, q, 8)
        o = harness.out_f64(out)
        assert np.isfinite(o).all()
        want, want_lse = harness.oracle_rows(w, rows, 0, loop, built.lengths, 1, vla.POLICY_FULL, 0)
        got = np.array([o[b, i, h] for (b, i, h) in rows])
        assert np.abs(got - want).max() <= TOL_BF16
        got_lse = lse.cpu().numpy()
        assert np.abs(np.array([got_lse[b, i, h] for (b, i, h) in rows]) - want_lse).max() <= 1e-3
    built.cache.close()


def test_timing_events_stamp_the_launch_and_change_nothing():
    """lkv_attend's optional event pair is stamped by the attention launch itself: the elapsed time is positive and
    the outputs equal those of the same call without events, bit for bit (decode with splits and the merge)."""
    w = _ragged(96)
    lengths = [100, 257, 40]
    built = harness.build_plain(w, lengths=lengths, layers=(1,), policy=vla.POLICY_RIPE, window=20)
    q = harness.gpu_queries(built, 1, 2, 1)
    a, _, _ = _attend(built, 1, 2, q, 3)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    ev1.record()  # torch creates the HIP events on first record
    out = torch.empty_like(q)
    ws = torch.empty(max(4, built.cache.lkv_workspace_bytes(1, 2, built.seqs, split_k=3)), dtype=torch.uint8,
                     device="cuda")
    built.cache.lkv_attend(1, 2, built.seqs, q, out, split_k=3, workspace=ws, ev_begin=ev0.cuda_event,
                           ev_end=ev1.cuda_event)
    torch.cuda.synchronize()
    assert ev0.elapsed_time(ev1) > 0
    assert torch.equal(out, a)
    built.cache.close()


def test_binding_refuses_undersized_buffers_before_any_launch():
    """A q, out, lse or append buffer smaller than the call's documented shape, or of the wrong element type, raises
    ValueError in the binding (the library takes bare addresses); the cache stays usable and a correct call after
    the refusals still matches the earlier result."""
    w = _ragged(96)
    built = harness.build_plain(w, lengths=[100, 40], layers=(1,), policy=vla.POLICY_RIPE, window=20)
    q = harness.gpu_queries(built, 1, 2, 1)
    a, _, _ = _attend(built, 1, 2, q, 1)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match=r"^out holds"):
        built.cache.lkv_attend(1, 2, built.seqs, q, out[:1], split_k=1)
    with pytest.raises(ValueError, match=r"^q has element type"):
        built.cache.lkv_attend(1, 2, built.seqs, q.float(), out, split_k=1)
    with pytest.raises(ValueError, match=r"^lse holds"):
        built.cache.lkv_attend(1, 2, built.seqs, q, out, split_k=1,
                               lse=torch.empty(1, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match=r"^out must be contiguous"):
        built.cache.lkv_attend(1, 2, built.seqs, q, out.transpose(2, 3), split_k=1)
    kv = torch.empty((4, w.hkv, w.head_dim), dtype=q.dtype, device="cuda")
    with pytest.raises(ValueError, match=r"^v holds"):
        built.cache.lkv_append_plane(built.seqs[0], 1, w.n_loops - 1, 100, kv, kv[:2])
    built.cache.lkv_attend(1, 2, built.seqs, q, out, split_k=1)
    torch.cuda.synchronize()
    assert torch.equal(out, a)
    built.cache.close()


def test_split_merge_is_deterministic():
    """Split partials are merged by log-sum-exp with the parts summed in index order (LoopKV page, Sec. 3.4): 40
    repeats of the same 8-split call give the same bits, calls with other split counts on the same (layer, loop) in
    between change nothing, and sampled rows match the oracle."""
    w = synth.Workload("det", 8, 1, 3, 8, 128, 900, synth.DT_BF16, "ripe", 40, 1, 16, synth.MODE_RIPEN, 1.0)
    built = harness.build_plain(w, lengths=[900, 517, 33, 700, 129, 16, 899, 640], shuffle=True, poison=True)
    q = harness.gpu_queries(built, 0, 1, 1)
    ref, ref_lse, _ = _attend(built, 0, 1, q, 8)
    for rep in range(40):
        if rep % 10 == 5:
            _attend(built, 0, 1, q, 3 + rep // 10)  # other split counts in between
        out, lse, _ = _attend(built, 0, 1, q, 8)
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), rep
    want, _ = harness.oracle_rows(w, [(b, 0, h) for b in range(8) for h in (0, 7)], 0, 1, built.lengths, 1,
                                  vla.POLICY_RIPE, 40)
    o = harness.out_f64(ref)
    got = np.array([o[b, 0, h] for b in range(8) for h in (0, 7)])
    assert np.abs(got - want).max() <= TOL_BF16
    built.cache.close()


@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 20), (vla.POLICY_RIPE, 0)])
def test_traced_physical_slots_hold_the_oracle_planes_keys(policy, W):
    """The physical half of the index trace, checked by content: for every key position j a row reads, the pool
    bytes at the traced physical page and slot (head 0's K row) equal, bit for bit, the generator's key of
    position j in the plane the oracle names (RIPE page, Sec. 2 policy pi and Eq. (9) with the block rule).  This
    pins the page resolution to the oracle and the seeded generator, not to the library's own tables."""
    w = _ragged(96)
    lengths = [1, 15, 16, 17, 100, 257]
    built = harness.build_plain(w, lengths=lengths, layers=(1,), policy=policy, window=W, shuffle=True,
                                poison=True)
    pool = built.cache._keep[0].cpu().numpy()
    page_bytes = vla.LoopCache.sizes(built.cache.cfg).page_bytes
    D, R = w.head_dim, w.n_loops
    for loop in (0, 2, R - 1):
        q = harness.gpu_queries(built, 1, loop, 1)
        _, _, tr = _attend(built, 1, loop, q, 2, trace_len=max(lengths))
        t = tr.cpu().numpy()
        for b, L in enumerate(lengths):
            pm = oracle.plane_map(policy, loop, R, L - 1, L - 1, L, W)
            np.testing.assert_array_equal(t[b, 0, :L, 0], pm)
            for plane in set(pm.tolist()):
                want = synth.kv(w.dtype, w.seed, synth.T_K, built.rows[b], 1, plane, w.hkv, D, 0, L, w.mode, R,
                                w.scale, heads=[0])[:, 0, :]  # bf16 bits [L][D]
                for j in np.flatnonzero(pm == plane):
                    phys, slot = divmod(int(t[b, 0, j, 1]), 16)
                    off = phys * page_bytes + slot * D * 2  # head 0's K block: [token][channel]
                    got = pool[off:off + D * 2].view(np.uint16)
                    assert np.array_equal(got, want[j]), (loop, b, j, plane)
    built.cache.close()
