"""GPU parity of LoopKV-style quantised cells (INT4 / INT2 / shared; bit-plane V with the
fixed hot rule s >= m0 - offset and the page's running-maximum rule) through the C-ABI against the fp64 oracle.

Outputs: max-abs 2e-2 (bf16 out).  Hot masks: bit-exact for every far token whose score
lies outside a 1e-4 band around the threshold (both sides compute the score in a
different rounding order; inside the band either bit is accepted and counted)."""
import math

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _cells_wl(batch=3):
    return synth.Workload("cells", batch, 2, 4, 2, 128, 1000, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN,
                          1.0, quant=True, sink=4, tail=128)


def _attend_cells(bc, layer, loop, offset, split_k=0, v_rule=vla.VRULE_FIXED, v_tau=14.0):
    w = bc.w
    n = len(bc.seqs)
    q = harness.gpu_queries(bc, layer, loop, 1)
    out = torch.empty_like(q)
    lse = torch.empty((n, 1, w.n_heads), dtype=torch.float32, device="cuda")
    max_far = max(bc.lengths) - w.sink - w.tail
    words = (max_far + 31) // 32
    mask = torch.empty((n, w.n_heads, words), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(4, bc.cache.lkv_workspace_bytes(layer, loop, bc.seqs, split_k=split_k)) + (1 << 20),
                     dtype=torch.uint8, device="cuda")
    bc.cache.lkv_attend(layer, loop, bc.seqs, q, out, split_k=split_k, v_thresh_offset=offset, lse=lse,
                        workspace=ws, mask_trace=mask, v_rule=v_rule, v_tau=v_tau)
    torch.cuda.synchronize()
    return harness.out_f64(out), lse.cpu().numpy(), mask.cpu().numpy().view(np.uint32)


def _bits(words, n_far):
    b = np.unpackbits(words.view(np.uint8), bitorder="little")
    return b[:n_far]


PLAN = np.array([[synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED, synth.CELL_INT4],
                 [synth.CELL_SHARED, synth.CELL_INT4, synth.CELL_INT2, synth.CELL_INT4]], dtype=np.int8)


@pytest.mark.parametrize("offset", [4.0, 1.0, math.inf, -math.inf])
def test_cells_every_kind(offset):
    """Ragged lengths (133 = sink + tail + 1: one far token; a partial last code page; 1000), every cell kind,
    offsets 4 (the workload's rule), 1 (many cold tokens), +inf (all hot), -inf (all cold)."""
    w = _cells_wl()
    lengths = [133, 300, 1000]
    bc = harness.build_cells(w, lengths=lengths, layers=(0, 1), plan=PLAN)
    band_hits = 0
    for layer in (0, 1):
        for loop in range(4):
            for split_k in (1, 3):
                out, lse, mask = _attend_cells(bc, layer, loop, offset, split_k)
                assert np.isfinite(out).all()
                for b, L in enumerate(lengths):
                    n_far = L - w.sink - w.tail
                    for h in range(w.n_heads):
                        want, want_lse, hot, s_far, thr = harness.cell_oracle_row(bc, b, layer, loop, h, offset)
                        err = np.abs(out[b, 0, h] - want).max()
                        assert err <= TOL, (layer, loop, split_k, b, h, err)
                        assert abs(lse[b, 0, h] - want_lse) <= 1e-2
                        got = _bits(mask[b, h], n_far)
                        near = np.abs(s_far - thr) <= BAND if np.isfinite(thr) else np.zeros(n_far, bool)
                        assert np.array_equal(got[~near], hot[~near]), (layer, loop, b, h)
                        band_hits += int(near.sum())
    assert band_hits < 5
    bc.cache.close()


@pytest.mark.parametrize("split_k", [0, 2, 5, 16, 64])
def test_cells_far_shares(split_k):
    """How a row's far pages are shared: the far blocks and the near block take equal shares of the code pages
    plus the near work, so with many splits most blocks get no page or one, and a wave's run of pages in the
    pipelined loops is empty, one page, or a few (lengths 133: one far token; 164: exactly one code page; 229:
    four pages, the last partial; 420; 1000), for every cell kind at the fixed rule (offset 4) and the
    library's own split choice (0): outputs within 2e-2 of the oracle, hot masks bit-exact outside a 1e-4
    band around the threshold."""
    w = _cells_wl(5)
    lengths = [133, 164, 229, 420, 1000]
    bc = harness.build_cells(w, lengths=lengths, layers=(0, 1), plan=PLAN)
    band_hits = 0
    for layer in (0, 1):
        for loop in range(4):
            out, lse, mask = _attend_cells(bc, layer, loop, 4.0, split_k)
            assert np.isfinite(out).all()
            for b, L in enumerate(lengths):
                n_far = L - w.sink - w.tail
                for h in range(w.n_heads):
                    want, want_lse, hot, s_far, thr = harness.cell_oracle_row(bc, b, layer, loop, h, 4.0)
                    assert np.abs(out[b, 0, h] - want).max() <= TOL, (layer, loop, split_k, b, h)
                    assert abs(lse[b, 0, h] - want_lse) <= 1e-2
                    got = _bits(mask[b, h], n_far)
                    near = np.abs(s_far - thr) <= BAND
                    assert np.array_equal(got[~near], hot[~near]), (layer, loop, split_k, b, h)
                    band_hits += int(near.sum())
    assert band_hits < 5
    bc.cache.close()


def test_all_hot_cell_reads_full_int4_codes_bitwise_equal_to_negative_infinite_threshold():
    """LoopKV page, App. I: with the threshold at -inf (every token hot) the reader equals the plain reader
    of both V planes; the same kernel with any offset >= the whole score range gives the same bits."""
    w = _cells_wl(2)
    bc = harness.build_cells(w, lengths=[500, 700], layers=(0,), plan=PLAN)
    a, _, ma = _attend_cells(bc, 0, 0, math.inf, 2)
    b, _, mb = _attend_cells(bc, 0, 0, 1e9, 2)
    assert np.array_equal(a, b) and np.array_equal(ma, mb)
    bc.cache.close()


@pytest.mark.slow
@pytest.mark.parametrize("layer", [0, 14])
def test_loopkv_full_shape_sampled(layer):
    """The LoopKV-shaped workload at full length: 16 sequences, L = 16384 (sink 4, far 16252, tail 128),
    16 heads x 128, the seeded plan's cells of one layer's four loops (layer 0: four INT4 cells; layer 14: INT2,
    shared, shared, INT4); sampled rows and their masks with the hot-mask trace on (the traced kernel
    instance), and sampled rows in the launch configuration the benchmark times (untraced kernel, the
    library's split choice), under the fixed rule and under the page's running rule."""
    w = synth.WORKLOADS["loopkv_cells"]
    plan = synth.cell_plan(w.seed, w.n_layers, w.n_loops)
    bc = harness.build_cells(w, layers=(layer,), plan=plan)
    rng = np.random.default_rng(4 + layer)
    n_far = w.length - w.sink - w.tail
    for loop in range(w.n_loops):
        out, lse, mask = _attend_cells(bc, layer, loop, 4.0)
        assert np.isfinite(out).all()
        q = harness.gpu_queries(bc, layer, loop, 1)
        plain = torch.empty_like(q)
        ws = torch.empty(bc.cache.lkv_workspace_bytes(layer, loop, bc.seqs) + 4, dtype=torch.uint8, device="cuda")
        bc.cache.lkv_attend(layer, loop, bc.seqs, q, plain, workspace=ws, v_thresh_offset=4.0)
        torch.cuda.synchronize()
        plain = harness.out_f64(plain)
        assert np.isfinite(plain).all()
        # the page's running rule (tau 14) in the same launch configuration: untraced, the library's split
        # count, read back from the workspace size ([rows][S + 1][d + 1] fp32)
        S = bc.cache.lkv_workspace_bytes(layer, loop, bc.seqs) // (w.batch * w.n_heads * (w.head_dim + 1) * 4) - 1
        run = torch.empty_like(q)
        bc.cache.lkv_attend(layer, loop, bc.seqs, q, run, workspace=ws, v_rule=vla.VRULE_RUNNING, v_tau=14.0)
        torch.cuda.synchronize()
        run = harness.out_f64(run)
        assert np.isfinite(run).all()
        for _ in range(4):
            b, h = int(rng.integers(w.batch)), int(rng.integers(w.n_heads))
            want, want_lse, hot, s_far, thr = harness.cell_oracle_row(bc, b, layer, loop, h, 4.0)
            assert np.abs(out[b, 0, h] - want).max() <= TOL
            assert np.abs(plain[b, 0, h] - want).max() <= TOL
            a = harness.cell_inputs(bc, b, layer, loop, h)
            want_run = oracle.cell_row_running(a["q"], a["k_near"], a["v_near"], a["kc"], a["ks"], a["kz"], a["vc"],
                                               a["vs"], a["vz"], a["sink"], a["tail"], a["kind"], 14.0, S)[0]
            assert np.abs(run[b, 0, h] - want_run).max() <= TOL, (layer, loop, S, b, h)
            got = _bits(mask[b, h], n_far)
            near = np.abs(s_far - thr) <= BAND
            assert np.array_equal(got[~near], hot[~near])
    bc.cache.close()


@pytest.mark.parametrize("tau", [14.0, 2.0, 0.5])
@pytest.mark.parametrize("split_k", [0, 1, 3, 7])
def test_cells_running_rule(tau, split_k):
    """The LoopKV page's own V-precision rule (Sec. 3.3, App. E Algorithm 1): each far split walks its pages in
    order with a running maximum m; a token is hot iff s >= max(m, m0) - tau ln 2.  Outputs vs the oracle's rule
    with the same page partition (max-abs 2e-2) and hot masks bit-exact outside a 1e-4 band around each token's
    threshold; INT2 cells read their whole codes.  split_k 0: the library's split count."""
    w = _cells_wl()
    lengths = [133, 300, 1000]
    bc = harness.build_cells(w, lengths=lengths, layers=(0, 1), plan=PLAN)
    band_hits, cold = 0, 0
    for layer in (0, 1):
        for loop in range(4):
            n = len(bc.seqs)
            q = harness.gpu_queries(bc, layer, loop, 1)
            out = torch.empty_like(q)
            words = (max(lengths) - w.sink - w.tail + 31) // 32
            mask = torch.empty((n, w.n_heads, words), dtype=torch.int32, device="cuda")
            ws_bytes = bc.cache.lkv_workspace_bytes(layer, loop, bc.seqs, split_k=split_k)
            ws = torch.empty(ws_bytes + 4, dtype=torch.uint8, device="cuda")
            bc.cache.lkv_attend(layer, loop, bc.seqs, q, out, split_k=split_k, workspace=ws, mask_trace=mask,
                                v_rule=vla.VRULE_RUNNING, v_tau=tau)
            torch.cuda.synchronize()
            o = harness.out_f64(out)
            m = mask.cpu().numpy().view(np.uint32)
            # the call's far splits: split_k, at most the longest row's code pages (shorter rows leave splits empty)
            S = min(split_k, max((L - w.sink - w.tail + 31) // 32 for L in lengths))
            if split_k == 0:  # the library's choice, read back from the workspace size [rows][S + 1][d + 1] fp32
                S = ws_bytes // (n * w.n_heads * (w.head_dim + 1) * 4) - 1
            for b, L in enumerate(lengths):
                n_far = L - w.sink - w.tail
                for h in range(w.n_heads):
                    a = harness.cell_inputs(bc, b, layer, loop, h)
                    want, _, hot, n_cold, thr = oracle.cell_row_running(
                        a["q"], a["k_near"], a["v_near"], a["kc"], a["ks"], a["kz"], a["vc"], a["vs"], a["vz"],
                        a["sink"], a["tail"], a["kind"], tau, S)
                    assert np.abs(o[b, 0, h] - want).max() <= TOL, (layer, loop, b, h)
                    g = np.arange(n_far) // 32
                    s_far = (a["kz"][g] + a["ks"][g] * a["kc"]) @ a["q"] / math.sqrt(w.head_dim)
                    got = _bits(m[b, h], n_far)
                    near = np.abs(s_far - thr) <= BAND if a["kind"] != oracle.CELL_INT2 else np.zeros(n_far, bool)
                    assert np.array_equal(got[~near], hot[~near]), (layer, loop, b, h)
                    band_hits += int(near.sum())
                    cold += n_cold
    assert band_hits < 5
    if tau <= 2.0:
        assert cold > 0
    bc.cache.close()


def test_running_rule_infinite_tau_is_the_all_hot_reader():
    """LoopKV page, Sec. 3.3 and App. I: at tau = infinity the running rule keeps every far token hot, so the
    cell equals the reader of both V planes (the fixed rule at offset +inf): masks bit for bit, outputs to
    rounding.  The fixed rule lets the near block take a share of the far pages, the running rule keeps equal
    runs per far split (whose running maxima define its hot sets), so the online softmax references and the
    fp16 rounding of the value weights (relative 2^-12) differ: outputs within one bf16 step plus 1e-4 (the
    weights' rounding, ~3e-5 on cancelling channels), lse within 1e-5."""
    w = _cells_wl(3)
    bc = harness.build_cells(w, lengths=[133, 640, 1000], layers=(0, 1), plan=PLAN)
    for layer in (0, 1):
        for loop in range(4):
            for split_k in (1, 4):
                a, la, ma = _attend_cells(bc, layer, loop, math.inf, split_k)
                b, lb, mb = _attend_cells(bc, layer, loop, 4.0, split_k, v_rule=vla.VRULE_RUNNING, v_tau=math.inf)
                assert np.array_equal(ma, mb), (layer, loop, split_k)
                assert np.all(np.abs(a - b) <= np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -7 + 1e-4), (layer, loop)
                assert np.abs(la - lb).max() <= 1e-5, (layer, loop, split_k)
    bc.cache.close()


@pytest.mark.parametrize("tau", [5.0, 3.0])
def test_running_rule_hot_set_within_fixed_rule_when_tau_ln2_below_offset(tau):
    """When tau ln 2 <= offset the page's threshold max(m, m0) - tau ln 2 is never below the fixed m0 - offset,
    so every token the running rule keeps hot is hot under the fixed rule (both masks come from the same
    kernel's scores, so the inclusion is exact); with offset 4 and tau 5 or 3 the running rule turns cold
    at least as many tokens."""
    w = _cells_wl(3)
    lengths = [300, 777, 1000]
    bc = harness.build_cells(w, lengths=lengths, layers=(0,), plan=PLAN)
    strict = 0
    for loop in range(4):
        if PLAN[0, loop] == synth.CELL_INT2:
            continue
        for split_k in (1, 3):
            _, _, mf = _attend_cells(bc, 0, loop, 4.0, split_k)
            _, _, mr = _attend_cells(bc, 0, loop, 4.0, split_k, v_rule=vla.VRULE_RUNNING, v_tau=tau)
            for b, L in enumerate(lengths):
                n_far = L - w.sink - w.tail
                for h in range(w.n_heads):
                    f, r = _bits(mf[b, h], n_far), _bits(mr[b, h], n_far)
                    assert not np.any(r & ~f), (loop, split_k, b, h)
                    strict += int(np.sum(f & ~r))
    assert strict > 0
    bc.cache.close()


@pytest.mark.parametrize("rule,tau", [("fixed", 0.0), ("running", 14.0), ("running", 3.0)])
def test_cells_32_sink_keys(rule, tau):
    """The LoopKV page seeds its hot test with the largest of 32 sink scores (App. E); sink 32 spans two plain
    pages.  Lengths 161 (= 32 + 128 + 1: one far token), 420 and 1000; fixed rule (offset 4) and the running
    rule (tau 14 and 3) vs the oracle with the same far partition: outputs within 2e-2, hot masks bit-exact
    outside a 1e-4 band around each token's threshold."""
    w = synth.Workload("cells32", 3, 1, 4, 2, 128, 1000, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN,
                       1.0, quant=True, sink=32, tail=128)
    lengths = [161, 420, 1000]
    bc = harness.build_cells(w, lengths=lengths, layers=(0,), plan=PLAN[:1])
    band_hits = 0
    for loop in range(4):
        for split_k in (1, 3):
            if rule == "fixed":
                out, _, mask = _attend_cells(bc, 0, loop, 4.0, split_k)
            else:
                out, _, mask = _attend_cells(bc, 0, loop, 4.0, split_k, v_rule=vla.VRULE_RUNNING, v_tau=tau)
            S = min(split_k, max((L - w.sink - w.tail + 31) // 32 for L in lengths))
            for b, L in enumerate(lengths):
                n_far = L - w.sink - w.tail
                for h in range(w.n_heads):
                    a = harness.cell_inputs(bc, b, 0, loop, h)
                    if rule == "fixed":
                        want, _, hot, s_far, thr = harness.cell_oracle_row(bc, b, 0, loop, h, 4.0)
                        thr = np.full(n_far, thr)
                    else:
                        want, _, hot, _, thr = oracle.cell_row_running(
                            a["q"], a["k_near"], a["v_near"], a["kc"], a["ks"], a["kz"], a["vc"], a["vs"], a["vz"],
                            a["sink"], a["tail"], a["kind"], tau, S)
                        g = np.arange(n_far) // 32
                        s_far = (a["kz"][g] + a["ks"][g] * a["kc"]) @ a["q"] / math.sqrt(w.head_dim)
                    assert np.abs(out[b, 0, h] - want).max() <= TOL, (loop, split_k, b, h)
                    got = _bits(mask[b, h], n_far)
                    near = (np.abs(s_far - thr) <= BAND) if a["kind"] != oracle.CELL_INT2 else np.zeros(n_far, bool)
                    assert np.array_equal(got[~near], hot[~near]), (loop, split_k, b, h)
                    band_hits += int(near.sum())
    assert band_hits < 5
    bc.cache.close()
