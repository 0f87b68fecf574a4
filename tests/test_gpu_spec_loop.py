"""A multi-step synthetic run of the RIPE page's self-speculative step (Sec. 4, Algorithm 1) on the GPU: draft
passes, block verification at every loop, seeded acceptance, commit and truncate, repeated.  At every step the
verify outputs equal the oracle's one-token-at-a-time decoding of the same tokens (Prop. 1, W >= gamma), the
draft outputs equal the oracle's draft rows, the logical bytes follow Eq. (10) and the pages in use are exactly
the deepest plane of every position plus the window ring."""
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


def _host_planes(sl, b, layer, loop, hk, n):
    R = sl.w.n_loops
    return (sl.host_kv(synth.T_K, b, layer, loop, hk, n), sl.host_kv(synth.T_V, b, layer, loop, hk, n),
            sl.host_kv(synth.T_K, b, layer, R - 1, hk, n), sl.host_kv(synth.T_V, b, layer, R - 1, hk, n))


@pytest.mark.parametrize("max_gamma,W,G", [(7, 7, 1), (6, 16, 2), (7, 3, 1)])
def test_self_speculative_loop(max_gamma, W, G):
    """Ten steps with a block length gamma drawn per step in [1, max_gamma] (Algorithm 1 takes gamma <= W; the
    W = 3 case also draws gamma > W on purpose).  Where W >= gamma, every verify row equals the oracle's
    sequential decoding of the same token (Prop. 1).  Where W < gamma, the verify rows equal the oracle's block
    pass (block tokens read plane r of earlier block tokens) and, as the discussion of Prop. 1 predicts, differ
    from sequential decoding for the rows that see an earlier block token more than W positions back."""
    w = synth.Workload("spec", 3, 2, 4, 2 * G, 64, 0, synth.DT_F32, "ripe", W, max_gamma + 1, 16, synth.MODE_RIPEN,
                       0.25, n_kv_heads=2)
    sl = harness.SpecLoop(w, [23, 40, 61], max_gamma=max_gamma, d=2, window=W, seed=max_gamma + W)
    R, H, HK, D = w.n_loops, w.n_heads, w.hkv, w.head_dim
    group = H // HK
    es = 4
    gammas = []
    for step in range(10):
        gamma = sl.draw_gamma()
        gammas.append(gamma)
        lens = list(sl.lengths)
        # ---- draft passes (cached positions at plane R, the block from scratch)
        for i in sorted({1, gamma}):
            res = sl.draft_pass(i)
            torch.cuda.synchronize()
            layer, loop = 1, 1
            out = harness.out_f64(res[(layer, loop)][0])
            for b, L in enumerate(lens):
                for h in (0, H - 1):
                    hk = h // group
                    n = L + i
                    ko, vo, kd, vd = _host_planes(sl, b, layer, loop, hk, n)
                    sk = synth.kv(w.dtype, 0, synth.T_DRAFTK, sl._row(b, L), layer, loop, HK, D, L, i,
                                  synth.MODE_PLAIN, R, w.scale, heads=[hk])[:, 0]
                    sv = synth.kv(w.dtype, 0, synth.T_DRAFTV, sl._row(b, L), layer, loop, HK, D, L, i,
                                  synth.MODE_PLAIN, R, w.scale, heads=[hk])[:, 0]
                    ko[L:], vo[L:] = harness.to_f64(sk, w.dtype), harness.to_f64(sv, w.dtype)
                    q = sl.query(b, layer, loop, h, L + i - 1, salt=1)
                    want, _ = oracle.attend_row(q, ko, vo, kd, vd, n - 1, L, oracle.RIPE, loop, R, 0)
                    assert np.abs(out[b, 0, h] - want).max() <= 1e-5, (step, i, b, h)
        # ---- verify the block [x, drafts] at every loop
        outs = sl.verify_pass(gamma)
        torch.cuda.synchronize()
        n_dep = 0
        for (layer, loop), o in outs.items():
            if layer == 0 and loop not in (0, R - 1):
                continue
            got = harness.out_f64(o)
            for b, L in enumerate(lens):
                n = L + gamma + 1
                for hk in range(HK):
                    ko, vo, kd, vd = _host_planes(sl, b, layer, loop, hk, n)
                    for h in range(hk * group, hk * group + group):
                        for i in range(gamma + 1):
                            t = L + i
                            q = sl.query(b, layer, loop, h, t)
                            seq, _ = oracle.attend_row(q, ko[:t + 1], vo[:t + 1], kd[:t + 1], vd[:t + 1], t, t,
                                                       oracle.RIPE, loop, R, W)
                            if W >= gamma:  # Prop. 1: the block pass is sequential decoding
                                assert np.abs(got[b, i, h] - seq).max() <= 1e-5, (step, layer, loop, b, i, h)
                                continue
                            blk, _ = oracle.attend_row(q, ko[:t + 1], vo[:t + 1], kd[:t + 1], vd[:t + 1], t, L,
                                                       oracle.RIPE, loop, R, W)
                            assert np.abs(got[b, i, h] - blk).max() <= 1e-5, (step, layer, loop, b, i, h)
                            if i > W and loop != R - 1:  # an earlier block token lies more than W back
                                assert np.abs(got[b, i, h] - seq).max() > 1e-3, (step, layer, loop, b, i, h)
                                n_dep += 1
        if W < gamma:
            assert n_dep > 0
        # ---- accept, commit, truncate; accounting
        sl.accept(gamma)
        m = sl.cache.lkv_mem_stats()
        bpt = 2 * HK * D * es
        assert m["logical_bytes"] == sum(bpt * w.n_layers * (L + (R - 1) * min(W, L)) for L in sl.lengths)
        assert m["pages_in_use"] == sl.expected_pages()
    assert len(set(gammas)) > 1  # block lengths did vary
    if W < max_gamma:
        assert any(g > W for g in gammas) and any(g <= W for g in gammas)
    sl.cache.close()
