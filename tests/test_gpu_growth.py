"""Scores that keep growing page after page, through the C-ABI against the fp64 oracle.

Keys carry a ramp along a fixed direction u of their KV head and the queries point along u, so a column's maximum
score rises by up to ~4 natural units per 16-token page (bf16 inputs built here from a seeded numpy generator and
fed to both sides).  The MFMA kernels (verify, grouped-query decode) keep a lazy reference maximum and rescale what
they have accumulated only when a column's maximum passes it by a margin; with these inputs that happens every one
to four pages, and the columns grow at different rates (queries of a block, or query heads of a group, with
different norms), so waves hold columns that rescale next to columns that do not.  A missing or wrong rescale
leaves early pages weighted e^5 or more too high, far outside the 2e-2 bar; the VALU decode kernel runs the same
inputs.  Exact softmax attention is the definition (RIPE page, Eq. (9) for the plane of each key)."""
import numpy as np
import pytest

import harness
import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

R = 2  # loops: plane 0 is the attending loop's own, plane 1 the deepest


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _bf16(x):
    """numpy fp32 -> (bf16 CPU tensor, its exact fp64 values)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t, t.float().numpy().astype(np.float64)


def _inputs(seed, lengths, hq, hkv, d, q_len, rate=0.25):
    """K, V of both planes [b][plane][L][hkv][d] and queries [b][q_len][hq][d], bf16 (tensors and fp64 values).
    Key j of KV head h is 0.5 N(0,1) + rate j u_h; query column c (block row i, head h) is (0.35 + 0.65 c / n_cols)
    sqrt(d) u_{h // G} + 0.3 N(0,1), so its score climbs by ~rate (0.35..1) per position."""
    rng = np.random.default_rng(seed)
    G = hq // hkv
    u = rng.standard_normal((hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    ks, vs, qs = [], [], []
    for L in lengths:
        kb, vb = [], []
        for _plane in range(R):
            k = 0.5 * rng.standard_normal((L, hkv, d)) + rate * np.arange(L)[:, None, None] * u[None]
            kb.append(_bf16(k))
            vb.append(_bf16(rng.standard_normal((L, hkv, d))))
        ks.append(kb)
        vs.append(vb)
        n_cols = q_len * G
        q = np.empty((q_len, hq, d))
        for i in range(q_len):
            for h in range(hq):
                c = i * G + h % G
                q[i, h] = (0.35 + 0.65 * c / max(1, n_cols - 1)) * np.sqrt(d) * u[h // G] + \
                    0.3 * rng.standard_normal(d)
        qs.append(_bf16(q))
    return ks, vs, qs


def _build(lengths, hq, hkv, d, q_len, policy, W, ks, vs):
    w = synth.Workload("growth", len(lengths), 1, R, hq, d, max(lengths), synth.DT_BF16,
                       "ripe" if policy == vla.POLICY_RIPE else "full", W, q_len, 16, synth.MODE_PLAIN, 1.0,
                       n_kv_heads=hkv)
    n_pages = harness.pages_needed(w, lengths, (0,), list(range(R)), policy, W, q_len)
    cfg = vla.LoopCache.config(n_layers=1, n_loops=R, n_heads_q=hq, n_heads_kv=hkv, head_dim=d,
                               kv_dtype=synth.DT_BF16, policy=policy, window=W, max_seqs=len(lengths),
                               max_len=max(lengths), max_block=q_len, poison=1, shuffle_seed=0x5EED)
    cache = vla.LoopCache.on_device(cfg, n_pages)
    seqs = []
    for b, L in enumerate(lengths):
        s = cache.lkv_add_seq()
        seqs.append(s)
        order = [R - 1, 0] if policy == vla.POLICY_RIPE else [0, R - 1]
        for p in order:
            a = harness.ripe_window_start(L, q_len, W) if (policy == vla.POLICY_RIPE and p < R - 1) else 0
            kt, vt = ks[b][p][0][a:].cuda(), vs[b][p][0][a:].cuda()
            cache.lkv_append_plane(s, 0, p, a, kt, vt)
            if policy == vla.POLICY_RIPE and p == R - 1:
                cache.lkv_commit(s, L - q_len)
        if policy != vla.POLICY_RIPE:
            cache.lkv_commit(s, L - q_len)
    torch.cuda.synchronize()
    return cache, seqs


def _check(lengths, hq, hkv, d, q_len, policy, W, mode, split_ks, seed, kernel=vla.KERNEL_AUTO):
    ks, vs, qs = _inputs(seed, lengths, hq, hkv, d, q_len)
    cache, seqs = _build(lengths, hq, hkv, d, q_len, policy, W, ks, vs)
    G = hq // hkv
    want = np.zeros((len(lengths), q_len, hq, d))
    want_lse = np.zeros((len(lengths), q_len, hq))
    for b, L in enumerate(lengths):
        t0 = L - q_len
        for i in range(q_len):
            for h in range(hq):
                hk = h // G
                o, lse = oracle.attend_row(qs[b][1][i, h], ks[b][0][1][:, hk], vs[b][0][1][:, hk],
                                           ks[b][R - 1][1][:, hk], vs[b][R - 1][1][:, hk], t0 + i, t0, policy, 0, R,
                                           W)
                want[b, i, h], want_lse[b, i, h] = o, lse
    q = torch.stack([x[0] for x in qs]).cuda()
    for split_k in split_ks:
        out = torch.empty_like(q)
        lse = torch.empty((len(lengths), q_len, hq), dtype=torch.float32, device="cuda")
        wsb = cache.lkv_workspace_bytes(0, 0, seqs, q_len=q_len, mode=mode, split_k=split_k)
        ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
        cache.lkv_attend(0, 0, seqs, q, out, q_len=q_len, mode=mode, split_k=split_k, lse=lse, workspace=ws,
                         kernel=kernel)
        torch.cuda.synchronize()
        got = harness.out_f64(out)
        assert np.isfinite(got).all()
        assert np.abs(got - want).max() <= 2e-2, split_k
        assert np.abs(lse.cpu().numpy() - want_lse).max() <= 2e-2 * max(1.0, np.abs(want_lse).max() / 64), split_k
    cache.close()


@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 20)])
@pytest.mark.parametrize("hq,hkv,d", [(2, 2, 96), (8, 2, 64), (8, 2, 128)])
def test_verify_with_growing_scores(policy, W, hq, hkv, d):
    """q = 8 blocks: one query head per tile (hq = hkv), or the G = 4 heads of a KV head over two tiles."""
    _check([8, 97, 300], hq, hkv, d, 8, policy, W, vla.MODE_VERIFY, (1, 3), seed=11)


@pytest.mark.parametrize("kernel", ["tile", "valu"])
@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 20)])
@pytest.mark.parametrize("G,d", [(4, 64), (8, 128), (4, 256)])
def test_grouped_decode_with_growing_scores(policy, W, G, d, kernel):
    """q = 1 on a grouped-query cache: the MFMA tile kernel (G columns; two page buffers up to d = 128, one at
    d = 256) and the VALU decode kernel."""
    _check([1, 97, 300], 2 * G, 2, d, 1, policy, W, vla.MODE_DECODE, (1, 3), seed=12,
           kernel=vla.KERNEL_VALU if kernel == "valu" else vla.KERNEL_AUTO)


@pytest.mark.parametrize("policy,W", [(vla.POLICY_FULL, 0), (vla.POLICY_RIPE, 20)])
def test_multihead_decode_with_growing_scores(policy, W):
    """q = 1 on a multi-head cache (VALU decode kernel, split-K and the merge)."""
    _check([1, 97, 300], 4, 4, 96, 1, policy, W, vla.MODE_DECODE, (1, 4), seed=13)
