"""Quantised cells whose far scores keep growing page after page, through the C-ABI against the fp64 oracle.

The far key metadata carries a ramp: the zero point of code page p of head h is 0.3 N(0,1) + (r_h p - 3) u_h, with
u_h a unit vector, and the query points along u_h, so the head's far scores start about 3 natural units low and
climb by about r_h per 32-token page (0.6, 1.5, 3 and 4.5 units for the four heads).  The far loop keeps a lazy
reference maximum per row and rescales what it has accumulated only when a page's maximum passes that reference
(set 2 base-2 units above the maximum that last moved it), so the steep heads rescale on every page and the
shallow one every two or three pages: both the rescale and its skip run.  A missing or wrong rescale weights the
earlier pages e^0.6 or more off, far outside the 2e-2 bar.  The codes and metadata are
built here from a seeded numpy generator and fed to both sides.  INT2 and INT4 cells are checked under the fixed
rule at offset 1 (the first pages cold, later pages hot) and under the running rule, over 1 and 3 far splits and
the library's own count.  Definition: LoopKV page, Sec. 3.1-3.3 (a decoded key or value is z + sigma c, sink and
tail exact) and App. E Algorithm 1 (the running rule)."""
import math

import numpy as np
import pytest

import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

H, D, SINK, TAIL = 4, 128, 4, 32
RATES = (0.6, 1.5, 3.0, 4.5)  # natural units of score growth per code page, per head
PLAN = np.array([[synth.CELL_INT2, synth.CELL_INT4]], dtype=np.int8)  # loop 0 INT2, loop 1 INT4
LENGTHS = [SINK + TAIL + 32 * 20 + 7, SINK + TAIL + 32 * 9 + 31, SINK + TAIL + 1]
TOL = 2e-2
BAND = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t, t.float().numpy().astype(np.float64)


def _f16(x):
    """fp16 bits (int16) and their exact fp64 values."""
    h = np.asarray(x, dtype=np.float16)
    return h.view(np.int16), h.astype(np.float64)


def _cell_data(rng, L, bits, u):
    n_far = L - SINK - TAIL
    n_cp = (n_far + 31) // 32
    kc = rng.integers(0, 1 << bits, (n_cp * 32, H, D), dtype=np.uint8)
    vc = rng.integers(0, 1 << bits, (n_cp * 32, H, D), dtype=np.uint8)
    pages = np.arange(n_cp)[:, None, None]
    ramp = (np.array(RATES)[None, :, None] * pages - 3.0) * u[None]
    ks_bits, ks = _f16(0.02 + 0.05 * rng.random((n_cp, H, D)))
    kz_bits, kz = _f16(0.3 * rng.standard_normal((n_cp, H, D)) + ramp)
    vs_bits, vs = _f16(0.05 + 0.1 * rng.random((n_cp * 32, H, D // 32)))
    vz_bits, vz = _f16(0.5 * rng.standard_normal((n_cp * 32, H, D // 32)))
    return dict(n_far=n_far, n_cp=n_cp, kc=kc, vc=vc, km=np.stack([ks_bits, kz_bits], -1),
                vm=np.stack([vs_bits, vz_bits], -1), ks=ks, kz=kz, vs=vs, vz=vz)


def _near_pages(L):
    return len(set(range((SINK - 1) // 16 + 1)) | set(range((L - TAIL) // 16, (L - 1) // 16 + 1)))


@pytest.fixture(scope="module")
def built():
    rng = np.random.default_rng(0xC311)
    u = rng.standard_normal((H, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    n_near = sum(_near_pages(L) for L in LENGTHS) * 2
    n2 = n4 = sum((L - SINK - TAIL + 31) // 32 for L in LENGTHS)
    cfg = vla.LoopCache.config(n_layers=1, n_loops=2, n_heads_q=H, n_heads_kv=H, head_dim=D,
                               kv_dtype=synth.DT_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=len(LENGTHS),
                               max_len=max(LENGTHS), max_block=1, quant=1, sink=SINK, tail=TAIL)
    cache = vla.LoopCache.on_device(cfg, n_near, n4, n2)
    cache.lkv_set_plan(PLAN)
    seqs, data, near, qs = [], {}, {}, {}
    for b, L in enumerate(LENGTHS):
        s = cache.lkv_add_seq()
        seqs.append(s)
        for loop in (0, 1):
            kn = np.zeros((L, H, D))
            vn = np.zeros((L, H, D))
            for (p0, n) in ((0, SINK), (L - TAIL, TAIL)):
                kt, kv64 = _bf16(0.5 * rng.standard_normal((n, H, D)))
                vt, vv64 = _bf16(rng.standard_normal((n, H, D)))
                kn[p0:p0 + n], vn[p0:p0 + n] = kv64, vv64
                cache.lkv_append_plane(s, 0, loop, p0, kt.cuda(), vt.cuda())
            d = _cell_data(rng, L, 2 if loop == 0 else 4, u)
            cache.lkv_append_coded(s, 0, loop, 0, d["n_cp"], torch.from_numpy(d["kc"]).cuda(),
                                   torch.from_numpy(np.ascontiguousarray(d["km"])).cuda(),
                                   torch.from_numpy(d["vc"]).cuda(),
                                   torch.from_numpy(np.ascontiguousarray(d["vm"])).cuda())
            data[b, loop], near[b, loop] = d, (kn, vn)
            qs[b, loop] = _bf16(math.sqrt(D) * u + 0.3 * rng.standard_normal((H, D)))
    torch.cuda.synchronize()
    yield cache, seqs, data, near, qs
    cache.close()


def _query(built, b, loop, qmul):
    """The row's query (bf16 tensor, fp64 values), times qmul and rounded to bf16 again."""
    t, v = built[4][b, loop]
    return (t, v) if qmul == 1.0 else _bf16(v * qmul)


def _attend(built, loop, split_k, traced=True, qmul=1.0, **kw):
    """One call (with the hot-mask trace, or the untraced kernel the benchmark times); the far split count."""
    cache, seqs, _, _, _ = built
    n = len(seqs)
    q = torch.stack([_query(built, b, loop, qmul)[0] for b in range(n)])[:, None].cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full((n, 1, H), float("nan"), dtype=torch.float32, device="cuda")
    words = (max(LENGTHS) - SINK - TAIL + 31) // 32
    mask = torch.full((n, H, words), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    wsb = cache.lkv_workspace_bytes(0, loop, seqs, split_k=split_k)
    ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
    cache.lkv_attend(0, loop, seqs, q, out, split_k=split_k, lse=lse, workspace=ws,
                     mask_trace=mask if traced else None, **kw)
    torch.cuda.synchronize()
    S = split_k if split_k > 0 else wsb // (n * H * (D + 1) * 4) - 1  # the library's far splits, from the size
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), mask.cpu().numpy().view(np.uint32),
            min(S, max((L - SINK - TAIL + 31) // 32 for L in LENGTHS)))


def _oracle_args(built, b, loop, h, qmul=1.0):
    _, _, data, near, _ = built
    d = data[b, loop]
    n_far = d["n_far"]
    kn, vn = near[b, loop]
    return (_query(built, b, loop, qmul)[1][h], kn[:, h], vn[:, h], d["kc"][:n_far, h], d["ks"][:, h], d["kz"][:, h],
            d["vc"][:n_far, h], d["vs"][:n_far, h], d["vz"][:n_far, h], SINK, TAIL,
            oracle.CELL_INT2 if loop == 0 else oracle.CELL_INT4)


def _far_scores(args):
    q, kc, ks, kz = args[0], args[3], args[4], args[5]
    g = np.arange(kc.shape[0]) // 32
    return (kz[g] + ks[g] * kc) @ q / math.sqrt(D)


def _check(got_o, got_lse, got_mask, want_o, want_lse, hot, thr, args, loop):
    """Output and lse against the oracle; the INT4 cell's hot mask (loop 1) when a mask is given, returning the
    number of tokens inside the rounding band (INT2 cells read their whole codes)."""
    assert np.isfinite(got_o).all()
    assert np.abs(got_o - want_o).max() <= TOL
    assert abs(got_lse - want_lse) <= 2e-2 * max(1.0, abs(want_lse) / 64)
    if loop == 1 and got_mask is not None:
        n_far = args[3].shape[0]
        got = np.unpackbits(got_mask.view(np.uint8), bitorder="little")[:n_far]
        near = np.abs(_far_scores(args) - thr) <= BAND
        assert np.array_equal(got[~near], hot[~near])
        return int(near.sum())
    return 0


@pytest.mark.parametrize("split_k", [0, 1, 3])
@pytest.mark.parametrize("loop", [0, 1])
def test_growing_far_scores_fixed_rule(built, loop, split_k):
    """Fixed rule at offset 1: every row within 2e-2 of the oracle (lse within 2e-2 scaled by |lse| / 64, the
    scores reaching ~90), INT4 hot masks bit-exact outside the 1e-4 band, early pages cold and later pages hot;
    the untraced kernel (the one the benchmark times) within the same bar."""
    o, lse, mask, _ = _attend(built, loop, split_k, v_thresh_offset=1.0)
    o2, lse2, _, _ = _attend(built, loop, split_k, traced=False, v_thresh_offset=1.0)
    band, cold, hot_n = 0, 0, 0
    for b, L in enumerate(LENGTHS):
        for h in range(H):
            args = _oracle_args(built, b, loop, h)
            want, want_lse, hot, n_cold = oracle.cell_row(*args, 1.0)
            m0 = (args[1][:SINK] @ args[0] / math.sqrt(D)).max()
            band += _check(o[b, 0, h], lse[b, 0, h], mask[b, h], want, want_lse, hot, m0 - 1.0, args, loop)
            _check(o2[b, 0, h], lse2[b, 0, h], None, want, want_lse, hot, m0 - 1.0, args, 0)
            cold += n_cold
            hot_n += int(hot.sum())
    assert band < 3
    if loop == 1:
        assert cold > 0 and hot_n > 0


@pytest.mark.parametrize("split_k", [0, 1, 3])
@pytest.mark.parametrize("tau", [14.0, 2.0])
def test_growing_far_scores_running_rule(built, tau, split_k):
    """The running rule (App. E Algorithm 1) on the INT4 cell: each far split's running maximum climbs with the
    scores, so its threshold moves on every page; outputs and masks against the oracle's rule with the same
    page partition; the untraced kernel's outputs within the same bar."""
    o, lse, mask, S = _attend(built, 1, split_k, v_rule=vla.VRULE_RUNNING, v_tau=tau)
    o2, lse2, _, _ = _attend(built, 1, split_k, traced=False, v_rule=vla.VRULE_RUNNING, v_tau=tau)
    band = 0
    for b, L in enumerate(LENGTHS):
        for h in range(H):
            args = _oracle_args(built, b, 1, h)
            want, want_lse, hot, _, thr = oracle.cell_row_running(*args, tau, S)
            band += _check(o[b, 0, h], lse[b, 0, h], mask[b, h], want, want_lse, hot, thr, args, 1)
            _check(o2[b, 0, h], lse2[b, 0, h], None, want, want_lse, hot, thr, args, 0)
    assert band < 3


@pytest.mark.parametrize("qmul", [0.0, 2.0 ** -12, 700.0, 2.0 ** 12])
def test_int2_query_magnitudes(built, qmul):
    """The INT2 far loop carries the query as exact fp16 pairs under a power-of-two row scale that puts its
    largest element in [512, 1024): queries 2^-12, 700 and 2^12 times as large (700: a scale that is no power of
    two, rounded to bf16 on both sides) give every row within 2e-2 of the oracle, lse within 2e-2 of |lse| / 64;
    an all-zero query (no scale to take: every score 0, the mean of the row's values) the same."""
    o, lse, _, _ = _attend(built, 0, 0, traced=False, qmul=qmul, v_thresh_offset=1.0)
    for b, L in enumerate(LENGTHS):
        for h in range(H):
            args = _oracle_args(built, b, 0, h, qmul)
            want, want_lse, hot, _ = oracle.cell_row(*args, 1.0)
            _check(o[b, 0, h], lse[b, 0, h], None, want, want_lse, hot, 0.0, args, 0)
