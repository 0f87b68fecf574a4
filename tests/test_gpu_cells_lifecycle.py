"""The quantised-cache lifecycle on the GPU (LoopKV page, Sec. 3.4 and Sec. 4: when a page leaves the exact
window its cell's codec quantises it into the cell's pool and the bf16 block is released).

Sequences grow step by step: each step appends 1-4 new positions to every loop's exact plane, lkv_window_exit
encodes every far position that left the tail (re-encoding the partial last code page as it fills) and returns
exact pages no cell reads any more, and then every loop attends.  At every step and for every (sequence, loop,
head) the output, lse and hot mask equal the oracle's cell routine fed the oracle codec's codes of the same exact
values (page by page from the far start, the final loop's codes for a shared cell); the code pages read back
equal the oracle codec byte for byte; and the exact and code pages in use are exactly what the release rule
leaves."""
import numpy as np
import pytest

import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SINK, TAIL, H, D, R = 4, 64, 4, 128, 4
PLAN = [synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED, synth.CELL_INT4]
OKIND = {synth.CELL_INT4: oracle.CELL_INT4, synth.CELL_INT2: oracle.CELL_INT2, synth.CELL_SHARED: oracle.CELL_SHARED}
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _src(loop):
    return R - 1 if PLAN[loop] == synth.CELL_SHARED else loop


def _bits(loop):
    return 2 if PLAN[_src(loop)] == synth.CELL_INT2 else 4


class Exact:
    """Exact bf16 keys and values of every (sequence, loop), fp32 [max_len][H][D], from the generator."""

    def __init__(self, n_seqs, max_len):
        self.k, self.v = {}, {}
        for b in range(n_seqs):
            for r in range(R):
                for t, dst in ((synth.T_K, self.k), (synth.T_V, self.v)):
                    dst[b, r] = synth.f32_from_bf16(synth.kv(synth.DT_BF16, 0, t, b, 0, r, H, D, 0, max_len))


class Codes:
    """The oracle codec's codes of each far page of each (sequence, source loop, head), cached per complete
    page; the partial last page is encoded again from its valid tokens."""

    def __init__(self, ex):
        self.ex, self.done = ex, {}

    def page(self, b, src, h, p, n_valid):
        key = (b, src, h, p)
        if key in self.done and self.done[key][0] == n_valid:
            return self.done[key][1]
        a = SINK + 32 * p
        kc, km, vc, vm = oracle.kivi_encode(self.ex.k[b, src][a:a + n_valid, h], self.ex.v[b, src][a:a + n_valid, h],
                                            2 if PLAN[src] == synth.CELL_INT2 else 4)
        self.done[key] = (n_valid, (kc, km, vc, vm))
        return kc, km, vc, vm

    def far(self, b, src, h, n_far):
        """Codes and fp64 metadata of far positions [0, n_far) in the oracle cell routine's arrays."""
        n_pg = (n_far + 31) // 32
        kc = np.zeros((n_far, D), np.uint8)
        vc = np.zeros((n_far, D), np.uint8)
        ks, kz = np.zeros((n_pg, D)), np.zeros((n_pg, D))
        vs, vz = np.zeros((n_far, D // 32)), np.zeros((n_far, D // 32))
        for p in range(n_pg):
            f0, f1 = 32 * p, min(n_far, 32 * p + 32)
            c_k, m_k, c_v, m_v = self.page(b, src, h, p, f1 - f0)
            kc[f0:f1], vc[f0:f1] = c_k, c_v
            ks[p], kz[p] = synth.f64_from_f16(m_k[:, 0]), synth.f64_from_f16(m_k[:, 1])
            vs[f0:f1], vz[f0:f1] = synth.f64_from_f16(m_v[..., 0]), synth.f64_from_f16(m_v[..., 1])
        return kc, ks, kz, vc, vs, vz


def _expected_pages(lengths):
    """(exact pages, INT4 code pages, INT2 code pages) the release rule leaves."""
    plain = c4 = c2 = 0
    for L in lengths:
        fe = max(0, L - TAIL - SINK)
        whole = SINK + fe // 32 * 32
        for r in range(R):
            limit = SINK + fe if PLAN[r] == synth.CELL_SHARED else whole
            for P in range((L + 15) // 16):
                if not (P * 16 >= SINK and (P + 1) * 16 <= limit):
                    plain += 1
            if PLAN[r] == synth.CELL_INT4:
                c4 += (fe + 31) // 32
            elif PLAN[r] == synth.CELL_INT2:
                c2 += (fe + 31) // 32
    return plain, c4, c2


def test_cells_grow_through_window_exits():
    L0 = [140, 203]
    n_steps = 45
    rng = np.random.default_rng(21)
    max_len = max(L0) + 4 * n_steps + 16
    cfg = vla.LoopCache.config(n_layers=1, n_loops=R, n_heads_q=H, n_heads_kv=H, head_dim=D, kv_dtype=vla.DTYPE_BF16,
                               policy=vla.POLICY_FULL, window=0, max_seqs=len(L0), max_len=max_len, max_block=1,
                               quant=1, sink=SINK, tail=TAIL, poison=1, shuffle_seed=77)
    n_cp = (max_len + 31) // 32
    cache = vla.LoopCache.on_device(cfg, len(L0) * R * ((max_len + 15) // 16), len(L0) * 2 * n_cp,
                                    len(L0) * n_cp)
    cache.lkv_set_plan(np.array([PLAN], dtype=np.int8))
    ex = Exact(len(L0), max_len)
    codes = Codes(ex)
    st = torch.cuda.current_stream().cuda_stream
    seqs = [cache.lkv_add_seq() for _ in L0]
    lengths = [0] * len(L0)

    def append(b, n):
        p0 = lengths[b]
        for r in range(R):
            k = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
            v = torch.empty_like(k)
            synth.gpu_kv(k.data_ptr(), synth.DT_BF16, 0, synth.T_K, b, 0, r, H, D, p0, n, synth.MODE_PLAIN, R, 1.0, st)
            synth.gpu_kv(v.data_ptr(), synth.DT_BF16, 0, synth.T_V, b, 0, r, H, D, p0, n, synth.MODE_PLAIN, R, 1.0, st)
            cache.lkv_append_plane(seqs[b], 0, r, p0, k, v)
        lengths[b] += n

    for b, L in enumerate(L0):
        append(b, L)
        cache.lkv_window_exit(seqs[b])
    torch.cuda.synchronize()

    n_checked_codes = 0
    for step in range(n_steps + 1):
        if step > 0:
            for b in range(len(L0)):
                append(b, int(rng.integers(1, 5)))
            # the far history grew: attending before the window exit is refused
            with pytest.raises(vla.LkvError) as e:
                q = torch.zeros((len(L0), 1, H, D), dtype=torch.bfloat16, device="cuda")
                cache.lkv_attend(0, 0, seqs, q, torch.empty_like(q), split_k=1,
                                 workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
            assert e.value.status == vla.LKV_ESTATE
            for b in range(len(L0)):
                cache.lkv_window_exit(seqs[b])
        torch.cuda.synchronize()
        m = cache.lkv_mem_stats()
        assert (m["pages_in_use"], m["code4_in_use"], m["code2_in_use"]) == _expected_pages(lengths), step
        n_far = [L - SINK - TAIL for L in lengths]
        words = (max(n_far) + 31) // 32
        for loop in range(R):
            q = torch.empty((len(L0), 1, H, D), dtype=torch.bfloat16, device="cuda")
            synth.gpu_q(q.data_ptr(), synth.DT_BF16, 0, list(range(len(L0))), [L - 1 for L in lengths], 0, loop, 1, H,
                        D, 1.0, st)
            out = torch.empty_like(q)
            lse = torch.empty((len(L0), 1, H), dtype=torch.float32, device="cuda")
            mask = torch.empty((len(L0), H, words), dtype=torch.int32, device="cuda")
            split_k = 1 + step % 3
            wsb = cache.lkv_workspace_bytes(0, loop, seqs, split_k=split_k)
            ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
            cache.lkv_attend(0, loop, seqs, q, out, split_k=split_k, lse=lse, workspace=ws, mask_trace=mask,
                             v_thresh_offset=4.0)
            torch.cuda.synchronize()
            o = out.float().cpu().numpy().astype(np.float64)
            gl = lse.cpu().numpy()
            bits = np.unpackbits(mask.cpu().numpy().view(np.uint8), bitorder="little").reshape(len(L0), H, words * 32)
            qh = synth.f32_from_bf16(synth.q(synth.DT_BF16, 0, list(range(len(L0))), [L - 1 for L in lengths], 0, loop,
                                             1, H, D)).astype(np.float64)
            src = _src(loop)
            for b, L in enumerate(lengths):
                for h in range(H):
                    kc, ks, kz, vc, vs, vz = codes.far(b, src, h, n_far[b])
                    kn = ex.k[b, loop][:L, h].astype(np.float64)
                    vn = ex.v[b, loop][:L, h].astype(np.float64)
                    want, want_lse, hot, _ = oracle.cell_row(qh[b, 0, h], kn, vn, kc, ks, kz, vc, vs, vz, SINK, TAIL,
                                                             OKIND[PLAN[loop]], 4.0)
                    assert np.abs(o[b, 0, h] - want).max() <= TOL, (step, loop, b, h)
                    assert abs(gl[b, 0, h] - want_lse) <= 1e-3, (step, loop, b, h)
                    # hot bits: exact outside a 1e-4 band around the threshold
                    g = np.arange(n_far[b]) // 32
                    s_far = (kz[g] + ks[g] * kc) @ qh[b, 0, h] / np.sqrt(D)
                    thr = (kn[:SINK] @ qh[b, 0, h] / np.sqrt(D)).max() - 4.0
                    got_hot = bits[b, h, :n_far[b]].astype(bool)
                    bad = (got_hot != hot.astype(bool)) & (np.abs(s_far - thr) > 1e-4)
                    assert not bad.any(), (step, loop, b, h, np.flatnonzero(bad)[:5])
        # code pages read back equal the oracle codec byte for byte (every few steps)
        if step % 9 == 0:
            for b, L in enumerate(lengths):
                nf = n_far[b]
                n_pg = (nf + 31) // 32
                for r in range(R):
                    if PLAN[r] == synth.CELL_SHARED:
                        continue
                    kc = torch.empty((n_pg * 32, H, D), dtype=torch.uint8, device="cuda")
                    vc = torch.empty_like(kc)
                    km = torch.empty((n_pg, H, D, 2), dtype=torch.int16, device="cuda")
                    vm = torch.empty((n_pg * 32, H, D // 32, 2), dtype=torch.int16, device="cuda")
                    cache.lkv_read_coded(seqs[b], 0, r, 0, n_pg, kc, km, vc, vm)
                    torch.cuda.synchronize()
                    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
                    km = km.cpu().numpy().view(np.uint16)
                    vm = vm.cpu().numpy().view(np.uint16)
                    for h in range(H):
                        for p in range(n_pg):
                            nv = min(32, nf - 32 * p)
                            c_k, m_k, c_v, m_v = codes.page(b, r, h, p, nv)
                            sl = slice(32 * p, 32 * p + nv)
                            assert np.array_equal(kc[sl, h], c_k) and np.array_equal(vc[sl, h], c_v), (step, b, r, p)
                            assert np.array_equal(km[p, h], m_k) and np.array_equal(vm[sl, h], m_v), (step, b, r, p)
                            assert not kc[32 * p + nv:32 * p + 32, h].any() and not vm[32 * p + nv:32 * p + 32, h].any()
                            n_checked_codes += 1
    assert n_checked_codes > 0
    # positions that left the tail can no longer be appended or truncated away
    b = 0
    k = torch.zeros((1, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vla.LkvError) as e:
        cache.lkv_append_plane(seqs[b], 0, 0, SINK + 1, k, k)
    assert e.value.status == vla.LKV_ESTATE
    with pytest.raises(vla.LkvError) as e:
        cache.lkv_truncate(seqs[b], lengths[b] - 40)
    assert e.value.status in (vla.LKV_ESTATE, vla.LKV_EINVAL)
    cache.close()
