"""GPU window-exit codec (LoopKV page, Sec. 3.1 and 3.3) through the C-ABI: codes and fp16 metadata written by
lkv_encode_pages must equal the oracle's CPU codec byte for byte; lkv_read_coded inverts lkv_append_coded's
packing exactly; attention over GPU-encoded cells matches the oracle run on the oracle's own codes."""
import math

import numpy as np
import pytest

import harness
import oracle
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PLAN = np.array([[synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED, synth.CELL_INT4]], dtype=np.int8)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _cache(w, lengths, plan):
    n_cp = max((L - w.sink - w.tail + 31) // 32 for L in lengths)
    cfg = vla.LoopCache.config(n_layers=plan.shape[0], n_loops=plan.shape[1], n_heads_q=w.n_heads,
                               n_heads_kv=w.n_heads, head_dim=w.head_dim, kv_dtype=synth.DT_BF16,
                               policy=vla.POLICY_FULL, window=0, max_seqs=len(lengths), max_len=max(lengths),
                               max_block=1, quant=1, sink=w.sink, tail=w.tail)
    n_near = len(lengths) * plan.size * 10
    cache = vla.LoopCache.on_device(cfg, n_near, len(lengths) * plan.size * n_cp, len(lengths) * plan.size * n_cp)
    cache.lkv_set_plan(plan)
    return cache


def _far_values(w, b, layer, loop, L, seed=0):
    """Exact bf16 keys and values of the far positions [sink, L - tail) on the device and as fp32 on the host."""
    n_far = L - w.sink - w.tail
    st = torch.cuda.current_stream().cuda_stream
    k = torch.empty((n_far, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    synth.gpu_kv(k.data_ptr(), synth.DT_BF16, seed, synth.T_K, b, layer, loop, w.n_heads, w.head_dim, w.sink, n_far,
                 synth.MODE_PLAIN, w.n_loops, w.scale, st)
    synth.gpu_kv(v.data_ptr(), synth.DT_BF16, seed, synth.T_V, b, layer, loop, w.n_heads, w.head_dim, w.sink, n_far,
                 synth.MODE_PLAIN, w.n_loops, w.scale, st)
    hk = synth.f32_from_bf16(synth.kv(synth.DT_BF16, seed, synth.T_K, b, layer, loop, w.n_heads, w.head_dim, w.sink,
                                      n_far))
    hv = synth.f32_from_bf16(synth.kv(synth.DT_BF16, seed, synth.T_V, b, layer, loop, w.n_heads, w.head_dim, w.sink,
                                      n_far))
    return k, v, hk, hv


def _read(cache, w, seq, layer, loop, n_cp):
    H, D = w.n_heads, w.head_dim
    kc = torch.empty((n_cp * 32, H, D), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    km = torch.empty((n_cp, H, D, 2), dtype=torch.int16, device="cuda")
    vm = torch.empty((n_cp * 32, H, D // 32, 2), dtype=torch.int16, device="cuda")
    cache.lkv_read_coded(seq, layer, loop, 0, n_cp, kc, km, vc, vm)
    torch.cuda.synchronize()
    return (kc.cpu().numpy(), km.cpu().numpy().view(np.uint16), vc.cpu().numpy(), vm.cpu().numpy().view(np.uint16))


def _oracle_codes(hk, hv, bits):
    """Oracle codec page by page and head by head: arrays shaped like lkv_read_coded's (valid tokens only)."""
    n_far, H, D = hk.shape
    n_cp = (n_far + 31) // 32
    kc = np.zeros((n_far, H, D), np.uint8)
    vc = np.zeros((n_far, H, D), np.uint8)
    km = np.zeros((n_cp, H, D, 2), np.uint16)
    vm = np.zeros((n_far, H, D // 32, 2), np.uint16)
    for p in range(n_cp):
        t0, t1 = 32 * p, min(n_far, 32 * p + 32)
        for h in range(H):
            a, b_, c, d = oracle.kivi_encode(hk[t0:t1, h], hv[t0:t1, h], bits)
            kc[t0:t1, h], km[p, h], vc[t0:t1, h], vm[t0:t1, h] = a, b_, c, d
    return kc, km, vc, vm


@pytest.mark.parametrize("L", [133, 300, 1000])
def test_gpu_codec_is_byte_identical_to_the_oracle_codec(L):
    """Far lengths 1 (a single-token page), 168 (partial last page) and 868; INT4 and INT2 cells."""
    w = synth.Workload("codec", 1, 1, 4, 2, 128, L, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN, 1.0,
                       quant=True, sink=4, tail=128)
    cache = _cache(w, [L], PLAN)
    seq = cache.lkv_add_seq()
    n_far = L - w.sink - w.tail
    n_cp = (n_far + 31) // 32
    for loop in (0, 1, 3):
        bits = 2 if PLAN[0, loop] == synth.CELL_INT2 else 4
        k, v, hk, hv = _far_values(w, 0, 0, loop, L)
        cache.lkv_encode_pages(seq, 0, loop, 0, n_cp, n_far - 32 * (n_cp - 1), k, v)
        gkc, gkm, gvc, gvm = _read(cache, w, seq, 0, loop, n_cp)
        okc, okm, ovc, ovm = _oracle_codes(hk, hv, bits)
        np.testing.assert_array_equal(gkc[:n_far], okc)
        np.testing.assert_array_equal(gvc[:n_far], ovc)
        np.testing.assert_array_equal(gkm, okm)
        np.testing.assert_array_equal(gvm[:n_far], ovm)
        assert not gkc[n_far:].any() and not gvc[n_far:].any() and not gvm[n_far:].any()
    with pytest.raises(vla.LkvError) as e:
        cache.lkv_encode_pages(seq, 0, 2, 0, n_cp, 1, k, v)  # shared cell: stores nothing
    assert e.value.status == vla.LKV_EINVAL
    cache.close()


def test_read_coded_inverts_the_packing():
    w = synth.Workload("codec", 2, 1, 4, 2, 128, 700, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN, 1.0,
                       quant=True, sink=4, tail=128)
    cache = _cache(w, [700], PLAN)
    seq = cache.lkv_add_seq()
    n_cp = (700 - 132 + 31) // 32
    st = torch.cuda.current_stream().cuda_stream
    for loop in (0, 1):
        bits = 2 if PLAN[0, loop] == synth.CELL_INT2 else 4
        H, D = w.n_heads, w.head_dim
        kc = torch.empty((n_cp * 32, H, D), dtype=torch.uint8, device="cuda")
        vc = torch.empty_like(kc)
        km = torch.empty((n_cp, H, D, 2), dtype=torch.int16, device="cuda")
        vm = torch.empty((n_cp * 32, H, D // 32, 2), dtype=torch.int16, device="cuda")
        synth.gpu_codes(kc.data_ptr(), 0, synth.T_KCODE, 0, 0, loop, H, D, 4, n_cp * 32, bits, st)
        synth.gpu_codes(vc.data_ptr(), 0, synth.T_VCODE, 0, 0, loop, H, D, 4, n_cp * 32, bits, st)
        synth.gpu_meta(km.data_ptr(), 0, 0, 0, 0, loop, H, D, 0, n_cp, bits, st)
        synth.gpu_meta(vm.data_ptr(), 0, 1, 0, 0, loop, H, D // 32, 0, n_cp * 32, bits, st)
        cache.lkv_append_coded(seq, 0, loop, 0, n_cp, kc, km, vc, vm)
        got = _read(cache, w, seq, 0, loop, n_cp)
        for a, b in zip(got, (kc, km, vc, vm)):
            np.testing.assert_array_equal(a, b.cpu().numpy().view(a.dtype))
    cache.close()


@pytest.mark.parametrize("offset", [4.0, 1.0])
def test_attention_over_gpu_encoded_cells(offset):
    """Cells whose far pages were encoded on the GPU from exact keys and values: attention and hot masks match
    the oracle's cell routine on the oracle codec's codes (max-abs 2e-2; masks exact outside a 1e-4 band)."""
    w = synth.Workload("codec", 2, 1, 4, 2, 128, 600, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN, 1.0,
                       quant=True, sink=4, tail=128)
    lengths = [600, 333]
    cache = _cache(w, lengths, PLAN)
    st = torch.cuda.current_stream().cuda_stream
    host = {}
    seqs = []
    for b, L in enumerate(lengths):
        s = cache.lkv_add_seq()
        seqs.append(s)
        n_far = L - w.sink - w.tail
        n_cp = (n_far + 31) // 32
        for loop in range(4):
            for (p0, n) in ((0, w.sink), (L - w.tail, w.tail)):
                kk = torch.empty((n, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
                vv = torch.empty_like(kk)
                synth.gpu_kv(kk.data_ptr(), synth.DT_BF16, 0, synth.T_K, b, 0, loop, w.n_heads, w.head_dim, p0, n,
                             synth.MODE_PLAIN, 4, 1.0, st)
                synth.gpu_kv(vv.data_ptr(), synth.DT_BF16, 0, synth.T_V, b, 0, loop, w.n_heads, w.head_dim, p0, n,
                             synth.MODE_PLAIN, 4, 1.0, st)
                cache.lkv_append_plane(s, 0, loop, p0, kk, vv)
            if PLAN[0, loop] == synth.CELL_SHARED:
                continue
            k, v, hk, hv = _far_values(w, b, 0, loop, L)
            cache.lkv_encode_pages(s, 0, loop, 0, n_cp, n_far - 32 * (n_cp - 1), k, v)
            host[(b, loop)] = (hk, hv)
    torch.cuda.synchronize()
    bc = harness.BuiltCells(cache, w, seqs, lengths, [0], PLAN)
    D = w.head_dim
    for loop in range(4):
        src = 3 if PLAN[0, loop] == synth.CELL_SHARED else loop
        bits = 2 if PLAN[0, src] == synth.CELL_INT2 else 4
        kind = {synth.CELL_INT4: oracle.CELL_INT4, synth.CELL_INT2: oracle.CELL_INT2,
                synth.CELL_SHARED: oracle.CELL_SHARED}[int(PLAN[0, loop])]
        q = harness.gpu_queries(bc, 0, loop, 1)
        out = torch.empty_like(q)
        words = (max(lengths) - 132 + 31) // 32
        mask = torch.empty((2, w.n_heads, words), dtype=torch.int32, device="cuda")
        ws = torch.empty(cache.lkv_workspace_bytes(0, loop, seqs) + 4, dtype=torch.uint8, device="cuda")
        cache.lkv_attend(0, loop, seqs, q, out, v_thresh_offset=offset, workspace=ws, mask_trace=mask)
        torch.cuda.synchronize()
        o = harness.out_f64(out)
        m = mask.cpu().numpy().view(np.uint32)
        for b, L in enumerate(lengths):
            hk, hv = host[(b, src)]
            n_far = L - 132
            okc, okm, ovc, ovm = _oracle_codes(hk, hv, bits)
            for h in range(w.n_heads):
                a = harness.cell_inputs(bc, b, 0, loop, h)  # query, sink and tail from the generator
                f64 = np.vectorize(oracle.f32_from_f16, otypes=[np.float64])
                ks, kz = f64(okm[:, h, :, 0]), f64(okm[:, h, :, 1])
                vs, vz = f64(ovm[:, h, :, 0]), f64(ovm[:, h, :, 1])
                want, _, hot, _ = oracle.cell_row(a["q"], a["k_near"], a["v_near"], okc[:, h], ks, kz, ovc[:, h], vs,
                                                  vz, 4, 128, kind, offset)
                assert np.abs(o[b, 0, h] - want).max() <= 2e-2, (loop, b, h)
                g = np.arange(n_far) // 32
                s_far = (kz[g] + ks[g] * okc[:, h]) @ a["q"] / math.sqrt(D)
                thr = (a["k_near"][:4] @ a["q"] / math.sqrt(D)).max() - offset
                got = np.unpackbits(m[b, h].view(np.uint8), bitorder="little")[:n_far]
                near = np.abs(s_far - thr) <= 1e-4
                assert np.array_equal(got[~near], hot[~near])
    cache.close()
