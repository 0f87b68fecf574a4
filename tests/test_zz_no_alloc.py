"""The attend entry point that allocates nothing (lkv_attend_noalloc) against lkv_attend with a caller
workspace: same kernels, so the outputs must match bit for bit.  Two calls in a row on each cache, the second
with a smaller input (fewer sequences, fewer splits), so stale partials left in the library's fixed scratch by
the first call would show.  Plain decode and verify with split partials (RIPE page, Eq. (9) and Algorithm 1;
split merge of the LoopKV page, Sec. 3.4) and quantised cells, whose far splits and near block always write
partials (LoopKV page, Sec. 3.1-3.4)."""
import numpy as np
import pytest
import torch

import harness
import synth
import verify_attention_loop_amd as vla

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _pair(cache, layer, loop, seqs, q, mode, q_len, split_k, **kw):
    """(lkv_attend out, lse, mask) and (lkv_attend_noalloc out, lse, mask) of one call."""
    res = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], q_len, q.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
        extra = dict(kw)
        if "mask_trace" in kw:
            extra["mask_trace"] = torch.full_like(kw["mask_trace"], 0x5A5A5A5A)
        if noalloc:
            cache.lkv_attend_noalloc(layer, loop, seqs, q, out, q_len=q_len, mode=mode, split_k=split_k, lse=lse,
                                     **extra)
        else:
            wsb = cache.lkv_workspace_bytes(layer, loop, seqs, q_len=q_len, mode=mode, split_k=split_k)
            ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
            cache.lkv_attend(layer, loop, seqs, q, out, q_len=q_len, mode=mode, split_k=split_k, lse=lse,
                             workspace=ws, **extra)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone(), extra.get("mask_trace")))
    return res


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


@pytest.mark.parametrize("mode", ["decode", "verify"])
def test_noalloc_matches_workspace_call_plain(mode):
    k = 8 if mode == "verify" else 1
    md = vla.MODE_VERIFY if mode == "verify" else vla.MODE_DECODE
    w = synth.Workload("noalloc", 4, 1, 4, 6, 96, 300, synth.DT_BF16, "ripe", 20, k, 16, synth.MODE_RIPEN, 1.0)
    lengths = [300, 170, 45, 100]
    built = harness.build_plain(w, lengths=lengths, q_len=k, shuffle=True, poison=True)
    for loop in (0, w.n_loops - 1):
        q = harness.gpu_queries(built, 0, loop, k)
        # first call: every sequence, 5 splits; second: a smaller call, 2 sequences and 3 splits
        for seqs, split_k in ((built.seqs, 5), (built.seqs[1:3], 3)):
            qq = q[[built.seqs.index(s) for s in seqs]].contiguous()
            a, b = _pair(built.cache, 0, loop, seqs, qq, md, k, split_k)
            assert torch.isfinite(a[0].float()).all()
            _same(a, b)
    built.cache.close()


def test_noalloc_matches_workspace_call_cells():
    w = synth.Workload("noalloc_cells", 3, 1, 4, 4, 128, 460, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN,
                       1.0, quant=True, sink=4, tail=32)
    bc = harness.build_cells(w, lengths=[460, 300, 200], plan=np.array([[synth.CELL_INT4, synth.CELL_SHARED,
                                                                          synth.CELL_INT2, synth.CELL_INT4]]))
    words = (460 - 4 - 32 + 31) // 32
    for loop in range(4):
        q = torch.empty((3, 1, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        synth.gpu_q(q.data_ptr(), synth.DT_BF16, 0, [0, 1, 2], [L - 1 for L in bc.lengths], 0, loop, 1, w.n_heads,
                    w.head_dim, 1.0, torch.cuda.current_stream().cuda_stream)
        for seqs, split_k in ((bc.seqs, 6), (bc.seqs[1:], 2)):
            qq = q[[bc.seqs.index(s) for s in seqs]].contiguous()
            mask = torch.empty((len(seqs), w.n_heads, words), dtype=torch.int32, device="cuda")
            a, b = _pair(bc.cache, 0, loop, seqs, qq, vla.MODE_DECODE, 1, split_k, mask_trace=mask)
            assert torch.isfinite(a[0].float()).all()
            _same(a, b)
    bc.cache.close()


def test_noalloc_refuses_a_workspace_and_oversized_calls():
    w = synth.Workload("noalloc", 4, 1, 4, 6, 96, 300, synth.DT_BF16, "ripe", 20, 1, 16, synth.MODE_RIPEN, 1.0)
    built = harness.build_plain(w, lengths=[300, 200])
    q = harness.gpu_queries(built, 0, 0, 1)
    out = torch.empty_like(q)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        built.cache.lkv_attend_noalloc(0, 0, built.seqs, q, out, split_k=4, workspace=ws)
    built.cache.close()
