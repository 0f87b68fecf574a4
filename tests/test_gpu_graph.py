"""The attend calls are capturable: every device write the library issues is a kernel (block-table rows travel
as kernel arguments, trace buffers are cleared by a fill kernel), with no allocation and no copy from pageable
host memory.  A step of decode calls over a RIPE cache, a verify pass, and quantised-cell calls are captured
into a HIP graph and replayed three times, with eager work and synchronisation between the replays; every
replay must equal the eager result bit for bit."""
import numpy as np
import pytest

import harness
import synth
import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _replays_equal_eager(run, outs):
    """run(): issues the calls on the current stream.  Eager reference, then capture and three replays."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), (rep, i)
        run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("G", [1, 4])
def test_graph_decode_and_verify(G):
    n_heads, n_kv = (4, 4) if G == 1 else (8, 2)
    w = synth.Workload("graph", 3, 2, 4, n_heads, 64, 300, synth.DT_BF16, "ripe", 20, 1, 16, synth.MODE_RIPEN, 1.0,
                       n_kv_heads=n_kv)
    lengths = [40, 150, 300]
    built = harness.build_plain(w, lengths=lengths, layers=(0, 1), policy=vla.POLICY_RIPE, window=20, q_len=8,
                                shuffle=True, poison=True, max_block=8)
    calls = [(layer, loop) for loop in range(w.n_loops) for layer in range(2)]
    qs = [harness.gpu_queries(built, layer, loop, 1) for (layer, loop) in calls]
    outs = [torch.empty_like(q) for q in qs]
    wsb = built.cache.lkv_workspace_bytes(0, 0, built.seqs, split_k=2)
    ws = torch.empty(max(4, wsb), dtype=torch.uint8, device="cuda")
    # a verify pass over the last 8 positions of every sequence at loop 1
    qv = harness.gpu_queries(built, 0, 1, 8)
    ov = torch.empty_like(qv)
    wsv = torch.empty(max(4, built.cache.lkv_workspace_bytes(0, 1, built.seqs, q_len=8, mode=vla.MODE_VERIFY,
                                                             split_k=2)), dtype=torch.uint8, device="cuda")

    def run():
        for (layer, loop), q, o in zip(calls, qs, outs):
            built.cache.lkv_attend(layer, loop, built.seqs, q, o, split_k=2, workspace=ws)
        built.cache.lkv_attend(0, 1, built.seqs, qv, ov, q_len=8, mode=vla.MODE_VERIFY, split_k=2, workspace=wsv)

    outs = outs + [ov]

    _replays_equal_eager(run, outs)
    built.cache.close()


def test_graph_cells():
    w = synth.Workload("graphc", 2, 1, 4, 2, 128, 600, synth.DT_BF16, "full", 0, 1, 16, synth.MODE_PLAIN, 1.0,
                       quant=True, sink=4, tail=128)
    plan = np.array([[synth.CELL_INT4, synth.CELL_INT2, synth.CELL_SHARED, synth.CELL_INT4]], dtype=np.int8)
    bc = harness.build_cells(w, lengths=[300, 600], layers=(0,), plan=plan)
    qs = [harness.gpu_queries(bc, 0, loop, 1) for loop in range(4)]
    outs = [torch.empty_like(q) for q in qs]
    ws = torch.empty(bc.cache.lkv_workspace_bytes(0, 0, bc.seqs, split_k=3) + 4, dtype=torch.uint8, device="cuda")

    def run():
        for loop, (q, o) in enumerate(zip(qs, outs)):
            bc.cache.lkv_attend(0, loop, bc.seqs, q, o, split_k=3, workspace=ws, v_thresh_offset=1.0)

    _replays_equal_eager(run, outs)
    bc.cache.close()
