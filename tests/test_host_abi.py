"""Host-side tests of the C-ABI library: exports, allocator, tables, window ring,
accounting and error paths.  No GPU: only calls that do host bookkeeping are made,
on arenas whose addresses are never dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import verify_attention_loop_amd as vla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vla.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return vla.load()


def test_library_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "loopattn.h")).read()
    declared = set(re.findall(r"^(?:lkv_status|const char\*)\s+(lkv_\w+)\(", hdr, flags=re.M))
    assert declared, "no declarations parsed"
    assert declared == set(vla.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_probe_read_checks_arguments_before_any_launch(lib):
    """The read probe refuses NULL pointers and sizes that are not a positive multiple of its chunk, on
    the host (no device call is made for these)."""
    assert vla.PROBE_CHUNK == 16384
    buf, sink = 1 << 40, 1 << 41  # never dereferenced
    for nbytes in (0, 100, vla.PROBE_CHUNK - 16, vla.PROBE_CHUNK + 16, 3 * vla.PROBE_CHUNK // 2):
        assert lib.lkv_probe_read(buf, nbytes, sink, 0, 0, 0) == vla.LKV_EINVAL, nbytes
    assert lib.lkv_probe_read(0, vla.PROBE_CHUNK, sink, 0, 0, 0) == vla.LKV_EINVAL
    assert lib.lkv_probe_read(buf, vla.PROBE_CHUNK, 0, 0, 0, 0) == vla.LKV_EINVAL
    assert lib.lkv_probe_read(buf, vla.PROBE_CHUNK << 31, sink, 0, 0, 0) == vla.LKV_EINVAL


class HostArenas:
    """Fake device arenas: host buffers whose addresses the host-only calls never read."""

    def __init__(self, cfg, n_pages, n4=0, n2=0):
        s = vla.LoopCache.sizes(cfg)
        self.meta = np.zeros(max(256, s.meta_bytes), dtype=np.uint8)
        base = 1 << 40  # never dereferenced
        self.ar = vla.lkv_arenas(base, n_pages * s.page_bytes, base + (1 << 38), n4 * s.code4_page_bytes,
                                 base + (1 << 39), n2 * s.code2_page_bytes, self.meta.ctypes.data, s.meta_bytes)
        self.sizes = s


def make(n_pages=64, **kw):
    base = dict(n_layers=2, n_loops=4, n_heads_q=2, n_heads_kv=2, head_dim=64, kv_dtype=vla.DTYPE_BF16,
                policy=vla.POLICY_RIPE, window=16, max_seqs=4, max_len=256, max_block=8)
    base.update(kw)
    cfg = vla.LoopCache.config(**base)
    ha = HostArenas(cfg, n_pages)
    c = vla.LoopCache(cfg, ha.ar, 0)
    c._host_arenas = ha
    return c


def test_page_size_and_table_bytes(lib):
    cfg = vla.LoopCache.config(n_layers=4, n_loops=32, n_heads_q=55, n_heads_kv=55, head_dim=96,
                               kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_RIPE, window=64, max_seqs=32,
                               max_len=1024, max_block=8)
    s = vla.LoopCache.sizes(cfg)
    assert s.page_bytes == 2 * 55 * 16 * 96 * 2
    # deepest plane: 64 pages per sequence; window ring: ceil((64 + 8) / 16) + 1 = 6 pages
    row = lambda n: (32 * n * 4 + 255) // 256 * 256
    assert s.meta_bytes == 4 * (row(64) + 31 * row(6))


def test_sequence_slots_and_errors_leave_handle_usable(lib):
    c = make()
    ids = [c.lkv_add_seq() for _ in range(4)]
    assert ids == [0, 1, 2, 3]
    with pytest.raises(vla.LkvError) as e:
        c.lkv_add_seq()
    assert e.value.status == vla.LKV_ENOMEM
    c.lkv_free_seq(2)
    assert c.lkv_add_seq() == 2
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(0, 5, 0, 0, 4)  # bad layer
    assert e.value.status == vla.LKV_EINVAL
    c.lkv_reserve(0, 0, 3, 0, 20)
    assert c.lkv_seq_info(0) == (20, 0)


def test_append_without_gap_and_pool_exhaustion(lib):
    c = make(n_pages=5, policy=vla.POLICY_FULL)
    s = c.lkv_add_seq()
    c.lkv_reserve(s, 0, 1, 0, 40)  # 3 pages
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(s, 0, 1, 50, 4)  # gap after position 40
    assert e.value.status == vla.LKV_ESTATE
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(s, 0, 2, 0, 48)  # 3 more pages, only 2 free
    assert e.value.status == vla.LKV_ENOMEM
    assert c.lkv_mem_stats()["pages_in_use"] == 3  # the failed call allocated nothing
    c.lkv_reserve(s, 0, 2, 0, 32)
    assert c.lkv_mem_stats()["pages_in_use"] == 5


def test_window_ring_commit_and_ewindow(lib):
    """RIPE page, Sec. 4 and Algorithm 1 (window slide): non-deepest planes are kept for the last W positions only;
    committing drops the planes of positions older than W, and their pages return to the pool."""
    W = 16
    c = make(n_pages=200, window=W, max_block=8)
    s = c.lkv_add_seq()
    R = 4
    # prefill 100 positions of the deepest plane, window planes only for the last W
    c.lkv_reserve(s, 0, R - 1, 0, 100)
    c.lkv_commit(s, 100)
    for p in range(R - 1):
        with pytest.raises(vla.LkvError) as e:
            c.lkv_reserve(s, 0, p, 100 - W - 1, 5)
        assert e.value.status == vla.LKV_EWINDOW
        c.lkv_reserve(s, 0, p, 100 - W, W)
    used = c.lkv_mem_stats()["pages_in_use"]
    # decode 200 more tokens one at a time: ring pages are recycled, the deepest plane grows
    for n in range(100, 250):
        for p in range(R):
            c.lkv_reserve(s, 0, p, n, 1)
        c.lkv_commit(s, n + 1)
    st = c.lkv_mem_stats()
    deep_pages = (250 + 15) // 16
    ring_pages = st["pages_in_use"] - deep_pages
    assert ring_pages <= (R - 1) * ((W + 8 + 15) // 16 + 1)
    assert st["pages_in_use"] > used
    # a position older than the window can no longer be written in a non-deepest plane
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(s, 0, 0, 250 - W - 1, 1)
    assert e.value.status == vla.LKV_EWINDOW


def test_truncate_rolls_back_a_block(lib):
    c = make(n_pages=100, window=16, max_block=8)
    s = c.lkv_add_seq()
    for p in range(4):
        c.lkv_reserve(s, 0, p, 0 if p == 3 else 0, 40)
    c.lkv_commit(s, 32)
    for p in range(4):
        c.lkv_reserve(s, 0, p, 40, 8)  # block of 8
    assert c.lkv_seq_info(s) == (48, 32)
    before = c.lkv_mem_stats()["pages_in_use"]
    c.lkv_truncate(s, 41)  # accept 1 token of the block
    assert c.lkv_seq_info(s) == (41, 32)
    assert c.lkv_mem_stats()["pages_in_use"] <= before
    with pytest.raises(vla.LkvError) as e:
        c.lkv_truncate(s, 30)  # below committed
    assert e.value.status == vla.LKV_EINVAL


def test_logical_bytes_follow_eq3_and_eq10(lib):
    """RIPE page, Eq. (3) and Eq. (10) for the core layers: the full cache holds R planes per position,
    RIPE the deepest plane plus R-1 planes for min(W, L) positions."""
    for policy in (vla.POLICY_FULL, vla.POLICY_RIPE):
        c = make(n_pages=400, policy=policy, window=16, n_layers=2, n_loops=4, head_dim=64, n_heads_kv=2,
                 n_heads_q=2)
        b = oracle.kv_bytes_per_layer_token(2, 64)
        for L in (5, 16, 100):
            s = c.lkv_add_seq()
            c.lkv_reserve(s, 0, 3, 0, L)
            got = c.lkv_mem_stats()["logical_bytes"]
            want = (oracle.mem_full(L, b, 0, 0, 2, 4) if policy == vla.POLICY_FULL
                    else oracle.mem_ripe(L, b, 0, 0, 2, 4, 16))
            assert got == want, (policy, L)
            c.lkv_free_seq(s)


def test_debug_resolve_matches_policy_and_tables(lib):
    """The host index function names the plane of Eq. (9) (with the block rule) and the physical page
    that the block table holds for it."""
    R, W = 4, 16
    c = make(n_pages=300, window=W, max_block=8, shuffle_seed=7)
    s = c.lkv_add_seq()
    L = 90
    c.lkv_reserve(s, 0, R - 1, 0, L)
    c.lkv_commit(s, L - 8)
    for p in range(R - 1):
        c.lkv_reserve(s, 0, p, L - 8 - W, W + 8)
    t0 = L - 8
    phys_seen = {}
    for r in range(R):
        for t in range(t0, L):
            for j in range(t + 1):
                plane, phys, slot = c.lkv_debug_resolve(s, 0, r, t, t0, j)
                assert plane == oracle.oracle_plane(oracle.RIPE, r, R, t, t0, j, W)
                assert slot == j % 16 and phys >= 0
                key = (plane, j // 16)
                assert phys_seen.setdefault(key, phys) == phys
    # distinct (plane, page) pairs never share a physical page
    assert len(set(phys_seen.values())) == len(phys_seen)


def test_shuffled_pool_hands_out_a_permutation(lib):
    c = make(n_pages=64, policy=vla.POLICY_FULL, shuffle_seed=123, max_len=1024)
    s = c.lkv_add_seq()
    c.lkv_reserve(s, 0, 0, 0, 1024)
    phys = [c.lkv_debug_resolve(s, 0, 0, 1023, 1023, j * 16)[1] for j in range(64)]
    assert sorted(phys) == list(range(64)) and phys != list(range(64))


def test_config_validation(lib):
    cfg = vla.LoopCache.config(n_layers=1, n_loops=4, n_heads_q=3, n_heads_kv=2, head_dim=64,
                               kv_dtype=vla.DTYPE_BF16, policy=0, window=0, max_seqs=1, max_len=16, max_block=1)
    with pytest.raises(vla.LkvError):
        vla.LoopCache.sizes(cfg)  # heads not divisible
    cfg.n_heads_q = 2
    cfg.head_dim = 80
    with pytest.raises(vla.LkvError):
        vla.LoopCache.sizes(cfg)
    cfg.head_dim = 64
    cfg.max_block = 17
    with pytest.raises(vla.LkvError):
        vla.LoopCache.sizes(cfg)
    cfg.max_block = 1
    cfg.head_dim = 256  # bf16 plain planes take head dim 256 (the Dory shape) ...
    assert vla.LoopCache.sizes(cfg).page_bytes == 2 * 2 * 16 * 256 * 2
    cfg.kv_dtype = vla.DTYPE_F32  # ... fp32 caches do not
    with pytest.raises(vla.LkvError):
        vla.LoopCache.sizes(cfg)
    cfg.kv_dtype = vla.DTYPE_BF16
    cfg.quant, cfg.sink, cfg.tail = 1, 4, 8  # nor do quantised cells
    with pytest.raises(vla.LkvError):
        vla.LoopCache.sizes(cfg)


def test_sink_range(lib):
    """Quantised cells take 1..64 exact sink positions (the LoopKV page's own rule seeds m0 from 32)."""
    def cfg(sink):
        return vla.LoopCache.config(n_layers=1, n_loops=2, n_heads_q=4, n_heads_kv=4, head_dim=128,
                                    kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=2,
                                    max_len=400, max_block=1, quant=1, sink=sink, tail=128)
    for ok in (1, 4, 32, 64):
        vla.LoopCache.sizes(cfg(ok))
    for bad in (0, 65, -1):
        with pytest.raises(vla.LkvError):
            vla.LoopCache.sizes(cfg(bad))


def test_plan_rules(lib):
    cfg = vla.LoopCache.config(n_layers=2, n_loops=4, n_heads_q=16, n_heads_kv=16, head_dim=128,
                               kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=2,
                               max_len=400, max_block=1, quant=1, sink=4, tail=128)
    ha = HostArenas(cfg, 10, 10, 10)
    c = vla.LoopCache(cfg, ha.ar, 0)
    plan = np.full((2, 4), vla.CELL_INT4, dtype=np.int8)
    plan[0, 3] = vla.CELL_SHARED
    with pytest.raises(vla.LkvError) as e:
        c.lkv_set_plan(plan)  # the final loop is the source of shared cells
    assert e.value.status == vla.LKV_EINVAL
    plan[0, 3] = vla.CELL_INT4
    plan[0, 1] = vla.CELL_SHARED
    plan[1, 0] = vla.CELL_INT2
    c.lkv_set_plan(plan)
    assert ha.sizes.code4_page_bytes == 16 * 160 * 32  # LoopKV page App. C: 2.5 KiB per token and layer
    assert ha.sizes.code2_page_bytes == 16 * 96 * 32   # 1.5 KiB


def test_quant_workspace_matches_the_cell_split_rule(lib):
    """lkv_workspace_bytes sizes a quantised-cell call by the split rule lkv_attend uses for every cell kind and
    V-precision rule: min(64, 1280 / (seqs * heads) - 1) far splits (at least 1), at most one per code page, plus
    the near part."""
    cfg = vla.LoopCache.config(n_layers=1, n_loops=2, n_heads_q=4, n_heads_kv=4, head_dim=128,
                               kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=3, max_len=2000,
                               max_block=1, quant=1, sink=4, tail=128)
    s = vla.LoopCache.sizes(cfg)
    meta = np.zeros(max(256, s.meta_bytes), dtype=np.uint8)
    base = 1 << 40
    ar = vla.lkv_arenas(base, 256 * s.page_bytes, base + (1 << 38), 256 * s.code4_page_bytes, base + (1 << 39),
                        256 * s.code2_page_bytes, meta.ctypes.data, s.meta_bytes)
    c = vla.LoopCache(cfg, ar, 0)
    seqs = [c.lkv_add_seq() for _ in range(3)]
    for sq, L in zip(seqs, (2000, 400, 140)):
        c.lkv_reserve(sq, 0, 0, 0, L)
    rows = 3 * 4
    n_cp = (2000 - 132 + 31) // 32
    S = min(64, max(1, 1280 // rows - 1), n_cp)
    assert c.lkv_workspace_bytes(0, 0, seqs) == rows * (S + 1) * 129 * 4
    assert c.lkv_workspace_bytes(0, 0, seqs[2:], split_k=5) == 4 * (1 + 1) * 129 * 4  # 1 code page caps the splits
    # 256 rows: 1280 / 256 - 1 = 4 far splits (five workgroups per row, one resident generation)
    cfg = vla.LoopCache.config(n_layers=1, n_loops=2, n_heads_q=16, n_heads_kv=16, head_dim=128,
                               kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=16, max_len=1000,
                               max_block=1, quant=1, sink=4, tail=128)
    s = vla.LoopCache.sizes(cfg)
    meta = np.zeros(max(256, s.meta_bytes), dtype=np.uint8)
    ar = vla.lkv_arenas(base, 1024 * s.page_bytes, base + (1 << 38), 1024 * s.code4_page_bytes, base + (1 << 39),
                        1024 * s.code2_page_bytes, meta.ctypes.data, s.meta_bytes)
    c = vla.LoopCache(cfg, ar, 0)
    seqs = [c.lkv_add_seq() for _ in range(16)]
    for sq in seqs:
        c.lkv_reserve(sq, 0, 0, 0, 1000)
    assert c.lkv_workspace_bytes(0, 0, seqs) == 256 * (4 + 1) * 129 * 4


@pytest.mark.parametrize("gamma,W", [(4, 8), (7, 7), (2, 40), (9, 4)])
def test_speculative_steps_keep_exactly_the_ripe_pages(lib, gamma, W):
    """Host bookkeeping of many self-speculative steps (RIPE page, Sec. 4 and Algorithm 1) with a block length
    drawn per step in [1, gamma] (also above W in the last case): reserve the block's planes at every loop, accept
    a seeded prefix, commit and truncate.  After every step the pages in use are the
    deepest plane of every position plus the window ring of every other plane, the logical bytes follow Eq. (10),
    and every cached position that the next token (at position len) reads resolves to a resident page of the
    plane the policy names."""
    R, n_layers, L0 = 4, 2, [5, 33, 70]
    c = make(n_pages=4096, n_layers=n_layers, n_loops=R, window=W, max_block=gamma + 1, max_len=2048, max_seqs=3)
    seqs = [c.lkv_add_seq() for _ in L0]
    lens = list(L0)
    for s, L in zip(seqs, lens):
        for layer in range(n_layers):
            c.lkv_reserve(s, layer, R - 1, 0, L)
        c.lkv_commit(s, L)  # the window is measured from the committed length
        for layer in range(n_layers):
            for plane in range(R - 1):
                lo = max(0, L - W)
                c.lkv_reserve(s, layer, plane, lo, L - lo)
    rng = np.random.default_rng(gamma * 100 + W)
    b_tok = 2 * 2 * 64 * 2
    drawn = set()
    for step in range(60):
        g = int(rng.integers(1, gamma + 1))  # this step's block length g + 1
        drawn.add(g)
        for b, s in enumerate(seqs):
            for loop in range(R):
                for layer in range(n_layers):
                    c.lkv_reserve(s, layer, loop, lens[b], g + 1)
            a = int(rng.integers(0, g + 1))
            new_len = lens[b] + 1 + a
            c.lkv_commit(s, new_len)
            c.lkv_truncate(s, new_len)
            lens[b] = new_len
            assert c.lkv_seq_info(s) == (new_len, new_len)
        want = 0
        for L in lens:
            lo = max(0, L - W)
            want += n_layers * ((L + 15) // 16 + (R - 1) * ((L - 1) // 16 - lo // 16 + 1))
        assert c.lkv_mem_stats()["pages_in_use"] == want
        assert c.lkv_mem_stats()["logical_bytes"] == sum(b_tok * n_layers * (L + (R - 1) * min(W, L)) for L in lens)
        for s, L in zip(seqs, lens):
            t = L  # the next token x sits at position L; it reads cached positions 0..L-1
            for loop in (0, R - 2, R - 1):
                for j in range(L):
                    plane, phys, slot = c.lkv_debug_resolve(s, 1, loop, t, t, j)
                    assert plane == oracle.oracle_plane(oracle.RIPE, loop, R, t, t, j, W)
                    assert phys >= 0 and slot == j % 16
    assert len(drawn) > 1  # the block length varied


def test_binding_rejects_host_noncontiguous_and_undersized_tensors():
    """The binding hands the library bare addresses, so it checks tensor arguments first: a host tensor, a
    non-contiguous view, a wrong element type or too few elements raise ValueError; None and int addresses pass."""
    torch = pytest.importorskip("torch")
    need = vla._need
    need(None, "x", 10, 4)
    need(1234, "x", 10, 4)
    with pytest.raises(ValueError, match="device tensor"):
        need(torch.zeros(16), "x", 10, 4)

    class FakeDev:  # a stand-in with the tensor attributes the check reads (no GPU here)
        is_cuda = True

        def __init__(self, n, es, dtype, contiguous=True):
            self.n, self.es, self.dtype, self.c = n, es, dtype, contiguous

        def is_contiguous(self):
            return self.c

        def element_size(self):
            return self.es

        def numel(self):
            return self.n

    need(FakeDev(10, 2, torch.bfloat16), "q", 10, 2, (torch.bfloat16,))
    with pytest.raises(ValueError, match="contiguous"):
        need(FakeDev(10, 2, torch.bfloat16, contiguous=False), "q", 10, 2, (torch.bfloat16,))
    with pytest.raises(ValueError, match="element type"):
        need(FakeDev(10, 2, torch.float16), "q", 10, 2, (torch.bfloat16,))
    with pytest.raises(ValueError, match="element type"):
        need(FakeDev(10, 4, torch.float32), "q", 10, 2, (torch.bfloat16,))
    with pytest.raises(ValueError, match="needs 11"):
        need(FakeDev(10, 2, torch.bfloat16), "q", 11, 2, (torch.bfloat16,))
    need(FakeDev(3, 8, torch.float64), "workspace", 0, None)


def test_commit_is_monotone(lib):
    """RIPE page, Algorithm 1: the window only slides forward.  A commit below the committed length is refused,
    since the ring pages of positions that left the window were already returned to the pool; after the refusal
    the cache still holds what it held, and a later forward commit works."""
    W = 16
    c = make(n_pages=100, window=W, max_block=8)
    s = c.lkv_add_seq()
    c.lkv_reserve(s, 0, 3, 0, 100)
    c.lkv_commit(s, 100)
    for p in range(3):
        c.lkv_reserve(s, 0, p, 100 - W, W)
    used = c.lkv_mem_stats()["pages_in_use"]
    with pytest.raises(vla.LkvError) as e:
        c.lkv_commit(s, 50)
    assert e.value.status == vla.LKV_EINVAL
    assert c.lkv_seq_info(s) == (100, 100)
    assert c.lkv_mem_stats()["pages_in_use"] == used
    # the truncate that could have followed a backwards commit is refused as well (below committed)
    with pytest.raises(vla.LkvError) as e:
        c.lkv_truncate(s, 60)
    assert e.value.status == vla.LKV_EINVAL
    # appending the next position and committing forward still works
    for p in range(4):
        c.lkv_reserve(s, 0, p, 100, 1)
    c.lkv_commit(s, 101)
    assert c.lkv_seq_info(s) == (101, 101)


def test_noalloc_refuses_workspace_and_oversized_calls_before_device_work(lib):
    """lkv_attend_noalloc takes no workspace, and a call whose split partials exceed its fixed scratch is refused
    on the host with EINVAL (no device is touched: this runs without a GPU)."""
    c = make(n_pages=400, n_heads_q=55, n_heads_kv=55, head_dim=96, max_seqs=16, max_len=256)
    seqs = [c.lkv_add_seq() for _ in range(16)]
    for s in seqs:
        c.lkv_reserve(s, 0, 3, 0, 64)
    per_split = 16 * 8 * 55 * 97 * 4  # verify blocks of 8 rows
    assert vla.NOALLOC_SCRATCH_BYTES == 32 << 20
    a, _ids = c._args(0, 3, seqs, 1 << 40, 1 << 41, q_len=8, mode=vla.MODE_VERIFY, split_k=64)
    assert 64 * per_split > vla.NOALLOC_SCRATCH_BYTES
    assert lib.lkv_attend_noalloc(c.h, ctypes.byref(a), 0) == vla.LKV_EINVAL
    assert b"scratch" in lib.lkv_last_error(c.h)
    a, _ids = c._args(0, 3, seqs, 1 << 40, 1 << 41, split_k=2)
    a.workspace, a.workspace_bytes = 1 << 42, 1 << 20
    assert lib.lkv_attend_noalloc(c.h, ctypes.byref(a), 0) == vla.LKV_EINVAL
    assert b"no workspace" in lib.lkv_last_error(c.h)


def test_quantised_plane_appends_keep_sink_then_tail_without_gaps(lib):
    """Quantised caches hold the exact sink and tail in their bf16 planes (LoopKV page, Sec. 3.2): after the sink the
    far history may be skipped (it comes as code pages), but any other gap is refused, and the tail grows one
    position after another."""
    cfg = vla.LoopCache.config(n_layers=1, n_loops=4, n_heads_q=2, n_heads_kv=2, head_dim=128,
                               kv_dtype=vla.DTYPE_BF16, policy=vla.POLICY_FULL, window=0, max_seqs=2, max_len=512,
                               max_block=1, quant=1, sink=4, tail=32)
    ha = HostArenas(cfg, 64, 16, 16)
    c = vla.LoopCache(cfg, ha.ar, 0)
    c._host_arenas = ha
    c.lkv_set_plan(np.array([[vla.CELL_INT4, vla.CELL_INT2, vla.CELL_SHARED, vla.CELL_INT4]], dtype=np.int8))
    s = c.lkv_add_seq()
    c.lkv_reserve(s, 0, 0, 0, 4)          # sink
    c.lkv_reserve(s, 0, 0, 200 - 32, 32)  # tail of a 200-token sequence; the far history comes as codes
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(s, 0, 0, 205, 1)    # a gap after the tail
    assert e.value.status == vla.LKV_ESTATE
    c.lkv_reserve(s, 0, 0, 200, 3)        # the tail grows
    assert c.lkv_seq_info(s) == (203, 0)
    s2 = c.lkv_add_seq()
    c.lkv_reserve(s2, 0, 1, 0, 2)
    with pytest.raises(vla.LkvError) as e:
        c.lkv_reserve(s2, 0, 1, 3, 1)     # a gap inside the sink
    assert e.value.status == vla.LKV_ESTATE
