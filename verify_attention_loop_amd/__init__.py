"""Python binding of libloopattn (loop-aware attention over a looped model's
multi-plane KV cache, MI355X / gfx950).

Argument marshalling only: every call goes through the C-ABI declared in
``include/loopattn.h``; every step of the attention path runs in the library's
HIP kernels.  PyTorch provides device memory (the arenas, inputs, outputs) and
the stream.  If the library is not built this module raises on first use; it
has no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopattn.so")

LKV_OK, LKV_EINVAL, LKV_ENOMEM, LKV_ESTATE, LKV_EWINDOW, LKV_EDEVICE, LKV_EUNSUPPORTED = range(7)
DTYPE_F32, DTYPE_BF16 = 0, 1
POLICY_FULL, POLICY_RIPE = 0, 1
MODE_DECODE, MODE_VERIFY, MODE_DRAFT = 0, 1, 2
CELL_BF16, CELL_INT4, CELL_INT2, CELL_SHARED = 0, 1, 2, 3
VRULE_FIXED, VRULE_RUNNING = 0, 1
KERNEL_AUTO, KERNEL_VALU = 0, 1
PAGE_TOKENS, CODE_PAGE_TOKENS = 16, 32
NOALLOC_SCRATCH_BYTES = 32 << 20  # LKV_NOALLOC_SCRATCH_BYTES

EXPORTS = [
    "lkv_sizes", "lkv_create", "lkv_destroy", "lkv_add_seq", "lkv_free_seq", "lkv_reserve", "lkv_append_plane",
    "lkv_commit", "lkv_truncate", "lkv_set_plan", "lkv_append_coded", "lkv_encode_pages", "lkv_read_coded",
    "lkv_window_exit",
    "lkv_workspace_bytes", "lkv_attend", "lkv_attend_noalloc",
    "lkv_mem_stats", "lkv_debug_resolve", "lkv_seq_info", "lkv_last_error", "lkv_status_str", "lkv_probe_read",
]


class lkv_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_loops", "n_heads_q", "n_heads_kv", "head_dim", "page_size", "kv_dtype", "policy", "window",
        "max_seqs", "max_len", "max_block", "quant", "sink", "tail", "poison")] + [("shuffle_seed", ctypes.c_uint64)]


class lkv_arenas(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("pages_bytes", ctypes.c_size_t),
                ("codes4", ctypes.c_void_p), ("codes4_bytes", ctypes.c_size_t),
                ("codes2", ctypes.c_void_p), ("codes2_bytes", ctypes.c_size_t),
                ("meta", ctypes.c_void_p), ("meta_bytes", ctypes.c_size_t)]


class lkv_size_info(ctypes.Structure):
    _fields_ = [("page_bytes", ctypes.c_size_t), ("code4_page_bytes", ctypes.c_size_t),
                ("code2_page_bytes", ctypes.c_size_t), ("meta_bytes", ctypes.c_size_t)]


class lkv_attend_args(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("loop", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("seq_ids", ctypes.POINTER(ctypes.c_int32)), ("q_len", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("window", ctypes.c_int32), ("split_k", ctypes.c_int32), ("v_thresh_offset", ctypes.c_float),
                ("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("draft_k", ctypes.c_void_p), ("draft_v", ctypes.c_void_p), ("draft_len", ctypes.c_int32),
                ("index_trace", ctypes.c_void_p), ("trace_len", ctypes.c_int32), ("mask_trace", ctypes.c_void_p),
                ("ev_begin", ctypes.c_void_p), ("ev_end", ctypes.c_void_p),
                ("v_rule", ctypes.c_int32), ("v_tau", ctypes.c_float),
                ("waves", ctypes.c_int32), ("kernel", ctypes.c_int32)]


class lkv_mem_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("logical_bytes", "pages_in_use", "pages_total", "code4_in_use",
                                               "code4_total", "code2_in_use", "code2_total")]


class LkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


_LIB = None


def load():
    """Load libloopattn.so (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    i32, vp, st = ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    P = ctypes.POINTER
    sig = {
        "lkv_sizes": [P(lkv_config), P(lkv_size_info)],
        "lkv_create": [P(lkv_config), P(lkv_arenas), ctypes.c_int, P(vp)],
        "lkv_destroy": [vp],
        "lkv_add_seq": [vp, P(i32)],
        "lkv_free_seq": [vp, i32],
        "lkv_reserve": [vp, i32, i32, i32, i32, i32],
        "lkv_append_plane": [vp, i32, i32, i32, i32, i32, vp, vp, vp],
        "lkv_commit": [vp, i32, i32],
        "lkv_truncate": [vp, i32, i32],
        "lkv_set_plan": [vp, P(ctypes.c_int8)],
        "lkv_append_coded": [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp],
        "lkv_encode_pages": [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp],
        "lkv_read_coded": [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp],
        "lkv_window_exit": [vp, i32, vp],
        "lkv_workspace_bytes": [vp, P(lkv_attend_args), P(ctypes.c_size_t)],
        "lkv_attend": [vp, P(lkv_attend_args), vp],
        "lkv_attend_noalloc": [vp, P(lkv_attend_args), vp],
        "lkv_mem_stats": [vp, P(lkv_mem_info)],
        "lkv_debug_resolve": [vp, i32, i32, i32, i32, i32, i32, i32, P(i32), P(i32), P(i32)],
        "lkv_seq_info": [vp, i32, P(i32), P(i32)],
        "lkv_probe_read": [vp, ctypes.c_size_t, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = st
    L.lkv_last_error.argtypes = [vp]
    L.lkv_last_error.restype = ctypes.c_char_p
    L.lkv_status_str.argtypes = [st]
    L.lkv_status_str.restype = ctypes.c_char_p
    _LIB = L
    return L


def _ptr(x) -> int:
    """Device address of a tensor (or an int address, or None -> 0)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _need(t, name: str, n_elems: int, elem_bytes: int, dtypes=None):
    """A tensor argument must be a contiguous device tensor of the documented element type holding at
    least n_elems elements: the library takes bare addresses and sizes its kernels from the call's
    arguments, so a smaller buffer would be read or written past its end.  None and int addresses pass
    through (the caller vouches for them)."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_bytes is not None and (t.element_size() != elem_bytes or (dtypes is not None and t.dtype not in dtypes)):
        raise ValueError(f"{name} has element type {t.dtype}, expected {elem_bytes}-byte {dtypes or ''}")
    if t.numel() < n_elems:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n_elems}")


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


PROBE_CHUNK = 16384  # LKV_PROBE_CHUNK


def lkv_probe_read(buf, nbytes: int, sink, ev_begin=0, ev_end=0, stream=None):
    """One streaming read of the first nbytes of device tensor buf (a positive multiple of PROBE_CHUNK)
    on the stream: the achievable HBM read rate that the attention kernels are compared with.  sink is
    a device tensor of at least one 4-byte word; ev_begin / ev_end are HIP event handles (or 0) that the
    launch stamps with its own start and end."""
    _need(buf, "buf", nbytes, None)
    if buf is not None and not isinstance(buf, int) and buf.numel() * buf.element_size() < nbytes:
        raise ValueError(f"buf holds {buf.numel() * buf.element_size()} bytes, the call reads {nbytes}")
    _need(sink, "sink", 1, 4)
    rc = load().lkv_probe_read(_ptr(buf), nbytes, _ptr(sink), ev_begin or 0, ev_end or 0, _stream(stream))
    if rc != 0:
        raise LkvError(rc, f"lkv_probe_read: {load().lkv_status_str(rc).decode()}")


class LoopCache:
    """A handle over caller-owned arenas.  Method names follow the C-ABI (lkv_*)."""

    def __init__(self, cfg: lkv_config, arenas: lkv_arenas, device: int = 0, keep=()):
        self.lib = load()
        self.cfg = cfg
        self.arenas = arenas
        self._keep = list(keep)  # tensors backing the arenas
        h = ctypes.c_void_p()
        rc = self.lib.lkv_create(ctypes.byref(cfg), ctypes.byref(arenas), device, ctypes.byref(h))
        if rc != LKV_OK:
            raise LkvError(rc, "lkv_create: " + self.lib.lkv_status_str(rc).decode())
        self.h = h

    # -- construction helpers
    @staticmethod
    def config(**kw) -> lkv_config:
        c = lkv_config()
        c.page_size = PAGE_TOKENS
        c.max_block = 1
        for k, v in kw.items():
            setattr(c, k, v)
        return c

    @staticmethod
    def sizes(cfg: lkv_config) -> lkv_size_info:
        s = lkv_size_info()
        rc = load().lkv_sizes(ctypes.byref(cfg), ctypes.byref(s))
        if rc != LKV_OK:
            raise LkvError(rc, "lkv_sizes: invalid configuration")
        return s

    @classmethod
    def on_device(cls, cfg: lkv_config, n_pages: int, n_code4: int = 0, n_code2: int = 0, device: int = 0):
        """Allocate the arenas as torch uint8 tensors on cuda:device and create the cache."""
        import torch
        s = cls.sizes(cfg)
        dev = torch.device("cuda", device)
        pages = torch.empty(max(1, n_pages * s.page_bytes), dtype=torch.uint8, device=dev)
        c4 = torch.empty(max(1, n_code4 * s.code4_page_bytes), dtype=torch.uint8, device=dev) if n_code4 else None
        c2 = torch.empty(max(1, n_code2 * s.code2_page_bytes), dtype=torch.uint8, device=dev) if n_code2 else None
        meta = torch.empty(max(256, s.meta_bytes), dtype=torch.uint8, device=dev)
        ar = lkv_arenas(pages.data_ptr(), n_pages * s.page_bytes,
                        c4.data_ptr() if c4 is not None else 0, n_code4 * s.code4_page_bytes,
                        c2.data_ptr() if c2 is not None else 0, n_code2 * s.code2_page_bytes,
                        meta.data_ptr(), s.meta_bytes)
        return cls(cfg, ar, device, keep=[t for t in (pages, c4, c2, meta) if t is not None])

    def close(self):
        if getattr(self, "h", None):
            self.lib.lkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc != LKV_OK:
            raise LkvError(rc, f"{what}: {self.lib.lkv_last_error(self.h).decode()}")

    # -- C-ABI calls
    def lkv_add_seq(self) -> int:
        s = ctypes.c_int32()
        self._check(self.lib.lkv_add_seq(self.h, ctypes.byref(s)), "lkv_add_seq")
        return s.value

    def lkv_free_seq(self, seq: int):
        self._check(self.lib.lkv_free_seq(self.h, seq), "lkv_free_seq")

    def lkv_reserve(self, seq: int, layer: int, plane: int, pos0: int, n_tok: int):
        self._check(self.lib.lkv_reserve(self.h, seq, layer, plane, pos0, n_tok), "lkv_reserve")

    def _kv_types(self):
        import torch
        return (4, (torch.float32,)) if self.cfg.kv_dtype == DTYPE_F32 else (2, (torch.bfloat16,))

    def lkv_append_plane(self, seq: int, layer: int, plane: int, pos0: int, k, v, stream=None):
        n_tok = k.shape[0]
        row = self.cfg.n_heads_kv * self.cfg.head_dim
        eb, dt = self._kv_types()
        _need(k, "k", n_tok * row, eb, dt)
        _need(v, "v", n_tok * row, eb, dt)
        self._check(self.lib.lkv_append_plane(self.h, seq, layer, plane, pos0, n_tok, _ptr(k), _ptr(v),
                                              _stream(stream)), "lkv_append_plane")

    def lkv_commit(self, seq: int, new_len: int):
        self._check(self.lib.lkv_commit(self.h, seq, new_len), "lkv_commit")

    def lkv_truncate(self, seq: int, new_len: int):
        self._check(self.lib.lkv_truncate(self.h, seq, new_len), "lkv_truncate")

    def lkv_set_plan(self, kinds):
        import numpy as np
        a = np.ascontiguousarray(kinds, dtype=np.int8)
        self._check(self.lib.lkv_set_plan(self.h, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))), "lkv_set_plan")

    def _coded_args(self, n_pages, k_codes, k_meta, v_codes, v_meta):
        hkv, d = self.cfg.n_heads_kv, self.cfg.head_dim
        _need(k_codes, "k_codes", n_pages * CODE_PAGE_TOKENS * hkv * d, 1)
        _need(k_meta, "k_meta", n_pages * hkv * d * 2, 2)
        _need(v_codes, "v_codes", n_pages * CODE_PAGE_TOKENS * hkv * d, 1)
        _need(v_meta, "v_meta", n_pages * CODE_PAGE_TOKENS * hkv * (d // 32) * 2, 2)

    def lkv_append_coded(self, seq: int, layer: int, loop: int, page0: int, n_pages: int, k_codes, k_meta, v_codes,
                         v_meta, stream=None):
        self._coded_args(n_pages, k_codes, k_meta, v_codes, v_meta)
        self._check(self.lib.lkv_append_coded(self.h, seq, layer, loop, page0, n_pages, _ptr(k_codes), _ptr(k_meta),
                                              _ptr(v_codes), _ptr(v_meta), _stream(stream)), "lkv_append_coded")

    def lkv_encode_pages(self, seq: int, layer: int, loop: int, page0: int, n_pages: int, n_valid_last: int, k, v,
                         stream=None):
        import torch
        n_tok = max(0, (n_pages - 1) * CODE_PAGE_TOKENS + n_valid_last)
        row = self.cfg.n_heads_kv * self.cfg.head_dim
        _need(k, "k", n_tok * row, 2, (torch.bfloat16,))
        _need(v, "v", n_tok * row, 2, (torch.bfloat16,))
        self._check(self.lib.lkv_encode_pages(self.h, seq, layer, loop, page0, n_pages, n_valid_last, _ptr(k), _ptr(v),
                                              _stream(stream)), "lkv_encode_pages")

    def lkv_read_coded(self, seq: int, layer: int, loop: int, page0: int, n_pages: int, k_codes, k_meta, v_codes,
                       v_meta, stream=None):
        self._coded_args(n_pages, k_codes, k_meta, v_codes, v_meta)
        self._check(self.lib.lkv_read_coded(self.h, seq, layer, loop, page0, n_pages, _ptr(k_codes), _ptr(k_meta),
                                            _ptr(v_codes), _ptr(v_meta), _stream(stream)), "lkv_read_coded")

    def lkv_window_exit(self, seq: int, stream=None):
        self._check(self.lib.lkv_window_exit(self.h, seq, _stream(stream)), "lkv_window_exit")

    def _args(self, layer, loop, seq_ids, q, out, q_len=1, mode=MODE_DECODE, window=-1, split_k=0,
              v_thresh_offset=4.0, lse=None, workspace=None, draft_k=None, draft_v=None, draft_len=0,
              index_trace=None, trace_len=0, mask_trace=None, ev_begin=None, ev_end=None, v_rule=VRULE_FIXED,
              v_tau=14.0, waves=0, kernel=KERNEL_AUTO):
        ids = (ctypes.c_int32 * len(seq_ids))(*seq_ids)
        a = lkv_attend_args()
        a.layer, a.loop, a.n_seqs, a.seq_ids = layer, loop, len(seq_ids), ids
        a.q_len, a.mode, a.window, a.split_k, a.v_thresh_offset = q_len, mode, window, split_k, v_thresh_offset
        a.q, a.out, a.lse = _ptr(q), _ptr(out), _ptr(lse)
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        a.draft_k, a.draft_v, a.draft_len = _ptr(draft_k), _ptr(draft_v), draft_len
        a.index_trace, a.trace_len, a.mask_trace = _ptr(index_trace), trace_len, _ptr(mask_trace)
        a.ev_begin = ev_begin or 0
        a.ev_end = ev_end or 0
        a.v_rule, a.v_tau = v_rule, v_tau
        a.waves, a.kernel = waves, kernel
        return a, ids

    def lkv_workspace_bytes(self, layer, loop, seq_ids, q_len=1, mode=MODE_DECODE, split_k=0) -> int:
        a, _ids = self._args(layer, loop, seq_ids, None, None, q_len=q_len, mode=mode, split_k=split_k)
        n = ctypes.c_size_t()
        self._check(self.lib.lkv_workspace_bytes(self.h, ctypes.byref(a), ctypes.byref(n)), "lkv_workspace_bytes")
        return n.value

    def _attend_buffers(self, a, q, out, kw):
        """Sizes of the call's tensors, from the same arguments the library sizes its kernels by."""
        import torch
        c = self.cfg
        n, k, hq, hkv, d = a.n_seqs, max(1, a.q_len), c.n_heads_q, c.n_heads_kv, c.head_dim
        eb, dt = self._kv_types()
        _need(q, "q", n * k * hq * d, eb, dt)
        _need(out, "out", n * k * hq * d, eb, dt)
        _need(kw.get("lse"), "lse", n * k * hq, 4, (torch.float32,))
        _need(kw.get("workspace"), "workspace", 0, None)  # its size in bytes is passed and checked by the library
        if a.draft_len > 0:
            _need(kw.get("draft_k"), "draft_k", n * a.draft_len * hkv * d, eb, dt)
            _need(kw.get("draft_v"), "draft_v", n * a.draft_len * hkv * d, eb, dt)
        if a.trace_len > 0:
            _need(kw.get("index_trace"), "index_trace", n * k * a.trace_len * 2, 4, (torch.int32,))
        if kw.get("mask_trace") is not None and c.quant:
            far = max(max(0, self.lkv_seq_info(a.seq_ids[b])[0] - c.sink - c.tail) for b in range(n))
            _need(kw.get("mask_trace"), "mask_trace", n * hq * ((far + 31) // 32), 4)

    def lkv_attend(self, layer, loop, seq_ids, q, out, stream=None, **kw):
        a, _ids = self._args(layer, loop, seq_ids, q, out, **kw)
        if not 1 <= a.n_seqs <= self.cfg.max_seqs:
            raise ValueError(f"n_seqs {a.n_seqs} outside [1, {self.cfg.max_seqs}]")
        self._attend_buffers(a, q, out, kw)
        self._check(self.lib.lkv_attend(self.h, ctypes.byref(a), _stream(stream)), "lkv_attend")

    def lkv_attend_noalloc(self, layer, loop, seq_ids, q, out, stream=None, **kw):
        """lkv_attend without a workspace: the split partials live in the library's fixed device scratch
        (nothing is allocated).  Calls that overlap on one GPU race."""
        if kw.get("workspace") is not None:
            raise ValueError("lkv_attend_noalloc takes no workspace")
        a, _ids = self._args(layer, loop, seq_ids, q, out, **kw)
        if not 1 <= a.n_seqs <= self.cfg.max_seqs:
            raise ValueError(f"n_seqs {a.n_seqs} outside [1, {self.cfg.max_seqs}]")
        self._attend_buffers(a, q, out, kw)
        self._check(self.lib.lkv_attend_noalloc(self.h, ctypes.byref(a), _stream(stream)), "lkv_attend_noalloc")

    def lkv_mem_stats(self) -> dict:
        m = lkv_mem_info()
        self._check(self.lib.lkv_mem_stats(self.h, ctypes.byref(m)), "lkv_mem_stats")
        return {n: getattr(m, n) for n, _ in lkv_mem_info._fields_}

    def lkv_debug_resolve(self, seq, layer, loop, t, t0, j, window=-1):
        p, ph, sl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(self.lib.lkv_debug_resolve(self.h, seq, layer, loop, t, t0, j, window, ctypes.byref(p),
                                               ctypes.byref(ph), ctypes.byref(sl)), "lkv_debug_resolve")
        return p.value, ph.value, sl.value

    def lkv_seq_info(self, seq):
        n, c = ctypes.c_int32(), ctypes.c_int32()
        self._check(self.lib.lkv_seq_info(self.h, seq, ctypes.byref(n), ctypes.byref(c)), "lkv_seq_info")
        return n.value, c.value
