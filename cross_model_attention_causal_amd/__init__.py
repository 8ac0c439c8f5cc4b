"""Python binding of ``libcma.so``: cross-model reuse of causal attention maps on MI355X.

Argument marshalling only. Every step of the path runs in the library's HIP
kernels; torch tensors provide device memory and the current HIP stream. There
is no fallback: if the library is missing or a tensor is not on the GPU, the
call raises.

Entry points (same names as the C ABI in ``include/cma.h``):
``attn_maps``, ``head_map_cosine``, ``block_compress``, ``mapped_av``,
``onehot_mix``, ``mapped_layers``; ``Varlen`` describes packed sequences.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcma.so")

CMA_OK, CMA_EINVAL, CMA_EUNSUPPORTED, CMA_ENOSPC, CMA_EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
DENSE, PACKED = 0, 1
SRC_DENSE, SRC_BSR = 0, 1
V_TOKEN_MAJOR, V_KEY_MAJOR, V_TILED, V_PAGED = 0, 1, 2, 3
BLOCK = 64

EXPORTS = [
    "cma_version", "cma_last_error", "cma_maps_elems", "cma_attn_maps",
    "cma_head_map_cosine_workspace", "cma_head_map_cosine", "cma_head_map_fused_workspace", "cma_head_map_fused", "cma_bsr_max_blocks", "cma_bsr_capacity",
    "cma_block_compress_workspace", "cma_block_compress", "cma_block_compress_noalloc", "cma_mapped_av_workspace",
    "cma_mapped_av", "cma_mapped_av_indexed_workspace", "cma_mapped_av_indexed", "cma_tile_v", "cma_tile_v_paged", "cma_onehot_mix", "cma_mapped_layers", "cma_timing_enable",
    "cma_timing_collect", "cma_timing_get", "cma_timing_name", "cma_timing_reset",
    "cma_prefix_hashes", "cma_fnv1a64", "cma_prefix_index_create", "cma_prefix_index_destroy",
    "cma_prefix_index_insert", "cma_prefix_index_lookup", "cma_prefix_index_erase", "cma_prefix_index_evict_lru",
    "cma_prefix_index_size",
]


class CmaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"cma status {status}: {msg}")
        self.status = status


class _CVarlen(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p), ("seqused_q", ctypes.c_void_p),
                ("seqused_k", ctypes.c_void_p), ("max_seqlen_q", ctypes.c_int32),
                ("max_seqlen_k", ctypes.c_int32), ("total_q", ctypes.c_int64),
                ("total_k", ctypes.c_int64)]


class _CMapsSrc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("maps", ctypes.c_void_p), ("maps_dt", ctypes.c_int),
                ("layout", ctypes.c_int), ("head_stride", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("vals", ctypes.c_void_p), ("n_block_rows", ctypes.c_int32),
                ("row_end", ctypes.c_void_p), ("n_key_blocks", ctypes.c_int32)]


class _CPagedV(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("page_stride", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load ``libcma.so`` and declare its C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python __graft_entry__.py` or "
                          "`python cross_model_attention_causal_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    F = ctypes.c_float
    sig = {
        "cma_version": (ctypes.c_int, []),
        "cma_last_error": (ctypes.c_char_p, []),
        "cma_maps_elems": (I64, [I32, P, P, ctypes.c_int]),
        "cma_attn_maps": (ctypes.c_int, [P, P, ctypes.c_int, I32, I32, P, P, P, P, ctypes.c_int,
                                         ctypes.c_int, I64, P]),
        "cma_head_map_cosine_workspace": (SZ, [I32, I32, I32, I64, ctypes.c_int]),
        "cma_head_map_cosine": (ctypes.c_int, [P, P, ctypes.c_int, I32, I32, I32, I64, I64, I64,
                                               I64, I64, P, P, P, P, SZ, P]),
        "cma_head_map_fused_workspace": (SZ, [I32, I32, I32, I32]),
        "cma_head_map_fused": (ctypes.c_int, [P, P, I32, I32, P, P, P, I64, I32, P, P, P, P, P, SZ, P]),
        "cma_bsr_max_blocks": (I64, [I32, I32, P]),
        "cma_bsr_capacity": (I64, [I32, I32, P, P]),
        "cma_block_compress_workspace": (SZ, [I32, I32, I32, I64]),
        "cma_block_compress": (ctypes.c_int, [P, P, ctypes.c_int, I32, I32, P, P, P, F, I32, P, P,
                                              P, I64, P, P, P, P, SZ, P]),
        "cma_block_compress_noalloc": (ctypes.c_int, [P, P, ctypes.c_int, I32, I32, P, P, P, F, I32, P, P,
                                                      P, I64, P, P, P, P]),
        "cma_mapped_av_workspace": (SZ, [P, I32, I32, I64, ctypes.c_int]),
        "cma_mapped_av": (ctypes.c_int, [P, I32, P, I64, I32, I32, P, ctypes.c_int, ctypes.c_int, I32, P,
                                         P, ctypes.c_int, P, SZ, P]),
        "cma_mapped_av_indexed_workspace": (SZ, [P, I32, I32, I32, I32, ctypes.c_int]),
        "cma_mapped_av_indexed": (ctypes.c_int, [P, I32, P, I64, I32, I32, P, ctypes.c_int, ctypes.c_int, I32,
                                                 P, P, ctypes.c_int, P, SZ, P]),
        "cma_tile_v": (ctypes.c_int, [P, ctypes.c_int, I32, I32, P, I32, P, P]),
        "cma_tile_v_paged": (ctypes.c_int, [P, ctypes.c_int, I32, I32, P, P, P]),
        "cma_onehot_mix": (ctypes.c_int, [P, I32, I32, I32, P, P]),
        "cma_mapped_layers": (ctypes.c_int, [I32, D, P, I32]),
        "cma_mapping_plan": (ctypes.c_int, [I32, P, I32, I32, P, P]),
        "cma_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "cma_timing_collect": (ctypes.c_int, []),
        "cma_timing_get": (D, [ctypes.c_char_p, ctypes.POINTER(I64)]),
        "cma_timing_name": (ctypes.c_char_p, [ctypes.c_int]),
        "cma_timing_reset": (None, []),
        "cma_prefix_hashes": (ctypes.c_int, [P, I64, ctypes.c_uint64, P]),
        "cma_fnv1a64": (ctypes.c_uint64, [P, SZ]),
        "cma_prefix_index_create": (P, [I32, I64]),
        "cma_prefix_index_destroy": (None, [P]),
        "cma_prefix_index_insert": (ctypes.c_int, [P, I32, ctypes.c_uint64, P, P]),
        "cma_prefix_index_lookup": (I64, [P, I32, P, I64, P, P]),
        "cma_prefix_index_erase": (ctypes.c_int, [P, I32, ctypes.c_uint64]),
        "cma_prefix_index_evict_lru": (ctypes.c_int, [P, P, P, P, P]),
        "cma_prefix_index_size": (I64, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != CMA_OK:
        raise CmaError(status, _lib.cma_last_error().decode())


def _torch():
    import torch
    return torch


def _dev_ptr(t, name):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class Varlen:
    """Packed sequences: start rows ``cu_q``/``cu_k`` (host sequences of n+1 ints)
    and optional used lengths ``used_q``/``used_k`` (host sequences of n ints).

    Device copies are made once; host copies size the outputs.
    """

    def __init__(self, cu_q, cu_k=None, used_q=None, used_k=None, device="cuda"):
        torch = _torch()
        self.cu_q_host = np.asarray(cu_q, dtype=np.int64)
        self.cu_k_host = np.asarray(cu_k if cu_k is not None else cu_q, dtype=np.int64)
        n = len(self.cu_q_host) - 1
        self.n_seqs = n
        if used_k is None and cu_k is None:
            used_k = used_q  # keys share the query layout
        self.lens_q = np.asarray(used_q if used_q is not None else np.diff(self.cu_q_host), dtype=np.int64)
        self.lens_k = np.asarray(used_k if used_k is not None else np.diff(self.cu_k_host), dtype=np.int64)
        mk = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device=device)
        self.cu_q = mk(self.cu_q_host)
        self.cu_k = mk(self.cu_k_host)
        self.used_q = mk(self.lens_q) if used_q is not None else None
        self.used_k = mk(self.lens_k) if used_k is not None else None
        self.max_q = int(self.lens_q.max()) if n else 0
        self.max_k = int(self.lens_k.max()) if n else 0
        self.n_block_rows = int(sum((int(x) + BLOCK - 1) // BLOCK for x in self.lens_q))
        self.n_key_blocks = int(sum((int(x) + BLOCK - 1) // BLOCK for x in self.lens_k))

    @staticmethod
    def from_lengths(lens_q, lens_k=None, device="cuda"):
        cu_q = np.concatenate([[0], np.cumsum(lens_q)])
        cu_k = np.concatenate([[0], np.cumsum(lens_k)]) if lens_k is not None else None
        return Varlen(cu_q, cu_k, device=device)

    def c(self, total_q, total_k):
        v = _CVarlen()
        v.n_seqs = self.n_seqs
        v.cu_seqlens_q = self.cu_q.data_ptr()
        v.cu_seqlens_k = self.cu_k.data_ptr()
        v.seqused_q = self.used_q.data_ptr() if self.used_q is not None else None
        v.seqused_k = self.used_k.data_ptr() if self.used_k is not None else None
        v.max_seqlen_q = self.max_q
        v.max_seqlen_k = self.max_k
        v.total_q = int(total_q)
        v.total_k = int(total_k)
        return v

    def maps_elems(self, layout):
        lib = load_library()
        lq = np.ascontiguousarray(self.lens_q, dtype=np.int32)
        lk = np.ascontiguousarray(self.lens_k, dtype=np.int32)
        r = lib.cma_maps_elems(self.n_seqs, lq.ctypes.data, lk.ctypes.data, layout)
        if r < 0:
            raise ValueError("inconsistent sequence lengths")
        return int(r)


def _need(t, name, n):
    """The C ABI takes raw pointers: check here that ``t`` holds at least ``n`` elements."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _check_rows(vl, Tq, Tk):
    """Every sequence's used rows must lie inside the packed tensors."""
    if vl.n_seqs and (int(np.max(vl.cu_q_host[:-1] + vl.lens_q)) > Tq or
                      int(np.max(vl.cu_k_host[:-1] + vl.lens_k)) > Tk):
        raise ValueError("a sequence's rows run past the end of the packed q/k/v tensors")


def attn_maps(q, k, scale, bias, vl: Varlen, layout=PACKED, out_dtype=None, out=None):
    """Causal maps of every (head, sequence); returns ``[H, head_stride]`` (see cma.h)."""
    torch = _torch()
    lib = load_library()
    H, Tq, d = q.shape
    if k.dim() != 3 or k.shape[0] < H or k.shape[2] != d:
        raise ValueError(f"k must be [>= {H}, Tk, {d}] (got {tuple(k.shape)})")
    _need(scale, "scale", H)
    _need(bias, "bias", H)
    _check_rows(vl, Tq, k.shape[1])
    out_dtype = out_dtype or torch.bfloat16
    stride = vl.maps_elems(layout)
    if out is None:
        out = torch.empty((H, stride), dtype=out_dtype, device=q.device)
    _need(out, "out", H * stride)
    cvl = vl.c(Tq, k.shape[1])
    _check(lib.cma_attn_maps(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dt(q), H, d, ctypes.byref(cvl),
                             _dev_ptr(scale, "scale"), _dev_ptr(bias, "bias"), _dev_ptr(out, "out"),
                             _dt(out), layout, out.shape[1], _stream()))
    return out


def head_map_cosine(recv, send, n_batch, n_recv, n_send, length, recv_hstride, recv_bstride,
                    send_hstride, send_bstride, want_cos=True, want_margin=True):
    """Cosine head map of ``n_batch`` problems; ``recv``/``send`` are base tensors
    addressed with element strides. Returns (cos or None, argmax int32, margin or None)."""
    torch = _torch()
    lib = load_library()
    dev = recv.device
    dt = _dt(recv)
    if n_batch > 0 and n_recv > 0 and n_send > 0:
        _need(recv, "recv", (n_recv - 1) * recv_hstride + (n_batch - 1) * recv_bstride + length)
        _need(send, "send", (n_send - 1) * send_hstride + (n_batch - 1) * send_bstride + length)
    ws_bytes = lib.cma_head_map_cosine_workspace(n_batch, n_recv, n_send, length, dt)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    cos = torch.empty((n_batch, n_recv, n_send), dtype=torch.float32, device=dev) if want_cos else None
    arg = torch.empty((n_batch, n_recv), dtype=torch.int32, device=dev)
    mar = torch.empty((n_batch, n_recv), dtype=torch.float32, device=dev) if want_margin else None
    _check(lib.cma_head_map_cosine(recv.data_ptr(), send.data_ptr(), dt, n_batch, n_recv, n_send,
                                   length, recv_hstride, recv_bstride, send_hstride, send_bstride,
                                   _dev_ptr(cos, "cos"), _dev_ptr(arg, "argmax"),
                                   _dev_ptr(mar, "margin"), ws.data_ptr(), ws_bytes, _stream()))
    return cos, arg, mar


def head_map_fused(recv_q, recv_k, recv_scale, recv_bias, send_maps, n_send, vl: Varlen, want_cos=True,
                   want_margin=True, workspace: Workspace | None = None):
    """Cosine head map with the receivers' maps formed on chip (never stored): one
    problem per sequence of ``vl``; ``send_maps`` as ``attn_maps(..., layout=DENSE)``
    wrote them (bf16 [>= n_send, head_stride]). Returns (cos or None, argmax, margin
    or None), each with a leading sequence dimension."""
    torch = _torch()
    lib = load_library()
    H, Tq, d = recv_q.shape
    if recv_k.dim() != 3 or recv_k.shape[0] < H or recv_k.shape[2] != d:
        raise ValueError(f"recv_k must be [>= {H}, Tk, {d}]")
    _need(recv_scale, "recv_scale", H)
    _need(recv_bias, "recv_bias", H)
    _check_rows(vl, Tq, recv_k.shape[1])
    stride = vl.maps_elems(DENSE)
    if send_maps.dim() != 2 or send_maps.shape[0] < n_send or send_maps.shape[1] < stride:
        raise ValueError(f"send_maps must be [>= {n_send}, >= {stride}] (dense maps)")
    dev = recv_q.device
    B = vl.n_seqs
    ws_bytes = lib.cma_head_map_fused_workspace(B, H, n_send, vl.max_q)
    ws = (workspace or Workspace()).get(max(1, ws_bytes), dev)
    cos = torch.empty((B, H, n_send), dtype=torch.float32, device=dev) if want_cos else None
    arg = torch.empty((B, H), dtype=torch.int32, device=dev)
    mar = torch.empty((B, H), dtype=torch.float32, device=dev) if want_margin else None
    cvl = vl.c(Tq, recv_k.shape[1])
    _check(lib.cma_head_map_fused(_dev_ptr(recv_q, "recv_q"), _dev_ptr(recv_k, "recv_k"), H, d,
                                  _dev_ptr(recv_scale, "recv_scale"), _dev_ptr(recv_bias, "recv_bias"),
                                  _dev_ptr(send_maps, "send_maps"), send_maps.shape[1], n_send, ctypes.byref(cvl),
                                  _dev_ptr(cos, "cos"), _dev_ptr(arg, "argmax"), _dev_ptr(mar, "margin"),
                                  ws.data_ptr(), ws.numel(), _stream()))
    return cos, arg, mar


def bsr_max_blocks(n_heads, lens, lens_k=None):
    """Most blocks a compression can keep (``lens_k``: key lengths of prefill chunks)."""
    lib = load_library()
    a = np.ascontiguousarray(lens, dtype=np.int32)
    if lens_k is None:
        return int(lib.cma_bsr_max_blocks(n_heads, len(a), a.ctypes.data))
    b = np.ascontiguousarray(lens_k, dtype=np.int32)
    r = int(lib.cma_bsr_capacity(n_heads, len(a), a.ctypes.data, b.ctypes.data))
    if r < 0:
        raise ValueError("inconsistent lengths")
    return r


class Workspace:
    """Reusable device scratch for repeated calls (no allocation once large enough)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)
        return self.buf


def block_compress(q, k, scale, bias, vl: Varlen, tau, capacity=None, want_mass=False,
                   want_stats=False, workspace: Workspace | None = None, bsr=None, no_alloc=False):
    """Two-phase block-sparse compression. Returns a dict with row_ptr, col_idx,
    vals (bf16 [capacity, 64, 64]), nnz (device int32[1]) and optional masses/stats.
    ``bsr`` may pass preallocated output arrays to reuse. ``no_alloc`` calls
    ``cma_block_compress_noalloc`` (the library's static scratch, no workspace)."""
    torch = _torch()
    lib = load_library()
    H, Tq, d = q.shape
    dev = q.device
    if k.dim() != 3 or k.shape[0] < H or k.shape[2] != d:
        raise ValueError(f"k must be [>= {H}, Tk, {d}] (got {tuple(k.shape)})")
    _need(scale, "scale", H)
    _need(bias, "bias", H)
    _check_rows(vl, Tq, k.shape[1])
    nbr = vl.n_block_rows
    if bsr is not None:
        _need(bsr["row_ptr"], "row_ptr", H * nbr + 1)
        _need(bsr["col_idx"], "col_idx", bsr["capacity"])
        _need(bsr["vals"], "vals", bsr["capacity"] * BLOCK * BLOCK)
    if bsr is None:
        if capacity is None:
            capacity = bsr_max_blocks(H, vl.lens_q, vl.lens_k)
        bsr = dict(row_ptr=torch.empty(H * nbr + 1, dtype=torch.int32, device=dev),
                   col_idx=torch.empty(max(1, capacity), dtype=torch.int32, device=dev),
                   vals=torch.empty((max(1, capacity), BLOCK, BLOCK), dtype=torch.bfloat16, device=dev),
                   nnz=torch.empty(1, dtype=torch.int32, device=dev), capacity=capacity)
    # block masses: block-row r of a sequence with kb0 = (nk - nq) / 64 holds kb0 + r + 1
    n_tri = 0
    for nq_, nk_ in zip(vl.lens_q, vl.lens_k):
        R = (int(nq_) + BLOCK - 1) // BLOCK
        n_tri += R * max(0, (int(nk_) - int(nq_)) // BLOCK) + R * (R + 1) // 2
    mass = torch.empty((H, n_tri), dtype=torch.float32, device=dev) if want_mass else None
    stats = torch.empty((H, Tq, 2), dtype=torch.float32, device=dev) if want_stats else None
    cvl = vl.c(Tq, k.shape[1])
    head = (_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dt(q), H, d, ctypes.byref(cvl), _dev_ptr(scale, "scale"),
            _dev_ptr(bias, "bias"), float(tau), nbr, _dev_ptr(bsr["row_ptr"], "row_ptr"),
            _dev_ptr(bsr["col_idx"], "col_idx"), _dev_ptr(bsr["vals"], "vals"), bsr["capacity"],
            _dev_ptr(bsr["nnz"], "nnz"), _dev_ptr(mass, "block_mass"), _dev_ptr(stats, "row_stats"))
    if no_alloc:
        _check(lib.cma_block_compress_noalloc(*head, _stream()))
    else:
        ws_bytes = lib.cma_block_compress_workspace(H, nbr, vl.max_q, Tq)
        ws = (workspace or Workspace()).get(ws_bytes, dev)
        _check(lib.cma_block_compress(*head, ws.data_ptr(), ws.numel(), _stream()))
    out = dict(bsr)
    out.update(block_mass=mass, row_stats=stats, n_block_rows=nbr, n_key_blocks=vl.n_key_blocks, n_heads=H)
    return out


def mapped_av(src, n_send, M, n_recv, v, vl: Varlen, out_dtype=None, M_seq_stride=None,
              workspace: Workspace | None = None, out=None, q_rows=None, v_layout=V_TOKEN_MAJOR,
              k_rows=None, v_heads=None, split_rows=True):
    """O_h = (sum_j M[h, j] A_j) V_{h // g}, g = n_recv // v_heads (grouped V;
    default v_heads = n_recv). ``M`` is fp32 mixing weights [B, n_recv, n_send],
    or int32 sender indices [B, n_recv] (one sender per receiver head, e.g. the
    cosine argmax: O_h = A_{M[h]} V_{h // g}, block-sparse source only; then
    ``M_seq_stride`` counts int32 entries). ``src`` is either a block_compress result
    (dict with row_ptr/col_idx/vals/n_block_rows, optionally row_end and
    n_key_blocks) or ``("dense", maps, layout)``.
    ``v`` is [v_heads, Tk, d] (V_TOKEN_MAJOR), [v_heads, d, Tk] (V_KEY_MAJOR),
    [v_heads, n_key_blocks, 64 * 128] (V_TILED) or a dict ``{"pages": [v_heads,
    n_pages, 64 * 128], "table": int32 [n_seqs, stride]}`` (V_PAGED); the last two
    serve block-sparse sources only and need ``k_rows`` (Tk). ``q_rows`` is the
    row count of the output tensor (default: Tk). With a dense source the call
    passes the library a workspace in which a launch of few rows splits each row's
    keys over several workgroups; ``split_rows=False`` passes none."""
    torch = _torch()
    lib = load_library()
    pv = None
    dev = v["pages"].device if v_layout == V_PAGED else v.device
    if v_layout == V_PAGED:
        pages, table = v["pages"], v["table"]
        if k_rows is None:
            raise ValueError("V_PAGED needs k_rows (the key rows of the packed sequences)")
        if table.dim() != 2 or table.dtype != torch.int32 or table.shape[0] < vl.n_seqs:
            raise ValueError("the page table must be int32 [n_seqs, stride]")
        H, d, Tk = pages.shape[0], 128, k_rows
        pv = _CPagedV()
        pv.pages = _dev_ptr(pages, "pages")
        pv.page_table = _dev_ptr(table, "page table")
        pv.page_stride = table.shape[1]
        pv.n_pages = pages.shape[1]
        vdt, vptr = _dt(pages), ctypes.addressof(pv)
    elif v_layout == V_KEY_MAJOR:
        H, d, Tk = v.shape
    elif v_layout == V_TILED:
        H, d = v.shape[0], 128
        if k_rows is None:
            raise ValueError("V_TILED needs k_rows (the key rows of the packed sequences)")
        Tk = k_rows
    else:
        H, Tk, d = v.shape
    if pv is None:
        vdt, vptr = _dt(v), _dev_ptr(v, "v")
    n_v = n_recv if v_heads is None else int(v_heads)
    if n_v < 1 or n_recv % n_v:
        raise ValueError(f"v_heads ({n_v}) must be >= 1 and divide n_recv ({n_recv})")
    if H < n_v:
        raise ValueError(f"v holds {H} heads, {n_v} are needed")
    out_dtype = out_dtype or (torch.bfloat16 if pv is not None else v.dtype)
    Tq = q_rows if q_rows is not None else Tk
    _check_rows(vl, Tq, Tk)
    if out is None:
        out = torch.empty((n_recv, Tq, d), dtype=out_dtype, device=dev)
    _need(out, "out", n_recv * Tq * d)
    s = _CMapsSrc()
    if isinstance(src, dict):
        nkb = int(src.get("n_key_blocks") or vl.n_key_blocks)
        if v_layout == V_TILED:
            _need(v, "v", n_v * nkb * BLOCK * 128)
        row_end = src.get("row_end")
        _need(src["row_ptr"], "row_ptr", n_send * src["n_block_rows"] + (0 if row_end is not None else 1))
        _need(row_end, "row_end", n_send * src["n_block_rows"])
        s.kind = SRC_BSR
        s.row_ptr = _dev_ptr(src["row_ptr"], "row_ptr")
        s.col_idx = _dev_ptr(src["col_idx"], "col_idx")
        s.vals = _dev_ptr(src["vals"], "vals")
        s.n_block_rows = src["n_block_rows"]
        s.row_end = _dev_ptr(row_end, "row_end")
        s.n_key_blocks = nkb
    else:
        _, maps, layout = src
        if maps.dim() != 2 or maps.shape[0] < n_send or maps.shape[1] < vl.maps_elems(layout):
            raise ValueError(f"maps must be [>= {n_send}, >= {vl.maps_elems(layout)}] (got {tuple(maps.shape)})")
        s.kind = SRC_DENSE
        s.maps = _dev_ptr(maps, "maps")
        s.maps_dt = _dt(maps)
        s.layout = layout
        s.head_stride = maps.shape[1]
    cvl = vl.c(Tq, Tk)
    if M.dtype == torch.int32:
        if s.kind != SRC_BSR:
            raise ValueError("sender indices need a block-sparse source")
        if M_seq_stride is None:
            M_seq_stride = 0 if M.shape[0] == 1 else n_recv
        _need(M, "sender", M_seq_stride * max(0, vl.n_seqs - 1) + n_recv)
        ws_bytes = lib.cma_mapped_av_indexed_workspace(ctypes.byref(s), n_recv, n_v, d, vl.n_seqs, v_layout)
        ws = (workspace or Workspace()).get(ws_bytes, dev) if ws_bytes else None
        _check(lib.cma_mapped_av_indexed(ctypes.byref(s), n_send, _dev_ptr(M, "sender"), M_seq_stride, n_recv,
                                         n_v, vptr, vdt, v_layout, d, ctypes.byref(cvl),
                                         _dev_ptr(out, "out"), _dt(out),
                                         ws.data_ptr() if ws is not None else None,
                                         ws.numel() if ws is not None else 0, _stream()))
        return out
    if M_seq_stride is None:
        M_seq_stride = 0 if M.shape[0] == 1 else n_recv * n_send
    _need(M, "M", M_seq_stride * max(0, vl.n_seqs - 1) + n_recv * n_send)
    ws_bytes = lib.cma_mapped_av_workspace(ctypes.byref(s), n_v, d, Tk, v_layout)
    if s.kind == SRC_DENSE and not split_rows:
        ws_bytes = 0
    ws = (workspace or Workspace()).get(ws_bytes, dev) if ws_bytes else None
    _check(lib.cma_mapped_av(ctypes.byref(s), n_send, _dev_ptr(M, "M"), M_seq_stride, n_recv, n_v,
                             vptr, vdt, v_layout, d, ctypes.byref(cvl),
                             _dev_ptr(out, "out"), _dt(out),
                             ws.data_ptr() if ws is not None else None,
                             ws.numel() if ws is not None else 0, _stream()))
    return out


def tile_v(v, vl: Varlen, n_block_rows, v_layout=V_TOKEN_MAJOR, out=None):
    """V ([H, Tk, 128] token-major or [H, 128, Tk] key-major, bf16) in the tiled
    operand order [H, n_key_blocks, 64 * 128] that ``mapped_av`` takes with
    ``v_layout=V_TILED`` (then also pass ``k_rows`` = Tk). ``n_block_rows``: the
    key blocks (``vl.n_key_blocks``; for whole prompts the block-rows)."""
    torch = _torch()
    lib = load_library()
    if v_layout == V_KEY_MAJOR:
        H, d, Tk = v.shape
    else:
        H, Tk, d = v.shape
    if out is None:
        out = torch.empty((H, n_block_rows, BLOCK * d), dtype=v.dtype, device=v.device)
    _need(out, "out", H * n_block_rows * BLOCK * d)
    _check_rows(vl, Tk, Tk)
    cvl = vl.c(Tk, Tk)
    _check(lib.cma_tile_v(_dev_ptr(v, "v"), v_layout, H, d, ctypes.byref(cvl), n_block_rows,
                          _dev_ptr(out, "out"), _stream()))
    return out


def tile_v_paged(v, vl: Varlen, pages, table, v_layout=V_TOKEN_MAJOR):
    """Write V's 64-key blocks into the pages of a paged V cache: key block c of
    sequence s goes to page ``table[s, c]`` of ``pages`` ([H, n_pages, 64 * 128]
    bf16), as ``mapped_av`` reads it with ``v_layout=V_PAGED``."""
    lib = load_library()
    if v_layout == V_KEY_MAJOR:
        H, d, Tk = v.shape
    else:
        H, Tk, d = v.shape
    torch = _torch()
    if table.dim() != 2 or table.dtype != torch.int32 or table.shape[0] < vl.n_seqs:
        raise ValueError("the page table must be int32 [n_seqs, stride]")
    if pages.shape[0] < H or pages.shape[2] != BLOCK * d:
        raise ValueError("pages must be [>= H, n_pages, 64 * d]")
    _check_rows(vl, Tk, Tk)
    pv = _CPagedV()
    pv.pages = _dev_ptr(pages, "pages")
    pv.page_table = _dev_ptr(table, "page table")
    pv.page_stride = table.shape[1]
    pv.n_pages = pages.shape[1]
    cvl = vl.c(Tk, Tk)
    _check(lib.cma_tile_v_paged(_dev_ptr(v, "v"), v_layout, H, d, ctypes.byref(cvl), ctypes.byref(pv), _stream()))
    return pages


def prefix_hashes(tokens, seed=0):
    """Chain hashes (uint64) of the whole 64-token blocks of a token sequence."""
    lib = load_library()
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros(max(1, t.size // 64), dtype=np.uint64)
    _check(lib.cma_prefix_hashes(t.ctypes.data, t.size, ctypes.c_uint64(seed & (2 ** 64 - 1)), out.ctypes.data))
    return out[: t.size // 64]


class PrefixIndex:
    """Host-side prefix-hash index of cached block-rows (see cma.h): per (layer,
    prefix hash), every sender head's (first block in the pool, block count)."""

    def __init__(self, n_heads, capacity):
        self.lib = load_library()
        self.n_heads = int(n_heads)
        self.h = self.lib.cma_prefix_index_create(self.n_heads, int(capacity))
        if not self.h:
            raise CmaError(CMA_EINVAL, "cma_prefix_index_create failed")

    def close(self):
        if self.h:
            self.lib.cma_prefix_index_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def __len__(self):
        return int(self.lib.cma_prefix_index_size(self.h))

    def insert(self, layer, h, begin, count):
        b = np.ascontiguousarray(begin, dtype=np.int32)
        c = np.ascontiguousarray(count, dtype=np.int32)
        if b.size != self.n_heads or c.size != self.n_heads:
            raise ValueError(f"begin and count need {self.n_heads} entries")
        return self.lib.cma_prefix_index_insert(self.h, int(layer), ctypes.c_uint64(int(h)), b.ctypes.data,
                                                c.ctypes.data)

    def lookup(self, layer, hashes):
        """(hits, begin [hits, n_heads], count [hits, n_heads]) for the leading run of hits."""
        hs = np.ascontiguousarray(hashes, dtype=np.uint64)
        b = np.zeros((max(1, hs.size), self.n_heads), dtype=np.int32)
        c = np.zeros_like(b)
        n = self.lib.cma_prefix_index_lookup(self.h, int(layer), hs.ctypes.data, hs.size, b.ctypes.data, c.ctypes.data)
        if n < 0:
            raise CmaError(int(n), "cma_prefix_index_lookup failed")
        return int(n), b[:n], c[:n]

    def erase(self, layer, h):
        return self.lib.cma_prefix_index_erase(self.h, int(layer), ctypes.c_uint64(int(h)))

    def evict_lru(self):
        """((layer, hash), begin, count) of the evicted entry, or None if empty."""
        layer, h = ctypes.c_int32(0), ctypes.c_uint64(0)
        b = np.zeros(self.n_heads, dtype=np.int32)
        c = np.zeros_like(b)
        r = self.lib.cma_prefix_index_evict_lru(self.h, ctypes.byref(layer), ctypes.byref(h), b.ctypes.data,
                                                c.ctypes.data)
        return ((int(layer.value), int(h.value)), b, c) if r == 1 else None


def onehot_mix(argmax, n_send):
    torch = _torch()
    lib = load_library()
    B, Hr = argmax.shape
    M = torch.empty((B, Hr, n_send), dtype=torch.float32, device=argmax.device)
    _check(lib.cma_onehot_mix(_dev_ptr(argmax, "argmax"), B, Hr, n_send, _dev_ptr(M, "M"), _stream()))
    return M


def mapped_layers(n_layers, ratio):
    lib = load_library()
    buf = (ctypes.c_int32 * max(1, n_layers))()
    n = lib.cma_mapped_layers(n_layers, float(ratio), buf, n_layers)
    if n < 0:
        raise CmaError(n, lib.cma_last_error().decode())
    return [int(buf[i]) for i in range(n)]


def mapping_plan(prompt_lens, tau_e, tau_t):
    """IAM's tau_e / tau_t thresholds per request: (tokens to generate before the
    head map is built, leading context tokens the similarity uses), as lists."""
    lib = load_library()
    p = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    gen = np.zeros(p.size, dtype=np.int32)
    sim = np.zeros(p.size, dtype=np.int32)
    _check(lib.cma_mapping_plan(p.size, p.ctypes.data, int(tau_e), int(tau_t), gen.ctypes.data, sim.ctypes.data))
    return [int(v) for v in gen], [int(v) for v in sim]


def timing_enable(on=True):
    """Bracket every library kernel launch with HIP events on its own stream."""
    load_library().cma_timing_enable(1 if on else 0)


def timing_collect():
    """Wait for recorded events and return {kernel: (total_ms, launches)} so far."""
    lib = load_library()
    _check(lib.cma_timing_collect())
    out = {}
    i = 0
    while True:
        name = lib.cma_timing_name(i)
        if name is None:
            break
        n = ctypes.c_int64(0)
        ms = lib.cma_timing_get(name, ctypes.byref(n))
        out[name.decode()] = (ms, int(n.value))
        i += 1
    return out


def timing_reset():
    load_library().cma_timing_reset()
