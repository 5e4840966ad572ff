"""ctypes binding of libcrisp.so (the C ABI declared in include/crisp.h).

Argument marshalling only: every function here forwards device pointers,
sizes and torch's current HIP stream to the library, and raises CrispError
on a non-zero status.  Nothing is computed on the host, and there is no
fallback: if the library is missing, every call fails loudly.

Functions keep the C names.  Tensors must be contiguous and live on the GPU
that is current.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcrisp.so")

CRISP_OK = 0
STATUS_NAMES = {0: "CRISP_OK", 1: "CRISP_ERR_NULL", 2: "CRISP_ERR_SHAPE", 3: "CRISP_ERR_PARAM",
                4: "CRISP_ERR_ALIGN", 5: "CRISP_ERR_WORKSPACE", 6: "CRISP_ERR_DEVICE", 7: "CRISP_ERR_LAUNCH"}

ROUTE_PE, ROUTE_VS = 0, 1
ROUTE_AUTO, ROUTE_FORCE_VS, ROUTE_FORCE_PE = 0, 1, 2
NF_MEDIAN, NF_MEAN = 0, 1


class CrispError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


class crisp_dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("scale", ctypes.c_float)]


class crisp_cfg(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("alpha", ctypes.c_float), ("gamma_pe", ctypes.c_float),
                ("kmin_blocks", ctypes.c_int32), ("sink_width", ctypes.c_int32), ("recency_width", ctypes.c_int32),
                ("nf_stat", ctypes.c_int32), ("route_override", ctypes.c_int32)]


class crisp_blocks(ctypes.Structure):
    _fields_ = [("count", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("v_score", ctypes.c_void_p),
                ("s_score", ctypes.c_void_p), ("floor_v", ctypes.c_void_p), ("floor_s", ctypes.c_void_p),
                ("v_mask", ctypes.c_void_p), ("s_mask", ctypes.c_void_p), ("n_v", ctypes.c_void_p),
                ("n_s", ctypes.c_void_p)]


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "crisp_proxy": (ctypes.c_int, [ctypes.POINTER(crisp_dims), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "crisp_proxy_scratch_bytes": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_route": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), _P, _P, _P, _P, _P]),
    "crisp_route_cols": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), _P, _P, _P, _P]),
    "crisp_proxy_cols": (ctypes.c_int, [ctypes.POINTER(crisp_dims), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "crisp_select_tokens": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), _P, _P, _P, _P,
                                           _P, ctypes.POINTER(crisp_blocks), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "crisp_sparse_attn_cols": (ctypes.c_int, [ctypes.POINTER(crisp_dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "crisp_route_jsd": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.c_float, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "crisp_route_jsd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_select": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), _P, _P, _P, _P, _P,
                                    ctypes.POINTER(crisp_blocks), _P, ctypes.c_size_t, _P]),
    "crisp_select_gamma": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), ctypes.c_float, _P,
                                          _P, _P, _P, _P, ctypes.POINTER(crisp_blocks), _P, ctypes.c_size_t, _P]),
    "crisp_select_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_select_noalloc": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), _P, _P, _P, _P,
                                            _P, ctypes.POINTER(crisp_blocks), _P]),
    "crisp_list_capacity": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_sparse_attn": (ctypes.c_int, [ctypes.POINTER(crisp_dims), _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                         _P, ctypes.c_size_t, _P]),
    "crisp_dense_attn": (ctypes.c_int, [ctypes.POINTER(crisp_dims), _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                        ctypes.c_size_t, _P]),
    "crisp_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_prefill": (ctypes.c_int, [ctypes.POINTER(crisp_dims), ctypes.POINTER(crisp_cfg), ctypes.c_int32, _P, _P,
                                     _P, ctypes.POINTER(crisp_blocks), _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                     ctypes.c_size_t, _P]),
    "crisp_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(crisp_dims)]),
    "crisp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "crisp_abi_version": (ctypes.c_int32, []),
}


def lib() -> ctypes.CDLL:
    """Load libcrisp.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libcrisp.so not found at {LIB_PATH}: build it with "
                               "`python -m dynamic_sparse_attention_proxy_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int):
    if status != CRISP_OK:
        raise CrispError(fn, status, lib().crisp_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcrisp must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def num_blocks(seq_len: int, block: int = 128) -> int:
    """Key/query blocks of a sequence: the last one is partial when `block`
    does not divide `seq_len`."""
    return -(-seq_len // block)


def make_dims(num_q_heads: int, num_kv_heads: int, seq_len: int, head_dim: int = 128, block: int = 128,
              scale: Optional[float] = None) -> crisp_dims:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return crisp_dims(num_q_heads, num_kv_heads, seq_len, head_dim, block, scale)


def make_cfg(tau: float = 0.5, alpha: float = 1.25, gamma_pe: float = 0.95, kmin_blocks: int = 8,
             sink_width: int = 128, recency_width: int = 128, nf_stat: int = NF_MEDIAN,
             route_override: int = ROUTE_AUTO) -> crisp_cfg:
    return crisp_cfg(tau, alpha, gamma_pe, kmin_blocks, sink_width, recency_width, nf_stat, route_override)


def crisp_proxy_scratch_bytes(dims: crisp_dims) -> int:
    return int(lib().crisp_proxy_scratch_bytes(ctypes.byref(dims)))


def crisp_select_workspace_bytes(dims: crisp_dims) -> int:
    return int(lib().crisp_select_workspace_bytes(ctypes.byref(dims)))


def crisp_prefill_workspace_bytes(dims: crisp_dims) -> int:
    return int(lib().crisp_prefill_workspace_bytes(ctypes.byref(dims)))


def crisp_list_capacity(dims: crisp_dims) -> int:
    return int(lib().crisp_list_capacity(ctypes.byref(dims)))


def crisp_abi_version() -> int:
    return int(lib().crisp_abi_version())


def crisp_proxy(dims: crisp_dims, q, k, attn_map, row_lse=None, partials=None, stream=None, block_mass=None):
    nbytes = partials.numel() * partials.element_size() if partials is not None else 0
    _check("crisp_proxy", lib().crisp_proxy(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(attn_map), _ptr(block_mass),
                                            _ptr(row_lse), _ptr(partials), nbytes, _stream(stream)))


def crisp_route(dims: crisp_dims, cfg: crisp_cfg, attn_map, c_struct, route, stream=None, block_mass=None):
    _check("crisp_route", lib().crisp_route(ctypes.byref(dims), ctypes.byref(cfg), _ptr(attn_map), _ptr(block_mass),
                                            _ptr(c_struct), _ptr(route), _stream(stream)))


def crisp_route_cols(dims: crisp_dims, cfg: crisp_cfg, col_mass, c_struct, route, stream=None):
    _check("crisp_route_cols", lib().crisp_route_cols(ctypes.byref(dims), ctypes.byref(cfg), _ptr(col_mass),
                                                      _ptr(c_struct), _ptr(route), _stream(stream)))


def crisp_proxy_cols(dims: crisp_dims, q, k, block_mass, col_mass, row_lse=None, partials=None, stream=None):
    nbytes = partials.numel() * partials.element_size() if partials is not None else 0
    _check("crisp_proxy_cols", lib().crisp_proxy_cols(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(block_mass),
                                                      _ptr(col_mass), _ptr(row_lse), _ptr(partials), nbytes,
                                                      _stream(stream)))


def crisp_route_jsd_workspace_bytes(dims: crisp_dims) -> int:
    return int(lib().crisp_route_jsd_workspace_bytes(ctypes.byref(dims)))


def crisp_route_jsd(dims: crisp_dims, tau_jsd: float, q, k, block_mass, js_dist, route, workspace, estimate=None,
                    stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("crisp_route_jsd", lib().crisp_route_jsd(ctypes.byref(dims), ctypes.c_float(tau_jsd), _ptr(q), _ptr(k),
                                                    _ptr(block_mass), _ptr(js_dist), _ptr(route), _ptr(estimate),
                                                    _ptr(workspace), nbytes, _stream(stream)))


def _blocks(out: dict) -> crisp_blocks:
    b = crisp_blocks()
    for name, _ in crisp_blocks._fields_:
        t = out.get(name)
        setattr(b, name, None if t is None else _ptr(t).value)
    return b


def crisp_select(dims: crisp_dims, cfg: crisp_cfg, q, k, attn_map, route, out: dict, workspace, stream=None,
                 block_mass=None):
    b = _blocks(out)
    _check("crisp_select", lib().crisp_select(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                              _ptr(attn_map), _ptr(block_mass), _ptr(route), ctypes.byref(b),
                                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)))


# CRISP_NOALLOC_SCRATCH_BYTES of include/crisp.h: the largest selection
# workspace crisp_select_noalloc serves from its static per-device scratch.
NOALLOC_SCRATCH_BYTES = 32 << 20


def crisp_select_noalloc(dims: crisp_dims, cfg: crisp_cfg, q, k, attn_map, route, out: dict, stream=None,
                         block_mass=None):
    b = _blocks(out)
    _check("crisp_select_noalloc", lib().crisp_select_noalloc(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                                              _ptr(attn_map), _ptr(block_mass), _ptr(route),
                                                              ctypes.byref(b), _stream(stream)))


def crisp_select_gamma(dims: crisp_dims, cfg: crisp_cfg, gamma: float, q, k, attn_map, route, out: dict,
                       workspace, stream=None, block_mass=None):
    b = _blocks(out)
    _check("crisp_select_gamma", lib().crisp_select_gamma(ctypes.byref(dims), ctypes.byref(cfg), gamma, _ptr(q),
                                                          _ptr(k), _ptr(attn_map), _ptr(block_mass), _ptr(route),
                                                          ctypes.byref(b), _ptr(workspace),
                                                          workspace.numel() * workspace.element_size(),
                                                          _stream(stream)))


def crisp_select_tokens(dims: crisp_dims, cfg: crisp_cfg, q, k, block_mass, col_mass, route, out: dict, cols,
                        ncols, col_below, workspace, stream=None):
    b = _blocks(out)
    _check("crisp_select_tokens", lib().crisp_select_tokens(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                                            _ptr(block_mass), _ptr(col_mass), _ptr(route),
                                                            ctypes.byref(b), _ptr(cols), _ptr(ncols),
                                                            _ptr(col_below), _ptr(workspace),
                                                            workspace.numel() * workspace.element_size(),
                                                            _stream(stream)))


def crisp_attn_workspace_bytes(dims: crisp_dims) -> int:
    return int(lib().crisp_attn_workspace_bytes(ctypes.byref(dims)))


def _attn_workspace(dims, out, workspace):
    # the attention kernels' work queue; a fresh one per call unless given
    if workspace is None:
        workspace = torch.empty(crisp_attn_workspace_bytes(dims), dtype=torch.uint8, device=out.device)
    return workspace


def crisp_sparse_attn_cols(dims: crisp_dims, q, k, v, count, idx, cols, col_below, out, lse, stream=None,
                           workspace=None):
    if out.dtype != torch.float32:
        raise TypeError("crisp_sparse_attn_cols updates an fp32 output in place")
    ws = _attn_workspace(dims, out, workspace)
    _check("crisp_sparse_attn_cols", lib().crisp_sparse_attn_cols(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                                                  _ptr(count), _ptr(idx), _ptr(cols),
                                                                  _ptr(col_below), _ptr(out), _ptr(lse), _ptr(ws),
                                                                  ws.numel() * ws.element_size(), _stream(stream)))


def crisp_sparse_attn(dims: crisp_dims, q, k, v, count, idx, out, lse=None, stream=None, workspace=None):
    out_fp32 = 1 if out.dtype == torch.float32 else 0
    ws = _attn_workspace(dims, out, workspace)
    _check("crisp_sparse_attn", lib().crisp_sparse_attn(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(count),
                                                        _ptr(idx), _ptr(out), out_fp32, _ptr(lse), _ptr(ws),
                                                        ws.numel() * ws.element_size(), _stream(stream)))


def crisp_dense_attn(dims: crisp_dims, q, k, v, out, lse=None, stream=None, workspace=None):
    out_fp32 = 1 if out.dtype == torch.float32 else 0
    ws = _attn_workspace(dims, out, workspace)
    _check("crisp_dense_attn", lib().crisp_dense_attn(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                      out_fp32, _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                                      _stream(stream)))


# --------------------------------------------------------------------------
# Buffer bundle for one layer (device memory from torch; no computation).
# --------------------------------------------------------------------------


class CrispBuffers:
    """Device buffers of one layer's CRISP chain, allocated once and reused.

    The proxy map itself (4 * 128 * n * Hq bytes) is only allocated with
    `with_map=True`; the chain otherwise runs on the block masses."""

    def __init__(self, dims: crisp_dims, device=None, out_dtype=torch.bfloat16, diagnostics: bool = True,
                 with_map: bool = False, tokens: bool = False):
        dev = torch.device("cuda") if device is None else torch.device(device)
        hq, n = dims.num_q_heads, dims.seq_len
        N = num_blocks(n, dims.block)
        f32, i32 = torch.float32, torch.int32
        self.dims = dims
        self.attn_map = torch.empty((hq, dims.block, n), dtype=f32, device=dev) if with_map else None
        self.block_mass = torch.empty((4, hq, N), dtype=f32, device=dev)
        self.row_lse = torch.empty((hq, dims.block), dtype=f32, device=dev)
        # one buffer for the one-call layer; the step-by-step calls use its
        # start as the proxy scratch and, from the scratch size rounded up to
        # 256 bytes, the selection workspace (crisp.h guarantees the room)
        self.prefill_workspace = torch.empty(crisp_prefill_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        ps, ws = crisp_proxy_scratch_bytes(dims), crisp_select_workspace_bytes(dims)
        off = -(-ps // 256) * 256
        self.partials = self.prefill_workspace[:ps]
        self.workspace = self.prefill_workspace[off:off + ws]
        self.c_struct = torch.empty((hq,), dtype=f32, device=dev)
        self.route = torch.empty((hq,), dtype=i32, device=dev)
        self.blocks = {"count": torch.empty((hq, N), dtype=i32, device=dev),
                       "idx": torch.empty((crisp_list_capacity(dims),), dtype=i32, device=dev)}
        if diagnostics:
            self.blocks.update({
                "v_score": torch.empty((hq, N), dtype=f32, device=dev),
                "s_score": torch.empty((hq, N), dtype=f32, device=dev),
                "floor_v": torch.empty((hq,), dtype=f32, device=dev),
                "floor_s": torch.empty((hq,), dtype=f32, device=dev),
                "v_mask": torch.empty((hq, N), dtype=i32, device=dev),
                "s_mask": torch.empty((hq, N), dtype=i32, device=dev),
                "n_v": torch.empty((hq,), dtype=i32, device=dev),
                "n_s": torch.empty((hq,), dtype=i32, device=dev),
            })
        if tokens:  # token-granular vertical selection; its attention output is fp32
            self.col_mass = torch.empty((hq, n), dtype=f32, device=dev)
            self.cols = torch.empty((hq, n), dtype=i32, device=dev)
            self.ncols = torch.empty((hq,), dtype=i32, device=dev)
            self.col_below = torch.empty((hq, N), dtype=i32, device=dev)
            out_dtype = f32
        self.out = torch.empty((hq, n, dims.head_dim), dtype=out_dtype, device=dev)
        self.lse = torch.empty((hq, n), dtype=f32, device=dev)
        self.attn_workspace = torch.empty(crisp_attn_workspace_bytes(dims), dtype=torch.uint8, device=dev)


# Context-length gate (ai.info summary: "Main Findings" puts the crossover
# where sparse prefill starts to pay between 8K and 64K, and "Why This
# Matters" suggests gating sparse prefill on a context-length threshold).
# The gate lives in the library's crisp_prefill; None here asks for its
# default, CRISP_DENSE_BELOW_DEFAULT (16384 tokens).
DENSE_BELOW = 16384  # the library default, mirrored for reporting and tests


def crisp_prefill(dims: crisp_dims, cfg: crisp_cfg, q, k, v, bufs: CrispBuffers, gamma: Optional[float] = None,
                  stream=None, use_map: bool = False, dense_below: Optional[int] = None):
    """One layer's path on `stream`.

    With no map in `bufs` and no `gamma`, this is the library's one-call
    layer (crisp_prefill in the C ABI): below the context-length gate
    (`dense_below` tokens, None for the library default) the dense kernel
    alone, else proxy -> route -> select -> block-sparse attention on the
    block masses.  With a map in bufs (CrispBuffers(with_map=True)) or a
    `gamma` (the gamma-cumulative comparison chain), the same steps are
    called one by one and never gated; routing and selection then read the
    block masses unless `use_map` asks for the materialised map."""
    if gamma is None and bufs.attn_map is None and not use_map:
        b = _blocks(bufs.blocks)
        out_fp32 = 1 if bufs.out.dtype == torch.float32 else 0
        ws = bufs.prefill_workspace
        _check("crisp_prefill", lib().crisp_prefill(ctypes.byref(dims), ctypes.byref(cfg),
                                                    -1 if dense_below is None else int(dense_below), _ptr(q),
                                                    _ptr(k), _ptr(v), ctypes.byref(b), _ptr(bufs.block_mass),
                                                    _ptr(bufs.c_struct), _ptr(bufs.route), _ptr(bufs.out), out_fp32,
                                                    _ptr(bufs.lse), _ptr(ws), ws.numel(), _stream(stream)))
        return bufs.out
    if use_map and bufs.attn_map is None:
        raise ValueError("use_map needs CrispBuffers(with_map=True)")
    mass = None if use_map else bufs.block_mass
    amap = bufs.attn_map if use_map else None
    crisp_proxy(dims, q, k, bufs.attn_map, bufs.row_lse, bufs.partials, stream, block_mass=bufs.block_mass)
    crisp_route(dims, cfg, amap, bufs.c_struct, bufs.route, stream, block_mass=mass)
    if gamma is None:
        crisp_select(dims, cfg, q, k, amap, bufs.route, bufs.blocks, bufs.workspace, stream, block_mass=mass)
    else:
        crisp_select_gamma(dims, cfg, gamma, q, k, amap, bufs.route, bufs.blocks, bufs.workspace, stream,
                           block_mass=mass)
    crisp_sparse_attn(dims, q, k, v, bufs.blocks["count"], bufs.blocks["idx"], bufs.out, bufs.lse, stream,
                      workspace=bufs.attn_workspace)
    return bufs.out


def crisp_prefill_tokens(dims: crisp_dims, cfg: crisp_cfg, q, k, v, bufs: CrispBuffers, stream=None):
    """One layer with token-granular vertical selection: proxy with column
    masses -> route -> select (kept columns; slash bands as in the block
    rule) -> tile attention -> the kept columns merged in.  bufs must come
    from CrispBuffers(tokens=True); the output is fp32."""
    if not hasattr(bufs, "cols"):
        raise ValueError("crisp_prefill_tokens needs CrispBuffers(tokens=True)")
    crisp_proxy_cols(dims, q, k, bufs.block_mass, bufs.col_mass, bufs.row_lse, bufs.partials, stream)
    crisp_route(dims, cfg, None, bufs.c_struct, bufs.route, stream, block_mass=bufs.block_mass)
    crisp_select_tokens(dims, cfg, q, k, bufs.block_mass, bufs.col_mass, bufs.route, bufs.blocks, bufs.cols,
                        bufs.ncols, bufs.col_below, bufs.workspace, stream)
    crisp_sparse_attn(dims, q, k, v, bufs.blocks["count"], bufs.blocks["idx"], bufs.out, bufs.lse, stream,
                      workspace=bufs.attn_workspace)
    crisp_sparse_attn_cols(dims, q, k, v, bufs.blocks["count"], bufs.blocks["idx"], bufs.cols, bufs.col_below,
                           bufs.out, bufs.lse, stream, workspace=bufs.attn_workspace)
    return bufs.out
