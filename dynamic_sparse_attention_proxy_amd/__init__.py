"""CRISP sparse prefill on AMD MI355X: Python binding of ``libcrisp.so``.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C-ABI declared in ``include/crisp.h``.  PyTorch supplies device
memory and the stream.  Importing works without a GPU; calling a compute
entry point without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcrisp.so")

F32, BF16 = 0, 1
SELECT_NOISE_FLOOR, SELECT_KEEP_ALL, SELECT_CUMULATIVE = 0, 1, 2

STATUS = {0: "CRISP_OK", -1: "CRISP_ERR_NULL", -2: "CRISP_ERR_SHAPE", -3: "CRISP_ERR_DTYPE",
          -4: "CRISP_ERR_CONFIG", -5: "CRISP_ERR_WORKSPACE", -6: "CRISP_ERR_CAPACITY", -7: "CRISP_ERR_HIP",
          -8: "CRISP_ERR_ALIGN", -9: "CRISP_ERR_SCRATCH"}

EXPORTS = ["crisp_workspace_size", "crisp_index_capacity", "crisp_route", "crisp_select_indices",
           "crisp_sparse_prefill", "crisp_sparse_prefill_noalloc", "crisp_dense_prefill", "crisp_route_jsd",
           "crisp_tile_layout_of", "crisp_status_string"]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("w_sink", ctypes.c_int32), ("w_local", ctypes.c_int32),
                ("tau_num", ctypes.c_uint32), ("tau_den", ctypes.c_uint32),
                ("alpha_num", ctypes.c_uint32), ("alpha_den", ctypes.c_uint32),
                ("gamma_num", ctypes.c_uint32), ("gamma_den", ctypes.c_uint32),
                ("select_mode", ctypes.c_int32)]


class RelBias(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("offsets", ctypes.c_void_p), ("values", ctypes.c_void_p)]


class IndexSets(ctypes.Structure):
    _fields_ = [("route", ctypes.c_void_p), ("cstruct_num", ctypes.c_void_p), ("mass_v", ctypes.c_void_p),
                ("mass_s", ctypes.c_void_p), ("mass_total", ctypes.c_void_p), ("vs_count", ctypes.c_void_p),
                ("vs_vertical", ctypes.c_void_p), ("vs_slash", ctypes.c_void_p),
                ("pe_rowptr", ctypes.c_void_p), ("pe_col", ctypes.c_void_p), ("pe_cap", ctypes.c_int64)]


class TileLayout(ctypes.Structure):
    _fields_ = [("list_offset", ctypes.c_int64), ("count_offset", ctypes.c_int64), ("list_stride", ctypes.c_int64),
                ("n_lists", ctypes.c_int32), ("pair_lists", ctypes.c_int32)]


class CrispError(RuntimeError):
    pass


_lib = None


def load_library(path: str = None):
    """Load libcrisp.so (built by ``dynamic_sparse_attention_proxy_amd.build``, or the
    build named by the CRISP_LIB environment variable); raise if missing."""
    global _lib
    path = path or os.environ.get("CRISP_LIB") or LIB_PATH
    if _lib is None:
        # torch first, so that the library binds to the HIP runtime torch brings
        # rather than pulling in the system's ahead of it (the two do not mix in
        # one process: kernel launches then fail)
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise CrispError(f"{path} is missing: build it with `python -m dynamic_sparse_attention_proxy_amd.build`")
        lib = ctypes.CDLL(path)
        P, S, C = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Config)
        lib.crisp_workspace_size.argtypes = [S, C]
        lib.crisp_workspace_size.restype = ctypes.c_size_t
        lib.crisp_index_capacity.argtypes = [S, C]
        lib.crisp_index_capacity.restype = ctypes.c_int64
        lib.crisp_route.argtypes = [S, C, P, P, ctypes.POINTER(RelBias), P, ctypes.c_size_t,
                                    ctypes.POINTER(IndexSets), P]
        lib.crisp_route.restype = ctypes.c_int
        lib.crisp_select_indices.argtypes = [S, C, P, P, P, ctypes.c_size_t, ctypes.POINTER(IndexSets), P]
        lib.crisp_select_indices.restype = ctypes.c_int
        lib.crisp_sparse_prefill.argtypes = [S, C, P, P, P, ctypes.POINTER(RelBias), ctypes.POINTER(IndexSets), P,
                                             ctypes.c_size_t, P, P]
        lib.crisp_sparse_prefill.restype = ctypes.c_int
        lib.crisp_sparse_prefill_noalloc.argtypes = [S, C, P, P, P, ctypes.POINTER(RelBias),
                                                     ctypes.POINTER(IndexSets), P, P]
        lib.crisp_sparse_prefill_noalloc.restype = ctypes.c_int
        lib.crisp_dense_prefill.argtypes = [S, C, P, P, P, ctypes.POINTER(RelBias), P, ctypes.c_size_t, P, P]
        lib.crisp_dense_prefill.restype = ctypes.c_int
        lib.crisp_route_jsd.argtypes = [S, C, ctypes.c_uint32, ctypes.c_uint32, P, P, ctypes.POINTER(IndexSets), P,
                                        ctypes.c_size_t, P, P, P, P]
        lib.crisp_route_jsd.restype = ctypes.c_int
        lib.crisp_tile_layout_of.argtypes = [S, C, ctypes.POINTER(TileLayout)]
        lib.crisp_tile_layout_of.restype = ctypes.c_int
        lib.crisp_status_string.argtypes = [ctypes.c_int]
        lib.crisp_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(code: int, what: str):
    if code != 0:
        msg = load_library().crisp_status_string(code).decode()
        raise CrispError(f"{what}: {STATUS.get(code, code)} ({msg})")


@dataclass
class LayerSpec:
    """Shape and hyper-parameters of one prefill layer."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    dtype: int  # F32 or BF16
    block: int = 128
    w_sink: int = 128
    w_local: int = 128
    tau: tuple = (1, 10)
    alpha: tuple = (1, 1)
    gamma: tuple = (19, 20)
    select_mode: int = SELECT_NOISE_FLOOR

    def shape(self) -> Shape:
        return Shape(self.batch, self.n_q_heads, self.n_kv_heads, self.seq_len, self.head_dim, self.dtype)

    def config(self) -> Config:
        return Config(self.block, self.w_sink, self.w_local, self.tau[0], self.tau[1], self.alpha[0],
                      self.alpha[1], self.gamma[0], self.gamma[1], self.select_mode)

    @property
    def num_blocks(self) -> int:
        return (self.seq_len + self.block - 1) // self.block

    @property
    def heads(self) -> int:
        return self.batch * self.n_q_heads


def workspace_size(spec: LayerSpec) -> int:
    return int(load_library().crisp_workspace_size(ctypes.byref(spec.shape()), ctypes.byref(spec.config())))


def index_capacity(spec: LayerSpec) -> int:
    return int(load_library().crisp_index_capacity(ctypes.byref(spec.shape()), ctypes.byref(spec.config())))


class Buffers:
    """Device buffers for one layer: routing outputs, index sets and workspace (torch tensors)."""

    def __init__(self, spec: LayerSpec, device="cuda"):
        import torch
        bh, nb = spec.heads, spec.num_blocks
        cap = index_capacity(spec)
        if cap < 0:
            raise CrispError("invalid layer spec")
        i32, i64 = torch.int32, torch.int64
        self.spec = spec
        self.route = torch.zeros(bh, dtype=torch.uint8, device=device)
        self.cstruct_num = torch.zeros(bh, dtype=i64, device=device)
        self.mass_v = torch.zeros(bh, nb, dtype=i64, device=device)
        self.mass_s = torch.zeros(bh, nb, dtype=i64, device=device)
        self.mass_total = torch.zeros(bh, dtype=i64, device=device)
        self.vs_count = torch.zeros(bh, 2, dtype=i32, device=device)
        self.vs_vertical = torch.zeros(bh, nb, dtype=i32, device=device)
        self.vs_slash = torch.zeros(bh, nb, dtype=i32, device=device)
        self.pe_rowptr = torch.zeros(bh, nb + 1, dtype=i32, device=device)
        self.pe_col = torch.zeros(bh, cap, dtype=i32, device=device)
        self.pe_cap = cap
        self.ws_bytes = workspace_size(spec)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def index_sets(self) -> IndexSets:
        return IndexSets(self.route.data_ptr(), self.cstruct_num.data_ptr(), self.mass_v.data_ptr(),
                         self.mass_s.data_ptr(), self.mass_total.data_ptr(), self.vs_count.data_ptr(),
                         self.vs_vertical.data_ptr(), self.vs_slash.data_ptr(), self.pe_rowptr.data_ptr(),
                         self.pe_col.data_ptr(), self.pe_cap)


def _tensor(t, numel, dtype, what):
    """Device pointer of t after checking what the C-ABI assumes of it (device memory,
    contiguous, element type, element count); raises CrispError otherwise."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise CrispError(f"{what}: expected a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise CrispError(f"{what}: expected a contiguous tensor")
    if t.dtype != dtype:
        raise CrispError(f"{what}: expected {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise CrispError(f"{what}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _act_dtype(spec: LayerSpec):
    import torch
    return torch.bfloat16 if spec.dtype == BF16 else torch.float32


def _qkvo(spec: LayerSpec, **tensors):
    """Pointers of q / o ([batch, n_q_heads, seq_len, head_dim]) and k / v
    ([batch, n_kv_heads, seq_len, head_dim]) in the spec's element type."""
    dt = _act_dtype(spec)
    per_head = spec.seq_len * spec.head_dim
    out = {}
    for name, t in tensors.items():
        heads = spec.n_q_heads if name in ("q", "o") else spec.n_kv_heads
        out[name] = _tensor(t, spec.batch * heads * per_head, dt, name)
    return out


def _bias(spec: LayerSpec, offsets, values) -> RelBias:
    import torch
    if offsets is None or offsets.numel() == 0:
        return RelBias(0, None, None)
    count = int(offsets.shape[-1])
    n = spec.heads * count
    return RelBias(count, _tensor(offsets, n, torch.int32, "bias_offsets"),
                   _tensor(values, n, torch.float32, "bias_values"))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def route(spec: LayerSpec, q, k, bufs: Buffers, bias_offsets=None, bias_values=None, stream=None):
    """crisp_route: proxy map of the last query block, C_struct and route bits into ``bufs``."""
    idx = bufs.index_sets()
    b = _bias(spec, bias_offsets, bias_values)
    p = _qkvo(spec, q=q, k=k)
    _check(load_library().crisp_route(ctypes.byref(spec.shape()), ctypes.byref(spec.config()), p["q"], p["k"],
                                      ctypes.byref(b), bufs.ws.data_ptr(), bufs.ws_bytes, ctypes.byref(idx),
                                      _stream(stream)), "crisp_route")


def select_indices(spec: LayerSpec, q, k, bufs: Buffers, stream=None):
    """crisp_select_indices: VS block lists (Eq. 3-4) and PE block sets (Alg. 4) into ``bufs``."""
    idx = bufs.index_sets()
    p = _qkvo(spec, q=q, k=k)
    _check(load_library().crisp_select_indices(ctypes.byref(spec.shape()), ctypes.byref(spec.config()), p["q"],
                                               p["k"], bufs.ws.data_ptr(), bufs.ws_bytes, ctypes.byref(idx),
                                               _stream(stream)), "crisp_select_indices")


def sparse_prefill(spec: LayerSpec, q, k, v, o, bufs: Buffers, bias_offsets=None, bias_values=None,
                   stream=None):
    """crisp_sparse_prefill: attention over the selected blocks, written into ``o``."""
    idx = bufs.index_sets()
    b = _bias(spec, bias_offsets, bias_values)
    p = _qkvo(spec, q=q, k=k, v=v, o=o)
    _check(load_library().crisp_sparse_prefill(ctypes.byref(spec.shape()), ctypes.byref(spec.config()), p["q"],
                                               p["k"], p["v"], ctypes.byref(b), ctypes.byref(idx),
                                               bufs.ws.data_ptr(), bufs.ws_bytes, p["o"], _stream(stream)),
           "crisp_sparse_prefill")


def sparse_prefill_noalloc(spec: LayerSpec, q, k, v, o, bufs: Buffers, bias_offsets=None, bias_values=None,
                           stream=None):
    """crisp_sparse_prefill_noalloc: the same attention with the library's static scratch
    (no workspace; ``bufs`` supplies only the index sets)."""
    idx = bufs.index_sets()
    b = _bias(spec, bias_offsets, bias_values)
    p = _qkvo(spec, q=q, k=k, v=v, o=o)
    _check(load_library().crisp_sparse_prefill_noalloc(ctypes.byref(spec.shape()), ctypes.byref(spec.config()),
                                                       p["q"], p["k"], p["v"], ctypes.byref(b), ctypes.byref(idx),
                                                       p["o"], _stream(stream)), "crisp_sparse_prefill_noalloc")


def dense_prefill(spec: LayerSpec, q, k, v, o, bufs: Buffers, bias_offsets=None, bias_values=None,
                  stream=None):
    """crisp_dense_prefill: full causal attention with the same tile engine (``bufs`` supplies the workspace)."""
    b = _bias(spec, bias_offsets, bias_values)
    p = _qkvo(spec, q=q, k=k, v=v, o=o)
    _check(load_library().crisp_dense_prefill(ctypes.byref(spec.shape()), ctypes.byref(spec.config()), p["q"],
                                              p["k"], p["v"], ctypes.byref(b), bufs.ws.data_ptr(), bufs.ws_bytes,
                                              p["o"], _stream(stream)), "crisp_dense_prefill")


def route_jsd(spec: LayerSpec, q, k, bufs: Buffers, route_out, jsd_out, tau_jsd=(1, 100), pooled_out=None,
              stream=None):
    """crisp_route_jsd: the divergence router on the proxy that ``route`` left in ``bufs``.
    route_out [BH] uint8, jsd_out [BH] int64 (JSD = value * 2^-53), pooled_out [BH, N_b]
    int64 or None."""
    import torch
    idx = bufs.index_sets()
    p = _qkvo(spec, q=q, k=k)
    bh = spec.heads
    r_ptr = _tensor(route_out, bh, torch.uint8, "route_out")
    j_ptr = _tensor(jsd_out, bh, torch.int64, "jsd_out")
    p_ptr = None if pooled_out is None else _tensor(pooled_out, bh * spec.num_blocks, torch.int64, "pooled_out")
    _check(load_library().crisp_route_jsd(ctypes.byref(spec.shape()), ctypes.byref(spec.config()), tau_jsd[0],
                                          tau_jsd[1], p["q"], p["k"], ctypes.byref(idx), bufs.ws.data_ptr(),
                                          bufs.ws_bytes, r_ptr, j_ptr, p_ptr, _stream(stream)), "crisp_route_jsd")


def tile_layout(spec: LayerSpec) -> dict:
    """crisp_tile_layout_of: where crisp_sparse_prefill keeps its key-tile lists inside the workspace."""
    out = TileLayout()
    _check(load_library().crisp_tile_layout_of(ctypes.byref(spec.shape()), ctypes.byref(spec.config()),
                                               ctypes.byref(out)), "crisp_tile_layout_of")
    return {name: int(getattr(out, name)) for name, _ in TileLayout._fields_}


def tile_lists(spec: LayerSpec, bufs: Buffers):
    """The key-tile lists the last crisp_sparse_prefill call left in ``bufs.ws``, as int32
    device tensors (lists [n_lists, list_stride], counts [n_lists, N_b]) viewing the workspace."""
    import torch
    lay = tile_layout(spec)
    n, stride, nb = lay["n_lists"], lay["list_stride"], spec.num_blocks
    lists = bufs.ws[lay["list_offset"]: lay["list_offset"] + 4 * n * stride].view(torch.int32).view(n, stride)
    counts = bufs.ws[lay["count_offset"]: lay["count_offset"] + 4 * n * nb].view(torch.int32).view(n, nb)
    return lay, lists, counts


def prefill(spec: LayerSpec, q, k, v, o, bufs: Buffers, bias_offsets=None, bias_values=None, stream=None):
    """One layer of the sparse path: route, select, sparse attention (Alg. 1)."""
    route(spec, q, k, bufs, bias_offsets, bias_values, stream)
    select_indices(spec, q, k, bufs, stream)
    sparse_prefill(spec, q, k, v, o, bufs, bias_offsets, bias_values, stream)
