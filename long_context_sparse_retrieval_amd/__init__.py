"""Python binding of librtp.so: RTPurbo's sparse-attention decode step on MI355X.

Thin ctypes marshalling over the C ABI declared in include/rtp.h (same names,
without the ``rtp_`` prefix).  Every step of the computation runs in the HIP
kernels of librtp.so; PyTorch only provides device memory and the current
stream.  Importing works without a GPU; the first call fails loudly if the
library was not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

__all__ = [
    "Layer", "RtpError", "library_path", "load", "num_retrieval", "workspace_bytes", "workspace",
    "rope_keys", "index_keys", "index_score", "topp_select", "sparse_attn", "swa_attn", "dense_attn",
    "decode_step", "decode_step_static", "append_kv", "prefill_attn", "cluster_workspace", "cluster_build", "cluster_step", "kv_rows",
    "kv_shape", "SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "librtp.so")
_lib = None

SYMBOLS = ("rtp_num_retrieval", "rtp_workspace_bytes", "rtp_workspace_init", "rtp_status_str", "rtp_rope_keys",
           "rtp_index_keys", "rtp_append_kv", "rtp_index_score", "rtp_topp_select", "rtp_sparse_attn", "rtp_swa_attn",
           "rtp_dense_attn", "rtp_prefill_attn", "rtp_decode_step", "rtp_cluster_workspace_bytes",
           "rtp_cluster_build", "rtp_cluster_step", "rtp_kv_rows", "rtp_decode_step_static")


class RtpError(RuntimeError):
    pass


class _CLayer(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("R", ctypes.c_int32), ("nq", ctypes.c_int32), ("N", ctypes.c_int64), ("Ncap", ctypes.c_int64),
        ("head_mode", ctypes.POINTER(ctypes.c_int8)), ("p", ctypes.c_double), ("window", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("idx_group", ctypes.c_int32),
        ("top_k", ctypes.c_int64), ("local_ring", ctypes.c_int32), ("scan_tile", ctypes.c_int32),
        ("swa_chunk", ctypes.c_int32), ("pf_qch", ctypes.c_int32),
    ]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load librtp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RtpError(f"{_LIB_PATH} is missing: build it with `python -m long_context_sparse_retrieval_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32p = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
    L = ctypes.POINTER(_CLayer)
    sig = {
        "rtp_num_retrieval": (ctypes.c_int32, [L]),
        "rtp_workspace_bytes": (ctypes.c_size_t, [L]),
        "rtp_kv_rows": (ctypes.c_int64, [L]),
        "rtp_workspace_init": (ctypes.c_int, [vp, ctypes.c_size_t, vp]),
        "rtp_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "rtp_rope_keys": (ctypes.c_int, [L, vp, vp, i64, i64, vp]),
        "rtp_index_keys": (ctypes.c_int, [L, vp, vp, vp, i64, i64, vp]),
        "rtp_append_kv": (ctypes.c_int, [L, vp, vp, vp, vp, vp, vp, i64, i64, vp]),
        "rtp_index_score": (ctypes.c_int, [L, vp, vp, vp, vp, vp]),
        "rtp_topp_select": (ctypes.c_int, [L, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]),
        "rtp_sparse_attn": (ctypes.c_int, [L, vp, vp, vp, vp, vp, i64, vp, vp, ctypes.c_size_t, vp]),
        "rtp_swa_attn": (ctypes.c_int, [L, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "rtp_dense_attn": (ctypes.c_int, [L, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "rtp_prefill_attn": (ctypes.c_int, [L, vp, vp, vp, vp, ctypes.c_int32, vp]),
        "rtp_decode_step": (ctypes.c_int, [L, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp, vp]),
        "rtp_decode_step_static": (ctypes.c_int, [L, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
        "rtp_cluster_workspace_bytes": (ctypes.c_size_t, [L, ctypes.c_int32]),
        "rtp_cluster_build": (ctypes.c_int, [L, vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp,
                                             ctypes.c_size_t, vp]),
        "rtp_cluster_step": (ctypes.c_int, [L, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                            ctypes.c_size_t, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _ = i32p
    _lib = lib
    return lib


@dataclass
class Layer:
    """One attention layer of the step (mirrors ``rtp_layer``)."""
    B: int
    Hq: int
    Hkv: int
    N: int
    head_mode: list
    nq: int = 1
    Ncap: int | None = None
    p: float = 0.9
    window: int = 4096
    n_sink: int = 4
    rope_theta: float = 1.0e6
    D: int = 128
    R: int = 16
    idx_group: int = 1        # retrieval heads sharing one indexer-key head (1 or Hq // Hkv)
    top_k: int = 0            # 0: Top-P with mass p; > 0: fixed top-k on the histogram order
    local_ring: int = 0       # 1: all-local KV groups keep only n_sink + window rows (K/V caches [B, kv_rows, D])
    scan_tile: int = 0        # tuning (0 = the library's choice): positions per indexer scan tile
    swa_chunk: int = 0        # tuning: cache rows per window workgroup
    pf_qch: int = 0           # tuning: queries per chunked-prefill selection chunk
    # the C struct of the current field values and the head_mode array it points
    # to (not an init field: dataclasses.replace gives the copy its own)
    _memo: dict = field(default_factory=dict, init=False, repr=False, compare=False)

    @property
    def cap_rows(self) -> int:
        return self.N if self.Ncap is None else self.Ncap

    @property
    def Hr(self) -> int:
        return int(sum(1 for h in self.head_mode if h))

    @property
    def Hi(self) -> int:
        """Indexer-key heads (rows of k_idx / w_k)."""
        return self.Hr // max(1, self.idx_group)

    def _key(self) -> tuple:
        return (self.B, self.Hq, self.Hkv, self.D, self.R, self.nq, self.N, self.cap_rows, tuple(self.head_mode),
                self.p, self.window, self.n_sink, self.rope_theta, self.idx_group, self.top_k, self.local_ring,
                self.scan_tile, self.swa_chunk, self.pf_qch)

    def c(self) -> _CLayer:
        """The C struct of the current field values (rebuilt only when a field changed)."""
        key = self._key()
        if self._memo.get("key") != key:
            hm = (ctypes.c_int8 * len(self.head_mode))(*[int(h) for h in self.head_mode])
            cl = _CLayer(self.B, self.Hq, self.Hkv, self.D, self.R, self.nq, self.N, self.cap_rows,
                         ctypes.cast(hm, ctypes.POINTER(ctypes.c_int8)), self.p, self.window, self.n_sink,
                         self.rope_theta, self.idx_group, self.top_k, self.local_ring, self.scan_tile,
                         self.swa_chunk, self.pf_qch)
            self._memo.clear()
            self._memo.update(key=key, c=cl, head_mode=hm)
        return self._memo["c"]


def _check(status: int, what: str):
    if status != 0:
        msg = load().rtp_status_str(status).decode()
        raise RtpError(f"{what}: {msg} ({status})")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None, dtype, shape=None, name="tensor") -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def num_retrieval(layer: Layer) -> int:
    return int(load().rtp_num_retrieval(ctypes.byref(layer.c())))


def workspace_bytes(layer: Layer) -> int:
    n = int(load().rtp_workspace_bytes(ctypes.byref(layer.c())))
    if n == 0:
        raise RtpError("invalid layer")
    return n


def workspace(layer: Layer, device="cuda") -> torch.Tensor:
    """A prepared workspace for ``layer`` (allocated by torch, filled by the library)."""
    n = workspace_bytes(layer)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    _check(load().rtp_workspace_init(ws.data_ptr(), n, _stream()), "rtp_workspace_init")
    return ws


def cluster_workspace(layer: Layer, K: int, device="cuda") -> torch.Tensor:
    """A prepared workspace for the cluster-index calls of ``layer`` with K clusters
    (it also serves every call ``workspace(layer)`` serves)."""
    n = int(load().rtp_cluster_workspace_bytes(ctypes.byref(layer.c()), int(K)))
    if n == 0:
        raise RtpError("invalid layer or cluster count")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    _check(load().rtp_workspace_init(ws.data_ptr(), n, _stream()), "rtp_workspace_init")
    return ws


def cluster_build(layer: Layer, k_idx, K: int, iters: int, ws) -> dict:
    """Cluster index of positions 0..N-1 of every (sequence, indexer-key head):
    centroids [B, Hi, K, R] bf16, counts [B, Hi, K], offsets [B, Hi, K+1] and
    members [B, Hi, N] (positions grouped by cluster, ascending in each)."""
    dev = k_idx.device
    ki = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx")
    cent = torch.empty((layer.B, layer.Hi, K, layer.R), dtype=torch.bfloat16, device=dev)
    counts = torch.empty((layer.B, layer.Hi, K), dtype=torch.int32, device=dev)
    offsets = torch.empty((layer.B, layer.Hi, K + 1), dtype=torch.int32, device=dev)
    members = torch.empty((layer.B, layer.Hi, layer.N), dtype=torch.int32, device=dev)
    _check(load().rtp_cluster_build(ctypes.byref(layer.c()), ki, int(K), int(iters), cent.data_ptr(),
                                    counts.data_ptr(), offsets.data_ptr(), members.data_ptr(), ws.data_ptr(),
                                    ws.numel(), _stream()), "rtp_cluster_build")
    return dict(K=int(K), centroids=cent, counts=counts, offsets=offsets, members=members)


def cluster_step(layer: Layer, q_pre, w_q, index: dict, k, v, ws, out=None, idx=None, count=None) -> torch.Tensor:
    """Decode step over a cluster index: retrieval heads attend over the members of
    their hit clusters, local heads over window + sinks; writes every row of out."""
    K = index["K"]
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    wq = _ptr(w_q, torch.bfloat16, (layer.Hr, layer.D, layer.R), "w_q")
    cent = _ptr(index["centroids"], torch.bfloat16, (layer.B, layer.Hi, K, layer.R), "centroids")
    cnt = _ptr(index["counts"], torch.int32, (layer.B, layer.Hi, K), "counts")
    offs = _ptr(index["offsets"], torch.int32, (layer.B, layer.Hi, K + 1), "offsets")
    mem = _ptr(index["members"], torch.int32, (layer.B, layer.Hi, layer.N), "members")
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.empty((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    cap = 0
    ip = cp = None
    if idx is not None:
        cap = int(idx.shape[-1])
        ip = _ptr(idx, torch.int32, (layer.B, layer.Hr, layer.nq, cap), "idx")
    if count is not None:
        cp = _ptr(count, torch.int32, (layer.B, layer.Hr, layer.nq), "count")
    _check(load().rtp_cluster_step(ctypes.byref(layer.c()), q, wq, int(K), cent, cnt, offs, mem, kp, vp, op, ip, cp,
                                   cap, ws.data_ptr(), ws.numel(), _stream()), "rtp_cluster_step")
    return out


def _cache_shape(layer: Layer, heads: int, width: int):
    return (layer.B, heads, layer.cap_rows, width)


def kv_rows(layer: Layer) -> int:
    """K/V cache rows per sequence in the layer's layout (rtp_kv_rows)."""
    r = int(load().rtp_kv_rows(ctypes.byref(layer.c())))
    if r < 0:
        _check(r, "rtp_kv_rows")
    return r


def kv_shape(layer: Layer) -> tuple:
    """Shape of the K/V caches: [B, Hkv, Ncap, D], or [B, kv_rows, D] with local_ring."""
    if layer.local_ring:
        layer.c()                                   # refreshes the memo when a field changed
        if "rows" not in layer._memo:
            layer._memo["rows"] = kv_rows(layer)
        return (layer.B, layer._memo["rows"], layer.D)
    return _cache_shape(layer, layer.Hkv, layer.D)


def rope_keys(layer: Layer, k_pre: torch.Tensor, k_out: torch.Tensor | None = None, n0: int = 0,
              n1: int | None = None) -> torch.Tensor:
    """Post-RoPE key cache rows [n0, n1) from pre-RoPE keys (may be in place)."""
    shp = _cache_shape(layer, layer.Hkv, layer.D)
    a = _ptr(k_pre, torch.bfloat16, shp, "k_pre")
    if k_out is None:
        k_out = torch.empty_like(k_pre)
    b = _ptr(k_out, torch.bfloat16, shp, "k_out")
    n1 = layer.cap_rows if n1 is None else n1
    _check(load().rtp_rope_keys(ctypes.byref(layer.c()), a, b, n0, n1, _stream()), "rtp_rope_keys")
    return k_out


def index_keys(layer: Layer, k_pre: torch.Tensor, w_k: torch.Tensor, k_idx: torch.Tensor | None = None,
               n0: int = 0, n1: int | None = None) -> torch.Tensor:
    """Indexer-key cache rows [n0, n1): bf16(k_pre . W_k) per retrieval head."""
    a = _ptr(k_pre, torch.bfloat16, _cache_shape(layer, layer.Hkv, layer.D), "k_pre")
    w = _ptr(w_k, torch.bfloat16, (layer.Hi, layer.D, layer.R), "w_k")
    if k_idx is None:
        k_idx = torch.zeros(_cache_shape(layer, layer.Hi, layer.R), dtype=torch.bfloat16, device=k_pre.device)
    b = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx")
    n1 = layer.cap_rows if n1 is None else n1
    _check(load().rtp_index_keys(ctypes.byref(layer.c()), a, w, b, n0, n1, _stream()), "rtp_index_keys")
    return k_idx


def append_kv(layer: Layer, k_new: torch.Tensor, v_new: torch.Tensor, w_k, k_cache: torch.Tensor,
              v_cache: torch.Tensor, k_idx, n0: int) -> None:
    """Write positions n0 .. n0 + n_new - 1 of every cache in one launch: post-RoPE keys,
    values and (for retrieval layers) indexer keys, from the new tokens' pre-RoPE keys
    and values [B, Hkv, n_new, D]."""
    if k_new.dim() != 4:
        raise ValueError("k_new must be [B, Hkv, n_new, D]")
    n_new = int(k_new.shape[2])
    shp_new = (layer.B, layer.Hkv, n_new, layer.D)
    a = _ptr(k_new, torch.bfloat16, shp_new, "k_new")
    b = _ptr(v_new, torch.bfloat16, shp_new, "v_new")
    kc = _ptr(k_cache, torch.bfloat16, kv_shape(layer), "k_cache")
    vc = _ptr(v_cache, torch.bfloat16, kv_shape(layer), "v_cache")
    w = ki = None
    if layer.Hi:
        w = _ptr(w_k, torch.bfloat16, (layer.Hi, layer.D, layer.R), "w_k")
        ki = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx")
    _check(load().rtp_append_kv(ctypes.byref(layer.c()), a, b, w, kc, vc, ki, n0, n_new, _stream()),
           "rtp_append_kv")


def index_score(layer: Layer, q_pre, w_q, k_idx, logits=None) -> torch.Tensor:
    """Indexer scores [B, Hr, nq, N] fp32 (eq. 4); -inf beyond each query's position."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    w = _ptr(w_q, torch.bfloat16, (layer.Hr, layer.D, layer.R), "w_q")
    k = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx")
    if logits is None:
        logits = torch.empty((layer.B, layer.Hr, layer.nq, layer.N), dtype=torch.float32, device=q_pre.device)
    o = _ptr(logits, torch.float32, (layer.B, layer.Hr, layer.nq, layer.N), "logits")
    _check(load().rtp_index_score(ctypes.byref(layer.c()), q, w, k, o, _stream()), "rtp_index_score")
    return logits


def topp_select(layer: Layer, logits, cap: int, ws, idx=None, count=None):
    """Histogram Top-P sets of given scores: (idx [B,Hr,nq,cap] int32, count [B,Hr,nq] int32)."""
    dev = logits.device
    lg = _ptr(logits, torch.float32, (layer.B, layer.Hr, layer.nq, layer.N), "logits")
    if idx is None:
        idx = torch.full((layer.B, layer.Hr, layer.nq, max(cap, 1)), -1, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.zeros((layer.B, layer.Hr, layer.nq), dtype=torch.int32, device=dev)
    ip = _ptr(idx, torch.int32, None, "idx")
    if idx.numel() < layer.B * layer.Hr * layer.nq * cap:
        raise ValueError("idx smaller than [B, Hr, nq, cap]")
    cp = _ptr(count, torch.int32, (layer.B, layer.Hr, layer.nq), "count")
    _check(load().rtp_topp_select(ctypes.byref(layer.c()), lg, ip, cp, cap, ws.data_ptr(), ws.numel(), _stream()),
           "rtp_topp_select")
    return idx, count


def sparse_attn(layer: Layer, q_pre, k, v, idx, count, ws, out=None) -> torch.Tensor:
    """Sparse attention of the retrieval heads over given sets (eq. 5); writes their rows of out."""
    cap = idx.shape[-1]
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    ip = _ptr(idx, torch.int32, (layer.B, layer.Hr, layer.nq, cap), "idx")
    cp = _ptr(count, torch.int32, (layer.B, layer.Hr, layer.nq), "count")
    if out is None:
        out = torch.zeros((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    _check(load().rtp_sparse_attn(ctypes.byref(layer.c()), q, kp, vp, ip, cp, cap, op, ws.data_ptr(), ws.numel(),
                                  _stream()), "rtp_sparse_attn")
    return out


def swa_attn(layer: Layer, q_pre, k, v, ws, out=None) -> torch.Tensor:
    """Sliding-window attention with sinks of the local heads; writes their rows of out."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.zeros((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    _check(load().rtp_swa_attn(ctypes.byref(layer.c()), q, kp, vp, op, ws.data_ptr(), ws.numel(), _stream()),
           "rtp_swa_attn")
    return out


def dense_attn(layer: Layer, q_pre, k, v, ws, out=None) -> torch.Tensor:
    """Dense attention of every head over every cached position (the comparator); writes every row of out."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.empty((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    _check(load().rtp_dense_attn(ctypes.byref(layer.c()), q, kp, vp, op, ws.data_ptr(), ws.numel(), _stream()),
           "rtp_dense_attn")
    return out


def prefill_attn(layer: Layer, q_pre, k, v, out=None, all_dense: bool = False) -> torch.Tensor:
    """Causal attention of the layer's nq queries on the matrix cores: retrieval heads
    over every earlier position, local heads over window + sinks (every head dense
    when all_dense); writes every row of out."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.empty((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    _check(load().rtp_prefill_attn(ctypes.byref(layer.c()), q, kp, vp, op, int(bool(all_dense)), _stream()),
           "rtp_prefill_attn")
    return out


def decode_step(layer: Layer, q_pre, w_q, k_idx, k, v, ws, out=None, idx=None, count=None,
                phase_event: torch.cuda.Event | None = None) -> torch.Tensor:
    """One fused decode step (eq. 4-5 + SWA): returns out [B, Hq, 1, D] fp32."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    w = _ptr(w_q, torch.bfloat16, (layer.Hr, layer.D, layer.R), "w_q") if layer.Hr else None
    ki = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx") if layer.Hr else None
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.empty((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    cap = 0
    ip = cp = None
    if idx is not None:
        cap = idx.shape[-1]
        ip = _ptr(idx, torch.int32, (layer.B, layer.Hr, layer.nq, cap), "idx")
    if count is not None:
        cp = _ptr(count, torch.int32, (layer.B, layer.Hr, layer.nq), "count")
    ev = None
    if phase_event is not None:
        ev = phase_event.cuda_event
        if not ev:
            raise ValueError("phase_event must have been recorded once (torch creates events lazily)")
    _check(load().rtp_decode_step(ctypes.byref(layer.c()), q, w, ki, kp, vp, op, ip, cp, cap, ws.data_ptr(),
                                  ws.numel(), ev, _stream()), "rtp_decode_step")
    return out


STATIC_SCRATCH_BYTES = 64 << 20     # RTP_STATIC_SCRATCH_BYTES


def decode_step_static(layer: Layer, q_pre, w_q, k_idx, k, v, out=None, idx=None, count=None) -> torch.Tensor:
    """rtp_decode_step_static: the decode step on the library's static device
    scratch (no workspace argument; allocates nothing on the library side).
    Layers whose workspace exceeds STATIC_SCRATCH_BYTES raise RtpError."""
    q = _ptr(q_pre, torch.bfloat16, (layer.B, layer.Hq, layer.nq, layer.D), "q_pre")
    w = _ptr(w_q, torch.bfloat16, (layer.Hr, layer.D, layer.R), "w_q") if layer.Hr else None
    ki = _ptr(k_idx, torch.bfloat16, _cache_shape(layer, layer.Hi, layer.R), "k_idx") if layer.Hr else None
    kp = _ptr(k, torch.bfloat16, kv_shape(layer), "k")
    vp = _ptr(v, torch.bfloat16, kv_shape(layer), "v")
    if out is None:
        out = torch.empty((layer.B, layer.Hq, layer.nq, layer.D), dtype=torch.float32, device=q_pre.device)
    op = _ptr(out, torch.float32, (layer.B, layer.Hq, layer.nq, layer.D), "out")
    cap = 0
    ip = cp = None
    if idx is not None:
        cap = idx.shape[-1]
        ip = _ptr(idx, torch.int32, (layer.B, layer.Hr, layer.nq, cap), "idx")
    if count is not None:
        cp = _ptr(count, torch.int32, (layer.B, layer.Hr, layer.nq), "count")
    _check(load().rtp_decode_step_static(ctypes.byref(layer.c()), q, w, ki, kp, vp, op, ip, cp, cap, _stream()),
           "rtp_decode_step_static")
    return out
