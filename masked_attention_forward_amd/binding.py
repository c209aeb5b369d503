"""ctypes binding to libfa.so (include/fa.h). Argument marshalling only.

Every computation runs in the library's HIP kernels; this module turns torch tensors into raw
pointers and sizes, passes torch's current HIP stream, and raises on a non-zero status. If
the library is missing it raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))

FA_LAYOUTS = {"BNSD": 0, "BSND": 1, "TND": 2}
_DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULLPTR", 2: "FA_ERR_PARAM_INVALID",
                3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_HIP", 5: "FA_ERR_WORKSPACE"}


class FaDims(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int64), ("N", ctypes.c_int64),
                ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("T_q", ctypes.c_int64), ("T_kv", ctypes.c_int64)]


class FaPlanStats(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("work_items", ctypes.c_int64), ("kv_tiles_visited", ctypes.c_int64),
                ("kv_tiles_full", ctypes.c_int64), ("kv_tiles_total", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("launch_order", ctypes.c_int32),
                ("edge_skip", ctypes.c_int32)]


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_status_str(status)})")


class FaKvCacheDims(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int64),
                ("k_head_size", ctypes.c_int64), ("v_head_size", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("elem_bytes", ctypes.c_int32), ("slot_bytes", ctypes.c_int32)]


CACHE_LAYOUTS = {"Norm": 0, "NHSD": 1}


class FaPagedKv(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("cache_layout", ctypes.c_int32), ("reserved", ctypes.c_int32)]

_LIB = None


def library_path() -> str:
    return os.environ.get("FA_LIBRARY") or os.path.join(HERE, "lib", "libfa.so")


def load_library():
    """Load libfa.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libfa.so is not built ({path}); run `python -m masked_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pdims = ctypes.POINTER(FaDims)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    lib.fa_fwd_workspace_size.argtypes = [pdims, i32, i32, pi64, pi64, ctypes.POINTER(sz)]
    lib.fa_fwd_workspace_size.restype = i32
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, pdims, i32, i32, i64, i64, pi64, pi64, pi64,
                           vp, i32, vp, pi64, ctypes.c_float, vp, sz, vp]
    lib.fa_fwd.restype = i32
    lib.fa_mask_probe.argtypes = [pdims, i32, i32, i64, i64, pi64, pi64, pi64, vp, pi64, vp, vp,
                                  vp, sz, vp]
    lib.fa_mask_probe.restype = i32
    lib.fa_tile_shape.argtypes = [pdims, i32, pi64, pi64, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                  pi64, pi64]
    lib.fa_tile_shape.restype = i32
    lib.fa_plan_stats_get.argtypes = [pdims, i32, i32, i64, i64, pi64, pi64, pi64, i32, i32,
                                      ctypes.c_float, ctypes.POINTER(FaPlanStats)]
    lib.fa_plan_stats_get.restype = i32
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_scatter_kv_cache.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(FaKvCacheDims), i32, vp]
    lib.fa_scatter_kv_cache.restype = i32
    ppaged = ctypes.POINTER(FaPagedKv)
    lib.fa_fwd_paged_workspace_size.argtypes = [pdims, i32, i32, pi64, pi64, ppaged, ctypes.POINTER(sz)]
    lib.fa_fwd_paged_workspace_size.restype = i32
    lib.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, pdims, i32, i32, i64, i64, pi64, pi64, pi64,
                                 vp, i32, vp, pi64, ppaged, ctypes.c_float, vp, sz, vp]
    lib.fa_fwd_paged.restype = i32
    lib.fa_fwd_mask_workspace_size.argtypes = [pdims, i32, pi64, ctypes.POINTER(sz)]
    lib.fa_fwd_mask_workspace_size.restype = i32
    lib.fa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, pdims, i32, i32, i64, i64, pi64, pi64, pi64,
                                   vp, i32, vp, pi64, ctypes.c_float, vp]
    lib.fa_fwd_noalloc.restype = i32
    lib.fa_bwd_workspace_size.argtypes = [pdims, i32, i32, pi64, pi64, ctypes.POINTER(sz)]
    lib.fa_bwd_workspace_size.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, pdims, i32, i32, i64, i64, pi64, pi64, pi64,
                           vp, i32, vp, pi64, ctypes.c_float, vp, sz, vp]
    lib.fa_bwd.restype = i32
    lib.fa_exp2_rate_probe.argtypes = [vp, i32, i32, pi64, vp]
    lib.fa_exp2_rate_probe.restype = i32
    _LIB = lib
    return lib


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def _i64(seq: Optional[Sequence[int]]):
    if seq is None:
        return None
    vals = [int(x) for x in seq]
    return (ctypes.c_int64 * max(len(vals), 1))(*vals)


def _layout_code(layout) -> int:
    if isinstance(layout, str):
        return FA_LAYOUTS[layout]
    return int(layout)


def make_dims(dtype, layout, *, B=0, N=1, Sq=0, Skv=0, D=1, T_q=0, T_kv=0) -> FaDims:
    code = _DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return FaDims(code, B, N, Sq, Skv, D, T_q, T_kv)


def dims_of(q: torch.Tensor, k: torch.Tensor, layout, actual_seq_qlen=None) -> FaDims:
    """fa_dims for q / k in `layout` (shapes only)."""
    lay = _layout_code(layout)
    if q.dtype not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if lay == 0:
        B, N, Sq, D = q.shape
        return make_dims(q.dtype, lay, B=B, N=N, Sq=Sq, Skv=k.shape[2], D=D)
    if lay == 1:
        B, Sq, N, D = q.shape
        return make_dims(q.dtype, lay, B=B, N=N, Sq=Sq, Skv=k.shape[1], D=D)
    T_q, N, D = q.shape
    B = len(actual_seq_qlen) if actual_seq_qlen is not None else 0
    return make_dims(q.dtype, lay, B=B, N=N, D=D, T_q=T_q, T_kv=k.shape[0])


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_device_tensor(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _kv_shape_of(q, layout, skv_or_tkv):
    """The shape k and v must have, given q in `layout` and the key count (Skv, or T_kv for TND)."""
    lay = _layout_code(layout)
    if lay == 0:
        B, N, _, D = q.shape
        return (B, N, skv_or_tkv, D)
    if lay == 1:
        B, _, N, D = q.shape
        return (B, skv_or_tkv, N, D)
    _, N, D = q.shape
    return (skv_or_tkv, N, D)


def check_shapes(q, k, v, out, softmax_lse, layout, *, atten_mask=None, mask_bcast=None) -> None:
    """Raises ValueError unless k, v, out, softmax_lse (and atten_mask, when given) have the
    shapes the C ABI derives from q and k: every extent the kernels use comes from q's and k's
    shapes, so a shorter v, out, lse or mask would be read or written past its end."""
    lay = _layout_code(layout)
    want_dim = 3 if lay == 2 else 4
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t is not None and t.dim() != want_dim:
            raise ValueError(f"{name} must be {want_dim}-D in layout {layout}, got {tuple(t.shape)}")
    skv = k.shape[0] if lay == 2 else (k.shape[2] if lay == 0 else k.shape[1])
    kv_want = _kv_shape_of(q, layout, skv)
    if tuple(k.shape) != kv_want:
        raise ValueError(f"k must have shape {kv_want} for q {tuple(q.shape)} ({layout}), got {tuple(k.shape)}")
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    if out is not None and tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if softmax_lse is not None and tuple(softmax_lse.shape) != lse_shape(q, layout):
        raise ValueError(f"softmax_lse must have shape {lse_shape(q, layout)}, got {tuple(softmax_lse.shape)}")
    if atten_mask is not None:
        if lay == 2:
            raise ValueError("atten_mask needs the BNSD or BSND layout")
        B = q.shape[0]
        N = q.shape[1] if lay == 0 else q.shape[2]
        Sq = q.shape[2] if lay == 0 else q.shape[1]
        bc = list(mask_bcast) if mask_bcast is not None else [0, 0]
        m_want = (1 if bc[0] else B, 1 if bc[1] else N, Sq, skv)
        if tuple(atten_mask.shape) != m_want:
            raise ValueError(f"atten_mask must have shape {m_want} (mask_bcast {bc}), got {tuple(atten_mask.shape)}")


def fa_fwd_workspace_size(dims: FaDims, layout, sparse_mode: int, actual_seq_qlen=None,
                          actual_seq_kvlen=None) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    st = lib.fa_fwd_workspace_size(ctypes.byref(dims), _layout_code(layout), int(sparse_mode),
                                   _i64(actual_seq_qlen), _i64(actual_seq_kvlen), ctypes.byref(out))
    if st != 0:
        raise FaError(st, "fa_fwd_workspace_size")
    return int(out.value)


def fa_fwd_mask_workspace_size(dims: FaDims, layout, mask_bcast=None) -> int:
    """Workspace bytes of a mode-1 call with this mask broadcast (exact; fa_fwd_workspace_size
    assumes an unbroadcast mask)."""
    lib = load_library()
    out = ctypes.c_size_t(0)
    st = lib.fa_fwd_mask_workspace_size(ctypes.byref(dims), _layout_code(layout), _i64(mask_bcast),
                                        ctypes.byref(out))
    if st != 0:
        raise FaError(st, "fa_fwd_mask_workspace_size")
    return int(out.value)


def fa_fwd(q, k, v, out, softmax_lse, *, layout="BNSD", sparse_mode: int = 0, pre_tokens: int = 0,
           next_tokens: int = 0, actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None,
           alibi_slopes: Optional[torch.Tensor] = None, alibi_mode="right",
           atten_mask: Optional[torch.Tensor] = None, mask_bcast=None, scale: float,
           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Calls fa_fwd on device tensors. Raises FaError on a non-zero status.

    alibi_mode: "right", "sqrt" or "left" (or the FA_ALIBI_* code)."""
    check_shapes(q, k, v, out, softmax_lse, layout, atten_mask=atten_mask, mask_bcast=mask_bcast)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_device_tensor(name, t, q.dtype)
    _check_device_tensor("softmax_lse", softmax_lse, torch.float32)
    _check_device_tensor("alibi_slopes", alibi_slopes, torch.float32)
    if atten_mask is not None:
        _check_device_tensor("atten_mask", atten_mask)
        if atten_mask.dtype not in (torch.uint8, torch.bool):
            raise TypeError("atten_mask must be uint8 or bool")
    dims = dims_of(q, k, layout, actual_seq_qlen)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(softmax_lse), ctypes.byref(dims),
                    _layout_code(layout), int(sparse_mode), int(pre_tokens), int(next_tokens),
                    _i64(actual_seq_qlen), _i64(actual_seq_kvlen), _i64(prefix), _ptr(alibi_slopes),
                    _alibi_code(alibi_mode), _ptr(atten_mask), _i64(mask_bcast), float(scale), _ptr(workspace), ws_bytes,
                    stream if stream is not None else _stream(q.device))
    if st != 0:
        raise FaError(st, "fa_fwd")


FA_NOALLOC_SCRATCH_BYTES = 16 << 20


def fa_fwd_noalloc(q, k, v, out, softmax_lse, *, layout="BNSD", sparse_mode: int = 0, pre_tokens: int = 0,
                   next_tokens: int = 0, actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None,
                   alibi_slopes: Optional[torch.Tensor] = None, alibi_mode="right",
                   atten_mask: Optional[torch.Tensor] = None, mask_bcast=None, scale: float, stream=None) -> None:
    """Calls fa_fwd_noalloc: fa_fwd with its workspace in the library's own device array (no
    allocation anywhere). Raises FaError on a non-zero status (FA_ERR_WORKSPACE when the
    problem needs more than FA_NOALLOC_SCRATCH_BYTES of workspace)."""
    check_shapes(q, k, v, out, softmax_lse, layout, atten_mask=atten_mask, mask_bcast=mask_bcast)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_device_tensor(name, t, q.dtype)
    _check_device_tensor("softmax_lse", softmax_lse, torch.float32)
    _check_device_tensor("alibi_slopes", alibi_slopes, torch.float32)
    if atten_mask is not None:
        _check_device_tensor("atten_mask", atten_mask)
        if atten_mask.dtype not in (torch.uint8, torch.bool):
            raise TypeError("atten_mask must be uint8 or bool")
    dims = dims_of(q, k, layout, actual_seq_qlen)
    st = lib.fa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(softmax_lse), ctypes.byref(dims),
                            _layout_code(layout), int(sparse_mode), int(pre_tokens), int(next_tokens),
                            _i64(actual_seq_qlen), _i64(actual_seq_kvlen), _i64(prefix), _ptr(alibi_slopes),
                            _alibi_code(alibi_mode), _ptr(atten_mask), _i64(mask_bcast), float(scale),
                            stream if stream is not None else _stream(q.device))
    if st != 0:
        raise FaError(st, "fa_fwd_noalloc")


ALIBI_MODES = {"right": 0, "sqrt": 1, "left": 2}


def _alibi_code(mode) -> int:
    if isinstance(mode, str):
        if mode not in ALIBI_MODES:
            raise ValueError(f"alibi_mode must be one of {sorted(ALIBI_MODES)}")
        return ALIBI_MODES[mode]
    return int(mode)


def fa_scatter_kv_cache(key, key_cache, slot_mapping, value=None, value_cache=None, *, layout="Norm",
                        stream=None) -> None:
    """Writes key[t] (and value[t]) into the cache slot slot_mapping[t] (in place).

    key / value: [num_tokens, N, D]; caches: [num_blocks, block_size, N, D] ("Norm") or
    [num_blocks, N, block_size, D] ("NHSD"); slot_mapping int32 or int64 [num_tokens]."""
    lib = load_library()
    if layout not in CACHE_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(CACHE_LAYOUTS)}")
    if (value is None) != (value_cache is None):
        raise ValueError("value and value_cache go together")
    for name, t in (("key", key), ("key_cache", key_cache), ("value", value), ("value_cache", value_cache)):
        _check_device_tensor(name, t, key.dtype)
    _check_device_tensor("slot_mapping", slot_mapping)
    if slot_mapping.dtype not in (torch.int32, torch.int64) or slot_mapping.dim() != 1:
        raise TypeError("slot_mapping must be a 1-D int32 or int64 tensor")
    if key.dim() != 3 or key_cache.dim() != 4:
        raise ValueError("key must be [num_tokens, N, D] and key_cache 4-D")
    t, n, dk = key.shape
    nb = key_cache.shape[0]
    bs = key_cache.shape[1] if layout == "Norm" else key_cache.shape[2]
    want = (nb, bs, n, dk) if layout == "Norm" else (nb, n, bs, dk)
    if tuple(key_cache.shape) != want or slot_mapping.shape[0] != t:
        raise ValueError(f"shapes: key {tuple(key.shape)}, key_cache {tuple(key_cache.shape)}, "
                         f"slot_mapping {tuple(slot_mapping.shape)}")
    dv = 0
    if value is not None:
        dv = value.shape[-1]
        want_v = (nb, bs, n, dv) if layout == "Norm" else (nb, n, bs, dv)
        if tuple(value.shape) != (t, n, dv) or tuple(value_cache.shape) != want_v:
            raise ValueError(f"shapes: value {tuple(value.shape)}, value_cache {tuple(value_cache.shape)}")
    dims = FaKvCacheDims(t, n, dk, dv, nb, bs, key.element_size(), slot_mapping.element_size())
    st = lib.fa_scatter_kv_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(slot_mapping), ctypes.byref(dims), CACHE_LAYOUTS[layout],
                                 stream if stream is not None else _stream(key.device))
    if st != 0:
        raise FaError(st, "fa_scatter_kv_cache")


def fa_exp2_rate_probe(out: torch.Tensor, iters: int, *, stream=None) -> int:
    """Launch the exp2-throughput kernel over out.numel() // 256 workgroups (out: float32 on the
    GPU); returns the number of exponentials the launch evaluates."""
    _check_device_tensor("out", out, torch.float32)
    if out.numel() == 0 or out.numel() % 256:
        raise ValueError("out must hold a positive multiple of 256 floats")
    n = ctypes.c_int64(0)
    st = load_library().fa_exp2_rate_probe(_ptr(out), out.numel() // 256, int(iters), ctypes.byref(n),
                                           stream if stream is not None else _stream(out.device))
    if st != 0:
        raise FaError(st, "fa_exp2_rate_probe")
    return n.value


def paged_kv(block_table: Optional[torch.Tensor], key_cache: torch.Tensor, *, cache_layout="Norm",
             max_blocks_per_seq: Optional[int] = None) -> FaPagedKv:
    """fa_paged_kv for a cache tensor ([num_blocks, block_size, N, D] for "Norm",
    [num_blocks, N, block_size, D] for "NHSD") and an int32 block table [B, max_blocks_per_seq]."""
    if cache_layout not in CACHE_LAYOUTS:
        raise ValueError(f"cache_layout must be one of {sorted(CACHE_LAYOUTS)}")
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be 4-D")
    nb = key_cache.shape[0]
    bs = key_cache.shape[1] if cache_layout == "Norm" else key_cache.shape[2]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1] if block_table is not None and block_table.dim() == 2 else 1
    return FaPagedKv(block_table.data_ptr() if block_table is not None and block_table.numel() else None,
                     int(max_blocks_per_seq), int(nb), int(bs), CACHE_LAYOUTS[cache_layout], 0)


def paged_dims(q: torch.Tensor, layout, *, kv_seqlen: int = 0, actual_seq_qlen=None,
               actual_seq_kvlen=None) -> FaDims:
    """fa_dims of a paged call: q's shape, and Skv = kv_seqlen (BNSD / BSND) or
    T_kv = actual_seq_kvlen[-1] (TND)."""
    lay = _layout_code(layout)
    if q.dtype not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if lay == 0:
        B, N, Sq, D = q.shape
        return make_dims(q.dtype, lay, B=B, N=N, Sq=Sq, Skv=int(kv_seqlen), D=D)
    if lay == 1:
        B, Sq, N, D = q.shape
        return make_dims(q.dtype, lay, B=B, N=N, Sq=Sq, Skv=int(kv_seqlen), D=D)
    T_q, N, D = q.shape
    B = len(actual_seq_qlen) if actual_seq_qlen is not None else 0
    T_kv = int(actual_seq_kvlen[-1]) if actual_seq_kvlen is not None and len(actual_seq_kvlen) else 0
    return make_dims(q.dtype, lay, B=B, N=N, D=D, T_q=T_q, T_kv=T_kv)


def fa_fwd_paged_workspace_size(dims: FaDims, layout, sparse_mode: int, paged: FaPagedKv,
                                actual_seq_qlen=None, actual_seq_kvlen=None) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    st = lib.fa_fwd_paged_workspace_size(ctypes.byref(dims), _layout_code(layout), int(sparse_mode),
                                         _i64(actual_seq_qlen), _i64(actual_seq_kvlen), ctypes.byref(paged),
                                         ctypes.byref(out))
    if st != 0:
        raise FaError(st, "fa_fwd_paged_workspace_size")
    return int(out.value)


def fa_fwd_paged(q, key_cache, value_cache, block_table, out, softmax_lse, *, layout="BNSD",
                 cache_layout="Norm", kv_seqlen: int = 0, sparse_mode: int = 0, pre_tokens: int = 0,
                 next_tokens: int = 0, actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None,
                 alibi_slopes: Optional[torch.Tensor] = None, alibi_mode="right",
                 atten_mask: Optional[torch.Tensor] = None, mask_bcast=None, scale: float,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Calls fa_fwd_paged: K / V from paged caches through an int32 block table
    [B, max_blocks_per_seq]. kv_seqlen is Skv for BNSD / BSND (TND uses actual_seq_kvlen)."""
    if q.dim() != (3 if _layout_code(layout) == 2 else 4):
        raise ValueError(f"q has the wrong rank for layout {layout}: {tuple(q.shape)}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if tuple(softmax_lse.shape) != lse_shape(q, layout):
        raise ValueError(f"softmax_lse must have shape {lse_shape(q, layout)}, got {tuple(softmax_lse.shape)}")
    if atten_mask is not None:
        lay = _layout_code(layout)
        if lay == 2:
            raise ValueError("atten_mask needs the BNSD or BSND layout")
        bc = list(mask_bcast) if mask_bcast is not None else [0, 0]
        Nq = q.shape[1] if lay == 0 else q.shape[2]
        Sq = q.shape[2] if lay == 0 else q.shape[1]
        m_want = (1 if bc[0] else q.shape[0], 1 if bc[1] else Nq, Sq, int(kv_seqlen))
        if tuple(atten_mask.shape) != m_want:
            raise ValueError(f"atten_mask must have shape {m_want} (mask_bcast {bc}), got {tuple(atten_mask.shape)}")
    lib = load_library()
    for name, t in (("q", q), ("key_cache", key_cache), ("value_cache", value_cache), ("out", out)):
        _check_device_tensor(name, t, q.dtype)
    _check_device_tensor("softmax_lse", softmax_lse, torch.float32)
    _check_device_tensor("block_table", block_table, torch.int32)
    _check_device_tensor("alibi_slopes", alibi_slopes, torch.float32)
    if atten_mask is not None:
        _check_device_tensor("atten_mask", atten_mask)
        if atten_mask.dtype not in (torch.uint8, torch.bool):
            raise TypeError("atten_mask must be uint8 or bool")
    if key_cache.shape != value_cache.shape:
        raise ValueError("key_cache and value_cache must have one shape")
    head = key_cache.shape[2] if cache_layout == "Norm" else key_cache.shape[1]
    if key_cache.shape[3] != q.shape[-1] or head != (q.shape[1] if _layout_code(layout) != 1 else q.shape[2]):
        raise ValueError(f"cache {tuple(key_cache.shape)} does not match q {tuple(q.shape)} ({layout}, {cache_layout})")
    dims = paged_dims(q, layout, kv_seqlen=kv_seqlen, actual_seq_qlen=actual_seq_qlen,
                      actual_seq_kvlen=actual_seq_kvlen)
    if block_table is not None and block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    pk = paged_kv(block_table, key_cache, cache_layout=cache_layout)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.fa_fwd_paged(_ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(out), _ptr(softmax_lse),
                          ctypes.byref(dims), _layout_code(layout), int(sparse_mode), int(pre_tokens),
                          int(next_tokens), _i64(actual_seq_qlen), _i64(actual_seq_kvlen), _i64(prefix),
                          _ptr(alibi_slopes), _alibi_code(alibi_mode), _ptr(atten_mask), _i64(mask_bcast),
                          ctypes.byref(pk), float(scale), _ptr(workspace), ws_bytes,
                          stream if stream is not None else _stream(q.device))
    if st != 0:
        raise FaError(st, "fa_fwd_paged")


def paged_attention(q, key_cache, value_cache, block_table, *, layout="BNSD", cache_layout="Norm",
                    kv_seqlen: int = 0, sparse_mode: int = 0, scale: float, **kw):
    """Allocates out / softmax_lse / workspace and runs fa_fwd_paged. Returns (out, softmax_lse)."""
    out = torch.empty_like(q)
    lse = torch.empty(lse_shape(q, layout), dtype=torch.float32, device=q.device)
    dims = paged_dims(q, layout, kv_seqlen=kv_seqlen, actual_seq_qlen=kw.get("actual_seq_qlen"),
                      actual_seq_kvlen=kw.get("actual_seq_kvlen"))
    pk = paged_kv(block_table, key_cache, cache_layout=cache_layout)
    ws = fa_fwd_paged_workspace_size(dims, layout, sparse_mode, pk, kw.get("actual_seq_qlen"),
                                     kw.get("actual_seq_kvlen"))
    workspace = torch.empty(ws, dtype=torch.uint8, device=q.device) if ws else None
    fa_fwd_paged(q, key_cache, value_cache, block_table, out, lse, layout=layout, cache_layout=cache_layout,
                 kv_seqlen=kv_seqlen, sparse_mode=sparse_mode, scale=scale, workspace=workspace, **kw)
    return out, lse


def fa_bwd_workspace_size(dims: FaDims, layout, sparse_mode: int, actual_seq_qlen=None,
                          actual_seq_kvlen=None) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    st = lib.fa_bwd_workspace_size(ctypes.byref(dims), _layout_code(layout), int(sparse_mode),
                                   _i64(actual_seq_qlen), _i64(actual_seq_kvlen), ctypes.byref(out))
    if st != 0:
        raise FaError(st, "fa_bwd_workspace_size")
    return int(out.value)


def fa_bwd(q, k, v, out, softmax_lse, dout, dq, dk, dv, *, layout="BNSD", sparse_mode: int = 0,
           pre_tokens: int = 0, next_tokens: int = 0, actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None,
           alibi_slopes: Optional[torch.Tensor] = None, alibi_mode="right",
           atten_mask: Optional[torch.Tensor] = None, mask_bcast=None, scale: float,
           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Calls fa_bwd: dq, dk, dv (written in full) from the forward's inputs, its out and
    softmax_lse, and dout. Raises FaError on a non-zero status."""
    check_shapes(q, k, v, out, softmax_lse, layout, atten_mask=atten_mask, mask_bcast=mask_bcast)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_device_tensor(name, t, q.dtype)
    _check_device_tensor("softmax_lse", softmax_lse, torch.float32)
    _check_device_tensor("alibi_slopes", alibi_slopes, torch.float32)
    if atten_mask is not None:
        _check_device_tensor("atten_mask", atten_mask)
        if atten_mask.dtype not in (torch.uint8, torch.bool):
            raise TypeError("atten_mask must be uint8 or bool")
    for name, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")
    dims = dims_of(q, k, layout, actual_seq_qlen)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(softmax_lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                    ctypes.byref(dims), _layout_code(layout), int(sparse_mode), int(pre_tokens), int(next_tokens),
                    _i64(actual_seq_qlen), _i64(actual_seq_kvlen), _i64(prefix), _ptr(alibi_slopes),
                    _alibi_code(alibi_mode), _ptr(atten_mask), _i64(mask_bcast), float(scale), _ptr(workspace), ws_bytes,
                    stream if stream is not None else _stream(q.device))
    if st != 0:
        raise FaError(st, "fa_bwd")


def flash_attention_backward(q, k, v, out, lse, dout, *, layout="BNSD", sparse_mode: int = 0, scale: float, **kw):
    """Allocates dq / dk / dv / workspace and runs fa_bwd. Returns (dq, dk, dv)."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dims = dims_of(q, k, layout, kw.get("actual_seq_qlen"))
    ws = fa_bwd_workspace_size(dims, layout, sparse_mode, kw.get("actual_seq_qlen"), kw.get("actual_seq_kvlen"))
    workspace = torch.empty(ws, dtype=torch.uint8, device=q.device) if ws else None
    fa_bwd(q, k, v, out, lse, dout, dq, dk, dv, layout=layout, sparse_mode=sparse_mode, scale=scale,
           workspace=workspace, **kw)
    return dq, dk, dv


def lse_shape(q, layout, actual_seq_qlen=None):
    lay = _layout_code(layout)
    if lay == 0:
        return (q.shape[0], q.shape[1], q.shape[2])
    if lay == 1:
        return (q.shape[0], q.shape[2], q.shape[1])
    return (q.shape[1], q.shape[0])


def flash_attention(q, k, v, *, layout="BNSD", sparse_mode: int = 0, scale: float, **kw):
    """Allocates out / softmax_lse / workspace and runs fa_fwd. Returns (out, softmax_lse)."""
    out = torch.empty_like(q)
    lse = torch.empty(lse_shape(q, layout), dtype=torch.float32, device=q.device)
    dims = dims_of(q, k, layout, kw.get("actual_seq_qlen"))
    if sparse_mode == 1:
        ws = fa_fwd_mask_workspace_size(dims, layout, kw.get("mask_bcast"))
    else:
        ws = fa_fwd_workspace_size(dims, layout, sparse_mode, kw.get("actual_seq_qlen"),
                                   kw.get("actual_seq_kvlen"))
    workspace = torch.empty(ws, dtype=torch.uint8, device=q.device) if ws else None
    fa_fwd(q, k, v, out, lse, layout=layout, sparse_mode=sparse_mode, scale=scale,
           workspace=workspace, **kw)
    return out, lse


def fa_tile_shape(dims: FaDims, layout, actual_seq_qlen=None, actual_seq_kvlen=None):
    """(block_m, block_n, n_qtiles_total, n_kvtiles_max)."""
    lib = load_library()
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    nq, nk = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.fa_tile_shape(ctypes.byref(dims), _layout_code(layout), _i64(actual_seq_qlen),
                           _i64(actual_seq_kvlen), ctypes.byref(bm), ctypes.byref(bn),
                           ctypes.byref(nq), ctypes.byref(nk))
    if st != 0:
        raise FaError(st, "fa_tile_shape")
    return bm.value, bn.value, nq.value, nk.value


def fa_plan_stats(dims: FaDims, layout, sparse_mode: int, *, pre_tokens=0, next_tokens=0,
                  actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None, has_alibi=False,
                  has_mask=False, scale=1.0) -> dict:
    """Host-side plan summary of a fa_fwd call (no device work)."""
    lib = load_library()
    s = FaPlanStats()
    st = lib.fa_plan_stats_get(ctypes.byref(dims), _layout_code(layout), int(sparse_mode),
                               int(pre_tokens), int(next_tokens), _i64(actual_seq_qlen),
                               _i64(actual_seq_kvlen), _i64(prefix), int(has_alibi), int(has_mask),
                               float(scale), ctypes.byref(s))
    if st != 0:
        raise FaError(st, "fa_plan_stats_get")
    return {f: getattr(s, f) for f, _ in FaPlanStats._fields_}


def fa_mask_probe(dims: FaDims, layout, sparse_mode: int, *, device, pre_tokens=0, next_tokens=0,
                  actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None, atten_mask=None,
                  mask_bcast=None, tiles: bool = True):
    """Runs fa_mask_probe; returns (row_visible_counts, tile_class or None) on `device`."""
    lib = load_library()
    lay = _layout_code(layout)
    if lay == 2:
        counts = torch.empty((dims.N, dims.T_q), dtype=torch.int64, device=device)
    else:
        counts = torch.empty((dims.B, dims.N, dims.Sq), dtype=torch.int64, device=device)
    tile = None
    if tiles:
        _, _, nq, nk = fa_tile_shape(dims, layout, actual_seq_qlen, actual_seq_kvlen)
        if sparse_mode == 1:
            nq *= dims.N    # mode 1: one map row per (batch, head, q tile)
        tile = torch.empty((nq, nk), dtype=torch.uint8, device=device)
    if sparse_mode == 1:
        ws = fa_fwd_mask_workspace_size(dims, layout, mask_bcast)
    else:
        ws = fa_fwd_workspace_size(dims, layout, sparse_mode, actual_seq_qlen, actual_seq_kvlen)
    workspace = torch.empty(ws, dtype=torch.uint8, device=device) if ws else None
    st = lib.fa_mask_probe(ctypes.byref(dims), lay, int(sparse_mode), int(pre_tokens), int(next_tokens),
                           _i64(actual_seq_qlen), _i64(actual_seq_kvlen), _i64(prefix),
                           _ptr(atten_mask), _i64(mask_bcast), _ptr(counts), _ptr(tile),
                           _ptr(workspace), ws, _stream(device))
    if st != 0:
        raise FaError(st, "fa_mask_probe")
    return counts, tile
