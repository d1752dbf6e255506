"""Paged GQA / MLA decode attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libdecode_attn.so`` (the C ABI declared in
``include/decode_attn.h``).  Every step of the computation runs in the HIP
kernels; this module only turns torch tensors into pointers, shapes and a
stream.  There is no CPU fallback: if the library is missing, importing the
binding raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecode_attn.so")

DA_F32, DA_BF16, DA_FP8_E4M3 = 0, 1, 2
STATUS = {0: "DA_OK", -1: "DA_ERR_NULL", -2: "DA_ERR_SHAPE", -3: "DA_ERR_DTYPE", -4: "DA_ERR_UNSUPPORTED",
          -5: "DA_ERR_WORKSPACE", -6: "DA_ERR_HIP", -7: "DA_ERR_DATA",
          -8: "DA_ERR_SCRATCH"}

EXPORTS = ("decode_attn_paged", "decode_attn_paged_rows", "decode_attn_mla", "decode_attn_mla_rows", "decode_attn_plan", "paged_kv_gather",
           "decode_kv_append", "decode_kv_append_mla",
           "decode_attn_default_workers", "decode_attn_status_str", "decode_attn_last_hip_error",
           "decode_attn_timer_begin", "decode_attn_timer_end",
           "decode_attn_workspace_size", "decode_attn_paged_ws", "decode_attn_mla_ws", "decode_attn_validate_inputs",
           "decode_attn_paged_noalloc", "decode_attn_kernel_name")


class PagedDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("workers", ctypes.c_int32), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class MLADesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("latent_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("workers", ctypes.c_int32)]


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        text = _lib.decode_attn_status_str(status).decode() if _lib is not None else ""
        extra = ""
        if status == -6 and _lib is not None:
            extra = f" (hip error {_lib.decode_attn_last_hip_error()})"
        super().__init__(f"{what}: {STATUS.get(status, status)}: {text}{extra}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_471_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.decode_attn_paged.argtypes = [ctypes.POINTER(PagedDesc), vp, vp, vp, vp, f32, vp, vp, vp]
    lib.decode_attn_paged.restype = ctypes.c_int
    lib.decode_attn_paged_rows.argtypes = [ctypes.POINTER(PagedDesc), i32, vp, vp, vp, vp, f32, vp, vp, vp]
    lib.decode_attn_paged_rows.restype = ctypes.c_int
    lib.decode_attn_mla.argtypes = [ctypes.POINTER(MLADesc), vp, vp, vp, vp, f32, vp, vp, vp]
    lib.decode_attn_mla.restype = ctypes.c_int
    lib.decode_attn_mla_rows.argtypes = [ctypes.POINTER(MLADesc), i32, vp, vp, vp, vp, f32, vp, vp, vp]
    lib.decode_attn_mla_rows.restype = ctypes.c_int
    lib.decode_attn_plan.argtypes = [i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.decode_attn_plan.restype = ctypes.c_int
    lib.paged_kv_gather.argtypes = [ctypes.POINTER(PagedDesc), i32, vp, vp, vp, vp, vp]
    lib.decode_kv_append.argtypes = [ctypes.POINTER(PagedDesc), vp, vp, vp, vp, vp, vp]
    lib.decode_kv_append.restype = ctypes.c_int
    lib.decode_kv_append_mla.argtypes = [ctypes.POINTER(MLADesc), vp, vp, vp, vp, vp]
    lib.decode_kv_append_mla.restype = ctypes.c_int
    lib.paged_kv_gather.restype = ctypes.c_int
    lib.decode_attn_default_workers.argtypes = [ctypes.POINTER(PagedDesc), ctypes.POINTER(MLADesc),
                                                ctypes.POINTER(i32)]
    lib.decode_attn_default_workers.restype = ctypes.c_int
    lib.decode_attn_status_str.argtypes = [ctypes.c_int]
    lib.decode_attn_status_str.restype = ctypes.c_char_p
    lib.decode_attn_last_hip_error.argtypes = []
    lib.decode_attn_last_hip_error.restype = ctypes.c_int
    lib.decode_attn_timer_begin.argtypes = [i32]
    lib.decode_attn_timer_begin.restype = ctypes.c_int
    lib.decode_attn_timer_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    lib.decode_attn_timer_end.restype = ctypes.c_int
    sz = ctypes.c_size_t
    lib.decode_attn_workspace_size.argtypes = [ctypes.POINTER(PagedDesc), ctypes.POINTER(MLADesc), i32,
                                               ctypes.POINTER(sz)]
    lib.decode_attn_workspace_size.restype = ctypes.c_int
    lib.decode_attn_paged_ws.argtypes = [ctypes.POINTER(PagedDesc), i32, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.decode_attn_paged_ws.restype = ctypes.c_int
    lib.decode_attn_mla_ws.argtypes = [ctypes.POINTER(MLADesc), i32, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.decode_attn_mla_ws.restype = ctypes.c_int
    lib.decode_attn_paged_noalloc.argtypes = [ctypes.POINTER(PagedDesc), i32, vp, vp, vp, vp, f32, vp, vp, vp]
    lib.decode_attn_paged_noalloc.restype = ctypes.c_int
    lib.decode_attn_validate_inputs.argtypes = [ctypes.POINTER(PagedDesc), ctypes.POINTER(MLADesc), vp, vp, vp]
    lib.decode_attn_validate_inputs.restype = ctypes.c_int
    lib.decode_attn_kernel_name.argtypes = [ctypes.POINTER(PagedDesc), ctypes.POINTER(MLADesc), i32]
    lib.decode_attn_kernel_name.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib():
    return _lib


# ----------------------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# torch's current stream as a raw handle, without building a Stream object
# (about 0.1 us against 2.7 us per call); absent from some torch builds
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device_index: int = -1) -> Optional[int]:
    """The HIP stream handle to launch on: the given stream (a torch stream or
    a raw handle), else torch's current stream on device `device_index` (the
    current device when negative)."""
    if stream is None:
        if device_index < 0:
            device_index = torch.cuda.current_device()
        if _RAW_STREAM is not None:
            return _RAW_STREAM(device_index)
        return torch.cuda.current_stream(device_index).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dtype_tag(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DA_F32
    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(status: int, what: str):
    if status != 0:
        raise DecodeAttnError(status, what)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _want(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_index_args(B: int, page_table: torch.Tensor, seq_lens: torch.Tensor, what: str = "seq_lens"):
    """page_table int32 [B][max_pages] and seq_lens (or positions) int32 [B]."""
    pts = page_table.shape
    if not (page_table.dtype == torch.int32 and len(pts) == 2 and pts[0] == B):
        raise ValueError(f"page_table must be int32 [{B}][max_pages], got {page_table.dtype} {tuple(pts)}")
    if pts[1] < 1:
        raise ValueError("page_table needs at least one column")
    if not (seq_lens.dtype == torch.int32 and seq_lens.shape == (B,)):
        raise ValueError(f"{what} must be int32 [{B}], got {seq_lens.dtype} {tuple(seq_lens.shape)}")


def _check_out_lse(out: Optional[torch.Tensor], lse: Optional[torch.Tensor], out_shape, out_dtype, lse_shape):
    if out is not None and not (out.dtype == out_dtype and out.shape == out_shape):
        raise ValueError(f"out must be {out_dtype} {tuple(out_shape)}, got {out.dtype} {tuple(out.shape)}")
    if lse is not None and not (lse.dtype == torch.float32 and lse.shape == lse_shape):
        raise ValueError(f"lse must be float32 {tuple(lse_shape)}, got {lse.dtype} {tuple(lse.shape)}")


def _check_paged_args(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                      out: Optional[torch.Tensor], lse: Optional[torch.Tensor], k_scale, v_scale):
    """Shapes and dtypes of a GQA call, q [B][Hq][D] or [B][n][Hq][D]; raises
    ValueError before any pointer reaches the library (which sees only
    pointers and the descriptor).  Messages are formatted only on failure."""
    qs = q.shape
    if len(qs) not in (3, 4):
        raise ValueError(f"q must be [B][Hq][D] or [B][rows][Hq][D], got {tuple(qs)}")
    qd = q.dtype
    if qd is not torch.float32 and qd is not torch.bfloat16:
        raise ValueError(f"q must be float32 or bfloat16, got {qd}")
    B, Hq, D = qs[0], qs[-2], qs[-1]
    ks = kv_pages.shape
    if not (len(ks) == 5 and ks[1] == 2 and ks[4] == D):
        raise ValueError(f"kv_pages must be [num_pages][2][Hkv][P][{D}], got {tuple(ks)}")
    Hkv = ks[2]
    if not (Hkv >= 1 and Hq % Hkv == 0):
        raise ValueError(f"{Hq} query heads are not a multiple of {Hkv} KV heads")
    kd = kv_pages.dtype
    fp8 = kd in _FP8
    if qd is torch.float32:
        if kd is not torch.float32:
            raise ValueError(f"float32 q needs a float32 cache, got {kd}")
    elif not (kd is torch.bfloat16 or fp8):
        raise ValueError(f"bfloat16 q needs a bfloat16 or fp8-e4m3 cache, got {kd}")
    if fp8:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if not (sc is not None and sc.dtype == torch.float32 and sc.shape == (Hkv,)):
                raise ValueError(f"an fp8 cache needs {name} float32 [{Hkv}], got "
                                 f"{None if sc is None else (sc.dtype, tuple(sc.shape))}")
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale apply to fp8 caches only")
    _check_index_args(B, page_table, seq_lens)
    _check_out_lse(out, lse, qs, qd, qs[:-1])


def _check_mla_args(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    v_dim: int, out: Optional[torch.Tensor], lse: Optional[torch.Tensor]):
    """Shapes and dtypes of an MLA call, q [B][H][576] or [B][n][H][576]."""
    qs = q.shape
    if len(qs) not in (3, 4):
        raise ValueError(f"q must be [B][H][Dk] or [B][rows][H][Dk], got {tuple(qs)}")
    if q.dtype is not torch.bfloat16:
        raise ValueError(f"MLA q must be bfloat16, got {q.dtype}")
    Dk = qs[-1]
    ks = kv_pages.shape
    if not (len(ks) == 3 and kv_pages.dtype is torch.bfloat16):
        raise ValueError(f"MLA kv_pages must be bfloat16 [num_pages][P][{Dk}], got {kv_pages.dtype} {tuple(ks)}")
    if ks[2] != Dk:
        raise ValueError(f"the cache's latent width {ks[2]} differs from q's {Dk}")
    if not (1 <= v_dim <= Dk):
        raise ValueError(f"v_dim {v_dim} must lie in [1, {Dk}]")
    _check_index_args(qs[0], page_table, seq_lens)
    _check_out_lse(out, lse, qs[:-1] + (v_dim,), torch.bfloat16, qs[:-1])


def paged_desc(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, *, k_scale=None, v_scale=None,
               workers: int = 0) -> PagedDesc:
    B, Hq, D = q.shape
    num_pages, two, Hkv, P, D2 = kv_pages.shape
    if two != 2 or D2 != D:
        raise ValueError(f"kv_pages must be [num_pages][2][Hkv][P][{D}], got {tuple(kv_pages.shape)}")
    return PagedDesc(B, Hq, Hkv, D, P, num_pages, page_table.shape[1], dtype_tag(q), dtype_tag(kv_pages),
                     workers, _ptr(k_scale), _ptr(v_scale))


def decode_attn_paged(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                      scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      workers: int = 0, want_lse: bool = True, stream=None):
    """Paged GQA decode attention.  q [B][Hq][D] (fp32 or bf16); kv_pages
    [num_pages][2][Hkv][P][D] with P = 16, 32, ..., 256 (fp32, bf16, or fp8-e4m3 as
    float8_e4m3fn/uint8 with k_scale/v_scale [Hkv] fp32); page_table int32
    [B][max_pages]; seq_lens int32 [B].
    Returns (out [B][Hq][D] in q's dtype, lse [B][Hq] fp32 or None)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [B][Hq][D], got {tuple(q.shape)}")
    _check_paged_args(q, kv_pages, page_table, seq_lens, out, lse, k_scale, v_scale)
    _need_cuda(q, kv_pages, page_table, seq_lens, k_scale, v_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _need_cuda(out, lse)
    d = paged_desc(q, kv_pages, page_table, k_scale=k_scale, v_scale=v_scale, workers=workers)
    st = _lib.decode_attn_paged(ctypes.byref(d), _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                                float(scale), _ptr(out), _ptr(lse), _stream(stream, q.get_device()))
    _check(st, "decode_attn_paged")
    return out, lse


def decode_attn_paged_rows(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                           seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, *, k_scale: Optional[torch.Tensor] = None,
                           v_scale: Optional[torch.Tensor] = None, workers: int = 0, want_lse: bool = True,
                           stream=None):
    """Paged GQA decode attention with several query rows per request.  q
    [B][n][Hq][D]: row i of request b is the token at position seq_lens[b] - n + i
    and sees positions up to its own.  Returns (out [B][n][Hq][D] in q's dtype,
    lse [B][n][Hq] fp32 or None)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B][rows][Hq][D], got {tuple(q.shape)}")
    _check_paged_args(q, kv_pages, page_table, seq_lens, out, lse, k_scale, v_scale)
    _need_cuda(q, kv_pages, page_table, seq_lens, k_scale, v_scale)
    B, n, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, n, Hq), dtype=torch.float32, device=q.device)
    _need_cuda(out, lse)
    d = paged_desc(q[:, 0], kv_pages, page_table, k_scale=k_scale, v_scale=v_scale, workers=workers)
    st = _lib.decode_attn_paged_rows(ctypes.byref(d), n, _ptr(q), _ptr(kv_pages), _ptr(page_table),
                                     _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _stream(stream, q.get_device()))
    _check(st, "decode_attn_paged_rows")
    return out, lse


def decode_attn_mla(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    scale: float, v_dim: int = 512, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, *, workers: int = 0,
                    want_lse: bool = True, stream=None):
    """Absorbed MLA decode.  q bf16 [B][H][576]; kv_pages bf16 [num_pages][P][576].
    Returns (out bf16 [B][H][v_dim], lse fp32 [B][H] or None)."""
    if q.dim() != 3:
        raise ValueError(f"q must be [B][H][Dk], got {tuple(q.shape)}")
    _check_mla_args(q, kv_pages, page_table, seq_lens, v_dim, out, lse)
    _need_cuda(q, kv_pages, page_table, seq_lens)
    B, H, Dk = q.shape
    if out is None:
        out = torch.empty((B, H, v_dim), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need_cuda(out, lse)
    num_pages, P, Dk2 = kv_pages.shape
    d = MLADesc(B, H, Dk, v_dim, P, num_pages, page_table.shape[1], workers)
    st = _lib.decode_attn_mla(ctypes.byref(d), _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                              float(scale), _ptr(out), _ptr(lse), _stream(stream, q.get_device()))
    _check(st, "decode_attn_mla")
    return out, lse


def decode_attn_mla_rows(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                         seq_lens: torch.Tensor, scale: float, v_dim: int = 512, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, *, workers: int = 0, want_lse: bool = True,
                         stream=None):
    """Absorbed MLA decode with several query rows per request.  q bf16
    [B][n][H][576]: row i of request b sees latent positions up to
    seq_lens[b] - n + i.  Returns (out bf16 [B][n][H][v_dim], lse fp32 [B][n][H] or None)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B][rows][H][576], got {tuple(q.shape)}")
    _check_mla_args(q, kv_pages, page_table, seq_lens, v_dim, out, lse)
    _need_cuda(q, kv_pages, page_table, seq_lens)
    B, n, H, Dk = q.shape
    if out is None:
        out = torch.empty((B, n, H, v_dim), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=q.device)
    _need_cuda(out, lse)
    num_pages, P, Dk2 = kv_pages.shape
    d = MLADesc(B, H, Dk, v_dim, P, num_pages, page_table.shape[1], workers)
    st = _lib.decode_attn_mla_rows(ctypes.byref(d), n, _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                                   float(scale), _ptr(out), _ptr(lse), _stream(stream, q.get_device()))
    _check(st, "decode_attn_mla_rows")
    return out, lse


def decode_attn_plan(seq_lens: torch.Tensor, page_size: int, units: int, workers: int, stream=None):
    """Run the split-KV planner alone; returns its outputs as int32 tensors."""
    _want(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1,
          f"seq_lens must be int32 [B], got {seq_lens.dtype} {tuple(seq_lens.shape)}")
    _need_cuda(seq_lens)
    B = seq_lens.shape[0]
    dev = seq_lens.device
    z = lambda *s: torch.zeros(s, dtype=torch.int32, device=dev)
    active, cuts, cursors = z(1), z(workers + 1), z(workers + 1, 4)
    fw, count = z(B * units), z(B * units)
    st = _lib.decode_attn_plan(B, _ptr(seq_lens), page_size, units, workers, _ptr(active), _ptr(cuts),
                               _ptr(cursors), _ptr(fw), _ptr(count), _stream(stream, seq_lens.get_device()))
    _check(st, "decode_attn_plan")
    return dict(active=active, cuts=cuts, cursors=cursors, first_worker=fw, piece_count=count)


def paged_kv_gather(kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, mla: bool = False,
                    stream=None) -> torch.Tensor:
    """Dense copy of every live token through the kernels' address function.
    GQA: [B][max_pages*P][2][Hkv][D]; MLA: [B][max_pages*P][Dk]; rows past L are zero."""
    _want(kv_pages.dim() == (3 if mla else 5), f"kv_pages has the wrong rank: {tuple(kv_pages.shape)}")
    _check_index_args(page_table.shape[0] if page_table.dim() == 2 else -1, page_table, seq_lens)
    _need_cuda(kv_pages, page_table, seq_lens)
    B, maxp = page_table.shape
    if mla:
        num_pages, P, Dk = kv_pages.shape
        dense = torch.zeros((B, maxp * P, Dk), dtype=kv_pages.dtype, device=kv_pages.device)
        d = PagedDesc(B, 1, 1, Dk, P, num_pages, maxp, DA_BF16, dtype_tag(kv_pages), 0, None, None)
    else:
        num_pages, _, Hkv, P, D = kv_pages.shape
        dense = torch.zeros((B, maxp * P, 2, Hkv, D), dtype=kv_pages.dtype, device=kv_pages.device)
        d = PagedDesc(B, Hkv, Hkv, D, P, num_pages, maxp, DA_F32, dtype_tag(kv_pages), 0, None, None)
    st = _lib.paged_kv_gather(ctypes.byref(d), 1 if mla else 0, _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                              _ptr(dense), _stream(stream, kv_pages.get_device()))
    _check(st, "paged_kv_gather")
    return dense


def decode_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                     positions: torch.Tensor, *, k_scale: Optional[torch.Tensor] = None,
                     v_scale: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Write each request's new K/V ([B][Hkv][D], fp32 or bf16) at token positions[b]
    of its paged history in kv_pages [num_pages][2][Hkv][P][D] (fp32, bf16, or fp8
    with k_scale/v_scale [Hkv]); a negative position skips the request.  In place;
    returns kv_pages."""
    _want(k_new.dim() == 3 and kv_pages.dim() == 5, "k_new must be [B][Hkv][D], kv_pages [num_pages][2][Hkv][P][D]")
    B, Hkv, D = k_new.shape
    num_pages, two, Hkv2, P, D2 = kv_pages.shape
    if two != 2 or Hkv2 != Hkv or D2 != D or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new, v_new must be [B][Hkv][D] matching kv_pages [num_pages][2][Hkv][P][D]")
    _want(k_new.dtype == v_new.dtype and k_new.dtype in (torch.float32, torch.bfloat16),
          f"k_new and v_new must share one dtype, float32 or bfloat16: {k_new.dtype}, {v_new.dtype}")
    fp8 = kv_pages.dtype in _FP8
    if fp8:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            _want(sc is not None and sc.dtype == torch.float32 and tuple(sc.shape) == (Hkv,),
                  f"an fp8 cache needs {name} float32 [{Hkv}]")
    else:
        _want(k_scale is None and v_scale is None, "k_scale / v_scale apply to fp8 caches only")
    _check_index_args(B, page_table, positions, "positions")
    _need_cuda(k_new, v_new, kv_pages, page_table, positions, k_scale, v_scale)
    d = PagedDesc(B, Hkv, Hkv, D, P, num_pages, page_table.shape[1], dtype_tag(k_new), dtype_tag(kv_pages), 0,
                  _ptr(k_scale), _ptr(v_scale))
    st = _lib.decode_kv_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(kv_pages), _ptr(page_table),
                               _ptr(positions), _stream(stream, kv_pages.get_device()))
    _check(st, "decode_kv_append")
    return kv_pages


def decode_kv_append_mla(latent_new: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                         positions: torch.Tensor, stream=None) -> torch.Tensor:
    """Write each request's new bf16 latent ([B][576]) at token positions[b] of its
    paged history in kv_pages [num_pages][P][576]; in place; returns kv_pages."""
    _want(latent_new.dim() == 2 and kv_pages.dim() == 3, "latent_new must be [B][576], kv_pages [num_pages][P][576]")
    B, Dk = latent_new.shape
    num_pages, P, Dk2 = kv_pages.shape
    if Dk2 != Dk:
        raise ValueError("latent_new [B][576] must match kv_pages [num_pages][P][576]")
    _want(latent_new.dtype == torch.bfloat16 and kv_pages.dtype == torch.bfloat16,
          f"latent_new and kv_pages must be bfloat16, got {latent_new.dtype}, {kv_pages.dtype}")
    _check_index_args(B, page_table, positions, "positions")
    _need_cuda(latent_new, kv_pages, page_table, positions)
    d = MLADesc(B, 128, Dk, 512, P, num_pages, page_table.shape[1], 0)
    st = _lib.decode_kv_append_mla(ctypes.byref(d), _ptr(latent_new), _ptr(kv_pages), _ptr(page_table),
                                   _ptr(positions), _stream(stream, kv_pages.get_device()))
    _check(st, "decode_kv_append_mla")
    return kv_pages


def default_workers(q: torch.Tensor = None, kv_pages: torch.Tensor = None, page_table: torch.Tensor = None,
                    *, mla_desc: Optional[MLADesc] = None, k_scale=None, v_scale=None) -> int:
    out = ctypes.c_int32(0)
    if mla_desc is not None:
        st = _lib.decode_attn_default_workers(None, ctypes.byref(mla_desc), ctypes.byref(out))
    else:
        d = paged_desc(q, kv_pages, page_table, k_scale=k_scale, v_scale=v_scale)
        st = _lib.decode_attn_default_workers(ctypes.byref(d), None, ctypes.byref(out))
    _check(st, "decode_attn_default_workers")
    return int(out.value)


def kernel_name(desc, q_rows: int = 1) -> Optional[str]:
    """The attention kernel a call with this descriptor (PagedDesc or MLADesc)
    and q_rows query rows runs, or None when the call would be refused (host
    query)."""
    if isinstance(desc, MLADesc):
        r = _lib.decode_attn_kernel_name(None, ctypes.byref(desc), int(q_rows))
    else:
        r = _lib.decode_attn_kernel_name(ctypes.byref(desc), None, int(q_rows))
    return None if r is None else r.decode()


def _rows_view(q: torch.Tensor) -> torch.Tensor:
    """[B][Hq][D] -> [B][1][Hq][D]; [B][n][Hq][D] as is."""
    return q.unsqueeze(1) if q.dim() == 3 else q


def workspace_size(desc, q_rows: int = 1) -> int:
    """Device workspace bytes one call with this descriptor (PagedDesc or
    MLADesc) and q_rows query rows needs (host query)."""
    out = ctypes.c_size_t(0)
    if isinstance(desc, MLADesc):
        st = _lib.decode_attn_workspace_size(None, ctypes.byref(desc), int(q_rows), ctypes.byref(out))
    else:
        st = _lib.decode_attn_workspace_size(ctypes.byref(desc), None, int(q_rows), ctypes.byref(out))
    _check(st, "decode_attn_workspace_size")
    return int(out.value)


def decode_attn_paged_ws(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                         scale: float, workspace: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                         *, k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                         workers: int = 0, stream=None):
    """decode_attn_paged / decode_attn_paged_rows with a caller-owned workspace
    (a byte tensor of at least workspace_size(...) bytes); q [B][Hq][D] or
    [B][n][Hq][D], out shaped like q.  Allocates nothing."""
    _want(out is not None, "the _ws entry points write into a caller-owned out")
    _check_paged_args(q, kv_pages, page_table, seq_lens, out, lse, k_scale, v_scale)
    _want(workspace.dim() == 1, "workspace must be a flat byte tensor")
    _need_cuda(q, kv_pages, page_table, seq_lens, k_scale, v_scale, workspace, out, lse)
    q4 = _rows_view(q)
    d = paged_desc(q4[:, 0], kv_pages, page_table, k_scale=k_scale, v_scale=v_scale, workers=workers)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.decode_attn_paged_ws(ctypes.byref(d), q4.shape[1], _ptr(q), _ptr(kv_pages), _ptr(page_table),
                                   _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _ptr(workspace), nbytes,
                                   _stream(stream, q.get_device()))
    _check(st, "decode_attn_paged_ws")
    return out, lse


# bytes of the device scratch array behind decode_attn_paged_noalloc (one per device)
NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_attn_paged_noalloc(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                              seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                              lse: Optional[torch.Tensor] = None, *, k_scale: Optional[torch.Tensor] = None,
                              v_scale: Optional[torch.Tensor] = None, workers: int = 0, stream=None):
    """decode_attn_paged / decode_attn_paged_rows for callers that cannot
    allocate: the workspace is the library's static per-device scratch
    (NOALLOC_SCRATCH_BYTES); q [B][Hq][D] or [B][n][Hq][D], out shaped like q
    and owned by the caller.  Calls that may overlap on one device race."""
    _want(out is not None, "decode_attn_paged_noalloc writes into a caller-owned out")
    _check_paged_args(q, kv_pages, page_table, seq_lens, out, lse, k_scale, v_scale)
    _need_cuda(q, kv_pages, page_table, seq_lens, k_scale, v_scale, out, lse)
    q4 = _rows_view(q)
    d = paged_desc(q4[:, 0], kv_pages, page_table, k_scale=k_scale, v_scale=v_scale, workers=workers)
    st = _lib.decode_attn_paged_noalloc(ctypes.byref(d), q4.shape[1], _ptr(q), _ptr(kv_pages), _ptr(page_table),
                                        _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _stream(stream, q.get_device()))
    _check(st, "decode_attn_paged_noalloc")
    return out, lse


def decode_attn_mla_ws(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                       scale: float, workspace: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                       *, v_dim: int = 512, workers: int = 0, stream=None):
    """decode_attn_mla / decode_attn_mla_rows with a caller-owned workspace;
    q [B][H][576] or [B][n][H][576].  Allocates nothing."""
    _want(out is not None, "the _ws entry points write into a caller-owned out")
    _check_mla_args(q, kv_pages, page_table, seq_lens, v_dim, out, lse)
    _want(workspace.dim() == 1, "workspace must be a flat byte tensor")
    _need_cuda(q, kv_pages, page_table, seq_lens, workspace, out, lse)
    q4 = _rows_view(q)
    B, n, H, Dk = q4.shape
    num_pages, P, _ = kv_pages.shape
    d = MLADesc(B, H, Dk, v_dim, P, num_pages, page_table.shape[1], workers)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.decode_attn_mla_ws(ctypes.byref(d), n, _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(seq_lens),
                                 float(scale), _ptr(out), _ptr(lse), _ptr(workspace), nbytes, _stream(stream, q.get_device()))
    _check(st, "decode_attn_mla_ws")
    return out, lse


def validate_inputs(desc, page_table: torch.Tensor, seq_lens: torch.Tensor, stream=None) -> int:
    """Debug check of lengths and used page ids (synchronises); returns the
    status (0, or -7 = DA_ERR_DATA when a precondition fails)."""
    _check_index_args(desc.batch, page_table, seq_lens)
    _need_cuda(page_table, seq_lens)
    if isinstance(desc, MLADesc):
        return _lib.decode_attn_validate_inputs(None, ctypes.byref(desc), _ptr(page_table), _ptr(seq_lens),
                                                _stream(stream, page_table.get_device()))
    return _lib.decode_attn_validate_inputs(ctypes.byref(desc), None, _ptr(page_table), _ptr(seq_lens),
                                            _stream(stream, page_table.get_device()))


def timer_begin(max_launches: int):
    """Time the main attention kernel of each following call (see decode_attn.h)."""
    _check(_lib.decode_attn_timer_begin(int(max_launches)), "decode_attn_timer_begin")


def timer_end():
    """Returns (summed kernel milliseconds, number of timed launches)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(_lib.decode_attn_timer_end(ctypes.byref(ms), ctypes.byref(n)), "decode_attn_timer_end")
    return ms.value, n.value


__all__ = ["timer_begin", "timer_end", "decode_attn_paged", "decode_attn_paged_rows", "decode_attn_mla",
           "decode_attn_mla_rows", "decode_attn_plan", "paged_kv_gather", "default_workers",
           "PagedDesc", "MLADesc", "DecodeAttnError", "LIB_PATH", "EXPORTS", "lib", "decode_kv_append", "decode_kv_append_mla",
           "workspace_size", "decode_attn_paged_ws", "decode_attn_mla_ws", "validate_inputs",
           "decode_attn_paged_noalloc", "NOALLOC_SCRATCH_BYTES", "kernel_name"]
