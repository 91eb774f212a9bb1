"""Python binding of libsparse3d.so (argument marshalling only).

Every function here has the name of the C entry point it wraps.  Torch provides
device memory and the current stream; all computation happens in the library's
HIP kernels.  If the library is not built, loading fails with an ImportError:
there is no fallback path.

Layouts are plain tuples ``(frames, tokens, stride, specials)``.  Tensors are
contiguous ``[heads, frames*stride, 64]`` on one HIP device.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "Sparse3dError", "library", "sparse3d_abi_version", "sparse3d_status_string",
    "sparse3d_tile_scores", "sparse3d_select_topk", "sparse3d_sparse_attn_fwd",
    "sparse3d_dense_attn_fwd", "sparse3d_subsample_layout", "sparse3d_grid_subsample_kv",
    "sparse3d_cast", "sparse3d_select_topk_per_head", "sparse3d_frame_attn_fwd",
    "sparse3d_discarded_mean", "Sga", "sparse3d_selection_transpose", "sparse3d_sparse_attn_bwd",
    "kmax_for", "LN64",
]

LN64 = math.log(64.0)
TILE = 64
HEAD_DIM = 64
F32, BF16 = 0, 1
_LIBPATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse3d.so")
_lib = None


class Sparse3dError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sparse3d status {status}: {msg}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("stride", ctypes.c_int32), ("specials", ctypes.c_int32)]


class _Sga(ctypes.Structure):
    _fields_ = [("k_full", ctypes.c_void_p), ("v_full", ctypes.c_void_p),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("window", ctypes.c_int32),
                ("kmean", ctypes.c_void_p), ("vmean", ctypes.c_void_p), ("mean_bias", ctypes.c_float)]


_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
_LP = ctypes.POINTER(_Layout)
_SP = ctypes.POINTER(_Sga)

_SIGS = {
    "sparse3d_abi_version": ([], ctypes.c_int),
    "sparse3d_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sparse3d_tile_scores": ([_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _LP, _LP, _f32,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "sparse3d_select_topk": ([_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp],
                             ctypes.c_int),
    "sparse3d_sparse_attn_fwd": ([_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _LP, _LP, _vp,
                                  _vp, _i32, _vp, _vp, _f32, _f32, _SP, _vp, ctypes.c_int, _vp, _vp],
                                 ctypes.c_int),
    "sparse3d_dense_attn_fwd": ([_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _LP, _LP, _f32, _SP, _vp,
                                 ctypes.c_int, _vp, _vp], ctypes.c_int),
    "sparse3d_discarded_mean": ([_vp, _vp, ctypes.c_int, _i32, _i32, _LP, _i32, _i32, _i32, _vp, _vp,
                                 _vp], ctypes.c_int),
    "sparse3d_selection_transpose": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "sparse3d_sparse_attn_bwd": ([_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _LP, _LP,
                                  _vp, _vp, _i32, _vp, _vp, _vp, _vp, _f32, _f32, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp], ctypes.c_int),
    "sparse3d_subsample_layout": ([_LP, _i32, _i32, _i32, _i32, _LP], ctypes.c_int),
    "sparse3d_grid_subsample_kv": ([_vp, _vp, ctypes.c_int, _i32, _i32, _LP, _i32, _i32, _i32,
                                    _vp, _vp, _LP, _vp], ctypes.c_int),
    "sparse3d_cast": ([_vp, ctypes.c_int64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "sparse3d_select_topk_per_head": ([_vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp],
                                      ctypes.c_int),
    "sparse3d_frame_attn_fwd": ([_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _LP, _LP, _f32, _vp,
                                 ctypes.c_int, _vp, _vp], ctypes.c_int),
}


def library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsparse3d.so once (ImportError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIBPATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m dynamic_block_sparse_tile_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise Sparse3dError(status, library().sparse3d_status_string(status).decode())


def _lay(t: Sequence[int]) -> _Layout:
    f, n, p, s = (int(x) for x in t)
    return _Layout(f, n, p, s)


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {x.dtype} (bfloat16 or float32)")


def _dev(x: torch.Tensor, name: str) -> torch.Tensor:
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _rows(lay) -> int:
    return int(lay[0]) * int(lay[2])


def _expect(x: Optional[torch.Tensor], name: str, shape: Sequence[int], dtypes) -> None:
    """Shape and dtype of one argument against what the layouts and sizes imply; runs
    before anything touches the device, so a mismatched tensor never reaches a kernel."""
    if x is None:
        return
    want = tuple(int(d) for d in shape)
    if tuple(x.shape) != want:
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {want}")
    if x.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {x.dtype}, expected one of {[str(d) for d in dtypes]}")


_OPERAND = (torch.bfloat16, torch.float32)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _operands(q, k, v, qlay, klay, heads=None):
    """q: [H, qlay rows, 64] in bf16 or fp32; k (and v): [H, klay rows, 64] in q's dtype."""
    if q.dim() != 3:
        raise ValueError(f"q must be [heads, rows, {HEAD_DIM}], got shape {tuple(q.shape)}")
    H = q.shape[0] if heads is None else heads
    _expect(q, "q", (H, _rows(qlay), HEAD_DIM), _OPERAND)
    _expect(k, "k", (H, _rows(klay), HEAD_DIM), (q.dtype,))
    _expect(v, "v", (H, _rows(klay), HEAD_DIM), (q.dtype,))
    devs = {x.device for x in (q, k, v) if x is not None}
    if len(devs) > 1:
        raise ValueError("q, k and v must be on one device")
    return H


def _same_device(ref: torch.Tensor, *xs) -> None:
    for x in xs:
        if x is not None and x.device != ref.device:
            raise ValueError("every tensor of a call must be on one device")


def _stream(x: torch.Tensor) -> int:
    return torch.cuda.current_stream(x.device).cuda_stream


def _ptr(x: Optional[torch.Tensor]) -> Optional[int]:
    return None if x is None else x.data_ptr()


class Sga:
    """Subsample completion for the attention calls: the own key of dropped positions
    (k_full/v_full: K and V before the subsample) and/or one mean pair (kmean/vmean from
    ``sparse3d_discarded_mean``, logit offset mean_bias = ln |D|)."""

    def __init__(self, grid, window, k_full=None, v_full=None, kmean=None, vmean=None,
                 mean_bias: float = 0.0):
        self.grid, self.window = tuple(grid), int(window)
        self.k_full, self.v_full, self.kmean, self.vmean = k_full, v_full, kmean, vmean
        self.mean_bias = float(mean_bias)

    def _c(self, q):
        H = q.shape[0]
        for x, n in ((self.k_full, "k_full"), (self.v_full, "v_full")):
            _expect(x, n, q.shape, (q.dtype,))
        for x, n in ((self.kmean, "kmean"), (self.vmean, "vmean")):
            _expect(x, n, (H, HEAD_DIM), _F32)
        _same_device(q, self.k_full, self.v_full, self.kmean, self.vmean)
        for x, n in ((self.k_full, "k_full"), (self.v_full, "v_full"), (self.kmean, "kmean"),
                     (self.vmean, "vmean")):
            if x is not None:
                _dev(x, n)
        return _Sga(_ptr(self.k_full), _ptr(self.v_full), self.grid[0], self.grid[1], self.window,
                    _ptr(self.kmean), _ptr(self.vmean), self.mean_bias)


def _sga_ref(sga, q):
    return None if sga is None else ctypes.byref(sga._c(q))


def sparse3d_abi_version() -> int:
    return library().sparse3d_abi_version()


def sparse3d_status_string(status: int) -> str:
    return library().sparse3d_status_string(status).decode()


def _tiles(lay) -> int:
    return lay[0] * lay[2] // TILE


def sparse3d_tile_scores(q: torch.Tensor, k: torch.Tensor, qlay, klay=None,
                         v: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                         operand_means: bool = False):
    """Pooled tile summaries and tile scores.  Returns (qbar, kbar, vbar|None, scores); with
    ``operand_means`` also (kbar_op, vbar_op|None), the key/value means in q's dtype (the
    landmark means the attention calls take), written by the same pooling pass."""
    klay = qlay if klay is None else klay
    H = _operands(q, k, v, qlay, klay)
    _dev(q, "q"), _dev(k, "k")
    if v is not None:
        _dev(v, "v")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale
    Tq, Tk = _tiles(qlay), _tiles(klay)
    f = dict(device=q.device, dtype=torch.float32)
    qbar = torch.empty((H, Tq, HEAD_DIM), **f)
    kbar = torch.empty((H, Tk, HEAD_DIM), **f)
    vbar = torch.empty((H, Tk, HEAD_DIM), **f) if v is not None else None
    scores = torch.empty((H, Tq, Tk), **f)
    kop = vop = None
    if operand_means:
        kop = torch.empty((H, Tk, HEAD_DIM), device=q.device, dtype=q.dtype)
        vop = torch.empty((H, Tk, HEAD_DIM), device=q.device, dtype=q.dtype) if v is not None else None
    ql, kl = _lay(qlay), _lay(klay)
    _check(library().sparse3d_tile_scores(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), H, q.shape[2], TILE, ctypes.byref(ql), ctypes.byref(kl),
        scale, _ptr(qbar), _ptr(kbar), _ptr(vbar), _ptr(scores), _ptr(kop), _ptr(vop), _stream(q)))
    if operand_means:
        return qbar, kbar, vbar, scores, kop, vop
    return qbar, kbar, vbar, scores


def kmax_for(k_tiles: int, k: int, tiles_per_frame: int, anchor_frame: int) -> int:
    """Size of the index table's last axis: min(Tk, k + anchor tiles)."""
    return min(k_tiles, max(k, 0) + (tiles_per_frame if anchor_frame >= 0 else 0))


def sparse3d_select_topk(scores: torch.Tensor, k: int, tiles_per_frame: int, anchor_frame: int = 0,
                         kmax: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k key tiles per query tile united with the anchor frame.  Returns (idx, cnt)."""
    if scores.dim() != 3:
        raise ValueError(f"scores must be [heads, q_tiles, k_tiles], got shape {tuple(scores.shape)}")
    _expect(scores, "scores", scores.shape, _F32)
    _dev(scores, "scores")
    H, Tq, Tk = scores.shape
    kmax = kmax_for(Tk, k, tiles_per_frame, anchor_frame) if kmax is None else kmax
    idx = torch.empty((H, Tq, max(kmax, 0)), device=scores.device, dtype=torch.int32)
    cnt = torch.empty((H, Tq), device=scores.device, dtype=torch.int32)
    _check(library().sparse3d_select_topk(
        _ptr(scores), H, Tq, Tk, k, tiles_per_frame, anchor_frame,
        _ptr(idx) if kmax > 0 else None, _ptr(cnt), kmax, _stream(scores)))
    return idx, cnt


def sparse3d_select_topk_per_head(scores: torch.Tensor, ks: Sequence[int], tiles_per_frame: int,
                                  anchor_frame: int = 0, kmax: Optional[int] = None):
    """Top-k_h key tiles per query tile of head h, united with the anchor frame."""
    if scores.dim() != 3:
        raise ValueError(f"scores must be [heads, q_tiles, k_tiles], got shape {tuple(scores.shape)}")
    _expect(scores, "scores", scores.shape, _F32)
    _dev(scores, "scores")
    H, Tq, Tk = scores.shape
    ks = [int(x) for x in ks]
    if len(ks) != H:
        raise ValueError(f"need one budget per head ({H}), got {len(ks)}")
    kmax = kmax_for(Tk, max(ks), tiles_per_frame, anchor_frame) if kmax is None else kmax
    idx = torch.empty((H, Tq, max(kmax, 0)), device=scores.device, dtype=torch.int32)
    cnt = torch.empty((H, Tq), device=scores.device, dtype=torch.int32)
    karr = (ctypes.c_int32 * H)(*ks)
    _check(library().sparse3d_select_topk_per_head(
        _ptr(scores), H, Tq, Tk, ctypes.cast(karr, ctypes.c_void_p), tiles_per_frame, anchor_frame,
        _ptr(idx) if kmax > 0 else None, _ptr(cnt), kmax, _stream(scores)))
    return idx, cnt


def _out_dtype(q, out_dtype):
    od = q.dtype if out_dtype is None else out_dtype
    if od not in _OPERAND:
        raise TypeError(f"out_dtype must be bfloat16 or float32, not {od}")
    return od, (BF16 if od == torch.bfloat16 else F32)


def sparse3d_sparse_attn_fwd(q, k, v, qlay, klay, idx, cnt, kbar=None, vbar=None,
                             landmark_bias: float = LN64, scale: Optional[float] = None,
                             out_dtype=None, return_lse: bool = False, sga: Optional[Sga] = None):
    """Attention over specials + selected tiles (+ landmarks when kbar/vbar are given).

    kbar/vbar are the tile means in q's dtype (for bf16, ``sparse3d_cast`` of the fp32
    means that ``sparse3d_tile_scores`` returns)."""
    H = _operands(q, k, v, qlay, klay)
    _out_dtype(q, out_dtype)
    if idx.dim() != 3:
        raise ValueError(f"idx must be [heads, q_tiles, kmax], got shape {tuple(idx.shape)}")
    Tq, Tk = _tiles(qlay), _tiles(klay)
    _expect(idx, "idx", (H, Tq, idx.shape[2]), _I32)
    _expect(cnt, "cnt", (H, Tq), _I32)
    if (kbar is None) != (vbar is None):
        raise ValueError("kbar and vbar go together")
    # landmark means in the operand dtype (for bf16: sparse3d_cast of the fp32 means)
    _expect(kbar, "kbar", (H, Tk, HEAD_DIM), (q.dtype,))
    _expect(vbar, "vbar", (H, Tk, HEAD_DIM), (q.dtype,))
    _same_device(q, idx, cnt, kbar, vbar)
    sga_c = _sga_ref(sga, q)
    for x, n in ((q, "q"), (k, "k"), (v, "v"), (idx, "idx"), (cnt, "cnt")):
        _dev(x, n)
    if kbar is not None:
        _dev(kbar, "kbar"), _dev(vbar, "vbar")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale
    od, odc = _out_dtype(q, out_dtype)
    out = torch.empty(q.shape, device=q.device, dtype=od)
    lse = torch.empty(q.shape[:2], device=q.device, dtype=torch.float32) if return_lse else None
    ql, kl = _lay(qlay), _lay(klay)
    kmax = idx.shape[2]
    _check(library().sparse3d_sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), H, q.shape[2], TILE, ctypes.byref(ql), ctypes.byref(kl),
        _ptr(idx) if kmax > 0 else None, _ptr(cnt), kmax, _ptr(kbar), _ptr(vbar), landmark_bias,
        scale, sga_c, _ptr(out), odc, _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def sparse3d_cast(x: torch.Tensor, dtype) -> torch.Tensor:
    """fp32 tensor -> new tensor of `dtype` (bfloat16: round to nearest even)."""
    if x.dtype != torch.float32:
        raise TypeError("sparse3d_cast converts from float32")
    if dtype not in _OPERAND:
        raise TypeError(f"sparse3d_cast converts to bfloat16 or float32, not {dtype}")
    _dev(x, "x")
    out = torch.empty(x.shape, device=x.device, dtype=dtype)
    _check(library().sparse3d_cast(_ptr(x), x.numel(), _dt(out), _ptr(out), _stream(x)))
    return out


def sparse3d_dense_attn_fwd(q, k, v, qlay, klay=None, scale: Optional[float] = None,
                            out_dtype=None, return_lse: bool = False, sga: Optional[Sga] = None):
    """Dense global attention over every valid key (the library's own baseline)."""
    klay = qlay if klay is None else klay
    H = _operands(q, k, v, qlay, klay)
    _out_dtype(q, out_dtype)
    sga_c = _sga_ref(sga, q)
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(x, n)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale
    od, odc = _out_dtype(q, out_dtype)
    out = torch.empty(q.shape, device=q.device, dtype=od)
    lse = torch.empty(q.shape[:2], device=q.device, dtype=torch.float32) if return_lse else None
    ql, kl = _lay(qlay), _lay(klay)
    _check(library().sparse3d_dense_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), H, q.shape[2], ctypes.byref(ql), ctypes.byref(kl),
        scale, sga_c, _ptr(out), odc, _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def sparse3d_frame_attn_fwd(q, k, v, qlay, klay=None, scale: Optional[float] = None,
                            out_dtype=None, return_lse: bool = False):
    """Attention of every valid query over the valid keys of its own frame only."""
    klay = qlay if klay is None else klay
    H = _operands(q, k, v, qlay, klay)
    _out_dtype(q, out_dtype)
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(x, n)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale
    od, odc = _out_dtype(q, out_dtype)
    out = torch.empty(q.shape, device=q.device, dtype=od)
    lse = torch.empty(q.shape[:2], device=q.device, dtype=torch.float32) if return_lse else None
    ql, kl = _lay(qlay), _lay(klay)
    _check(library().sparse3d_frame_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), H, q.shape[2], ctypes.byref(ql), ctypes.byref(kl),
        scale, _ptr(out), odc, _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def sparse3d_discarded_mean(k, v, lay, grid: Tuple[int, int], window: int):
    """Mean key and value of the patch rows the grid subsample drops (all frames, per head):
    (kmean [H, 64] fp32, vmean [H, 64] fp32, |D|)."""
    H = _operands(k, k, v, lay, lay)
    _dev(k, "k"), _dev(v, "v")
    kmean = torch.empty((H, HEAD_DIM), device=k.device, dtype=torch.float32)
    vmean = torch.empty_like(kmean)
    il = _lay(lay)
    _check(library().sparse3d_discarded_mean(_ptr(k), _ptr(v), _dt(k), H, k.shape[2], ctypes.byref(il),
                                             grid[0], grid[1], window, _ptr(kmean), _ptr(vmean),
                                             _stream(k)))
    gh, gw = grid
    kept = -(-gh // window) * -(-gw // window)
    return kmean, vmean, int(lay[0]) * (gh * gw - kept)


def sparse3d_selection_transpose(idx: torch.Tensor, cnt: torch.Tensor, k_tiles: int):
    """For each head and key tile, the ascending query tiles that selected it (CSR with end
    offsets).  Returns (t_end int32 [H, k_tiles], t_list int32 [H, q_tiles * kmax])."""
    if idx.dim() != 3:
        raise ValueError(f"idx must be [heads, q_tiles, kmax], got shape {tuple(idx.shape)}")
    H, Tq, kmax = idx.shape
    _expect(idx, "idx", idx.shape, _I32)
    _expect(cnt, "cnt", (H, Tq), _I32)
    _same_device(idx, cnt)
    _dev(idx, "idx"), _dev(cnt, "cnt")
    t_end = torch.empty((H, k_tiles), device=idx.device, dtype=torch.int32)
    t_list = torch.empty((H, Tq * max(kmax, 0)), device=idx.device, dtype=torch.int32)
    _check(library().sparse3d_selection_transpose(_ptr(idx) if kmax > 0 else None, _ptr(cnt), H, Tq,
                                                  k_tiles, kmax, _ptr(t_end),
                                                  _ptr(t_list) if kmax > 0 else None, _stream(idx)))
    return t_end, t_list


def sparse3d_sparse_attn_bwd(q, k, v, out, dout, lse, qlay, klay, idx, cnt, t_end, t_list,
                             kbar=None, vbar=None, landmark_bias: float = LN64,
                             scale: Optional[float] = None):
    """Gradients of the sparse attention, selection fixed.  Returns (dq, dk, dv, delta), fp32;
    with landmarks (kbar/vbar as given to the forward) (dq, dk, dv, delta, dkbar, dvbar),
    where dk/dv already include the means' gradients spread over the member rows."""
    H = _operands(q, k, v, qlay, klay)
    if idx.dim() != 3:
        raise ValueError(f"idx must be [heads, q_tiles, kmax], got shape {tuple(idx.shape)}")
    Tq, Tk = _tiles(qlay), _tiles(klay)
    _expect(idx, "idx", (H, Tq, idx.shape[2]), _I32)
    _expect(cnt, "cnt", (H, Tq), _I32)
    _expect(out, "out", q.shape, (q.dtype,))
    _expect(dout, "dout", q.shape, (q.dtype,))
    _expect(lse, "lse", q.shape[:2], _F32)
    _expect(t_end, "t_end", (H, Tk), _I32)
    _expect(t_list, "t_list", (H, Tq * idx.shape[2]), _I32)
    if (kbar is None) != (vbar is None):
        raise ValueError("kbar and vbar go together")
    _expect(kbar, "kbar", (H, Tk, HEAD_DIM), (q.dtype,))
    _expect(vbar, "vbar", (H, Tk, HEAD_DIM), (q.dtype,))
    _same_device(q, out, dout, lse, idx, cnt, t_end, t_list, kbar, vbar)
    for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (lse, "lse"),
                 (idx, "idx"), (cnt, "cnt"), (t_end, "t_end"), (t_list, "t_list")):
        _dev(x, n)
    if kbar is not None:
        _dev(kbar, "kbar"), _dev(vbar, "vbar")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale
    f = dict(device=q.device, dtype=torch.float32)
    dq = torch.empty(q.shape, **f)
    dk = torch.empty(k.shape, **f)
    dv = torch.empty(v.shape, **f)
    delta = torch.empty(q.shape[:2], **f)
    dkbar = torch.empty((H, Tk, HEAD_DIM), **f) if kbar is not None else None
    dvbar = torch.empty((H, Tk, HEAD_DIM), **f) if kbar is not None else None
    ql, kl = _lay(qlay), _lay(klay)
    kmax = idx.shape[2]
    _check(library().sparse3d_sparse_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dt(q), H, q.shape[2], TILE,
        ctypes.byref(ql), ctypes.byref(kl), _ptr(idx) if kmax > 0 else None, _ptr(cnt), kmax,
        _ptr(t_end), _ptr(t_list) if kmax > 0 else None, _ptr(kbar), _ptr(vbar), landmark_bias, scale,
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), _ptr(dkbar), _ptr(dvbar), _stream(q)))
    if kbar is not None:
        return dq, dk, dv, delta, dkbar, dvbar
    return dq, dk, dv, delta


def sparse3d_subsample_layout(lay, grid_h: int, grid_w: int, window: int, tile: int = TILE):
    """Key/value layout after the grid subsample, as a (frames, tokens, stride, specials) tuple."""
    src, dst = _lay(lay), _Layout()
    _check(library().sparse3d_subsample_layout(ctypes.byref(src), grid_h, grid_w, window, tile,
                                               ctypes.byref(dst)))
    return (dst.frames, dst.tokens, dst.stride, dst.specials)


def sparse3d_grid_subsample_kv(k, v, lay, grid: Tuple[int, int], window: int):
    """Thin keys/values on the patch grid.  Returns (k_sub, v_sub, layout_sub)."""
    H = _operands(k, k, v, lay, lay)
    _dev(k, "k"), _dev(v, "v")
    out_lay = sparse3d_subsample_layout(lay, grid[0], grid[1], window)
    rows = out_lay[0] * out_lay[2]
    k2 = torch.empty((H, rows, k.shape[2]), device=k.device, dtype=k.dtype)
    v2 = torch.empty_like(k2)
    il, ol = _lay(lay), _lay(out_lay)
    _check(library().sparse3d_grid_subsample_kv(
        _ptr(k), _ptr(v), _dt(k), H, k.shape[2], ctypes.byref(il), grid[0], grid[1], window,
        _ptr(k2), _ptr(v2), ctypes.byref(ol), _stream(k)))
    return k2, v2, out_lay
