"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before touching the GPU."""
import ctypes
import math
import os
import re

import pytest

from dynamic_block_sparse_tile_amd import sparse3d as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse3d.h")

NULL = None
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_HIP, ERR_ALIAS = 0, 1, 2, 3, 4, 5
FAKE = 0x7F0000000000        # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse3d_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return S.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(S._SIGS), "binding signatures must cover the header exactly"


def test_library_resolves_every_symbol_at_load():
    # RTLD_NOW: an undefined symbol in the built library fails here, on the CPU
    ctypes.CDLL(S._LIBPATH, mode=os.RTLD_NOW)


def test_version_and_status(lib):
    assert lib.sparse3d_abi_version() == 5
    for st in range(6):
        assert lib.sparse3d_status_string(st)
    assert lib.sparse3d_status_string(99) == b"unknown status"


def L(f=2, n=256, p=256, s=0):
    return ctypes.byref(S._Layout(f, n, p, s))


def scores_call(lib, q=FAKE, k=FAKE, v=NULL, dt=1, H=2, d=64, tile=64, ql=None, kl=None,
                qbar=FAKE + 10**9, kbar=FAKE + 2 * 10**9, vbar=NULL, sc=FAKE + 3 * 10**9, kop=NULL, vop=NULL):
    return lib.sparse3d_tile_scores(q, k, v, dt, H, d, tile, ql or L(), kl or L(), 0.125,
                                    qbar, kbar, vbar, sc, kop, vop, NULL)


def test_tile_scores_validation(lib):
    assert scores_call(lib, q=NULL) == ERR_NULL
    assert scores_call(lib, sc=NULL) == ERR_NULL
    assert scores_call(lib, v=FAKE + 4 * 10**9) == ERR_NULL            # v without vbar
    assert scores_call(lib, d=32) == ERR_UNSUP
    assert scores_call(lib, tile=32) == ERR_UNSUP
    assert scores_call(lib, dt=7) == ERR_UNSUP
    assert scores_call(lib, H=0) == ERR_SHAPE
    assert scores_call(lib, ql=L(p=200)) == ERR_SHAPE                   # stride % 64
    assert scores_call(lib, ql=L(n=300)) == ERR_SHAPE                   # tokens > stride
    assert scores_call(lib, ql=L(s=256)) == ERR_SHAPE                   # specials >= tokens
    assert scores_call(lib, kl=L(f=3, n=256, p=256)) == ERR_SHAPE       # frame counts differ
    assert scores_call(lib, sc=FAKE + 100) == ERR_ALIAS                 # scores overlaps q
    assert lib.sparse3d_tile_scores(FAKE, FAKE, NULL, 1, 2, 64, 64, NULL, L(), 0.1, FAKE + 10**9,
                                    FAKE + 2 * 10**9, NULL, FAKE + 3 * 10**9, NULL, NULL, NULL) == ERR_NULL
    # the means in the operand dtype: value means need the values, no overlap with anything
    assert scores_call(lib, vop=FAKE + 5 * 10**9) == ERR_NULL
    assert scores_call(lib, kop=FAKE + 2 * 10**9 + 64) == ERR_ALIAS      # inside kbar
    assert scores_call(lib, kop=FAKE + 64) == ERR_ALIAS                  # inside q
    assert scores_call(lib, v=FAKE + 4 * 10**9, vbar=FAKE + 5 * 10**9, kop=FAKE + 6 * 10**9,
                       vop=FAKE + 6 * 10**9 + 32) == ERR_ALIAS            # kop and vop overlap


def topk_call(lib, sc=FAKE, H=2, tq=8, tk=8, k=4, tpf=4, anchor=0, idx=FAKE + 10**9,
              cnt=FAKE + 2 * 10**9, kmax=8):
    return lib.sparse3d_select_topk(sc, H, tq, tk, k, tpf, anchor, idx, cnt, kmax, NULL)


def test_select_validation(lib):
    assert topk_call(lib, sc=NULL) == ERR_NULL
    assert topk_call(lib, cnt=NULL) == ERR_NULL
    assert topk_call(lib, idx=NULL) == ERR_NULL
    assert topk_call(lib, kmax=7) == ERR_SHAPE                          # k + anchor tiles = 8
    assert topk_call(lib, anchor=-1, kmax=3) == ERR_SHAPE
    assert topk_call(lib, tpf=3) == ERR_SHAPE                           # 8 % 3
    assert topk_call(lib, anchor=2) == ERR_SHAPE                        # only 2 frames
    assert topk_call(lib, anchor=-2) == ERR_SHAPE
    assert topk_call(lib, k=-1) == ERR_SHAPE
    assert topk_call(lib, tk=12289 * 1, tpf=12289, kmax=8, anchor=-1) == ERR_UNSUP
    assert topk_call(lib, idx=FAKE + 64) == ERR_ALIAS


def attn_call(lib, q=FAKE, k=FAKE + 10**9, v=FAKE + 2 * 10**9, dt=1, H=2, d=64, tile=64,
              ql=None, kl=None, idx=FAKE + 3 * 10**9, cnt=FAKE + 4 * 10**9, kmax=8, kbar=NULL,
              vbar=NULL, out=FAKE + 5 * 10**9, odt=1, lse=NULL, bias=4.1588830833596715,
              scale=0.125, sga=NULL):
    return lib.sparse3d_sparse_attn_fwd(q, k, v, dt, H, d, tile, ql or L(), kl or L(), idx, cnt,
                                        kmax, kbar, vbar, bias, scale, sga, out, odt, lse, NULL)


def test_attn_validation(lib):
    assert attn_call(lib, v=NULL) == ERR_NULL
    assert attn_call(lib, out=NULL) == ERR_NULL
    assert attn_call(lib, cnt=NULL) == ERR_NULL
    assert attn_call(lib, idx=NULL) == ERR_NULL
    assert attn_call(lib, kbar=FAKE + 6 * 10**9) == ERR_NULL            # kbar without vbar
    assert attn_call(lib, kmax=-1) == ERR_SHAPE
    assert attn_call(lib, odt=5) == ERR_UNSUP
    assert attn_call(lib, d=128) == ERR_UNSUP
    assert attn_call(lib, kl=L(f=3)) == ERR_SHAPE
    assert attn_call(lib, out=FAKE + 64) == ERR_ALIAS                   # out overlaps q
    assert attn_call(lib, lse=FAKE + 5 * 10**9 + 128) == ERR_ALIAS      # lse overlaps out
    assert lib.sparse3d_dense_attn_fwd(FAKE, FAKE, NULL, 1, 2, 64, L(), L(), 0.1, NULL, FAKE + 10**9, 1,
                                       NULL, NULL) == ERR_NULL
    assert lib.sparse3d_dense_attn_fwd(FAKE, FAKE, FAKE, 1, 2, 64, L(), L(), 0.1, NULL, FAKE + 64, 1,
                                       NULL, NULL) == ERR_ALIAS
    # a masked logit is -inf; only a finite positive scale keeps it out of the softmax
    for bad in (0.0, -0.125, float("inf"), float("nan")):
        assert attn_call(lib, scale=bad) == ERR_UNSUP
        assert lib.sparse3d_dense_attn_fwd(FAKE, FAKE, FAKE, 1, 2, 64, L(), L(), bad, NULL,
                                           FAKE + 10**9 * 5, 1, NULL, NULL) == ERR_UNSUP
    lm = dict(kbar=FAKE + 6 * 10**9, vbar=FAKE + 7 * 10**9)
    assert attn_call(lib, bias=float("inf"), **lm) == ERR_UNSUP
    assert attn_call(lib, bias=float("nan"), **lm) == ERR_UNSUP
    # out or lse must not overlap the landmark means ([2, 8, 64] bf16 = 2 KiB each)
    assert attn_call(lib, kbar=FAKE + 5 * 10**9 + 1024, vbar=FAKE + 7 * 10**9) == ERR_ALIAS
    assert attn_call(lib, lse=FAKE + 8 * 10**9, kbar=FAKE + 6 * 10**9,
                     vbar=FAKE + 8 * 10**9 - 64) == ERR_ALIAS


def test_per_head_select_validation(lib):
    def call(ks, kmax=8, anchor=0, tpf=4, k_ptr=None):
        arr = (ctypes.c_int32 * len(ks))(*ks)
        return lib.sparse3d_select_topk_per_head(FAKE, len(ks), 8, 16, k_ptr if k_ptr is not None else
                                                 ctypes.cast(arr, ctypes.c_void_p), tpf, anchor,
                                                 FAKE + 10**9, FAKE + 2 * 10**9, kmax, NULL)
    assert lib.sparse3d_select_topk_per_head(FAKE, 2, 8, 8, NULL, 4, 0, FAKE + 10**9,
                                             FAKE + 2 * 10**9, 8, NULL) == ERR_NULL
    assert call([2, -1]) == ERR_SHAPE                          # a negative budget
    assert call([2, 5], kmax=8) == ERR_SHAPE                   # largest budget 5 + 4 anchor tiles > 8
    assert call([2, 4], kmax=7) == ERR_SHAPE
    assert call([], kmax=8) == ERR_SHAPE                       # no heads
    assert call([1, 2], anchor=4) == ERR_SHAPE                 # only 4 frames of 4 tiles


def test_frame_attn_validation(lib):
    fa = lib.sparse3d_frame_attn_fwd
    assert fa(FAKE, FAKE, NULL, 1, 2, 64, L(), L(), 0.1, FAKE + 10**9, 1, NULL, NULL) == ERR_NULL
    assert fa(FAKE, FAKE, FAKE, 1, 2, 64, L(), L(f=3), 0.1, FAKE + 10**9, 1, NULL, NULL) == ERR_SHAPE
    assert fa(FAKE, FAKE, FAKE, 1, 2, 32, L(), L(), 0.1, FAKE + 10**9, 1, NULL, NULL) == ERR_UNSUP
    assert fa(FAKE, FAKE, FAKE, 1, 2, 64, L(), L(), 0.0, FAKE + 10**9, 1, NULL, NULL) == ERR_UNSUP
    assert fa(FAKE, FAKE, FAKE, 1, 2, 64, L(), L(), 0.1, FAKE + 64, 1, NULL, NULL) == ERR_ALIAS


def _sga(k_full=NULL, v_full=NULL, grid=(4, 4), window=2, kmean=NULL, vmean=NULL, bias=3.0):
    return ctypes.byref(S._Sga(k_full, v_full, grid[0], grid[1], window, kmean, vmean, bias))


def test_sga_validation(lib):
    # queries: 2 frames x (2 specials + 4x4 patches) in stride 64; keys: the 2x2 subsample
    ql = L(f=2, n=18, p=64, s=2)
    kl_ok = L(f=2, n=6, p=64, s=2)
    call = lambda sga, kl=None, out=FAKE + 5 * 10**9: attn_call(lib, ql=ql, kl=kl or kl_ok, sga=sga,
                                                                 kmax=2, out=out)
    assert call(_sga(k_full=FAKE + 6 * 10**9)) == ERR_NULL                  # own key without values
    assert call(_sga(kmean=FAKE + 7 * 10**9)) == ERR_NULL                   # mean key without value
    assert call(_sga(), kl=L(f=2, n=7, p=64, s=2)) == ERR_SHAPE             # keys are not that subsample
    assert call(_sga(grid=(3, 5))) == ERR_SHAPE                             # grid does not tile the frame
    assert call(_sga(window=0)) == ERR_SHAPE
    assert call(_sga(kmean=FAKE + 7 * 10**9, vmean=FAKE + 8 * 10**9, bias=float("nan"))) == ERR_UNSUP
    assert call(_sga(kmean=FAKE + 5 * 10**9 + 256, vmean=FAKE + 8 * 10**9)) == ERR_ALIAS   # inside out
    assert call(_sga(k_full=FAKE + 6 * 10**9, v_full=FAKE + 5 * 10**9 + 64)) == ERR_ALIAS
    dense = lambda sga: lib.sparse3d_dense_attn_fwd(FAKE, FAKE + 10**9, FAKE + 2 * 10**9, 1, 2, 64, ql,
                                                    L(f=2, n=5, p=64, s=2), 0.1, sga, FAKE + 5 * 10**9,
                                                    1, NULL, NULL)
    assert dense(_sga()) == ERR_SHAPE


def test_discarded_mean_validation(lib):
    dm = lambda k=FAKE, km=FAKE + 10**9, vm=FAKE + 2 * 10**9, grid=(4, 4), window=2, lay=None: \
        lib.sparse3d_discarded_mean(k, FAKE + 3 * 10**9, 1, 2, 64, lay or L(f=2, n=18, p=64, s=2),
                                    grid[0], grid[1], window, km, vm, NULL)
    assert dm(k=NULL) == ERR_NULL
    assert dm(km=NULL) == ERR_NULL
    assert dm(grid=(4, 5)) == ERR_SHAPE
    assert dm(window=0) == ERR_SHAPE
    assert dm(km=FAKE + 64) == ERR_ALIAS                                    # means inside k
    assert dm(vm=FAKE + 10**9 + 128) == ERR_ALIAS                           # the two means overlap


def test_transpose_validation(lib):
    tr = lambda idx=FAKE, cnt=FAKE + 10**9, H=2, tq=8, tk=8, kmax=4, te=FAKE + 2 * 10**9, tl=FAKE + 3 * 10**9: \
        lib.sparse3d_selection_transpose(idx, cnt, H, tq, tk, kmax, te, tl, NULL)
    assert tr(cnt=NULL) == ERR_NULL
    assert tr(te=NULL) == ERR_NULL
    assert tr(tl=NULL) == ERR_NULL
    assert tr(kmax=-1) == ERR_SHAPE
    assert tr(H=0) == ERR_SHAPE
    assert tr(tq=16385) == ERR_UNSUP
    assert tr(tl=FAKE + 64) == ERR_ALIAS                                  # list inside idx


def test_backward_validation(lib):
    ql = L()
    def bwd(q=FAKE, out=FAKE + 3 * 10**9, dout=FAKE + 4 * 10**9, lse=FAKE + 5 * 10**9, dt=1, kmax=8,
            dq=FAKE + 9 * 10**9, dk=FAKE + 10 * 10**9, dv=FAKE + 11 * 10**9, delta=FAKE + 12 * 10**9,
            scale=0.125, d=64, kbar=NULL, vbar=NULL, bias=math.log(64.0), dkbar=NULL, dvbar=NULL):
        return lib.sparse3d_sparse_attn_bwd(q, FAKE + 10**9, FAKE + 2 * 10**9, out, dout, lse, dt, 2, d, 64,
                                            ql, ql, FAKE + 6 * 10**9, FAKE + 7 * 10**9, kmax,
                                            FAKE + 8 * 10**9, FAKE + 13 * 10**9, kbar, vbar, bias, scale,
                                            dq, dk, dv, delta, dkbar, dvbar, NULL)
    assert bwd(out=NULL) == ERR_NULL
    assert bwd(lse=NULL) == ERR_NULL
    assert bwd(delta=NULL) == ERR_NULL
    assert bwd(dt=0) == ERR_UNSUP                                          # fp32 operands
    assert bwd(d=32) == ERR_UNSUP
    assert bwd(scale=0.0) == ERR_UNSUP
    assert bwd(dq=FAKE + 64) == ERR_ALIAS                                  # dq inside q
    assert bwd(dk=FAKE + 9 * 10**9 + 64) == ERR_ALIAS                     # dk inside dq
    assert bwd(delta=FAKE + 5 * 10**9 + 4) == ERR_ALIAS                   # delta inside lse
    assert bwd(kmax=8001) == ERR_UNSUP
    # landmarks: means in, their gradients out
    lm = dict(kbar=FAKE + 14 * 10**9, vbar=FAKE + 15 * 10**9, dkbar=FAKE + 16 * 10**9, dvbar=FAKE + 17 * 10**9)
    # a call that passed every check would launch on these fake addresses: the cases that
    # must get past a check end on the aliasing test, which comes last
    late = dict(delta=FAKE + 5 * 10**9 + 4)                                # delta inside lse
    assert bwd(**lm, **late) == ERR_ALIAS
    assert bwd(**{**lm, "vbar": NULL}) == ERR_NULL                         # kbar without vbar
    assert bwd(**{**lm, "dkbar": NULL}) == ERR_NULL                        # no room for the gradients
    assert bwd(**{**lm, "dvbar": NULL}) == ERR_NULL
    assert bwd(**{**lm, "bias": math.inf}) == ERR_UNSUP
    assert bwd(bias=math.inf, **late) == ERR_ALIAS                         # no landmarks: bias unused
    assert bwd(**{**lm, "kmax": 7801}) == ERR_UNSUP                        # list + bitmap exceed LDS
    assert bwd(**{**lm, "kmax": 7800}, **late) == ERR_ALIAS
    assert bwd(**{**lm, "dkbar": FAKE + 14 * 10**9 + 128}) == ERR_ALIAS   # dkbar inside kbar
    assert bwd(**{**lm, "dvbar": FAKE + 16 * 10**9 + 4}) == ERR_ALIAS     # dvbar inside dkbar
    assert bwd(**{**lm, "dk": FAKE + 17 * 10**9}) == ERR_ALIAS            # dk on dvbar
    assert bwd(**{**lm, "dq": FAKE + 15 * 10**9}) == ERR_ALIAS            # dq on vbar


def test_cast_validation(lib):
    cast = lib.sparse3d_cast
    assert cast(FAKE, -1, 1, FAKE + 10**9, NULL) == ERR_SHAPE
    assert cast(FAKE, 16, 5, FAKE + 10**9, NULL) == ERR_UNSUP
    assert cast(NULL, 16, 1, FAKE + 10**9, NULL) == ERR_NULL
    assert cast(FAKE, 16, 1, NULL, NULL) == ERR_NULL
    assert cast(FAKE, 16, 1, FAKE + 32, NULL) == ERR_ALIAS              # dst inside src
    assert cast(NULL, 0, 1, NULL, NULL) == OK                          # nothing to do, no launch


def test_subsample_layout_host_only(lib):
    out = S._Layout()
    lay = S._Layout(256, 1374, 1408, 5)
    assert lib.sparse3d_subsample_layout(ctypes.byref(lay), 37, 37, 2, 64, ctypes.byref(out)) == OK
    assert (out.frames, out.tokens, out.stride, out.specials) == (256, 366, 384, 5)
    assert lib.sparse3d_subsample_layout(ctypes.byref(lay), 37, 37, 3, 64, ctypes.byref(out)) == OK
    assert (out.tokens, out.stride) == (5 + 13 * 13, 192)
    assert lib.sparse3d_subsample_layout(ctypes.byref(lay), 36, 37, 2, 64, ctypes.byref(out)) == ERR_SHAPE
    assert lib.sparse3d_subsample_layout(ctypes.byref(lay), 37, 37, 0, 64, ctypes.byref(out)) == ERR_SHAPE
    assert lib.sparse3d_subsample_layout(NULL, 37, 37, 2, 64, ctypes.byref(out)) == ERR_NULL
    bad = S._Layout(256, 366, 384, 5)
    assert lib.sparse3d_grid_subsample_kv(FAKE, FAKE + 10**10, 1, 16, 64, ctypes.byref(lay), 37, 37, 2,
                                          FAKE + 2 * 10**10, FAKE + 3 * 10**10, ctypes.byref(S._Layout(256, 366, 448, 5)),
                                          NULL) == ERR_SHAPE
    assert lib.sparse3d_grid_subsample_kv(FAKE, FAKE + 10**10, 1, 16, 64, ctypes.byref(lay), 37, 37, 2,
                                          FAKE + 64, FAKE + 3 * 10**10, ctypes.byref(bad), NULL) == ERR_ALIAS


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 256, 64)
    with pytest.raises(ValueError):
        S.sparse3d_tile_scores(x, x, (2, 256, 256, 0))


def test_size_caps_of_the_kernels(lib):
    # score matrix: 64 score rows per wave are addressed with 32-bit offsets, so key tiles
    # are capped at 2^23; query tiles at 65535 grid rows of 128
    big_k = L(f=131072, n=64, p=8192)                     # 2^24 key tiles
    assert scores_call(lib, ql=L(f=131072, n=64, p=64), kl=big_k) == ERR_UNSUP
    assert scores_call(lib, ql=L(f=131072, n=64, p=4096), kl=L(f=131072, n=64, p=64)) == ERR_UNSUP
    # attention: one head of K/V (or Q) must stay below 2^24 rows of 128 bytes
    wide = L(f=2, n=256, p=(1 << 23) + 64)                # 2^24 + 128 rows
    dense = lambda ql, kl: lib.sparse3d_dense_attn_fwd(FAKE, FAKE + 10**10, FAKE + 2 * 10**10, 1, 2, 64, ql,
                                                       kl, 0.125, NULL, FAKE + 3 * 10**10, 1, NULL, NULL)
    frame = lambda ql, kl: lib.sparse3d_frame_attn_fwd(FAKE, FAKE + 10**10, FAKE + 2 * 10**10, 1, 2, 64, ql,
                                                       kl, 0.125, FAKE + 3 * 10**10, 1, NULL, NULL)
    assert dense(L(), wide) == ERR_UNSUP
    assert dense(wide, L()) == ERR_UNSUP
    assert frame(L(), wide) == ERR_UNSUP
    ok = L(f=2, n=256, p=1 << 23)                          # exactly 2^24 rows: allowed
    assert dense(L(), ok) != ERR_UNSUP


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def test_binding_checks_shapes_and_dtypes_before_the_device():
    """Every wrapper compares its tensors with the layouts and sizes before it touches the
    device: a too-short operand, a dtype mismatch or an int64 index table raises here, with
    CPU tensors, long before a kernel could read past an allocation."""
    import torch
    lay = (2, 256, 256, 0)
    q = _cpu(2, 512, 64)
    with pytest.raises(ValueError, match="shape"):
        S.sparse3d_tile_scores(q, _cpu(2, 448, 64), lay)                  # k shorter than its layout
    with pytest.raises(ValueError, match="shape"):
        S.sparse3d_tile_scores(_cpu(2, 512, 32), _cpu(2, 512, 32), lay)   # head_dim 32
    with pytest.raises(TypeError, match="dtype"):
        S.sparse3d_tile_scores(q, _cpu(2, 512, 64, dtype=torch.float32), lay)
    with pytest.raises(TypeError, match="dtype"):
        S.sparse3d_tile_scores(_cpu(2, 512, 64, dtype=torch.float16), _cpu(2, 512, 64, dtype=torch.float16), lay)
    with pytest.raises(TypeError, match="dtype"):
        S.sparse3d_select_topk(_cpu(2, 8, 8), 4, 4)                          # bf16 scores
    idx, cnt = _cpu(2, 8, 8, dtype=torch.int32), _cpu(2, 8, dtype=torch.int32)
    attn = lambda **kw: S.sparse3d_sparse_attn_fwd(kw.get("q", q), kw.get("k", q), kw.get("v", q), lay, lay,
                                                    kw.get("idx", idx), kw.get("cnt", cnt),
                                                    kbar=kw.get("kbar"), vbar=kw.get("vbar"),
                                                    out_dtype=kw.get("out_dtype"))
    with pytest.raises(TypeError, match="idx"):
        attn(idx=_cpu(2, 8, 8, dtype=torch.int64))
    with pytest.raises(TypeError, match="cnt"):
        attn(cnt=_cpu(2, 8, dtype=torch.int64))
    with pytest.raises(ValueError, match="cnt"):
        attn(cnt=_cpu(2, 7, dtype=torch.int32))
    with pytest.raises(ValueError, match="idx"):
        attn(idx=_cpu(3, 8, 8, dtype=torch.int32))
    with pytest.raises(ValueError, match="v has shape"):
        attn(v=_cpu(2, 256, 64))
    with pytest.raises(TypeError, match="v has dtype"):
        attn(v=_cpu(2, 512, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="kbar"):
        attn(kbar=_cpu(2, 7, 64), vbar=_cpu(2, 8, 64))
    with pytest.raises(TypeError, match="kbar"):
        attn(kbar=_cpu(2, 8, 64, dtype=torch.float32), vbar=_cpu(2, 8, 64, dtype=torch.float32))
    with pytest.raises(TypeError, match="out_dtype"):
        attn(out_dtype=torch.float16)
    with pytest.raises(ValueError, match="device"):
        attn()                                                              # right shapes, host memory
    with pytest.raises(ValueError, match="shape"):
        S.sparse3d_dense_attn_fwd(q, _cpu(2, 500, 64), q, lay)
    with pytest.raises(ValueError, match="shape"):
        S.sparse3d_frame_attn_fwd(q, q, _cpu(1, 512, 64), lay)
    with pytest.raises(TypeError, match="cnt"):
        S.sparse3d_selection_transpose(idx, _cpu(2, 8, dtype=torch.int64), 8)
    bwd = lambda **kw: S.sparse3d_sparse_attn_bwd(q, q, q, kw.get("out", q), kw.get("dout", q),
                                                  kw.get("lse", _cpu(2, 512, dtype=torch.float32)), lay, lay,
                                                  idx, cnt, kw.get("t_end", _cpu(2, 8, dtype=torch.int32)),
                                                  kw.get("t_list", _cpu(2, 64, dtype=torch.int32)))
    with pytest.raises(ValueError, match="lse"):
        bwd(lse=_cpu(2, 511, dtype=torch.float32))
    with pytest.raises(TypeError, match="dout"):
        bwd(dout=_cpu(2, 512, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="t_list"):
        bwd(t_list=_cpu(2, 63, dtype=torch.int32))
    with pytest.raises(ValueError, match="device"):
        bwd()
    with pytest.raises(ValueError, match="kbar and vbar"):
        S.sparse3d_sparse_attn_bwd(q, q, q, q, q, _cpu(2, 512, dtype=torch.float32), lay, lay, idx, cnt,
                                   _cpu(2, 8, dtype=torch.int32), _cpu(2, 64, dtype=torch.int32),
                                   kbar=_cpu(2, 8, 64))
    with pytest.raises(TypeError, match="vbar"):
        S.sparse3d_sparse_attn_bwd(q, q, q, q, q, _cpu(2, 512, dtype=torch.float32), lay, lay, idx, cnt,
                                   _cpu(2, 8, dtype=torch.int32), _cpu(2, 64, dtype=torch.int32),
                                   kbar=_cpu(2, 8, 64), vbar=_cpu(2, 8, 64, dtype=torch.float32))
    sga = S.Sga((16, 16), 2, kmean=_cpu(2, 63, dtype=torch.float32), vmean=_cpu(2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="kmean"):
        S.sparse3d_dense_attn_fwd(q, q, q, lay, sga=sga)
    with pytest.raises(TypeError):
        S.sparse3d_cast(_cpu(4, dtype=torch.float32), torch.float16)


def test_validation_under_sanitizers(tmp_path):
    """The host-side checks (plain C++, no HIP) built with AddressSanitizer and
    UndefinedBehaviorSanitizer and driven over sweeps of extreme, null and aliased
    arguments: no undefined behaviour, no memory error, a status code for every call."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++ on this machine")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "dynamic_block_sparse_tile_amd", "csrc")
    exe = str(tmp_path / "sanitize_validate")
    build = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                            "-I", os.path.join(root, "include"), "-I", csrc,
                            os.path.join(root, "tests", "sanitize_validate.cpp"),
                            os.path.join(csrc, "validate.cpp"), "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    # the sanitizer runtime need not come first among preloaded libraries
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-1000:], run.stderr[-3000:])
    assert "outside the status codes 0, well-formed accepted 4 of 4" in run.stdout
