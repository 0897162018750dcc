"""The C ABI library loads, exports every declared entry point, and rejects bad arguments on
the host before any launch (these calls never reach the GPU, so they run on CPU)."""
import ctypes

import pytest

import sparse_moe_expert_top_amd as moe
from sparse_moe_expert_top_amd import _lib

OK, ENULL, ESHAPE, EUNSUP, EWS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def test_every_declared_symbol_is_exported(lib):
    names = moe.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib._SIGS, f"binding lacks {n}"


def test_status_strings(lib):
    for s in range(7):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"
    assert lib.moe_version() >= 100
    assert lib.moe_last_hip_error() == 0


def _ws(which, **kw):
    out = ctypes.c_size_t(0)
    args = dict(T=0, E_loc=1, k=1, d=64, H=64, R_cap=0)
    args.update(kw)
    st = moe.load().moe_workspace_size(which, args["T"], args["E_loc"], args["k"], args["d"],
                                       args["H"], args["R_cap"], ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    assert _ws(_lib.MOE_WS_SITU_GLU_FWD, T=10) == (OK, 0)
    assert _ws(_lib.MOE_WS_SITU_GLU_BWD, T=10) == (OK, 0)
    st, b = _ws(_lib.MOE_WS_PERMUTE, T=1000, E_loc=28)
    assert st == OK and b >= 28 * 4 * 4 and b % 256 == 0
    st, b = _ws(_lib.MOE_WS_DOWN_COMBINE, d=3584, H=3072, R_cap=1000)
    assert st == OK and b >= 1000 * 3584 * 4                           # fp32 rows
    st, b = _ws(_lib.MOE_WS_EXPERT_BWD, d=3584, H=3072, R_cap=1000)
    assert st == OK and b >= 1000 * 6144 * 2 + 1000 * 3584 * 4
    assert _ws(_lib.MOE_WS_EXPERT_BWD, d=100, H=3072, R_cap=10)[0] == EUNSUP
    assert _ws(_lib.MOE_WS_PERMUTE, E_loc=0)[0] == ESHAPE
    assert _ws(77)[0] == ESHAPE
    assert moe.load().moe_workspace_size(1, 0, 1, 1, 64, 64, 0, None) == ENULL


def test_route_rejects(lib):
    P = ctypes.c_void_p(16)
    assert lib.moe_route_topk(P, -1, 8, 2, P, P, None) == ESHAPE
    assert lib.moe_route_topk(P, 4, 8, 9, P, P, None) == ESHAPE       # k > E
    assert lib.moe_route_topk(P, 4, 8, 0, P, P, None) == ESHAPE
    assert lib.moe_route_topk(P, 4, 2000, 2, P, P, None) == EUNSUP    # E > 1024
    assert lib.moe_route_topk(P, 4, 64, 33, P, P, None) == EUNSUP     # k > 32
    assert lib.moe_route_topk(None, 4, 8, 2, P, P, None) == ENULL
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == OK  # empty: nothing to do


def test_permute_rejects(lib):
    P = ctypes.c_void_p(256)
    args = [P, P, 16, 2, 0, 4, 32, P, P, P, P, P, P, 1 << 20, None]
    assert lib.moe_permute(*args[:5], 0, *args[6:]) == ESHAPE          # E_loc = 0
    a = list(args); a[4] = -1
    assert lib.moe_permute(*a) == ESHAPE
    a = list(args); a[13] = 0
    assert lib.moe_permute(*a) == EWS
    a = list(args); a[11] = None
    assert lib.moe_permute(*a) == ENULL                                # status flag
    a = list(args); a[3] = 40
    assert lib.moe_permute(*a) == EUNSUP                               # k > 32


def test_gemm_and_situ_reject(lib):
    P = ctypes.c_void_p(256)
    U = ctypes.c_void_p(258)                                           # not 16-byte aligned
    gu = lib.moe_grouped_gemm_gate_up
    assert gu(P, 50, P, P, 4, 100, 100, 64, P, 4.0, 25.0, P, P, None) == EUNSUP
    assert gu(P, 50, P, P, 4, 100, 128, 64, P, 4.0, 25.0, U, P, None) == EUNSUP
    assert gu(P, 50, P, None, 4, 100, 128, 64, P, 4.0, 25.0, P, P, None) == ENULL
    assert gu(P, 50, P, P, 4, 100, 128, 64, P, -1.0, 25.0, P, P, None) == ESHAPE
    assert gu(P, -1, P, P, 4, 100, 128, 64, P, 4.0, 25.0, P, P, None) == ESHAPE
    assert lib.situ_glu_fwd(P, 10, 12, 4.0, 25.0, P, None, 0, None) == EUNSUP     # H % 8
    assert lib.situ_glu_fwd(None, 10, 16, 4.0, 25.0, P, None, 0, None) == ENULL
    assert lib.situ_glu_bwd(P, P, -5, 16, 4.0, 25.0, P, None, 0, None) == ESHAPE
    assert lib.situ_glu_fwd(None, 0, 16, 4.0, 25.0, None, None, 0, None) == OK
    assert lib.moe_unpermute(P, P, None, 4, 2, 12, P, None) == EUNSUP             # n % 8
    assert lib.moe_grouped_gemm_down_combine(P, P, P, P, 8, 2, 4, 16, 64, 128, P, P, P, 0, None) == EWS
    assert lib.moe_router_bwd(None, P, 4, 2, P, None) == ENULL


def test_expert_bwd_rejects(lib):
    P = ctypes.c_void_p(256)
    base = [P, P, P, P, P, P, P, 8, 2, 4, 16, 128, 64, P, P, 4.0, 25.0, P, P, P, P, P, 1 << 30, None]
    a = list(base); a[22] = 10
    assert lib.moe_expert_bwd(*a) == EWS
    a = list(base); a[11] = 96
    assert lib.moe_expert_bwd(*a) == EUNSUP
    a = list(base); a[13] = None
    assert lib.moe_expert_bwd(*a) == ENULL
    a = list(base); a[8] = 0
    assert lib.moe_expert_bwd(*a) == ESHAPE


def test_mxfp8_entry_points_reject(lib):
    P = ctypes.c_void_p(256)
    U = ctypes.c_void_p(264)                                           # 8- but not 16-byte aligned
    # standalone quantizer / dequantizer
    assert lib.moe_mxfp8_quantize(P, 10, 48, P, P, None) == EUNSUP    # n % 32
    assert lib.moe_mxfp8_quantize(P, -1, 64, P, P, None) == ESHAPE
    assert lib.moe_mxfp8_quantize(P, 10, 64, P, None, None) == ENULL
    assert lib.moe_mxfp8_quantize(P, 10, 64, U, P, None) == EUNSUP    # codes alignment
    assert lib.moe_mxfp8_quantize(None, 0, 64, None, None, None) == OK
    assert lib.moe_mxfp8_dequantize(P, P, 10, 40, P, None) == EUNSUP
    assert lib.moe_mxfp8_dequantize(P, None, 10, 64, P, None) == ENULL
    assert lib.moe_mxfp8_dequantize(P, P, 0, 64, None, None) == OK
    # gate/up writing MXFP8 h
    gu = lib.moe_grouped_gemm_gate_up_mx
    assert gu(P, 50, P, P, 4, 100, 100, 64, P, 4.0, 25.0, P, P, P, None) == EUNSUP   # d % 64
    assert gu(P, 50, P, P, 4, 100, 128, 64, P, 4.0, 25.0, P, None, P, None) == ENULL # scales
    assert gu(P, 50, P, P, 4, 100, 128, 64, P, 4.0, 25.0, U, P, P, None) == EUNSUP   # codes alignment
    assert gu(P, 50, P, P, 4, 100, 128, 64, P, 4.0, 0.0, P, P, P, None) == ESHAPE    # linear_beta
    assert gu(P, 50, None, P, 4, 0, 128, 64, P, 4.0, 25.0, None, None, None, None) == OK   # R_cap = 0
    assert gu(P, 1 << 24, P, P, 4, 100, 128, 64, P, 4.0, 25.0, P, P, P, None) == EUNSUP  # T rows
    # backward reading MXFP8 h
    base = [P, P, P, P, P, P, P, P, 8, 2, 4, 16, 128, 64, P, P, 4.0, 25.0, P, P, P, P, P,
            1 << 30, None]
    bw = lib.moe_expert_bwd_mx
    a = list(base); a[23] = 10
    assert bw(*a) == EWS
    a = list(base); a[3] = None                                        # h_scales
    assert bw(*a) == ENULL
    a = list(base); a[12] = 96
    assert bw(*a) == EUNSUP
    a = list(base); a[9] = 0
    assert bw(*a) == ESHAPE


def test_w4a8_entry_points_reject(lib):
    """Host-side validation of the MXFP4 codec and the W4A8 GEMMs (nothing is launched)."""
    P = ctypes.c_void_p(256)
    U16 = ctypes.c_void_p(264)                                         # 8- but not 16-byte aligned
    U4 = ctypes.c_void_p(258)                                          # not 4-byte aligned
    assert lib.moe_mxfp4_quantize(P, 10, 48, P, P, None) == EUNSUP    # n % 32
    assert lib.moe_mxfp4_quantize(P, -1, 64, P, P, None) == ESHAPE
    assert lib.moe_mxfp4_quantize(P, 10, 64, P, None, None) == ENULL
    assert lib.moe_mxfp4_quantize(U16, 10, 64, P, P, None) == EUNSUP  # v alignment
    assert lib.moe_mxfp4_quantize(P, 10, 64, U4, P, None) == EUNSUP   # codes alignment
    assert lib.moe_mxfp4_quantize(None, 0, 64, None, None, None) == OK
    assert lib.moe_mxfp4_dequantize(P, P, 10, 40, P, None) == EUNSUP
    assert lib.moe_mxfp4_dequantize(P, None, 10, 64, P, None) == ENULL
    assert lib.moe_mxfp4_dequantize(P, P, 0, 64, None, None) == OK
    gu = lib.moe_grouped_gemm_gate_up_w4a8
    #        xc xs  T    tok off E_loc R_cap d   H   wc ws beta  lbeta ac as stream
    ok = [P, P, 100, P, P, 4, 100, 256, 128, P, P, 4.0, 25.0, P, P, None]
    def g(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return gu(*a)
    assert g(a7=192) == EUNSUP                                         # d % 128
    assert g(a8=64) == EUNSUP                                          # H % 128
    assert g(a2=-1) == ESHAPE
    assert g(a2=1 << 25) == EUNSUP                                     # T * d >= 2^32
    assert g(a12=0.0) == ESHAPE                                        # linear_beta
    assert g(a10=None) == ENULL                                        # weight scales
    assert g(a14=None) == ENULL                                        # a scales
    assert g(a0=U16) == EUNSUP                                         # x codes alignment
    assert g(a1=U4) == EUNSUP                                          # x scales alignment
    assert g(a13=U16) == EUNSUP                                        # a codes alignment
    assert g(a6=0, a0=None, a1=None, a3=None, a13=None, a14=None) == OK   # R_cap = 0
    dn = lib.moe_grouped_gemm_down_combine_w4a8
    #          ac as off gate slot T   k  E_loc R_cap H    d   wc ws y  ws   bytes  stream
    okd = [P, P, P, P, P, 100, 2, 4, 100, 128, 256, P, P, P, P, 1 << 30, None]
    def dd(**kw):
        a = list(okd)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return dn(*a)
    assert dd(a9=192) == EUNSUP                                        # H % 128
    assert dd(a15=10) == EWS
    assert dd(a1=None) == ENULL
    assert dd(a12=None) == ENULL
    assert dd(a1=U4) == EUNSUP
    assert dd(a8=1 << 24, a9=1024) == EWS      # R_cap * H >= 2^32 is supported; ws too small
    assert dd(a6=0) == ESHAPE


def test_gate_up_rejects_token_rows_past_4gib(lib):
    """The gather addresses token rows with 32-bit byte offsets: T * max(d, 2H) * 2 >= 2^32 is
    refused before any launch (d = 128, H = 64: T = 2^24 is the first such T)."""
    P = ctypes.c_void_p(256)
    gu = lib.moe_grouped_gemm_gate_up
    assert gu(P, (1 << 24) - 1, P, P, 4, 0, 128, 64, P, 4.0, 25.0, P, P, None) == OK   # R_cap = 0
    assert gu(P, 1 << 24, P, P, 4, 100, 128, 64, P, 4.0, 25.0, P, P, None) == EUNSUP
    assert gu(P, 1 << 24, P, P, 4, 0, 128, 64, P, 4.0, 25.0, P, P, None) == EUNSUP
    # 2H decides when it exceeds d: d = 64, H = 1024 -> T = 2^20
    assert gu(P, 1 << 20, P, P, 4, 100, 64, 1024, P, 4.0, 25.0, P, P, None) == EUNSUP


def _wsp(which, passes, **kw):
    out = ctypes.c_size_t(0)
    args = dict(T=0, E_loc=1, k=1, d=64, H=64, R_cap=0)
    args.update(kw)
    st = moe.load().moe_workspace_size_passes(which, args["T"], args["E_loc"], args["k"],
                                              args["d"], args["H"], args["R_cap"], passes,
                                              ctypes.byref(out))
    return st, out.value


def test_workspace_size_passes():
    kw = dict(d=3584, H=3072, R_cap=1000)
    for which in (_lib.MOE_WS_DOWN_COMBINE, _lib.MOE_WS_EXPERT_BWD):
        assert _wsp(which, 1, **kw) == _ws(which, **kw)
        sizes = [_wsp(which, p, **kw)[1] for p in (1, 2, 3, 14, 100)]
        assert all(a >= b for a, b in zip(sizes, sizes[1:]))             # more passes, less memory
        assert sizes[-2] == sizes[-1]                                      # 256-column floor
    assert _wsp(_lib.MOE_WS_DOWN_COMBINE, 2, **kw)[1] == 1000 * 1792 * 4  # windows of 1792
    assert _wsp(_lib.MOE_WS_DOWN_COMBINE, 14, **kw)[1] == 1000 * 256 * 4
    assert _wsp(_lib.MOE_WS_DOWN_COMBINE, 0, **kw)[0] == ESHAPE
    assert _wsp(_lib.MOE_WS_PERMUTE, 1, **kw)[0] == ESHAPE
    assert _wsp(_lib.MOE_WS_DOWN_COMBINE, 2, d=100, H=64, R_cap=10)[0] == EUNSUP


def test_down_combine_accepts_any_window_workspace(lib):
    """A workspace below one window of 256 fp32 columns is refused; from there up every size
    is accepted (here with R_cap = 0 nothing is launched, so the null stream is never used)."""
    P = ctypes.c_void_p(256)
    dn = lib.moe_grouped_gemm_down_combine
    #            a  off gate slot T  k  E_loc R_cap H    d    w  y  ws bytes stream
    assert dn(P, P, P, P, 0, 2, 4, 16, 64, 512, P, P, P, 16 * 256 * 4 - 1, None) == EWS
    bw = lib.moe_expert_bwd
    st, need = _wsp(_lib.MOE_WS_EXPERT_BWD, 100, d=512, H=64, R_cap=16)
    base = [P, P, P, P, P, P, P, 0, 2, 4, 16, 512, 64, P, P, 4.0, 25.0, P, P, P, P, P, need - 1,
            None]
    assert bw(*base) == EWS


def test_wrappers_check_shapes_before_any_call():
    """The Python binding rejects buffers too small for the row capacity (or of the wrong
    shape) before it reaches the library, so an undersized buffer can never become an
    out-of-bounds device access; shape checks run before the device check (CPU tensors)."""
    import torch
    T, d, H, E_loc, k, R_cap = 8, 64, 64, 4, 2, 16
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    x = torch.zeros(T, d, dtype=bf)
    w_gu = torch.zeros(E_loc, 2 * H, d, dtype=bf)
    w_down = torch.zeros(E_loc, d, H, dtype=bf)
    off = torch.zeros(E_loc + 1, dtype=i32)
    tok = torch.zeros(R_cap, dtype=i32)
    perm = dict(offsets=off, row_token=tok, row_gate=torch.zeros(R_cap, dtype=f32),
                slot_row=torch.zeros(T, k, dtype=i32))
    h = torch.zeros(R_cap, 2 * H, dtype=bf)
    a = torch.zeros(R_cap, H, dtype=bf)

    def shape_err(fn, *args, **kw):
        with pytest.raises(ValueError, match="shape"):
            fn(*args, **kw)

    gu = _lib.moe_grouped_gemm_gate_up
    shape_err(gu, x[:, :32].contiguous(), tok, off, w_gu, R_cap, h=h, a=a)         # x (T, d)
    shape_err(gu, x, tok[:R_cap - 1].contiguous(), off, w_gu, R_cap, h=h, a=a)     # row_token
    shape_err(gu, x, tok, off, w_gu, R_cap, h=h[:R_cap - 1].contiguous(), a=a)     # h rows
    shape_err(gu, x, tok, off, w_gu, R_cap, h=h, a=a[:, :32].contiguous())         # a columns
    shape_err(gu, x, tok, off[:E_loc].contiguous(), w_gu, R_cap, h=h, a=a)         # offsets
    with pytest.raises(ValueError, match="GPU tensor"):
        gu(x, tok, off, w_gu, R_cap, h=h, a=a)                                      # shapes fine
    dn = _lib.moe_grouped_gemm_down_combine
    shape_err(dn, a[:R_cap - 1].contiguous(), off, perm["row_gate"], perm["slot_row"], w_down,
              R_cap)
    shape_err(dn, a, off, perm["row_gate"][:3].contiguous(), perm["slot_row"], w_down, R_cap)
    bw = _lib.moe_expert_bwd
    shape_err(bw, x, x, h[:R_cap - 1].contiguous(), perm, w_gu, w_down, R_cap)
    bad = dict(perm, row_token=tok[:4].contiguous())
    shape_err(bw, x, x, h, bad, w_gu, w_down, R_cap)
    shape_err(bw, x, x[:T - 1].contiguous(), h, perm, w_gu, w_down, R_cap)
    gmx = _lib.moe_grouped_gemm_gate_up_mx
    shape_err(gmx, x, tok, off, w_gu, R_cap,
              h_codes=torch.zeros(R_cap - 1, 2 * H, dtype=torch.uint8))


def test_expert_bwd_stages_rejects(lib):
    P = ctypes.c_void_p(256)
    #       dy x  h  hc hs tok gate slot off T  k  E_loc R_cap d   H   wgu wd beta lbeta
    base = [P, P, P, None, None, P, P, P, P, 8, 2, 4, 16, 128, 64, P, P, 4.0, 25.0,
            P, P, P, P, P, 1 << 30, 31, None]
    #       dx dwg dwd dp ws bytes stages stream
    def st(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.moe_expert_bwd_stages(*a)
    assert st(a25=0) == ESHAPE                                         # no stage
    assert st(a25=32) == ESHAPE                                        # unknown stage bit
    assert st(a3=P, a4=P) == ESHAPE                                    # both forms of h
    assert st(a2=None) == ENULL                                        # no form of h
    assert st(a2=None, a3=P) == ENULL                                  # codes without scales
    assert st(a24=10) == EWS
    assert st(a13=96) == EUNSUP


def test_noalloc_down_combine_rejects(lib):
    """The allocation-free down combine refuses more rows than its static scratch holds for one
    256-column window (65536 at d >= 256), and the usual bad arguments, before any launch."""
    P = ctypes.c_void_p(256)
    na = lib.moe_grouped_gemm_down_combine_noalloc
    #            a  off gate slot T  k  E_loc R_cap   H   d    w  y  stream
    assert na(P, P, P, P, 8, 2, 4, 65537, 64, 512, P, P, None) == EWS
    assert na(P, P, P, P, 8, 2, 4, 1 << 20, 64, 128, P, P, None) == EWS   # d < 256: 128 columns
    assert na(P, P, P, P, 8, 2, 4, -1, 64, 512, P, P, None) == ESHAPE
    assert na(P, P, P, P, 8, 2, 4, 0, 64, 100, P, P, None) == EUNSUP       # d % 64
    assert na(P, None, P, P, 8, 2, 4, 0, 64, 512, P, P, None) == ENULL     # offsets
    assert na(P, P, P, P, 8, 2, 4, 0, 64, 512, None, P, None) == ENULL     # w_down
