"""GPU parity: every libmoe.so entry point against the fp64 oracle (mode S).

Bars: integer outputs (indices, offsets, rows, slots) bit-exact; bf16 outputs and the fp32
weight gradients max|gpu - oracle| / max|oracle| <= 1e-2; fp32 gates and dp <= 2e-3.
Small shapes are compared in full; the full-size workloads (one expert-parallel rank,
skewed routing, large context) run in the benchmark's launch configuration and are compared
on sampled tokens, rows and weight-gradient columns, plus properties that hold at any size.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import LAYER_CONFIGS, LayerConfig, SITU_CONFIGS, layer_inputs, situ_inputs
from tests._helpers import rel_err, BF16_TOL, FP32_TOL, sub_perm, oracle_route_perm

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    import sparse_moe_expert_top_amd as m
    m.load()
    return m


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16(t):
    return oracle.bf16_widen(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def layer_shape(m, cfg, T=None):
    return m.LayerShape(T=cfg.T if T is None else T, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo,
                        E_loc=cfg.E_loc, d=cfg.d, H=cfg.H, beta=cfg.beta,
                        linear_beta=cfg.linear_beta)


def run_layer(m, cfg, inp, R_cap=None, h_store="bf16", **buf_kw):
    """Forward + backward through LayerBuffers (the benchmark's launch configuration). The
    forward's activation `a` shares memory with the backward workspace, so a copy taken after
    the forward is kept as buf.a_fwd."""
    buf = m.LayerBuffers(layer_shape(m, cfg, inp["x"].shape[0]), R_cap=R_cap, h_store=h_store,
                         **buf_kw)
    t = dict(x=dev_bf16(inp["x"]), logits=dev(inp["logits"]), w_gu=dev_bf16(inp["w_gu"]),
             w_down=dev_bf16(inp["w_down"]), dy=dev_bf16(inp["dy"]))
    buf.forward(t["x"], t["logits"], t["w_gu"], t["w_down"])
    buf.a_fwd = buf.a.clone()
    if buf.combine_passes == 1:
        buf.rows_fwd = rows_f32(buf, cfg.d)
    buf.backward(t["dy"], t["x"], t["w_gu"], t["w_down"])
    torch.cuda.synchronize()
    return buf, t


def bf16_half_step(v):
    """Half the spacing of the bf16 grid at |v| (8 significant bits; 2^-134 below 2^-126)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def rows_f32(buf, n):
    """The fp32 rows the down GEMM left in the combine's workspace (one pass: [R_cap, n])."""
    R = buf.R_cap
    return buf.ws_down[: R * n * 4].view(torch.float32).view(R, n).cpu().numpy().astype(np.float64)


def check_rounded_once(y, rows, slot_row, what):
    """The combine rounds each output once: y[t] is the bf16 rounding (nearest, ties to even)
    of the fp32 sum of the token's fp32 rows in slot order. The exact sum S of those rows (fp64
    here) and the fp32 sum differ by at most (k - 1) 2^-24 sum|rows|, so y must lie within half
    a bf16 step of S plus that; rows rounded to bf16 before the sum would miss it by up to k
    half steps of the terms. Also checks that the rows are not bf16 values themselves."""
    T, k = slot_row.shape
    S = np.zeros_like(y)
    M = np.zeros_like(y)
    for j in range(k):
        r = slot_row[:, j]
        m = r >= 0
        S[m] += rows[r[m]]
        M[m] += np.abs(rows[r[m]])
    bound = bf16_half_step(S) + (k - 1) * 2.0 ** -24 * M + 2.0 ** -149
    err = np.abs(y - S)
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:3])
    used = np.unique(slot_row[slot_row >= 0])
    if len(used):
        low = rows[used].astype(np.float32).view(np.uint32) & 0xFFFF
        assert np.mean(low != 0) > 0.9, (what, "rows look bf16-rounded")


def rel_to_sum(got, exact):
    """max|got - exact| / max|exact|: against the oracle's fp64 sum before its final rounding
    (reported; half a bf16 step at the top of the range is 2^-8 = 3.9e-3 of the maximum)."""
    m = float(np.max(np.abs(exact))) if exact.size else 0.0
    return 0.0 if m == 0.0 else float(np.max(np.abs(np.asarray(got, np.float64) - exact)) / m)


def check_route_perm(buf, idx, gates, perm, R_cap=None):
    assert np.array_equal(buf.topk_idx.cpu().numpy(), idx)
    assert rel_err(buf.gates.cpu().numpy(), gates) <= FP32_TOL
    R = perm["R"]
    off = buf.perm["offsets"].cpu().numpy()
    assert np.array_equal(off, perm["offsets"])
    assert np.array_equal(buf.perm["row_token"][:R].cpu().numpy(), perm["row_token"])
    assert np.array_equal(buf.perm["slot_row"].cpu().numpy(), perm["slot_row"])
    # row_gate is the GPU's own gate of that route, bit for bit
    g_gpu = buf.gates.cpu().numpy()
    sr = perm["slot_row"]
    t, j = np.nonzero(sr >= 0)
    assert np.array_equal(buf.perm["row_gate"][:R].cpu().numpy()[sr[t, j]], g_gpu[t, j])
    assert int(buf.perm["status"].item()) == 0


# ------------------------------------------------------------------------------- SiTU-GLU
@pytest.mark.parametrize("R,H,rows_per_launch", [(1000, 192, 0), (37, 64, 0), (1, 8, 0),
                                                 (1000, 192, 300), (1000, 192, 1)])
def test_situ_glu_small(moe, R, H, rows_per_launch):
    """rows_per_launch > 0 caps the rows of one launch (MOE_SITU_ROWS_PER_LAUNCH), so the
    split across launches that very large inputs take (below 2^32 chunks each) is exercised:
    4 launches of 300, 300, 300 and 100 rows, or one launch per row."""
    say(f"situ_glu R={R} H={H} rows_per_launch={rows_per_launch}")
    inp = situ_inputs(R, H, seed=3)
    h = dev_bf16(inp["h"])
    da = dev_bf16(inp["da"])
    if rows_per_launch:
        os.environ["MOE_SITU_ROWS_PER_LAUNCH"] = str(rows_per_launch)
    try:
        a = moe.situ_glu_fwd(h)
        dh = moe.situ_glu_bwd(h, da)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("MOE_SITU_ROWS_PER_LAUNCH", None)
    hf = oracle.bf16_widen(inp["h"])
    ref_a = oracle.bf16_round(oracle.situ_glu_fwd(hf, H))
    ref_dh = oracle.bf16_round(oracle.situ_glu_bwd(hf, oracle.bf16_widen(inp["da"]), H))
    assert rel_err(host_bf16(a), ref_a) <= BF16_TOL
    assert rel_err(host_bf16(dh), ref_dh) <= BF16_TOL


def test_situ_glu_extremes(moe):
    """Saturated and special inputs stay finite and match the oracle's limits."""
    H = 8
    g = np.array([0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 200.0, -200.0, 3e38, -3e38, 0.5, -1.2188,
                  4.0, -4.0, 30.0, -30.0], np.float32)
    l = np.array([0.0, 1.0, -1.0, 1e4, -1e4, 3e38, -3e38, 25.0, 0.5, -0.5, 100.0, 2.0, -60.0,
                  60.0, 1e-20, 7.0], np.float32)
    from moe_inputs import f32_to_bf16_bits
    hb = f32_to_bf16_bits(np.concatenate([g.reshape(2, 8), l.reshape(2, 8)], axis=1))
    da = f32_to_bf16_bits(np.ones((2, 8), np.float32))
    a = moe.situ_glu_fwd(dev_bf16(hb))
    dh = moe.situ_glu_bwd(dev_bf16(hb), dev_bf16(da))
    torch.cuda.synchronize()
    ga, gdh = host_bf16(a), host_bf16(dh)
    assert np.all(np.isfinite(ga)) and np.all(np.isfinite(gdh))
    hf = oracle.bf16_widen(hb)
    ref_a = oracle.bf16_round(oracle.situ_glu_fwd(hf, H))
    ref_dh = oracle.bf16_round(oracle.situ_glu_bwd(hf, oracle.bf16_widen(da), H))
    np.testing.assert_allclose(ga, ref_a, rtol=1e-2, atol=1e-35)   # fp32 denormals may flush
    np.testing.assert_allclose(gdh, ref_dh, rtol=1e-2, atol=1e-6)


@pytest.mark.parametrize("beta,linear_beta", [(3.0, 10.0), (1.0, 1.0), (7.5, 40.0)])
def test_situ_glu_other_coefficients(moe, beta, linear_beta):
    """beta != 4 takes the kernels' other path (exp(-|g|) evaluated on its own rather than as
    the square of exp(-|g|/2)), and every coefficient enters the scaled terms: random rows and
    the saturated and special inputs against the oracle at the same coefficients."""
    say(f"situ_glu beta={beta} linear_beta={linear_beta}")
    inp = situ_inputs(1000, 192, seed=5)
    h, da = dev_bf16(inp["h"]), dev_bf16(inp["da"])
    a = moe.situ_glu_fwd(h, beta=beta, linear_beta=linear_beta)
    dh = moe.situ_glu_bwd(h, da, beta=beta, linear_beta=linear_beta)
    torch.cuda.synchronize()
    hf = oracle.bf16_widen(inp["h"])
    ref_a = oracle.bf16_round(oracle.situ_glu_fwd(hf, 192, beta, linear_beta))
    ref_dh = oracle.bf16_round(oracle.situ_glu_bwd(hf, oracle.bf16_widen(inp["da"]), 192, beta,
                                                   linear_beta))
    assert rel_err(host_bf16(a), ref_a) <= BF16_TOL
    assert rel_err(host_bf16(dh), ref_dh) <= BF16_TOL
    from moe_inputs import f32_to_bf16_bits
    g = np.array([0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 200.0, -200.0, 3e38, -3e38, 0.5, -1.2188,
                  4.0, -4.0, 30.0, -30.0], np.float32)
    l = np.array([0.0, 1.0, -1.0, 1e4, -1e4, 3e38, -3e38, 25.0, 0.5, -0.5, 100.0, 2.0, -60.0,
                  60.0, 1e-20, 7.0], np.float32)
    hb = f32_to_bf16_bits(np.concatenate([g.reshape(2, 8), l.reshape(2, 8)], axis=1))
    db = f32_to_bf16_bits(np.ones((2, 8), np.float32))
    a = moe.situ_glu_fwd(dev_bf16(hb), beta=beta, linear_beta=linear_beta)
    dh = moe.situ_glu_bwd(dev_bf16(hb), dev_bf16(db), beta=beta, linear_beta=linear_beta)
    torch.cuda.synchronize()
    ga, gdh = host_bf16(a), host_bf16(dh)
    assert np.all(np.isfinite(ga)) and np.all(np.isfinite(gdh))
    hf = oracle.bf16_widen(hb)
    np.testing.assert_allclose(ga, oracle.bf16_round(oracle.situ_glu_fwd(hf, 8, beta, linear_beta)),
                               rtol=1e-2, atol=1e-35)
    np.testing.assert_allclose(
        gdh, oracle.bf16_round(oracle.situ_glu_bwd(hf, oracle.bf16_widen(db), 8, beta, linear_beta)),
        rtol=1e-2, atol=1e-6)


def test_situ_glu_full_size_sampled(moe):
    """h bf16 [131072, 6144] ~ N(0, 9), da [131072, 3072]: the streaming configuration; the
    oracle checks 4096 sampled rows."""
    cfg = SITU_CONFIGS["situ"]
    R, H = cfg["R"], cfg["H"]
    say(f"situ_glu full R={R} H={H}")
    inp = situ_inputs(R, H, seed=0, h_std=cfg["h_std"])
    h = dev_bf16(inp["h"])
    da = dev_bf16(inp["da"])
    a = moe.situ_glu_fwd(h)
    dh = moe.situ_glu_bwd(h, da)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(R, 4096, replace=False))
    rows = np.concatenate([rows, [0, R - 1]])
    hf = oracle.bf16_widen(inp["h"][rows])
    ref_a = oracle.bf16_round(oracle.situ_glu_fwd(hf, H))
    ref_dh = oracle.bf16_round(oracle.situ_glu_bwd(hf, oracle.bf16_widen(inp["da"][rows]), H))
    ridx = torch.from_numpy(rows).cuda()
    assert rel_err(host_bf16(a[ridx]), ref_a) <= BF16_TOL
    assert rel_err(host_bf16(dh[ridx]), ref_dh) <= BF16_TOL
    assert bool(torch.isfinite(a.float()).all()) and bool(torch.isfinite(dh.float()).all())


# ------------------------------------------------------------------------------- routing
@pytest.mark.parametrize("name", ["tiny", "shard", "skew", "large"])
def test_route_and_permute(moe, name):
    cfg = LAYER_CONFIGS[name]
    say(f"route/permute {name}")
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.bias:
        from moe_inputs import zipf_bias
        logits += zipf_bias(cfg.E)[None, :]
    idx, gates = oracle.route_topk(logits, cfg.k)
    g_idx, g_gates = moe.moe_route_topk(dev(logits), cfg.k)
    assert np.array_equal(g_idx.cpu().numpy(), idx)
    assert rel_err(g_gates.cpu().numpy(), gates) <= FP32_TOL
    assert float((g_gates.sum(1) - 1).abs().max()) <= 1e-5
    perm = oracle.permute(idx, gates, cfg.e_lo, cfg.E_loc)
    R_cap = cfg.T * cfg.k
    out = moe.moe_permute(g_idx, g_gates, cfg.e_lo, cfg.E_loc, R_cap)
    torch.cuda.synchronize()
    assert np.array_equal(out["offsets"].cpu().numpy(), perm["offsets"])
    assert np.array_equal(out["row_token"][:perm["R"]].cpu().numpy(), perm["row_token"])
    assert np.array_equal(out["slot_row"].cpu().numpy(), perm["slot_row"])
    assert int(out["status"].item()) == 0


def test_route_ties(moe):
    """Equal logits (and -0.0 vs +0.0) resolve to the lower expert index."""
    rng = np.random.default_rng(5)
    L = rng.integers(-2, 3, size=(513, 130)).astype(np.float32)
    L[0] = 0.0
    L[1, ::2] = -0.0
    for k in (1, 7, 32):
        idx, gates = oracle.route_topk(L, k)
        g_idx, g_gates = moe.moe_route_topk(dev(L), k)
        assert np.array_equal(g_idx.cpu().numpy(), idx)
        assert rel_err(g_gates.cpu().numpy(), gates) <= FP32_TOL


@pytest.mark.parametrize("T,E,k", [(1000, 1024, 32), (777, 1000, 16), (300, 65, 1), (300, 64, 32),
                                   (500, 100, 32), (257, 896, 16), (129, 33, 33 - 1),
                                   # E <= 32: one lane per token
                                   (600, 28, 16), (300, 32, 32), (257, 1, 1), (300, 7, 3),
                                   (300, 17, 17), (100, 16, 8), (70, 9, 9), (1000, 8, 2)])
def test_route_shapes(moe, T, E, k):
    """Envelope edges of the router: E not a multiple of 64, E = 1024, k = 1 and k = 32, and
    rows that force the many-ties path (all equal; few distinct levels), next to rows with
    extreme but finite values, signed zeros and subnormals."""
    say(f"route T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 7 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[0] = 1.5                                                  # every logit equal
    L[1] = rng.integers(0, 3, size=E).astype(np.float32)        # three levels: >64 ties at the cut
    L[2, ::3] = -0.0
    L[2, 1::3] = 0.0
    L[3] = rng.choice(np.array([-3e38, 3e38, 1e-40, -1e-40, 0.0], np.float32), size=E)
    L[4] = np.arange(E, dtype=np.float32)[::-1] * 1e-3          # strictly decreasing by index
    idx, gates = oracle.route_topk(L, k)
    g_idx, g_gates = moe.moe_route_topk(dev(L), k)
    assert np.array_equal(g_idx.cpu().numpy(), idx)
    assert rel_err(g_gates.cpu().numpy(), gates) <= FP32_TOL
    assert float((g_gates.sum(1) - 1).abs().max()) <= 1e-5


def test_permute_capacity_overflow(moe):
    """R_cap below the routed rows: flag raised, offsets clamped, dropped routes get -1."""
    cfg = LAYER_CONFIGS["tiny"]
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    idx, gates = oracle.route_topk(logits, cfg.k)
    perm = oracle.permute(idx, gates, 0, cfg.E_loc)
    R_cap = perm["R"] - 100
    g_idx, g_gates = moe.moe_route_topk(dev(logits), cfg.k)
    out = moe.moe_permute(g_idx, g_gates, 0, cfg.E_loc, R_cap)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 1
    assert np.array_equal(out["offsets"].cpu().numpy(), np.minimum(perm["offsets"], R_cap))
    sr = out["slot_row"].cpu().numpy()
    ref = np.where(perm["slot_row"] < R_cap, perm["slot_row"], -1)
    assert np.array_equal(sr, ref)
    assert np.array_equal(out["row_token"][:R_cap].cpu().numpy(), perm["row_token"][:R_cap])


@pytest.mark.parametrize("T,k,n", [(50, 5, 64), (40, 32, 3584), (3, 1, 8), (17, 9, 136)])
def test_unpermute(moe, T, k, n):
    """Combine: k = 32 (every lane of the slot load), several batches of four local slots
    per token, rows narrower than a wave and a row of 3584 columns."""
    say(f"unpermute T={T} k={k} n={n}")
    rng = np.random.default_rng(2 + k)
    from moe_inputs import f32_to_bf16_bits
    rows = f32_to_bf16_bits(rng.standard_normal((300, n)).astype(np.float32))
    slot_row = rng.integers(-1, 300, size=(T, k)).astype(np.int32)
    slot_row[0] = -1                       # a token with no local slot
    w = rng.random(300).astype(np.float32)
    out = moe.moe_unpermute(dev_bf16(rows), dev(slot_row), dev(w))
    out_nw = moe.moe_unpermute(dev_bf16(rows), dev(slot_row))
    torch.cuda.synchronize()
    ref = oracle.bf16_round(oracle.unpermute_sum(rows, slot_row, w.astype(np.float64)))
    assert rel_err(host_bf16(out), ref) <= BF16_TOL
    ref = oracle.bf16_round(oracle.unpermute_sum(rows, slot_row))
    assert rel_err(host_bf16(out_nw), ref) <= BF16_TOL


def test_router_bwd(moe):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((100, 20)).astype(np.float32)
    idx, gates = oracle.route_topk(logits, 6)
    dp = rng.standard_normal((100, 6)).astype(np.float32)
    g_idx, g_gates = moe.moe_route_topk(dev(logits), 6)
    out = moe.moe_router_bwd(g_gates, dev(dp))
    torch.cuda.synchronize()
    assert rel_err(out.cpu().numpy(), oracle.router_bwd(gates, dp)) <= FP32_TOL


# ------------------------------------------------------------------------------- layer, full compare
MID = LayerConfig("mid", T=2048, d=256, H=192, E=16, k=4, e_lo=2, E_loc=10)
# every GEMM spans two or more N tiles (gate/up 5 pair tiles, down and dX 3, dA 3 with a
# half tile, dW_down 3 x 3, dW_gu 5 x 3) and the zipf bias makes the experts' rows uneven
MULTI = LayerConfig("multi_tile", T=1536, d=768, H=640, E=8, k=2, e_lo=0, E_loc=8, bias="zipf")
SMALL_CASES = {
    "tiny": LAYER_CONFIGS["tiny"],
    "mid": MID,                                                           # several tiles + ragged tails
    "multi_tile": MULTI,
    "one_token": LayerConfig("one_token", T=1, d=128, H=64, E=8, k=3, e_lo=0, E_loc=8),
    "k_eq_E": LayerConfig("k_eq_E", T=64, d=64, H=128, E=6, k=6, e_lo=0, E_loc=6),
    "none_local": LayerConfig("none_local", T=128, d=128, H=64, E=64, k=2, e_lo=60, E_loc=4),
    "skew_tail_small": LayerConfig("skew_tail_small", T=512, d=128, H=64, E=64, k=4, e_lo=20,
                                   E_loc=8, bias="zipf"),
    # the largest k: up to 32 local slots per token in the router, permute and both combines
    "k32": LayerConfig("k32", T=200, d=128, H=64, E=48, k=32, e_lo=4, E_loc=40),
}


def compare_full(m, cfg, inp, R_cap=None, **buf_kw):
    idx, gates, perm = oracle_route_perm(inp, cfg)
    buf, t = run_layer(m, cfg, inp, R_cap, **buf_kw)
    check_route_perm(buf, idx, gates, perm)
    f = oracle.expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta, mode="S")
    b = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta,
                                mode="S")
    R = perm["R"]
    gy, gdx = host_bf16(buf.y), host_bf16(buf.dx)
    errs = dict(
        h=rel_err(host_bf16(buf.h[:R]), f["h"]) if R else 0.0,
        y=rel_err(gy, f["y"]),
        dx=rel_err(gdx, b["dx"]),
        dw_gu=rel_err(buf.dw_gu.cpu().numpy(), b["dw_gu"]),
        dw_down=rel_err(buf.dw_down.cpu().numpy(), b["dw_down"]),
        dp=rel_err(buf.dp.cpu().numpy(), b["dp"]),
    )
    if R:
        errs["a"] = rel_err(host_bf16(buf.a_fwd[:R]), f["a"])
    if buf.combine_passes == 1:
        check_rounded_once(gy, buf.rows_fwd, perm["slot_row"], f"{cfg.name} y")
    once = dict(y=rel_to_sum(gy, f["y_sum"]), dx=rel_to_sum(gdx, b["dx_sum"]))
    say(cfg.name, "R", R, {k: f"{v:.2e}" for k, v in errs.items()},
        "vs pre-rounding sums:", {k: f"{v:.2e}" for k, v in once.items()})
    for k_, v in errs.items():
        assert v <= (FP32_TOL if k_ == "dp" else BF16_TOL), (k_, v)
    return buf, t, perm


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_layer_full(moe, name):
    cfg = SMALL_CASES[name]
    say(f"layer full {name}")
    inp = layer_inputs(cfg, seed=0)
    if name == "none_local":              # no token may pick the local window
        inp["logits"][:, cfg.e_lo:cfg.e_lo + cfg.E_loc] -= 100.0
    buf, t, perm = compare_full(moe, cfg, inp)
    if name == "none_local":
        assert perm["R"] == 0
        assert not bool(buf.y.any()) and not bool(buf.dx.any()) and not bool(buf.dp.any())
        assert not bool(buf.dw_gu.any()) and not bool(buf.dw_down.any())


# mid's shape with coefficients other than beta = 4, linear_beta = 25
COEF_CASE = LayerConfig("mid_coef", T=2048, d=256, H=192, E=16, k=4, e_lo=2, E_loc=10,
                        beta=2.5, linear_beta=12.0)


def test_layer_other_coefficients(moe):
    """beta = 2.5, linear_beta = 12: the gate/up epilogue's forward and the dA epilogue's
    backward on the kernels' beta != 4 path, every output compared in full with the oracle at
    the same coefficients."""
    say(f"layer full {COEF_CASE.name}")
    compare_full(moe, COEF_CASE, layer_inputs(COEF_CASE, seed=2))


def random_layer_configs(n=32, seed=7):
    """Seeded small shapes inside the library's envelope (d, H multiples of 64; k <= E):
    ragged N tiles of every GEMM, K extents of 2..18 stages of 32, 1..40 experts with
    uneven rows, local windows anywhere in the expert range."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 192, 320, 448, 576]))
        H = int(rng.choice([64, 128, 192, 320, 448, 576]))
        E = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(E, 8) + 1))
        E_loc = int(rng.integers(1, E + 1))
        e_lo = int(rng.integers(0, E - E_loc + 1))
        T = int(rng.choice([int(rng.integers(1, 16)), int(rng.integers(16, 1500))]))
        bias = "zipf" if rng.random() < 0.3 else None
        out.append(LayerConfig(f"rand{i}", T=T, d=d, H=H, E=E, k=k, e_lo=e_lo, E_loc=E_loc,
                               bias=bias))
    return out


@pytest.mark.parametrize("cfg", random_layer_configs(), ids=lambda c: c.name)
def test_layer_random_shapes(moe, cfg):
    """Every element of y, dx, h, a, dW and dp against the oracle on seeded random shapes."""
    say(f"layer random {cfg}")
    compare_full(moe, cfg, layer_inputs(cfg, seed=1))


def test_layer_exact_capacity(moe):
    """R_cap equal to the routed rows (the tightest legal buffers), found on the device."""
    inp = layer_inputs(MID, seed=1)
    _, _, perm = oracle_route_perm(inp, MID)
    R = moe.LayerBuffers.routed_rows(layer_shape(moe, MID), dev(inp["logits"]))
    assert R == perm["R"]
    compare_full(moe, MID, inp, R_cap=R)


def test_layer_combine_passes_bit_identical(moe):
    """The combines in 1, 2 or 3 passes over the output columns (d = 768: windows of 768, 512
    + 256, 256) and with or without the forward/backward memory overlay give bit-identical
    results; the one-pass run is also compared with the oracle."""
    inp = layer_inputs(MULTI, seed=6)
    _, _, perm = oracle_route_perm(inp, MULTI)
    ref, _, _ = compare_full(moe, MULTI, inp, R_cap=perm["R"], alias=False)
    for passes, alias in ((2, True), (3, True), (3, False)):
        say(f"combine passes {passes} alias {alias}")
        buf, _ = run_layer(moe, MULTI, inp, R_cap=perm["R"], alias=alias, combine_passes=passes)
        for name in ("y", "dx", "dw_gu", "dw_down", "dp", "h"):
            assert torch.equal(getattr(buf, name), getattr(ref, name)), (passes, alias, name)
        assert torch.equal(buf.a_fwd, ref.a_fwd)
    # the backward in separate stage calls (as the benchmark times it) is the same backward
    buf, t = run_layer(moe, MULTI, inp, R_cap=perm["R"])
    for name in ("dx", "dw_gu", "dw_down", "dp"):
        getattr(buf, name).zero_()
    for st in (moe.MOE_BWD_DA, moe.MOE_BWD_DW_DOWN, moe.MOE_BWD_DW_GU,
               moe.MOE_BWD_DX | moe.MOE_BWD_DP):
        buf.backward(t["dy"], t["x"], t["w_gu"], t["w_down"], stages=st)
    torch.cuda.synchronize()
    for name in ("dx", "dw_gu", "dw_down", "dp"):
        assert torch.equal(getattr(buf, name), getattr(ref, name)), ("stages", name)


def test_layer_deterministic_and_recompute_exact(moe):
    """Repeat runs are bit-identical; the activation recomputed from h equals the stored one;
    dy x 2 doubles dx, dW and dp exactly (power-of-two scaling is exact)."""
    inp = layer_inputs(MID, seed=2)
    buf, t = run_layer(moe, MID, inp)
    R = buf.rows()
    y1, dx1 = buf.y.clone(), buf.dx.clone()
    dwg1, dwd1, dp1 = buf.dw_gu.clone(), buf.dw_down.clone(), buf.dp.clone()
    a1 = buf.a_fwd[:R].clone()
    buf.step(t["x"], t["logits"], t["w_gu"], t["w_down"], t["dy"])
    torch.cuda.synchronize()
    for u, v in ((y1, buf.y), (dx1, buf.dx), (dwg1, buf.dw_gu), (dwd1, buf.dw_down), (dp1, buf.dp)):
        assert torch.equal(u, v)
    a_re = moe.situ_glu_fwd(buf.h[:R].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a_re.view(torch.int16), a1.view(torch.int16))
    buf.backward(t["dy"] * 2, t["x"], t["w_gu"], t["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(buf.dx.float(), dx1.float() * 2)
    assert torch.equal(buf.dw_gu, dwg1 * 2) and torch.equal(buf.dw_down, dwd1 * 2)
    assert torch.equal(buf.dp, dp1 * 2)


def test_layer_token_permutation(moe):
    """Permuting tokens permutes y and dx rows and leaves dW bit-identical."""
    inp = layer_inputs(MID, seed=4)
    buf, t = run_layer(moe, MID, inp)
    y1, dx1, dw1 = buf.y.clone(), buf.dx.clone(), buf.dw_gu.clone()
    perm_t = np.random.default_rng(0).permutation(MID.T)
    inp2 = dict(inp)
    for key in ("x", "logits", "dy"):
        inp2[key] = inp[key][perm_t]
    buf2, _ = run_layer(moe, MID, inp2)
    pt = torch.from_numpy(perm_t).cuda()
    assert torch.equal(buf2.y, y1[pt]) and torch.equal(buf2.dx, dx1[pt])
    # dW sums rows in token order within an expert, which the permutation changes: compare
    # to the bf16 bar instead of bitwise
    assert rel_err(buf2.dw_gu.cpu().numpy(), dw1.cpu().numpy()) <= 1e-5


# ------------------------------------------------------------------------------- layer, full-size sampled
def check_h_codes(got_c, got_s, h_ref, what):
    """The saved h as MXFP8 (codes, scale bytes) against the oracle's MXFP8 of its own bf16 h.
    The GPU's bf16 h can sit one bf16 step from the oracle's where its fp32 sum lies next to a
    rounding boundary; that moves an E4M3 code by one step at most or, when a block's largest
    magnitude crosses a power of two, its scale byte by one (the block's largest value may
    then move by two steps of the finer grid, its saturation band). Bound per element: two
    E4M3 steps at the larger of the two scales plus one bf16 step of h. Nearly all codes and
    scale bytes must be identical."""
    ref_c, ref_s = oracle.mxfp8.quantize(h_ref)
    g = oracle.mxfp8.dequantize(got_c, got_s)
    r = oracle.mxfp8.dequantize(ref_c, ref_s)
    X = np.maximum(got_s, ref_s).astype(np.int64).repeat(32, axis=1) - 127
    tol = 2.0 * e4m3_step(r, X) + 2.0 ** -7 * np.abs(h_ref)
    diff = np.abs(g - r)
    same_c = float(np.mean(got_c == ref_c))
    same_s = float(np.mean(got_s == ref_s))
    say(what, f"h codes identical {same_c:.5f}, scale bytes identical {same_s:.5f}, worst "
        f"|dh|/tol {float(np.max(diff / tol)):.3f}")
    assert not (diff > tol).any(), (what, np.argwhere(diff > tol)[:5])
    assert np.all(np.abs(got_s.astype(np.int64) - ref_s.astype(np.int64)) <= 1), what
    assert same_c >= 0.999 and same_s >= 0.999, (what, same_c, same_s)


def compare_sampled(m, cfg, n_tok=128, n_exp=4, n_col=14, seed=0, h_store="bf16", repeats=0):
    """Sampled comparison at full size: tokens (all their local rows), their rows' h and a,
    and the weight-gradient columns of sampled experts (incl. empty ones). h_store="mxfp8"
    runs the MXFP8-store path; its stored codes are checked within a bound and its weight-
    gradient columns are taken in whole 32-column blocks (a block shares one scale).
    repeats > 0 runs that many more steps on the same inputs and requires every output
    tensor to be bit-identical to the first step's."""
    mx = h_store == "mxfp8"
    say(f"layer sampled {cfg.name} ({h_store}): generating inputs")
    inp = layer_inputs(cfg, seed=0)
    say(f"layer sampled {cfg.name}: oracle routing")
    idx, gates, perm = oracle_route_perm(inp, cfg)
    say(f"layer sampled {cfg.name}: GPU step (R={perm['R']})")
    buf, t = run_layer(m, cfg, inp, h_store=h_store)
    check_route_perm(buf, idx, gates, perm)
    rng = np.random.default_rng(seed)
    local_tok = np.unique(perm["row_token"]) if perm["R"] else np.zeros(0, int)
    toks = np.concatenate([rng.choice(local_tok, min(n_tok, len(local_tok)), replace=False),
                           rng.choice(cfg.T, 8, replace=False), [0, cfg.T - 1]])
    sub, rows = sub_perm(perm, toks)
    say(f"layer sampled {cfg.name}: oracle on {len(rows)} rows")
    f = oracle.expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], sub, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta, mode="S")
    b = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], sub, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta,
                                mode="S", h_store=h_store)
    toks = np.unique(toks)
    tt = torch.from_numpy(toks).cuda()
    rr = torch.from_numpy(rows).cuda()
    gy, gdx = host_bf16(buf.y[tt]), host_bf16(buf.dx[tt])
    errs = dict(
        y=rel_err(gy, f["y"][toks]),
        dx=rel_err(gdx, b["dx"][toks]),
        dp=rel_err(buf.dp[tt].cpu().numpy(), b["dp"][toks]),
        a=rel_err(host_bf16(buf.a_fwd[rr]), f["a"]),
    )
    once = dict(y=rel_to_sum(gy, f["y_sum"][toks]))
    if mx:
        check_h_codes(buf.h_codes[rr].cpu().numpy(), buf.h_scales[rr].cpu().numpy(), f["h"],
                      f"{cfg.name} sampled")
    else:
        errs["h"] = rel_err(host_bf16(buf.h[rr]), f["h"])
        once["dx"] = rel_to_sum(gdx, b["dx_sum"][toks])
    # weight gradients: sampled experts x intermediate columns (all rows of the expert)
    counts = np.diff(perm["offsets"])
    exps = list(rng.choice(cfg.E_loc, n_exp, replace=False))
    if np.any(counts == 0):
        exps.append(int(np.nonzero(counts == 0)[0][0]))
    if mx:
        nb = cfg.H // 32
        blk = np.unique(np.concatenate([rng.choice(nb, 2, replace=False), [0, nb - 1]]))
        cols = (blk[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    else:
        cols = np.unique(np.concatenate([rng.choice(cfg.H, n_col, replace=False), [0, cfg.H - 1]]))
    dwg = buf.dw_gu
    dwd = buf.dw_down
    ref_gu_all, ref_dn_all, got_gu_all, got_dn_all = [], [], [], []
    for e in exps:
        say(f"layer sampled {cfg.name}: dW expert {e} rows {counts[e]}")
        gu, dn = oracle.dw_columns(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, int(e),
                                   cols, cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta,
                                   h_store=h_store)
        ci = torch.from_numpy(np.concatenate([cols, cfg.H + cols])).cuda()
        got_gu_all.append(dwg[int(e)][ci].cpu().numpy())
        got_dn_all.append(dwd[int(e)][:, torch.from_numpy(cols).cuda()].cpu().numpy())
        ref_gu_all.append(gu)
        ref_dn_all.append(dn)
    errs["dw_gu"] = rel_err(np.stack(got_gu_all), np.stack(ref_gu_all))
    errs["dw_down"] = rel_err(np.stack(got_dn_all), np.stack(ref_dn_all))
    say(cfg.name, "R", perm["R"], {k: f"{v:.2e}" for k, v in errs.items()},
        "vs pre-rounding sums:", {k: f"{v:.2e}" for k, v in once.items()})
    for k_, v in errs.items():
        assert v <= (FP32_TOL if k_ == "dp" else BF16_TOL), (k_, v)
    # properties over the whole tensors
    nonlocal_tok = np.setdiff1d(np.arange(cfg.T), local_tok)
    if len(nonlocal_tok):
        nt = torch.from_numpy(nonlocal_tok).cuda()
        assert not bool(buf.y[nt].any()) and not bool(buf.dx[nt].any())
    for tname in ("y", "dx", "dp", "dw_gu", "dw_down"):
        assert bool(torch.isfinite(getattr(buf, tname).float()).all()), tname
    if np.any(counts == 0):
        for e in np.nonzero(counts == 0)[0]:
            assert not bool(dwg[int(e)].any()) and not bool(dwd[int(e)].any())
    if repeats:
        first = {n_: getattr(buf, n_).clone() for n_ in ("y", "dx", "dp", "dw_gu", "dw_down")}
        for i in range(repeats):
            say(f"layer sampled {cfg.name}: repeat {i + 1} of {repeats}")
            buf.step(t["x"], t["logits"], t["w_gu"], t["w_down"], t["dy"])
            torch.cuda.synchronize()
            for n_, v in first.items():
                got = getattr(buf, n_)
                if v.dtype == torch.bfloat16:
                    got, v = got.view(torch.int16), v.view(torch.int16)
                assert torch.equal(got, v), (cfg.name, "repeat", i + 1, n_)


@pytest.mark.parametrize("name", ["shard", "skew", "skew_mid", "skew_tail", "large"])
def test_layer_full_size_sampled(moe, name):
    """At shard and large, three more steps must reproduce every output bit for bit (the
    persistent kernels' tile order, the scan-based permutation and the slot-order combines
    are deterministic)."""
    compare_sampled(moe, LAYER_CONFIGS[name], repeats=3 if name in ("shard", "large") else 0)
    torch.cuda.empty_cache()


def test_layer_mxfp8_full_size_sampled(moe):
    """The MXFP8-store path at the shard workload's full size, on the workload's own inputs."""
    compare_sampled(moe, LAYER_CONFIGS["shard"], h_store="mxfp8")
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ router backward, end to end
ROUTER_CASES = {
    "tiny": LAYER_CONFIGS["tiny"],
    # the large-context workload's shapes (16 of 28 local experts, every route local) at 512
    # tokens, so the oracle runs the whole layer
    "large_512": LayerConfig("large_512", T=512, d=3584, H=3072, E=28, k=16, e_lo=0, E_loc=28),
}


@pytest.mark.parametrize("name", list(ROUTER_CASES))
def test_router_bwd_end_to_end(moe, name):
    """dp from the layer's backward feeds the router backward: dlogits against the oracle's
    router_bwd of its own gates and dp (every route is local, so dp is complete)."""
    cfg = ROUTER_CASES[name]
    say(f"router bwd end to end {name}")
    inp = layer_inputs(cfg, seed=0)
    idx, gates, perm = oracle_route_perm(inp, cfg)
    assert perm["R"] == cfg.T * cfg.k
    buf, t = run_layer(moe, cfg, inp)
    check_route_perm(buf, idx, gates, perm)
    dl = moe.moe_router_bwd(buf.gates, buf.dp)
    torch.cuda.synchronize()
    say(f"router bwd end to end {name}: oracle")
    b = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta,
                                mode="S")
    ref = oracle.router_bwd(gates, b["dp"])
    errs = dict(dp=rel_err(buf.dp.cpu().numpy(), b["dp"]), dlogits=rel_err(dl.cpu().numpy(), ref))
    say(name, {k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["dp"] <= FP32_TOL and errs["dlogits"] <= FP32_TOL
    # softmax gradient: each token's dlogits sum to zero
    assert float(dl.double().sum(1).abs().max()) <= 1e-5 * float(dl.abs().max())


# ------------------------------------------------------------------ MXFP8 storage of the saved h
def test_mxfp8_quantize_dequantize(moe):
    """The standalone quantizer is bit-exact with the oracle's MXFP8 (codes and scale bytes)
    and the dequantizer returns the stored values exactly."""
    from moe_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(11)
    rows, n = 300, 256
    v = rng.standard_normal((rows, n)).astype(np.float32)
    v *= np.exp(rng.uniform(-30, 30, size=(rows, 1))).astype(np.float32)
    v[0, :32] = 0.0                                      # all-zero block
    v[1, :32] = -0.0                                     # negative zeros
    v[2, 5] = 1e4                                        # one outlier: the rest of the block is small
    v[3, ::7] *= 600.0                                   # several values in the saturation band
    v[4, :64] = rng.standard_normal(64).astype(np.float32) * 1e-38   # subnormal fp32 range
    vb = f32_to_bf16_bits(v)
    codes, scales = moe.moe_mxfp8_quantize(dev_bf16(vb))
    back = moe.moe_mxfp8_dequantize(codes, scales)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.mxfp8.quantize(oracle.bf16_widen(vb))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    ref_v = oracle.mxfp8.dequantize(ref_c, ref_s)
    got_v = host_bf16(back)
    big = np.abs(ref_v) >= 2.0 ** -126
    assert np.array_equal(got_v[big], ref_v[big])
    assert np.all(np.abs(got_v[~big] - ref_v[~big]) <= 2.0 ** -126)


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_layer_mxfp8_store(moe, name):
    """Layer with the saved h stored as MXFP8: the stored codes and scales equal the oracle's
    MXFP8 of its bf16 h (dyadic inputs make h exact on both sides); the forward is bit-identical
    to the bf16-store path; the backward matches the oracle recomputing from the stored h."""
    from moe_inputs import dyadic_layer_inputs
    cfg = SMALL_CASES[name]
    say(f"layer mxfp8 {name}")
    inp = dyadic_layer_inputs(cfg, seed=0)
    idx, gates, perm = oracle_route_perm(inp, cfg)
    shape = moe.LayerShape(T=cfg.T, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo, E_loc=cfg.E_loc, d=cfg.d,
                           H=cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta)
    t = dict(x=dev_bf16(inp["x"]), logits=dev(inp["logits"]), w_gu=dev_bf16(inp["w_gu"]),
             w_down=dev_bf16(inp["w_down"]), dy=dev_bf16(inp["dy"]))
    buf = moe.LayerBuffers(shape, h_store="mxfp8")
    buf.forward(t["x"], t["logits"], t["w_gu"], t["w_down"])
    a_mx = buf.a.clone()
    buf.backward(t["dy"], t["x"], t["w_gu"], t["w_down"])
    ref16 = moe.LayerBuffers(shape)
    ref16.forward(t["x"], t["logits"], t["w_gu"], t["w_down"])
    torch.cuda.synchronize()
    check_route_perm(buf, idx, gates, perm)
    R = perm["R"]
    f = oracle.expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta, mode="S")
    assert np.array_equal(host_bf16(ref16.h[:R]), f["h"])          # h is exact on both sides
    ref_c, ref_s = oracle.mxfp8.quantize(f["h"])
    assert np.array_equal(buf.h_codes[:R].cpu().numpy(), ref_c)
    assert np.array_equal(buf.h_scales[:R].cpu().numpy(), ref_s)
    assert torch.equal(a_mx[:R].view(torch.int16), ref16.a[:R].view(torch.int16))
    assert torch.equal(buf.y.view(torch.int16), ref16.y.view(torch.int16))
    b = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta,
                                mode="S", h_store="mxfp8")
    errs = dict(dx=rel_err(host_bf16(buf.dx), b["dx"]),
                dw_gu=rel_err(buf.dw_gu.cpu().numpy(), b["dw_gu"]),
                dw_down=rel_err(buf.dw_down.cpu().numpy(), b["dw_down"]),
                dp=rel_err(buf.dp.cpu().numpy(), b["dp"]))
    say(name, "R", R, {k: f"{v:.2e}" for k, v in errs.items()})
    for k_, v in errs.items():
        assert v <= (FP32_TOL if k_ == "dp" else BF16_TOL), (k_, v)
    # the stored form matters: the oracle's bf16-store backward differs from the MXFP8 one
    b16 = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                  beta=cfg.beta, linear_beta=cfg.linear_beta,
                                  mode="S")
    assert rel_err(b16["dp"], b["dp"]) > FP32_TOL


@pytest.mark.parametrize("name", ["tiny", "mid", "multi_tile", "mid_coef"])
def test_layer_mxfp8_store_general(moe, name):
    """The MXFP8-store layer on the workloads' own inputs (x ~ N(0,1), weights N(0, 1/fan_in)):
    the stored codes within the bound of check_h_codes; y, a and h's forward as in the
    bf16-store path; dx, dW and dp against the oracle recomputing from its own stored h.
    mid_coef takes the MXFP8 epilogues' beta != 4 path."""
    cfg = COEF_CASE if name == "mid_coef" else SMALL_CASES[name]
    say(f"layer mxfp8 general {name}")
    inp = layer_inputs(cfg, seed=0)
    idx, gates, perm = oracle_route_perm(inp, cfg)
    buf, t = run_layer(moe, cfg, inp, h_store="mxfp8")
    check_route_perm(buf, idx, gates, perm)
    ref16, _ = run_layer(moe, cfg, inp)
    R = perm["R"]
    f = oracle.expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta, mode="S")
    check_h_codes(buf.h_codes[:R].cpu().numpy(), buf.h_scales[:R].cpu().numpy(), f["h"], name)
    assert torch.equal(buf.a_fwd[:R].view(torch.int16), ref16.a_fwd[:R].view(torch.int16))
    assert torch.equal(buf.y.view(torch.int16), ref16.y.view(torch.int16))
    b = oracle.expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                beta=cfg.beta, linear_beta=cfg.linear_beta,
                                mode="S", h_store="mxfp8")
    errs = dict(dx=rel_err(host_bf16(buf.dx), b["dx"]),
                dw_gu=rel_err(buf.dw_gu.cpu().numpy(), b["dw_gu"]),
                dw_down=rel_err(buf.dw_down.cpu().numpy(), b["dw_down"]),
                dp=rel_err(buf.dp.cpu().numpy(), b["dp"]))
    say(name, "R", R, {k: f"{v:.2e}" for k, v in errs.items()})
    for k_, v in errs.items():
        assert v <= (FP32_TOL if k_ == "dp" else BF16_TOL), (k_, v)


# ------------------------------------------------------------------ W4A8 forward (MXFP4 weights)
W4A8_CASES = {
    "w4a8_tiny": LayerConfig("w4a8_tiny", T=256, d=256, H=128, E=8, k=2, e_lo=0, E_loc=8),
    # several m- and n-tiles, ragged experts, five K stages, a partial gate/up tile pair
    "w4a8_mid": LayerConfig("w4a8_mid", T=2048, d=640, H=384, E=16, k=4, e_lo=2, E_loc=10),
    "w4a8_none_local": LayerConfig("w4a8_none_local", T=128, d=128, H=128, E=64, k=2, e_lo=60,
                                   E_loc=4),
    "w4a8_one_token": LayerConfig("w4a8_one_token", T=1, d=128, H=128, E=8, k=3, e_lo=0,
                                  E_loc=8),
    "w4a8_k_eq_E": LayerConfig("w4a8_k_eq_E", T=64, d=128, H=256, E=6, k=6, e_lo=0, E_loc=6),
    # the SiTU-GLU epilogue on the kernels' beta != 4 path
    "w4a8_coef": LayerConfig("w4a8_coef", T=512, d=256, H=128, E=8, k=2, e_lo=0, E_loc=8,
                             beta=3.0, linear_beta=10.0),
    # K a multiple of 512 (at most 3584): the kernels' per-tile scale block instead of
    # per-stage scale loads; one 16-byte chunk of scales per row, and 7 (d = 3584, every
    # chunk of a row) with 3 for down (H = 1536)
    "w4a8_sb": LayerConfig("w4a8_sb", T=1024, d=512, H=512, E=8, k=2, e_lo=0, E_loc=8),
    "w4a8_sb_deep": LayerConfig("w4a8_sb_deep", T=300, d=3584, H=1536, E=4, k=2, e_lo=0,
                                E_loc=4),
    # K a multiple of 512 but above 3584 (32 stages): gate/up keeps the per-stage scale loads
    "w4a8_k4096": LayerConfig("w4a8_k4096", T=256, d=4096, H=256, E=4, k=2, e_lo=0, E_loc=4),
}


def e4m3_step(v, X):
    """Spacing of the E4M3 grid (scaled by 2^X) at magnitude |v|."""
    a = np.abs(v) / np.ldexp(1.0, X)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(np.int64) + X)


def check_a_codes(got_c, got_s, f, rows, H, beta, what):
    """a as MXFP8 against the oracle's (f: oracle result, rows: its rows to compare).

    The GPU takes h from the block-scaled MFMA, whose per-block sums deviate from exact ones
    by up to about 2^-12.7 of the sum of the products' magnitudes (measured), then rounds h
    and a to bf16 and encodes a; a code may therefore differ from the oracle's where a value
    sits near a rounding boundary. Bound per element: one E4M3 step of either side, one bf16
    step of a, and the h error carried through SiTU-GLU, |da| <= 1.2 |l| dg + min(beta, |g|) dl
    with dh = 2^-11 sum|x8 w4| + one bf16 step of h. Nearly all codes must be identical."""
    from oracle import mxfp8
    ref_c, ref_s = f["a_codes"][rows], f["a_scales"][rows]
    if ref_c.size == 0:
        return
    g = mxfp8.dequantize(got_c, got_s)
    r = mxfp8.dequantize(ref_c, ref_s)
    X = np.maximum(got_s, ref_s).astype(np.int64).repeat(32, axis=1) - 127
    hg, hl = f["h"][rows][:, :H], f["h"][rows][:, H:]
    mg, ml = f["h_mag"][rows][:, :H], f["h_mag"][rows][:, H:]
    dg = 2.0 ** -11 * mg + 2.0 ** -7 * np.abs(hg)
    dl = 2.0 ** -11 * ml + 2.0 ** -7 * np.abs(hl)
    tol = (np.maximum(e4m3_step(r, X), e4m3_step(g, X)) + 2.0 ** -7 * np.abs(r)
           + 1.2 * np.abs(hl) * dg + np.minimum(beta, np.abs(hg)) * dl)
    diff = np.abs(g - r)
    bad = diff > tol
    same = float(np.mean(got_c == ref_c))
    worst = np.unravel_index(np.argmax(diff / tol), diff.shape)
    say(what, f"a codes identical {same:.5f}, scales identical {float(np.mean(got_s == ref_s)):.5f},"
        f" worst |da|/tol {float(diff[worst] / tol[worst]):.3f} at {worst}: gpu {g[worst]:.6g}"
        f" oracle {r[worst]:.6g} tol {tol[worst]:.3g} step {e4m3_step(r, X)[worst]:.3g}"
        f" h {hg[worst]:.6g},{hl[worst]:.6g} sum|x w| {mg[worst]:.4g},{ml[worst]:.4g}")
    assert not bad.any(), (what, np.argwhere(bad)[:5])
    assert same >= 0.99, (what, same)


def run_w4a8(m, cfg, inp, R_cap=None):
    shape = m.LayerShape(T=inp["x"].shape[0], E=cfg.E, k=cfg.k, e_lo=cfg.e_lo, E_loc=cfg.E_loc,
                         d=cfg.d, H=cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta)
    buf = m.LayerBuffers(shape, R_cap=R_cap)
    x, logits = dev_bf16(inp["x"]), dev(inp["logits"])
    w4 = m.W4A8Weights(dev_bf16(inp["w_gu"]), dev_bf16(inp["w_down"]))
    buf.forward_w4a8(x, logits, w4)
    torch.cuda.synchronize()
    return buf, w4


def test_mxfp4_quantize_dequantize(moe):
    """The weight quantizer is bit-exact with the oracle's MXFP4 (packed codes and scale
    bytes) and the dequantizer returns the stored values exactly."""
    from moe_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(12)
    rows, n = 300, 256
    v = rng.standard_normal((rows, n)).astype(np.float32)
    v *= np.exp(rng.uniform(-30, 30, size=(rows, 1))).astype(np.float32)
    v[0, :32] = 0.0
    v[1, :32] = -0.0
    v[2, 5] = 1e4                                        # one outlier: the rest of the block rounds to 0
    v[3, ::5] *= 7.0                                     # values in the saturation band
    v[4, :64] = rng.standard_normal(64).astype(np.float32) * 1e-38
    tab = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5], np.float32)
    v[5, :16], v[5, 16:32] = tab, -tab                   # every rounding midpoint, scale X = 0
    vb = f32_to_bf16_bits(v)
    codes, scales = moe.moe_mxfp4_quantize(dev_bf16(vb))
    back = moe.moe_mxfp4_dequantize(codes, scales)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.mxfp4.quantize(oracle.bf16_widen(vb))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(host_bf16(back), oracle.mxfp4.dequantize(ref_c, ref_s))


def compare_w4a8_full(m, cfg, inp, R_cap=None):
    idx, gates, perm = oracle_route_perm(inp, cfg)
    buf, w4 = run_w4a8(m, cfg, inp, R_cap)
    check_route_perm(buf, idx, gates, perm)
    ref_xc, ref_xs = oracle.mxfp8.quantize(oracle.bf16_widen(inp["x"]))
    assert np.array_equal(buf.x_codes.cpu().numpy(), ref_xc)
    assert np.array_equal(buf.x_scales.cpu().numpy(), ref_xs)
    wq = [oracle.mxfp4.quantize(oracle.bf16_widen(inp[k_])) for k_ in ("w_gu", "w_down")]
    assert np.array_equal(w4.gu_codes.cpu().numpy(), wq[0][0])
    assert np.array_equal(w4.gu_scales.cpu().numpy(), wq[0][1])
    assert np.array_equal(w4.down_codes.cpu().numpy(), wq[1][0])
    assert np.array_equal(w4.down_scales.cpu().numpy(), wq[1][1])
    f = oracle.w4a8.expert_layer_fwd_w4a8(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                                           cfg.beta, cfg.linear_beta)
    R = perm["R"]
    check_a_codes(buf.a_codes[:R].cpu().numpy(), buf.a_scales[:R].cpu().numpy(), f,
                  np.arange(R), cfg.H, cfg.beta, cfg.name)
    gy = host_bf16(buf.y)
    err = rel_err(gy, f["y"])
    check_rounded_once(gy, rows_f32(buf, cfg.d), perm["slot_row"], f"{cfg.name} y")
    once = rel_to_sum(gy, f["y_sum"])
    say(cfg.name, "R", R, f"y {err:.2e}, vs pre-rounding sum {once:.2e}")
    assert err <= BF16_TOL
    return buf, perm


@pytest.mark.parametrize("name", list(W4A8_CASES))
def test_w4a8_forward(moe, name):
    cfg = W4A8_CASES[name]
    say(f"w4a8 full {name}")
    inp = layer_inputs(cfg, seed=0)
    if name == "w4a8_none_local":
        inp["logits"][:, cfg.e_lo:cfg.e_lo + cfg.E_loc] -= 100.0
    buf, perm = compare_w4a8_full(moe, cfg, inp)
    if name == "w4a8_none_local":
        assert perm["R"] == 0 and not bool(buf.y.any())


def test_w4a8_scales_4_byte_aligned(moe):
    """The C ABI lets the scale arrays be 4-byte aligned. The GEMMs then load each stage's
    scale bytes per row instead of keeping the 16-byte-loaded scale block, with the same
    products in the same order: gate/up's a codes and scales and down's y from 4-byte (not
    16-byte) aligned copies of every scale array equal the aligned run's bit for bit (a shape
    whose K suits the scale block, which test_w4a8_forward[w4a8_sb] compares with the
    oracle)."""
    cfg = W4A8_CASES["w4a8_sb"]
    inp = layer_inputs(cfg, seed=5)
    buf, w4 = run_w4a8(moe, cfg, inp)
    R = buf.rows()
    assert R > 0

    def off4(t):
        flat = torch.empty(t.numel() + 32, dtype=torch.uint8, device=t.device)
        base = (-flat.data_ptr()) % 16 + 4
        v = flat[base:base + t.numel()].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 == 4
        return v

    a_c, a_s = moe.moe_grouped_gemm_gate_up_w4a8(
        buf.x_codes, off4(buf.x_scales), buf.perm["row_token"], buf.perm["offsets"],
        w4.gu_codes, off4(w4.gu_scales), buf.R_cap, cfg.beta, cfg.linear_beta)
    y = moe.moe_grouped_gemm_down_combine_w4a8(
        buf.a_codes, off4(buf.a_scales), buf.perm["offsets"], buf.perm["row_gate"],
        buf.perm["slot_row"], w4.down_codes, off4(w4.down_scales), buf.R_cap)
    torch.cuda.synchronize()
    assert torch.equal(a_c[:R], buf.a_codes[:R])
    assert torch.equal(a_s[:R], buf.a_scales[:R])
    assert torch.equal(y.view(torch.int16), buf.y.view(torch.int16))


def test_w4a8_exact_capacity(moe):
    """R_cap equal to the routed rows (the tightest legal buffers)."""
    cfg = W4A8_CASES["w4a8_mid"]
    inp = layer_inputs(cfg, seed=3)
    _, _, perm = oracle_route_perm(inp, cfg)
    compare_w4a8_full(moe, cfg, inp, R_cap=perm["R"])


def test_w4a8_rows_past_4gib(moe):
    """W4A8 with activation codes past 4 GiB: 140000 tokens routed to all 8 experts of H =
    4096 give R * H = 4.6e9 bytes of a codes, so the down GEMM's rows of the last expert lie
    beyond 2^32 bytes from the array's start. Tokens late in the batch (whose last-expert rows
    are there) are compared with the oracle over all 8 experts."""
    cfg = LayerConfig("w4a8_past_4gib", T=140000, d=256, H=4096, E=8, k=8, e_lo=0, E_loc=8)
    say("w4a8 rows past 4 GiB: generating inputs")
    inp = layer_inputs(cfg, seed=3)
    idx, gates, perm = oracle_route_perm(inp, cfg)
    assert perm["R"] * cfg.H > (1 << 32)
    say(f"w4a8 rows past 4 GiB: GPU forward (R={perm['R']})")
    buf, w4 = run_w4a8(moe, cfg, inp)
    check_route_perm(buf, idx, gates, perm)
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(np.arange(cfg.T - 20000, cfg.T), 12, replace=False))
    sub, rows = sub_perm(perm, toks)
    assert rows.max() * cfg.H >= (1 << 32)
    say(f"w4a8 rows past 4 GiB: oracle on {len(rows)} rows")
    f = oracle.w4a8.expert_layer_fwd_w4a8(inp["x"], inp["w_gu"], inp["w_down"], sub, cfg.H,
                                           cfg.beta, cfg.linear_beta)
    tt = torch.from_numpy(toks).cuda()
    rr = torch.from_numpy(rows).cuda()
    check_a_codes(buf.a_codes[rr].cpu().numpy(), buf.a_scales[rr].cpu().numpy(), f,
                  np.arange(len(rows)), cfg.H, cfg.beta, "past 4 GiB")
    err = rel_err(host_bf16(buf.y[tt]), f["y"][toks])
    say("w4a8 rows past 4 GiB", len(toks), "tokens", f"y {err:.2e}")
    assert err <= BF16_TOL
    del buf, w4
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["shard", "skew_tail"])
def test_w4a8_full_size_sampled(moe, name):
    """The W4A8 forward at a full-size workload (one rank's shard; the skewed window with
    empty experts), compared on tokens whose local routes all go to two sampled experts of at
    most 2000 rows (the oracle quantizes only those experts' weights), plus properties of the
    whole output."""
    cfg = LAYER_CONFIGS[name]
    say(f"w4a8 sampled {name}: generating inputs")
    inp = layer_inputs(cfg, seed=0)
    idx, gates, perm = oracle_route_perm(inp, cfg)
    say(f"w4a8 sampled {name}: GPU forward (R={perm['R']})")
    buf, w4 = run_w4a8(moe, cfg, inp)
    check_route_perm(buf, idx, gates, perm)
    rng = np.random.default_rng(0)
    off = perm["offsets"]
    counts = np.diff(off)
    small = np.nonzero((counts > 0) & (counts <= 2000))[0]
    exps = set(int(e) for e in rng.choice(small, min(2, len(small)), replace=False))
    row_exp = np.repeat(np.arange(cfg.E_loc), np.diff(off))
    tok_all = perm["row_token"][: perm["R"]]
    ok = np.ones(cfg.T, bool)
    ok[tok_all[~np.isin(row_exp, list(exps))]] = False       # a route outside the sampled experts
    cand = np.intersect1d(np.nonzero(ok)[0], tok_all)
    toks = np.concatenate([rng.choice(cand, min(40, len(cand)), replace=False),
                           rng.choice(np.setdiff1d(np.arange(cfg.T), tok_all), 4, replace=False)])
    sub, rows = sub_perm(perm, toks)
    say(f"w4a8 sampled {name}: oracle on {len(rows)} rows of experts {sorted(exps)}")
    # the oracle reads w[e] only for experts with rows, which in `sub` are the sampled ones
    w_gu = {e: inp["w_gu"][e] for e in exps}
    w_down = {e: inp["w_down"][e] for e in exps}
    f = oracle.w4a8.expert_layer_fwd_w4a8(inp["x"], w_gu, w_down, sub, cfg.H, cfg.beta,
                                           cfg.linear_beta)
    toks = np.unique(toks)
    tt = torch.from_numpy(toks).cuda()
    rr = torch.from_numpy(rows).cuda()
    check_a_codes(buf.a_codes[rr].cpu().numpy(), buf.a_scales[rr].cpu().numpy(), f,
                  np.arange(len(rows)), cfg.H, cfg.beta, f"{name} sampled")
    err = rel_err(host_bf16(buf.y[tt]), f["y"][toks])
    say(f"w4a8 {name} sampled", len(toks), "tokens", f"y {err:.2e}")
    assert err <= BF16_TOL
    nonlocal_tok = torch.from_numpy(np.setdiff1d(np.arange(cfg.T), tok_all)).cuda()
    assert not bool(buf.y[nonlocal_tok].any())
    assert bool(torch.isfinite(buf.y.float()).all())
    del buf, w4
    torch.cuda.empty_cache()
