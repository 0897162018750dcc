"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins: closed forms, limits, a special case that reduces to a library
routine, brute force on tiny inputs, finite differences, autograd, and the numbers the
pages print (tests/golden/page_numbers.json). CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (bf16_round, situ_glu_fwd, situ_glu_bwd, route_topk, permute,
                    expert_layer_fwd, expert_layer_bwd, token_layer_fwd, token_layer_bwd,
                    dw_columns, router_bwd, unpermute_sum)
from moe_inputs import LAYER_CONFIGS, LayerConfig, layer_inputs, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


# ----------------------------------------------------------------------------- bf16 storage
def test_bf16_round_matches_torch_on_fp32_values():
    """fp32 -> bf16 is a single rounding; torch's cast (RNE) is the library reference."""
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),       # fp32 subnormals
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895313e38, 3.4e38, -3.4e38,
                  1e-45, -1e-45, 65504.0], dtype=np.float32),
    ])
    ours = bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)


def test_bf16_round_is_direct_from_fp64():
    """1 + 2^-8 + 2^-30 is above the bf16 tie, so direct rounding gives 1 + 2^-7; rounding
    via fp32 first would land on the tie 1 + 2^-8 and then round to even (1.0)."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_round(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0            # exact tie -> even
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7


def test_bf16_widen_matches_torch_on_every_bit_pattern():
    """All 65,536 bf16 bit patterns widen to the value torch assigns them (its bfloat16 view of
    the same bits, cast to fp64): zeros of both signs, subnormals, normals, infinities and
    NaNs. A wrong shift, byte order or view fails here, independently of the oracle's other
    helpers, which all decode through this function."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_widen(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert ours.dtype == np.float64 and ours.shape == (1 << 16,)
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127 and np.array_equal(np.isnan(ours), nan)
    # spot values from the format's definition
    assert ours[0x3F80] == 1.0 and ours[0xBF80] == -1.0 and ours[0x0001] == 2.0 ** -133
    assert ours[0x7F7F] == (2.0 - 2.0 ** -7) * 2.0 ** 127 and ours[0x7F80] == np.inf


def test_layer_sums_are_rounded_once():
    """The forward's y and the backward's dx are their pre-rounding sums rounded once: in mode
    S, y = bf16(y_sum) and dx = bf16(dx_sum) exactly; in mode X the sums are the outputs; and
    the mode-S sums stay within the storage roundings (h, a, dh to bf16) of the exact ones."""
    cfg = LayerConfig("s", T=40, d=64, H=64, E=6, k=3, e_lo=1, E_loc=4)
    inp = layer_inputs(cfg, seed=5)
    idx, gates = route_topk(inp["logits"], cfg.k)
    perm = permute(idx, gates, cfg.e_lo, cfg.E_loc)
    fs = expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="S")
    fx = expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="X")
    bs = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="S")
    bx = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="X")
    assert np.array_equal(fs["y"], bf16_round(fs["y_sum"]))
    assert np.array_equal(bs["dx"], bf16_round(bs["dx_sum"]))
    assert np.array_equal(fx["y"], fx["y_sum"]) and np.array_equal(bx["dx"], bx["dx_sum"])
    assert not np.array_equal(fs["y_sum"], fs["y"])          # the rounding is not a no-op
    for s_, x_ in ((fs["y_sum"], fx["y"]), (bs["dx_sum"], bx["dx"])):
        assert np.max(np.abs(s_ - x_)) <= 2.0 ** -6 * np.max(np.abs(x_))


# ----------------------------------------------------------------------------- SiTU-GLU
def _h(g, l):
    g = np.atleast_1d(np.asarray(g, np.float64))
    l = np.atleast_1d(np.asarray(l, np.float64))
    return np.stack([g, l], axis=-1), 1


def test_situ_zero_rows():
    """a(0, l) = 0 and a(g, 0) = 0: tanh(0) = 0 in both factors."""
    g = np.linspace(-50, 50, 1001)
    h, H = _h(g, np.zeros_like(g))
    assert np.all(situ_glu_fwd(h, H) == 0)
    h, H = _h(np.zeros_like(g), g)
    assert np.all(situ_glu_fwd(h, H) == 0)


def test_situ_closed_form_points():
    """lin'(25 atanh(1/2)) = 12.5 exactly in real arithmetic; gate' -> beta, 0 and
    lin' -> +-linear_beta in the saturation limits; slopes at zero are 1/2 and 1."""
    l = 25.0 * math.atanh(0.5)
    g_big = 60.0
    h, H = _h([g_big], [l])
    # gate'(60) = 4 tanh(15) sigmoid(60) = 4 to 1e-12
    assert situ_glu_fwd(h, H)[0] == pytest.approx(4.0 * 12.5, rel=1e-12)
    h, H = _h([-60.0, 60.0], [1e4, -1e4])
    a = situ_glu_fwd(h, H)
    assert -1e-20 < a[0] <= 0.0            # gate'(-60) ~ -4 e^-60 -> 0 from below, times +25
    assert a[1] == pytest.approx(-100.0, rel=1e-12)
    # slope at g = 0 with lin' = 1: choose l = 25 atanh(1/25) so lin'(l) = 1
    l1 = 25.0 * math.atanh(1.0 / 25.0)
    h, H = _h([0.0], [l1])
    dh = situ_glu_bwd(h, np.ones((1, 1)), H)
    assert dh[0, 0] == pytest.approx(0.5, rel=1e-14)      # d gate'/dg (0) = sigmoid(0) = 1/2
    h, H = _h([60.0], [0.0])
    dh = situ_glu_bwd(h, np.ones((1, 1)), H)
    assert dh[0, 1] == pytest.approx(4.0, rel=1e-12)      # gate'(60) * d lin'/dl (0) = 4 * 1


def test_situ_swiglu_limit_matches_torch_silu():
    """With beta, linear_beta -> infinity, beta tanh(g/beta) -> g and lin' -> l, so SiTU-GLU
    becomes SwiGLU silu(gate) * linear; torch.nn.functional.silu is the library reference.
    Catches a swapped gate/linear half, a missing sigmoid, or a wrong product."""
    rng = np.random.default_rng(2)
    H = 37
    h = rng.standard_normal((50, 2 * H)) * 3.0
    ours = situ_glu_fwd(h, H, beta=1e8, linear_beta=1e8)
    t = torch.from_numpy(h)
    ref = (torch.nn.functional.silu(t[:, :H]) * t[:, H:]).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_situ_bounds_and_extremes():
    """|gate'| < beta and |lin'| < linear_beta, so |a| < 100; extreme inputs stay finite;
    gate' has its minimum -0.26977 near g = -1.2188 and d gate'/dg lies in [-0.1054, 0.9264]."""
    g = np.linspace(-400, 400, 400001)
    h, H = _h(g, np.full_like(g, 1e6))
    a = situ_glu_fwd(h, H)
    assert np.all(np.isfinite(a)) and np.max(np.abs(a)) <= 100.0
    h, H = _h(np.array([-1e30, 1e30, -3e38, 3e38]), np.array([1e30, -1e30, 0.5, 0.5]))
    assert np.all(np.isfinite(situ_glu_fwd(h, H)))
    gg = np.linspace(-3, 0, 300001)
    gate = situ_glu_fwd(_h(gg, np.full_like(gg, 1e9))[0], 1) / 25.0
    i = int(np.argmin(gate))
    assert gate[i] == pytest.approx(-0.26977, abs=5e-6)
    assert gg[i] == pytest.approx(-1.2188, abs=2e-4)
    gw = np.linspace(-30, 30, 600001)
    l1 = 25.0 * math.atanh(1.0 / 25.0)
    dg = situ_glu_bwd(_h(gw, np.full_like(gw, l1))[0], np.ones((gw.size, 1)), 1)[:, 0]
    assert dg.min() == pytest.approx(-0.1054, abs=1e-4)
    assert dg.max() == pytest.approx(0.9264, abs=1e-4)


def test_situ_bwd_matches_central_differences():
    """The hand-derived backward equals central differences of the forward."""
    rng = np.random.default_rng(3)
    H = 16
    h = rng.standard_normal((40, 2 * H)) * 3.0
    da = rng.standard_normal((40, H))
    dh = situ_glu_bwd(h, da, H)
    eps = 1e-6
    fd = np.zeros_like(h)
    for c in range(2 * H):
        hp, hm = h.copy(), h.copy()
        hp[:, c] += eps
        hm[:, c] -= eps
        fd[:, c] = np.sum(da * (situ_glu_fwd(hp, H) - situ_glu_fwd(hm, H)), axis=1) / (2 * eps)
    np.testing.assert_allclose(dh, fd, rtol=1e-6, atol=1e-8)


def test_situ_bwd_matches_autograd():
    """torch autograd of the activation (fp64) is an independent derivative."""
    rng = np.random.default_rng(4)
    H = 24
    h = rng.standard_normal((30, 2 * H)) * 4.0
    da = rng.standard_normal((30, H))
    t = torch.tensor(h, requires_grad=True)
    g, l = t.split(H, dim=-1)
    out = torch.mul(torch.sigmoid(g) * torch.tanh(g / 4.0) * 4.0, torch.tanh(l / 25.0) * 25.0)
    out.backward(torch.from_numpy(da))
    np.testing.assert_allclose(situ_glu_bwd(h, da, H), t.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(situ_glu_fwd(h, H), out.detach().numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("beta,linear_beta", [(3.0, 10.0), (1.0, 1.0), (7.5, 40.0)])
def test_situ_other_coefficients_match_autograd(beta, linear_beta):
    """The coefficients are parameters of the op ("Frontier-scale RL with Kimi K3", section
    "Streaming activations"): with beta != 4 and linear_beta != 25 the oracle's forward and
    backward equal torch's fp64 composition of the same formula and its autograd."""
    rng = np.random.default_rng(6)
    H = 20
    h = rng.standard_normal((30, 2 * H)) * 5.0
    da = rng.standard_normal((30, H))
    t = torch.tensor(h, requires_grad=True)
    g, l = t.split(H, dim=-1)
    out = torch.mul(torch.sigmoid(g) * torch.tanh(g / beta) * beta,
                    torch.tanh(l / linear_beta) * linear_beta)
    out.backward(torch.from_numpy(da))
    np.testing.assert_allclose(situ_glu_fwd(h, H, beta, linear_beta), out.detach().numpy(),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(situ_glu_bwd(h, da, H, beta, linear_beta), t.grad.numpy(),
                               rtol=1e-12, atol=1e-14)
    # and they differ from the default coefficients' results on these inputs
    assert not np.allclose(situ_glu_fwd(h, H, beta, linear_beta), situ_glu_fwd(h, H))


def test_naive_activation_saves_six_fp32_copies():
    """The pages say autograd keeps 6 fp32 copies of [R, H] for the naive activation and that
    the bf16 [R, 2H] input is 1/6 of that. Count autograd's saved storages."""
    R, H = 64, 48
    x = torch.randn(R, 2 * H, dtype=torch.bfloat16, requires_grad=True)
    seen = {}

    def pack(t):
        seen[t.untyped_storage().data_ptr()] = t.untyped_storage().nbytes()
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        xf = x.float()
        g, l = xf[:, :H], xf[:, H:]
        gate = torch.tanh(g / 4.0) * 4.0 * torch.sigmoid(g)
        lin = torch.tanh(l / 25.0) * 25.0
        (gate * lin).to(x.dtype)
    big = [n for n in seen.values() if n == R * H * 4]
    assert len(big) == 6
    assert sum(big) == 6 * (R * 2 * H * 2)         # six fp32 [R,H] == 6x the bf16 [R,2H] input


# ----------------------------------------------------------------------------- routing
def _brute_topk(L, k):
    idx = np.zeros((L.shape[0], k), np.int32)
    for t in range(L.shape[0]):
        order = sorted(range(L.shape[1]), key=lambda e: (-float(L[t, e]), e))
        idx[t] = order[:k]
    return idx


def test_route_matches_brute_force_with_ties():
    rng = np.random.default_rng(5)
    L = rng.integers(-3, 4, size=(200, 12)).astype(np.float32)   # many ties
    L[0, :] = 0.0
    L[1, ::2] = -0.0                                               # -0.0 ties +0.0
    for k in (1, 3, 12):
        idx, gates = route_topk(L, k)
        assert np.array_equal(idx, _brute_topk(L, k))
    assert list(route_topk(np.array([[1, 3, 3, 2, 3]], np.float32), 3)[0][0]) == [1, 2, 4]
    assert route_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 1)[0][0, 0] == 0


def test_route_matches_torch_topk_and_softmax():
    """Distinct values: torch.topk's sorted output is the unique order; softmax over the kept
    values equals torch.softmax."""
    rng = np.random.default_rng(6)
    L = rng.standard_normal((300, 896)).astype(np.float32)
    idx, gates = route_topk(L, 16)
    tv, ti = torch.topk(torch.from_numpy(L).double(), 16, dim=-1, sorted=True)
    assert np.array_equal(idx, ti.numpy())
    np.testing.assert_allclose(gates, torch.softmax(tv, dim=-1).numpy(), rtol=1e-14)
    np.testing.assert_allclose(gates.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(gates > 0) and np.all(np.diff(gates, axis=1) <= 0)


# ----------------------------------------------------------------------------- permute
def _check_perm_invariants(idx, gates, e_lo, E_loc, perm):
    off, rt, rg, sr = perm["offsets"], perm["row_token"], perm["row_gate"], perm["slot_row"]
    local = (idx >= e_lo) & (idx < e_lo + E_loc)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == local.sum() == perm["R"]
    t, j = np.nonzero(sr >= 0)
    assert np.array_equal(sr >= 0, local)
    assert np.array_equal(rt[sr[t, j]], t)                     # slot_row and row_token inverse
    assert np.array_equal(rg[sr[t, j]], gates[t, j])
    assert sorted(sr[t, j].tolist()) == list(range(perm["R"]))


def test_permute_matches_stable_argsort():
    """Rows are a stable sort, by expert, of the local routes listed in token-major order."""
    rng = np.random.default_rng(7)
    L = rng.standard_normal((500, 40)).astype(np.float32)
    idx, gates = route_topk(L, 6)
    for e_lo, E_loc in ((0, 40), (8, 10), (35, 5)):
        perm = permute(idx, gates, e_lo, E_loc)
        _check_perm_invariants(idx, gates, e_lo, E_loc, perm)
        t, j = np.nonzero((idx >= e_lo) & (idx < e_lo + E_loc))     # token-major order
        order = np.argsort(idx[t, j], kind="stable")
        assert np.array_equal(perm["row_token"], t[order])
        counts = np.bincount(idx[t, j] - e_lo, minlength=E_loc)
        assert np.array_equal(perm["offsets"], np.concatenate([[0], np.cumsum(counts)]))


def test_permute_empty_window():
    idx = np.array([[0, 1], [1, 2]], np.int32)
    gates = np.full((2, 2), 0.5)
    perm = permute(idx, gates, 5, 3)
    assert perm["R"] == 0 and np.all(perm["offsets"] == 0) and np.all(perm["slot_row"] == -1)


# ----------------------------------------------------------------------------- layer
TINYCFG = LayerConfig("t", T=8, d=8, H=4, E=4, k=2, e_lo=0, E_loc=4)


def _setup(cfg, T=None, seed=0):
    inp = layer_inputs(cfg, seed=seed, T=T)
    idx, gates = route_topk(inp["logits"], cfg.k)
    perm = permute(idx, gates, cfg.e_lo, cfg.E_loc)
    return inp, idx, gates, perm


@pytest.mark.parametrize("mode", ["X", "S"])
def test_grouped_equals_per_token_loop(mode):
    """The grouped computation equals the routing snippet's per-token loop."""
    cfg = LayerConfig("g", T=64, d=32, H=16, E=12, k=3, e_lo=2, E_loc=7)
    inp, idx, gates, perm = _setup(cfg)
    fwd = expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode=mode)
    bwd = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                           mode=mode)
    for t in range(cfg.T):
        y_t = token_layer_fwd(inp["x"][t], idx[t], gates[t], inp["w_gu"], inp["w_down"],
                              cfg.e_lo, cfg.H, mode=mode)
        dx_t, dp_t = token_layer_bwd(inp["x"][t], inp["dy"][t], idx[t], gates[t], inp["w_gu"],
                                     inp["w_down"], cfg.e_lo, cfg.H, mode=mode)
        tol = 1e-12 if mode == "X" else 1e-2    # S: a rare bf16 tie flip from BLAS order
        np.testing.assert_allclose(fwd["y"][t], y_t, rtol=tol, atol=tol)
        np.testing.assert_allclose(bwd["dx"][t], dx_t, rtol=tol, atol=tol)
        np.testing.assert_allclose(bwd["dp"][t], dp_t, rtol=1e-10 if mode == "X" else 1e-3,
                                   atol=1e-12 if mode == "X" else 1e-4)


def test_layer_bwd_matches_finite_differences():
    """Central differences of L = <dy, y> (mode X) w.r.t. x, W_gate, W_up, W_down and the
    gates p; the p derivative checks dp = <W_down^T dy, a>."""
    cfg = TINYCFG
    inp, idx, gates, perm = _setup(cfg)
    H = cfg.H
    x = oracle.bf16_widen(inp["x"])
    wgu = oracle.bf16_widen(inp["w_gu"])
    wd = oracle.bf16_widen(inp["w_down"])
    dy = oracle.bf16_widen(inp["dy"])

    def loss(x_, wgu_, wd_, perm_):
        return float(np.sum(dy * expert_layer_fwd(x_, wgu_, wd_, perm_, H, mode="X")["y"]))

    g = expert_layer_bwd(x, dy, wgu, wd, perm, H, mode="X")
    eps = 1e-6
    rng = np.random.default_rng(8)
    for name, arr, grad in (("x", x, g["dx"]), ("w_gu", wgu, g["dw_gu"]),
                            ("w_down", wd, g["dw_down"])):
        for _ in range(12):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += eps
            am[pos] -= eps
            args_p = dict(x=x, w_gu=wgu, w_down=wd)
            args_m = dict(x=x, w_gu=wgu, w_down=wd)
            args_p[name], args_m[name] = ap, am
            fd = (loss(args_p["x"], args_p["w_gu"], args_p["w_down"], perm) -
                  loss(args_m["x"], args_m["w_gu"], args_m["w_down"], perm)) / (2 * eps)
            assert grad[pos] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, pos)
    for r in range(perm["R"]):
        pp, pm = dict(perm), dict(perm)
        pp["row_gate"] = perm["row_gate"].copy()
        pm["row_gate"] = perm["row_gate"].copy()
        pp["row_gate"][r] += eps
        pm["row_gate"][r] -= eps
        fd = (loss(x, wgu, wd, pp) - loss(x, wgu, wd, pm)) / (2 * eps)
        assert g["dp_rows"][r] == pytest.approx(fd, rel=1e-6, abs=1e-8)


def test_dp_rewrite_identity():
    """<dy, o_e> (direct form) equals <W_down^T dy, a_e> (rewritten form) per route."""
    cfg = LayerConfig("g", T=40, d=24, H=12, E=6, k=2, e_lo=0, E_loc=6)
    inp, idx, gates, perm = _setup(cfg)
    fwd = expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="X")
    bwd = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                           mode="X")
    dy = oracle.bf16_widen(inp["dy"])
    for e in range(cfg.E_loc):
        r0, r1 = perm["offsets"][e], perm["offsets"][e + 1]
        o = fwd["a"][r0:r1] @ oracle.bf16_widen(inp["w_down"][e]).T
        direct = np.sum(dy[perm["row_token"][r0:r1]] * o, axis=1)
        np.testing.assert_allclose(bwd["dp_rows"][r0:r1], direct, rtol=1e-12, atol=1e-13)


def test_layer_bwd_matches_autograd():
    """torch autograd (fp64) of the per-token layer gives dx, dW and dp independently."""
    cfg = LayerConfig("g", T=24, d=16, H=8, E=5, k=2, e_lo=1, E_loc=3)
    inp, idx, gates, perm = _setup(cfg)
    H = cfg.H
    x = torch.tensor(oracle.bf16_widen(inp["x"]), requires_grad=True)
    wgu = torch.tensor(oracle.bf16_widen(inp["w_gu"]), requires_grad=True)
    wd = torch.tensor(oracle.bf16_widen(inp["w_down"]), requires_grad=True)
    p = torch.tensor(gates, requires_grad=True)
    dy = torch.tensor(oracle.bf16_widen(inp["dy"]))
    loss = 0
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = int(idx[t, j]) - cfg.e_lo
            if 0 <= e < cfg.E_loc:
                hh = wgu[e] @ x[t]
                act = (4 * torch.tanh(hh[:H] / 4) * torch.sigmoid(hh[:H])) * (25 * torch.tanh(hh[H:] / 25))
                loss = loss + p[t, j] * torch.dot(dy[t], wd[e] @ act)
    loss.backward()
    g = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, H, mode="X")
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw_gu"], wgu.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dw_down"], wd.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dp"], p.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_mode_s_rounds_only_stored_tensors():
    cfg = TINYCFG
    inp, idx, gates, perm = _setup(cfg)
    f = expert_layer_fwd(inp["x"], inp["w_gu"], inp["w_down"], perm, cfg.H, mode="S")
    for name in ("h", "a", "y"):
        assert np.array_equal(f[name], bf16_round(f[name])), name
    b = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H,
                         mode="S", keep=True)
    assert np.array_equal(b["dx"], bf16_round(b["dx"]))
    assert np.array_equal(b["dh"], bf16_round(b["dh"]))
    assert not np.array_equal(b["dw_gu"], bf16_round(b["dw_gu"]))   # fp32-style gradient


def test_dw_columns_equals_full():
    cfg = LayerConfig("g", T=48, d=16, H=8, E=6, k=2, e_lo=0, E_loc=6)
    inp, idx, gates, perm = _setup(cfg)
    full = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H)
    for e in range(cfg.E_loc):
        cols = np.array([0, 3, 7])
        gu, dn = dw_columns(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, e, cols,
                            cfg.H)
        np.testing.assert_allclose(gu[:3], full["dw_gu"][e][cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(gu[3:], full["dw_gu"][e][cfg.H + cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dn, full["dw_down"][e][:, cols], rtol=1e-9, atol=1e-12)


def test_empty_expert_gets_zero_gradient():
    cfg = LayerConfig("g", T=16, d=8, H=4, E=40, k=2, e_lo=0, E_loc=40)
    inp, idx, gates, perm = _setup(cfg)
    counts = np.diff(perm["offsets"])
    assert np.any(counts == 0)
    g = expert_layer_bwd(inp["x"], inp["dy"], inp["w_gu"], inp["w_down"], perm, cfg.H)
    for e in np.nonzero(counts == 0)[0]:
        assert not np.any(g["dw_gu"][e]) and not np.any(g["dw_down"][e])


def test_unpermute_sum_brute_force():
    rng = np.random.default_rng(9)
    rows = rng.standard_normal((10, 5))
    slot_row = np.array([[0, -1], [3, 9], [-1, -1], [1, 2]], np.int32)
    w = rng.random(10)
    out = unpermute_sum(rows, slot_row, w)
    for t in range(4):
        ref = sum((w[r] * rows[r] for r in slot_row[t] if r >= 0), np.zeros(5))
        np.testing.assert_allclose(out[t], ref, rtol=1e-15)


def test_router_bwd_matches_autograd_and_fd():
    """Gradient through the softmax over the kept logits (top-k set fixed)."""
    rng = np.random.default_rng(10)
    L = rng.standard_normal((20, 10)).astype(np.float32)
    idx, gates = route_topk(L, 4)
    dp = rng.standard_normal((20, 4))
    ours = router_bwd(gates, dp)
    v = torch.tensor(np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), 1),
                     requires_grad=True)
    torch.softmax(v, dim=-1).backward(torch.from_numpy(dp))
    np.testing.assert_allclose(ours, v.grad.numpy(), rtol=1e-12, atol=1e-14)
    # finite differences through route_topk with perturbations that keep the top-k set
    eps = 1e-4
    for t in range(5):
        for j in range(4):
            Lp = L.astype(np.float64).copy()
            Lm = Lp.copy()
            Lp[t, idx[t, j]] += eps
            Lm[t, idx[t, j]] -= eps
            # evaluate the gates on the same index set
            vp = np.take_along_axis(Lp, idx.astype(np.int64), 1)[t]
            vm = np.take_along_axis(Lm, idx.astype(np.int64), 1)[t]
            sp = np.exp(vp - vp.max()); sp /= sp.sum()
            sm = np.exp(vm - vm.max()); sm /= sm.sum()
            assert ours[t, j] == pytest.approx(np.dot(dp[t], sp - sm) / (2 * eps), rel=1e-6,
                                               abs=1e-9)


# ----------------------------------------------------------------------------- page numbers
def test_page_numbers_fix_the_shapes():
    g = json.load(open(GOLDEN))
    rh = g["rows_and_hidden"]
    R = rh["tokens_per_gpu"] * rh["topk"]
    H = rh["H"]
    naive = rh["naive_saved_fp32_copies"] * R * H * 4
    saved = R * 2 * H * 2
    assert naive / 1e9 > rh["naive_hbm_lower_bound_GB"]              # ">100GB"
    assert saved * 6 == naive                                         # "1/6"
    assert abs((naive - saved) / 1e9 - rh["hbm_saved_approx_GB"]) < 10  # "about 90GB"
    assert abs(100 * (naive - saved) / 1e9 / rh["gpu_hbm_GB"] - rh["share_saved_approx_pct"]) < 4
    led = g["expert_ledger"]
    n = led["moe_layers"] * led["experts"] * np.prod(led["expert_shape"])
    assert round(n / 1e12, 2) == led["routed_params_T_approx"]
    pt = g["per_token_moe_values"]
    assert round(16 * 3584 / 1000) == pt["dispatch_copy_and_outputs_each_k"]
    ep = g["expert_parallel"]
    assert led["experts"] // ep["ep_size"] == ep["local_experts"]
    shard = LAYER_CONFIGS["shard"]
    assert (shard.d, shard.H, shard.E, shard.k, shard.E_loc) == (
        led["expert_shape"][1], led["expert_shape"][2], g["routing"]["experts"],
        g["routing"]["topk"], ep["local_experts"])
    sd = g["situ_defaults"]
    assert (shard.beta, shard.linear_beta) == (sd["beta"], sd["linear_beta"])


# ------------------------------------------------------------------ MXFP8 storage of h
def test_mx_e4m3_decode_matches_torch():
    """All 256 E4M3 codes decode as torch's float8_e4m3fn (OCP E4M3) does."""
    from oracle import mxfp8
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = mxfp8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_mx_e4m3_encode_matches_torch():
    """Round to nearest, ties to even, on fp32 inputs inside +-448: torch's cast is the
    independent reference (every representable value, every midpoint, random values)."""
    from oracle import mxfp8
    pos = mxfp8.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([pos, -pos, mids, -mids, rng.uniform(-448, 448, 50000),
                        rng.standard_normal(50000) * 1e-2]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mxfp8.e4m3_encode(x.astype(np.float64)), ref)


def test_mx_e4m3_saturation_and_zero_sign():
    from oracle import mxfp8
    got = mxfp8.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, -500.0, 0.0, -0.0, -1e-5]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80]


def test_mx_scale_exponent_rule():
    """X = floor(log2 amax) - 8, clamped to [-127, 127]; zero blocks take -127."""
    from oracle import mxfp8
    amax = np.array([1.0, 0.75, 448.0, 511.0, 512.0, 0.0, 2.0 ** -130, 3e38, 2.0 ** -119])
    assert list(mxfp8.block_scale_exp(amax)) == [-8, -9, 0, 0, 1, -127, -127, 119, -127]


def test_mx_roundtrip_bounds():
    """Per block: the largest magnitude lands in [256, 512) times 2^X; elements at or below
    448 * 2^X are within half a quantum (2^-4 relative for normals, 2^(X-10) absolute for
    subnormals); elements above saturate to 448 * 2^X; representable values are exact."""
    from oracle import mxfp8
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, size=(64, 1)))
    c, s = mxfp8.quantize(v)
    d = mxfp8.dequantize(c, s)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    sc = np.ldexp(1.0, X)
    amax = np.abs(v).reshape(64, 8, 32).max(-1).repeat(32, axis=1)
    assert np.all((amax / sc >= 256) & (amax / sc < 512))
    sat = np.abs(v) > 448 * sc
    assert np.all(np.abs(d[sat]) == 448 * sc[sat])
    ok = ~sat
    err = np.abs(d - v)[ok]
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(v[ok]), 2.0 ** -10 * sc[ok]) * (1 + 1e-12))
    exact = mxfp8.e4m3_decode(rng.integers(0, 127, size=(16, 64)).astype(np.uint8)) * 2.0 ** 5
    exact[:, ::32] = 448.0 * 2.0 ** 5                    # fixes each block's scale at X = 5
    assert np.array_equal(mxfp8.roundtrip(exact), exact)


def test_mx_layer_bwd_reduces_to_bf16_store_on_representable_h():
    """With weights that make every h exactly representable in MXFP8, the MXFP8 store
    changes nothing; with general weights the gradients move by at most a few percent."""
    from oracle import layer, mxfp8
    rng = np.random.default_rng(2)
    T, d, H, E, k = 48, 32, 64, 4, 2
    x = np.zeros((T, d)); x[np.arange(T), np.arange(T) % d] = 1.0          # one-hot rows
    w_gu = mxfp8.e4m3_decode(rng.integers(0, 127, size=(E, 2 * H, d)).astype(np.uint8))
    w_gu *= np.where(rng.random(w_gu.shape) < 0.5, -1.0, 1.0) * 2.0 ** -4
    w_gu[:, ::32, :] = 448 * 2.0 ** -4      # every 32-row block holds its amax: X = -4, exact
    w_down = rng.standard_normal((E, d, H)) * 0.1
    dy = rng.standard_normal((T, d))
    idx = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], 1).astype(np.int32)
    gates = np.full((T, k), 0.5)
    perm = oracle.permute(idx, gates, 0, E)
    # one-hot rows: h[r] is a column of w_gu[e], so each 32-column block of h is representable
    ref = layer.expert_layer_bwd(x, dy, w_gu, w_down, perm, H, mode="X")
    got = layer.expert_layer_bwd(x, dy, w_gu, w_down, perm, H, mode="X", h_store="mxfp8")
    h = np.concatenate([x[perm["row_token"][perm["offsets"][e]:perm["offsets"][e + 1]]] @ w_gu[e].T
                        for e in range(E)])
    assert np.array_equal(mxfp8.roundtrip(h), h)
    for key in ("dx", "dw_gu", "dw_down", "dp"):
        assert np.array_equal(got[key], ref[key]), key
    w2 = rng.standard_normal((E, 2 * H, d)) * 0.3
    x2 = rng.standard_normal((T, d))
    r2 = layer.expert_layer_bwd(x2, dy, w2, w_down, perm, H, mode="X")
    g2 = layer.expert_layer_bwd(x2, dy, w2, w_down, perm, H, mode="X", h_store="mxfp8")
    for key in ("dx", "dw_gu", "dw_down", "dp"):
        e = np.max(np.abs(g2[key] - r2[key])) / np.max(np.abs(r2[key]))
        assert 0 < e < 0.1, (key, e)


# ------------------------------------------------------------------ W4A8 (MXFP4 weights)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]     # OCP MX v1.0, FP4 E2M1 magnitudes


def _e2m1_nearest(v):
    """Brute force: the E2M1 code nearest to v (|v| capped at 6), ties to the even code."""
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(a - E2M1_TABLE[c]), c % 2))
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def _e4m3_nearest(v):
    """Brute force over the 127 finite E4M3 magnitudes, ties to the even code, saturating."""
    mags = [(1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7) if c >> 3 else (c & 7) * 2.0 ** -9
            for c in range(127)]
    a = min(abs(v), 448.0)
    best = min(range(127), key=lambda c: (abs(a - mags[c]), c % 2))
    return mags[best] * (-1.0 if math.copysign(1.0, v) < 0 else 1.0)


def _mx_block_scalar(vals, emax, nearest_value):
    """One MX block quantized with scalar loops: X from math.frexp of the largest magnitude."""
    amax = max(abs(v) for v in vals)
    X = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - emax))
    return [nearest_value(v / 2.0 ** X) * 2.0 ** X for v in vals]


def test_mx4_e2m1_decode_table():
    """The 16 codes decode to the format's table, sign in bit 3 (code 8 is -0)."""
    from oracle import mxfp4
    got = mxfp4.e2m1_decode(np.arange(16))
    assert list(got[:8]) == E2M1_TABLE
    assert list(got[8:]) == [-v for v in E2M1_TABLE]
    assert math.copysign(1.0, got[8]) == -1.0


def test_mx4_e2m1_encode_brute_force():
    """Vectorised encoder = scalar brute force on every value, every midpoint, the
    saturation band, signed zeros and random values."""
    from oracle import mxfp4
    tab = np.array(E2M1_TABLE)
    mids = (tab[1:] + tab[:-1]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([tab, -tab, mids, -mids, [6.5, 7.0, 7.99, 100.0, -9.0, 0.0, -0.0, -0.1],
                        rng.uniform(-8, 8, 4000), rng.standard_normal(1000) * 0.3])
    got = mxfp4.e2m1_encode(x)
    ref = np.array([_e2m1_nearest(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)
    # ties to even: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    assert list(mxfp4.e2m1_decode(mxfp4.e2m1_encode(mids))) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_mx4_scale_exponent_rule():
    """X = floor(log2 amax) - 2, clamped to [-127, 127]; zero blocks take -127."""
    from oracle import mxfp4
    amax = np.array([1.0, 4.0, 7.99, 8.0, 0.75, 0.0, 2.0 ** -130, 3e38, 2.0 ** -124])
    assert list(mxfp4.block_scale_exp(amax)) == [-2, 0, 0, 1, -3, -127, -127, 125, -126]


def test_mx4_packing_layout():
    """Element 2j in the low nibble of byte j, 2j+1 in the high nibble; unpack inverts."""
    from oracle import mxfp4
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    assert list(mxfp4.pack(codes)[0]) == [0x21, 0x43, 0x0F]
    assert np.array_equal(mxfp4.unpack(mxfp4.pack(codes)), codes)
    v = np.zeros((1, 32))
    v[0, 0], v[0, 1] = 6.0, -0.5                          # X = 0: codes 7 and 9
    c, s = mxfp4.quantize(v)
    assert c[0, 0] == 0x97 and s[0, 0] == 127 and np.all(c[0, 1:] == 0)


def test_mx4_roundtrip_bounds():
    """Per block the largest magnitude lands in [4, 8) times 2^X; elements above 6 * 2^X
    saturate; the rest are within half a step (2^-2 relative at or above 2^X, 2^(X-2)
    absolute below); representable blocks come back exactly."""
    from oracle import mxfp4
    rng = np.random.default_rng(6)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, size=(64, 1)))
    c, s = mxfp4.quantize(v)
    d = mxfp4.dequantize(c, s)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    sc = np.ldexp(1.0, X)
    amax = np.abs(v).reshape(64, 8, 32).max(-1).repeat(32, axis=1)
    assert np.all((amax / sc >= 4) & (amax / sc < 8))
    sat = np.abs(v) > 6 * sc
    assert np.all(np.abs(d[sat]) == 6 * sc[sat])
    ok = ~sat
    err = np.abs(d - v)[ok]
    assert np.all(err <= np.maximum(2.0 ** -2 * np.abs(v[ok]), 2.0 ** -2 * sc[ok]) * (1 + 1e-12))
    exact = mxfp4.e2m1_decode(rng.integers(0, 16, size=(16, 64))) * 2.0 ** -3
    exact[:, ::32] = 6.0 * 2.0 ** -3                     # fixes each block's scale at X = -3
    assert np.array_equal(mxfp4.roundtrip(exact), exact)


def test_w4a8_forward_brute_force_tiny():
    """The W4A8 forward against scalar loops over tokens, slots, outputs and reductions,
    with scalar MX quantizers written from the formats (brute-force nearest codes)."""
    from oracle import w4a8
    from oracle.situ import situ_glu_fwd
    rng = np.random.default_rng(7)
    T, d, H, E, k = 5, 64, 32, 3, 2
    x = rng.standard_normal((T, d)) * 0.7
    w_gu = rng.standard_normal((E, 2 * H, d)) * 0.2
    w_down = rng.standard_normal((E, d, H)) * 0.2
    idx = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]], np.int32)
    gates = rng.uniform(0.2, 0.8, size=(T, k))
    perm = oracle.permute(idx, gates, 0, E)
    got = w4a8.expert_layer_fwd_w4a8(x, w_gu, w_down, perm, H)

    def q8_row(row):
        return sum((_mx_block_scalar(list(row[b:b + 32]), 8, _e4m3_nearest)
                    for b in range(0, len(row), 32)), [])

    def q4_row(row):
        nearest = lambda v: math.copysign(E2M1_TABLE[_e2m1_nearest(v) & 7], 1.0) * (
            -1.0 if _e2m1_nearest(v) & 8 else 1.0)
        return sum((_mx_block_scalar(list(row[b:b + 32]), 2, nearest)
                    for b in range(0, len(row), 32)), [])

    y = np.zeros((T, d))
    for t in range(T):
        x8 = q8_row(x[t])
        for j in range(k):
            e = int(idx[t, j])
            h = [sum(x8[c] * q4 for c, q4 in enumerate(q4_row(w_gu[e, n]))) for n in range(2 * H)]
            h = bf16_round(np.array(h))
            a = bf16_round(situ_glu_fwd(h[None, :], H)[0])
            a8 = q8_row(a)
            for n in range(d):
                w4 = q4_row(w_down[e, n])
                y[t, n] += gates[t, j] * sum(a8[c] * w4[c] for c in range(H))
    assert np.allclose(got["y"], bf16_round(y), rtol=0, atol=1e-12 * np.max(np.abs(y)))


def test_w4a8_lossless_inputs_reduce_to_bf16_layer():
    """With x and the weights exactly representable in MXFP8 / MXFP4, the W4A8 forward has
    the bf16 layer's h and a bit for bit, and its y differs from the bf16 layer's only by
    the MXFP8 rounding of a: |dy| <= sum_e p sum_c |a8 - a| |w_down|, each |a8 - a| within
    the E4M3 bound (half a step, or the clip to 448 * 2^X), plus one bf16 step of each y."""
    from oracle import layer, mxfp4, mxfp8, w4a8
    rng = np.random.default_rng(8)
    T, d, H, E, k = 40, 64, 64, 4, 2
    x = mxfp8.e4m3_decode(rng.integers(0, 127, size=(T, d)).astype(np.uint8)) * 2.0 ** -8
    x *= np.where(rng.random(x.shape) < 0.5, -1.0, 1.0)
    x[:, ::32] = 448 * 2.0 ** -8                          # every block's scale fixed: exact
    w_gu = mxfp4.e2m1_decode(rng.integers(0, 16, size=(E, 2 * H, d))) * 2.0 ** -4
    w_gu[:, :, ::32] = 6.0 * 2.0 ** -4
    w_down = mxfp4.e2m1_decode(rng.integers(0, 16, size=(E, d, H))) * 2.0 ** -5
    w_down[:, :, ::32] = -6.0 * 2.0 ** -5
    assert np.array_equal(mxfp8.roundtrip(x), x) and np.array_equal(mxfp4.roundtrip(w_gu), w_gu)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.uniform(0.1, 0.9, size=(T, k))
    perm = oracle.permute(idx, gates, 0, E)
    got = w4a8.expert_layer_fwd_w4a8(x, w_gu, w_down, perm, H)
    ref = layer.expert_layer_fwd(x, w_gu, w_down, perm, H, mode="S")
    assert np.array_equal(got["h"], ref["h"]) and np.array_equal(got["a"], ref["a"])
    a8 = mxfp8.dequantize(got["a_codes"], got["a_scales"])
    X = (got["a_scales"].astype(np.int64) - 127).repeat(32, axis=1)
    sc = np.ldexp(1.0, X)
    sat = np.abs(ref["a"]) > 448 * sc                   # clipped to 448 * 2^X
    step = np.where(sat, np.abs(ref["a"]) - 448 * sc,
                    np.maximum(2.0 ** -4 * np.abs(ref["a"]), 2.0 ** -10 * sc))
    assert np.all(np.abs(a8 - ref["a"]) <= step)
    assert np.any(a8 != ref["a"])                          # a itself is generally not representable
    bound = np.zeros((T, d))
    off = perm["offsets"]
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        bound[perm["row_token"][r0:r1]] += perm["row_gate"][r0:r1, None] * (
            step[r0:r1] @ np.abs(w_down[e]).T)
    dy = np.abs(got["y"] - ref["y"])
    assert np.all(dy <= bound + 2.0 ** -7 * np.abs(ref["y"]) + 1e-30)
    assert np.max(dy) > 0
