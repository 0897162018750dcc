"""Routed-expert layer forward and backward in fp64 (test infrastructure only).

Definition ("Kimi K3 ... Memory", section "MoE 反向", the expert forward equation): for a
token routed to expert e with input x_e,
    a_e = SiTU(W_gate_e x_e, W_up_e x_e),   o_e = W_down_e a_e,   y = sum_{e in top-k} p_e o_e,
with a_e the expert's activation ("act_output") and p_e the router-normalised probability.
Backward with the loss L = <dy, y> (so dL/dy = dy), same section, the p-gradient rewrite:
    dL/dp_e = <dL/dy, o_e> = <W_down_e^T dL/dy, a_e>,   dL/da_e = p_e W_down_e^T dL/dy,
so o_e is never needed; the pre-activation h = [W_gate x ; W_up x] is the one saved tensor
("Frontier-scale RL with Kimi K3", "Streaming activations"), tanh and sigmoid are
recomputed from it, and the dispatch is redone from the pre-dispatch input ("MoE 反向",
second saving).

Readings (the pages are silent): weight gradients are full fp32-style overwrites
(the second page keeps gradients in FP32); y, dx, dp are this GPU's partial sums over its
local experts, zero for non-local routes; an expert with no rows gets a zero gradient.

`mode="S"` rounds to bf16 where the layer stores bf16 (h, a, dh, y, dx); `mode="X"` is exact.
"""
import numpy as np

from . import mxfp8
from .bf16 import bf16_round, bf16_widen
from .situ import situ_glu_fwd, situ_glu_bwd


def _f64(a):
    a = np.asarray(a)
    return bf16_widen(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _maybe_round(v, mode):
    return bf16_round(v) if mode == "S" else v


def expert_layer_fwd(x, w_gu, w_down, perm, H, beta=4.0, linear_beta=25.0, mode="S",
                     keep=True):
    """Grouped forward, one local expert at a time.

    x [T,d] (bf16 bits or float), w_gu [E_loc,2H,d], w_down [E_loc,d,H], perm from
    `permute`. Returns dict(y [T,d], y_sum [T,d], h [R,2H], a [R,H]) (h, a only when
    keep=True); y_sum is the fp64 sum over routes before y's own rounding (y = y_sum in mode
    "X", y = bf16(y_sum) in mode "S").
    """
    xf = _f64(x)
    T, d = xf.shape
    off, row_token, row_gate = perm["offsets"], perm["row_token"], perm["row_gate"]
    E_loc = len(off) - 1
    R = int(off[-1])
    y = np.zeros((T, d))
    h_all = np.zeros((R, 2 * H)) if keep else None
    a_all = np.zeros((R, H)) if keep else None
    for e in range(E_loc):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        tok = row_token[r0:r1]
        X = xf[tok]
        h = _maybe_round(X @ _f64(w_gu[e]).T, mode)
        a = _maybe_round(situ_glu_fwd(h, H, beta, linear_beta), mode)
        o = a @ _f64(w_down[e]).T
        y[tok] += row_gate[r0:r1, None] * o      # a token occurs at most once per expert
        if keep:
            h_all[r0:r1] = h
            a_all[r0:r1] = a
    return dict(y=_maybe_round(y, mode), y_sum=y, h=h_all, a=a_all)


def _stored_h(h, h_store):
    """The pre-activation the backward reads: as saved in bf16, or after MXFP8 storage."""
    return mxfp8.roundtrip(h) if h_store == "mxfp8" else h


def expert_layer_bwd(x, dy, w_gu, w_down, perm, H, beta=4.0, linear_beta=25.0, mode="S",
                     keep=False, h_store="bf16"):
    """Grouped backward with dL/dy = dy; recomputes h from x (the re-dispatch).

    h_store="mxfp8": the saved h went through MXFP8 storage (oracle.mxfp8), so the
    activation and its gradient are recomputed from the stored value.
    Returns dict(dx [T,d], dx_sum [T,d], dw_gu [E_loc,2H,d], dw_down [E_loc,d,H], dp [T,k],
    dp_rows [R]) and dh [R,2H] when keep=True; dx_sum is the fp64 sum over routes before dx's
    own rounding.
    """
    xf = _f64(x)
    dyf = _f64(dy)
    T, d = xf.shape
    off, row_token, row_gate = perm["offsets"], perm["row_token"], perm["row_gate"]
    slot_row = perm["slot_row"]
    E_loc = len(off) - 1
    R = int(off[-1])
    dx = np.zeros((T, d))
    dw_gu = np.zeros((E_loc, 2 * H, d))
    dw_down = np.zeros((E_loc, d, H))
    dp_rows = np.zeros(R)
    dh_all = np.zeros((R, 2 * H)) if keep else None
    for e in range(E_loc):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        tok = row_token[r0:r1]
        p = row_gate[r0:r1, None]
        X, dY = xf[tok], dyf[tok]
        Wgu, Wd = _f64(w_gu[e]), _f64(w_down[e])
        h = _stored_h(_maybe_round(X @ Wgu.T, mode), h_store)
        a = _maybe_round(situ_glu_fwd(h, H, beta, linear_beta), mode)
        G = dY @ Wd                                   # W_down^T dy, per row [n, H]
        dp_rows[r0:r1] = np.sum(G * a, axis=1)        # <W_down^T dy, a>
        dh = _maybe_round(situ_glu_bwd(h, p * G, H, beta, linear_beta), mode)
        dw_down[e] = (p * dY).T @ a
        dw_gu[e] = dh.T @ X
        dx[tok] += dh @ Wgu
        if keep:
            dh_all[r0:r1] = dh
    dp = np.where(slot_row >= 0, dp_rows[np.maximum(slot_row, 0)] if R else 0.0, 0.0)
    return dict(dx=_maybe_round(dx, mode), dx_sum=dx, dw_gu=dw_gu, dw_down=dw_down, dp=dp,
                dp_rows=dp_rows, dh=dh_all)


def _token_expert(xt, Wgu, Wd, H, beta, linear_beta, mode):
    h = _maybe_round(Wgu @ xt, mode)
    a = _maybe_round(situ_glu_fwd(h, H, beta, linear_beta), mode)
    return h, a, Wd @ a


def token_layer_fwd(x_t, idx_t, gates_t, w_gu, w_down, e_lo, H, beta=4.0, linear_beta=25.0,
                    mode="S"):
    """One token, written as the routing snippet's loop: y = sum_i gate_i expert_{idx_i}(x).

    Only local experts (e_lo <= idx < e_lo + E_loc) contribute. Returns y [d] fp64.
    """
    xt = _f64(x_t)
    E_loc = len(w_gu)
    y = np.zeros_like(xt)
    for j in range(len(idx_t)):
        e = int(idx_t[j]) - e_lo
        if 0 <= e < E_loc:
            _, _, o = _token_expert(xt, _f64(w_gu[e]), _f64(w_down[e]), H, beta, linear_beta,
                                    mode)
            y = y + gates_t[j] * o
    return _maybe_round(y, mode)


def token_layer_bwd(x_t, dy_t, idx_t, gates_t, w_gu, w_down, e_lo, H, beta=4.0,
                    linear_beta=25.0, mode="S"):
    """One token's dx [d] and dp [k] (zero for non-local slots), vector by vector."""
    xt, dyt = _f64(x_t), _f64(dy_t)
    E_loc = len(w_gu)
    dx = np.zeros_like(xt)
    dp = np.zeros(len(idx_t))
    for j in range(len(idx_t)):
        e = int(idx_t[j]) - e_lo
        if not 0 <= e < E_loc:
            continue
        Wgu, Wd = _f64(w_gu[e]), _f64(w_down[e])
        h, a, _ = _token_expert(xt, Wgu, Wd, H, beta, linear_beta, mode)
        G = Wd.T @ dyt
        dp[j] = G @ a
        dh = _maybe_round(situ_glu_bwd(h, gates_t[j] * G, H, beta, linear_beta), mode)
        dx = dx + Wgu.T @ dh
    return _maybe_round(dx, mode), dp


def dw_columns(x, dy, w_gu, w_down, perm, e, cols, H, beta=4.0, linear_beta=25.0, mode="S",
               h_store="bf16"):
    """Weight gradients of local expert e restricted to intermediate columns `cols`.

    Returns (dw_gu_rows [2*len(cols), d] = rows cols then H+cols of dW_gu[e],
             dw_down_cols [d, len(cols)] = columns cols of dW_down[e]).
    SiTU-GLU is elementwise, so column j of h, a, dh depends only on columns j and j+H.
    With h_store="mxfp8" the columns must cover whole 32-column blocks (a block shares one
    scale), in ascending order.
    """
    cols = np.asarray(cols, dtype=np.int64)
    if h_store == "mxfp8":
        assert len(cols) % mxfp8.BLOCK == 0 and np.all(cols.reshape(-1, mxfp8.BLOCK) ==
                                                      cols.reshape(-1, mxfp8.BLOCK)[:, :1] +
                                                      np.arange(mxfp8.BLOCK))
        assert np.all(cols.reshape(-1, mxfp8.BLOCK)[:, 0] % mxfp8.BLOCK == 0)
    off, row_token, row_gate = perm["offsets"], perm["row_token"], perm["row_gate"]
    r0, r1 = int(off[e]), int(off[e + 1])
    d = w_gu.shape[2]
    if r1 == r0:
        return np.zeros((2 * len(cols), d)), np.zeros((d, len(cols)))
    tok = row_token[r0:r1]
    X = _f64(np.asarray(x)[tok])
    dY = _f64(np.asarray(dy)[tok])
    p = row_gate[r0:r1, None]
    Wsel = _f64(np.concatenate([w_gu[e][cols], w_gu[e][H + cols]], axis=0))   # [2c, d]
    Wd = _f64(w_down[e][:, cols])                                              # [d, c]
    c = len(cols)
    h = _stored_h(_maybe_round(X @ Wsel.T, mode), h_store)                     # [n, 2c]
    a = _maybe_round(situ_glu_fwd(h, c, beta, linear_beta), mode)
    G = dY @ Wd
    dh = _maybe_round(situ_glu_bwd(h, p * G, c, beta, linear_beta), mode)
    return dh.T @ X, (p * dY).T @ a


def unpermute_sum(rows, slot_row, row_weight=None):
    """out[t] = sum over local slots j of w(row) * rows[slot_row[t, j]] (fp64)."""
    rf = _f64(rows)
    slot_row = np.asarray(slot_row)
    T, k = slot_row.shape
    out = np.zeros((T, rf.shape[1]))
    for j in range(k):
        r = slot_row[:, j]
        m = r >= 0
        w = 1.0 if row_weight is None else np.asarray(row_weight, np.float64)[r[m]][:, None]
        out[m] += w * rf[r[m]]
    return out


def router_bwd(gates, dp):
    """Gradient of the loss w.r.t. the k kept logits through the softmax over them.

    With p = softmax(v) over the kept values v: dL/dv_j = p_j (dL/dp_j - sum_i p_i dL/dp_i).
    Logits that were not kept do not reach the output and get no gradient.
    """
    p = np.asarray(gates, np.float64)
    g = np.asarray(dp, np.float64)
    return p * (g - np.sum(p * g, axis=-1, keepdims=True))
