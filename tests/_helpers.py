"""Shared plumbing for the tests: host<->device copies, error metrics, oracle sub-problems."""
import numpy as np

import oracle


def rel_err(gpu, ref):
    """max|gpu - ref| / max|ref|; when ref is all zero, max|gpu| (which must then be 0)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    m = np.max(np.abs(ref))
    if m == 0:
        return float(np.max(np.abs(gpu)))
    return float(np.max(np.abs(gpu - ref)) / m)


BF16_TOL = 1e-2      # bf16 outputs (h, a, y, dx, dh) and the fp32 weight gradients
FP32_TOL = 2e-3      # fp32 gates and dp


def sub_perm(perm, tokens):
    """Restrict a permutation to the rows of `tokens` (keeps expert grouping and order).

    Rows are independent in the layer, so the oracle run on this sub-permutation gives the
    exact outputs of those tokens. Returns (sub, rows) where rows are the full-perm rows kept.
    """
    tokens = np.asarray(sorted(set(int(t) for t in tokens)))
    keep = np.isin(perm["row_token"][: perm["R"]], tokens)
    rows = np.nonzero(keep)[0]
    off = perm["offsets"]
    E_loc = len(off) - 1
    counts = np.array([np.sum(keep[off[e]:off[e + 1]]) for e in range(E_loc)])
    new_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_map = -np.ones(perm["R"] + 1, np.int64)
    row_map[rows] = np.arange(len(rows))
    sr = perm["slot_row"].copy()
    T = sr.shape[0]
    mask_tok = np.zeros(T, bool)
    mask_tok[tokens] = True
    new_sr = np.where((sr >= 0) & mask_tok[:, None], row_map[np.maximum(sr, 0)], -1).astype(np.int32)
    sub = dict(offsets=new_off, row_token=perm["row_token"][rows], row_gate=perm["row_gate"][rows],
               slot_row=new_sr, R=len(rows))
    return sub, rows


def oracle_route_perm(inp, cfg):
    idx, gates = oracle.route_topk(inp["logits"], cfg.k)
    perm = oracle.permute(idx, gates, cfg.e_lo, cfg.E_loc)
    return idx, gates, perm
