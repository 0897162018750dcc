"""Dispatch metadata: local-route filter and stable sort by expert (test infrastructure only).

The grouped GEMM runs over a copy of the tokens arranged by expert ("Kimi K3 ... Memory",
"MoE 反向", second saving: only the pre-dispatch input is kept and the dispatch is redone in
the backward). On one GPU the dispatch is this permutation.

Reading: keep the routes whose expert lies in [e_lo, e_lo + E_loc); rows are grouped by
local expert in increasing expert order, and within an expert by increasing token index.
A token picks an expert at most once, so this order is unique. Gates of the kept routes are
not renormalised.
"""
import numpy as np


def permute(idx, gates, e_lo, E_loc):
    """Return dict(offsets [E_loc+1], row_token [R], row_gate [R], slot_row [T,k], R).

    slot_row[t, j] is the row of route (t, j), or -1 when that expert is not local.
    """
    idx = np.asarray(idx)
    gates = np.asarray(gates, dtype=np.float64)
    T, k = idx.shape
    for t in range(T) if T * k <= 4096 else []:
        assert len(set(idx[t].tolist())) == k, "a token must pick distinct experts"
    slot_row = np.full((T, k), -1, dtype=np.int32)
    offsets = np.zeros(E_loc + 1, dtype=np.int64)
    tok_parts, gate_parts = [], []
    base = 0
    for e in range(E_loc):
        t_sel, j_sel = np.nonzero(idx == e_lo + e)     # row-major: ascending token
        assert np.all(np.diff(t_sel) > 0), "a token must pick an expert at most once"
        n = t_sel.size
        slot_row[t_sel, j_sel] = base + np.arange(n, dtype=np.int32)
        tok_parts.append(t_sel.astype(np.int32))
        gate_parts.append(gates[t_sel, j_sel])
        base += n
        offsets[e + 1] = base
    row_token = np.concatenate(tok_parts) if tok_parts else np.zeros(0, np.int32)
    row_gate = np.concatenate(gate_parts) if gate_parts else np.zeros(0)
    return dict(offsets=offsets.astype(np.int32), row_token=row_token, row_gate=row_gate,
                slot_row=slot_row, R=int(base))
