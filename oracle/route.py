"""Top-k routing with a softmax over the kept logits, fp64 (test infrastructure only).

Definition ("Inside Kimi K3", "Idea One", routing snippet): the router scores every expert,
the k highest scores are kept, and the gates are a softmax over those k values only; the
token's output is the gate-weighted sum of the chosen experts' outputs. The second page
("Kimi K3 ... Memory", "MoE 反向") calls these gates the router-normalised probabilities p_e.

Readings where the pages are silent (the snippet's top-k fixes neither):
  * order: value descending, equal values broken by the lower expert index; slot j of a
    token holds its j-th pick in that order (-0.0 and +0.0 compare equal);
  * logits must be finite (asserted);
  * softmax subtracts the maximum (the first pick) before exponentiating.
The selection is decided on the float32 logits themselves (widening to fp64 is exact and
keeps every comparison), so it is the same decision the GPU takes.
"""
import numpy as np


def route_topk(logits, k):
    """Return (idx int32 [T,k], gates fp64 [T,k]) for float32 logits [T, E]."""
    L = np.asarray(logits, dtype=np.float64)
    assert L.ndim == 2 and 1 <= k <= L.shape[1]
    assert np.all(np.isfinite(L)), "router logits must be finite"
    T, E = L.shape
    col = np.broadcast_to(np.arange(E), (T, E))
    # primary key: -logit (descending logit); secondary: expert index ascending.
    order = np.lexsort((col, -L), axis=-1)
    idx = order[:, :k].astype(np.int32)
    vals = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    m = vals[:, :1]
    w = np.exp(vals - m)
    gates = w / w.sum(axis=1, keepdims=True)
    return idx, gates
