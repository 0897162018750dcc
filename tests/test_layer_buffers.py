"""Host-side sizing of LayerBuffers (CPU: buffers on torch's meta device, so nothing is
allocated; the sizes come from the library's host-only workspace queries)."""
import pytest

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_expert_top_amd")


def shape(T, E, k, E_loc, d, H):
    return moe.LayerShape(T=T, E=E, k=k, e_lo=0, E_loc=E_loc, d=d, H=H, beta=4.0,
                          linear_beta=25.0)


def test_backward_passes_keep_the_backward_within_the_forward():
    # large context: one dX window would need 42.2 GB against the forward's 32.2 GB, so the
    # combine splits into two 1792-column windows (30.9 GB)
    s = shape(98304, 28, 16, 28, 3584, 3072)
    b = moe.LayerBuffers(s, R_cap=1572864, device="meta")
    assert b.bwd_passes == 2
    fwd = b.a.numel() * 2 + b.ws_down.numel()
    assert b.ws_bwd.numel() <= fwd and b.arena.numel() == max(fwd, b.ws_bwd.numel())
    one = moe.workspace_size_passes(moe.MOE_WS_EXPERT_BWD, 1, T=s.T, E_loc=s.E_loc, k=s.k,
                                    d=s.d, H=s.H, R_cap=1572864)
    assert one > fwd + (1 << 30)


def test_backward_passes_stay_at_one_below_a_gib():
    # shard: splitting would save 0.1 GB, below the 1 GiB threshold
    b = moe.LayerBuffers(shape(32768, 896, 16, 28, 3584, 3072), R_cap=16456, device="meta")
    assert b.bwd_passes == 1


def test_backward_passes_explicit_and_unaliased():
    s = shape(98304, 28, 16, 28, 3584, 3072)
    assert moe.LayerBuffers(s, R_cap=1572864, device="meta", bwd_passes=3).bwd_passes == 3
    b = moe.LayerBuffers(s, R_cap=1572864, device="meta", alias=False)
    assert b.bwd_passes == 1 and b.arena is None
