"""The allocation-free down GEMM + combine (moe_grouped_gemm_down_combine_noalloc), called
through the C ABI, against moe_grouped_gemm_down_combine with a caller workspace: bit-identical
y on two calls in a row, the second smaller, and the refusal of row counts beyond its static
scratch. Callers that cannot allocate are what this entry point is for."""
import sys

import numpy as np
import pytest
import torch

from moe_inputs import LayerConfig, layer_inputs

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


# first call: R = 65536 rows of d = 1024, so its fp32 rows (256 MiB) need four 256-column
# windows of the 64 MiB scratch; second call: 512 rows of d = 256, one window
CASES = [LayerConfig("noalloc_big", T=8192, d=1024, H=256, E=8, k=8, e_lo=0, E_loc=8),
         LayerConfig("noalloc_small", T=256, d=256, H=128, E=8, k=2, e_lo=0, E_loc=8)]


def run_both(m, cfg, seed):
    inp = layer_inputs(cfg, seed=seed)
    x, w_gu, w_down = dev_bf16(inp["x"]), dev_bf16(inp["w_gu"]), dev_bf16(inp["w_down"])
    logits = torch.from_numpy(inp["logits"]).cuda()
    R_cap = cfg.T * cfg.k
    idx, gates = m.moe_route_topk(logits, cfg.k)
    perm = m.moe_permute(idx, gates, cfg.e_lo, cfg.E_loc, R_cap)
    _, a = m.moe_grouped_gemm_gate_up(x, perm["row_token"], perm["offsets"], w_gu, R_cap)
    y_ws = m.moe_grouped_gemm_down_combine(a, perm["offsets"], perm["row_gate"],
                                           perm["slot_row"], w_down, R_cap)
    y_na = torch.full_like(y_ws, float("nan"))
    m._lib.moe_grouped_gemm_down_combine_noalloc(a, perm["offsets"], perm["row_gate"],
                                                 perm["slot_row"], w_down, R_cap, y=y_na)
    torch.cuda.synchronize()
    R = int(perm["offsets"][-1].item())
    return y_ws, y_na, R


def test_noalloc_matches_workspace_call_twice(moe):
    for i, cfg in enumerate(CASES):
        say(f"noalloc call {i + 1}: {cfg.name} T={cfg.T} d={cfg.d} H={cfg.H}")
        y_ws, y_na, R = run_both(moe, cfg, seed=7 + i)
        assert R > 0 and bool(y_ws.abs().sum() > 0)
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), cfg.name
        say(f"noalloc call {i + 1}: R={R} identical")
    assert R == CASES[1].T * CASES[1].k                 # every route of the second call local


def test_noalloc_refuses_rows_beyond_scratch(moe):
    """65536 rows of one 256-column window fill the 64 MiB scratch; one more row is refused
    before anything is launched (the buffers are never touched)."""
    T, k, E_loc, d, H = 40000, 2, 4, 512, 128
    a = torch.zeros((65537, H), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(E_loc + 1, dtype=torch.int32, device="cuda")
    gate = torch.zeros(65537, dtype=torch.float32, device="cuda")
    slot = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((E_loc, d, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe._lib.moe_grouped_gemm_down_combine_noalloc(a, off, gate, slot, w, 65537)
    assert e.value.status == 4
