"""Seeded synthetic inputs for the routed-expert layer and the standalone SiTU-GLU op.

This module is shared by the fp64 oracle tests, the GPU parity tests and the benchmark.
It draws random numbers and stores them in the dtypes the layer consumes; it holds none of
the layer's own arithmetic (no routing, no activation, no contraction).

Workload shapes follow the pages:
  * "Kimi K3 ... Memory" (blog.javazero.top), parameter ledger: routed experts of shape
    3 x 3584 x 3072 (latent d = 3584, expert intermediate H = 3072), 896 experts;
    ledger sliders: expert-parallel size 32, hence 896 / 32 = 28 experts per GPU.
  * "Inside Kimi K3" (dramitakapoor.com), "Idea One" routing snippet: top-16 of 896 scores.
  * "Frontier-scale RL with Kimi K3" (appliedcompute.com), "Streaming activations":
    R = tokens per GPU x 16 rows, H = 3072, on the order of 100k tokens per GPU.

Recipe (the pages name no RNG, so this choice is ours): numpy PCG64 seeded with 0, values
drawn as float32 standard normals and scaled in float32, bf16 tensors rounded from float32
with round-to-nearest-even and returned as raw uint16 bit patterns. Draw order for the layer
is logits, x, W_gate, W_up, W_down, dy; only the local experts' weights are drawn. Weight
std is fan_in ** -0.5 (d for W_gate and W_up, H for W_down).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerConfig", "LAYER_CONFIGS", "SITU_CONFIGS", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "layer_inputs", "situ_inputs", "zipf_bias",
]


@dataclass(frozen=True)
class LayerConfig:
    """Shapes of one routed-expert layer call on one GPU's share of experts."""
    name: str
    T: int          # tokens on this GPU
    d: int          # latent (expert input/output) dimension
    H: int          # expert intermediate dimension
    E: int          # experts the router scores
    k: int          # experts kept per token
    e_lo: int = 0   # first local expert
    E_loc: int = 0  # number of local experts
    bias: str | None = None   # "zipf": logits + 2 ln(1/(e+1))
    beta: float = 4.0
    linear_beta: float = 25.0
    note: str = field(default="", compare=False)

    @property
    def local_range(self):
        return range(self.e_lo, self.e_lo + self.E_loc)


LAYER_CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, d=128, H=64, E=8, k=2, e_lo=0, E_loc=8,
                        note="256 tokens, d=128, H=64, 8 experts, top-2"),
    "shard": LayerConfig("shard", T=32768, d=3584, H=3072, E=896, k=16, e_lo=0, E_loc=28,
                         note="one expert-parallel rank: 32768 tokens, top-16 of 896, local experts 0..27"),
    "skew": LayerConfig("skew", T=32768, d=3584, H=3072, E=896, k=16, e_lo=0, E_loc=28,
                        bias="zipf", note="shard shapes, logits + 2 ln(1/(e+1)), local experts 0..27"),
    "skew_mid": LayerConfig("skew_mid", T=32768, d=3584, H=3072, E=896, k=16, e_lo=28, E_loc=28,
                            bias="zipf", note="skewed logits, local experts 28..55"),
    "skew_tail": LayerConfig("skew_tail", T=32768, d=3584, H=3072, E=896, k=16, e_lo=84, E_loc=28,
                             bias="zipf", note="skewed logits, local experts 84..111 (some empty)"),
    "large": LayerConfig("large", T=98304, d=3584, H=3072, E=28, k=16, e_lo=0, E_loc=28,
                         note="98304 tokens already dispatched, 16 of 28 local experts"),
}

SITU_CONFIGS = {
    # Standalone streaming SiTU-GLU: h bf16 [131072, 6144] ~ N(0, 3^2), da bf16 [131072, 3072] ~ N(0,1)
    "situ": dict(R=131072, H=3072, h_std=3.0),
    "situ_small": dict(R=1000, H=192, h_std=3.0),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporaries on multi-GB arrays
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 26
    for s in range(0, flat_u.size, step):
        x = flat_u[s:s + step]
        lsb = (x >> np.uint32(16)) & np.uint32(1)
        r = (x + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        nan = (x & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = np.where(nan, (x >> np.uint32(16)) | np.uint32(0x40), r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(E: int) -> np.ndarray:
    """Per-expert logit bias b_e = 2 ln(1/(e+1)), e = 0..E-1, as float32."""
    e = np.arange(E, dtype=np.float64)
    return (2.0 * np.log(1.0 / (e + 1.0))).astype(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def layer_inputs(cfg: LayerConfig | str, seed: int = 0, T: int | None = None) -> dict:
    """Draw (logits, x, w_gu, w_down, dy) for one layer call.

    Returns a dict of numpy arrays:
      logits  float32 [T, E]
      x       uint16 (bf16 bits) [T, d]
      w_gu    uint16 [E_loc, 2H, d]   rows 0..H-1 are W_gate, rows H..2H-1 are W_up
      w_down  uint16 [E_loc, d, H]
      dy      uint16 [T, d]
    `T` overrides the token count (same recipe, fewer tokens) for reduced-size parity runs.
    """
    if isinstance(cfg, str):
        cfg = LAYER_CONFIGS[cfg]
    T = cfg.T if T is None else T
    rng = np.random.default_rng(seed)
    logits = _normal(rng, (T, cfg.E), 1.0)
    if cfg.bias == "zipf":
        logits += zipf_bias(cfg.E)[None, :]
    x = f32_to_bf16_bits(_normal(rng, (T, cfg.d), 1.0))
    sg = cfg.d ** -0.5
    w_gate = f32_to_bf16_bits(_normal(rng, (cfg.E_loc, cfg.H, cfg.d), sg))
    w_up = f32_to_bf16_bits(_normal(rng, (cfg.E_loc, cfg.H, cfg.d), sg))
    w_gu = np.concatenate([w_gate, w_up], axis=1)
    del w_gate, w_up
    w_down = f32_to_bf16_bits(_normal(rng, (cfg.E_loc, cfg.d, cfg.H), cfg.H ** -0.5))
    dy = f32_to_bf16_bits(_normal(rng, (T, cfg.d), 1.0))
    return dict(logits=logits, x=x, w_gu=w_gu, w_down=w_down, dy=dy)


def dyadic_layer_inputs(cfg: LayerConfig | str, seed: int = 0) -> dict:
    """layer_inputs with x and w_gu on coarse dyadic grids, so every partial sum of
    h = x . w_gu^T is exact in fp32 (x in {0, +-1, +-2} 2^-3, w_gu in {-7..7} 2^-7; the sum
    over d <= 4096 terms needs at most 17 significant bits). Any correct GEMM then produces
    the same h, and so the same bf16 h, as the fp64 oracle: used where the stored form of h
    is compared bit for bit. logits, w_down and dy are drawn as in layer_inputs."""
    if isinstance(cfg, str):
        cfg = LAYER_CONFIGS[cfg]
    assert cfg.d <= 4096
    out = layer_inputs(cfg, seed)
    rng = np.random.default_rng(seed + 1000)
    x = rng.integers(-2, 3, size=(cfg.T, cfg.d)).astype(np.float32) * 0.125
    w_gu = rng.integers(-7, 8, size=(cfg.E_loc, 2 * cfg.H, cfg.d)).astype(np.float32) / 128.0
    out["x"] = f32_to_bf16_bits(x)
    out["w_gu"] = f32_to_bf16_bits(w_gu)
    return out


def situ_inputs(R: int, H: int, seed: int = 0, h_std: float = 3.0) -> dict:
    """Draw h bf16 [R, 2H] ~ N(0, h_std^2) and da bf16 [R, H] ~ N(0, 1), in that order."""
    rng = np.random.default_rng(seed)
    h = f32_to_bf16_bits(_normal(rng, (R, 2 * H), h_std))
    da = f32_to_bf16_bits(_normal(rng, (R, H), 1.0))
    return dict(h=h, da=da)
