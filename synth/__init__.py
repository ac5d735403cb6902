"""Seeded synthetic inputs for the low-rank binary (LRB) linear layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds only input synthesis: random numbers, the bf16 rounding
used to *make* bf16 inputs, and the SplitMix64 counter generator.  It contains
none of the method's arithmetic (no packing, no sign application, no products).

Workload shapes follow the Llama-2 7B / 70B linear layers that the NanoQuant
pages evaluate on (research.samsung.com blog "NanoQuant: Efficient Sub-1-Bit
Quantization of Large Language Models", section 4 "Results").  Trained weights
and WikiText-2 data are not available; seeded synthetic values of the same
shapes stand in for them.

Recipe (every draw is reproducible from BASE_SEED):
  * generators are numpy PCG64 seeded from children of SeedSequence(BASE_SEED)
    keyed by a short text tag, so each matrix/vector has its own stream;
  * latent factors U [d_out][r], V [d_in][r]: fp32 N(0,1) (their signs are iid
    Rademacher);
  * scales: 0.02*|N(0,1)| fp32, or exp(N(-4, 0.5)) fp32 ("log-normal" set);
  * activations: N(0,1) rounded to bf16 (round-to-nearest-even), optionally with
    1% of positions per token replaced by +-20 (20 sigma outliers);
  * 70B-shaped sign words: low 32 bits of SplitMix64 of (seed + word index),
    identical on host (here) and on the GPU (the library's fill routine).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260206

# --------------------------------------------------------------------------
# seeded streams
# --------------------------------------------------------------------------


def _tag_key(tag: str) -> list[int]:
    h = hashlib.sha256(tag.encode()).digest()
    return [int.from_bytes(h[i:i + 4], "little") for i in range(0, 16, 4)]


def rng(tag: str, base_seed: int = BASE_SEED) -> np.random.Generator:
    """PCG64 generator for a named stream (child of SeedSequence(base_seed))."""
    ss = np.random.SeedSequence(entropy=base_seed, spawn_key=tuple(_tag_key(tag)))
    return np.random.Generator(np.random.PCG64(ss))


def seed64(tag: str, base_seed: int = BASE_SEED) -> int:
    """A 64-bit seed for a SplitMix64 word stream, derived like rng()."""
    ss = np.random.SeedSequence(entropy=base_seed, spawn_key=tuple(_tag_key(tag)))
    lo, hi = (int(v) for v in ss.generate_state(2, np.uint32))
    return (hi << 32) | lo


# --------------------------------------------------------------------------
# bf16 (used only to manufacture bf16 inputs)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit patterns.

    NaN inputs are not produced by this module and are not handled specially.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values that are exactly representable in bf16 (RNE of the input)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# --------------------------------------------------------------------------
# SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014; constants of Vigna's public-domain splitmix64)
# --------------------------------------------------------------------------

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, index: np.ndarray) -> np.ndarray:
    """Output number index+1 of a SplitMix64 stream started at `seed`.

    state_i = seed + (index + 1) * GAMMA (mod 2^64); output = mix(state_i).
    Vectorised over `index` (uint64 array); all arithmetic wraps mod 2^64.
    """
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (idx + np.uint64(1)) * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def random_words(seed: int, index: np.ndarray) -> np.ndarray:
    """uint32 sign words: the low 32 bits of splitmix64(seed, index)."""
    return (splitmix64(seed, index) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------


def normal_f32(tag: str, shape) -> np.ndarray:
    return rng(tag).standard_normal(shape, dtype=np.float32)


def scales_halfnormal(tag: str, n: int) -> np.ndarray:
    """0.02 * |N(0,1)| as fp32."""
    return (np.float32(0.02) * np.abs(normal_f32(tag, n))).astype(np.float32)


def scales_lognormal(tag: str, n: int, mu: float = -4.0, sigma: float = 0.5) -> np.ndarray:
    """exp(N(mu, sigma^2)) as fp32."""
    g = rng(tag).standard_normal(n)  # fp64 draw, then exp, then round to fp32
    return np.exp(mu + sigma * g).astype(np.float32)


def activations(tag: str, T: int, d: int, dtype: str = "bf16",
                outlier_frac: float = 0.0, outlier_mag: float = 20.0) -> np.ndarray:
    """x [T][d] ~ N(0,1), as fp32 or bf16-rounded fp32 values.

    With outlier_frac > 0: per token, floor(outlier_frac*d) positions drawn
    uniformly without replacement are set to +-outlier_mag (random sign).
    """
    g = rng(tag)
    x = g.standard_normal((T, d), dtype=np.float32)
    n_out = int(np.floor(outlier_frac * d))
    if n_out > 0:
        for t in range(T):
            pos = g.choice(d, size=n_out, replace=False)
            sgn = np.where(g.random(n_out) < 0.5, -1.0, 1.0).astype(np.float32)
            x[t, pos] = sgn * np.float32(outlier_mag)
    if dtype == "bf16":
        x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class LayerShape:
    name: str
    d_out: int
    d_in: int
    r: int


def rank_for_bits(d_out: int, d_in: int, frac: float = 1.0, multiple: int = 64) -> int:
    """r = floor(frac * d_out*d_in/(d_out+d_in) / multiple) * multiple.

    frac=1.0 gives ~1 bit/weight of sign storage; frac=0.55 the 0.55-bit variant.
    """
    return int(np.floor(frac * d_out * d_in / (d_out + d_in) / multiple)) * multiple


def llama2_70b_layer(frac: float = 1.0) -> list[LayerShape]:
    """The seven linears of one Llama-2-70B decoder layer, in execution order."""
    h, kv, ff = 8192, 1024, 28672
    shapes = [("q", h, h), ("k", kv, h), ("v", kv, h), ("o", h, h),
              ("gate", ff, h), ("up", ff, h), ("down", h, ff)]
    return [LayerShape(n, o, i, rank_for_bits(o, i, frac)) for n, o, i in shapes]


@dataclass
class Config:
    key: str
    description: str
    layers: list = field(default_factory=list)  # LayerShape list
    T: tuple = (1,)
    x_dtype: str = "bf16"
    scale_kind: str = "halfnormal"
    outlier_frac: float = 0.0
    n_layers: int = 1
    words: str = "latent"  # "latent": pack from fp32 latent; "splitmix": words drawn directly


CONFIGS = {
    "single": Config("single", "single LRB linear 256x256, r=64, fp32 x",
                     [LayerShape("w", 256, 256, 64)], (1,), "f32"),
    "7b_attn": Config("7b_attn", "Llama-2-7B attention projection 4096x4096, r=2048",
                      [LayerShape("attn", 4096, 4096, 2048)], (1,), "bf16"),
    "7b_mlp": Config("7b_mlp", "Llama-2-7B MLP set at ~0.8 bit, r=2368, 1% 20-sigma outliers",
                     [LayerShape("gate", 11008, 4096, 2368), LayerShape("up", 11008, 4096, 2368),
                      LayerShape("down", 4096, 11008, 2368)], (1, 8), "bf16",
                     scale_kind="lognormal", outlier_frac=0.01),
    "70b_stack": Config("70b_stack", "Llama-2-70B linear stack, 80 layers, ~1.0 bit",
                        llama2_70b_layer(1.0), (1,), "bf16", n_layers=80, words="splitmix"),
    "70b_stack_055": Config("70b_stack_055", "Llama-2-70B linear stack, 80 layers, 0.55 bit",
                            llama2_70b_layer(0.55), (1,), "bf16", n_layers=80, words="splitmix"),
    "70b_prefill": Config("70b_prefill", "Llama-2-70B-shaped prefill, T=2048, ~1.0 bit",
                          llama2_70b_layer(1.0), (2048,), "bf16", n_layers=80, words="splitmix"),
}


def stack_config(frac: float) -> Config:
    """The 80-layer Llama-2-70B-shaped stack with every rank at `frac` times its
    ~1-bit value (1.0 and 0.55 are the named configs; other fractions are the
    rank-sweep stacks)."""
    if frac == 1.0:
        return CONFIGS["70b_stack"]
    if frac == 0.55:
        return CONFIGS["70b_stack_055"]
    return Config(f"70b_stack_{frac}", f"Llama-2-70B linear stack, {frac} x the 1-bit rank",
                  llama2_70b_layer(frac), (1,), "bf16", n_layers=80, words="splitmix")


def scales(cfg: Config, tag: str, n: int) -> np.ndarray:
    if cfg.scale_kind == "lognormal":
        return scales_lognormal(tag, n)
    return scales_halfnormal(tag, n)


def lrb_inputs(cfg: Config, layer: LayerShape, layer_idx: int = 0) -> dict:
    """Latent factors and scales for one linear of a 'latent' config."""
    base = f"{cfg.key}/{layer_idx}/{layer.name}"
    out = {
        "s1": scales(cfg, base + "/s1", layer.d_out),
        "s2": scales(cfg, base + "/s2", layer.d_in),
    }
    if cfg.words == "latent":
        out["U_latent"] = normal_f32(base + "/U", (layer.d_out, layer.r))
        out["V_latent"] = normal_f32(base + "/V", (layer.d_in, layer.r))
    else:
        out["u_seed"] = seed64(base + "/U")
        out["v_seed"] = seed64(base + "/V")
    return out


def x_for(cfg: Config, d_in: int, T: int, tag: str = "x") -> np.ndarray:
    return activations(f"{cfg.key}/{tag}/{d_in}/{T}", T, d_in, cfg.x_dtype, cfg.outlier_frac)
