"""Seeded synthetic workloads: shapes and bf16 inputs, nothing else.

This module holds none of the method's arithmetic.  It draws random inputs
with NumPy, rounds them once to bfloat16 (nearest, ties to even) and returns
the raw bf16 bit patterns as uint16, which the oracle and the HIP library
both consume byte for byte.

The pages evaluate trained models (Qwen3 / Qwen3.5 / Gemma-4 families) on
agentic and long-context suites ([GS-EN] s.4 Experimental Results); none of
that is available here, so LLM-shaped GEMMs with synthetic activations and
weights stand in for them.  The shapes are those of a Llama-3-8B-like and a
Llama-3-70B-like decoder layer.

Recipe (per tensor): ``default_rng(SeedSequence([seed, cfg, tensor_id, role]))``
(role 0 = activation, 1 = weight), float32 draws in chunks of 1024 rows,
outlier columns chosen without replacement and multiplied by the factor,
then one rounding to bf16.  Configuration 1 instead uses ``default_rng(0)``
with draw order activations, outlier columns, weights.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# tensor ids for the per-layer activations and weights
ACTS = ("x_qkv", "x_o", "x_gu", "x_down")
PROJ_INPUT = {"q": "x_qkv", "k": "x_qkv", "v": "x_qkv", "o": "x_o",
              "gate": "x_gu", "up": "x_gu", "down": "x_down"}
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, nearest with ties to even (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerShape:
    d_model: int
    d_kv: int
    d_ffn: int

    def proj_nk(self, proj: str):
        d, kv, f = self.d_model, self.d_kv, self.d_ffn
        return {"q": (d, d), "k": (kv, d), "v": (kv, d), "o": (d, d),
                "gate": (f, d), "up": (f, d), "down": (d, f)}[proj]

    def act_k(self, act: str) -> int:
        return self.d_ffn if act == "x_down" else self.d_model


LLAMA8B = LayerShape(4096, 1024, 14336)
LLAMA70B = LayerShape(8192, 1024, 28672)


@dataclass(frozen=True)
class Dist:
    kind: str              # "normal" or "student_t"
    df: float = 0.0
    std: float = 1.0       # N(0, std^2); for student_t the scale after unit-variance
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    M: tuple               # token counts (decode: several batch sizes)
    layer: LayerShape | None
    act: Dist
    weight: Dist
    fused_act_quant: bool = False
    decode: bool = False
    projs: tuple = PROJS
    weight_cfg: int | None = None  # draw weights with another config's seeds
    desc: str = ""
    extra: dict = field(default_factory=dict)

    def flops(self, M=None):
        M = self.M[0] if M is None else M
        return sum(2 * M * n * k for n, k in (self.layer.proj_nk(p) for p in self.projs))


CONFIGS = {
    1: Config(1, "single_linear_m128_k512_n512", (128,), None,
              Dist("normal", outlier_frac=4 / 512, outlier_factor=20.0),
              Dist("normal", std=0.02),
              desc="one NVFP4 linear, M=128, K=512, N=512"),
    2: Config(2, "llama8b_prefill_m4096", (4096,), LLAMA8B,
              Dist("normal", outlier_frac=0.01, outlier_factor=30.0),
              Dist("normal", std=0.02),
              desc="8B-shaped layer, seven projections, M=4096"),
    3: Config(3, "llama8b_longctx_m32768_fused", (32768,), LLAMA8B,
              Dist("student_t", df=4.0, std=1.0),
              Dist("normal", std=0.02), fused_act_quant=True,
              desc="8B-shaped layer, M=32768, act-quant fused into each GEMM"),
    4: Config(4, "llama8b_decode_bf16", (1, 4, 16, 32), LLAMA8B,
              Dist("normal"), Dist("normal", std=0.02), decode=True,
              projs=("q", "k", "gate", "down"), weight_cfg=2,
              desc="BF16 decode GEMV on the 8B-shaped weights, M in {1,4,16,32}"),
    5: Config(5, "llama70b_prefill_m16384", (16384,), LLAMA70B,
              Dist("student_t", df=3.0, std=1.0, outlier_frac=0.005, outlier_factor=50.0),
              Dist("normal", std=0.015),
              desc="70B-shaped layer slice, M=16384, heavy-tailed activations"),
}

_TENSOR_IDS = {name: i for i, name in enumerate(ACTS + PROJS)}


def _draw(rng: np.random.Generator, rows: int, cols: int, dist: Dist) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, 1024):
        r1 = min(rows, r0 + 1024)
        if dist.kind == "normal":
            out[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        elif dist.kind == "student_t":
            t = rng.standard_t(dist.df, size=(r1 - r0, cols))
            out[r0:r1] = t * np.sqrt((dist.df - 2.0) / dist.df)  # unit variance
        else:
            raise ValueError(dist.kind)
    if dist.std != 1.0:
        out *= np.float32(dist.std)
    if dist.outlier_frac > 0:
        n = int(round(dist.outlier_frac * cols))
        idx = rng.choice(cols, n, replace=False)
        out[:, idx] *= np.float32(dist.outlier_factor)
    return out


def activation(cfg: int, act: str = "x_qkv", M: int | None = None, seed: int = 0) -> np.ndarray:
    """bf16 bits [M][K] of one activation tensor of configuration ``cfg``."""
    c = CONFIGS[cfg]
    if cfg == 1:
        return _cfg1()[0]
    M = c.M[0] if M is None else M
    K = c.layer.act_k(act)
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, _TENSOR_IDS[act], 0, M]))
    return f32_to_bf16_bits(_draw(rng, M, K, c.act))


def weight(cfg: int, proj: str = "q", seed: int = 0) -> np.ndarray:
    """bf16 bits [N][K] of one projection weight of configuration ``cfg``."""
    c = CONFIGS[cfg]
    if cfg == 1:
        return _cfg1()[1]
    wcfg = c.weight_cfg or cfg
    wc = CONFIGS[wcfg]
    N, K = wc.layer.proj_nk(proj)
    rng = np.random.default_rng(np.random.SeedSequence([seed, wcfg, _TENSOR_IDS[proj], 1]))
    return f32_to_bf16_bits(_draw(rng, N, K, wc.weight))


_CFG1_CACHE = {}


def _cfg1():
    if "v" not in _CFG1_CACHE:
        rng = np.random.default_rng(0)
        x = rng.standard_normal((128, 512), dtype=np.float32)
        idx = rng.choice(512, 4, replace=False)
        x[:, idx] *= np.float32(20.0)
        w = rng.standard_normal((512, 512), dtype=np.float32) * np.float32(0.02)
        _CFG1_CACHE["v"] = (f32_to_bf16_bits(x), f32_to_bf16_bits(w))
    return _CFG1_CACHE["v"]


def random_bf16(shape, seed: int, scale: float = 1.0, kind: str = "normal") -> np.ndarray:
    """Generic seeded bf16 tensor for ragged / edge-case tests."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 99]))
    if kind == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif kind == "uniform":
        x = rng.uniform(-1, 1, size=shape).astype(np.float32)
    elif kind == "lognormal_mixed":
        # magnitudes spread over many binades, random signs: exercises every
        # group-scale exponent including E4M3 subnormals
        mag = np.exp(rng.normal(0.0, 6.0, size=shape)).astype(np.float32)
        x = np.where(rng.random(shape) < 0.5, -mag, mag).astype(np.float32)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(x * np.float32(scale))


def sha256(bits: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(bits).tobytes()).hexdigest()
