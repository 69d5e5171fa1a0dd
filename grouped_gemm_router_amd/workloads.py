"""Seeded synthetic inputs for the routed MoE expert layer.

This module only draws random inputs and stores them in the layouts the
layer consumes.  It holds none of the layer's arithmetic (no routing, no
softmax, no GEMM, no quantisation); both the GPU path and the CPU checker
read their inputs from here.

Shapes follow the model contracts listed in the LightMoE README (section
"Compatibility": hidden/intermediate 2048/512 with 256 experts, top-8, and
4096/1024 with 512 experts, top-10) and the 8,192-tokens, 128-experts/top-8
training setting of the LigerCute README (section "MoE performance").

Recipe (every tensor has its own counter-free numpy PCG64 stream, so any part
can be drawn alone and in any order):

* logits  fp32 [T, E]  ~ N(0, 1)                       stream [seed, 0]
* bias    fp32 [E]     = 0.5 * Zipf(a=1.1) per expert   stream [seed, 1]
  (added to every token's logits for the skewed configurations)
* X       bf16 [T, H]  ~ N(0, 1)                        stream [seed, 2]
* W_gate  bf16 [E, H, I] ~ N(0, std = 1/sqrt(H))        stream [seed, 3, e]
* W_up    bf16 [E, H, I] ~ N(0, std = 1/sqrt(H))        stream [seed, 4, e]
* W_down  bf16 [E, I, H] ~ N(0, std = 1/sqrt(I))        stream [seed, 5, e]
* dY      bf16 [T, H]  ~ N(0, 1)                        stream [seed, 6]

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even
from the fp32 draw).  Weights are drawn per expert so that a caller may draw
only some experts and fill the rest with a poison pattern.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

BF16_NAN_BITS = 0x7FC0


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts
    k: int          # experts per token
    dtype: str      # "bf16" or "mxfp8" (weights and activations of the expert GEMMs)
    logits: str     # "normal", "zipf" (N(0,1) + 0.5*Zipf(1.1) per expert) or "rankzipf"
    seed: int
    backward: bool = False
    activation: str = "swiglu"   # gated activation (swiglu, swiglu_clamp, swiglu_oai, geglu, reglu)
    act_limit: float = 0.0       # clamp of swiglu_clamp / swiglu_oai
    save_activations: bool = False   # training: the forward keeps G, U for the backward

    @property
    def A(self) -> int:
        """Routed rows (token-expert assignments), T*k."""
        return self.T * self.k

    @property
    def gated(self) -> bool:
        """Whether the experts have a gate weight (every activation but relu2)."""
        return self.activation != "relu2"

    @property
    def mats(self) -> tuple:
        """Names of the expert weight matrices."""
        return ("gate", "up", "down") if self.gated else ("up", "down")


CONFIGS = {
    "tiny": MoEConfig("tiny", 64, 256, 128, 8, 2, "bf16", "normal", 0),
    "prefill": MoEConfig("prefill", 4096, 2048, 512, 256, 8, "bf16", "zipf", 1),
    "decode": MoEConfig("decode", 32, 2048, 512, 256, 8, "bf16", "normal", 2),
    "large_mxfp8": MoEConfig("large_mxfp8", 8192, 4096, 1024, 512, 10, "mxfp8", "zipf", 3),
    "train": MoEConfig("train", 8192, 4096, 1024, 128, 8, "bf16", "normal", 4, backward=True),
    # the same training step with the projections kept from the forward instead of recomputed
    "train_saved": MoEConfig("train_saved", 8192, 4096, 1024, 128, 8, "bf16", "normal", 4, backward=True,
                             save_activations=True),
    # Diagnostic: prefill shapes with a milder per-rank bias, every expert active.
    "prefill_rankzipf": MoEConfig("prefill_rankzipf", 4096, 2048, 512, 256, 8, "bf16", "rankzipf", 1),
    # Diagnostic: the larger expert shapes of the LightMoE compatibility table (hidden / intermediate,
    # experts / top-k, activation), 4096 tokens, balanced routing.  The clamp of the bounded SwiGLU is
    # the value the pages give; SwiGLU-OAI's 7 is its public definition's (the pages give none).
    "h4096_i2048_e256_k6_clamp": MoEConfig("h4096_i2048_e256_k6_clamp", 4096, 4096, 2048, 256, 6, "bf16",
                                           "normal", 5, activation="swiglu_clamp", act_limit=10.0),
    "h6144_i2048_e256_k8": MoEConfig("h6144_i2048_e256_k8", 4096, 6144, 2048, 256, 8, "bf16", "normal", 6),
    "h6144_i3072_e128_k4_oai": MoEConfig("h6144_i3072_e128_k4_oai", 4096, 6144, 3072, 128, 4, "bf16",
                                         "normal", 7, activation="swiglu_oai", act_limit=7.0),
    # the two-weight ReLU^2 expert shape of the same table
    "h2688_i1856_e128_k6_relu2": MoEConfig("h2688_i1856_e128_k6_relu2", 4096, 2688, 1856, 128, 6, "bf16",
                                           "normal", 8, activation="relu2"),
}


def config(base: str, **over) -> MoEConfig:
    cfg = CONFIGS[base]
    return replace(cfg, **over) if over else cfg


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def make_logits(cfg: MoEConfig) -> np.ndarray:
    logits = _rng(cfg.seed, 0).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.logits == "zipf":
        bias = (0.5 * _rng(cfg.seed, 1).zipf(1.1, size=cfg.E)).astype(np.float32)
        logits += bias[None, :]
    elif cfg.logits == "rankzipf":
        bias = (-0.55 * np.log(np.arange(1, cfg.E + 1, dtype=np.float64) + 1.0)).astype(np.float32)
        logits += bias[None, :]
    elif cfg.logits != "normal":
        raise ValueError(cfg.logits)
    return np.ascontiguousarray(logits)


def make_x(cfg: MoEConfig) -> np.ndarray:
    return f32_to_bf16_bits(_rng(cfg.seed, 2).standard_normal((cfg.T, cfg.H), dtype=np.float32))


def make_dy(cfg: MoEConfig) -> np.ndarray:
    return f32_to_bf16_bits(_rng(cfg.seed, 6).standard_normal((cfg.T, cfg.H), dtype=np.float32))


_WEIGHT_STREAM = {"gate": 3, "up": 4, "down": 5}


def weight_shape(cfg: MoEConfig, name: str) -> tuple[int, int]:
    """[K, N] of one expert's matrix: gate/up are [H, I], down is [I, H]."""
    return (cfg.I, cfg.H) if name == "down" else (cfg.H, cfg.I)


def make_expert_weight(cfg: MoEConfig, name: str, e: int) -> np.ndarray:
    K, N = weight_shape(cfg, name)
    w = _rng(cfg.seed, _WEIGHT_STREAM[name], e).standard_normal((K, N), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(K))
    return f32_to_bf16_bits(w)


def make_weights(cfg: MoEConfig, name: str, experts=None, fill_bits: int = BF16_NAN_BITS,
                 threads: int | None = None) -> np.ndarray:
    """All experts' [E, K, N] bf16 bits.  With ``experts`` given, only those are
    drawn and every other expert is filled with ``fill_bits`` (NaN by default)."""
    K, N = weight_shape(cfg, name)
    out = np.empty((cfg.E, K, N), dtype=np.uint16)
    todo = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))
    if experts is not None:
        out[...] = np.uint16(fill_bits)

    def one(e):
        out[e] = make_expert_weight(cfg, name, e)

    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(one, todo))
    return out

