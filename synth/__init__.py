"""Seeded synthetic inputs for one-pass typed-decision scoring.

This module only draws random numbers: question tail lengths, option counts, candidate
token ids and bf16 tensors. It computes no step of the scoring method, so both the HIP
path and the CPU oracle can be fed from it without sharing any of the method's arithmetic.

The five workloads restate the shapes of the shared-prefix tail-prefill path described on
the blink.py page (thegovind/blink-4b): the "constants the deployment sets" section fixes
the 32768 padded-token budget, up to 255 options and up to 512 questions, and its
PREFIX_CACHE comment describes long multi-question documents whose prefix is encoded once.
The pages hold no dataset, so every tensor is N(0, sigma) noise of the stated shape.

Recipe (fixed draw order from one PCG64 stream seeded with 1000 + workload number):
tail lengths -> option counts -> candidate ids -> Q -> K_tail -> V_tail -> K_prefix ->
V_prefix -> H -> W_U. Integers are uniform and inclusive. Candidate ids are drawn per
question without replacement. Tensors are float32 normals rounded to bf16 with
round-to-nearest-even, padding rows included. Every padded-layout tensor needs the total
number of padded tokens, which the caller gets from a packer and passes in.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "config",
    "Tables",
    "draw_tables",
    "draw_tensors",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "rng_for",
]


@dataclass(frozen=True)
class Config:
    """One synthetic workload: attention shapes, question mix and readout shapes."""

    number: int
    name: str
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    prefix_len: int
    n_questions: int
    tail_lo: int
    tail_hi: int
    d_model: int
    vocab: int
    k_lo: int
    k_hi: int
    temperature: float
    w_u_std: float = 0.02
    qkv_std: float = 1.0
    hidden_std: float = 1.0
    token_budget: int = 32768
    max_rows: int = 0

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))


CONFIGS = {
    1: Config(1, "tiny", 4, 1, 64, 256, 4, 16, 48, 256, 1024, 2, 4, 1.0),
    2: Config(2, "4b_like", 32, 8, 128, 2048, 32, 64, 256, 2560, 151936, 2, 8, 1.0),
    3: Config(3, "long_document", 32, 8, 128, 18432, 64, 128, 512, 2560, 151936, 2, 26, 1.0),
    4: Config(4, "plain_max_packing", 32, 8, 128, 0, 512, 32, 256, 2560, 151936, 2, 255, 0.7),
    5: Config(5, "27b_like", 40, 8, 128, 65536, 16, 256, 1024, 5120, 151936, 2, 16, 1.0),
}


def config(number: int, **overrides) -> Config:
    """The numbered workload, optionally with fields replaced (for small test variants)."""
    cfg = CONFIGS[int(number)]
    return replace(cfg, **overrides) if overrides else cfg


def rng_for(cfg: Config, seed: int | None = None) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 + cfg.number if seed is None else seed))


@dataclass
class Tables:
    """Integer inputs of one request: per-question tail length and candidate ids (CSR)."""

    tail_len: np.ndarray  # int32 [n]
    n_options: np.ndarray  # int32 [n]
    cand_ids: np.ndarray  # int32 [sum K]
    cand_off: np.ndarray  # int32 [n + 1]


def draw_tables(cfg: Config, rng: np.random.Generator) -> Tables:
    n = cfg.n_questions
    tail_len = rng.integers(cfg.tail_lo, cfg.tail_hi, size=n, endpoint=True).astype(np.int32)
    n_options = rng.integers(cfg.k_lo, cfg.k_hi, size=n, endpoint=True).astype(np.int32)
    ids = [rng.choice(cfg.vocab, size=int(k), replace=False) for k in n_options]
    cand_ids = np.concatenate(ids).astype(np.int32) if ids else np.zeros(0, np.int32)
    cand_off = np.zeros(n + 1, np.int32)
    np.cumsum(n_options, out=cand_off[1:])
    return Tables(tail_len, n_options, cand_ids, cand_off)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    u = u + np.uint32(0x7FFF) + r
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float, chunk: int = 1 << 23) -> np.ndarray:
    """bf16 bits of N(0, std) float32 draws, generated in chunks to bound host memory."""
    total = int(np.prod(shape))
    out = np.empty(total, np.uint16)
    for start in range(0, total, chunk):
        stop = min(total, start + chunk)
        x = rng.standard_normal(stop - start, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[start:stop] = f32_to_bf16_bits(x)
    return out.reshape(shape)


TENSOR_ORDER = ("q", "k_tail", "v_tail", "k_prefix", "v_prefix", "hidden", "w_u")


def draw_tensors(cfg: Config, rng: np.random.Generator, total_padded_tokens: int,
                 parts=TENSOR_ORDER) -> dict:
    """bf16 bit arrays in the fixed order; parts not requested are still drawn (and dropped)
    so that the stream stays aligned, except trailing parts, which are not drawn at all."""
    t = int(total_padded_tokens)
    shapes = {
        "q": ((t, cfg.n_heads_q, cfg.head_dim), cfg.qkv_std),
        "k_tail": ((t, cfg.n_heads_kv, cfg.head_dim), cfg.qkv_std),
        "v_tail": ((t, cfg.n_heads_kv, cfg.head_dim), cfg.qkv_std),
        "k_prefix": ((cfg.prefix_len, cfg.n_heads_kv, cfg.head_dim), cfg.qkv_std),
        "v_prefix": ((cfg.prefix_len, cfg.n_heads_kv, cfg.head_dim), cfg.qkv_std),
        "hidden": ((t, cfg.d_model), cfg.hidden_std),
        "w_u": ((cfg.vocab, cfg.d_model), cfg.w_u_std),
    }
    wanted = set(parts)
    last = max(TENSOR_ORDER.index(p) for p in wanted) if wanted else -1
    out = {}
    for i, name in enumerate(TENSOR_ORDER[: last + 1]):
        shape, std = shapes[name]
        arr = _normal_bf16(rng, shape, std)
        if name in wanted:
            out[name] = arr
    return out


def draw_prefix_queries(cfg: Config, seed: int | None = None) -> np.ndarray:
    """Query rows of the shared prefix itself, bf16 bits [prefix_len, H_q, D] ~ N(0, 1), from
    their own PCG64 stream (seed 2000 + workload number by default). They are the inputs of
    the prefix's own causal prefill; the request's draws are not disturbed."""
    rng = np.random.Generator(np.random.PCG64(2000 + cfg.number if seed is None else seed))
    return _normal_bf16(rng, (cfg.prefix_len, cfg.n_heads_q, cfg.head_dim), 1.0)
