"""Seeded synthetic workloads for the routed MoE expert-FFN layer.

Shapes and value distributions follow the five workloads this layer is
measured on: a tiny correctness case, single-token decode (M=1), a small
batch (M=21, aligned with b=8), a Zipf-skewed batch (M=256, b=64) and an
MXFP8-weight batch (M=64). The large shapes (hidden 2048, per-expert
intermediate 768, 128 experts, top-8, AWQ-style int4 with group 128) are
those of the Qwen3-30B-A3B-class layer in "Route-Block Membership Selects
Packed-AWQ Arithmetic" (fixture paragraph) and of the Qwen-3-style decode in
the warp-decode blog ("La ruta convencional de MoE"). No trained weights are
used: every array is drawn from a seeded numpy PCG64 generator.

Conventions shared by both consumers (they define the input bytes only):
  * int4 weights: uint32 words ``q[e, n, kk // 8]`` in AWQ's interleaved
    nibble order (nibble slot i holds element [0, 2, 4, 6, 1, 3, 5, 7][i] of
    the word's eight). Drawing every word uniformly from [0, 2^32) draws each
    nibble independently from U{0..15}, whatever the order.
  * scales: fp16 ``s[e, n, kk // g]``; zero points: uint8 ``z[e, n, kk // g]``
    holding 0..15.
  * W13 has ``2I`` rows: rows ``0..I-1`` are the gate projection, rows
    ``I..2I-1`` the up projection; its reduction dimension is H. W2 has H
    rows and reduction dimension I.
  * activations: bf16 bit patterns (uint16), rounded to nearest even from
    fp32 N(0, 1) draws.
  * routing: fp32 router logits -> fp32 softmax -> top-k by descending
    probability (ties to the lower expert ID) -> weights renormalised to sum
    to one in fp32. IDs are int32 ``[M, k]``, weights fp32 ``[M, k]``.
  * MXFP8 weights: OCP E4M3FN codes ``[e, n, kk]`` (uint8) and one E8M0
    exponent byte per 32 consecutive reduction elements ``[e, n, kk // 32]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Stream identifiers keep weights, activations, logits and popularity
# independent for one seed.
_STREAM_WEIGHTS = 0
_STREAM_X = 1
_STREAM_LOGITS = 2
_STREAM_ZIPF = 3


@dataclass(frozen=True)
class Config:
    name: str
    M: int
    H: int
    I: int
    E: int
    k: int
    b: int
    g: int
    fmt: str = "int4"          # "int4" (AWQ-style) or "mxfp8"
    s_lo: float = 0.002        # int4 scale ~ U(s_lo, s_hi), stored fp16
    s_hi: float = 0.01
    zipf_s: float | None = None  # popularity exponent of the expert bias
    mx_sigma: float = 0.02     # MXFP8: fp32 weights ~ N(0, sigma) before quantisation


CONFIGS: dict[str, Config] = {
    # Tiny correctness case.
    "tiny": Config("tiny", M=4, H=256, I=128, E=8, k=2, b=8, g=64,
                   s_lo=0.005, s_hi=0.02),
    # Single-token decode on the 128-expert, top-8 layer.
    "decode_m1": Config("decode_m1", M=1, H=2048, I=768, E=128, k=8, b=8, g=128),
    # The 21-token batch aligned with b=8 (168 routes).
    "batch_m21": Config("batch_m21", M=21, H=2048, I=768, E=128, k=8, b=8, g=128),
    # 256 tokens with Zipf(1.1) expert popularity, aligned with b=64.
    "batch_m256_zipf": Config("batch_m256_zipf", M=256, H=2048, I=768, E=128, k=8,
                              b=64, g=128, zipf_s=1.1),
    # MXFP8 weights (E4M3 + E8M0 per 32), 64 tokens.
    "mxfp8_m64": Config("mxfp8_m64", M=64, H=2048, I=768, E=128, k=8, b=16, g=32,
                        fmt="mxfp8"),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


@dataclass
class PackedWeights:
    """One projection's resident weights for all E experts."""
    fmt: str
    N: int                    # output rows per expert
    K: int                    # reduction length
    g: int                    # elements per scale group
    q: np.ndarray             # int4: uint32 [E, N, K/8]; mxfp8: uint8 [E, N, K]
    s: np.ndarray             # int4: float16 [E, N, K/g]; mxfp8: uint8 E8M0 [E, N, K/32]
    z: np.ndarray | None      # int4: uint8 [E, N, K/g]; mxfp8: None

    def expert_bytes(self) -> int:
        """Bytes one expert's packed values, scales and zeros occupy."""
        n = self.q[0].nbytes + self.s[0].nbytes
        if self.z is not None:
            n += self.z[0].nbytes
        return int(n)


def _int4_projection(rng: np.random.Generator, E: int, N: int, K: int, g: int,
                     s_lo: float, s_hi: float) -> PackedWeights:
    q = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32)
    s = rng.uniform(s_lo, s_hi, size=(E, N, K // g)).astype(np.float32).astype(np.float16)
    z = rng.integers(0, 16, size=(E, N, K // g), dtype=np.uint8)
    return PackedWeights("int4", N, K, g, q, s, z)


def _mxfp8_projection(rng: np.random.Generator, E: int, N: int, K: int,
                      sigma: float) -> PackedWeights:
    """Quantise N(0, sigma) fp32 weights to E4M3 codes with an E8M0 scale per 32.

    The shared exponent of a block is floor(log2(max |w|)) - 8 (8 is the
    exponent of E4M3's largest normal, 448); values are scaled by 2^-exp,
    clamped to +-448 and cast with round-to-nearest-even. Only the codes and
    exponent bytes are inputs to the layer.
    """
    import torch  # the fp8 cast is torch's; used for data generation only

    codes = np.empty((E, N, K), dtype=np.uint8)
    exps = np.empty((E, N, K // 32), dtype=np.uint8)
    for e in range(E):
        w = rng.normal(0.0, sigma, size=(N, K // 32, 32)).astype(np.float32)
        amax = np.abs(w).max(axis=-1)
        with np.errstate(divide="ignore"):
            ex = np.where(amax > 0, np.floor(np.log2(amax)) - 8, -127).astype(np.int32)
        ex = np.clip(ex, -127, 127)
        scaled = np.clip(w / np.ldexp(np.float32(1), ex)[..., None], -448.0, 448.0)
        c = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn)
        codes[e] = c.view(torch.uint8).numpy().reshape(N, K)
        exps[e] = (ex + 127).astype(np.uint8)
    return PackedWeights("mxfp8", N, K, 32, codes, exps, None)


def make_weights(cfg: Config, seed: int, layer: int = 0) -> tuple[PackedWeights, PackedWeights]:
    """(W13, W2) for all experts of one layer."""
    rng = _rng(seed, _STREAM_WEIGHTS, layer)
    if cfg.fmt == "int4":
        w13 = _int4_projection(rng, cfg.E, 2 * cfg.I, cfg.H, cfg.g, cfg.s_lo, cfg.s_hi)
        w2 = _int4_projection(rng, cfg.E, cfg.H, cfg.I, cfg.g, cfg.s_lo, cfg.s_hi)
    elif cfg.fmt == "mxfp8":
        w13 = _mxfp8_projection(rng, cfg.E, 2 * cfg.I, cfg.H, cfg.mx_sigma)
        w2 = _mxfp8_projection(rng, cfg.E, cfg.H, cfg.I, cfg.mx_sigma)
    else:
        raise ValueError(f"unknown weight format {cfg.fmt!r}")
    return w13, w2


def zipf_bias(cfg: Config, seed: int) -> np.ndarray:
    """Per-expert logit bias ln(p_e), p_e proportional to rank_e^-s.

    Ranks 1..E are assigned to experts by a seeded permutation, so the most
    popular expert is not always expert 0.
    """
    assert cfg.zipf_s is not None
    ranks = _rng(seed, _STREAM_ZIPF).permutation(cfg.E) + 1
    return (-cfg.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)


def route(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 softmax, top-k by descending probability (ties: lower ID), renormalised."""
    logits = np.asarray(logits, dtype=np.float32)
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m, dtype=np.float32)
    p = (ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    order = np.argsort(-p, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return ids, w


def make_routing(cfg: Config, seed: int, index: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(topk_ids int32 [M, k], topk_w fp32 [M, k]) for routing draw ``index``."""
    logits = _rng(seed, _STREAM_LOGITS, index).standard_normal((cfg.M, cfg.E), dtype=np.float32)
    if cfg.zipf_s is not None:
        logits = logits + zipf_bias(cfg, seed)[None, :]
    return route(logits, cfg.k)


def make_x(cfg: Config, seed: int, index: int = 0, M: int | None = None) -> np.ndarray:
    """bf16 bit patterns [M, H] of N(0, 1) activations."""
    m = cfg.M if M is None else M
    a = _rng(seed, _STREAM_X, index).standard_normal((m, cfg.H), dtype=np.float32)
    return bf16_bits_from_f32(a)


@dataclass
class Workload:
    cfg: Config
    seed: int
    x: np.ndarray            # uint16 bf16 bits [M, H]
    topk_ids: np.ndarray     # int32 [M, k]
    topk_w: np.ndarray       # float32 [M, k]
    w13: PackedWeights
    w2: PackedWeights
    extra: dict = field(default_factory=dict)

    def touched_experts(self) -> np.ndarray:
        ids = self.topk_ids.reshape(-1)
        ids = ids[(ids >= 0) & (ids < self.cfg.E)]
        return np.unique(ids)


def make_workload(name_or_cfg, seed: int = 0, layer: int = 0, routing: int = 0) -> Workload:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    w13, w2 = make_weights(cfg, seed, layer)
    ids, w = make_routing(cfg, seed, routing)
    x = make_x(cfg, seed, routing)
    return Workload(cfg, seed, x, ids, w, w13, w2)
