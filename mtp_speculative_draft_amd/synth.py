"""Seeded synthetic inputs for the MTP draft-layer forward.

This module holds random draws, the bit packing of the weight formats and
plain data containers -- none of the forward's arithmetic.  Both the CPU
oracle (tests, benchmark baseline) and the HIP path are fed from here.

Weight formats (hf2q 0.1.1, src/serve/forward_mlx_shared.rs, `MlxAffineExtra`
and `MlxQWeight::from_mlx_affine_linear`):

* 4-bit affine, group 32: u32 codes ``[n, k/8]`` with element ``k`` in nibble
  ``k % 8`` of word ``k // 8`` (lowest nibble = lowest k); f32 scales and
  biases ``[n, k/32]``; value = scale * code + bias.
* 8-bit block, block 32: int8 codes ``[..., n, k]`` and f32 scales
  ``[..., n, k/32]``; value = scale * code.
* 4-bit affine expert stack with bf16 group constants (hf2q 0.1.1,
  `MlxAffineMoeStack`): u32 codes ``[E, n, k/8]`` in the 4-bit nibble order,
  bf16 scales and biases ``[E, n, k/32]`` stored as their 16 bits (the upper
  half of an f32); value = scale * code + bias.

Every generator takes a ``numpy.random.Generator`` so that callers fix the
draw order; ``rng(config, *extra)`` seeds one from ``SeedSequence`` entropy
``[1234 + config, *extra]``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 1234
GROUP = 32


def rng(config: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_BASE + int(config), *map(int, extra)]))


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Q4:
    codes: np.ndarray  # uint32 [n, k/8]
    scales: np.ndarray  # float32 [n, k/32]
    biases: np.ndarray  # float32 [n, k/32]

    @property
    def n(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k(self) -> int:
        return int(self.codes.shape[1]) * 8

    @property
    def nbytes(self) -> int:
        return int(self.codes.nbytes + self.scales.nbytes + self.biases.nbytes)


@dataclasses.dataclass
class Q8:
    codes: np.ndarray  # int8 [E, n, k] (E = 1 for a single matrix)
    scales: np.ndarray  # float32 [E, n, k/32]

    @property
    def n_experts(self) -> int:
        return int(self.codes.shape[0])

    @property
    def n(self) -> int:
        return int(self.codes.shape[1])

    @property
    def k(self) -> int:
        return int(self.codes.shape[2])

    @property
    def expert_nbytes(self) -> int:
        return int(self.codes[0].nbytes + self.scales[0].nbytes)


@dataclasses.dataclass
class Q4E:
    codes: np.ndarray  # uint32 [E, n, k/8]
    scales: np.ndarray  # uint16 (bf16 bits) [E, n, k/32]
    biases: np.ndarray  # uint16 (bf16 bits) [E, n, k/32]

    @property
    def n_experts(self) -> int:
        return int(self.codes.shape[0])

    @property
    def n(self) -> int:
        return int(self.codes.shape[1])

    @property
    def k(self) -> int:
        return int(self.codes.shape[2]) * 8

    @property
    def expert_nbytes(self) -> int:
        return int(self.codes[0].nbytes + self.scales[0].nbytes + self.biases[0].nbytes)


@dataclasses.dataclass
class DenseLayer:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    ffn_inter: int
    rope_theta: float
    eps: float
    gamma_e: np.ndarray
    gamma_h: np.ndarray
    gamma_attn: np.ndarray
    gamma_post: np.ndarray
    gamma_final: np.ndarray
    eh_proj: Q4
    wq: Q4
    wk: Q4
    wv: Q4
    wo: Q4
    gate: Q4
    up: Q4
    down: Q4
    lm_head: Q4
    # attention variant ([mtp.rs] `forward_full_attention`): per-head q/k
    # RMSNorm weights [head_dim], a gated q projection (per head: q rows then
    # gate rows) and a partial rotary dimension (0 = head_dim)
    gamma_q_head: Optional[np.ndarray] = None
    gamma_k_head: Optional[np.ndarray] = None
    q_gated: bool = False
    rotary_dim: int = 0
    # sliding-window attention ([mimo.rs] "window 128, sinks"): per-query-head
    # sink logits [n_heads] and the window (0 = none)
    sinks: Optional[np.ndarray] = None
    window: int = 0
    # MiMo draft geometry (head 192 / V 128): the V heads' width (0 = head_dim)
    v_head_dim: int = 0
    # multi-section rotary ([mtp.rs] `apply_imrope`, `mrope_section`): the
    # sizes of the first three position-id sections (with the position ids of
    # a call's rows given per call)
    mrope_section: tuple = (0, 0, 0, 0)

    def q4_weights(self):
        return [self.eh_proj, self.wq, self.wk, self.wv, self.wo, self.gate, self.up, self.down, self.lm_head]

    @property
    def weight_nbytes(self) -> int:
        return sum(w.nbytes for w in self.q4_weights()) + 5 * self.hidden * 4


# --------------------------------------------------------------------------
# packing (format only)
# --------------------------------------------------------------------------
def pack_q4(codes: np.ndarray) -> np.ndarray:
    """Pack uint8 codes [n, k] (values 0..15) into u32 [n, k/8], low nibble first."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    if k % 8:
        raise ValueError("k must be a multiple of 8")
    if codes.max(initial=0) > 15:
        raise ValueError("4-bit codes must lie in 0..15")
    byte = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(byte).view("<u4").reshape(n, k // 8).astype(np.uint32)


def unpack_q4_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_q4`` (format only): u32 [n, k/8] -> uint8 [n, k]."""
    b = np.ascontiguousarray(packed, dtype="<u4").view(np.uint8).reshape(packed.shape[0], -1)
    out = np.empty((packed.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def q4_weight(g: np.random.Generator, n: int, k: int) -> Q4:
    """codes ~ U{0..15}, scale ~ U(0.005, 0.02), bias = -8*scale + N(0, 1e-3)."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 32")
    # one uniform byte holds two independent uniform nibbles
    byte = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    codes = np.ascontiguousarray(byte).view("<u4").reshape(n, k // 8).copy()
    scales = g.uniform(0.005, 0.02, size=(n, k // GROUP)).astype(np.float32)
    biases = (-8.0 * scales.astype(np.float64) + g.normal(0.0, 1e-3, size=(n, k // GROUP))).astype(np.float32)
    return Q4(codes, scales, biases)


def q8_weight(g: np.random.Generator, n_experts: int, n: int, k: int) -> Q8:
    """codes ~ U{-127..127}, one scale ~ U(0.001, 0.01) per block of 32."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 32")
    codes = g.integers(-127, 128, size=(n_experts, n, k), dtype=np.int8)
    scales = g.uniform(0.001, 0.01, size=(n_experts, n, k // GROUP)).astype(np.float32)
    return Q8(codes, scales)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 nearest to each finite f32 (ties to even), as its 16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """The f32 that 16 bf16 bits stand for (format only)."""
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def q4e_weight(g: np.random.Generator, n_experts: int, n: int, k: int) -> Q4E:
    """codes ~ U{0..15}; scale ~ U(0.005, 0.02) and bias = -8*scale + N(0, 1e-3),
    each rounded to bf16."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 32")
    byte = g.integers(0, 256, size=(n_experts, n, k // 2), dtype=np.uint8)
    codes = np.ascontiguousarray(byte).view("<u4").reshape(n_experts, n, k // 8).copy()
    scales = g.uniform(0.005, 0.02, size=(n_experts, n, k // GROUP))
    biases = -8.0 * scales + g.normal(0.0, 1e-3, size=(n_experts, n, k // GROUP))
    return Q4E(codes, bf16_bits(scales.astype(np.float32)), bf16_bits(biases.astype(np.float32)))


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def gamma(g: np.random.Generator, h: int) -> np.ndarray:
    """Norm weight 1 + N(0, 0.1)."""
    return (1.0 + 0.1 * g.standard_normal(size=h)).astype(np.float32)


def dense_layer(g: np.random.Generator, hidden: int = 2048, n_heads: int = 16, n_kv_heads: int = 2,
                head_dim: int = 128, vocab: int = 151936, ffn_inter: int = 6144,
                rope_theta: float = 1.0e6, eps: float = 1e-6, q_gated: bool = False, qk_norm: bool = False,
                rotary_dim: int = 0, window: int = 0, sinks: bool = False, v_head_dim: int = 0,
                mrope_section=(0, 0, 0, 0)) -> DenseLayer:
    """Dense MTP draft layer with 4-bit weights (draw order fixed; the
    attention variant's head norm weights are drawn last, then the sinks,
    U(-1, 3) per query head)."""
    H = hidden
    gam = [gamma(g, H) for _ in range(5)]
    eh = q4_weight(g, H, 2 * H)
    dv = v_head_dim if v_head_dim > 0 else head_dim
    wq = q4_weight(g, n_heads * (head_dim + dv if q_gated else head_dim), H)
    wk = q4_weight(g, n_kv_heads * head_dim, H)
    wv = q4_weight(g, n_kv_heads * dv, H)
    wo = q4_weight(g, H, n_heads * dv)
    gate = q4_weight(g, ffn_inter, H)
    up = q4_weight(g, ffn_inter, H)
    down = q4_weight(g, H, ffn_inter)
    lm = q4_weight(g, vocab, H)
    gq = gamma(g, head_dim) if qk_norm else None
    gk = gamma(g, head_dim) if qk_norm else None
    sk = g.uniform(-1.0, 3.0, size=n_heads).astype(np.float32) if sinks else None
    return DenseLayer(H, n_heads, n_kv_heads, head_dim, vocab, ffn_inter, float(rope_theta), float(eps),
                      gam[0], gam[1], gam[2], gam[3], gam[4], eh, wq, wk, wv, wo, gate, up, down, lm,
                      gq, gk, bool(q_gated), int(rotary_dim), sk, int(window), int(v_head_dim),
                      tuple(int(v) for v in mrope_section))


def kv_cache(g: np.random.Generator, n_kv_heads: int, filled: int, capacity: int, head_dim: int,
             v_dim: int = 0):
    """K cache [n_kv, capacity, head_dim] and V cache [n_kv, capacity, v_dim or
    head_dim]: rows < filled ~ N(0,1), the rest zero."""
    dv = v_dim if v_dim > 0 else head_dim
    k = np.zeros((n_kv_heads, capacity, head_dim), dtype=np.float32)
    v = np.zeros((n_kv_heads, capacity, dv), dtype=np.float32)
    k[:, :filled] = normal(g, (n_kv_heads, filled, head_dim))
    v[:, :filled] = normal(g, (n_kv_heads, filled, dv))
    return k, v


@dataclasses.dataclass
class MoeInputs:
    """Routed FFN weights and input rows; the expert matrices are all Q8
    (8-bit experts) or all Q4E (4-bit experts with bf16 group constants)."""
    x: np.ndarray
    router: np.ndarray
    gate_exps: "Q8 | Q4E"
    up_exps: "Q8 | Q4E"
    down_exps: "Q8 | Q4E"
    sh_gate: "Optional[Q8 | Q4E]"
    sh_up: "Optional[Q8 | Q4E]"
    sh_down: "Optional[Q8 | Q4E]"
    top_k: int

    @property
    def n_experts(self) -> int:
        return self.gate_exps.n_experts

    @property
    def q4(self) -> bool:
        return isinstance(self.gate_exps, Q4E)


def moe_inputs(g: np.random.Generator, m: int, hidden: int = 2048, n_experts: int = 256, inter: int = 512,
               top_k: int = 8, shared_inter: Optional[int] = 512, q4: bool = False) -> MoeInputs:
    """q4: 4-bit experts with bf16 group constants instead of 8-bit ones."""
    draw = q4e_weight if q4 else q8_weight
    x = normal(g, (m, hidden))
    router = normal(g, (n_experts, hidden), 0.02)
    ge = draw(g, n_experts, inter, hidden)
    ue = draw(g, n_experts, inter, hidden)
    de = draw(g, n_experts, hidden, inter)
    if shared_inter:
        sg = draw(g, 1, shared_inter, hidden)
        su = draw(g, 1, shared_inter, hidden)
        sd = draw(g, 1, hidden, shared_inter)
    else:
        sg = su = sd = None
    return MoeInputs(x, router, ge, ue, de, sg, su, sd, top_k)


# --------------------------------------------------------------------------
# the five workloads (shapes and distributions of the pages' configurations)
# --------------------------------------------------------------------------
def config0_gemv():
    g = rng(0)
    w = q4_weight(g, 1024, 1024)
    x = normal(g, (1, 1024))
    return w, x


def config1_proj():
    g = rng(1)
    H = 2048
    e = normal(g, (4, H))
    h = normal(g, (4, H))
    ge = gamma(g, H)
    gh = gamma(g, H)
    w = q4_weight(g, H, 2 * H)
    return e, h, ge, gh, w


def config2_head(vocab: int = 151936, hidden: int = 2048):
    """Hidden rows, final-norm weight and lm_head (before any planting)."""
    g = rng(2)
    x = normal(g, (4, hidden))
    gf = gamma(g, hidden)
    lm = q4_weight(g, vocab, hidden)
    return x, gf, lm


def config3_moe(m: int = 4):
    return moe_inputs(rng(3), m)


@dataclasses.dataclass
class StepInputs:
    layer: DenseLayer
    e0: np.ndarray
    h0: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    cache_len: int
    capacity: int
    table: np.ndarray


def config4_step(seed_extra: int = 0, cache_len: int = 4096, capacity: int = 4104, **shape) -> StepInputs:
    """Dense draft step: layer weights, (e0, h0), the KV caches and a token
    embedding table [vocab, hidden] ~ N(0,1)."""
    g = rng(4, seed_extra) if seed_extra else rng(4)
    layer = dense_layer(g, **shape)
    e0 = normal(g, (1, layer.hidden))
    h0 = normal(g, (1, layer.hidden))
    kc, vc = kv_cache(g, layer.n_kv_heads, cache_len, capacity, layer.head_dim, layer.v_head_dim)
    table = normal(g, (layer.vocab, layer.hidden))
    return StepInputs(layer, e0, h0, kc, vc, cache_len, capacity, table)


def imrope_positions(g: np.random.Generator, m: int, base: int, spread: int = 64) -> np.ndarray:
    """Four rotary position ids per row (int32 [m, 4]): the row's sequence
    position base + r for the first id, the others drawn within +-spread of it
    (the distinct per-section ids of a multimodal token)."""
    p = np.empty((m, 4), dtype=np.int32)
    for r in range(m):
        p[r, 0] = base + r
        p[r, 1:] = base + r + g.integers(-spread, spread + 1, size=3)
    return np.maximum(p, 0)
