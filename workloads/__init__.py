"""Seeded synthetic inputs for the MoE layer forward (shared by tests and bench).

This module draws random numbers and packs them into the storage formats the
layer consumes.  It holds none of the layer's arithmetic: no routing, no
softmax, no FFN, no dequantisation.  Both the CPU oracle (``oracle/``) and the
HIP library receive exactly the arrays produced here.

Shapes follow the five MoE-layer workloads the pages study:

* ``tiny``            -- fp32, H=256, 8 experts top-2, I=512, one shared expert
                         (I_s=512), 16 tokens, experts 0-3 resident, LoRE r=8.
* ``dsv2_lite``       -- DeepSeek-V2-Lite shape (SPICE page, "MoE inference
                         I/O bottleneck": 64 experts, top-6): H=2048, I=1408,
                         two shared experts of 1408, unnormalised softmax
                         weights, 50% of experts resident, LoRE r=16.
* ``qwen2_57b``       -- Qwen2-57B-A14B shape: H=3584, 64 experts top-8,
                         I=2560, one shared expert of 20480 with a sigmoid
                         scalar gate, renormalised weights, 25% resident,
                         LoRE r=32.
* ``mixtral_floe``    -- Mixtral-8x7B FloE expert (FloE page, Sec. 1 "Hybrid
                         compression"): H=4096, 8 experts top-2, I=14336, up
                         projection stored as 2-bit asymmetric codes in groups
                         of 64 with fp16 scale and zero, keep 10% of channels.
* ``granite_prefill`` -- Granite-3B-A800M shape (APEX page, Sec. 1: 40 experts,
                         top-8): H=1536, I=512, 4096 tokens, a separate linear
                         prefetch router drawn N(0, 0.02) independently of the
                         router, per-token extra budget delta drawn from
                         Geometric(0.4) on {0,1,...} capped at N-k, and an
                         ordinal budget model (w_delta, theta).
* ``granite_prefill_distilled`` -- the same layer with the prefetch router
                         drawn correlated 0.97 with the router (APEX page,
                         Sec. 4.1 trains the prefetch router toward the
                         router's choices); used for the adaptive-budget
                         statistics, whose overlap is meaningless for an
                         unrelated router.

Layouts (all row-major, C order):

* ``x``             [T][H]
* ``w_router``      [E][H]           ``w_prefetch`` [E][H]  (expert e's row holds
                    the H weights of its logit, so logits = x W^T)
* ``w_gate``        [E][I][H]        (output channel i's H-vector contiguous)
* ``w_up``          [E][I][H]        (dense up only)
* ``w_down``        [E][H][I] dense; [E][I][H] for the FloE format, whose
                    selective loading wants one channel's down row contiguous
* ``up_q``          [E][I][H/4] uint8: code of input h in bits 2*(h%4)..+1 of
                    byte h/4
* ``up_scale``, ``up_zero`` [E][I][H/64] fp16 bit patterns (uint16)
* ``ws_gate``, ``ws_up`` [n_s][I_s][H];  ``ws_down`` [n_s][H][I_s]
* ``w_shared_gate`` [H]
* ``lore_A``        [E][r][H];  ``lore_B`` [E][H][r]
* ``resident``      one uint64 bit mask of resident experts (bit e = expert e)
* ``delta``         [T] int32 extra prefetch budget per token
* ``w_delta``, ``theta``  APEX ordinal budget model: [H] and [N-k+1] fp32

bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even from
the fp32 draw); fp32 tensors as float32.  Every tensor has its own seed stream
``SeedSequence([seed, tag, index])`` so an expert's weights can be drawn alone
(the oracle samples a few experts of the large workloads).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "Layer", "make_layer", "bf16_bits_from_f32",
    "fp16_bits_from_f32", "quantize_int2_g64", "draw_delta", "draw_resident", "draw_ordinal",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int
    shared_inter: int
    lore_rank: int
    renormalize: bool
    shared_gate: bool
    dtype: str                      # "f32" or "bf16"
    token_counts: Tuple[int, ...]
    modes: Tuple[str, ...]
    seed: int
    up_format: str = "dense"        # "dense" or "int2_g64"
    floe_keep: int = 0              # kept channels per (token, expert) pair
    resident_fixed: Optional[Tuple[int, ...]] = None
    resident_count: Optional[int] = None
    prefetch: bool = False          # draws w_prefetch and delta
    delta_p: float = 0.4
    prefetch_rho: float = 0.0       # correlation of the prefetch router with the router
    weight_std: float = 0.02
    hidden_std: float = 1.0
    lore_std: float = 0.01
    prev_noise: float = 0.33        # x_prev = x + prev_noise * N(0, hidden_std): cosine ~0.95

    @property
    def t_max(self) -> int:
        return max(self.token_counts)

    @property
    def delta_cap(self) -> int:
        return self.n_experts - self.top_k


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig(
        name="tiny", hidden=256, n_experts=8, top_k=2, inter=512, n_shared=1,
        shared_inter=512, lore_rank=8, renormalize=False, shared_gate=False,
        dtype="f32", token_counts=(16,), modes=("standard", "lore"), seed=0,
        resident_fixed=(0, 1, 2, 3)),
    "dsv2_lite": MoEConfig(
        name="dsv2_lite", hidden=2048, n_experts=64, top_k=6, inter=1408,
        n_shared=2, shared_inter=1408, lore_rank=16, renormalize=False,
        shared_gate=False, dtype="bf16", token_counts=(1, 8, 64),
        modes=("standard", "lore"), seed=1, resident_count=32),
    "qwen2_57b": MoEConfig(
        name="qwen2_57b", hidden=3584, n_experts=64, top_k=8, inter=2560,
        n_shared=1, shared_inter=20480, lore_rank=32, renormalize=True,
        shared_gate=True, dtype="bf16", token_counts=(1, 32, 256),
        modes=("standard", "lore"), seed=2, resident_count=16),
    "mixtral_floe": MoEConfig(
        name="mixtral_floe", hidden=4096, n_experts=8, top_k=2, inter=14336,
        n_shared=0, shared_inter=0, lore_rank=0, renormalize=True,
        shared_gate=False, dtype="bf16", token_counts=(1,), modes=("floe",),
        seed=3, up_format="int2_g64", floe_keep=1434),
    "granite_prefill": MoEConfig(
        name="granite_prefill", hidden=1536, n_experts=40, top_k=8, inter=512,
        n_shared=0, shared_inter=0, lore_rank=0, renormalize=True,
        shared_gate=False, dtype="bf16", token_counts=(4096,),
        modes=("standard", "stall_free"), seed=4, prefetch=True),
    "granite_prefill_distilled": MoEConfig(
        name="granite_prefill_distilled", hidden=1536, n_experts=40, top_k=8, inter=512,
        n_shared=0, shared_inter=0, lore_rank=0, renormalize=True,
        shared_gate=False, dtype="bf16", token_counts=(4096,),
        modes=("standard", "stall_free"), seed=4, prefetch=True, prefetch_rho=0.97),
}

# Seed-stream tags, one per tensor.
_TAG = {"x": 1, "w_router": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
        "ws_gate": 6, "ws_up": 7, "ws_down": 8, "w_shared_gate": 9,
        "lore_A": 10, "lore_B": 11, "resident": 12, "w_prefetch": 13,
        "delta": 14, "w_delta": 15, "theta": 16, "x_prev": 17, "calib": 18, "omega": 19}


def _rng(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _TAG[tag], idx]))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def fp16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def quantize_int2_g64(w: np.ndarray):
    """Asymmetric round-to-nearest 2-bit quantiser, groups of 64 along the last axis.

    FloE stores the up projection as HQQ INT2 (FloE page, Sec. 1 "ultra-low-bit
    quantisation"); HQQ's zero-point optimiser is not described there, so the
    plain min-max form is used: per group s = fp16((max-min)/3),
    z = fp16(-min/s), q = clamp(rint(w/s + z), 0, 3) using the fp16 s and z.
    A constant group gets s = 1, z = fp16(-min).  Returns (codes packed four to
    a byte, scale bits, zero bits).  The decoded weight is (q - z) * s.
    """
    w = np.asarray(w, dtype=np.float32)
    *lead, h = w.shape
    assert h % 64 == 0
    g = w.reshape(*lead, h // 64, 64)
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    flat = hi == lo
    s = np.where(flat, np.float32(1.0), (hi - lo) / np.float32(3.0)).astype(np.float16)
    s32 = s.astype(np.float32)
    z = (-lo / s32).astype(np.float16)
    z32 = z.astype(np.float32)
    q = np.clip(np.rint(g / s32[..., None] + z32[..., None]), 0, 3).astype(np.uint8)
    q = q.reshape(*lead, h // 4, 4)
    packed = (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)).astype(np.uint8)
    return packed, s.view(np.uint16), z.view(np.uint16)


def draw_resident(cfg: MoEConfig, seed: int) -> int:
    """Resident-expert bit mask: a fixed list, or round(f*E) experts drawn
    uniformly without replacement."""
    if cfg.resident_fixed is not None:
        ids = cfg.resident_fixed
    elif cfg.resident_count is not None:
        ids = _rng(seed, "resident").permutation(cfg.n_experts)[: cfg.resident_count]
    else:
        ids = range(cfg.n_experts)
    m = 0
    for e in ids:
        m |= 1 << int(e)
    return m


def draw_delta(cfg: MoEConfig, seed: int, T: int) -> np.ndarray:
    """Per-token extra prefetch budget: Geometric(p) on {0,1,...} (P(j)=p(1-p)^j),
    capped at N-k (the largest budget the APEX page allows)."""
    d = _rng(seed, "delta").geometric(cfg.delta_p, size=T) - 1
    return np.minimum(d, cfg.delta_cap).astype(np.int32)


def draw_ordinal(cfg: MoEConfig, seed: int, tau: float = 0.9):
    """Synthetic APEX ordinal budget model (the page trains it; no trained
    values exist here): w [H] ~ N(0, 1/H), so w.x has unit spread for unit x;
    theta [N-k+1] non-decreasing, theta_d = logit(tau) - 2 + sum of d steps
    drawn from 0.5 * U(0.5, 1.5), which puts the mean budget near 4 at tau.
    Returns (w fp32, theta fp32)."""
    w = _normal(_rng(seed, "w_delta"), (cfg.hidden,), 1.0 / np.sqrt(cfg.hidden))
    steps = _rng(seed, "theta").uniform(0.5, 1.5, size=cfg.delta_cap).astype(np.float32) * np.float32(0.5)
    base = np.float32(np.log(tau / (1.0 - tau)) - 2.0)
    theta = np.concatenate([[base], base + np.cumsum(steps, dtype=np.float32)]).astype(np.float32)
    return w, theta


class Layer:
    """Lazily drawn inputs of one MoE layer for a workload.

    Expert tensors are drawn per expert (``expert(name, e)``) so large layers
    can be sampled; ``full(name)`` stacks all experts.  ``x(T)`` is the first T
    rows of one T_max-row draw, so smaller batches are row prefixes.
    """

    def __init__(self, cfg: MoEConfig, seed: Optional[int] = None, threads: Optional[int] = None,
                 cache_bytes: int = 8 << 30):
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self.threads = threads or min(16, len(os.sched_getaffinity(0)))
        self._cache: Dict[Tuple[str, int], object] = {}
        self._cache_left = cache_bytes

    # ---- scalars / small tensors -------------------------------------------------
    def _to_storage(self, a: np.ndarray) -> np.ndarray:
        return a if self.cfg.dtype == "f32" else bf16_bits_from_f32(a)

    def x(self, T: Optional[int] = None) -> np.ndarray:
        key = ("x", 0)
        if key not in self._cache:
            a = _normal(_rng(self.seed, "x"), (self.cfg.t_max, self.cfg.hidden), self.cfg.hidden_std)
            self._cache[key] = self._to_storage(a)
        full = self._cache[key]
        return full if T is None else full[:T]

    def x_prev(self, T: Optional[int] = None) -> np.ndarray:
        """The previous layer's hidden state for the FloE intra-expert
        predictor: x + prev_noise * fresh N(0, hidden_std) noise, drawn in fp32
        from the fp32 x draw, then rounded to the storage dtype.  0.33 puts the
        cosine between the two near 0.95, the similarity of adjacent layers'
        hidden states on the FloE page."""
        key = ("x_prev", 0)
        if key not in self._cache:
            c = self.cfg
            shape = (c.t_max, c.hidden)
            x = _normal(_rng(self.seed, "x"), shape, c.hidden_std)
            nz = _normal(_rng(self.seed, "x_prev"), shape, c.hidden_std)
            self._cache[key] = self._to_storage((x + np.float32(c.prev_noise) * nz).astype(np.float32))
        full = self._cache[key]
        return full if T is None else full[:T]

    def calibration(self, N: int) -> np.ndarray:
        """LoRE calibration inputs: an orthogonal design of N = m*H rows, m
        blocks of sqrt(H) * Q with Q the Q factor of an H x H N(0,1) draw, so
        the rows have the norm of unit-variance hidden states and
        h^T h = N I in fp32 before rounding to the storage dtype."""
        H = self.cfg.hidden
        if N % H:
            raise ValueError("calibration size must be a multiple of hidden")
        rng = _rng(self.seed, "calib")
        blocks = []
        for _ in range(N // H):
            q, _ = np.linalg.qr(rng.standard_normal((H, H)))
            blocks.append((q * np.sqrt(H)).astype(np.float32))
        return self._to_storage(np.concatenate(blocks, axis=0))

    def omega(self, cols: int) -> np.ndarray:
        """Gaussian start block [H][cols] fp32 for the LoRE fit's subspace
        iteration (the random numbers the method draws)."""
        return _normal(_rng(self.seed, "omega"), (self.cfg.hidden, cols), 1.0)

    def w_router(self) -> np.ndarray:
        return self._small("w_router", (self.cfg.n_experts, self.cfg.hidden), self.cfg.weight_std)

    def w_prefetch(self) -> np.ndarray:
        """The separate linear prefetch router (APEX page, Sec. 4.1):
        rho * W_r + sqrt(1 - rho^2) * fresh N(0, weight_std) noise, drawn in
        fp32 before rounding to the storage dtype.  rho = 0 (the default) is
        an independent N(0, weight_std) router; rho = 0.97 stands in for one
        trained toward the router's choices (no trained weights exist here)
        and gives Granite-shaped inputs a long-tailed delta* (median 2, 98th
        percentile about 9)."""
        key = ("w_prefetch", 0)
        if key not in self._cache:
            c = self.cfg
            shape = (c.n_experts, c.hidden)
            wr = _normal(_rng(self.seed, "w_router"), shape, c.weight_std)
            nz = _normal(_rng(self.seed, "w_prefetch"), shape, c.weight_std)
            rho = np.float32(c.prefetch_rho)
            w = (rho * wr + np.float32(np.sqrt(1.0 - c.prefetch_rho ** 2)) * nz).astype(np.float32)
            self._cache[key] = self._to_storage(w)
        return self._cache[key]

    def w_shared_gate(self) -> np.ndarray:
        return self._small("w_shared_gate", (self.cfg.hidden,), self.cfg.weight_std)

    def resident(self) -> int:
        return draw_resident(self.cfg, self.seed)

    def delta(self, T: Optional[int] = None) -> np.ndarray:
        d = draw_delta(self.cfg, self.seed, self.cfg.t_max)
        return d if T is None else d[:T]

    def ordinal(self, tau: float = 0.9):
        """(w_delta in storage dtype, theta fp32) of the APEX budget model."""
        key = ("ordinal", 0)
        if key not in self._cache:
            w, th = draw_ordinal(self.cfg, self.seed, tau)
            self._cache[key] = (self._to_storage(w), th)
        return self._cache[key]

    def _small(self, name, shape, std):
        key = (name, 0)
        if key not in self._cache:
            self._cache[key] = self._to_storage(_normal(_rng(self.seed, name), shape, std))
        return self._cache[key]

    # ---- per-expert tensors ------------------------------------------------------
    def _shape(self, name: str):
        c = self.cfg
        H, I, r = c.hidden, c.inter, c.lore_rank
        return {
            "w_gate": (I, H), "w_up": (I, H),
            "w_down": (I, H) if c.up_format == "int2_g64" else (H, I),
            "ws_gate": (c.shared_inter, H), "ws_up": (c.shared_inter, H),
            "ws_down": (H, c.shared_inter),
            "lore_A": (r, H), "lore_B": (H, r),
        }[name]

    def _count(self, name: str) -> int:
        return self.cfg.n_shared if name.startswith("ws_") else self.cfg.n_experts

    def expert(self, name: str, e: int):
        """One expert's tensor.  For ``up_q`` / ``up_scale`` / ``up_zero`` the
        INT2 form of that expert's fp32 up weights."""
        key = (name, e)
        if key in self._cache:
            return self._cache[key]
        c = self.cfg
        if name in ("up_q", "up_scale", "up_zero"):
            w = _normal(_rng(self.seed, "w_up", e), self._shape("w_up"), c.weight_std)
            q, s, z = quantize_int2_g64(w)
            out = {"up_q": q, "up_scale": s, "up_zero": z}
            nb = q.nbytes + s.nbytes + z.nbytes
            if nb <= self._cache_left:
                self._cache_left -= nb
                for n, v in out.items():
                    self._cache[(n, e)] = v
            return out[name]
        std = c.lore_std if name.startswith("lore_") else c.weight_std
        a = self._to_storage(_normal(_rng(self.seed, name, e), self._shape(name), std))
        # Kept until the cache budget is spent; later draws are regenerated.
        if a.nbytes <= self._cache_left:
            self._cache[key] = a
            self._cache_left -= a.nbytes
        return a

    def w_up_f32(self, e: int) -> np.ndarray:
        """The unquantised fp32 up weights that the INT2 codes were made from."""
        return _normal(_rng(self.seed, "w_up", e), self._shape("w_up"), self.cfg.weight_std)

    def full(self, name: str) -> np.ndarray:
        n = self._count(name)
        with ThreadPoolExecutor(self.threads) as ex:
            parts = list(ex.map(lambda e: self.expert(name, e), range(n)))
        return np.stack(parts) if parts else np.zeros((0,) + self._shape(name), np.float32)

    def tensor_names(self):
        c = self.cfg
        names = ["w_gate", "w_down"]
        names += ["up_q", "up_scale", "up_zero"] if c.up_format == "int2_g64" else ["w_up"]
        if c.n_shared:
            names += ["ws_gate", "ws_up", "ws_down"]
        if c.lore_rank:
            names += ["lore_A", "lore_B"]
        return names


def make_layer(name_or_cfg, seed: Optional[int] = None, **overrides) -> Layer:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    return Layer(cfg, seed)
