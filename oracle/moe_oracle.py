"""Plain fp64 CPU oracle of one MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It is written from the pages alone, in
NumPy float64 from exactly decoded inputs, shares no code with the HIP library,
and is deliberately unoptimised: every step is its textbook definition or the
algorithm's steps in the pages' order.

Sources (cited by page title and section):

* [SPICE] "SPICE: Speculative Prefetching with Low-Rank Expert Surrogates and
  Heterogeneous Orchestration for MoE Inference Acceleration" (PaperDaily
  summary).  Sections "MoE inference I/O bottleneck" (router picks top-k of N
  experts per token), "Confidence-aware adaptive prefetch" (confidence = the
  probability mass on the predicted top-K), "LoRE low-rank surrogate" (a
  missing expert's output is replaced by y_shared + B_e A_e h).
* [FloE] "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" (Paper
  Notes).  Sec. 1 "Hybrid compression": contextual sparsification forward
  a^S(x) = (SiLU(x W_gate) * S_t(x W_up)) W_down with S_t a mask from the
  magnitude of the up output; up projection stored as INT2.
* [APEX] "APEX: Adaptive Expert Prefetching for Edge MoE Inference" (blog
  summary).  Sec. 1 (router picks top-k of N), Sec. 4.1 (prefetch router: a
  linear layer + softmax over experts), Sec. 4.2 (oracle budget delta*,
  prefetch list = top-(k+delta)), Sec. 4.3 (stall-free mode, Algorithm 1).

Readings where the pages are silent or garbled (each also listed in the design
notes):

* LoRE factor shapes: A_e is r x H and B_e is H x r, so B_e A_e h is an H-vector
  (the page prints the two shapes the other way round, which cannot multiply h).
* y_shared in the surrogate is the raw (ungated) sum of the shared-expert FFN
  outputs; a surrogate slot keeps the missing expert's own routing weight; h is
  the layer input x_t.
* Ties in every ranking go to the lower expert id (lower channel for FloE).  A
  decision whose deciding gap is below ``tie_margin`` (1e-4, absolute, in
  logits or |u|) is flagged as a near-tie: several answers are correct there.
* Stall-free: a substitute keeps its own original-router probability; weights
  are renormalised over the final set when the layer renormalises; the final
  slots are ordered by (-logit, id).
* FloE keeps ``floe_keep`` channels per (token, routed expert) pair, ranked by
  (-|u_i|, i); the gate is evaluated only where kept (SiLU(g)*0 = 0 elsewhere).
* INT2 up weights decode as (q - z) * s with q the 2-bit code of input h at bits
  2*(h%4) of byte h/4 and fp16 s, z per group of 64 consecutive inputs.
* Dense expert down weights are stored [H][I] (output row h holds the I inputs);
  FloE down weights are stored [I][H] (one channel's H-vector contiguous).
  Router and prefetch-router weights are stored [E][H].

* APEX's adaptive budget is the least delta with p_delta >= tau; when no
  delta in 0..N-k qualifies the budget is N-k (everything is prefetched).  Its
  near-tie is measured on the logit scale: |theta_d - s - logit(tau)| below
  ``tie_margin`` at the chosen d or at d - 1.

* FloE's intra-expert predictor applies the mask rule itself to h_l W_up^(l+1)
  (the previous layer's hidden state and this layer's INT2 up weights) for the
  experts this layer routes to; the inter-expert predictor that would guess
  those experts is a trained MLP and not modelled, so the experts are given.
  Recall is |predicted & true| / n_keep per (token, expert).  Compact packing
  gathers the kept channels' gate and down rows in ascending channel order.

* LoRE fitting minimises ||R - h (B A)^T||_F over rank-r maps on the rows it
  is given (R = y_e - y_shared): with G = h^T h / N and M = R^T h / N, the
  minimiser is B A = [M G^-1/2]_r G^-1/2 (reduced-rank regression: whiten the
  inputs, truncate the SVD, map back), B = U_r S_r and A = V_r^T G^-1/2 from
  the SVD U S V^T of M G^-1/2.  For an orthogonal design (G = I) this is the
  truncated SVD of M itself.

* SPICE's cost rule for a missed expert compares fetching it (W_e / B_pcie +
  T_gpu_e) with running it on the host (T_cpu_e + 2H / B_pcie).  W_e counts
  the expert's three matrices (gate, up, down) in the layer dtype; T_cpu_e
  and the 2H transfer scale with the expert's routed (token, expert) pairs
  (each pair's hidden state goes down and its output comes back), and
  T_cpu_e may also hold a fixed per-expert term (the weight reads); the fetch
  is taken only when strictly cheaper.  A resident expert, or one no token
  routes to, needs neither.  The page also ties the choice to the current
  PCIe pressure; the queue-aware form reads that as queues: experts are
  decided by decreasing pair count, each cost counting the time earlier
  decisions already put on the link or the host (the plain rule is the
  default and the first decision of either form).

* Stall-free with fewer than k prefetched experts (outside the page's domain:
  its lists hold k + delta >= k experts): Algorithm 1 then returns the whole
  prefetched set; the remaining slots take the best experts outside it by
  the original router's score (these would stall), and the token gets flag
  bit 32.

Flag bits per token: 1 route near-tie, 2 prefetch near-tie, 4 substitution
near-tie, 8 FloE mask near-tie, 16 prefetch-budget near-tie, 32 prefetched
set smaller than k (stall-free).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "FLAG_ROUTE", "FLAG_PREFETCH", "FLAG_SUBST", "FLAG_FLOE", "FLAG_SHORT",
    "bf16_to_f64", "fp16_to_f64", "decode", "silu", "sigmoid",
    "router_logits", "softmax", "rank_experts", "route_token",
    "prefetch_set", "prefetch_masks", "delta_star", "stall_free_select", "stall_free_fill",
    "FLAG_BUDGET", "adaptive_budget", "prefetch_overlap", "adaptive_prefetch",
    "permute", "swiglu_expert", "dequant_int2", "floe_expert",
    "floe_channel_mask", "floe_predict_masks", "mask_recall", "floe_pack",
    "lore_targets", "lore_fit",
    "shared_experts", "lore_residual", "layer_forward", "WeightSource",
    "OFFLOAD_NONE", "OFFLOAD_FETCH", "OFFLOAD_HOST", "offload_costs", "offload_plan",
]

FLAG_ROUTE, FLAG_PREFETCH, FLAG_SUBST, FLAG_FLOE = 1, 2, 4, 8
FLAG_BUDGET = 16
FLAG_SHORT = 32
MODES = ("standard", "lore", "stall_free", "floe")


# ---------------------------------------------------------------- decoding --
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float64 (exact: a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def silu(z):
    """SiLU(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


# ------------------------------------------------------------------ routing --
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] W_r[e, h]: the router is a linear head over the
    experts [APEX Sec. 1; SPICE "MoE inference I/O bottleneck"].  W_r is stored
    [E][H], one row of weights per expert."""
    return x @ w_router.T


def softmax(l: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis."""
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def rank_experts(score_row: Sequence[float]) -> List[int]:
    """All expert ids ordered by (-score, id): ties go to the lower id."""
    return sorted(range(len(score_row)), key=lambda e: (-float(score_row[e]), e))


def route_token(l_row: np.ndarray, k: int, renormalize: bool, margin: float):
    """Top-k routing of one token [APEX Sec. 1; SPICE "MoE inference I/O
    bottleneck"], with the SPICE confidence = probability mass on the chosen
    top-k [SPICE "Confidence-aware adaptive prefetch", Eq. 5].

    Returns (ids in rank order, weights, mass, near-tie flag)."""
    E = len(l_row)
    order = rank_experts(l_row)
    ids = order[:k]
    p = softmax(np.asarray(l_row, dtype=np.float64))
    mass = float(sum(p[e] for e in ids))
    w = [p[e] / mass for e in ids] if renormalize else [p[e] for e in ids]
    flag = k < E and (l_row[order[k - 1]] - l_row[order[k]]) < margin
    return ids, np.array(w), mass, bool(flag)


def prefetch_set(lp_row: np.ndarray, n: int, margin: float):
    """K_p = the top-n experts by the prefetch router's score; the prefetch
    router is linear + softmax and softmax keeps the order, so its logits rank
    the same [APEX Sec. 4.1, Sec. 4.2 top-(k+delta) list].  Returns (bit mask,
    near-tie flag)."""
    E = len(lp_row)
    order = rank_experts(lp_row)
    mask = 0
    for e in order[:n]:
        mask |= 1 << e
    flag = n < E and (lp_row[order[n - 1]] - lp_row[order[n]]) < margin
    return mask, bool(flag)


def prefetch_masks(x: np.ndarray, w_prefetch: np.ndarray, delta: np.ndarray, k: int,
                   margin: float = 1e-4):
    """Per-token prefetch masks top-(k + delta_t) of x W_p, and flag bit 2 for
    near-ties at the list's edge."""
    lp = router_logits(x, w_prefetch)
    masks, flags = [], []
    for t in range(x.shape[0]):
        m, f = prefetch_set(lp[t], k + int(delta[t]), margin)
        masks.append(m)
        flags.append(FLAG_PREFETCH if f else 0)
    return masks, np.array(flags, dtype=np.uint32), lp


def delta_star(routed: Sequence[int], lp_row: np.ndarray, k: int) -> int:
    """APEX oracle budget [Sec. 4.2]: the least delta in {0..N-k} such that the
    routed set lies inside the top-(k+delta) prefetch list."""
    E = len(lp_row)
    order = rank_experts(lp_row)
    for d in range(0, E - k + 1):
        if set(routed) <= set(order[: k + d]):
            return d
    raise AssertionError("unreachable: delta = N-k lists every expert")


def adaptive_budget(x_row: np.ndarray, w_delta: np.ndarray, theta: Sequence[float],
                    tau: float, margin: float = 1e-4):
    """APEX adaptive budget [Sec. 4.2]: an ordinal logistic CDF
    p_delta(x) = Pr(delta >= delta* | x) = sigmoid(theta_delta - w^T x) over
    delta = 0..N-k, and delta_hat(x) = the least delta with p_delta >= tau.
    theta has N-k+1 entries (non-decreasing on the page; the least qualifying
    delta is taken either way).  Returns (delta_hat, near-tie flag)."""
    s = float(np.dot(np.asarray(w_delta, dtype=np.float64), np.asarray(x_row, dtype=np.float64)))
    lt = math.log(tau / (1.0 - tau))
    d_hat = len(theta) - 1
    for d, th in enumerate(theta):
        if sigmoid(float(th) - s) >= tau:
            d_hat = d
            break
    near = abs(float(theta[d_hat]) - s - lt) < margin
    if d_hat > 0:
        near = near or abs(float(theta[d_hat - 1]) - s - lt) < margin
    return d_hat, bool(near)


def prefetch_overlap(routed: Sequence[int], mask: int) -> int:
    """Routed experts inside the prefetch list: the page's expert overlap of a
    token is this count over k [APEX Sec. 5.1]."""
    return sum(1 for e in routed if (mask >> int(e)) & 1)


def adaptive_prefetch(x: np.ndarray, w_prefetch: np.ndarray, w_delta: np.ndarray,
                      theta: Sequence[float], tau: float, k: int,
                      routed: Optional[np.ndarray] = None, margin: float = 1e-4):
    """Per token: delta_hat [Sec. 4.2], the top-(k + delta_hat) prefetch mask
    [Sec. 4.1], and, given the router's choices, delta* and the overlap.
    Returns (delta_hat, masks, flags, delta_star or None, overlap or None)."""
    lp = router_logits(x, w_prefetch)
    T = x.shape[0]
    d_hat = np.zeros(T, dtype=np.int32)
    flags = np.zeros(T, dtype=np.uint32)
    masks = []
    for t in range(T):
        d, fb = adaptive_budget(x[t], w_delta, theta, tau, margin)
        m, fp = prefetch_set(lp[t], k + d, margin)
        d_hat[t] = d
        masks.append(m)
        flags[t] = (FLAG_BUDGET if fb else 0) | (FLAG_PREFETCH if fp else 0)
    if routed is None:
        return d_hat, masks, flags, None, None
    ds = np.array([delta_star(routed[t], lp[t], k) for t in range(T)], dtype=np.int32)
    ov = np.array([prefetch_overlap(routed[t], masks[t]) for t in range(T)], dtype=np.int32)
    return d_hat, masks, flags, ds, ov


def stall_free_select(k_routed: Sequence[int], q_r: np.ndarray, k_prefetched: set,
                      margin: float):
    """Stall-free substitution [APEX Sec. 4.3, Algorithm 1].

    Every routed expert that was prefetched is kept; each missing one is
    replaced by the prefetched, not-kept expert with the highest score under
    the ORIGINAL router's softmax alpha = softmax(q_r).  Returns (final set,
    near-tie flag).  The flag is raised when the last chosen substitute and
    the best rejected candidate differ by less than ``margin`` in logits.
    """
    routed = set(k_routed)
    prefetched = set(k_prefetched)
    alpha = softmax(np.asarray(q_r, dtype=np.float64))
    if routed <= prefetched:
        return routed, False
    keep = routed & prefetched
    missing = routed - prefetched
    candidates = sorted(prefetched - keep, key=lambda e: (-alpha[e], e))
    n = len(missing)
    subs = candidates[:n]
    flag = len(candidates) > n and (q_r[candidates[n - 1]] - q_r[candidates[n]]) < margin
    return keep | set(subs), bool(flag)


def stall_free_fill(S: set, q_r: np.ndarray, k: int, margin: float):
    """Completes a stall-free set that Algorithm 1 left short: with fewer
    than k prefetched experts [APEX Sec. 4.3 assumes k + delta >= k] it
    returns the whole prefetched set; the missing k - |S| slots take the
    experts outside S with the highest original-router score (ties -> lower
    id).  Returns (set of k, near-tie flag between the last one taken and the
    next candidate)."""
    S = set(S)
    n = k - len(S)
    if n <= 0:
        return S, False
    rest = sorted((e for e in range(len(q_r)) if e not in S), key=lambda e: (-q_r[e], e))
    flag = len(rest) > n and (q_r[rest[n - 1]] - q_r[rest[n]]) < margin
    return S | set(rest[:n]), bool(flag)


# -------------------------------------------------------------- permutation --
def permute(ids: np.ndarray, exact: np.ndarray, n_experts: int):
    """Token->expert permutation: the exactly computed (token, slot) pairs,
    flattened as f = t*k + j, grouped by expert with f increasing inside each
    group.  Returns (offsets[E+1], perm[P] of f, inv[T*k] with -1 for pairs
    that are not computed exactly)."""
    flat_ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    flat_exact = np.asarray(exact, dtype=bool).reshape(-1)
    groups = [np.nonzero((flat_ids == e) & flat_exact)[0] for e in range(n_experts)]
    counts = np.array([len(g) for g in groups], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = (np.concatenate(groups) if len(groups) else np.zeros(0)).astype(np.int32)
    inv = np.full(flat_ids.shape[0], -1, dtype=np.int32)
    for p, f in enumerate(perm):
        inv[f] = p
    return offsets, perm, inv


# ---------------------------------------------------------------- expert FFN --
def swiglu_expert(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down_hi: np.ndarray) -> np.ndarray:
    """SwiGLU expert FFN on rows of x: (SiLU(x W_gate) * (x W_up)) W_down
    [FloE Sec. 1, sparsified forward with S_t = identity].  w_gate, w_up are
    stored [I][H]; w_down_hi is stored [H][I]."""
    g = x @ w_gate.T
    u = x @ w_up.T
    a = silu(g) * u
    return a @ w_down_hi.T


def dequant_int2(q_packed: np.ndarray, scale_bits: np.ndarray, zero_bits: np.ndarray) -> np.ndarray:
    """Decode 2-bit group-quantised weights [FloE Sec. 1, ultra-low-bit up
    projection]: code of input h is bits 2*(h%4)..2*(h%4)+1 of byte h/4; every
    64 consecutive inputs share an fp16 scale s and zero z; weight = (q - z) * s.
    Shapes: q [..., H/4], s and z [..., H/64] -> [..., H] float64."""
    q = np.asarray(q_packed, dtype=np.uint8)
    codes = np.stack([(q >> (2 * i)) & 3 for i in range(4)], axis=-1)
    codes = codes.reshape(*q.shape[:-1], q.shape[-1] * 4).astype(np.float64)
    s = np.repeat(fp16_to_f64(scale_bits), 64, axis=-1)
    z = np.repeat(fp16_to_f64(zero_bits), 64, axis=-1)
    return (codes - z) * s


def floe_channel_mask(x_t: np.ndarray, up_q, up_scale, up_zero, n_keep: int, margin: float):
    """FloE's channel mask S_t for one (token, expert) [FloE Sec. 1,
    contextual sparsification]: u = x W_up with INT2 W_up; keep the n_keep
    channels of largest |u|, ties to the lower channel.  Returns (keep
    ascending int32, near-tie flag at the mask edge, u)."""
    u = dequant_int2(up_q, up_scale, up_zero) @ x_t
    I = u.shape[0]
    order = sorted(range(I), key=lambda i: (-abs(u[i]), i))
    flag = n_keep < I and (abs(u[order[n_keep - 1]]) - abs(u[order[n_keep]])) < margin
    keep = np.sort(np.array(order[:n_keep], dtype=np.int64))
    return keep.astype(np.int32), bool(flag), u


def floe_predict_masks(h_prev: np.ndarray, ids: np.ndarray, up_q, up_scale, up_zero,
                       n_keep: int, margin: float):
    """FloE intra-expert predictor [FloE, "dual sparsity predictors",
    intra-expert, reuse-based]: the mask of layer l+1 is estimated before its
    input exists by applying the same top-|u| rule to h_l W_up^(l+1), the
    current layer's hidden state times the next layer's own (INT2) up
    projection -- no extra parameters.  ids [T][k] are the next layer's
    experts per token; up_q etc. index [E][I][...].  Returns (keep [T][k][n_keep],
    flags [T] with FLAG_FLOE at a near-tie)."""
    T, k = ids.shape
    keep = np.zeros((T, k, n_keep), dtype=np.int32)
    flags = np.zeros(T, dtype=np.uint32)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            kp, fl, _ = floe_channel_mask(h_prev[t], up_q[e], up_scale[e], up_zero[e], n_keep, margin)
            keep[t, j] = kp
            if fl:
                flags[t] |= FLAG_FLOE
    return keep, flags


def mask_recall(pred: Sequence[int], true: Sequence[int]) -> float:
    """Share of the true kept channels that the predicted set holds (the
    page's recall of the intra-expert predictor)."""
    t = set(int(c) for c in true)
    return len(t & set(int(c) for c in pred)) / len(t) if t else 1.0


def floe_pack(keep: np.ndarray, w_gate_e: np.ndarray, w_down_ih_e: np.ndarray):
    """Compact column packing [FloE, "system co-optimisation": the gate and
    down columns of the selected channels stored aligned so they move as one
    compact block]: the kept channels' gate rows [n_keep][H] and down rows
    [n_keep][H] (both stored channel-major), in the mask's ascending order."""
    kp = np.asarray(keep, dtype=np.int64)
    return np.asarray(w_gate_e)[kp].copy(), np.asarray(w_down_ih_e)[kp].copy()


def floe_expert(x_t: np.ndarray, w_gate: np.ndarray, up_q, up_scale, up_zero,
                w_down_ih: np.ndarray, n_keep: int, margin: float,
                force_keep: Optional[np.ndarray] = None):
    """FloE expert on one token [FloE Sec. 1, contextual sparsification]:
    u = x W_up with INT2 W_up; S_t keeps the n_keep channels of largest |u|
    (ties -> lower channel) and zeroes the rest; gate is applied only where
    kept; y = (SiLU(x W_gate) * S_t(u)) W_down.  w_gate is [I][H]; w_down_ih is
    [I][H] (channel rows).  Returns (y[H], u[I], keep ascending, flag)."""
    w_up = dequant_int2(up_q, up_scale, up_zero)
    u = w_up @ x_t
    I = u.shape[0]
    order = sorted(range(I), key=lambda i: (-abs(u[i]), i))
    flag = n_keep < I and (abs(u[order[n_keep - 1]]) - abs(u[order[n_keep]])) < margin
    keep = np.sort(np.array(order[:n_keep], dtype=np.int64)) if force_keep is None \
        else np.sort(np.asarray(force_keep, dtype=np.int64))
    g = w_gate[keep] @ x_t
    a = silu(g) * u[keep]
    y = a @ w_down_ih[keep]
    return y, u, keep.astype(np.int32), bool(flag)


def shared_experts(x: np.ndarray, ws_gate, ws_up, ws_down_hi, w_shared_gate=None):
    """Always-active shared experts [SPICE "LoRE low-rank surrogate": the shared
    expert is active for every token]: y_s = sum over shared experts of their
    SwiGLU FFN; gate g_s = sigmoid(x . w_sg) when the layer has a scalar shared
    gate, else 1.  Returns (y_s [T][H], g_s [T])."""
    T, H = x.shape
    y = np.zeros((T, H))
    for s in range(len(ws_gate)):
        y += swiglu_expert(x, ws_gate[s], ws_up[s], ws_down_hi[s])
    g = sigmoid(x @ w_shared_gate) if w_shared_gate is not None else np.ones(T)
    return y, g


def lore_targets(h: np.ndarray, w_gate_e, w_up_e, w_down_e, ws_gate, ws_up, ws_down) -> np.ndarray:
    """What LoRE must reproduce for expert e on calibration inputs h [N][H]
    [SPICE "LoRE low-rank surrogate": collect each expert's inputs and
    outputs and the shared experts' output]: y_e(h) - y_shared(h)."""
    y_e = swiglu_expert(h, w_gate_e, w_up_e, w_down_e)
    y_s, _ = shared_experts(h, ws_gate, ws_up, ws_down)
    return y_e - y_s


def lore_fit(h: np.ndarray, resid: np.ndarray, r: int):
    """LoRE fitting [SPICE "LoRE low-rank surrogate": minimise
    ||y_e - y_shared - B_e A_e h||^2 over the calibration set, solved by an
    SVD].  With R = resid [N][H_out] and the calibration inputs h [N][H_in]
    (full column rank), the objective is ||R - h W^T||_F^2 over maps W of
    rank <= r.  Writing G = h^T h / N and M = R^T h / N (the least-squares
    map is M G^-1), the objective equals N ||(W - M G^-1) G^1/2||_F^2 plus a
    constant, so the minimiser truncates the SVD of the whitened map
    M G^-1/2 = U S V^T (Eckart-Young) and maps back: W = U_r S_r V_r^T G^-1/2.
    G^-1/2 comes from the symmetric eigendecomposition of G.
    Returns (A = V_r^T G^-1/2 [r][H_in], B = U_r S_r [H_out][r], the r
    singular values of M G^-1/2, and the relative residual
    ||R - h (B A)^T||_F / ||R||_F on the calibration set)."""
    h = np.asarray(h, dtype=np.float64)
    R = np.asarray(resid, dtype=np.float64)
    N = h.shape[0]
    G = h.T @ h / N
    lam, Q = np.linalg.eigh(G)
    G_mhalf = (Q / np.sqrt(lam)) @ Q.T
    M = R.T @ h / N
    U, S, Vt = np.linalg.svd(M @ G_mhalf)
    B = U[:, :r] * S[:r]
    A = Vt[:r] @ G_mhalf
    pred = h @ (B @ A).T
    err = float(np.linalg.norm(R - pred) / np.linalg.norm(R))
    return A, B, S[:r].copy(), err


def lore_residual(x_t: np.ndarray, lore_a: np.ndarray, lore_b: np.ndarray) -> np.ndarray:
    """LoRE low-rank residual B_e (A_e h) with A_e [r][H], B_e [H][r] [SPICE
    "LoRE low-rank surrogate"]."""
    return lore_b @ (lore_a @ x_t)


# ------------------------------------------- missed experts: fetch or host --
OFFLOAD_NONE, OFFLOAD_FETCH, OFFLOAD_HOST = 0, 1, 2


def offload_costs(weight_bytes: float, hidden_bytes: float, n_pairs: int,
                  pcie_bytes_per_s: float, gpu_expert_s: float, cpu_pair_s: float,
                  cpu_expert_s: float = 0.0):
    """(fetch cost, host cost) in seconds of one missed expert [SPICE
    "CPU-GPU collaboration: handling prefetch misses", the per-expert cost
    comparison]: fetching moves the weights over the link and then runs the
    expert on the GPU; host execution runs it on the CPU (a fixed time per
    expert plus a time per routed pair) and moves each routed token's hidden
    state down and its output back."""
    fetch = weight_bytes / pcie_bytes_per_s + gpu_expert_s
    t_cpu = cpu_expert_s + n_pairs * cpu_pair_s
    host = t_cpu + 2 * n_pairs * hidden_bytes / pcie_bytes_per_s
    return fetch, host


def offload_plan(dims: dict, tokens: Sequence[int], resident: int, pcie_bytes_per_s: float,
                 gpu_expert_s: float, cpu_pair_s: float, cpu_expert_s: float = 0.0,
                 queue_aware: bool = False) -> List[int]:
    """Decision per expert: OFFLOAD_NONE (resident or not routed),
    OFFLOAD_FETCH when the fetch cost is strictly below the host cost, else
    OFFLOAD_HOST [SPICE "CPU-GPU collaboration: handling prefetch misses"].
    tokens[e] = routed (token, expert) pairs of expert e.

    queue_aware: the link and the host are queues ("PCIe pressure", Fig. 6
    of the same section): missed experts are taken by decreasing pair count
    (then id) and each side's cost includes what earlier decisions already
    put on that side."""
    elem = 2 if dims["dtype"] == "bf16" else 4
    w_bytes = 3 * dims["inter"] * dims["hidden"] * elem
    h_bytes = dims["hidden"] * elem
    out = [OFFLOAD_NONE] * len(tokens)
    missed = [e for e, n in enumerate(tokens) if n > 0 and not (resident >> e) & 1]
    if queue_aware:
        missed.sort(key=lambda e: (-tokens[e], e))
    link_busy = host_busy = 0.0
    for e in missed:
        fetch, host = offload_costs(w_bytes, h_bytes, tokens[e], pcie_bytes_per_s, gpu_expert_s,
                                    cpu_pair_s, cpu_expert_s)
        if queue_aware:
            fetch += link_busy
            host += host_busy
        if fetch < host:
            out[e] = OFFLOAD_FETCH
            link_busy = fetch
        else:
            out[e] = OFFLOAD_HOST
            host_busy = host
    return out


# ---------------------------------------------------------- weight access --
class WeightSource:
    """Uniform access to a layer's weights in storage form.

    ``src`` is either a mapping name -> stacked array, or an object with
    ``expert(name, e)`` (per-expert draw) plus ``w_router()`` etc."""

    def __init__(self, src, dtype: str, compute=np.float64):
        self.src = src
        self.dtype = dtype
        self.compute = compute
        self._memo: Dict = {}

    def small(self, name: str):
        if isinstance(self.src, dict):
            v = self.src.get(name)
        else:
            v = getattr(self.src, name)() if hasattr(self.src, name) else None
        return v

    def expert(self, name: str, e: int):
        if isinstance(self.src, dict):
            return self.src[name][e]
        return self.src.expert(name, e)

    def f64(self, name: str, e: int) -> np.ndarray:
        """Decoded float64 copy; small tensors are kept, large ones re-decoded
        on each request so a sampled forward of a large layer stays small."""
        key = (name, e)
        if key in self._memo:
            return self._memo[key]
        v = decode(self.expert(name, e), self.dtype).astype(self.compute, copy=False)
        if v.nbytes <= (1 << 22):
            self._memo[key] = v
        return v


# ------------------------------------------------------------- layer forward --
def layer_forward(x, weights, dims: dict, mode: str, resident=None,
                  force: Optional[dict] = None, tie_margin: float = 1e-4,
                  precision: str = "f64") -> dict:
    """One MoE layer forward, every step in fp64 (``precision="f32"`` runs
    the same steps on float32 copies of the decoded inputs: the timed CPU
    baseline, never a parity reference).

    x: [T][H] storage (bf16 bits or fp32); weights: mapping or per-expert source;
    dims: hidden, n_experts, top_k, inter, n_shared, shared_inter, lore_rank,
    renormalize, shared_gate, dtype, up_format, floe_keep.
    resident: int bit mask (one for all tokens) or a length-T sequence of masks
    (per token; the APEX prefetched set in mode stall_free).
    force: optional {"ids": {t: final ids}, "keep": {(t, j): channels}} to
    re-run with decisions taken elsewhere at flagged near-ties.

    Steps: router logits -> softmax -> top-k [APEX Sec. 1]; stall-free
    substitution [APEX Sec. 4.3]; residency split and LoRE surrogate for
    non-resident experts [SPICE "LoRE low-rank surrogate"]; permutation;
    SwiGLU experts, FloE experts [FloE Sec. 1]; shared experts; weighted
    combine out = g_s y_s + sum_j w_j yhat_j.
    """
    assert mode in MODES, mode
    force = force or {}
    dt = dims["dtype"]
    H, E, k = dims["hidden"], dims["n_experts"], dims["top_k"]
    cdt = {"f64": np.float64, "f32": np.float32}[precision]
    src = weights if isinstance(weights, WeightSource) else WeightSource(weights, dt, cdt)
    X = decode(x, dt).astype(cdt, copy=False)
    T = X.shape[0]
    w_router = decode(src.small("w_router"), dt).astype(cdt, copy=False)
    logits = router_logits(X, w_router)
    probs = softmax(logits)

    if resident is None:
        res = [(1 << E) - 1] * T
    elif isinstance(resident, (int, np.integer)):
        res = [int(resident)] * T
    else:
        res = [int(m) for m in resident]

    ids = np.zeros((T, k), dtype=np.int32)
    wts = np.zeros((T, k))
    mass = np.zeros(T)
    flags = np.zeros(T, dtype=np.uint32)
    n_subst = np.zeros(T, dtype=np.int32)
    for t in range(T):
        r_ids, r_w, m, f = route_token(logits[t], k, dims["renormalize"], tie_margin)
        mass[t] = m
        flags[t] |= FLAG_ROUTE if f else 0
        final = list(r_ids)
        if mode == "stall_free":
            kp = {e for e in range(E) if (res[t] >> e) & 1}
            S, fs = stall_free_select(r_ids, logits[t], kp, tie_margin)
            flags[t] |= FLAG_SUBST if fs else 0
            if len(S) < k:
                S, ff = stall_free_fill(S, logits[t], k, tie_margin)
                flags[t] |= FLAG_SHORT | (FLAG_SUBST if ff else 0)
            final = sorted(S, key=lambda e: (-logits[t][e], e))
            n_subst[t] = len(set(final) - set(r_ids))
        if t in force.get("ids", {}):
            final = [int(e) for e in force["ids"][t]]
        ids[t] = final
        pw = np.array([probs[t][e] for e in final])
        wts[t] = pw / pw.sum() if dims["renormalize"] else pw

    if mode == "lore":
        exact = np.array([[(res[t] >> int(ids[t, j])) & 1 for j in range(k)] for t in range(T)],
                         dtype=np.uint8)
    else:
        exact = np.ones((T, k), dtype=np.uint8)

    offsets, perm, inv = permute(ids, exact, E)

    # routed experts, exact pairs (grouped by expert; each pair is independent)
    y_pair = np.zeros((len(perm), H))
    floe_keep: Dict = {}
    floe_u: Dict = {}
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        if len(seg) == 0:
            continue
        toks = seg // k
        if mode == "floe":
            wg = src.f64("w_gate", e)
            wd = src.f64("w_down", e)
            for pos, f in zip(range(offsets[e], offsets[e + 1]), seg):
                t, j = int(f) // k, int(f) % k
                y, u, keep, fl = floe_expert(
                    X[t], wg, src.expert("up_q", e), src.expert("up_scale", e),
                    src.expert("up_zero", e), wd, dims["floe_keep"], tie_margin,
                    force.get("keep", {}).get((t, j)))
                y_pair[pos] = y
                floe_keep[(t, j)] = keep
                floe_u[(t, j)] = u
                flags[t] |= FLAG_FLOE if fl else 0
        else:
            y_pair[offsets[e]:offsets[e + 1]] = swiglu_expert(
                X[toks], src.f64("w_gate", e), src.f64("w_up", e), src.f64("w_down", e))

    # shared experts
    if dims["n_shared"] > 0:
        ws_g = [src.f64("ws_gate", s) for s in range(dims["n_shared"])]
        ws_u = [src.f64("ws_up", s) for s in range(dims["n_shared"])]
        ws_d = [src.f64("ws_down", s) for s in range(dims["n_shared"])]
        wsg = decode(src.small("w_shared_gate"), dt).astype(cdt, copy=False) if dims["shared_gate"] else None
        y_shared, g_shared = shared_experts(X, ws_g, ws_u, ws_d, wsg)
    else:
        y_shared, g_shared = np.zeros((T, H)), np.zeros(T)

    # LoRE residuals for non-exact slots
    lore = np.zeros((T, k, H))
    for t in range(T):
        for j in range(k):
            if not exact[t, j]:
                e = int(ids[t, j])
                lore[t, j] = lore_residual(X[t], src.f64("lore_A", e), src.f64("lore_B", e))

    # weighted combine
    out = np.zeros((T, H))
    for t in range(T):
        acc = g_shared[t] * y_shared[t]
        for j in range(k):
            if exact[t, j]:
                yj = y_pair[inv[t * k + j]]
            else:
                yj = y_shared[t] + lore[t, j]
            acc = acc + wts[t, j] * yj
        out[t] = acc

    return dict(out=out, logits=logits, probs=probs, ids=ids, weights=wts, mass=mass,
                flags=flags, exact=exact, offsets=offsets, perm=perm, inv=inv,
                y_pair=y_pair, y_shared=y_shared, g_shared=g_shared, lore=lore,
                floe_keep=floe_keep, floe_u=floe_u, n_subst=n_subst)
