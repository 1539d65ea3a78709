"""Shared helpers for the GPU parity tests: run the HIP layer through the C
ABI, run the oracle on the same inputs, and compare.

Decisions (expert ids, permutation, substitution, FloE channel sets) are
compared bit for bit where the oracle finds no near-tie; at a flagged near-tie
the GPU's decision must be admissible (within the margin of the oracle's), and
the oracle is re-run with the GPU's decisions so the outputs are still
compared.  Outputs are compared by relative Frobenius error.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle as O
import workloads as W
from workloads.device import dims_dict, mask_tensor, tensor, upload

import sparse_moe_layer_route_amd as M

TOL = {"f32": 1e-5, "bf16": 1e-2}
MARGIN = 1e-4

_dev_cache: Dict = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_weights(layer: W.Layer):
    key = (layer.cfg, layer.seed)
    if key not in _dev_cache:
        _dev_cache.clear()  # one layer's weights (and their packed copy) at a time
        torch.cuda.empty_cache()
        _dev_cache[key] = upload(layer, "cuda")
    return _dev_cache[key]


def default_layout(cfg) -> str:
    """The layout the bench runs: fragment-major expert matrices wherever the
    matrix-core kernels run (bf16, dense up), row-major elsewhere."""
    return "mfma16" if cfg.dtype == "bf16" and cfg.up_format == "dense" else "rows"


def packed_weights(layer: W.Layer, wdev=None):
    """The device weights with the expert matrices packed by moe_pack_weights
    (cached beside dev_weights when wdev is the layer's own)."""
    own = wdev is None
    wdev = dev_weights(layer) if own else wdev
    key = ("packed", layer.cfg, layer.seed)
    if own and key in _dev_cache:
        return _dev_cache[key]
    packed = M.pack_weights(M.Dims(**dims_dict(layer.cfg)), wdev)
    torch.cuda.synchronize()
    if own:
        _dev_cache[key] = packed
    return packed


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def out_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class GpuResult:
    out: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    exact: np.ndarray
    flags: np.ndarray
    logits: np.ndarray
    mass: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray
    keep: Optional[np.ndarray]
    masks: Optional[list]


def prefetch_masks_gpu(layer: W.Layer, T: int, wdev, delta=None):
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg))
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    d = torch.from_numpy(np.ascontiguousarray(layer.delta(T) if delta is None else delta)
                         .astype(np.int32)).cuda()
    mask = torch.empty(T, dtype=torch.int64, device="cuda")
    flags = torch.empty(T, dtype=torch.int32, device="cuda")
    M.moe_prefetch_mask(dims, T, x, wdev["w_prefetch"], d, mask, flags)
    torch.cuda.synchronize()
    masks = [int(v) for v in mask.cpu().numpy().view(np.uint64)]
    return masks, flags.cpu().numpy().view(np.uint32), mask


def prefetch_adaptive_gpu(layer: W.Layer, T: int, wdev, tau: float, theta=None, routed=None):
    """moe_prefetch_adaptive on the first T rows; returns (delta, masks,
    flags, delta_star or None, overlap or None) as numpy / int lists."""
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg))
    w_delta, th = layer.ordinal(tau)
    th = th if theta is None else np.asarray(theta, np.float32)
    # buffers hold at least one row, so T = 0 still passes valid pointers
    x = tensor(layer.x(max(T, 1)), cfg.dtype, "cuda")
    wd = tensor(w_delta, cfg.dtype, "cuda")
    th_d = torch.from_numpy(np.ascontiguousarray(th, np.float32)).cuda()
    delta = torch.full((max(T, 1),), -7, dtype=torch.int32, device="cuda")
    mask = torch.empty(max(T, 1), dtype=torch.int64, device="cuda")
    flags = torch.empty(max(T, 1), dtype=torch.int32, device="cuda")
    ids = ds = ov = None
    if routed is not None:
        ids = torch.zeros(max(T, 1) * cfg.top_k, dtype=torch.int32, device="cuda")
        ids[:T * cfg.top_k] = torch.from_numpy(np.ascontiguousarray(routed, np.int32).reshape(-1))
        ds = torch.full((max(T, 1),), -7, dtype=torch.int32, device="cuda")
        ov = torch.full((max(T, 1),), -7, dtype=torch.int32, device="cuda")
    M.moe_prefetch_adaptive(dims, T, x, wdev["w_prefetch"], wd, th_d, tau, delta, mask, flags,
                            topk_ids=ids, delta_star=ds, overlap=ov)
    torch.cuda.synchronize()
    masks = [int(v) for v in mask[:T].cpu().numpy().view(np.uint64)]
    return (delta[:T].cpu().numpy(), masks, flags[:T].cpu().numpy().view(np.uint32),
            None if ds is None else ds[:T].cpu().numpy(), None if ov is None else ov[:T].cpu().numpy())


def run_layer(layer: W.Layer, T: int, mode: str, wdev=None, dims_over=None,
              resident_masks=None, x_np=None, layout="rows") -> GpuResult:
    """moe_layer_forward on the first T rows of the layer's x; layout
    "mfma16" packs the expert matrices (of wdev, or the layer's own) first."""
    cfg = layer.cfg
    dd = dims_dict(cfg, **(dims_over or {}))
    dims = M.Dims(**dd, weight_layout=layout)
    wdev = wdev if wdev is not None else dev_weights(layer)
    if layout == "mfma16":
        wdev = packed_weights(layer, None if wdev is _dev_cache.get((cfg, layer.seed)) else wdev)
    x_np = layer.x(T) if x_np is None else x_np
    x = tensor(x_np, cfg.dtype, "cuda")
    k, E, H = dd["top_k"], dd["n_experts"], dd["hidden"]
    masks = None
    if mode == "lore":
        res = mask_tensor([layer.resident()], "cuda"); stride = 0
    elif mode == "stall_free":
        if resident_masks is None:
            masks, _, res = prefetch_masks_gpu(layer, T, wdev)
        else:
            masks = list(resident_masks); res = mask_tensor(masks, "cuda")
        stride = 1
    else:
        res = None; stride = 0
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if dd["dtype"] == "f32" else torch.bfloat16
    out = torch.empty(T, H, dtype=odt, device="cuda")
    dbg = dict(topk_ids=torch.empty(T * k, dtype=torch.int32, device="cuda"),
               topk_w=torch.empty(T * k, dtype=torch.float32, device="cuda"),
               exact=torch.empty(T * k, dtype=torch.uint8, device="cuda"),
               flags=torch.empty(T, dtype=torch.int32, device="cuda"),
               logits=torch.empty(T * E, dtype=torch.float32, device="cuda"),
               mass=torch.empty(T, dtype=torch.float32, device="cuda"),
               expert_offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               perm=torch.empty(max(T * k, 1), dtype=torch.int32, device="cuda"))
    if mode == "floe":
        dbg["floe_keep"] = torch.empty(T * k * dd["floe_keep"], dtype=torch.int32, device="cuda")
    M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, out, ws, debug=dbg)
    torch.cuda.synchronize()
    g = {n: t.cpu().numpy() for n, t in dbg.items()}
    keep = g["floe_keep"].reshape(T, k, dd["floe_keep"]) if mode == "floe" else None
    return GpuResult(out=out_to_np(out), ids=g["topk_ids"].reshape(T, k), w=g["topk_w"].reshape(T, k),
                  exact=g["exact"].reshape(T, k), flags=g["flags"].view(np.uint32),
                  logits=g["logits"].reshape(T, E), mass=g["mass"], offsets=g["expert_offsets"],
                  perm=g["perm"][: int(g["expert_offsets"][E])], keep=keep, masks=masks)


def admissible_topk(l: np.ndarray, chosen: Sequence[int], allowed: Sequence[int], margin: float) -> bool:
    """chosen is a top-|chosen| set of l over `allowed` up to the margin."""
    chosen = set(int(e) for e in chosen)
    if not chosen <= set(allowed):
        return False
    rest = [e for e in allowed if e not in chosen]
    if not rest:
        return True
    return min(l[e] for e in chosen) >= max(l[e] for e in rest) - margin


def _flag_gap_ok(gap: float) -> bool:
    """A flag that one side raises and the other does not must sit on its own
    threshold: the oracle's fp64 gap within 1% of the margin (fp32 logits
    carry about 1e-7 of rounding)."""
    return abs(gap - MARGIN) < 1e-2 * MARGIN


def check_decisions(layer: W.Layer, T: int, mode: str, g: GpuResult, dims_over=None,
                    x_np=None) -> dict:
    """Routing decisions for all T tokens: bit-exact unless the oracle flags a
    near-tie; admissible otherwise.  The GPU's flag bits 1 (route near-tie),
    4 (substitution near-tie) and 32 (short prefetched set) match the
    oracle's, except where the deciding gap sits on the margin itself.
    Returns counts."""
    cfg = layer.cfg
    dd = dims_dict(cfg, **(dims_over or {}))
    k, E = dd["top_k"], dd["n_experts"]
    X = O.decode(layer.x(T) if x_np is None else x_np, dd["dtype"])
    l = O.router_logits(X, O.decode(layer.w_router(), dd["dtype"]))
    np.testing.assert_allclose(g.logits, l, rtol=1e-4, atol=2e-5 * max(1.0, np.abs(l).max()))
    n_flag = n_exact = n_sub = n_short = 0
    res = layer.resident()
    for t in range(T):
        ids, w, mass, fl = O.route_token(l[t], k, dd["renormalize"], MARGIN)
        order = O.rank_experts(l[t])
        final, f2, short = list(ids), False, False
        gaps = {1: l[t][order[k - 1]] - l[t][order[k]] if k < E else np.inf}
        if mode == "stall_free":
            kp = {e for e in range(E) if (g.masks[t] >> e) & 1}
            S, f2 = O.stall_free_select(ids, l[t], kp, MARGIN)
            if len(S) < k:
                short = True
                n_short += 1
                S, f2 = O.stall_free_fill(S, l[t], k, MARGIN)
                rest = [e for e in order if e not in kp]
                need = k - len(kp)
                gaps[4] = l[t][rest[need - 1]] - l[t][rest[need]] if len(rest) > need else np.inf
            elif not set(ids) <= kp:
                cand = [e for e in order if e in kp]
                gaps[4] = l[t][cand[k - 1]] - l[t][cand[k]] if len(cand) > k else np.inf
            final = sorted(S, key=lambda e: (-l[t][e], e))
            n_sub += len(set(final) - set(ids))
        gids = [int(e) for e in g.ids[t]]
        if fl or f2:
            n_flag += 1
            if mode == "stall_free" and short:
                # every prefetched expert kept, the rest a top set of the others
                assert kp <= set(gids), (t, gids, final)
                assert admissible_topk(l[t], [e for e in gids if e not in kp],
                                       [e for e in range(E) if e not in kp], MARGIN), (t, gids, final)
            elif mode == "stall_free" and not set(ids) <= kp:
                assert admissible_topk(l[t], gids, sorted(kp), MARGIN), (t, gids, final)
            elif mode == "stall_free":
                # a route near-tie decides whether a substitution happens at all
                assert admissible_topk(l[t], gids, sorted(kp), MARGIN) or \
                    admissible_topk(l[t], gids, list(range(E)), MARGIN), (t, gids, final)
            else:
                assert admissible_topk(l[t], gids, list(range(E)), MARGIN), (t, gids, final)
        else:
            n_exact += 1
            assert gids == final, (t, gids, final)
        # flag bits against the oracle's
        want = (O.FLAG_ROUTE if fl else 0) | (O.FLAG_SUBST if f2 else 0) | (O.FLAG_SHORT if short else 0)
        got = int(g.flags[t]) & (O.FLAG_ROUTE | O.FLAG_SUBST | O.FLAG_SHORT)
        for bit in (O.FLAG_ROUTE, O.FLAG_SUBST):
            if (got ^ want) & bit:
                if bit == O.FLAG_SUBST and fl:
                    continue  # a route near-tie decides whether anything is substituted
                assert bit in gaps and _flag_gap_ok(gaps[bit]), (t, bit, got, want, gaps)
        assert bool(got & O.FLAG_SHORT) == short, t
        # slots are ordered by (-logit, id)
        assert all((l[t][gids[j]], -gids[j]) >= (l[t][gids[j + 1]], -gids[j + 1]) for j in range(k - 1)) \
            or (fl or f2)
        # weights = softmax of the GPU's decisions
        p = O.softmax(l[t])
        pw = np.array([p[e] for e in gids])
        if dd["renormalize"]:
            pw = pw / pw.sum()
        np.testing.assert_allclose(g.w[t], pw, rtol=2e-5, atol=1e-7)
        if mode != "stall_free":
            np.testing.assert_allclose(g.mass[t], sum(p[e] for e in ids), rtol=2e-5)
        ex = [((res >> e) & 1) if mode == "lore" else 1 for e in gids]
        assert list(g.exact[t]) == ex
    # permutation is a pure function of the GPU's ids / exact: bit-exact
    off, perm, inv = O.permute(g.ids, g.exact, E)
    np.testing.assert_array_equal(g.offsets, off)
    np.testing.assert_array_equal(g.perm, perm)
    return dict(flagged=n_flag, exact=n_exact, substituted_slots=n_sub, short_sets=n_short)


def oracle_forward_forced(layer: W.Layer, T: int, mode: str, g: GpuResult, sample: Sequence[int],
                          dims_over=None, weights=None, x_np=None):
    """The oracle on tokens `sample`, with the GPU's routing (and FloE mask)
    decisions forced, so a near-tie cannot split the comparison."""
    cfg = layer.cfg
    dd = dims_dict(cfg, **(dims_over or {}))
    x = (layer.x(T) if x_np is None else x_np)[list(sample)]
    src = weights if weights is not None else layer
    force = {"ids": {i: list(g.ids[t]) for i, t in enumerate(sample)}}
    if g.keep is not None:
        force["keep"] = {(i, j): g.keep[t, j] for i, t in enumerate(sample) for j in range(dd["top_k"])}
    res = layer.resident()
    if mode == "stall_free":
        res = [g.masks[t] for t in sample]
    return O.layer_forward(x, src, dd, mode, resident=res, force=force, tie_margin=MARGIN)


def check_floe_masks(layer: W.Layer, g: GpuResult, ref: dict, sample: Sequence[int]):
    """FloE kept channels: exact where the oracle sees no near-tie at the
    mask edge; admissible within the margin otherwise.  Flag bit 8 of a token
    matches the oracle's (some pair of the token at a near-tie), except where
    that pair's gap sits on the margin itself."""
    n_keep = g.keep.shape[2]
    n_tie = 0
    for i, t in enumerate(sample):
        any_edge, gaps = False, []
        for j in range(layer.cfg.top_k):
            u = ref["floe_u"][(i, j)]
            gk = np.asarray(g.keep[t, j])
            order = sorted(range(len(u)), key=lambda c: (-abs(u[c]), c))
            want = np.sort(order[:n_keep])
            gap = abs(u[order[n_keep - 1]]) - abs(u[order[n_keep]]) if n_keep < len(u) else np.inf
            edge = gap < MARGIN
            gaps.append(gap)
            any_edge |= edge
            assert np.all(np.diff(gk) > 0), "kept channels ascending and distinct"
            if edge:
                n_tie += 1
                mask = np.zeros(len(u), bool); mask[gk] = True
                assert np.abs(u[mask]).min() >= np.abs(u[~mask]).max() - MARGIN
            else:
                np.testing.assert_array_equal(gk, want)
        if bool(g.flags[t] & O.FLAG_FLOE) != any_edge:
            assert any(abs(gp - MARGIN) < 1e-2 * MARGIN for gp in gaps), (t, gaps)
    return n_tie
