"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs ``moe_layer_forward`` (or the individual entry points) on
seeded synthetic inputs, then checks decisions bit for bit (admissibility at
flagged near-ties) and outputs by relative Frobenius error (1e-5 for fp32,
1e-2 for bf16 with fp32 accumulation).  Full-size workloads compare every
token's decisions and every output row.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads.device import dims_dict, mask_tensor, tensor

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the -m gpu suite needs a GPU
    pytest.skip("no GPU", allow_module_level=True)

import sparse_moe_layer_route_amd as M  # noqa: E402
from gpu_harness import (MARGIN, TOL, check_decisions, check_floe_masks, default_layout,  # noqa: E402
                         dev_weights, oracle_forward_forced, packed_weights, prefetch_adaptive_gpu, prefetch_masks_gpu, rel_fro,
                         run_layer, say)


def _variant(base, **kw):
    return dataclasses.replace(W.CONFIGS[base], **kw)


# Small layers that still span several row tiles and end on ragged tails.
SMALL = {
    "tiny": W.CONFIGS["tiny"],
    "dsv2_small": _variant("dsv2_lite", name="dsv2_small", hidden=512, n_experts=16, top_k=4,
                           inter=384, shared_inter=256, token_counts=(37,), resident_count=8,
                           seed=101),
    "qwen2_small": _variant("qwen2_57b", name="qwen2_small", hidden=640, n_experts=24, top_k=8,
                            inter=320, shared_inter=1040, token_counts=(29,), resident_count=6,
                            seed=102),
    "granite_small": _variant("granite_prefill", name="granite_small", hidden=384, n_experts=40,
                              inter=144, token_counts=(203,), seed=103),
    # prefill-sized segments (grouped GEMM path): ~150 tokens per expert,
    # ragged m- and n-tiles, a shared expert of 320 channels over 300 tokens
    "prefill_small": _variant("dsv2_lite", name="prefill_small", hidden=256, n_experts=4, top_k=2,
                              inter=192, n_shared=1, shared_inter=320, token_counts=(300,),
                              resident_count=2, seed=106),
    # long routed segments on the decode kernels (more than one 16-token
    # tile per expert, at most four): gate/up waves with two row tiles,
    # down waves with four; ragged intermediate sizes
    "long_seg": _variant("qwen2_57b", name="long_seg", hidden=640, n_experts=8, top_k=4,
                         inter=336, shared_inter=528, token_counts=(64,), resident_count=4,
                         seed=108),
    # 65-128 tokens with the shared experts on the decode kernels: eight
    # 16-token tiles, two row strips x two k-splits per block
    # prefetch router and budget model on an fp32 layer, and on the full
    # DeepSeek-V2-Lite shape (64 experts: every lane of the ranking wave live)
    "f32_prefetch": _variant("tiny", name="f32_prefetch", n_experts=16, prefetch=True,
                             token_counts=(23,), seed=109),
    "dsv2_prefetch": _variant("dsv2_lite", name="dsv2_prefetch", prefetch=True,
                              token_counts=(64,), seed=110),
    "dsv2_t100": _variant("dsv2_lite", name="dsv2_t100", hidden=512, n_experts=16, top_k=4,
                          inter=384, shared_inter=256, token_counts=(100,), resident_count=8,
                          seed=107),
}
FLOE_SMALL = {
    "floe_small": _variant("mixtral_floe", name="floe_small", hidden=1024, n_experts=4, inter=1040,
                           floe_keep=104, token_counts=(5,), seed=104),
    "floe_wide": _variant("mixtral_floe", name="floe_wide", hidden=8192, n_experts=4, inter=512,
                          floe_keep=51, token_counts=(3,), seed=105),
    # FloE routed experts beside dense gated shared experts, bf16 and fp32
    "floe_shared": _variant("mixtral_floe", name="floe_shared", hidden=1024, n_experts=4,
                            inter=1040, floe_keep=104, n_shared=2, shared_inter=256,
                            shared_gate=True, token_counts=(7,), seed=111),
    "floe_shared_f32": _variant("mixtral_floe", name="floe_shared_f32", hidden=512, n_experts=4,
                                inter=528, floe_keep=53, n_shared=1, shared_inter=256,
                                dtype="f32", token_counts=(6,), seed=112),
    # the FloE limits: I = 16384 (16 channels per select thread, |u| row filling its LDS
    # stage) and H = 16384 (the packed x row of the up kernel)
    "floe_max_inter": _variant("mixtral_floe", name="floe_max_inter", hidden=512, n_experts=4,
                               inter=16384, floe_keep=1639, token_counts=(2,), seed=114),
    "floe_max_hidden": _variant("mixtral_floe", name="floe_max_hidden", hidden=16384, n_experts=4,
                                inter=256, floe_keep=26, token_counts=(2,), seed=115),
}


def _check_full(layer, T, mode, sample=None, dims_over=None, layout=None):
    layout = default_layout(layer.cfg) if layout is None else layout
    say(f"[parity] {layer.cfg.name} T={T} mode={mode} layout={layout}")
    g = run_layer(layer, T, mode, dims_over=dims_over, layout=layout)
    counts = check_decisions(layer, T, mode, g, dims_over=dims_over)
    sample = list(range(T)) if sample is None else sample
    ref = oracle_forward_forced(layer, T, mode, g, sample, dims_over=dims_over)
    err = rel_fro(g.out[sample], ref["out"])
    tol = TOL[dims_dict(layer.cfg, **(dims_over or {}))["dtype"]]
    # every row on its own too (a bad tile cannot hide in the whole-matrix norm)
    rows = [rel_fro(g.out[t], ref["out"][i]) for i, t in enumerate(sample)]
    say(f"    rel_fro={err:.3e} worst row {max(rows):.3e} tol={tol} decisions={counts}")
    assert np.all(np.isfinite(g.out))
    assert err <= tol, err
    assert max(rows) <= 3 * tol, (int(np.argmax(rows)), max(rows))
    if mode == "floe":
        check_floe_masks(layer, g, ref, sample)
    return g, ref


# ------------------------------------------------------------ small layers --
@pytest.mark.parametrize("name,mode", [
    ("tiny", "standard"), ("tiny", "lore"),
    ("dsv2_small", "standard"), ("dsv2_small", "lore"),
    ("qwen2_small", "standard"), ("qwen2_small", "lore"),
    ("granite_small", "standard"), ("granite_small", "stall_free"),
    ("prefill_small", "standard"), ("prefill_small", "lore"),
    ("dsv2_t100", "standard"), ("dsv2_t100", "lore"),
    ("long_seg", "standard"), ("long_seg", "lore"),
])
def test_small_layer_parity(name, mode):
    layer = W.Layer(SMALL[name])
    _check_full(layer, layer.cfg.t_max, mode)
    if default_layout(layer.cfg) != "rows":  # the row-major expert matrices too
        _check_full(layer, layer.cfg.t_max, mode, layout="rows")


@pytest.mark.parametrize("name", ["floe_small", "floe_wide", "floe_shared", "floe_shared_f32",
                                  "floe_max_inter", "floe_max_hidden"])
def test_floe_small_parity(name):
    layer = W.Layer(FLOE_SMALL[name])
    _check_full(layer, layer.cfg.t_max, "floe")


@pytest.mark.parametrize("keep", [1, 1040])
def test_floe_keep_extremes(keep):
    """keep = 1 (single channel) and keep = I (dense FFN on decoded up weights)."""
    layer = W.Layer(FLOE_SMALL["floe_small"])
    _check_full(layer, 5, "floe", dims_over={"floe_keep": keep})


@pytest.mark.parametrize("seed", [201, 202, 203])
def test_extra_seeds(seed):
    layer = W.Layer(dataclasses.replace(SMALL["dsv2_small"], seed=seed, token_counts=(19,)))
    _check_full(layer, 19, "lore")


# ----------------------------------------------------- full-size workloads --
@pytest.mark.parametrize("T", [1, 8, 64])
@pytest.mark.parametrize("mode", ["standard", "lore"])
def test_dsv2_lite(T, mode):
    layer = W.make_layer("dsv2_lite")
    _check_full(layer, T, mode)


@pytest.mark.parametrize("mode", ["standard", "lore"])
def test_dsv2_lite_long_segments(mode):
    """256 tokens: 24 pairs per routed expert on average, so the decode
    kernels take their long-segment form (two row strips per block, each
    wave over half of K), and the shared experts run on the grouped GEMM."""
    cfg = dataclasses.replace(W.CONFIGS["dsv2_lite"], token_counts=(256,))
    _check_full(W.Layer(cfg), 256, mode)


@pytest.mark.parametrize("T", [1, 32, 256])
@pytest.mark.parametrize("mode", ["standard", "lore"])
def test_qwen2_57b(T, mode):
    layer = W.make_layer("qwen2_57b")
    _check_full(layer, T, mode)


def test_mixtral_floe_batch1():
    """Batch-1 decode calls (T = 1), several tokens one at a time."""
    cfg = dataclasses.replace(W.CONFIGS["mixtral_floe"], token_counts=(1, 6))
    layer = W.Layer(cfg)
    wdev = dev_weights(layer)
    for t in range(6):
        x1 = layer.x()[t:t + 1]
        say(f"[parity] mixtral_floe token {t}")
        g = run_layer(layer, 1, "floe", wdev=wdev, x_np=x1)
        check_decisions(layer, 1, "floe", g, x_np=x1)
        ref = oracle_forward_forced(layer, 1, "floe", g, [0], x_np=x1)
        err = rel_fro(g.out, ref["out"])
        say(f"    rel_fro={err:.3e}")
        assert err <= TOL["bf16"]
        check_floe_masks(layer, g, ref, [0])


@pytest.mark.parametrize("mode", ["standard", "stall_free"])
def test_granite_prefill(mode):
    """The 4096-token Granite-shaped layer, every output row.  Stall-free runs
    on the independent N(0, 0.02) prefetch router, so about three quarters of
    the routed slots are substituted."""
    layer = W.make_layer("granite_prefill")
    T = 4096
    g, _ = _check_full(layer, T, mode)
    if mode == "stall_free":
        n_sub = sum(len(set(g.ids[t]) - set(np.argsort(-g.logits[t], kind="stable")[:8]))
                    for t in range(T))
        say(f"    substituted slots: {n_sub} of {T * 8}")
        assert n_sub > T * 8 // 2


# ----------------------------------------------------------- entry points --
def test_prefetch_mask_parity():
    layer = W.make_layer("granite_prefill")
    T = 4096
    wdev = dev_weights(layer)
    masks, flags, _ = prefetch_masks_gpu(layer, T, wdev)
    X = O.decode(layer.x(T), "bf16")
    om, of, _ = O.prefetch_masks(X, O.decode(layer.w_prefetch(), "bf16"), layer.delta(T), 8)
    lp = O.router_logits(X, O.decode(layer.w_prefetch(), "bf16"))
    n_tie = 0
    for t in range(T):
        if of[t]:
            n_tie += 1
            sel = [e for e in range(40) if (masks[t] >> e) & 1]
            rest = [e for e in range(40) if not (masks[t] >> e) & 1]
            assert len(sel) == 8 + layer.delta(T)[t]
            assert not rest or min(lp[t][sel]) >= max(lp[t][rest]) - 1e-4
        else:
            assert masks[t] == om[t], t
            assert flags[t] == 0
    say(f"    prefetch near-ties: {n_tie}")


@pytest.mark.parametrize("delta", [0, 32])
def test_prefetch_delta_extremes(delta):
    """delta = 0 lists exactly k experts; delta = N - k lists all of them, so
    stall-free equals standard."""
    layer = W.Layer(SMALL["granite_small"])
    T = layer.cfg.t_max
    wdev = dev_weights(layer)
    masks, _, _ = prefetch_masks_gpu(layer, T, wdev, delta=np.full(T, delta, np.int32))
    assert all(bin(m).count("1") == 8 + delta for m in masks)
    sf = run_layer(layer, T, "stall_free", resident_masks=masks)
    check_decisions(layer, T, "stall_free", sf)
    if delta == 32:
        st = run_layer(layer, T, "standard")
        np.testing.assert_array_equal(sf.ids, st.ids)
        np.testing.assert_array_equal(sf.out, st.out)


def _oracle_routed(layer, X, k):
    """The router's top-k by the oracle (inputs of the overlap diagnostics)."""
    lr = O.router_logits(X, O.decode(layer.w_router(), layer.cfg.dtype))
    return np.array([O.rank_experts(lr[t])[:k] for t in range(X.shape[0])], dtype=np.int32)


@pytest.mark.parametrize("name,T", [("granite_prefill_distilled", 4096), ("granite_small", 203),
                                    ("granite_small", 37), ("f32_prefetch", 23),
                                    ("dsv2_prefetch", 64)])
def test_prefetch_adaptive_parity(name, T):
    """Adaptive budget, list, delta* and overlap against the oracle, every
    token: exact where neither side flags a near-tie; at a budget near-tie
    (flag 16) the budgets differ by at most one and the list is still the
    top-(k + budget) of the prefetch logits."""
    layer = W.make_layer(name) if name in W.CONFIGS else W.Layer(SMALL[name])
    cfg, tau = layer.cfg, 0.9
    k, E = cfg.top_k, cfg.n_experts
    wdev = dev_weights(layer)
    X = O.decode(layer.x(T), cfg.dtype)
    Wp = O.decode(layer.w_prefetch(), cfg.dtype)
    w_delta, theta = layer.ordinal(tau)
    routed = _oracle_routed(layer, X, k)
    od, om, of, ods, oov = O.adaptive_prefetch(X, Wp, O.decode(w_delta, cfg.dtype), theta, tau, k,
                                               routed, MARGIN)
    gd, gm, gf, gds, gov = prefetch_adaptive_gpu(layer, T, wdev, tau, routed=routed)
    lp = O.router_logits(X, Wp)
    # theta_d - w.x - logit(tau) per token and budget: the oracle's budget
    # test on the logit scale (for the flag-threshold check below)
    g = (theta.astype(np.float64)[None, :] - (X @ O.decode(w_delta, cfg.dtype))[:, None]
         - np.log(tau / (1 - tau)))
    n_budget_tie = n_list_tie = 0
    for t in range(T):
        srt = np.sort(lp[t])[::-1]
        if (of[t] | gf[t]) & O.FLAG_BUDGET:
            n_budget_tie += 1
        if gd[t] != od[t]:  # a budget near-tie, raised on both sides
            assert gf[t] & O.FLAG_BUDGET and of[t] & O.FLAG_BUDGET, t
            assert abs(int(gd[t]) - int(od[t])) == 1, t
        if (gf[t] ^ of[t]) & O.FLAG_BUDGET:  # the flag itself sits on its threshold
            d = int(od[t])
            gap = min(abs(g[t, j]) for j in (d - 1, d) if j >= 0)
            assert abs(gap - MARGIN) < 1e-2 * MARGIN, t
        n = k + int(gd[t])
        assert bin(gm[t]).count("1") == n, t
        sel = [e for e in range(E) if (gm[t] >> e) & 1]
        rest = [e for e in range(E) if not (gm[t] >> e) & 1]
        if gd[t] == od[t] and not (of[t] & O.FLAG_PREFETCH):
            assert gm[t] == om[t], t
            assert gov[t] == oov[t], t
        else:
            n_list_tie += 1
            assert not rest or min(lp[t][sel]) >= max(lp[t][rest]) - MARGIN, t
            assert gov[t] == O.prefetch_overlap(routed[t], gm[t]), t
        if gds[t] != ods[t]:  # only where the deepest routed expert ties its neighbour
            lo = k - 1 + min(int(gds[t]), int(ods[t]))
            assert abs(int(gds[t]) - int(ods[t])) == 1 and srt[lo] - srt[lo + 1] < MARGIN, t
        # flag bits other than 2 and 16 are never set
        assert gf[t] & ~np.uint32(O.FLAG_PREFETCH | O.FLAG_BUDGET) == 0, t
    say(f"    {name} T={T}: mean budget {gd.mean():.2f}, overlap {gov.mean() / k:.3f}, "
        f"budget near-ties {n_budget_tie}, list near-ties {n_list_tie}")
    assert 0 < gd.mean() < E - k  # the synthetic model spreads the budget


@pytest.mark.parametrize("fill,expect", [(-1e4, "all"), (1e4, "zero")])
def test_prefetch_adaptive_extremes(fill, expect):
    """theta far below logit(tau) everywhere: no budget qualifies, so the
    budget is N - k and every expert is listed (every routed one covered);
    far above: budget 0, the list is the prefetch router's own top-k."""
    layer = W.Layer(SMALL["granite_small"])
    cfg = layer.cfg
    k, E, T = cfg.top_k, cfg.n_experts, 203
    X = O.decode(layer.x(T), cfg.dtype)
    routed = _oracle_routed(layer, X, k)
    theta = np.full(E - k + 1, fill, np.float32)
    gd, gm, gf, gds, gov = prefetch_adaptive_gpu(layer, T, dev_weights(layer), 0.9, theta=theta,
                                                 routed=routed)
    assert (gf & O.FLAG_BUDGET).sum() == 0
    if expect == "all":
        assert (gd == E - k).all() and all(m == (1 << E) - 1 for m in gm) and (gov == k).all()
    else:
        lp = O.router_logits(X, O.decode(layer.w_prefetch(), cfg.dtype))
        om, of, _ = O.prefetch_masks(X, O.decode(layer.w_prefetch(), cfg.dtype),
                                     np.zeros(T, np.int32), k)
        assert (gd == 0).all()
        for t in range(T):
            assert gm[t] == om[t] or of[t], t
        assert (gov <= k).all() and (gds >= 0).all()
        # covered exactly when delta* is 0
        assert ((gov == k) == (gds == 0)).all()
    # T = 0 enqueues nothing and succeeds
    out = prefetch_adaptive_gpu(layer, 0, dev_weights(layer), 0.9, routed=routed[:0])
    assert len(out[0]) == 0 and len(out[1]) == 0


def _pack_reference(src: np.ndarray) -> np.ndarray:
    """Fragment-major packing written from its definition: fragment (t, s),
    lane l, element j = W[16t + l%16][32s + 8(l/16) + j], zero outside."""
    G, R, K = src.shape
    RT, KS = -(-R // 16), -(-K // 32)
    pad = np.zeros((G, RT * 16, KS * 32), dtype=src.dtype)
    pad[:, :R, :K] = src
    out = np.zeros((G, RT, KS, 64, 8), dtype=src.dtype)
    for lane in range(64):
        rows = np.arange(RT) * 16 + lane % 16
        for s_ in range(KS):
            k0 = 32 * s_ + 8 * (lane // 16)
            out[:, :, s_, lane, :] = pad[:, rows, k0:k0 + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("G,R,K", [(3, 40, 72), (2, 64, 64), (1, 16, 8), (5, 48, 2048)])
def test_pack_weights_bit_exact(G, R, K):
    rng = np.random.default_rng(G * 1000 + R + K)
    src = rng.integers(0, 1 << 16, size=(G, R, K), dtype=np.uint16)
    d_src = torch.from_numpy(src.view(np.int16)).cuda()
    n = M.moe_pack_size(G, R, K)
    assert n == G * (-(-R // 16)) * 16 * (-(-K // 32)) * 32 * 2
    d_dst = torch.full((n // 2,), -1, dtype=torch.int16, device="cuda")
    M.moe_pack_weights(G, R, K, d_src, d_dst)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_dst.cpu().numpy().view(np.uint16), _pack_reference(src))


# ----------------------------------------------- FloE predictor and packing --
def _floe_layer_for(name):
    if name == "mixtral":
        return W.Layer(dataclasses.replace(W.CONFIGS["mixtral_floe"], token_counts=(1, 3)))
    return W.Layer(FLOE_SMALL[name])


def _floe_stack(layer, field):
    return np.stack([layer.expert(field, e) for e in range(layer.cfg.n_experts)])


def _floe_predict_gpu(layer, T, h_np, ids, wdev=None):
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg))
    k, nk = cfg.top_k, cfg.floe_keep
    ws = torch.empty(M.moe_workspace_size(dims, T, "floe"), dtype=torch.uint8, device="cuda")
    keep = torch.full((T * k * nk,), -3, dtype=torch.int32, device="cuda")
    flags = torch.zeros(T, dtype=torch.int32, device="cuda")
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1)).cuda()
    M.moe_floe_predict(dims, T, tensor(h_np, cfg.dtype, "cuda"),
                       dev_weights(layer) if wdev is None else wdev, d_ids, keep, flags, ws)
    torch.cuda.synchronize()
    return keep.cpu().numpy().reshape(T, k, nk), flags.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,T", [("floe_small", 5), ("floe_wide", 3), ("mixtral", 2)])
def test_floe_predict_parity(name, T):
    """Predicted masks from the previous layer's hidden state: every pair
    exact against the oracle's mask rule unless it flags a near-tie at the
    mask edge, admissible within the margin there."""
    layer = _floe_layer_for(name)
    cfg = layer.cfg
    k, nk = cfg.top_k, cfg.floe_keep
    X = O.decode(layer.x(T), cfg.dtype)
    Xp = O.decode(layer.x_prev(T), cfg.dtype)
    ids = _oracle_routed(layer, X, k)
    gk, gf = _floe_predict_gpu(layer, T, layer.x_prev(T), ids)
    n_tie, rec = 0, []
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            ok, ofl, u = O.floe_channel_mask(Xp[t], layer.expert("up_q", e), layer.expert("up_scale", e),
                                             layer.expert("up_zero", e), nk, MARGIN)
            assert np.all(np.diff(gk[t, j]) > 0)
            if ofl:
                n_tie += 1
                assert gf[t] & O.FLAG_FLOE
                mask = np.zeros(cfg.inter, bool)
                mask[gk[t, j]] = True
                assert np.abs(u[mask]).min() >= np.abs(u[~mask]).max() - MARGIN
            else:
                np.testing.assert_array_equal(gk[t, j], ok)
            tk, _, _ = O.floe_channel_mask(X[t], layer.expert("up_q", e), layer.expert("up_scale", e),
                                           layer.expert("up_zero", e), nk, MARGIN)
            rec.append(O.mask_recall(ok, tk))
    assert (gf & ~np.uint32(O.FLAG_FLOE)).sum() == 0
    say(f"    {name} T={T}: near-ties {n_tie}, oracle recall vs the true mask {np.mean(rec):.3f}")


@pytest.mark.parametrize("keep", [104, 105, 520])
def test_floe_select_exact_channel_ties(keep):
    """Exact |u| ties over many channels: every even up row is the same row and
    every odd row's codes equal its zero point (u = 0 up to rounding), so the
    520 even channels tie exactly and the channel select must keep the lowest
    `keep` of them (ties to the lower channel), as the oracle's rule does, and
    raise the mask-edge flag when the edge falls inside the tie.  This takes
    the select's equal-key ranking."""
    base = _floe_layer_for("floe_small")
    layer = W.Layer(dataclasses.replace(base.cfg, floe_keep=keep))
    cfg = layer.cfg
    T, k = 5, cfg.top_k
    q, sc, zp = layer.full("up_q").copy(), layer.full("up_scale").copy(), layer.full("up_zero").copy()
    q[:, 0::2], sc[:, 0::2], zp[:, 0::2] = q[:, :1], sc[:, :1], zp[:, :1]
    q[:, 1::2] = 0x55            # every 2-bit code 1
    zp[:, 1::2] = 0x3C00         # zero point 1.0 (fp16)
    wdev = dict(dev_weights(layer))
    wdev["up_q"] = tensor(q, cfg.dtype, "cuda")
    wdev["up_scale"] = tensor(sc, cfg.dtype, "cuda")
    wdev["up_zero"] = tensor(zp, cfg.dtype, "cuda")
    X = O.decode(layer.x(T), cfg.dtype)
    Xp = O.decode(layer.x_prev(T), cfg.dtype)
    ids = _oracle_routed(layer, X, k)
    gk, gf = _floe_predict_gpu(layer, T, layer.x_prev(T), ids, wdev)
    want = list(range(0, 2 * keep, 2))
    tie = keep < 520    # at 520 every tied channel is kept: no edge inside the tie
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            ok, ofl, _ = O.floe_channel_mask(Xp[t], q[e], sc[e], zp[e], keep, MARGIN)
            assert list(ok) == want and ofl == tie
            assert list(gk[t, j]) == want
        assert bool(gf[t] & O.FLAG_FLOE) == tie
    say(f"    exact channel ties, keep {keep}: lowest even channels kept on every pair")


@pytest.mark.parametrize("name,T", [("floe_small", 5), ("mixtral", 3)])
def test_floe_pack_bit_exact(name, T):
    """Compact gate/down rows of the oracle's predicted channels, bit for bit
    (a pure gather), including a slot with an invalid expert id and a channel
    past I, which give zero rows."""
    layer = _floe_layer_for(name)
    cfg = layer.cfg
    k, nk, H = cfg.top_k, cfg.floe_keep, cfg.hidden
    X = O.decode(layer.x(T), cfg.dtype)
    ids = _oracle_routed(layer, X, k)
    keep, _ = O.floe_predict_masks(O.decode(layer.x_prev(T), cfg.dtype), ids,
                                   _floe_stack(layer, "up_q"), _floe_stack(layer, "up_scale"),
                                   _floe_stack(layer, "up_zero"), nk, MARGIN)
    ids_in = ids.copy()
    ids_in[T - 1, k - 1] = cfg.n_experts          # invalid expert -> zero rows
    keep_in = keep.copy()
    keep_in[0, 0, nk - 1] = cfg.inter             # channel past I -> a zero row
    dims = M.Dims(**dims_dict(cfg))
    wdev = dev_weights(layer)
    gate = torch.full((T * k * nk * H,), 7, dtype=torch.int16, device="cuda")
    down = torch.full((T * k * nk * H,), 7, dtype=torch.int16, device="cuda")
    M.moe_floe_pack(dims, T, torch.from_numpy(ids_in.reshape(-1)).cuda(),
                    torch.from_numpy(keep_in.reshape(-1)).cuda(), wdev["w_gate"], wdev["w_down"],
                    gate, down)
    torch.cuda.synchronize()
    gg = gate.cpu().numpy().view(np.uint16).reshape(T, k, nk, H)
    gd = down.cpu().numpy().view(np.uint16).reshape(T, k, nk, H)
    for t in range(T):
        for j in range(k):
            if ids_in[t, j] >= cfg.n_experts:
                assert not gg[t, j].any() and not gd[t, j].any()
                continue
            e = int(ids_in[t, j])
            wg, wd = O.floe_pack(keep[t, j], layer.expert("w_gate", e), layer.expert("w_down", e))
            if t == 0 and j == 0:
                assert not gg[0, 0, nk - 1].any() and not gd[0, 0, nk - 1].any()
                wg, wd, gg_, gd_ = wg[:-1], wd[:-1], gg[0, 0, :-1], gd[0, 0, :-1]
            else:
                gg_, gd_ = gg[t, j], gd[t, j]
            np.testing.assert_array_equal(gg_, wg)
            np.testing.assert_array_equal(gd_, wd)


# ------------------------------------------------------------ LoRE fitting --
def _fit_gpu(dims, h_np, R_np, dtype, r, cols, n_iter, omega):
    N, H = R_np.shape
    h = tensor(h_np, dtype, "cuda")
    R = torch.from_numpy(np.ascontiguousarray(R_np, np.float32)).cuda()
    om = torch.from_numpy(np.ascontiguousarray(omega, np.float32)).cuda()
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    A = torch.empty(r * H, dtype=tdt, device="cuda")
    B = torch.empty(H * r, dtype=tdt, device="cuda")
    sig = torch.empty(r, dtype=torch.float32, device="cuda")
    err = torch.empty(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_lore_fit_size(H, N, r, cols), dtype=torch.uint8, device="cuda")
    M.moe_lore_fit(dims, N, h, R, r, cols, n_iter, om, A, B, sig, err, ws)
    torch.cuda.synchronize()
    return (A.float().cpu().numpy().reshape(r, H), B.float().cpu().numpy().reshape(H, r),
            sig.cpu().numpy(), float(err[0].cpu()))


def _orthogonal_rows(rng, N, H):
    return np.concatenate([np.linalg.qr(rng.standard_normal((H, H)))[0] * np.sqrt(H)
                           for _ in range(N // H)], axis=0)


@pytest.mark.parametrize("H,N,r,cols", [(256, 512, 8, 16), (192, 384, 5, 24)])
def test_lore_fit_planted_map(H, N, r, cols):
    """Targets from a planted rank-r map plus small noise (well separated
    singular values): the fitted B A, the singular values and the
    calibration error match the oracle's truncated SVD."""
    rng = np.random.default_rng(H + r)
    h = _orthogonal_rows(rng, N, H).astype(np.float32)
    U = np.linalg.qr(rng.standard_normal((H, r)))[0]
    V = np.linalg.qr(rng.standard_normal((H, r)))[0]
    M_true = (U * np.linspace(2.0, 1.0, r)) @ V.T
    R = (h.astype(np.float64) @ M_true.T + 0.01 * rng.standard_normal((N, H))).astype(np.float32)
    dims = M.Dims(hidden=H, n_experts=1, top_k=1, inter=16, dtype="f32")
    omega = rng.standard_normal((H, cols)).astype(np.float32)
    A, B, sig, err = _fit_gpu(dims, h, R, "f32", r, cols, 12, omega)
    oA, oB, osig, oerr = O.lore_fit(h.astype(np.float64), R.astype(np.float64), r)
    np.testing.assert_allclose(sig, osig, rtol=1e-4)
    assert abs(err - oerr) < 1e-4, (err, oerr)
    assert rel_fro(B @ A, oB @ oA) < 1e-4
    np.testing.assert_allclose(A @ A.T, np.eye(r), atol=1e-4)


def test_lore_targets_and_fit_on_an_expert():
    """The whole fit for one expert of a small DeepSeek-V2-Lite-shaped layer:
    targets y_e - y_s from the FFN kernels against the oracle's (bf16
    activation rounding on the GPU side), then singular values and the
    calibration error of rank-8 and rank-16 fits against the oracle's exact
    SVD (the spectrum of random experts is flat, so the factors themselves
    are only determined up to rotations within near-equal singular values and
    are not compared)."""
    layer = W.Layer(SMALL["dsv2_small"])
    cfg = layer.cfg
    N, e = 2 * cfg.hidden, 5
    dims = M.Dims(**dims_dict(cfg))
    h_np = layer.calibration(N)
    h = O.decode(h_np, cfg.dtype)
    D = lambda a: O.decode(a, cfg.dtype)
    R_o = O.lore_targets(h, D(layer.expert("w_gate", e)), D(layer.expert("w_up", e)),
                         D(layer.expert("w_down", e)), D(layer.full("ws_gate")), D(layer.full("ws_up")),
                         D(layer.full("ws_down")))
    wdev = dev_weights(layer)
    d1 = dataclasses.replace(dims, top_k=1)
    for layout, wts in (("rows", wdev), ("mfma16", packed_weights(layer))):
        dl = dataclasses.replace(d1, weight_layout=layout)
        ws = torch.empty(M.moe_workspace_size(dl, N, "standard"), dtype=torch.uint8, device="cuda")
        R = torch.empty(N * cfg.hidden, dtype=torch.float32, device="cuda")
        M.moe_lore_targets(dataclasses.replace(dims, weight_layout=layout), N,
                           tensor(h_np, cfg.dtype, "cuda"), wts, e, R, ws)
        torch.cuda.synchronize()
        R_g = R.cpu().numpy().reshape(N, cfg.hidden)
        say(f"    targets ({layout}): rel_fro {rel_fro(R_g, R_o):.2e}")
        assert rel_fro(R_g, R_o) < 1e-2
    omega = layer.omega(64)
    for r in (8, 16):
        _, _, sig, err = _fit_gpu(dims, h_np, R_g, cfg.dtype, r, 64, 20, omega)
        _, _, osig, oerr = O.lore_fit(h, R_o, r)
        say(f"    rank {r}: error {err:.4f} (oracle {oerr:.4f}), top sigma {sig[0]:.5f} ({osig[0]:.5f})")
        np.testing.assert_allclose(sig, osig, rtol=5e-3)
        assert abs(err - oerr) < 5e-3


# --------------------------------------------------------- graph capture --
@pytest.mark.parametrize("name,mode,layout", [("dsv2_small", "lore", "mfma16"),
                                              ("dsv2_prefetch", "standard", "mfma16"),
                                              ("granite_small", "stall_free", "rows"),
                                              ("tiny", "lore", "rows")])
def test_graph_replay_matches_eager(name, mode, layout):
    """One moe_layer_forward captured in a HIP graph (torch.cuda.CUDAGraph on
    the library's stream argument) and replayed three times, with eager work
    and synchronisations in between: every replay's output equals the eager
    call's bit for bit (the forward records kernels and no memset nodes)."""
    layer = W.make_layer(name) if name in W.CONFIGS else W.Layer(SMALL[name])
    cfg = layer.cfg
    T = cfg.t_max
    dd = dims_dict(cfg)
    dims = M.Dims(**dd, weight_layout=layout)
    wdev = packed_weights(layer) if layout == "mfma16" else dev_weights(layer)
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    if mode == "lore":
        res, stride = mask_tensor([layer.resident()], "cuda"), 0
    elif mode == "stall_free":
        _, _, res = prefetch_masks_gpu(layer, T, dev_weights(layer))
        stride = 1
    else:
        res, stride = None, 0
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    eager = torch.empty(T, cfg.hidden, dtype=odt, device="cuda")
    M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, eager, ws)
    torch.cuda.synchronize()
    ref = eager.clone()
    out = torch.zeros_like(eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, out, ws)  # warm-up on the side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, out, ws)
    for rep in range(3):
        out.zero_()
        eager.zero_()
        M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, eager, ws)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, mode, rep)
        assert torch.equal(eager, ref), (name, mode, rep)


def test_permute_parity_random():
    rng = np.random.default_rng(7)
    for T, k, E, p_exact in [(1, 1, 1, 1.0), (37, 6, 64, 0.5), (4096, 8, 40, 1.0), (300, 8, 64, 0.0),
                             (1000, 2, 8, 0.7), (5, 8, 64, 1.0), (128, 8, 16, 0.6), (129, 8, 16, 0.6),
                             (2999, 7, 64, 0.5), (512, 8, 64, 0.5), (4097, 1, 64, 0.5),
                             (256, 8, 64, 1.0)]:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        exact = (rng.random((T, k)) < p_exact).astype(np.uint8)
        d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
        d_ex = torch.from_numpy(exact.reshape(-1)).cuda()
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        ws = torch.empty(M.moe_workspace_size(M.Dims(hidden=64, n_experts=E, top_k=k, inter=16), T,
                                               "standard"), dtype=torch.uint8, device="cuda")
        M.moe_permute(T, k, E, d_ids, d_ex, off, perm, inv, ws)
        torch.cuda.synchronize()
        o_off, o_perm, o_inv = O.permute(ids, exact, E)
        np.testing.assert_array_equal(off.cpu().numpy(), o_off)
        np.testing.assert_array_equal(perm.cpu().numpy()[: len(o_perm)], o_perm)
        np.testing.assert_array_equal(inv.cpu().numpy(), o_inv)
        # the remaining entries list the non-exact pairs, grouped the same way
        _, m_perm, _ = O.permute(ids, 1 - exact, E)
        np.testing.assert_array_equal(perm.cpu().numpy()[len(o_perm):], m_perm)


def test_all_resident_reduces_to_standard_bitwise():
    layer = W.Layer(SMALL["dsv2_small"])
    T = layer.cfg.t_max
    allres = (1 << layer.cfg.n_experts) - 1
    st = run_layer(layer, T, "standard")
    lo = run_layer(W.Layer(dataclasses.replace(layer.cfg, resident_count=16)), T, "lore")
    sf = run_layer(layer, T, "stall_free", resident_masks=[allres] * T)
    for r in (lo, sf):
        np.testing.assert_array_equal(r.ids, st.ids)
        np.testing.assert_array_equal(r.out, st.out)


def test_nan_poisoned_missing_experts_are_never_read():
    """LORE never touches a non-resident expert's FFN weights."""
    layer = W.Layer(SMALL["dsv2_small"])
    T = layer.cfg.t_max
    wdev = dict(dev_weights(layer))
    base = run_layer(layer, T, "lore", wdev=wdev)
    res = layer.resident()
    poisoned = dict(wdev)
    for n in ("w_gate", "w_up", "w_down"):
        t = wdev[n].clone()
        for e in range(layer.cfg.n_experts):
            if not (res >> e) & 1:
                t[e] = float("nan")
        poisoned[n] = t
    p = run_layer(layer, T, "lore", wdev=poisoned)
    assert np.all(np.isfinite(p.out))
    np.testing.assert_array_equal(p.out, base.out)


def test_lore_zero_factors():
    """A = B = 0: every surrogate slot contributes w * y_shared."""
    layer = W.Layer(SMALL["dsv2_small"])
    T = layer.cfg.t_max
    wdev = dict(dev_weights(layer))
    wdev["lore_A"] = torch.zeros_like(wdev["lore_A"])
    wdev["lore_B"] = torch.zeros_like(wdev["lore_B"])
    g = run_layer(layer, T, "lore", wdev=wdev)
    w = {n: layer.full(n) for n in layer.tensor_names()}
    w["w_router"] = layer.w_router()
    w["lore_A"] = np.zeros_like(w["lore_A"]); w["lore_B"] = np.zeros_like(w["lore_B"])
    ref = oracle_forward_forced(layer, T, "lore", g, list(range(T)), weights=w)
    assert rel_fro(g.out, ref["out"]) <= TOL["bf16"]
    assert (g.exact == 0).any()


def test_exact_ties_go_to_lower_id():
    """Identical router columns give exactly equal logits; the lower id wins."""
    cfg = SMALL["tiny"]
    layer = W.Layer(cfg)
    wdev = dict(dev_weights(layer))
    wr = layer.w_router().copy()       # [E][H]
    wr[5] = wr[2]
    wr[7] = wr[0]
    wdev["w_router"] = tensor(wr, "f32", "cuda")
    g = run_layer(layer, 16, "standard", wdev=wdev)
    l = O.router_logits(O.decode(layer.x(16), "f32"), O.decode(wr, "f32"))
    for t in range(16):
        want = O.rank_experts(l[t])[:2]
        assert list(g.ids[t]) == want
        assert not (2 in want and 5 in want and list(want).index(5) < list(want).index(2))
        assert 5 not in g.ids[t] or 2 in g.ids[t]
        assert 7 not in g.ids[t] or 0 in g.ids[t]


@pytest.mark.parametrize("name,mode", [("qwen2_small", "lore"), ("prefill_small", "standard"),
                                       ("prefill_small", "lore")])
def test_unfused_entry_points_match_fused(name, mode):
    """route -> permute -> expert_ffn -> lore_surrogate -> combine matches
    moe_layer_forward: on the decode kernels (qwen2_small) and on the grouped
    GEMM with the shared experts' k-split (prefill_small), where the unfused
    expert_ffn writes fp32 rows and the fused standard forward bf16 rows."""
    layer = W.Layer(SMALL[name])
    say(f"[unfused] {name} {mode}")
    cfg = layer.cfg
    T, k, E, H = cfg.t_max, cfg.top_k, cfg.n_experts, cfg.hidden
    dims = M.Dims(**dims_dict(cfg))
    wdev = dev_weights(layer)
    x = tensor(layer.x(T), "bf16", "cuda")
    res = mask_tensor([layer.resident()], "cuda") if mode == "lore" else None
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    ex = torch.empty(T * k, dtype=torch.uint8, device="cuda")
    fl = torch.empty(T, dtype=torch.int32, device="cuda")
    lg = torch.empty(T * E, dtype=torch.float32, device="cuda")
    M.moe_route(dims, T, x, wdev["w_router"], res, 0, mode, ids, w, ex, fl, lg)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    M.moe_permute(T, k, E, ids, ex, off, perm, inv)
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    y = torch.empty(T * k, H, dtype=torch.float32, device="cuda")
    ys = torch.empty(T, H, dtype=torch.float32, device="cuda")
    gs = torch.empty(T, dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(dims, T, x, wdev, mode, off, perm, y, ys, gs, ws)
    lo = torch.empty(T, k, H, dtype=torch.float32, device="cuda")
    M.moe_lore_surrogate(dims, T, x, ids, ex, wdev["lore_A"], wdev["lore_B"], lo)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    M.moe_combine(dims, T, y, inv, w, ex, ys, gs, lo, out)
    torch.cuda.synchronize()
    fused = run_layer(layer, T, mode, wdev=wdev)
    # same decisions; the fused path computes B_e A_e x on the matrix cores
    # and the unfused one with vector FMAs, and rounds GEMM rows to bf16 when
    # no surrogate row follows, so outputs agree to rounding
    np.testing.assert_array_equal(ids.cpu().numpy().reshape(T, k), fused.ids)
    err = rel_fro(out.float().cpu().numpy(), fused.out)
    say(f"    rel_fro={err:.3e}")
    # bf16 GEMM rows in the fused forward: one more rounding of each routed
    # row, at most 2^-9 relative per element, on top of the output's own
    tol = 2.0 ** -8 if (name, mode) == ("prefill_small", "standard") else 2e-3
    assert err <= tol


def test_zero_tokens_enqueue_nothing():
    layer = W.Layer(SMALL["tiny"])
    dims = M.Dims(**dims_dict(layer.cfg))
    wdev = dev_weights(layer)
    x = torch.empty(0, 256, dtype=torch.float32, device="cuda")
    out = torch.empty(0, 256, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, M.moe_workspace_size(dims, 0, "standard")), dtype=torch.uint8, device="cuda")
    # a zero-size tensor may have a null data pointer; pass a valid one
    x1 = torch.empty(1, 256, dtype=torch.float32, device="cuda")
    M.moe_layer_forward(dims, 0, x1, wdev, None, 0, "standard", x1, ws)
    torch.cuda.synchronize()


def test_repeat_runs_bitwise_identical():
    layer = W.make_layer("granite_prefill")
    a = run_layer(layer, 4096, "stall_free")
    b = run_layer(layer, 4096, "stall_free")
    np.testing.assert_array_equal(a.out, b.out)
    np.testing.assert_array_equal(a.perm, b.perm)


# ------------------------------------- stall-free with short prefetched sets --
def test_stall_free_short_prefetched_sets():
    """Prefetched sets of every size from 0 to E: those smaller than k keep
    all their experts and fill the rest from outside by router score (flag
    32), the others follow Algorithm 1; outputs against the oracle."""
    layer = W.Layer(SMALL["granite_small"])
    cfg = layer.cfg
    T, E = cfg.t_max, cfg.n_experts
    rng = np.random.default_rng(31)
    masks = []
    for t in range(T):
        n = t % (E + 1)
        m = 0
        for e in rng.permutation(E)[:n]:
            m |= 1 << int(e)
        masks.append(m)
    g = run_layer(layer, T, "stall_free", resident_masks=masks)
    counts = check_decisions(layer, T, "stall_free", g)
    ref = oracle_forward_forced(layer, T, "stall_free", g, list(range(T)))
    err = rel_fro(g.out, ref["out"])
    say(f"    short sets: {counts}, rel_fro={err:.3e}")
    assert counts["short_sets"] > 0 and err <= TOL["bf16"]


# ------------------------------- unfused entry points against the oracle ----
def _route_permute(layer, T, mode, dims, wdev, x):
    cfg = layer.cfg
    k, E = cfg.top_k, cfg.n_experts
    res = mask_tensor([layer.resident()], "cuda") if mode == "lore" else None
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    ex = torch.empty(T * k, dtype=torch.uint8, device="cuda")
    fl = torch.zeros(T, dtype=torch.int32, device="cuda")
    lg = torch.empty(T * E, dtype=torch.float32, device="cuda")
    M.moe_route(dims, T, x, wdev["w_router"], res, 0, mode, ids, w, ex, fl, lg)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    M.moe_permute(T, k, E, ids, ex, off, perm, inv, ws)
    return ids, w, ex, fl, off, perm, inv, ws


def test_lore_surrogate_entry_against_oracle():
    """moe_lore_surrogate (the vector-FMA path) against the oracle's
    B_e (A_e x_t) for every non-resident slot, zeros elsewhere."""
    layer = W.Layer(SMALL["qwen2_small"])
    cfg = layer.cfg
    T, k, H = cfg.t_max, cfg.top_k, cfg.hidden
    dims = M.Dims(**dims_dict(cfg))
    wdev = dev_weights(layer)
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    ids, _, ex, _, _, _, _, _ = _route_permute(layer, T, "lore", dims, wdev, x)
    lo = torch.full((T, k, H), 7.0, dtype=torch.float32, device="cuda")
    M.moe_lore_surrogate(dims, T, x, ids, ex, wdev["lore_A"], wdev["lore_B"], lo)
    torch.cuda.synchronize()
    gids, gex = ids.cpu().numpy().reshape(T, k), ex.cpu().numpy().reshape(T, k)
    X = O.decode(layer.x(T), cfg.dtype)
    want = np.zeros((T, k, H))
    for t in range(T):
        for j in range(k):
            if not gex[t, j]:
                e = int(gids[t, j])
                want[t, j] = O.lore_residual(X[t], O.decode(layer.expert("lore_A", e), cfg.dtype),
                                             O.decode(layer.expert("lore_B", e), cfg.dtype))
    got = lo.cpu().numpy().astype(np.float64)
    err = rel_fro(got, want)
    say(f"    lore_surrogate rel_fro={err:.3e} over {int((gex == 0).sum())} surrogate slots")
    assert (gex == 0).any() and err <= 1e-5
    assert not got[gex == 1].any()


def test_combine_entry_against_oracle():
    """moe_combine fed the oracle's own intermediates (expert rows, weights,
    shared output and gate, LoRE residuals, rounded to fp32) reproduces the
    oracle's layer output."""
    layer = W.Layer(SMALL["qwen2_small"])
    cfg = layer.cfg
    T, k, H = cfg.t_max, cfg.top_k, cfg.hidden
    dims = M.Dims(**dims_dict(cfg))
    ref = O.layer_forward(layer.x(T), layer, dims_dict(cfg), "lore", resident=layer.resident())
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    y = np.zeros((T * k, H))
    y[: len(ref["perm"])] = ref["y_pair"]
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    M.moe_combine(dims, T, f32(y), torch.from_numpy(ref["inv"].astype(np.int32)).cuda(),
                  f32(ref["weights"].reshape(-1)), torch.from_numpy(ref["exact"].reshape(-1)).cuda(),
                  f32(ref["y_shared"]), f32(ref["g_shared"]), f32(ref["lore"]), out)
    torch.cuda.synchronize()
    err = rel_fro(out.float().cpu().numpy(), ref["out"])
    say(f"    combine rel_fro={err:.3e}")
    assert (ref["exact"] == 0).any() and err <= TOL["bf16"]


def test_expert_ffn_floe_entry_against_oracle():
    """moe_expert_ffn in FloE mode after moe_route / moe_permute: every pair's
    unweighted expert row and kept channels against the oracle's FloE expert
    (the oracle re-run on the GPU's kept channels at a flagged mask edge)."""
    layer = W.Layer(FLOE_SMALL["floe_small"])
    cfg = layer.cfg
    T, k, H, nk = cfg.t_max, cfg.top_k, cfg.hidden, cfg.floe_keep
    dims = M.Dims(**dims_dict(cfg))
    wdev = dev_weights(layer)
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    ids, _, _, fl, off, perm, _, ws = _route_permute(layer, T, "floe", dims, wdev, x)
    y = torch.empty(T * k, H, dtype=torch.float32, device="cuda")
    keep = torch.empty(T * k * nk, dtype=torch.int32, device="cuda")
    M.moe_expert_ffn(dims, T, x, wdev, "floe", off, perm, y, None, None, ws, floe_keep=keep, flags=fl)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy().reshape(T, k)
    gperm = perm.cpu().numpy()
    gkeep = keep.cpu().numpy().reshape(T, k, nk)
    gy = y.cpu().numpy()
    X = O.decode(layer.x(T), cfg.dtype)
    D = lambda n, e: O.decode(layer.expert(n, e), cfg.dtype)
    worst = 0.0
    for p in range(T * k):
        f = int(gperm[p]); t, j = f // k, f % k
        e = int(gids[t, j])
        yo, u, ko, flag = O.floe_expert(X[t], D("w_gate", e), layer.expert("up_q", e),
                                        layer.expert("up_scale", e), layer.expert("up_zero", e),
                                        D("w_down", e), nk, MARGIN, force_keep=gkeep[t, j])
        if not flag:
            _, _, k_free, _ = O.floe_expert(X[t], D("w_gate", e), layer.expert("up_q", e),
                                            layer.expert("up_scale", e), layer.expert("up_zero", e),
                                            D("w_down", e), nk, MARGIN)
            np.testing.assert_array_equal(gkeep[t, j], k_free)
        worst = max(worst, rel_fro(gy[p], yo))
    say(f"    floe expert rows: worst rel_fro {worst:.3e}")
    assert worst <= TOL["bf16"]


def test_lore_fit_non_orthogonal_design():
    """A Gaussian calibration design of 2H rows (h^T h far from N I): the
    GPU's whitened fit against the oracle's exact rank-r least squares on a
    planted low-rank map plus noise."""
    H, N, r, cols = 256, 512, 8, 24
    rng = np.random.default_rng(77)
    h = rng.standard_normal((N, H)).astype(np.float32)
    U = np.linalg.qr(rng.standard_normal((H, r)))[0]
    V = np.linalg.qr(rng.standard_normal((H, r)))[0]
    M_true = (U * np.linspace(2.0, 1.0, r)) @ V.T
    R = (h.astype(np.float64) @ M_true.T + 0.01 * rng.standard_normal((N, H))).astype(np.float32)
    dims = M.Dims(hidden=H, n_experts=1, top_k=1, inter=16, dtype="f32")
    omega = rng.standard_normal((H, cols)).astype(np.float32)
    A, B, sig, err = _fit_gpu(dims, h, R, "f32", r, cols, 12, omega)
    oA, oB, osig, oerr = O.lore_fit(h.astype(np.float64), R.astype(np.float64), r)
    say(f"    non-orthogonal design: error {err:.5f} (oracle {oerr:.5f}), sigma0 {sig[0]:.5f} ({osig[0]:.5f})")
    np.testing.assert_allclose(sig, osig, rtol=1e-3)
    assert abs(err - oerr) < 1e-4, (err, oerr)
    assert rel_fro(B @ A, oB @ oA) < 1e-3
