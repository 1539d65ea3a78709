"""Host half of the exact execution of missed experts, through the C ABI and
without a GPU [SPICE page, "CPU-GPU collaboration: handling prefetch
misses"]: the cost rule (moe_offload_plan) against the oracle's, and the host
SwiGLU FFN (moe_host_expert_ffn) against the oracle's expert FFN."""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads.device import dims_dict

import sparse_moe_layer_route_amd as M
from sparse_moe_layer_route_amd import binding as B


def _dims(cfg, **over):
    return M.Dims(**dims_dict(cfg, **over))


def test_plan_matches_oracle_rule():
    rng = np.random.default_rng(5)
    for case in range(300):
        cfg = W.CONFIGS[["tiny", "dsv2_lite", "qwen2_57b", "granite_prefill"][case % 4]]
        d = dims_dict(cfg)
        E = cfg.n_experts
        tokens = rng.integers(0, 40, E) * (rng.random(E) < 0.7)
        resident = int(rng.integers(0, 2**63)) & ((1 << E) - 1)
        Bw = 10 ** rng.uniform(8, 11)
        g = 10 ** rng.uniform(-7, -3)
        c = 10 ** rng.uniform(-7, -2)
        ce = 10 ** rng.uniform(-6, -2) if case % 2 else 0.0
        qa = bool(case % 3 == 0)
        want = O.offload_plan(d, [int(t) for t in tokens], resident, Bw, g, c, ce, qa)
        got = M.moe_offload_plan(_dims(cfg), tokens, resident,
                                 M.offload_cost(Bw, g, c, cpu_expert_s=ce, queue_aware=qa))
        assert list(got) == want, case


def test_plan_hand_boundary_and_checks():
    cfg = dataclasses.replace(W.CONFIGS["tiny"], hidden=64, inter=16, n_experts=8, dtype="bf16")
    dims = _dims(cfg, n_shared=0, shared_inter=0, lore_rank=0)
    # W_e = 6144 bytes, 256 bytes per pair: equal at 24 pairs -> host
    got = M.moe_offload_plan(dims, [23, 24, 25, 48, 0, 3, 30, 1], 0b0100000,
                             M.offload_cost(1e9, 0.0, 0.0))
    assert list(got) == [2, 2, 1, 1, 0, 0, 1, 2]
    for bad in (M.offload_cost(0.0, 0.0, 0.0), M.offload_cost(1e9, -1.0, 0.0),
                M.offload_cost(1e9, 0.0, float("nan")), M.offload_cost(float("inf"), 0.0, 0.0),
                M.offload_cost(1e9, 0.0, 0.0, cpu_expert_s=-1.0)):
        with pytest.raises(M.MoEError) as ei:
            M.moe_offload_plan(dims, [1] * 8, 0, bad)
        assert ei.value.status == B.MOE_EINVAL
    with pytest.raises(M.MoEError):
        M.moe_offload_plan(dims, [1, -1, 0, 0, 0, 0, 0, 0], 0, M.offload_cost(1e9, 0, 0))


def test_plan_queue_aware_hand_case():
    # the hand case of the oracle pin: four single-pair experts alternate
    cfg = dataclasses.replace(W.CONFIGS["tiny"], hidden=1024, inter=1024, n_experts=8)
    dims = _dims(cfg, n_shared=0, shared_inter=0, lore_rank=0)
    w_bytes = 3 * 1024 * 1024 * 4
    cost = M.offload_cost(float(w_bytes), 0.0, 0.9, queue_aware=True)
    got = M.moe_offload_plan(dims, [1, 1, 1, 1, 0, 0, 0, 0], 0, cost)
    assert list(got) == [2, 1, 2, 1, 0, 0, 0, 0]
    plain = M.moe_offload_plan(dims, [1, 1, 1, 1, 0, 0, 0, 0], 0,
                               M.offload_cost(float(w_bytes), 0.0, 0.9))
    assert list(plain) == [2, 2, 2, 2, 0, 0, 0, 0]


def _bf16_small():
    return W.make_layer(dataclasses.replace(
        W.CONFIGS["dsv2_lite"], name="dsv2_host", hidden=256, inter=192, n_experts=16,
        top_k=4, n_shared=0, shared_inter=0, lore_rank=0, token_counts=(12,), seed=41))


@pytest.mark.parametrize("which", ["tiny", "bf16"])
def test_host_ffn_matches_oracle(which):
    layer = W.make_layer("tiny") if which == "tiny" else _bf16_small()
    cfg = layer.cfg
    T = 12
    x = layer.x(T)
    wg, wu, wd = (layer.full(n) for n in ("w_gate", "w_up", "w_down"))
    rng = np.random.default_rng(7)
    n = 23                                   # unsorted pairs, experts repeated
    tok = rng.integers(0, T, n).astype(np.int32)
    ex = rng.integers(0, cfg.n_experts, n).astype(np.int32)
    dims = _dims(cfg)
    ws = np.zeros(M.moe_host_ffn_workspace_size(dims, n), np.uint8)
    y = np.zeros((n, cfg.hidden), np.float32)
    M.moe_host_expert_ffn(dims, T, x, {"w_gate": wg, "w_up": wu, "w_down": wd}, tok, ex, 3, y, ws)
    xf = O.decode(x, cfg.dtype)
    for i in range(n):
        e = ex[i]
        ref = O.swiglu_expert(xf[tok[i]][None], O.decode(wg[e], cfg.dtype),
                              O.decode(wu[e], cfg.dtype), O.decode(wd[e], cfg.dtype))[0]
        err = np.linalg.norm(y[i] - ref) / np.linalg.norm(ref)
        # fp32 sums; bf16 layers also round the SwiGLU product to bf16 (2^-9)
        assert err <= (1e-6 if cfg.dtype == "f32" else 4e-3), (i, err)
    # thread count does not change a bit
    for threads in (1, 8):
        y2 = np.zeros_like(y)
        M.moe_host_expert_ffn(dims, T, x, {"w_gate": wg, "w_up": wu, "w_down": wd}, tok, ex,
                              threads, y2, ws)
        assert np.array_equal(y2, y)


def test_host_ffn_checks():
    layer = W.make_layer("tiny")
    cfg = layer.cfg
    dims = _dims(cfg)
    T = 4
    x = layer.x(T)
    hw = {n: layer.full(n) for n in ("w_gate", "w_up", "w_down")}
    ws = np.zeros(M.moe_host_ffn_workspace_size(dims, 2), np.uint8)
    y = np.zeros((2, cfg.hidden), np.float32)
    for tok, ex in (([0, T], [0, 1]), ([0, 1], [0, cfg.n_experts]), ([-1, 0], [0, 0])):
        with pytest.raises(M.MoEError) as ei:
            M.moe_host_expert_ffn(dims, T, x, hw, tok, ex, 1, y, ws)
        assert ei.value.status == B.MOE_EINVAL
    small = np.zeros(64, np.uint8)
    with pytest.raises(M.MoEError) as ei:
        M.moe_host_expert_ffn(dims, T, x, hw, [0, 1], [0, 1], 1, y, small)
    assert ei.value.status == B.MOE_EWORKSPACE
    M.moe_host_expert_ffn(dims, T, x, hw, [], [], 1, y, ws)   # no pairs: nothing to do


def test_offload_workspace_sizes_grow_with_tokens():
    dims = _dims(W.CONFIGS["dsv2_lite"])
    d1, h1 = M.moe_offload_workspace_size(dims, 1)
    d64, h64 = M.moe_offload_workspace_size(dims, 64)
    assert 0 < d1 < d64 and 0 < h1 < h64
    assert d64 >= M.moe_workspace_size(dims, 64, "standard")
