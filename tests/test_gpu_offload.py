"""Exact execution of missed experts on the GPU [SPICE page, "CPU-GPU
collaboration: handling prefetch misses"]: moe_layer_forward_offload with
every non-resident expert slot on the GPU filled with NaN, so an expert that
is neither fetched nor run on the host poisons the output.  Each plan (all
fetched, all on the host, mixed by the cost rule) is checked against the
oracle's STANDARD forward, and against the GPU's own STANDARD forward on the
full weights."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads.device import dims_dict, tensor

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_moe_layer_route_amd as M  # noqa: E402
from gpu_harness import (TOL, dev_weights, oracle_forward_forced, out_to_np, rel_fro,  # noqa: E402
                         run_layer, say)

NAMES = ("w_gate", "w_up", "w_down")


def _pinned(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
        else torch.from_numpy(a)
    return t.pin_memory()


class Rig:
    """Host copies of the routed experts, device slots with the missed ones
    poisoned, and the workspaces for up to t_max tokens."""

    def __init__(self, layer, t_max):
        cfg = layer.cfg
        self.layer, self.cfg = layer, cfg
        self.dims = M.Dims(**dims_dict(cfg))
        self.res = layer.resident()
        self.host = {n: _pinned(layer.full(n), cfg.dtype) for n in NAMES}
        self.missing = [e for e in range(cfg.n_experts) if not (self.res >> e) & 1]
        self.wdev = dict(dev_weights(layer))
        self.poison()
        dev_b, host_b = M.moe_offload_workspace_size(self.dims, t_max)
        self.ws = torch.empty(dev_b, dtype=torch.uint8, device="cuda")
        self.hws = torch.empty(host_b, dtype=torch.uint8).pin_memory()

    def poison(self):
        for n in NAMES:
            t = self.wdev[n].clone()
            t[self.missing] = float("nan")
            self.wdev[n] = t
        torch.cuda.synchronize()

    def run(self, T, cost):
        cfg = self.cfg
        odt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        out = torch.full((T, cfg.hidden), float("nan"), dtype=odt, device="cuda")
        x = tensor(self.layer.x(T), cfg.dtype, "cuda")
        dec = np.zeros(cfg.n_experts, np.uint8)
        st = M.MoeOffloadStats()
        st.decision = dec.ctypes.data
        M.moe_layer_forward_offload(self.dims, T, x, self.wdev, self.host, self.res, cost, out,
                                    self.ws, self.hws, stats=st)
        torch.cuda.synchronize()
        return out_to_np(out), st, dec


def _expected_plan(rig, ids, cost):
    tokens = np.bincount(ids.reshape(-1), minlength=rig.cfg.n_experts)
    return O.offload_plan(dims_dict(rig.cfg), [int(v) for v in tokens], rig.res,
                          cost.pcie_bytes_per_s, cost.gpu_expert_s, cost.cpu_pair_s,
                          cost.cpu_expert_s, bool(cost.queue_aware)), tokens


def _check(rig, T, cost, g, ref, want_kind):
    out, st, dec = rig.run(T, cost)
    plan, tokens = _expected_plan(rig, g.ids, cost)
    assert list(dec) == plan
    missed = [e for e in range(rig.cfg.n_experts) if plan[e] != O.OFFLOAD_NONE]
    assert st.missed_experts == len(missed) > 0
    fetched = [e for e in missed if plan[e] == O.OFFLOAD_FETCH]
    hosted = [e for e in missed if plan[e] == O.OFFLOAD_HOST]
    assert st.fetched_experts == len(fetched) and st.host_experts == len(hosted)
    assert st.host_pairs == int(sum(tokens[e] for e in hosted))
    if want_kind == "fetch":
        assert not hosted
    elif want_kind == "host":
        assert not fetched
    elif len(missed) > 1:
        assert fetched and hosted, (fetched, hosted)
    assert np.isfinite(out).all()
    tol = TOL[rig.cfg.dtype]
    err_o = rel_fro(out, ref["out"])
    err_g = rel_fro(out, g.out)
    say(f"[offload] {rig.cfg.name} T={T} {want_kind}: fetched={len(fetched)} host={len(hosted)} "
        f"pairs={st.host_pairs} vs oracle {err_o:.2e} vs gpu {err_g:.2e} "
        f"route {st.route_ms:.3f} ms host {st.host_ms:.3f} ms parallel {st.parallel_ms:.3f} ms "
        f"wall {st.wall_ms:.3f} ms")
    assert err_o <= tol, err_o
    if not hosted:
        # fetched experts run through the same kernels on the same weights
        assert np.array_equal(out, g.out)
    else:
        assert err_g <= tol, err_g
    # fetched slots now hold the host weights; host-run experts were never copied
    for n in NAMES:
        for e in fetched:
            assert torch.equal(rig.wdev[n][e].cpu(), rig.host[n][e])
        for e in hosted:
            assert torch.isnan(rig.wdev[n][e]).all()
    rig.poison()
    return st


def _costs(cfg, ids, res):
    """Cost tables that fetch every missed expert, run every one on the host,
    and (when the missed experts' pair counts differ) split them: the host
    takes the experts with at most the median count, the GPU fetches the
    rest."""
    elem = 2 if cfg.dtype == "bf16" else 4
    w_s = 3 * cfg.inter * cfg.hidden * elem / 50e9       # W_e / B_pcie
    costs = {"fetch": M.offload_cost(50e9, 0.0, 1.0, 8),  # host time huge
             "host": M.offload_cost(50e9, 1.0, 0.0, 8),   # GPU time huge
             # host a little cheaper per expert, but the link and the host
             # fill up as queues: the experts alternate between the two
             "queued": M.offload_cost(50e9, 0.0, 0.0, 8, cpu_expert_s=0.9 * w_s,
                                      queue_aware=True)}
    tokens = np.bincount(ids.reshape(-1), minlength=cfg.n_experts)
    counts = sorted({int(tokens[e]) for e in range(cfg.n_experts)
                     if tokens[e] and not (res >> e) & 1})
    if len(counts) > 1:
        thr = counts[(len(counts) - 1) // 2]
        costs["mixed"] = M.offload_cost(50e9, 0.0, w_s / (thr + 0.5), 8)
    return costs


@pytest.mark.parametrize("name,T", [("dsv2_lite", 8), ("dsv2_lite", 1), ("tiny", 16)])
def test_offload_plans_match_standard(name, T):
    layer = W.make_layer(name)
    cfg = layer.cfg
    g = run_layer(layer, T, "standard")
    ref = oracle_forward_forced(layer, T, "standard", g, list(range(T)))
    rig = Rig(layer, T)
    costs = _costs(cfg, g.ids, rig.res)
    assert T == 1 or "mixed" in costs
    for kind, cost in costs.items():
        _check(rig, T, cost, g, ref, kind)


def test_offload_reuses_workspaces_across_batches():
    layer = W.make_layer("dsv2_lite")
    rig = Rig(layer, 64)
    for T, kind in ((64, "mixed"), (5, "host"), (64, "fetch"), (64, "queued")):
        g = run_layer(layer, T, "standard")
        ref = oracle_forward_forced(layer, T, "standard", g, list(range(T)))
        _check(rig, T, _costs(layer.cfg, g.ids, rig.res)[kind], g, ref, kind)


def test_offload_host_checks():
    layer = W.make_layer("tiny")
    cfg = layer.cfg
    rig = Rig(layer, 4)
    x = tensor(layer.x(4), cfg.dtype, "cuda")
    out = torch.empty(4, cfg.hidden, dtype=torch.float32, device="cuda")
    cost = M.offload_cost(50e9, 0.0, 0.0)
    small = torch.empty(64, dtype=torch.uint8).pin_memory()
    with pytest.raises(M.MoEError) as ei:
        M.moe_layer_forward_offload(rig.dims, 4, x, rig.wdev, rig.host, rig.res, cost, out,
                                    rig.ws, small)
    assert ei.value.status == M.binding.MOE_EWORKSPACE
    with pytest.raises(M.MoEError) as ei:
        M.moe_layer_forward_offload(rig.dims, 4, x, rig.wdev, rig.host, rig.res,
                                    M.offload_cost(0.0, 0.0, 0.0), out, rig.ws, rig.hws)
    assert ei.value.status == M.binding.MOE_EINVAL


def test_offload_without_misses_is_the_standard_forward():
    """All experts resident: nothing to fetch or run on the host, and the
    output is the STANDARD forward's bit for bit; T = 0 enqueues nothing."""
    layer = W.make_layer("dsv2_lite")
    cfg = layer.cfg
    T = 8
    g = run_layer(layer, T, "standard")
    rig = Rig(layer, T)
    rig.res = (1 << cfg.n_experts) - 1
    rig.wdev = dict(dev_weights(layer))          # every slot valid
    out, st, dec = rig.run(T, M.offload_cost(50e9, 0.0, 0.0, 4))
    assert st.missed_experts == 0 and st.fetched_experts == 0 and st.host_pairs == 0
    assert not dec.any()
    assert np.array_equal(out, g.out)
    x = tensor(layer.x(1), cfg.dtype, "cuda")
    o = torch.empty(1, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    M.moe_layer_forward_offload(rig.dims, 0, x, rig.wdev, rig.host, rig.res,
                                M.offload_cost(50e9, 0.0, 0.0), o, rig.ws, rig.hws)


def test_offload_single_host_thread_matches_many():
    """The host FFN's thread count does not change a bit of the output."""
    layer = W.make_layer("dsv2_lite")
    T = 5
    rig = Rig(layer, T)
    outs = []
    for threads in (1, 16):
        out, st, _ = rig.run(T, M.offload_cost(50e9, 1.0, 0.0, threads))
        assert st.host_pairs > 0 and st.fetched_experts == 0
        outs.append(out)
    assert np.array_equal(outs[0], outs[1])
