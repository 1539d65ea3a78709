"""moe_layer_forward_noalloc (the forward on the library's own scratch array)
against moe_layer_forward on a caller workspace: bit-identical outputs on two
calls in a row, the second with a smaller batch, and a batch too large for
the scratch array refused on the host."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.device import dims_dict, mask_tensor, tensor

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_moe_layer_route_amd as M  # noqa: E402
from gpu_harness import dev_weights, packed_weights, prefetch_masks_gpu, say  # noqa: E402


def _both(layer, T, mode, layout):
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg), weight_layout=layout)
    wdev = packed_weights(layer) if layout == "mfma16" else dev_weights(layer)
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    if mode == "lore":
        res, stride = mask_tensor([layer.resident()], "cuda"), 0
    elif mode == "stall_free":
        _, _, res = prefetch_masks_gpu(layer, T, dev_weights(layer))
        stride = 1
    else:
        res, stride = None, 0
    odt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    ref = torch.empty(T, cfg.hidden, dtype=odt, device="cuda")
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    M.moe_layer_forward(dims, T, x, wdev, res, stride, mode, ref, ws)
    out = torch.full_like(ref, float("nan"))
    M.moe_layer_forward_noalloc(dims, T, x, wdev, res, stride, mode, out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("name,mode,layout,T1,T2", [
    ("dsv2_lite", "lore", "mfma16", 64, 8),
    ("dsv2_lite", "standard", "mfma16", 64, 1),
    ("granite_small", "stall_free", "rows", 203, 37),
    ("tiny", "lore", "rows", 16, 5),
    ("floe_small", "floe", "rows", 6, 2),
])
def test_noalloc_matches_workspace_forward(name, mode, layout, T1, T2):
    import dataclasses
    if name == "granite_small":
        cfg = dataclasses.replace(W.CONFIGS["granite_prefill"], name="granite_small", hidden=384,
                                  inter=144, token_counts=(203,), seed=103)
        layer = W.Layer(cfg)
    elif name == "floe_small":
        # FloE with gated shared experts: the fused slice-sum + combine launch
        cfg = dataclasses.replace(W.CONFIGS["mixtral_floe"], name="floe_small_sh", hidden=1024,
                                  n_experts=4, inter=1040, floe_keep=104, n_shared=1,
                                  shared_inter=256, shared_gate=True, token_counts=(6,), seed=113)
        layer = W.Layer(cfg)
    else:
        layer = W.make_layer(name)
    for T in (T1, T2):
        say(f"[noalloc] {name} mode={mode} layout={layout} T={T}")
        ref, out = _both(layer, T, mode, layout)
        assert torch.equal(out, ref), (name, mode, T)


def test_noalloc_refuses_batches_beyond_its_scratch():
    layer = W.make_layer("granite_prefill")
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg))
    T = 4096
    assert M.moe_workspace_size(dims, T, "standard") > M.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(M.MoEError):
        M.moe_layer_forward_noalloc(dims, T, x, dev_weights(layer), None, 0, "standard", out)
