"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments on the host before any
HIP call (status codes from include/moe_route.h)."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_route_amd as M
from sparse_moe_layer_route_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_route.h")
L = B._lib
FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|int|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(M.EXPORTED) == names


def test_version_and_status_strings():
    assert M.moe_abi_version() == 2
    for s in range(5):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown status"


def dims(**kw):
    d = dict(hidden=256, n_experts=8, top_k=2, inter=512, n_shared=1, shared_inter=512,
             lore_rank=8, renormalize=False, shared_gate=False, floe_keep=0, dtype="f32")
    d.update(kw)
    return M.Dims(**d).c()


def ws_size(d, T, mode):
    n = ctypes.c_size_t(0)
    st = L.moe_workspace_size(ctypes.byref(d), T, mode, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(n_experts=65), B.MOE_EUNSUPPORTED), (dict(top_k=9), B.MOE_EUNSUPPORTED),
    (dict(top_k=9, n_experts=8), B.MOE_EUNSUPPORTED), (dict(hidden=250), B.MOE_EUNSUPPORTED),
    (dict(inter=500), B.MOE_EUNSUPPORTED), (dict(lore_rank=12), B.MOE_EUNSUPPORTED),
    (dict(lore_rank=128), B.MOE_EUNSUPPORTED), (dict(hidden=0), B.MOE_EINVAL),
    (dict(top_k=0), B.MOE_EINVAL), (dict(shared_inter=100), B.MOE_EUNSUPPORTED),
    (dict(tie_margin=-1.0), B.MOE_EINVAL), ({}, B.MOE_OK),
    (dict(weight_layout="mfma16"), B.MOE_EUNSUPPORTED),                  # fp32
    (dict(weight_layout="mfma16", dtype="bf16"), B.MOE_OK),
    (dict(weight_layout="mfma16", dtype="bf16", up_format="int2_g64"), B.MOE_EUNSUPPORTED),
])
def test_dims_validation(kw, status):
    assert ws_size(dims(**kw), 16, 0)[0] == status


def test_mode_validation():
    assert ws_size(dims(), 16, 3)[0] == B.MOE_EUNSUPPORTED            # FLOE needs INT2 up
    assert ws_size(dims(lore_rank=0), 16, 1)[0] == B.MOE_EUNSUPPORTED  # LORE needs factors
    fl = dims(up_format="int2_g64", floe_keep=600)
    assert ws_size(fl, 1, 3)[0] == B.MOE_EINVAL                        # keep > I
    assert ws_size(dims(up_format="int2_g64", floe_keep=51), 1, 3)[0] == B.MOE_OK
    assert ws_size(dims(up_format="int2_g64", floe_keep=51), 1, 0)[0] == B.MOE_EUNSUPPORTED
    # FloE keeps a whole |u| row and the packed x of a token in on-chip memory
    big_i = dims(up_format="int2_g64", floe_keep=51, inter=16384 + 64)
    big_h = dims(up_format="int2_g64", floe_keep=51, hidden=16384 + 64)
    assert ws_size(big_i, 1, 3)[0] == B.MOE_EUNSUPPORTED
    assert ws_size(big_h, 1, 3)[0] == B.MOE_EUNSUPPORTED
    assert ws_size(dims(up_format="int2_g64", floe_keep=51, hidden=16384), 1, 3)[0] == B.MOE_OK
    assert ws_size(dims(), 16, 7)[0] == B.MOE_EINVAL
    assert ws_size(dims(), -1, 0)[0] == B.MOE_EINVAL


def test_workspace_grows_with_tokens():
    a = ws_size(dims(), 1, 0)[1]; b = ws_size(dims(), 64, 0)[1]
    assert 0 < a < b and a % 256 == 0


def _weights(**over):
    w = {n: FAKE for n in B._WEIGHT_FIELDS}
    w.update(over)
    return B.MoeWeights(*[w[n] for n in B._WEIGHT_FIELDS])


def fwd(d, T, w, resident, stride, mode, out, ws, ws_bytes, x=FAKE):
    return L.moe_layer_forward(ctypes.byref(d), T, x, ctypes.byref(w), resident, stride, mode, out,
                               None, ws, ws_bytes, None)


def test_layer_forward_host_checks():
    d = dims()
    need = ws_size(d, 16, 1)[1]
    w = _weights()
    assert fwd(d, 16, w, FAKE, 0, 1, FAKE, FAKE, need - 1) == B.MOE_EWORKSPACE
    assert fwd(d, 16, w, None, 0, 1, FAKE, FAKE, need) == B.MOE_EINVAL        # LORE needs a mask
    assert fwd(d, 16, w, FAKE, 2, 1, FAKE, FAKE, need) == B.MOE_EINVAL        # stride 0 or 1
    assert fwd(d, 16, _weights(lore_A=None), FAKE, 0, 1, FAKE, FAKE, need) == B.MOE_EINVAL
    assert fwd(d, 16, _weights(w_up=None), FAKE, 0, 0, FAKE, FAKE, need) == B.MOE_EINVAL
    assert fwd(d, 16, w, FAKE, 0, 1, FAKE + 2, FAKE, need) == B.MOE_EINVAL    # misaligned out
    assert fwd(d, 16, w, FAKE, 0, 1, FAKE, FAKE, need, x=None) == B.MOE_EINVAL
    assert fwd(d, 16, _weights(ws_gate=None), FAKE, 0, 0, FAKE, FAKE, need) == B.MOE_EINVAL
    dg = dims(shared_gate=True)
    assert fwd(dg, 16, _weights(w_shared_gate=None), FAKE, 0, 0, FAKE, FAKE, need) == B.MOE_EINVAL
    # T = 0 with valid arguments enqueues nothing and succeeds (no GPU touched)
    assert fwd(d, 0, w, FAKE, 0, 1, FAKE, FAKE, need) == B.MOE_OK


def test_32bit_offset_limits():
    # T * k * max(H, I, n_s * I_s) must stay below 2^31
    d = dims(hidden=4096, inter=512, n_shared=0, shared_inter=0)
    big = (1 << 31) // (2 * 4096)          # k = 2
    assert ws_size(d, big - 1, 0)[0] == B.MOE_OK
    assert ws_size(d, big, 0)[0] == B.MOE_EUNSUPPORTED
    d = dims(hidden=256, inter=512, n_shared=2, shared_inter=1 << 20)   # wide shared block
    assert ws_size(d, 1 << 9, 0)[0] == B.MOE_EUNSUPPORTED
    assert ws_size(d, (1 << 9) - 1, 0)[0] == B.MOE_OK
    # one expert matrix past 2^31 elements
    assert ws_size(dims(hidden=1 << 16, inter=1 << 15), 1, 0)[0] == B.MOE_EUNSUPPORTED
    assert ws_size(dims(hidden=1 << 16, inter=(1 << 15) - 16), 1, 0)[0] == B.MOE_OK


def test_layout_field_out_of_range():
    d = dims(dtype="bf16")
    d.weight_layout = 7
    assert ws_size(d, 16, 0)[0] == B.MOE_EINVAL


def test_pack_size_and_checks():
    # rows padded to 16, cols to 32, 2 bytes each
    assert M.moe_pack_size(1, 40, 72) == 48 * 96 * 2
    assert M.moe_pack_size(3, 64, 2048) == 3 * 64 * 2048 * 2
    n = ctypes.c_size_t(0)
    for g, r, c in [(0, 16, 32), (1, 0, 32), (1, 16, 12), (1, 16, -8)]:
        assert L.moe_pack_size(g, r, c, ctypes.byref(n)) == B.MOE_EINVAL
    assert L.moe_pack_size(1, 16, 32, None) == B.MOE_EINVAL
    assert L.moe_pack_weights(1, 16, 32, None, FAKE, None) == B.MOE_EINVAL
    assert L.moe_pack_weights(1, 16, 32, FAKE, FAKE + 8, None) == B.MOE_EINVAL   # misaligned
    assert L.moe_pack_weights(1, 16, 32, FAKE, FAKE + 512, None) == B.MOE_EINVAL  # overlap
    assert L.moe_pack_weights(1, 16, 12, FAKE, FAKE + 4096, None) == B.MOE_EINVAL  # cols % 8


def test_pack_weights_binding_rejects_non_bf16():
    import torch
    d32 = M.Dims(hidden=256, n_experts=8, top_k=2, inter=512, dtype="f32")
    with pytest.raises(ValueError):
        M.pack_weights(d32, {})
    d16 = M.Dims(hidden=256, n_experts=8, top_k=2, inter=512, dtype="bf16")
    w = {"w_gate": torch.zeros(8 * 512 * 256, dtype=torch.float32)}
    with pytest.raises(ValueError):
        M.pack_weights(d16, w)


def test_floe_predict_and_pack_host_checks():
    fl = dims(dtype="bf16", up_format="int2_g64", floe_keep=16, n_shared=0, shared_inter=0)
    w = _weights()
    need = ws_size(fl, 16, 3)[1]
    pr, pk = L.moe_floe_predict, L.moe_floe_pack
    assert pr(ctypes.byref(fl), 16, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, need - 256,
              None) == B.MOE_EWORKSPACE
    assert pr(ctypes.byref(fl), 16, None, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, need,
              None) == B.MOE_EINVAL
    assert pr(ctypes.byref(fl), 16, FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, need,
              None) == B.MOE_EINVAL                                    # flags required
    assert pr(ctypes.byref(fl), 40000, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, 1 << 40,
              None) == B.MOE_EUNSUPPORTED                              # T*k > 65535
    assert pr(ctypes.byref(dims(dtype="bf16")), 16, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE,
              need, None) == B.MOE_EUNSUPPORTED                        # not the INT2 format
    assert pr(ctypes.byref(fl), 0, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, 1 << 20,
              None) == B.MOE_OK
    assert pk(ctypes.byref(fl), 16, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == B.MOE_EINVAL
    assert pk(ctypes.byref(fl), 40000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_EUNSUPPORTED
    assert pk(ctypes.byref(fl), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_OK


def test_lore_fit_host_checks():
    n = ctypes.c_size_t(0)
    assert L.moe_lore_fit_size(256, 512, 8, 16, ctypes.byref(n)) == B.MOE_OK and n.value > 256 * 256 * 4
    for args in [(256, 512, 0, 16), (256, 512, 17, 16), (256, 512, 8, 65), (32, 64, 8, 48),
                 (256, 0, 8, 16)]:
        assert L.moe_lore_fit_size(*args, ctypes.byref(n)) == B.MOE_EINVAL
    d = dims(dtype="bf16")
    fit = L.moe_lore_fit
    assert fit(ctypes.byref(d), 512, FAKE, FAKE, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
               None) == B.MOE_EWORKSPACE
    assert fit(ctypes.byref(d), 512, FAKE, None, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
               None) == B.MOE_EINVAL
    assert fit(ctypes.byref(d), 512, FAKE, FAKE, 8, 4, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
               None) == B.MOE_EINVAL                                    # cols < rank
    w = _weights()
    tg = L.moe_lore_targets
    assert tg(ctypes.byref(d), 64, FAKE, ctypes.byref(w), 8, FAKE, FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert tg(ctypes.byref(d), 64, FAKE, ctypes.byref(w), 1, FAKE, FAKE, 16, None) == B.MOE_EWORKSPACE
    assert tg(ctypes.byref(d), 0, FAKE, ctypes.byref(w), 1, FAKE, FAKE, 1 << 30, None) == B.MOE_OK


def test_entry_point_null_checks():
    d = dims()
    P = ctypes.c_void_p
    assert L.moe_route(ctypes.byref(d), 4, None, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None,
                       None) == B.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 4, FAKE, FAKE, None, 0, 2, FAKE, FAKE, FAKE, FAKE, None, None,
                       None) == B.MOE_EINVAL                                   # stall-free needs masks
    assert L.moe_route(ctypes.byref(d), 4, FAKE, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None,
                       None) == B.MOE_EINVAL                                   # logits are required
    assert L.moe_route(ctypes.byref(d), 0, FAKE, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                       None) == B.MOE_OK
    assert L.moe_permute(4, 9, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.MOE_EUNSUPPORTED
    assert L.moe_permute(4, 2, 65, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.MOE_EUNSUPPORTED
    assert L.moe_permute(4, 2, 8, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.MOE_EINVAL
    # more than 1024 pairs: the per-chunk histograms need the workspace
    assert L.moe_permute(600, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.MOE_EINVAL
    assert L.moe_permute(600, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == B.MOE_EWORKSPACE
    assert L.moe_prefetch_mask(ctypes.byref(d), 4, FAKE, FAKE, None, FAKE, FAKE, None) == B.MOE_EINVAL
    pa = L.moe_prefetch_adaptive
    for tau in (0.0, 1.0, -0.5, float("nan")):   # tau must lie in (0, 1)
        assert pa(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, tau, None, FAKE, FAKE, FAKE, None, None,
                  None) == B.MOE_EINVAL
    assert pa(ctypes.byref(d), 4, FAKE, FAKE, None, FAKE, 0.9, None, FAKE, FAKE, FAKE, None, None,
              None) == B.MOE_EINVAL                                   # w_delta required
    assert pa(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, 0.9, None, FAKE, FAKE, FAKE, FAKE, FAKE,
              None) == B.MOE_EINVAL                                   # diagnostics need topk_ids
    assert pa(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, 0.9, FAKE, FAKE, FAKE, FAKE, FAKE, None,
              None) == B.MOE_EINVAL                                   # both diagnostics or neither
    assert pa(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, 0.9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
              None) == B.MOE_OK
    assert L.moe_lore_surrogate(ctypes.byref(dims(lore_rank=0)), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None) == B.MOE_EUNSUPPORTED
    assert L.moe_combine(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                         None) == B.MOE_EINVAL
    w = _weights()
    assert L.moe_expert_ffn(ctypes.byref(d), 4, FAKE, ctypes.byref(w), 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None, None, FAKE, 0, None) == B.MOE_EWORKSPACE


def test_noalloc_forward_host_checks():
    """The allocation-free forward validates like moe_layer_forward and
    refuses a batch whose workspace exceeds its scratch array before
    touching the GPU (T = 0 returns at once)."""
    f = L.moe_layer_forward_noalloc
    d = dims()
    w = _weights()
    assert f(ctypes.byref(d), 16, FAKE, ctypes.byref(w), None, 0, 1, FAKE, None) == B.MOE_EINVAL
    assert f(ctypes.byref(d), 16, FAKE, ctypes.byref(w), FAKE, 0, 1, FAKE + 2, None) == B.MOE_EINVAL
    assert f(ctypes.byref(d), 0, FAKE, ctypes.byref(w), FAKE, 0, 1, FAKE, None) == B.MOE_OK
    big = dims(hidden=4096, inter=4096, n_shared=0, shared_inter=0)
    T = 8192
    assert ws_size(big, T, 0)[1] > M.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), T, FAKE, ctypes.byref(_weights()), None, 0, 0, FAKE, None) == B.MOE_EWORKSPACE
