"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example derived by hand from scalar closed forms, brute force over all subsets,
pure-Python loops on tiny shapes, identities, or reductions between modes.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------- hand example --
def _hand():
    with open(os.path.join(GOLD, "hand_example.json")) as f:
        g = json.load(f)
    w = {k: np.array(g[k], dtype=np.float32) for k in
         ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
          "lore_A", "lore_B")}
    return g, np.array(g["x"], dtype=np.float32), w


def _mask(ids):
    m = 0
    for e in ids:
        m |= 1 << e
    return m


def _hand_expected():
    """Worked by hand.  Logits are [2, 1, 0.5, 0] (x picks column 0 of W_r).
    Expert outputs with x = [1, 0]: g = gate[0], u = up[0], y = SiLU(g) u down.
    SiLU(z) = z sigma(z)."""
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    s1, sm1, s2 = 1 * sig(1), -1 * sig(-1), 2 * sig(2)
    y0 = (2 * s1, -2 * s1)            # g=1, u=2, down=[1,-1]
    y1 = (0.0, 4 * sm1)               # g=-1, u=1, down=[0,4]
    y2 = (s2, s2)                     # g=2, u=1, down=[1,1]
    ys = (2 * s1, 0.0)                # shared: g=1, u=1, down=[2,0]
    Z = math.exp(2) + math.exp(1) + math.exp(0.5) + 1.0
    p = [math.exp(2) / Z, math.exp(1) / Z, math.exp(0.5) / Z, 1.0 / Z]
    w_ren = (p[0] / (p[0] + p[1]), p[1] / (p[0] + p[1]))     # = sigma(1), sigma(-1)
    w_un = (p[0], p[1])
    comb = lambda w, ya, yb: tuple(ys[i] + w[0] * ya[i] + w[1] * yb[i] for i in range(2))
    lore1 = (ys[0] + 0.0, ys[1] + 1.0)   # B1 A1 x = [0,1] * (1*1)
    w_sf = (p[0] / (p[0] + p[2]), p[2] / (p[0] + p[2]))      # = sigma(1.5), sigma(-1.5)
    return dict(p=p, w_ren=w_ren, sig15=sig(1.5),
                standard_renorm=comb(w_ren, y0, y1), standard_unnorm=comb(w_un, y0, y1),
                lore=comb(w_ren, y0, lore1),
                lore_zero=comb(w_ren, y0, ys),
                stall_free=comb(w_sf, y0, y2))


def test_hand_example_closed_forms_match_decimal_values():
    # The closed forms above reproduce the decimal values worked out by hand.
    ex = _hand_expected()
    np.testing.assert_allclose(ex["p"], [0.5792585299413738, 0.2130973042886238,
                                         0.1292500485531628, 0.0783941172168397], rtol=1e-15)
    np.testing.assert_allclose(ex["w_ren"][0], 0.7310585786300049, rtol=1e-15)
    np.testing.assert_allclose(ex["standard_renorm"], [2.5310104480370557, -1.358211243291099], rtol=1e-14)
    np.testing.assert_allclose(ex["stall_free"], [2.978866562875048, -0.8740299323461453], rtol=1e-14)


@pytest.mark.parametrize("case", ["standard_renorm", "standard_unnorm", "lore", "lore_zero", "stall_free"])
def test_hand_example(case):
    g, x, w = _hand()
    dims = dict(g["dims"])
    ex = _hand_expected()
    if case == "standard_unnorm":
        dims["renormalize"] = False
    mode = {"standard_renorm": "standard", "standard_unnorm": "standard", "lore": "lore",
            "lore_zero": "lore", "stall_free": "stall_free"}[case]
    if case == "lore_zero":
        w["lore_A"] = np.zeros_like(w["lore_A"])
        w["lore_B"] = np.zeros_like(w["lore_B"])
    resident = None
    if mode == "lore":
        resident = _mask(g["resident_lore"])
    if mode == "stall_free":
        resident = [_mask(g["prefetched_stall_free"])]
    r = O.layer_forward(x, w, dims, mode, resident=resident)
    np.testing.assert_allclose(r["out"][0], ex[case], rtol=1e-14, atol=1e-15)
    # decisions
    if mode == "stall_free":
        assert list(r["ids"][0]) == [0, 2] and r["n_subst"][0] == 1
        np.testing.assert_allclose(r["weights"][0], [ex["sig15"], 1 - ex["sig15"]], rtol=1e-14)
    else:
        assert list(r["ids"][0]) == [0, 1]
    np.testing.assert_allclose(r["mass"][0], ex["p"][0] + ex["p"][1], rtol=1e-15)
    if mode == "lore":
        assert list(r["exact"][0]) == [1, 0]


# ------------------------------------------------------- routing pins ----
def _rand_logits(rng, T, E, scale=1.0):
    return rng.standard_normal((T, E)) * scale


@pytest.mark.parametrize("E,k", [(8, 2), (8, 3), (6, 1), (5, 5), (7, 4)])
def test_topk_is_max_mass_subset(E, k):
    """Brute force over all C(E,k) subsets: the routed set maximises the
    probability mass (no ties in continuous random logits)."""
    rng = np.random.default_rng(10 + E * 10 + k)
    for l in _rand_logits(rng, 50, E, 2.0):
        ids, w, mass, flag = O.route_token(l, k, False, 1e-4)
        p = np.exp(l - l.max()); p /= p.sum()
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(p[list(s)]))
        assert set(ids) == set(best)
        assert math.isclose(mass, sum(p[list(best)]), rel_tol=1e-12)
        # rank order: descending logit
        assert all(l[ids[i]] >= l[ids[i + 1]] for i in range(k - 1))


def test_topk_ties_go_to_lower_id():
    l = np.array([1.0, 3.0, 3.0, 0.5, 3.0])
    ids, _, _, flag = O.route_token(l, 2, False, 1e-4)
    assert ids == [1, 2] and flag  # 3.0 vs 3.0 at the cut: near-tie
    ids, _, _, flag = O.route_token(l, 3, False, 1e-4)
    assert ids == [1, 2, 4] and not flag


def test_weights_mass_identities():
    """Renormalised weights sum to 1; unnormalised sum to the SPICE confidence
    mass C in [k/E, 1]; softmax sums to 1 and ignores a logit shift."""
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (64, 6), (64, 8), (40, 8)]:
        for l in _rand_logits(rng, 20, E):
            _, wr, C, _ = O.route_token(l, k, True, 1e-4)
            _, wu, C2, _ = O.route_token(l, k, False, 1e-4)
            assert math.isclose(wr.sum(), 1.0, rel_tol=1e-12)
            assert math.isclose(wu.sum(), C, rel_tol=1e-12) and C == C2
            assert k / E - 1e-12 <= C <= 1.0 + 1e-12
            p = O.softmax(l)
            assert math.isclose(p.sum(), 1.0, rel_tol=1e-12)
            np.testing.assert_allclose(O.softmax(l + 7.25), p, rtol=1e-12)


def test_softmax_two_expert_closed_form():
    for a, b in [(0.0, 0.0), (1.0, -2.0), (30.0, 29.5)]:
        p = O.softmax(np.array([a, b]))
        assert math.isclose(p[0], 1.0 / (1.0 + math.exp(b - a)), rel_tol=1e-14)


def test_router_logits_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5)); wr = rng.standard_normal((4, 5))     # [E][H]
    l = O.router_logits(x, wr)
    for t in range(3):
        for e in range(4):
            assert math.isclose(l[t, e], sum(x[t, h] * wr[e, h] for h in range(5)), rel_tol=1e-12)


# ----------------------------------------------------- stall-free pins ----
def _masked_topk(l, allowed, k):
    return set(sorted(allowed, key=lambda e: (-l[e], e))[:k])


def test_stall_free_equals_topk_within_prefetched_set():
    """Algorithm 1 picks keep = routed and prefetched, and fills each miss with
    the best remaining prefetched expert.  Every routed expert outranks every
    non-routed one, so the result is the top-k of the router restricted to the
    prefetched set -- checked by brute force on random tiny layers."""
    rng = np.random.default_rng(5)
    for _ in range(400):
        E = int(rng.integers(3, 10)); k = int(rng.integers(1, E + 1))
        l = rng.standard_normal(E)
        routed = O.rank_experts(l)[:k]
        n = int(rng.integers(k, E + 1))
        kp = set(rng.permutation(E)[:n].tolist())
        S, _ = O.stall_free_select(routed, l, kp, 1e-4)
        assert len(S) == k and S <= kp
        assert S == _masked_topk(l, kp, k)
        assert set(routed) & kp <= S          # everything prefetched and routed is kept


def test_stall_free_literal_sets():
    l = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0])
    # all hit
    assert O.stall_free_select([0, 1], l, {0, 1, 5}, 1e-4) == ({0, 1}, False)
    # one miss (1), candidates {3, 5}: the higher score 3 substitutes
    assert O.stall_free_select([0, 1], l, {0, 3, 5}, 1e-4)[0] == {0, 3}
    # both missing, take the best two of {2, 4, 5}
    assert O.stall_free_select([0, 1], l, {2, 4, 5}, 1e-4)[0] == {2, 4}
    # near-tie between the last substitute and the next candidate is flagged
    l2 = np.array([5.0, 4.0, 1.0, 1.00005, 0.0])
    S, f = O.stall_free_select([0, 1], l2, {0, 2, 3}, 1e-4)
    assert S == {0, 3} and f


def test_delta_star_bounds_substitution():
    """With delta >= delta* the routed set is inside the prefetched list, so no
    substitution happens [APEX Sec. 4.2]; delta = N-k prefetches everything;
    a prefetch router equal to the router with delta = 0 prefetches K_r."""
    rng = np.random.default_rng(6)
    E, k = 12, 3
    for _ in range(100):
        l = rng.standard_normal(E); lp = rng.standard_normal(E)
        routed = O.rank_experts(l)[:k]
        ds = O.delta_star(routed, lp, k)
        for d in range(ds, E - k + 1):
            m, _ = O.prefetch_set(lp, k + d, 1e-4)
            kp = {e for e in range(E) if (m >> e) & 1}
            assert O.stall_free_select(routed, l, kp, 1e-4)[0] == set(routed)
        if ds > 0:
            m, _ = O.prefetch_set(lp, k + ds - 1, 1e-4)
            kp = {e for e in range(E) if (m >> e) & 1}
            assert not set(routed) <= kp
        m, _ = O.prefetch_set(l, k, 1e-4)
        assert {e for e in range(E) if (m >> e) & 1} == set(routed)


# ------------------------------------------------------ permutation pins --
def test_permutation_bucket_append_brute_force():
    """Against a list-append counting sort written with plain loops."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        T, k, E = int(rng.integers(1, 12)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        ids = rng.integers(0, E, size=(T, k))
        exact = rng.integers(0, 2, size=(T, k))
        off, perm, inv = O.permute(ids, exact, E)
        buckets = [[] for _ in range(E)]
        for t in range(T):
            for j in range(k):
                if exact[t, j]:
                    buckets[ids[t, j]].append(t * k + j)
        assert list(perm) == [f for b in buckets for f in b]
        assert list(off) == [sum(len(b) for b in buckets[:e]) for e in range(E + 1)]
        for f in range(T * k):
            if exact.reshape(-1)[f]:
                assert perm[inv[f]] == f
            else:
                assert inv[f] == -1


# --------------------------------------------------------------- FFN pins --
def test_swiglu_brute_force_loops():
    rng = np.random.default_rng(8)
    H, I, T = 5, 3, 2
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((I, H)); wu = rng.standard_normal((I, H)); wd = rng.standard_normal((H, I))
    y = O.swiglu_expert(x, wg, wu, wd)
    for t in range(T):
        a = []
        for i in range(I):
            g = sum(x[t, h] * wg[i, h] for h in range(H))
            u = sum(x[t, h] * wu[i, h] for h in range(H))
            a.append(g / (1 + math.exp(-g)) * u)
        for h in range(H):
            assert math.isclose(y[t, h], sum(a[i] * wd[h, i] for i in range(I)), rel_tol=1e-12)


def test_silu_sigmoid_closed_forms():
    assert O.silu(np.float64(0.0)) == 0.0
    assert math.isclose(O.silu(np.float64(1.0)), 0.7310585786300049, rel_tol=1e-15)
    assert O.silu(np.float64(-800.0)) == 0.0          # no NaN at the far tail
    assert O.silu(np.float64(800.0)) == 800.0
    assert O.sigmoid(np.float64(0.0)) == 0.5


def test_lore_brute_force_and_rank1():
    rng = np.random.default_rng(9)
    H, r = 6, 3
    x = rng.standard_normal(H); A = rng.standard_normal((r, H)); B = rng.standard_normal((H, r))
    res = O.lore_residual(x, A, B)
    for h in range(H):
        z = [sum(A[q, i] * x[i] for i in range(H)) for q in range(r)]
        assert math.isclose(res[h], sum(B[h, q] * z[q] for q in range(r)), rel_tol=1e-12)
    # rank 1, A = e_j^T, B = b  =>  residual = x_j b
    j = 4; b = rng.standard_normal(H)
    A1 = np.zeros((1, H)); A1[0, j] = 1.0
    np.testing.assert_allclose(O.lore_residual(x, A1, b[:, None]), x[j] * b, rtol=1e-15)


# -------------------------------------------------------------- INT2 pins --
def test_int2_unpack_and_dequant_closed_forms():
    # byte 0xE4 = 0b11_10_01_00 holds codes h0..h3 = 0, 1, 2, 3
    q = np.full((1, 16), 0xE4, dtype=np.uint8)            # H = 64
    s = np.array([[np.float16(2.0).view(np.uint16)]], dtype=np.uint16)
    z = np.array([[np.float16(1.5).view(np.uint16)]], dtype=np.uint16)
    w = O.dequant_int2(q, s, z)
    np.testing.assert_array_equal(w[0, :4], [-3.0, -1.0, 1.0, 3.0])
    np.testing.assert_array_equal(w[0], np.tile([-3.0, -1.0, 1.0, 3.0], 16))
    # a second group uses its own scale/zero
    q2 = np.zeros((1, 32), dtype=np.uint8); q2[0, 16:] = 0xFF      # group 1: all code 3
    s2 = np.array([[np.float16(1.0).view(np.uint16), np.float16(0.5).view(np.uint16)]])
    z2 = np.array([[np.float16(0.0).view(np.uint16), np.float16(1.0).view(np.uint16)]])
    w2 = O.dequant_int2(q2, s2, z2)
    assert np.all(w2[0, :64] == 0.0) and np.all(w2[0, 64:] == 1.0)


def test_quantiser_error_bound():
    """Round-to-nearest codes are within s/2 of the weight (the fp16 rounding
    of s and z adds a little; clamping only affects the group's extremes)."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((4, 256)).astype(np.float32) * 0.02
    q, s, z = W.quantize_int2_g64(w)
    wh = O.dequant_int2(q, s, z)
    sf = np.repeat(O.fp16_to_f64(s), 64, axis=-1)
    assert np.all(np.abs(wh - w) <= 0.5 * sf * (1 + 4e-3) + 1e-7)


def _floe_layer(rng, H=128, I=24, keep=5):
    q, s, z = W.quantize_int2_g64(rng.standard_normal((I, H)).astype(np.float32) * 0.1)
    wg = rng.standard_normal((I, H)) * 0.1
    wd = rng.standard_normal((I, H)) * 0.1
    return q, s, z, wg, wd


def test_floe_full_keep_equals_dense_swiglu():
    """keep = 100% makes FloE's forward the dense SwiGLU FFN on the decoded up
    weights [FloE Sec. 1, S_t = identity]."""
    rng = np.random.default_rng(12)
    q, s, z, wg, wd = _floe_layer(rng)
    x = rng.standard_normal(128)
    y, u, keep, _ = O.floe_expert(x, wg, q, s, z, wd, 24, 1e-4)
    dense = O.swiglu_expert(x[None], wg, O.dequant_int2(q, s, z), wd.T)[0]
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-14)
    assert list(keep) == list(range(24))


def test_floe_keep_one_closed_form_and_mask_rule():
    rng = np.random.default_rng(13)
    q, s, z, wg, wd = _floe_layer(rng)
    x = rng.standard_normal(128)
    y, u, keep, _ = O.floe_expert(x, wg, q, s, z, wd, 1, 1e-4)
    i = int(np.argmax(np.abs(u)))
    assert list(keep) == [i]
    g = float(wg[i] @ x)
    np.testing.assert_allclose(y, g / (1 + math.exp(-g)) * u[i] * wd[i], rtol=1e-12)
    # keep = 5: exactly the five largest |u|, listed ascending
    y5, u5, keep5, _ = O.floe_expert(x, wg, q, s, z, wd, 5, 1e-4)
    assert set(keep5) == set(np.argsort(-np.abs(u5), kind="stable")[:5]) and list(keep5) == sorted(keep5)


def test_floe_mask_brute_force_and_sign_scale_invariance():
    """The kept set is the n-subset with the largest sum of |u| (brute force
    over every 4-subset of 10 channels); it depends on |u| only, so x, -x and
    3x keep the same channels."""
    rng = np.random.default_rng(31)
    q, s, z, _, _ = _floe_layer(rng, H=64, I=10)
    x = rng.standard_normal(64)
    keep, _, u = O.floe_channel_mask(x, q, s, z, 4, 1e-4)
    best = max(itertools.combinations(range(10), 4), key=lambda c: sum(abs(u[i]) for i in c))
    assert list(keep) == sorted(best)
    for c in (-1.0, 3.0):
        assert list(O.floe_channel_mask(c * x, q, s, z, 4, 1e-4)[0]) == list(keep)


def test_floe_predictor_on_the_true_input_is_exact_and_recall_closed_forms():
    """With h_prev equal to the layer's own input the predicted masks are the
    layer's masks (recall 1); recall counts the shared channels over |true|."""
    rng = np.random.default_rng(32)
    E, I, H, keep = 3, 24, 128, 5
    layers = [_floe_layer(rng, H=H, I=I) for _ in range(E)]
    q = np.stack([l[0] for l in layers]); sc = np.stack([l[1] for l in layers])
    z = np.stack([l[2] for l in layers])
    x = rng.standard_normal((2, H))
    ids = np.array([[2, 0], [1, 2]])
    pk, fl = O.floe_predict_masks(x, ids, q, sc, z, keep, 1e-4)
    for t in range(2):
        for j in range(2):
            e = ids[t, j]
            _, _, kt, _ = O.floe_expert(x[t], layers[e][3], q[e], sc[e], z[e], layers[e][4], keep, 1e-4)
            assert list(pk[t, j]) == list(kt) and O.mask_recall(pk[t, j], kt) == 1.0
    assert O.mask_recall([1, 2, 3, 4], [5, 6, 7, 8]) == 0.0
    assert O.mask_recall([1, 2, 9, 8], [1, 2, 3, 4]) == 0.5
    # a far-off previous state predicts worse than a near one (same weights)
    near = x + 0.01 * rng.standard_normal(x.shape)
    r_near = np.mean([O.mask_recall(a, b) for a, b in
                      zip(O.floe_predict_masks(near, ids, q, sc, z, keep, 1e-4)[0].reshape(-1, keep),
                          pk.reshape(-1, keep))])
    assert r_near == 1.0


def test_floe_pack_reproduces_the_sparse_forward():
    """The compact gate and down blocks of the kept channels, used as a dense
    SwiGLU over n_keep channels, give FloE's output: a wrong, shuffled or
    transposed row selection would not."""
    rng = np.random.default_rng(33)
    q, s, z, wg, wd = _floe_layer(rng, H=128, I=24)
    x = rng.standard_normal(128)
    y, u, keep, _ = O.floe_expert(x, wg, q, s, z, wd, 6, 1e-4)
    gc, dc = O.floe_pack(keep, wg, wd)
    assert gc.shape == (6, 128) and dc.shape == (6, 128)
    y_c = (O.silu(gc @ x) * u[keep]) @ dc
    np.testing.assert_allclose(y_c, y, rtol=1e-12, atol=1e-14)


def _orthogonal_design(rng, N, H):
    blocks = [np.linalg.qr(rng.standard_normal((H, H)))[0] * np.sqrt(H) for _ in range(N // H)]
    return np.concatenate(blocks, axis=0)


def test_lore_fit_map_is_least_squares_under_orthogonal_design():
    """With h^T h = N I the map R^T h / N is lstsq's solution, and the rank-r
    residual obeys Eckart-Young: ||R - h M_r^T||^2 = ||R - h M^T||^2 +
    N * (sum of the dropped squared singular values)."""
    rng = np.random.default_rng(41)
    N, H, r = 64, 32, 5
    h = _orthogonal_design(rng, N, H)
    R = rng.standard_normal((N, H)) @ rng.standard_normal((H, H)) * 0.1 + rng.standard_normal((N, H)) * 0.05
    A, B, sig, err = O.lore_fit(h, R, r)
    M_ls = np.linalg.lstsq(h, R, rcond=None)[0].T
    np.testing.assert_allclose(R.T @ h / N, M_ls, rtol=1e-10, atol=1e-12)
    S = np.linalg.svd(M_ls, compute_uv=False)
    np.testing.assert_allclose(sig, S[:r], rtol=1e-12)
    full = np.linalg.norm(R - h @ M_ls.T) ** 2
    want = math.sqrt(full + N * float(np.sum(S[r:] ** 2))) / np.linalg.norm(R)
    assert abs(err - want) < 1e-10
    # the error never grows with the rank, and rank H reproduces the LS fit
    errs = [O.lore_fit(h, R, q)[3] for q in (1, 2, 5, 10, 32)]
    assert all(a >= b - 1e-12 for a, b in zip(errs, errs[1:]))
    assert abs(errs[-1] - math.sqrt(full) / np.linalg.norm(R)) < 1e-10


def test_lore_fit_recovers_an_exact_low_rank_map():
    rng = np.random.default_rng(42)
    N, H, r = 96, 48, 4
    h = _orthogonal_design(rng, N, H)
    M_true = rng.standard_normal((H, r)) @ rng.standard_normal((r, H))
    A, B, sig, err = O.lore_fit(h, h @ M_true.T, r)
    assert err < 1e-12
    np.testing.assert_allclose(B @ A, M_true, rtol=1e-10, atol=1e-10)
    assert A.shape == (r, H) and B.shape == (H, r)
    # A has orthonormal rows; B's columns carry the singular values
    np.testing.assert_allclose(A @ A.T, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(B, axis=0), sig, rtol=1e-12)


def test_lore_targets_are_expert_minus_shared():
    rng = np.random.default_rng(43)
    H, I, Is = 16, 8, 12
    wg, wu, wd = (rng.standard_normal(s) * 0.3 for s in ((I, H), (I, H), (H, I)))
    sg, su, sd = (rng.standard_normal(s) * 0.3 for s in ((1, Is, H), (1, Is, H), (1, H, Is)))
    h = rng.standard_normal((3, H))
    got = O.lore_targets(h, wg, wu, wd, sg, su, sd)
    for t in range(3):
        ye = sum(wd[:, i] * (h[t] @ wg[i]) / (1 + math.exp(-(h[t] @ wg[i]))) * (h[t] @ wu[i]) for i in range(I))
        ys = sum(sd[0][:, i] * (h[t] @ sg[0][i]) / (1 + math.exp(-(h[t] @ sg[0][i]))) * (h[t] @ su[0][i])
                 for i in range(Is))
        np.testing.assert_allclose(got[t], ye - ys, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- layer-level pins --
def _small_layer(name="tiny", **kw):
    cfg = W.CONFIGS[name]
    lay = W.make_layer(name, **kw)
    return lay


def _dims(cfg):
    return dict(hidden=cfg.hidden, n_experts=cfg.n_experts, top_k=cfg.top_k, inter=cfg.inter,
                n_shared=cfg.n_shared, shared_inter=cfg.shared_inter, lore_rank=cfg.lore_rank,
                renormalize=cfg.renormalize, shared_gate=cfg.shared_gate, dtype=cfg.dtype,
                up_format=cfg.up_format, floe_keep=cfg.floe_keep)


def _weights(lay):
    w = {n: lay.full(n) for n in lay.tensor_names()}
    w["w_router"] = lay.w_router()
    if lay.cfg.shared_gate:
        w["w_shared_gate"] = lay.w_shared_gate()
    return w


def test_all_resident_reduces_to_standard():
    lay = _small_layer(); cfg = lay.cfg; w = _weights(lay); x = lay.x()
    d = _dims(cfg)
    std = O.layer_forward(x, w, d, "standard")
    allres = (1 << cfg.n_experts) - 1
    lore = O.layer_forward(x, w, d, "lore", resident=allres)
    sf = O.layer_forward(x, w, d, "stall_free", resident=[allres] * x.shape[0])
    for r in (lore, sf):
        np.testing.assert_array_equal(r["ids"], std["ids"])
        np.testing.assert_array_equal(r["out"], std["out"])


def test_lore_zero_factors_give_shared_output_and_standard_when_experts_equal_shared():
    lay = _small_layer(); cfg = lay.cfg; w = _weights(lay); x = lay.x(); d = _dims(cfg)
    w["lore_A"] = np.zeros_like(w["lore_A"]); w["lore_B"] = np.zeros_like(w["lore_B"])
    r = O.layer_forward(x, w, d, "lore", resident=lay.resident())
    for t in range(x.shape[0]):
        for j in range(cfg.top_k):
            if not r["exact"][t, j]:
                np.testing.assert_array_equal(r["lore"][t, j], 0.0)
    # every routed expert equal to the single shared expert => LORE == STANDARD
    for n, sn in (("w_gate", "ws_gate"), ("w_up", "ws_up"), ("w_down", "ws_down")):
        w[n] = np.repeat(w[sn][:1], cfg.n_experts, axis=0)
    a = O.layer_forward(x, w, d, "lore", resident=lay.resident())
    b = O.layer_forward(x, w, d, "standard")
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    assert (a["exact"] == 0).any()


def test_batch_invariance():
    lay = _small_layer(); cfg = lay.cfg; w = _weights(lay); d = _dims(cfg)
    full = O.layer_forward(lay.x(), w, d, "lore", resident=lay.resident())
    for t in (0, 5, 15):
        one = O.layer_forward(lay.x()[t:t + 1], w, d, "lore", resident=lay.resident())
        np.testing.assert_allclose(one["out"][0], full["out"][t], rtol=1e-12, atol=1e-15)
        np.testing.assert_array_equal(one["ids"][0], full["ids"][t])


def test_expert_relabelling_equivariance():
    lay = _small_layer(); cfg = lay.cfg; w = _weights(lay); x = lay.x(); d = _dims(cfg)
    pi = np.random.default_rng(14).permutation(cfg.n_experts)     # new id j holds old expert pi[j]
    w2 = dict(w)
    w2["w_router"] = w["w_router"][pi]
    for n in ("w_gate", "w_up", "w_down", "lore_A", "lore_B"):
        w2[n] = w[n][pi]
    res = lay.resident()
    res2 = sum(1 << j for j in range(cfg.n_experts) if (res >> int(pi[j])) & 1)
    a = O.layer_forward(x, w, d, "lore", resident=res)
    b = O.layer_forward(x, w2, d, "lore", resident=res2)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(a["ids"], pi[b["ids"]])


def test_down_scaling_is_linear():
    lay = _small_layer(); cfg = lay.cfg; w = _weights(lay); x = lay.x(); d = _dims(cfg)
    a = O.layer_forward(x, w, d, "standard")
    w2 = dict(w); w2["w_down"] = w["w_down"] * 2; w2["ws_down"] = w["ws_down"] * 2
    b = O.layer_forward(x, w2, d, "standard")
    np.testing.assert_array_equal(b["out"], 2 * a["out"])


def test_shared_gate_closed_form():
    lay = _small_layer("tiny"); cfg = lay.cfg; w = _weights(lay); x = lay.x(); d = _dims(cfg)
    d2 = dict(d, shared_gate=True)
    w["w_shared_gate"] = np.zeros(cfg.hidden, dtype=np.float32)
    a = O.layer_forward(x, w, d2, "standard")     # sigma(0) = 1/2
    b = O.layer_forward(x, w, d, "standard")
    np.testing.assert_allclose(a["out"], b["out"] - 0.5 * b["y_shared"], rtol=1e-12, atol=1e-14)


def test_two_shared_experts_sum():
    lay = _small_layer("tiny"); cfg = lay.cfg; w = _weights(lay); x = lay.x(); d = _dims(cfg)
    w2 = dict(w)
    for n in ("ws_gate", "ws_up", "ws_down"):
        w2[n] = np.concatenate([w[n], w[n]], 0)
    d2 = dict(d, n_shared=2)
    a = O.layer_forward(x, w, d, "standard"); b = O.layer_forward(x, w2, d2, "standard")
    np.testing.assert_allclose(b["y_shared"], 2 * a["y_shared"], rtol=1e-12)


def _tiny_cfg(**kw):
    import dataclasses
    return dataclasses.replace(W.CONFIGS["tiny"], **kw)


def test_floe_layer_full_keep_equals_standard_on_decoded_up():
    """Layer level: FLOE with keep = I equals STANDARD run on the decoded INT2
    up weights and the [H][I] view of the channel-major down weights."""
    cfg = _tiny_cfg(name="tiny_floe", hidden=128, n_experts=4, top_k=2, inter=32, n_shared=0,
                    shared_inter=0, lore_rank=0, dtype="bf16", up_format="int2_g64",
                    floe_keep=32, renormalize=True, token_counts=(3,), modes=("floe",))
    lay = W.Layer(cfg, 21)
    w = _weights(lay); x = lay.x(); d = _dims(cfg)
    r = O.layer_forward(x, w, d, "floe")
    wd = dict(hidden=128, n_experts=4, top_k=2, inter=32, n_shared=0, shared_inter=0, lore_rank=0,
              renormalize=True, shared_gate=False, dtype="f32", up_format="dense", floe_keep=0)
    dense = {"w_router": O.bf16_to_f64(w["w_router"]), "w_gate": O.bf16_to_f64(w["w_gate"]),
             "w_up": O.dequant_int2(w["up_q"], w["up_scale"], w["up_zero"]),
             "w_down": np.transpose(O.bf16_to_f64(w["w_down"]), (0, 2, 1))}
    s = O.layer_forward(O.bf16_to_f64(x), dense, wd, "standard")
    np.testing.assert_array_equal(r["ids"], s["ids"])
    np.testing.assert_allclose(r["out"], s["out"], rtol=1e-12, atol=1e-14)


def test_stall_free_layer_uses_prefetch_masks():
    cfg = _tiny_cfg(name="tiny_sf", n_experts=8, top_k=2, n_shared=0, shared_inter=0, lore_rank=0,
                    renormalize=True, prefetch=True, modes=("standard", "stall_free"))
    lay = W.Layer(cfg, 22)
    w = _weights(lay); x = lay.x(); d = _dims(cfg)
    masks, pflags, lp = O.prefetch_masks(O.decode(x, "f32"), O.decode(lay.w_prefetch(), "f32"),
                                         np.zeros(x.shape[0], np.int32), cfg.top_k)
    r = O.layer_forward(x, w, d, "stall_free", resident=masks)
    l = r["logits"]
    for t in range(x.shape[0]):
        allowed = [e for e in range(8) if (masks[t] >> e) & 1]
        assert list(r["ids"][t]) == sorted(allowed, key=lambda e: (-l[t, e], e))[:2]
    assert r["n_subst"].sum() > 0


def test_workload_generator_shapes_and_determinism():
    for name, cfg in W.CONFIGS.items():
        lay = W.make_layer(name)
        assert lay.x().shape == (cfg.t_max, cfg.hidden)
        m = lay.resident()
        if cfg.resident_count:
            assert bin(m).count("1") == cfg.resident_count
        if cfg.prefetch:
            d = lay.delta()
            assert d.min() >= 0 and d.max() <= cfg.delta_cap
            assert abs(d.mean() - 1.5) < 0.15          # Geometric(0.4) on {0,1,...}: mean 1.5
    a = W.make_layer("tiny").expert("w_gate", 3); b = W.make_layer("tiny").expert("w_gate", 3)
    np.testing.assert_array_equal(a, b)
    assert W.make_layer("tiny").resident() == 0b1111
    # bf16 rounding is round-to-nearest-even
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20], dtype=np.float32)
    bits = W.bf16_bits_from_f32(v)
    np.testing.assert_array_equal(O.bf16_to_f64(bits), [1.0, 1.0, 1.0 + 4 * 2**-8, 1.0 + 2**-7])


# ------------------------------------------------- APEX adaptive budget --
def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_adaptive_budget_closed_forms():
    """delta_hat = min{d : sigmoid(theta_d - w.x) >= tau} [APEX Sec. 4.2], on
    scores whose value is exact: w = a e_0, x = b e_0, so w.x = a*b."""
    H = 8
    for a, b in [(0.5, 1.0), (-1.25, 2.0), (3.0, 0.75), (0.0, 5.0)]:
        w = np.zeros(H); w[0] = a
        x = np.zeros(H); x[0] = b
        s = a * b
        for tau in (0.6, 0.9, 0.97):
            lt = math.log(tau / (1 - tau))
            # constant theta: the first delta qualifies or none does (then N-k)
            for c in (-3.0, 0.0, 1.7, 6.0):
                th = [c] * 5
                d, _ = O.adaptive_budget(x, w, th, tau)
                assert d == (0 if _sig(c - s) >= tau else 4)
            # linear theta_d = a0 + g d: least integer d >= (s + logit(tau) - a0) / g
            for a0, g in [(-2.0, 0.5), (0.3, 1.1), (-5.0, 0.7)]:
                th = [a0 + g * d for d in range(33)]
                want = min(32, max(0, math.ceil((s + lt - a0) / g)))
                assert abs((s + lt - a0) / g - round((s + lt - a0) / g)) > 1e-6  # off a boundary
                d, _ = O.adaptive_budget(x, w, th, tau)
                assert d == want, (a, b, tau, a0, g)


def test_adaptive_budget_monotone():
    """A larger tau never lowers the budget; raising every threshold theta_d
    (more confidence at each budget) never raises it."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        H = 16
        x = rng.standard_normal(H)
        w = rng.standard_normal(H) / 4
        th = np.cumsum(rng.uniform(0, 1, 9)) - 3
        ds = [O.adaptive_budget(x, w, th, tau)[0] for tau in (0.5, 0.7, 0.9, 0.99)]
        assert ds == sorted(ds)
        assert O.adaptive_budget(x, w, th + 0.8, 0.9)[0] <= ds[2]


def test_overlap_full_exactly_when_budget_covers_delta_star():
    """The page's overlap is |K_r & K_p| / k; with the list top-(k + delta) it
    is complete exactly when delta >= delta* (the definition of delta*),
    checked on random tiny layers against a set intersection."""
    rng = np.random.default_rng(12)
    E, k, H = 9, 3, 12
    for _ in range(100):
        x = rng.standard_normal((4, H))
        wr = rng.standard_normal((E, H))
        wp = wr + rng.standard_normal((E, H)) * 0.7
        wd = rng.standard_normal(H) / 3
        th = np.cumsum(rng.uniform(0.2, 1.0, E - k + 1)) - 2
        routed = np.array([O.route_token(O.router_logits(x[t:t + 1], wr)[0], k, True, 1e-4)[0]
                           for t in range(4)])
        d_hat, masks, _, ds, ov = O.adaptive_prefetch(x, wp, wd, th, 0.9, k, routed=routed)
        lp = O.router_logits(x, wp)
        for t in range(4):
            order = sorted(range(E), key=lambda e: (-lp[t][e], e))
            kp = set(order[: k + int(d_hat[t])])
            assert masks[t] == _mask(kp)
            assert ov[t] == len(set(routed[t]) & kp)
            assert (ov[t] == k) == (d_hat[t] >= ds[t])


# ------------------------------------------- flag thresholds (bits 2, 8, 16) --
MARGIN = 1e-4


@pytest.mark.parametrize("gap,want", [(0.99e-4, True), (1.01e-4, False)])
def test_prefetch_edge_flag_sits_at_the_list_edge(gap, want):
    """Bit 2 is raised exactly when the list's last member and the first
    expert left out differ by less than the margin in prefetch logits; the
    same gap one place deeper or shallower in the ranking never raises it."""
    base = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0])
    n = 3
    lp = base.copy(); lp[3] = lp[2] - gap          # ranks n-1 and n
    m, f = O.prefetch_set(lp, n, MARGIN)
    assert m == 0b000111 and f is want
    lp = base.copy(); lp[4] = lp[3] - gap          # ranks n and n+1
    assert O.prefetch_set(lp, n, MARGIN) == (0b000111, False)
    lp = base.copy(); lp[2] = lp[1] - gap          # ranks n-2 and n-1
    assert O.prefetch_set(lp, n, MARGIN) == (0b000111, False)
    # through the per-token entry: x = [1] makes the logits the router column
    lp = base.copy(); lp[3] = lp[2] - gap
    masks, flags, _ = O.prefetch_masks(np.ones((1, 1)), lp[:, None], np.array([1]), 2, MARGIN)
    assert masks == [0b000111] and flags[0] == (O.FLAG_PREFETCH if want else 0)
    # a list of every expert has no edge
    assert O.prefetch_set(np.zeros(4), 4, MARGIN) == (0b1111, False)


def test_budget_flag_on_the_logit_scale_at_the_chosen_budget_and_the_one_below():
    """Bit 16: |theta_d - w.x - logit(tau)| below the margin at the chosen
    budget d or at d - 1; not at d + 1, and judged on the logit scale, not on
    the probability sigmoid(theta_d - w.x) (whose slope at tau = 0.9 is 0.09,
    so a logit gap of 5e-4 is a probability gap of 4.5e-5)."""
    tau = 0.9
    lt = math.log(tau / (1 - tau))
    w, x = np.array([0.75]), np.array([1.0])
    s = 0.75

    def budget(gaps):
        return O.adaptive_budget(x, w, [lt + s + g for g in gaps], tau, MARGIN)

    # the chosen budget (d = 1) sits just above the threshold
    assert budget([-1.0, 0.99e-4, 1.0]) == (1, True)
    assert budget([-1.0, 1.01e-4, 1.0]) == (1, False)
    # the budget below it (d - 1 = 0) sits just under the threshold
    assert budget([-0.99e-4, 1.0, 2.0]) == (1, True)
    assert budget([-1.01e-4, 1.0, 2.0]) == (1, False)
    # a near-threshold budget above the chosen one does not count
    assert budget([-1.0, 1.0, 0.5e-4]) == (1, False)
    # logit scale: a logit gap of 5e-4 is no near-tie although p moves by 4.5e-5
    d, f = budget([-1.0, 5e-4, 1.0])
    assert d == 1 and not f
    assert abs(O.sigmoid(lt + 5e-4) - tau) < MARGIN
    # no budget qualifies: N - k, flagged only if the last one is within the margin
    assert budget([-1.0, -2.0, -3.0]) == (2, False)
    assert budget([-1.0, -2.0, -0.5e-4]) == (2, True)


def _int2_group(q0, q1):
    """Codes of one 64-input group: input 0 -> q0, input 1 -> q1, the other
    62 inputs -> code 1 (weight 0 with zero point 1)."""
    b = np.full(16, 0b01010101, dtype=np.uint8)
    b[0] = q0 | (q1 << 2) | (1 << 4) | (1 << 6)
    return b


@pytest.mark.parametrize("eps,want", [(0.99e-4, True), (1.01e-4, False)])
def test_floe_mask_edge_flag_threshold(eps, want):
    """Bit 8: the n_keep-th and (n_keep+1)-th |u| differ by less than the
    margin.  Scale s = 1, zero z = 1 give weights q - 1 in {-1, 0, 1, 2};
    x = [1, eps, 0, ...] then gives u = [2, 1, -(1 - eps), 0]: |u| ranks
    channels 0, 1, 2, 3 and the gap at the edge of a 2-channel mask is eps."""
    one = np.float16(1.0).view(np.uint16)
    q = np.stack([_int2_group(3, 1), _int2_group(2, 1), _int2_group(0, 2), _int2_group(1, 1)])
    s = np.full((4, 1), one, dtype=np.uint16)
    z = np.full((4, 1), one, dtype=np.uint16)
    x = np.zeros(64); x[0] = 1.0; x[1] = eps
    keep, flag, u = O.floe_channel_mask(x, q, s, z, 2, MARGIN)
    np.testing.assert_allclose(u, [2.0, 1.0, -(1.0 - eps), 0.0], rtol=0, atol=1e-15)
    assert list(keep) == [0, 1] and flag is want
    # the same gap elsewhere in the ranking is no near-tie
    assert O.floe_channel_mask(x, q, s, z, 1, MARGIN)[1] is False
    assert O.floe_channel_mask(x, q, s, z, 3, MARGIN)[1] is False
    # the forward raises the same flag
    rng = np.random.default_rng(3)
    y, _, keep2, flag2 = O.floe_expert(x, rng.standard_normal((4, 64)), q, s, z,
                                       rng.standard_normal((4, 64)), 2, MARGIN)
    assert list(keep2) == [0, 1] and flag2 is want


# ----------------------------------------------- LoRE fit: exact least squares --
def _skewed_design(rng, N, H):
    """Correlated, unequally scaled inputs: far from an orthogonal design."""
    mix = rng.standard_normal((H, H)) * 0.3 + np.diag(np.linspace(0.5, 3.0, H))
    return rng.standard_normal((N, H)) @ mix


def test_lore_fit_full_rank_is_lstsq_on_a_non_orthogonal_design():
    rng = np.random.default_rng(44)
    N, H = 80, 24
    h = _skewed_design(rng, N, H)
    R = rng.standard_normal((N, H))
    A, B, sig, err = O.lore_fit(h, R, H)
    W_ls = np.linalg.lstsq(h, R, rcond=None)[0].T
    np.testing.assert_allclose(B @ A, W_ls, rtol=1e-8, atol=1e-10)
    want = np.linalg.norm(R - h @ W_ls.T) / np.linalg.norm(R)
    assert abs(err - want) < 1e-10


@pytest.mark.parametrize("r", [1, 3, 7])
def test_lore_fit_rank_r_matches_the_qr_route_and_is_optimal(r):
    """Rank-r least squares by a second route: with the thin QR h = Q_h R_h,
    ||R - h W^T|| = ||Q_h^T R - R_h W^T|| + const, so R_h W^T is the rank-r
    truncated SVD of C = Q_h^T R and W^T = R_h^-1 [C]_r.  Random rank-r
    perturbations of the result never lower the residual, and it beats the
    truncated SVD of the unwhitened map R^T h / N on this skewed design."""
    rng = np.random.default_rng(45 + r)
    N, H = 90, 20
    h = _skewed_design(rng, N, H)
    R = h @ rng.standard_normal((H, H)) * 0.2 + rng.standard_normal((N, H))
    A, B, sig, err = O.lore_fit(h, R, r)
    Qh, Rh = np.linalg.qr(h)
    Uc, Sc, Vct = np.linalg.svd(Qh.T @ R)
    Cr = (Uc[:, :r] * Sc[:r]) @ Vct[:r]
    W_qr = np.linalg.solve(Rh, Cr).T
    np.testing.assert_allclose(B @ A, W_qr, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(sig, Sc[:r] / math.sqrt(N), rtol=1e-10)
    loss = lambda W: np.linalg.norm(R - h @ W.T)
    base = loss(B @ A)
    for _ in range(20):
        dB = rng.standard_normal(B.shape) * 1e-3
        dA = rng.standard_normal(A.shape) * 1e-3
        assert loss((B + dB) @ (A + dA)) >= base - 1e-12
    U, S, Vt = np.linalg.svd(R.T @ h / N)
    naive = (U[:, :r] * S[:r]) @ Vt[:r]
    assert base < loss(naive)


# ------------------------------------- stall-free with a short prefetched set --
def test_stall_free_short_prefetched_set_literal_and_fill():
    """Fewer than k prefetched experts: Algorithm 1's sets give back the whole
    prefetched set (every prefetched expert is kept or substitutes), and the
    fill takes the best remaining experts by the original router's score."""
    l = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0])
    # routed {0, 1, 2}, prefetched {4, 5}: keep {}, missing {0, 1, 2}, subs {4, 5}
    S, _ = O.stall_free_select([0, 1, 2], l, {4, 5}, MARGIN)
    assert S == {4, 5}
    full, f = O.stall_free_fill(S, l, 3, MARGIN)
    assert full == {0, 4, 5} and not f
    # prefetched {1}: keep {1}; fill 0 and 2
    S, _ = O.stall_free_select([0, 1, 2], l, {1}, MARGIN)
    assert S == {1} and O.stall_free_fill(S, l, 3, MARGIN) == ({0, 1, 2}, False)
    # a near-tie between the last filled expert and the next one is flagged
    l2 = np.array([5.0, 4.0, 3.0, 3.0 - 0.5e-4, 1.0])
    assert O.stall_free_fill({4}, l2, 3, MARGIN) == ({0, 1, 4}, False)
    assert O.stall_free_fill({4}, l2, 4, MARGIN)[1] is True
    # a full set is returned unchanged
    assert O.stall_free_fill({1, 2, 3}, l, 3, MARGIN) == ({1, 2, 3}, False)


def test_stall_free_short_sets_brute_force_through_the_layer():
    """On random tiny layers and prefetched sets of every size: the layer's
    final set is the prefetched set plus the best outside it when the set is
    short (flag 32), else Algorithm 1's set; slots ordered by (-logit, id)."""
    rng = np.random.default_rng(46)
    H, I = 8, 4
    for trial in range(60):
        E = int(rng.integers(3, 9)); k = int(rng.integers(1, E + 1))
        w = {"w_router": rng.standard_normal((E, H)).astype(np.float32),
             "w_gate": rng.standard_normal((E, I, H)).astype(np.float32),
             "w_up": rng.standard_normal((E, I, H)).astype(np.float32),
             "w_down": rng.standard_normal((E, H, I)).astype(np.float32)}
        dims = dict(hidden=H, n_experts=E, top_k=k, inter=I, n_shared=0, shared_inter=0,
                    lore_rank=0, renormalize=True, shared_gate=False, dtype="f32",
                    up_format="dense", floe_keep=0)
        x = rng.standard_normal((3, H)).astype(np.float32)
        masks = [_mask(rng.permutation(E)[: int(rng.integers(0, E + 1))].tolist()) for _ in range(3)]
        r = O.layer_forward(x, w, dims, "stall_free", resident=masks)
        l = O.router_logits(x.astype(np.float64), w["w_router"].astype(np.float64))
        for t in range(3):
            kp = [e for e in range(E) if (masks[t] >> e) & 1]
            order = O.rank_experts(l[t])
            if len(kp) < k:
                want = set(kp) | set([e for e in order if e not in kp][: k - len(kp)])
                assert r["flags"][t] & O.FLAG_SHORT
            else:
                want = set(sorted(kp, key=lambda e: (-l[t][e], e))[:k])
                assert not r["flags"][t] & O.FLAG_SHORT
            assert set(r["ids"][t]) == want
            assert list(r["ids"][t]) == [e for e in order if e in want]


# ---- SPICE cost rule for missed experts ------------------------------------
# SPICE page, "CPU-GPU collaboration: handling prefetch misses": fetch when
# W_e / B_pcie + T_gpu_e is below T_cpu_e + 2H / B_pcie.

def test_offload_rule_hand_worked_boundary():
    # H = 64, I = 16, bf16: W_e = 3 * 16 * 64 * 2 = 6144 bytes, each pair moves
    # 2 * 64 * 2 = 256 bytes.  With no compute time on either side the rule
    # compares 6144 with 256 n: equal at n = 24 (not strictly cheaper: host),
    # fetch from n = 25.  A dropped factor 2 would move the edge to 48 and a
    # W_e of two matrices to 16.
    d = {"dtype": "bf16", "inter": 16, "hidden": 64}
    dec = O.offload_plan(d, [23, 24, 25, 48, 49], 0, 1.0e9, 0.0, 0.0)
    assert dec == [O.OFFLOAD_HOST, O.OFFLOAD_HOST, O.OFFLOAD_FETCH, O.OFFLOAD_FETCH,
                   O.OFFLOAD_FETCH]
    f, h = O.offload_costs(6144, 128, 24, 1.0e9, 0.0, 0.0)
    assert f == h == 6144 / 1.0e9


def test_offload_rule_compute_terms():
    # W_e / B = 4 s (4e9 bytes at 1e9 B/s), T_gpu = 0.5 s, host 1.5 s per pair
    # and negligible transfers: fetch 4.5 s against 1.5 n s -> host for n <= 3
    # (n = 3 ties at 4.5 s: host), fetch for n >= 4.
    d = {"dtype": "f32", "inter": 1, "hidden": 1}
    for n, want in ((1, O.OFFLOAD_HOST), (3, O.OFFLOAD_HOST), (4, O.OFFLOAD_FETCH)):
        f, h = O.offload_costs(4.0e9, 0.0, n, 1.0e9, 0.5, 1.5)
        assert f == 4.5 and h == 1.5 * n
        assert (O.OFFLOAD_FETCH if f < h else O.OFFLOAD_HOST) == want
    # through the plan: W_e there is 3 * 1 * 1 * 4 = 12 bytes, so fetching is
    # cheap unless the GPU time dominates
    assert O.offload_plan(d, [1], 0, 12.0, 2.0, 2.5) == [O.OFFLOAD_FETCH]   # 3.0 < 2.5 + 8/12
    assert O.offload_plan(d, [1], 0, 12.0, 2.5, 2.5) == [O.OFFLOAD_HOST]    # 3.5 > 3.1667


def test_offload_rule_fixed_host_term():
    # a fixed host time per expert (its weight reads) counts once, not per
    # pair: fetch 1.05 s against 0.6 + 0.1 n s (+ 8n bytes over the link) ->
    # host up to n = 4, fetch at n = 5.  Counted per pair (0.7 n s) it would
    # fetch from n = 2.
    d = {"dtype": "f32", "inter": 1, "hidden": 1}
    B = 12.0e9                                    # W_e = 12 bytes: 1 ns to fetch
    dec = O.offload_plan(d, [1, 3, 4, 5], 0, B, 1.05 - 1e-9, 0.1, cpu_expert_s=0.6)
    assert dec == [O.OFFLOAD_HOST, O.OFFLOAD_HOST, O.OFFLOAD_HOST, O.OFFLOAD_FETCH]
    f, h = O.offload_costs(12, 4, 4, B, 0.5, 0.1, 0.6)
    assert abs(h - (0.6 + 0.4 + 32 / B)) < 1e-15 and f == 12 / B + 0.5


def test_offload_rule_resident_and_unrouted_need_nothing():
    d = {"dtype": "bf16", "inter": 1408, "hidden": 2048}
    dec = O.offload_plan(d, [0, 5, 5, 0], 0b0010, 50e9, 1e-5, 1e-3)
    assert dec[0] == O.OFFLOAD_NONE and dec[1] == O.OFFLOAD_NONE and dec[3] == O.OFFLOAD_NONE
    assert dec[2] in (O.OFFLOAD_FETCH, O.OFFLOAD_HOST)


def test_offload_rule_switches_once_with_more_pairs():
    # the host cost grows with the expert's pairs, the fetch cost does not: as
    # pairs increase the decision can only move from host to fetch
    rng = np.random.default_rng(11)
    d = {"dtype": "bf16", "inter": 1408, "hidden": 2048}
    for _ in range(200):
        B = 10 ** rng.uniform(9, 11)
        g = 10 ** rng.uniform(-6, -3)
        c = 10 ** rng.uniform(-6, -2)
        dec = O.offload_plan(d, list(range(1, 65)), 0, B, g, c)
        first = next((i for i, v in enumerate(dec) if v == O.OFFLOAD_FETCH), len(dec))
        assert all(v == O.OFFLOAD_HOST for v in dec[:first])
        assert all(v == O.OFFLOAD_FETCH for v in dec[first:])


def test_offload_queue_aware_balances_link_and_host():
    # f32, H = I = 1000: W_e = 12e6 bytes at 12e6 B/s = 1 s per fetch; host
    # 0.9 s per pair plus 8e3 / 12e6 s of transfers per pair.  On its own
    # every single-pair expert goes to the host (0.9007 < 1); as queues:
    # e0 host (0.9007), e1 fetch (1 < 1.8013), e2 host (1.8013 < 2),
    # e3 fetch (2 < 2.702).
    d = {"dtype": "f32", "inter": 1000, "hidden": 1000}
    args = (0, 12e6, 0.0, 0.9)
    assert O.offload_plan(d, [1, 1, 1, 1], *args) == [O.OFFLOAD_HOST] * 4
    assert O.offload_plan(d, [1, 1, 1, 1], *args, queue_aware=True) == \
        [O.OFFLOAD_HOST, O.OFFLOAD_FETCH, O.OFFLOAD_HOST, O.OFFLOAD_FETCH]
    # order by decreasing pairs, then id: e1 (3 pairs: 2.7 s host) fetches,
    # e3 (2 pairs) then faces 2 s of fetches against 1.8013 s on the host,
    # e0 faces 2 s against 1.8013 + 0.9007, e2 then 3 s against 2.702
    assert O.offload_plan(d, [1, 3, 1, 2], *args, queue_aware=True) == \
        [O.OFFLOAD_FETCH, O.OFFLOAD_FETCH, O.OFFLOAD_HOST, O.OFFLOAD_HOST]
