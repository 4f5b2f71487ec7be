"""Pins of the CPU oracle to facts other than itself.

Each test pins one part of the layer against a hand-derived closed form, a
brute-force property, an invariant of the definition or an IEEE/NumPy library
routine, chosen so that a plausible slip (dropped term, wrong sign, transposed
operand, wrong tie rule, missing renormalization) fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs as mi
import oracle
from _layers import load_hand_fixture, oracle_layer_from_arrays, oracle_layer_from_config

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _random_arrays(rng, H, E, K, I, Is, rstd=0.05, estd=0.05):
    return dict(H=H, E=E, K=K, I=I, Is=Is,
                router_w=(rng.standard_normal((E, H)) * rstd).astype(np.float32),
                gate_vec=(rng.standard_normal(H) * rstd).astype(np.float32), router_bias=None,
                exp_gate=(rng.standard_normal((E, I, H)) * estd).astype(np.float32),
                exp_up=(rng.standard_normal((E, I, H)) * estd).astype(np.float32),
                exp_down=(rng.standard_normal((E, H, I)) * estd).astype(np.float32),
                sh_gate=(rng.standard_normal((Is, H)) * estd).astype(np.float32),
                sh_up=(rng.standard_normal((Is, H)) * estd).astype(np.float32),
                sh_down=(rng.standard_normal((H, Is)) * estd).astype(np.float32))


# ---------------------------------------------------------------- golden

def test_hand_fixture_closed_forms():
    a, exp = load_hand_fixture()
    L = oracle_layer_from_arrays(a)
    ids, wts, gate, y, y64 = L.forward(a["x"])
    np.testing.assert_array_equal(ids[0], exp["ids"])          # tie at the boundary: lower id kept
    np.testing.assert_allclose(wts[0], exp["wts"], rtol=0, atol=1e-15)
    assert abs(gate[0] - exp["gate"]) < 1e-15
    np.testing.assert_allclose(y64[0], exp["y"], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(y[0], exp["y"].astype(np.float32))


# ------------------------------------------------------------- selection

def test_selection_one_hot_permutation():
    """One-hot router rows through a random permutation: l_e = x[pi(e)] exactly."""
    rng = np.random.default_rng(1)
    H, E, K = 64, 64, 6
    pi = rng.permutation(H)
    a = _random_arrays(rng, H, E, K, 32, 32)
    a["router_w"] = np.zeros((E, H), np.float32)
    a["router_w"][np.arange(E), pi] = 1.0
    x = np.zeros((1, H), np.float32)
    x[0, pi] = (E - np.arange(E)) / E          # expert e gets logit (E-e)/E
    ids, wts, gate, logits = oracle_layer_from_arrays(a).route(x)
    np.testing.assert_array_equal(ids[0], np.arange(K))
    vals = np.array([(E - e) / E for e in range(K)], np.float32).astype(np.float64)
    ref = np.exp(vals - vals[0]) / np.exp(vals - vals[0]).sum()
    np.testing.assert_allclose(wts[0], ref, rtol=1e-14)
    np.testing.assert_array_equal(logits[0], x[0, pi].astype(np.float64))


@pytest.mark.parametrize("seed", range(20))
def test_selection_brute_force_properties(seed):
    """Integer logits with many exact ties; the selection must be the unique
    sequence ordered by (logit desc, id asc) that beats every unselected expert."""
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(2, 12))
    K = int(rng.integers(1, E + 1))
    H = 32
    a = _random_arrays(rng, H, E, K, 32, 32)
    vals = rng.integers(-3, 4, size=E).astype(np.float32)     # lots of ties
    a["router_w"] = np.zeros((E, H), np.float32)
    a["router_w"][:, 0] = vals
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    ids, wts, _, logits = oracle_layer_from_arrays(a).route(x)
    sel = list(ids[0])
    assert len(set(sel)) == K
    l = logits[0]

    def before(p, q):
        return l[p] > l[q] or (l[p] == l[q] and p < q)

    for i in range(K - 1):
        assert before(sel[i], sel[i + 1])
    for p in sel:
        for q in set(range(E)) - set(sel):
            assert before(p, q)
    # exhaustive: no other K-subset has a larger logit sum (ties broken by ids)
    import itertools
    best = max(itertools.combinations(range(E), K), key=lambda c: (sum(l[list(c)]), [-i for i in sorted(c)]))
    assert sorted(best) == sorted(sel)
    assert abs(wts[0].sum() - 1.0) < 1e-15


def test_selection_duplicate_rows_tie():
    """Two identical router rows give bit-equal logits; the lower id wins at the
    K boundary."""
    rng = np.random.default_rng(7)
    H, E, K = 128, 32, 5
    a = _random_arrays(rng, H, E, K, 32, 32)
    x = rng.standard_normal((1, H)).astype(np.float32)
    ids, _, _, _ = oracle_layer_from_arrays(a).route(x)
    sel = list(ids[0])
    for _ in range(100):                 # find a K-th expert with an unselected higher id
        lo = sel[K - 1]
        cands = [e for e in range(lo + 1, E) if e not in sel]
        if cands:
            break
        x = rng.standard_normal((1, H)).astype(np.float32)
        sel = list(oracle_layer_from_arrays(a).route(x)[0][0])
    hi = cands[0]
    a["router_w"][hi] = a["router_w"][lo]
    ids2, _, _, logits = oracle_layer_from_arrays(a).route(x)
    assert logits[0, lo] == logits[0, hi]
    np.testing.assert_array_equal(ids2[0], sel)          # hi ties with lo and loses
    # swap roles: give the lower id the copy and keep the higher one -> lower wins again
    b = dict(a)
    b["router_w"] = a["router_w"].copy()
    ids3, _, _, _ = oracle_layer_from_arrays(b).route(x)
    assert hi not in ids3[0]


def test_selection_all_experts():
    rng = np.random.default_rng(3)
    a = _random_arrays(rng, 64, 8, 8, 32, 32)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    ids, wts, _, logits = oracle_layer_from_arrays(a).route(x)
    for t in range(3):
        assert sorted(ids[t]) == list(range(8))
        assert np.all(np.diff(logits[t][ids[t]]) <= 0)
        assert abs(wts[t].sum() - 1) < 1e-14


def test_weights_ln2_and_k1():
    rng = np.random.default_rng(4)
    a = _random_arrays(rng, 32, 4, 2, 32, 32)
    a["router_w"] = np.zeros((4, 32), np.float32)
    a["router_w"][0, 0] = np.float32(math.log(2.0))
    a["router_w"][1, 0] = 0.0
    a["router_w"][2, 0] = -5.0
    a["router_w"][3, 0] = -6.0
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    ids, wts, _, _ = oracle_layer_from_arrays(a).route(x)
    np.testing.assert_array_equal(ids[0], [0, 1])
    np.testing.assert_allclose(wts[0], [2 / 3, 1 / 3], atol=1e-8)
    a["K"] = 1
    ids, wts, _, _ = oracle_layer_from_arrays(a).route(x)
    assert ids[0, 0] == 0 and wts[0, 0] == 1.0


def test_weights_not_renormalized_variant():
    """Without renormalization the weights are the full softmax entries."""
    rng = np.random.default_rng(5)
    a = _random_arrays(rng, 64, 16, 4, 32, 32)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    ids, wts, _, logits = oracle_layer_from_arrays(a, renormalize=0).route(x)
    for t in range(2):
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(wts[t], p[ids[t]], rtol=1e-13)
        assert wts[t].sum() < 1.0


def test_zero_input_and_bias_routing():
    """x = 0: every logit is the bias; with no bias all tie, ids = 0..K-1,
    weights exactly 1/K, gate exactly 1/2 and y exactly 0."""
    rng = np.random.default_rng(6)
    a = _random_arrays(rng, 64, 16, 4, 32, 32)
    x = np.zeros((1, 64), np.float32)
    ids, wts, gate, y, y64 = oracle_layer_from_arrays(a).forward(x)
    np.testing.assert_array_equal(ids[0], [0, 1, 2, 3])
    assert np.all(wts[0] == 0.25) and gate[0] == 0.5
    assert np.all(y64 == 0)
    a["router_bias"] = np.array([0, 5, -1, 3, 3, 7] + [0] * 10, np.float32)
    ids, wts, gate, _, _ = oracle_layer_from_arrays(a).forward(x)
    np.testing.assert_array_equal(ids[0], [5, 1, 3, 4])      # 3 and 4 tie: lower first


def test_shared_gate_closed_forms():
    rng = np.random.default_rng(8)
    a = _random_arrays(rng, 32, 4, 2, 32, 32)
    x = rng.standard_normal((1, 32)).astype(np.float32)
    a["gate_vec"] = np.zeros(32, np.float32)
    _, _, gate, _ = oracle_layer_from_arrays(a).route(x)
    assert gate[0] == 0.5
    a["gate_vec"][0] = 1.0
    x[0, 0] = np.float32(math.log(3.0))
    _, _, gate, _ = oracle_layer_from_arrays(a).route(x)
    assert abs(gate[0] - 0.75) < 1e-7                         # sigmoid(ln 3) = 3/4


# ------------------------------------------------------------ expert FFN

def _numpy_swiglu(G, U, D, x):
    """Dense SwiGLU MLP with NumPy float64 matrix products (library routine)."""
    G, U, D, x = (np.asarray(v, np.float64) for v in (G, U, D, x))
    a = G @ x
    c = U @ x
    return D @ ((a / (1.0 + np.exp(-a))) * c)


def test_single_expert_reduces_to_dense_swiglu():
    """E = K = 1 with a zero shared expert is one dense SwiGLU MLP (w = 1)."""
    rng = np.random.default_rng(9)
    H, I = 96, 64                                   # non-square: a transposed operand fails
    a = _random_arrays(rng, H, 1, 1, I, 32, estd=0.1)
    a["sh_down"][:] = 0
    x = rng.standard_normal((4, H)).astype(np.float32)
    ids, wts, _, y, y64 = oracle_layer_from_arrays(a).forward(x)
    for t in range(4):
        ref = _numpy_swiglu(a["exp_gate"][0], a["exp_up"][0], a["exp_down"][0], x[t])
        np.testing.assert_allclose(y64[t], ref, rtol=1e-12, atol=1e-14)
        assert wts[t, 0] == 1.0


def test_gate_preactivation_zero_kills_channel():
    rng = np.random.default_rng(10)
    a = _random_arrays(rng, 64, 2, 1, 32, 32)
    a["exp_gate"][:] = 0
    a["sh_gate"][:] = 0
    x = rng.standard_normal((2, 64)).astype(np.float32)
    _, _, _, _, y64 = oracle_layer_from_arrays(a).forward(x)
    assert np.all(y64 == 0)


def test_down_scaling_is_exact():
    rng = np.random.default_rng(11)
    a = _random_arrays(rng, 64, 8, 3, 32, 32)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    y1 = oracle_layer_from_arrays(a).forward(x)[4]
    a["exp_down"] = a["exp_down"] * 2
    a["sh_down"] = a["sh_down"] * 2
    y2 = oracle_layer_from_arrays(a).forward(x)[4]
    np.testing.assert_array_equal(y2, 2 * y1)


def test_identical_experts_make_routing_irrelevant():
    """All routed experts equal: y = FFN(x) * sum(w) + g * S(x) = FFN(x) + g * S(x)."""
    rng = np.random.default_rng(12)
    H, E, K, I, Is = 64, 16, 4, 32, 64
    a = _random_arrays(rng, H, E, K, I, Is, estd=0.1)
    for m in ("exp_gate", "exp_up", "exp_down"):
        a[m][:] = a[m][0]
    x = rng.standard_normal((5, H)).astype(np.float32)
    ids, wts, gate, y, y64 = oracle_layer_from_arrays(a).forward(x)
    for t in range(5):
        ref = (_numpy_swiglu(a["exp_gate"][0], a["exp_up"][0], a["exp_down"][0], x[t])
               + gate[t] * _numpy_swiglu(a["sh_gate"], a["sh_up"], a["sh_down"], x[t]))
        np.testing.assert_allclose(y64[t], ref, rtol=1e-12, atol=1e-13)


def test_zero_routed_down_leaves_gated_shared_expert():
    rng = np.random.default_rng(13)
    H = 64
    a = _random_arrays(rng, H, 8, 2, 32, 96, estd=0.1)
    a["exp_down"][:] = 0
    x = rng.standard_normal((3, H)).astype(np.float32)
    _, _, gate, _, y64 = oracle_layer_from_arrays(a).forward(x)
    z = x.astype(np.float64) @ a["gate_vec"].astype(np.float64)
    np.testing.assert_allclose(gate, 1 / (1 + np.exp(-z)), rtol=1e-14)
    for t in range(3):
        ref = gate[t] * _numpy_swiglu(a["sh_gate"], a["sh_up"], a["sh_down"], x[t])
        np.testing.assert_allclose(y64[t], ref, rtol=1e-12, atol=1e-14)


def test_tiny_workload_against_numpy_layer():
    """The tiny fp32 workload against an independent NumPy float64 layer
    (library matmuls, lexsort selection)."""
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    g, u, d = mi.expert_stacks(cfg)
    L = oracle_layer_from_config(cfg, dense=dense, stacks=(g, u, d))
    x = mi.activations(cfg, T=8)
    ids, wts, gate, y, y64 = L.forward(x)
    W = dense["router_w"].astype(np.float64)
    for t in range(8):
        xt = x[t].astype(np.float64)
        l = W @ xt
        order = np.lexsort((np.arange(cfg.E), -l))[: cfg.K]
        np.testing.assert_array_equal(ids[t], order)
        p = np.exp(l[order] - l[order].max())
        p /= p.sum()
        np.testing.assert_allclose(wts[t], p, rtol=1e-13)
        gt = 1 / (1 + np.exp(-(dense["gate_vec"].astype(np.float64) @ xt)))
        ref = sum(p[k] * _numpy_swiglu(g[order[k]], u[order[k]], d[order[k]], xt) for k in range(cfg.K))
        ref = ref + gt * _numpy_swiglu(dense["sh_gate"], dense["sh_up"], dense["sh_down"], xt)
        np.testing.assert_allclose(y64[t], ref, rtol=1e-11, atol=1e-14)


def test_bf16_widening_is_exact():
    """bf16 weights are widened exactly: a bf16 layer equals the fp32 layer
    holding the same values."""
    rng = np.random.default_rng(14)
    a = _random_arrays(rng, 64, 8, 2, 32, 32)
    b = dict(a)
    for k in ("router_w", "gate_vec", "exp_gate", "exp_up", "exp_down", "sh_gate", "sh_up", "sh_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
        a[k] = mi.bf16_bits_to_f32(b[k]).reshape(a[k].shape)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    ra = oracle_layer_from_arrays(a).forward(x)
    rb = oracle_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16").forward(x)
    for u, v in zip(ra, rb):
        np.testing.assert_array_equal(u, v)


def test_thread_count_does_not_change_results():
    cfg = mi.CONFIGS[0]
    L = oracle_layer_from_config(cfg)
    x = mi.activations(cfg, T=6)
    oracle.set_threads(1)
    r1 = L.forward(x)
    oracle.set_threads(4)
    r4 = L.forward(x)
    for u, v in zip(r1, r4):
        np.testing.assert_array_equal(u, v)


# ------------------------------------------------------------ fp16 / q2

def test_half_to_float_all_patterns():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(h) for h in range(65536)], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_float_to_half_matches_ieee_rne():
    rng = np.random.default_rng(15)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 0.05,
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),              # subnormal range
        rng.uniform(-70000, 70000, 2000).astype(np.float32),
        np.array([65504, 65519.996, 65520, 65536, 6.1035156e-05, 5.96e-08, 2.98e-08, 2.9802322e-08,
                  0.0, -0.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25], np.float32),
    ])
    # exact half-way cases between adjacent fp16 values
    h = rng.integers(0, 0x7bff, 3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, ((lo + hi) / 2).astype(np.float32)])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_q2_bit_layout_fixture():
    """Codes 0,1,2,3 repeated pack to 0xE4 bytes; scale 2^-6 -> 0x2400,
    min -2^-5 -> 0xA800 (hand-derived fp16 encodings)."""
    codes = np.tile(np.arange(4), 8)
    w = (codes * 2.0 ** -6 - 2.0 ** -5).astype(np.float32).reshape(1, 32)
    q = oracle.q2_quantize(w)
    assert list(q.codes[0]) == [0xE4] * 8
    assert q.scale[0, 0] == 0x2400 and q.minv[0, 0] == 0xA800
    np.testing.assert_array_equal(oracle.q2_dequantize(q), w)


def test_q2_exact_round_trip_dyadic_blocks():
    rng = np.random.default_rng(16)
    rows, cols = 16, 256
    codes = rng.integers(0, 4, (rows, cols))
    codes[:, ::32] = 0
    codes[:, 1::32] = 3                               # every block spans the full code range
    s = 2.0 ** rng.integers(-12, -3, (rows, cols // 32))
    m = rng.integers(-64, 64, (rows, cols // 32)) * 2.0 ** -10
    w = (codes * np.repeat(s, 32, axis=1) + np.repeat(m, 32, axis=1)).astype(np.float32)
    q = oracle.q2_quantize(w)
    np.testing.assert_array_equal(oracle.q2_dequantize(q), w)
    unpacked = np.stack([(q.codes >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(rows, cols)
    np.testing.assert_array_equal(unpacked, codes)


def test_q2_constant_block():
    """A constant block that fp16 represents exactly has scale 0, codes 0 and
    decodes exactly; a constant that fp16 cannot represent decodes to one
    constant value no farther from it than fp16 rounding."""
    w = np.full((2, 64), 0.01220703125, np.float32)     # 25 * 2^-11: exact in fp16
    w[1] = -3.5
    q = oracle.q2_quantize(w)
    assert np.all(q.scale == 0) and np.all(q.codes == 0)
    np.testing.assert_array_equal(oracle.q2_dequantize(q), w)
    w = np.full((1, 32), 0.0123, np.float32)
    wq = oracle.q2_dequantize(oracle.q2_quantize(w))
    assert np.all(wq == wq[0, 0])
    assert abs(float(wq[0, 0]) - 0.0123) <= abs(float(np.float16(0.0123)) - float(np.float32(0.0123)))


def test_q2_error_bound_random_blocks():
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    q = oracle.q2_quantize(w)
    wq = oracle.q2_dequantize(q).astype(np.float64)
    sf = np.repeat(q.scale.view(np.float16).astype(np.float64), 32, axis=1)
    mf = np.repeat(q.minv.view(np.float16).astype(np.float64), 32, axis=1)
    lo = np.repeat(w.reshape(64, 16, 32).min(axis=2).astype(np.float64), 32, axis=1)
    bound = 0.5 * np.abs(sf) + np.abs(lo - mf) + 0.002 * np.abs(sf) + 1e-9
    assert np.all(np.abs(w - wq) <= bound)
    codes = np.stack([(q.codes >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(64, 512)
    assert codes.min() == 0 and codes.max() == 3


def test_q2_rejects_non_finite():
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = np.inf
    with pytest.raises(ValueError):
        oracle.q2_quantize(w)


def test_q2_layer_equals_dequantized_fp32_layer():
    """A 2-bit layer is the fp32 layer holding the dequantized weights."""
    rng = np.random.default_rng(18)
    a = _random_arrays(rng, 64, 6, 2, 32, 32)
    qa = dict(a)
    qa["exp_gate"] = [oracle.q2_quantize(m) for m in a["exp_gate"]]
    qa["exp_up"] = [oracle.q2_quantize(m) for m in a["exp_up"]]
    qa["exp_down"] = [oracle.q2_quantize(m) for m in a["exp_down"]]
    fa = dict(a)
    fa["exp_gate"] = np.stack([oracle.q2_dequantize(q) for q in qa["exp_gate"]])
    fa["exp_up"] = np.stack([oracle.q2_dequantize(q) for q in qa["exp_up"]])
    fa["exp_down"] = np.stack([oracle.q2_dequantize(q) for q in qa["exp_down"]])
    x = rng.standard_normal((3, 64)).astype(np.float32)
    rq = oracle_layer_from_arrays(qa, expert_t="q2").forward(x)
    rf = oracle_layer_from_arrays(fa).forward(x)
    for u, v in zip(rq, rf):
        np.testing.assert_array_equal(u, v)


# ------------------------------------------- selection-only router bias

def test_hand_fixture_bias_selection_only():
    """hand_bias_select_only.json: a bias that ties two experts at the top;
    bias_mode 1 weighs them by their unbiased logits, bias_mode 0 by the
    biased (equal) ones."""
    a, exp = load_hand_fixture("hand_bias_select_only.json")
    for mode, e in ((1, exp), (0, exp["bias_mode_0"])):
        L = oracle_layer_from_arrays(dict(a, bias_mode=mode))
        ids, wts, gate, y, y64 = L.forward(a["x"])
        np.testing.assert_array_equal(ids[0], e["ids"])
        np.testing.assert_allclose(wts[0], e["wts"], rtol=0, atol=1e-15)
        assert abs(gate[0] - e["gate"]) < 1e-15
        np.testing.assert_allclose(y64[0], e["y"], rtol=1e-14, atol=1e-15)


def test_bias_selection_only_invariants():
    """bias 0: both modes equal the unbiased layer; a bias equal for every
    expert: the same selection and (mode 1) the same weights as no bias; any
    bias: both modes select the same experts, and mode 1's weights are the
    softmax of the unbiased logits of that selection."""
    rng = np.random.default_rng(77)
    a = _random_arrays(rng, 96, 40, 6, 32, 32, rstd=0.1)
    x = rng.standard_normal((12, 96)).astype(np.float32)
    plain = oracle_layer_from_arrays(a).forward(x)
    for mode in (0, 1):
        r = oracle_layer_from_arrays(dict(a, router_bias=np.zeros(40, np.float32), bias_mode=mode)).forward(x)
        for u, v in zip(plain, r):
            np.testing.assert_array_equal(u, v)
    const = oracle_layer_from_arrays(dict(a, router_bias=np.full(40, 0.75, np.float32), bias_mode=1)).forward(x)
    np.testing.assert_array_equal(const[0], plain[0])
    np.testing.assert_allclose(const[1], plain[1], rtol=0, atol=1e-15)
    b = rng.standard_normal(40).astype(np.float32)
    m0 = oracle_layer_from_arrays(dict(a, router_bias=b, bias_mode=0))
    m1 = oracle_layer_from_arrays(dict(a, router_bias=b, bias_mode=1))
    i0, w0, _, _ = m0.route(x)
    i1, w1, _, sel = m1.route(x)
    np.testing.assert_array_equal(i0, i1)
    assert not np.array_equal(i1, plain[0])                         # the bias changed some selections
    unb = sel - b.astype(np.float64)[None, :]                       # unbiased logits of every expert
    for t in range(x.shape[0]):
        v = unb[t, i1[t]]
        ref = np.exp(v - v.max()) / np.exp(v - v.max()).sum()
        np.testing.assert_allclose(w1[t], ref, rtol=1e-12, atol=1e-15)
        v0 = sel[t, i0[t]]
        np.testing.assert_allclose(w0[t], np.exp(v0 - v0.max()) / np.exp(v0 - v0.max()).sum(), rtol=1e-12)


# ------------------------------------------------ RMS norm and residual

def test_hand_fixture_norm_and_residual():
    """hand_norm_residual.json: mean(x^2) = 4 and eps = 12 make r = 1/4
    exactly; a missing sqrt, mean or eps changes every value."""
    a, exp = load_hand_fixture("hand_norm_residual.json")
    u = oracle.rmsnorm(a["x"], a["norm_w"], a["norm_eps"])
    ref_u = np.zeros(32, np.float32)
    ref_u[:8] = 1.0
    ref_u[0], ref_u[1] = 0.25, 0.5
    np.testing.assert_array_equal(u[0], ref_u)
    L = oracle_layer_from_arrays(a)
    ids, wts, gate, y, y64 = L.forward(a["x"])
    np.testing.assert_array_equal(ids[0], exp["ids"])
    np.testing.assert_allclose(wts[0], exp["wts"], rtol=0, atol=1e-15)
    assert abs(gate[0] - exp["gate"]) < 1e-15
    np.testing.assert_allclose(y64[0], exp["y"], rtol=1e-14, atol=1e-15)


def test_rmsnorm_properties():
    """Scaling x by a power of two leaves u unchanged (eps = 0); with gamma = 1
    and eps = 0 the mean square of u is 1; eps enters under the root (a row
    with mean square m and eps gives u = x / sqrt(m + eps)); an all-zero row
    with eps > 0 gives zeros."""
    rng = np.random.default_rng(8)
    H = 256
    x = rng.standard_normal((5, H)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, H).astype(np.float32)
    u = oracle.rmsnorm(x, g, 0.0)
    np.testing.assert_array_equal(oracle.rmsnorm(x * np.float32(8.0), g, 0.0), u)
    one = oracle.rmsnorm(x, np.ones(H, np.float32), 0.0).astype(np.float64)
    np.testing.assert_allclose((one ** 2).mean(axis=1), 1.0, rtol=1e-6)
    xc = np.full((1, H), 3.0, np.float32)                      # mean square 9, eps 7: r = 1/4
    np.testing.assert_array_equal(oracle.rmsnorm(xc, np.ones(H, np.float32), 7.0), np.full((1, H), 0.75, np.float32))
    np.testing.assert_array_equal(oracle.rmsnorm(np.zeros((1, H), np.float32), g, 1e-6), np.zeros((1, H), np.float32))


def test_norm_of_unit_rows_and_residual():
    """gamma = 1, eps = 0 and rows of +-1 (mean square 1): the norm is the
    identity, so the layer with norm and residual equals x plus the plain
    layer, to the rounding of the final sum; zero down matrices leave y = x
    exactly."""
    rng = np.random.default_rng(9)
    H = 128
    a = _random_arrays(rng, H, 24, 4, 64, 32)
    x = np.where(rng.random((6, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    plain = oracle_layer_from_arrays(a).forward(x)
    nr = oracle_layer_from_arrays(dict(a, norm_w=np.ones(H, np.float32), norm_eps=0.0, residual=1)).forward(x)
    np.testing.assert_array_equal(nr[0], plain[0])
    np.testing.assert_array_equal(nr[1], plain[1])
    np.testing.assert_allclose(nr[4], plain[4] + x.astype(np.float64), rtol=0, atol=1e-13)
    z = dict(a, exp_down=np.zeros_like(a["exp_down"]), sh_down=np.zeros_like(a["sh_down"]),
             norm_w=rng.uniform(0.5, 2.0, H).astype(np.float32), residual=1)
    xr = rng.standard_normal((6, H)).astype(np.float32)
    np.testing.assert_array_equal(oracle_layer_from_arrays(z).forward(xr)[3], xr)


# ------------------------------------------------------ b-bit quantizer

def _quant_cases():
    with open(os.path.join(os.path.dirname(__file__), "golden", "hand_quant_blocks.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _quant_cases(), ids=lambda c: c["name"])
def test_hand_fixture_quant_blocks(case):
    """hand_quant_blocks.json: ties to even, a block whose fp16 min lies above
    its maximum (negative step), and the 3- and 4-bit bit layouts."""
    w = np.array(case["w"], np.float32).reshape(1, 32)
    q = oracle.qb_quantize(w, case["bits"])
    assert list(q.codes[0]) == case["codes"]
    assert int(q.scale[0, 0]) == case["scale"] and int(q.minv[0, 0]) == case["min"]
    np.testing.assert_array_equal(oracle.qb_dequantize(q)[0], np.array(case["decoded"], np.float32))


def _unpack_codes(q):
    """Codes of a b-bit matrix read bit by bit (weight j of a block at bits b*j..)."""
    bits = q.bits
    nb = q.cols // 32
    raw = q.codes.reshape(q.rows, nb, 4 * bits)
    allbits = np.unpackbits(raw, axis=-1, bitorder="little").reshape(q.rows, nb, 32, bits)
    return (allbits * (1 << np.arange(bits))).sum(axis=-1).reshape(q.rows, q.cols)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_qb_exact_round_trip_dyadic_blocks(bits):
    rng = np.random.default_rng(40 + bits)
    rows, cols, top = 16, 256, (1 << bits) - 1
    codes = rng.integers(0, top + 1, (rows, cols))
    codes[:, ::32] = 0
    codes[:, 1::32] = top                               # every block spans the full code range
    s = 2.0 ** rng.integers(-12, -3, (rows, cols // 32))
    m = rng.integers(-64, 64, (rows, cols // 32)) * 2.0 ** -10
    w = (codes * np.repeat(s, 32, axis=1) + np.repeat(m, 32, axis=1)).astype(np.float32)
    q = oracle.qb_quantize(w, bits)
    assert q.codes.shape == (rows, cols * bits // 8)
    np.testing.assert_array_equal(oracle.qb_dequantize(q), w)
    np.testing.assert_array_equal(_unpack_codes(q), codes)


@pytest.mark.parametrize("bits", [3, 4])
def test_qb_error_bound_random_blocks(bits):
    """Each decoded weight lies within half a step of its input, plus the
    min's fp16 rounding and the step's; more bits give a smaller error."""
    rng = np.random.default_rng(50 + bits)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    q = oracle.qb_quantize(w, bits)
    wq = oracle.qb_dequantize(q).astype(np.float64)
    top = (1 << bits) - 1
    sf = np.repeat(q.scale.view(np.float16).astype(np.float64), 32, axis=1)
    mf = np.repeat(q.minv.view(np.float16).astype(np.float64), 32, axis=1)
    lo = np.repeat(w.reshape(64, 16, 32).min(axis=2).astype(np.float64), 32, axis=1)
    bound = 0.5 * np.abs(sf) + np.abs(lo - mf) + top * 0.001 * np.abs(sf) + 1e-9
    assert np.all(np.abs(w - wq) <= bound)
    c = _unpack_codes(q)
    assert c.min() == 0 and c.max() == top
    e_lo = np.abs(w - oracle.qb_dequantize(oracle.qb_quantize(w, bits - 1))).mean()
    assert np.abs(w - wq).mean() < 0.75 * e_lo


@pytest.mark.parametrize("wt", ["q3", "q4"])
def test_qb_layer_equals_dequantized_fp32_layer(wt):
    """A b-bit layer is the fp32 layer holding the dequantized weights."""
    bits = oracle.BITS[wt]
    rng = np.random.default_rng(60 + bits)
    a = _random_arrays(rng, 64, 6, 2, 32, 32)
    qa, fa = dict(a), dict(a)
    for k in ("exp_gate", "exp_up", "exp_down"):
        qa[k] = [oracle.qb_quantize(m, bits) for m in a[k]]
        fa[k] = np.stack([oracle.qb_dequantize(q) for q in qa[k]])
    x = rng.standard_normal((3, 64)).astype(np.float32)
    rq = oracle_layer_from_arrays(qa, expert_t=wt).forward(x)
    rf = oracle_layer_from_arrays(fa).forward(x)
    for u, v in zip(rq, rf):
        np.testing.assert_array_equal(u, v)
