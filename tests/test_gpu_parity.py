"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: router ids bit-identical (ordered), wts / gate / y within
|gpu - oracle| <= 1e-4 + 2e-3 |oracle| elementwise, 2-bit unpack bit-exact,
grouping (counting sort) bit-exact. Full-size workloads run in the same
launch configuration the benchmark times (back-to-back calls on one stream);
routing is checked on every row, y on every row the oracle finishes quickly.
"""
import os
import sys

import numpy as np
import pytest

import moe_inputs as mi
from _layers import (assert_parity, gpu_layer_from_arrays, gpu_layer_from_config, load_hand_fixture,
                     oracle_layer_from_arrays, oracle_layer_from_config, run_calls, tolerance_ok)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_decode_amd as moe
    moe.lib()   # fails loudly if the library is not built


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_ref(L, x):
    ids, wts, gate, y, y64 = L.forward(x)
    return ids, wts, gate, y64


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


# ------------------------------------------------------------- small cases

def test_hand_fixture():
    _say("case: hand fixture H=32 E=4 K=2")
    a, exp = load_hand_fixture()
    G = gpu_layer_from_arrays(a)
    ids, wts, gate, y = run_calls(G, a["x"], 1)
    np.testing.assert_array_equal(ids[0], exp["ids"])
    assert tolerance_ok(wts[0], exp["wts"]).all()
    assert tolerance_ok(gate[0], exp["gate"]).all()
    assert tolerance_ok(y[0], exp["y"]).all(), (y[0][:4], exp["y"][:4])


@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 6, 7, 8])
def test_tiny_fp32_workload(rows):
    _say(f"case: tiny fp32 workload, {rows} rows per call")
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    stacks = mi.expert_stacks(cfg)
    G = gpu_layer_from_config(cfg, dense, stacks)
    L = oracle_layer_from_config(cfg, dense=dense, stacks=stacks)
    x = mi.activations(cfg, T=64 + rows - 1)
    got = run_calls(G, x, rows)
    assert_parity(got, _oracle_ref(L, x), f"tiny rows={rows}")


def test_route_only_entry_point():
    _say("case: moe_route on the tiny workload")
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    G = gpu_layer_from_config(cfg, dense, mi.expert_stacks(cfg))
    L = oracle_layer_from_config(cfg, dense=dense, experts=[])
    x = mi.activations(cfg, T=37)
    ids, wts, gate = G.route(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ri, rw, rg, _ = L.route(x)
    np.testing.assert_array_equal(ids.cpu().numpy(), ri)
    assert tolerance_ok(wts.cpu().numpy(), rw).all()
    assert tolerance_ok(gate.cpu().numpy(), rg).all()


@pytest.mark.parametrize("layout", ["pairs64", "twins512"])
def test_duplicate_router_rows_tie_on_gpu(layout):
    """Bit-equal logits from duplicated router rows: the lower id must win
    on the GPU exactly as in the oracle, at every boundary position."""
    _say(f"case: exact-tie fixture {layout}")
    rng = np.random.default_rng(31)
    if layout == "pairs64":
        H, E, K = 256, 64, 6
        a = _random_arrays(rng, H, E, K, 64, 64)
        # pairs of identical rows across the whole expert range
        for lo, hi in [(1, 40), (5, 6), (10, 63), (20, 21), (33, 50)]:
            a["router_w"][hi] = a["router_w"][lo]
    else:
        # every logit has a twin 256 ids away: with K odd the K-th and the
        # (K+1)-th are always equal
        H, E, K = 128, 512, 5
        a = _random_arrays(rng, H, E, K, 32, 32)
        a["router_w"][256:] = a["router_w"][:256]
    x = rng.standard_normal((200, H)).astype(np.float32)
    L = oracle_layer_from_arrays(a)
    ri, _, _, logits = L.route(x)
    G = gpu_layer_from_arrays(a)
    ref = _oracle_ref(L, x)
    for rows in (1, 2, 3, 4, 200):   # decode, few-row calls and one prefill call
        got = run_calls(G, x, rows)
        np.testing.assert_array_equal(got[0], ri)
        assert_parity(got, ref, f"tie fixture rows={rows}")


@pytest.mark.parametrize("case", ["k_equals_e", "single_expert", "no_renorm", "bias", "zero_x", "zero_x_many", "wide"])
def test_edge_shapes(case):
    _say(f"case: edge {case}")
    rng = np.random.default_rng(hash(case) % 2 ** 32)
    renorm = 1
    if case == "k_equals_e":
        a = _random_arrays(rng, 64, 8, 8, 32, 32)
    elif case == "single_expert":
        a = _random_arrays(rng, 96, 1, 1, 64, 32)
    elif case == "no_renorm":
        a = _random_arrays(rng, 128, 32, 5, 64, 96)
        renorm = 0
    elif case == "bias":
        a = _random_arrays(rng, 128, 48, 7, 32, 64)
        a["router_bias"] = rng.standard_normal(48).astype(np.float32)
    elif case == "zero_x":
        a = _random_arrays(rng, 64, 16, 4, 32, 32)
    elif case == "zero_x_many":   # 512 equal logits: more candidates than a wave holds
        a = _random_arrays(rng, 64, 512, 10, 32, 32)
    else:   # wide: K = 16, E = 1024, odd intermediate sizes
        a = _random_arrays(rng, 256, 1024, 16, 96, 160, rstd=0.1)
    T = 9
    x = rng.standard_normal((T, a["H"])).astype(np.float32)
    if case.startswith("zero_x"):
        x[:] = 0
    L = oracle_layer_from_arrays(a, renormalize=renorm)
    G = gpu_layer_from_arrays(a, renormalize=renorm)
    ref = _oracle_ref(L, x)
    for rows in (1, 3, 4, 6, 8, T):   # decode, few-row launches of 3 and 4 rows, calls of 6, 8 and 9 rows
        assert_parity(run_calls(G, x, rows), ref, f"{case} rows={rows}")
    assert_parity(run_calls(G, x, T, force_path="prefill"), ref, f"{case} prefill")


def test_bf16_and_q2_small_shapes():
    """bf16 router/shared with bf16 and 2-bit experts at small, ragged sizes."""
    rng = np.random.default_rng(41)
    a = _random_arrays(rng, 320, 24, 5, 96, 64, rstd=0.05, estd=0.05)
    b = dict(a)
    for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    x = rng.standard_normal((11, 320)).astype(np.float32)
    _say("case: small bf16 experts")
    L = oracle_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    G = gpu_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    ref = _oracle_ref(L, x)
    for rows in (1, 2, 4, 11):
        assert_parity(run_calls(G, x, rows), ref, f"bf16 rows={rows}")
    assert_parity(run_calls(G, x, 11, force_path="prefill"), ref, "bf16 prefill")
    _say("case: small 2-bit experts")
    import oracle
    q = dict(b)
    q["exp_gate"] = [oracle.q2_quantize(m) for m in a["exp_gate"]]
    q["exp_up"] = [oracle.q2_quantize(m) for m in a["exp_up"]]
    q["exp_down"] = [oracle.q2_quantize(m) for m in a["exp_down"]]
    Lq = oracle_layer_from_arrays(q, router_t="bf16", expert_t="q2", shared_t="bf16")
    Gq = gpu_layer_from_arrays(dict(b, exp_gate=a["exp_gate"], exp_up=a["exp_up"], exp_down=a["exp_down"]),
                               router_t="bf16", expert_t="q2", shared_t="bf16")
    ref = _oracle_ref(Lq, x)
    for rows in (1, 3, 11):
        assert_parity(run_calls(Gq, x, rows), ref, f"q2 rows={rows}")
    assert_parity(run_calls(Gq, x, 11, force_path="prefill"), ref, "q2 prefill")


@pytest.mark.parametrize("fmt", ["q3", "q4"])
def test_block_formats_small_shapes(fmt):
    """3- and 4-bit experts on a small layer (H 320: ten blocks per row, a
    ragged last set of lanes): decode, few-row calls of 2, 3, 5 and 11 rows
    and the prefill path, with fp32 and bf16 shared experts."""
    import oracle
    bits = oracle.BITS[fmt]
    rng = np.random.default_rng(300 + bits)
    a = _random_arrays(rng, 320, 24, 5, 96, 64, rstd=0.05, estd=0.05)
    x = rng.standard_normal((11, 320)).astype(np.float32)
    for dense_t in ("f32", "bf16"):
        _say(f"case: small {fmt} experts, {dense_t} router and shared expert")
        b = dict(a)
        if dense_t == "bf16":
            for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down"):
                b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
        q = dict(b)
        for k in ("exp_gate", "exp_up", "exp_down"):
            q[k] = [oracle.qb_quantize(m, bits) for m in a[k]]
        L = oracle_layer_from_arrays(q, router_t=dense_t, expert_t=fmt, shared_t=dense_t)
        G = gpu_layer_from_arrays(b, router_t=dense_t, expert_t=fmt, shared_t=dense_t)
        ref = _oracle_ref(L, x)
        for rows in (1, 2, 3, 5, 11):
            assert_parity(run_calls(G, x, rows), ref, f"{fmt} {dense_t} rows={rows}")
        assert_parity(run_calls(G, x, 11, force_path="prefill"), ref, f"{fmt} {dense_t} prefill")


def test_path_boundaries():
    """Calls at the edges of the library's path choice on a 2-bit layer:
    5, 8 and 12 rows run as few-row launches of three (remainders of two,
    two and none), 13 rows as one prefill chunk; 13 rows forced through
    few-row launches (a remainder of one joining the last launch as four)
    must agree as well."""
    _say("case: path boundaries (5, 12, 13 rows)")
    import oracle
    rng = np.random.default_rng(43)
    a = _random_arrays(rng, 256, 32, 6, 128, 64, rstd=0.05, estd=0.05)
    b = dict(a)
    for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    q = dict(b)
    for k in ("exp_gate", "exp_up", "exp_down"):
        q[k] = [oracle.q2_quantize(m) for m in a[k]]
    L = oracle_layer_from_arrays(q, router_t="bf16", expert_t="q2", shared_t="bf16")
    G = gpu_layer_from_arrays(dict(b, exp_gate=a["exp_gate"], exp_up=a["exp_up"], exp_down=a["exp_down"]),
                              router_t="bf16", expert_t="q2", shared_t="bf16")
    x = rng.standard_normal((60, 256)).astype(np.float32)
    ref = _oracle_ref(L, x)
    for rows in (5, 8, 12, 13):
        assert_parity(run_calls(G, x, rows), ref, f"boundary rows={rows}")
    assert_parity(run_calls(G, x, 13, force_path="fewrow"), ref, "boundary rows=13 few-row")


@pytest.mark.parametrize("fmt", ["bf16", "q2", "q3", "q4"])
def test_wide_rows_and_large_pair_sets(fmt):
    """Rows wider than one chunk set per wave (H = 2112: the streamed gate/up
    path) and, at four rows with K = 16, more (slot, row) pairs than the down
    pass stages in LDS (h' read from L2); eight rows as launches of three,
    three and two."""
    _say(f"case: wide rows {fmt} H=2112 E=16 K=16 I=544 Is=96")
    rng = np.random.default_rng(77)
    a = _random_arrays(rng, 2112, 16, 16, 544, 96, rstd=0.05, estd=0.03)
    b = dict(a)
    for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    x = rng.standard_normal((8, 2112)).astype(np.float32)
    if fmt == "bf16":
        L = oracle_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
        G = gpu_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    else:
        import oracle
        ef = {k: [mi.bf16_bits_to_f32(m) for m in b[k]] for k in ("exp_gate", "exp_up", "exp_down")}
        q = dict(b)
        for k in ef:
            q[k] = [oracle.qb_quantize(m, oracle.BITS[fmt]) for m in ef[k]]
        L = oracle_layer_from_arrays(q, router_t="bf16", expert_t=fmt, shared_t="bf16")
        G = gpu_layer_from_arrays(dict(b, **{k: np.stack(v) for k, v in ef.items()}),
                                  router_t="bf16", expert_t=fmt, shared_t="bf16")
    ref = _oracle_ref(L, x)
    for rows in (1, 4, 8):
        assert_parity(run_calls(G, x, rows), ref, f"wide {fmt} rows={rows}")


def test_maximum_sizes():
    """The largest H, I and Is the ABI accepts (8192, 4096, 4096) with bf16
    weights: the streamed gate/up rows, the unstaged down pass (four rows) and
    the prefill GEMMs at their largest reduction depths."""
    H, E, K, I, Is = 8192, 4, 2, 4096, 4096
    _say(f"case: maximum sizes H={H} I={I} Is={Is} E={E} K={K}")
    rng = np.random.default_rng(4096)
    a = _random_arrays(rng, H, E, K, I, Is, rstd=0.02, estd=0.01)
    b = dict(a)
    for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    del a
    x = rng.standard_normal((7, H)).astype(np.float32)
    L = oracle_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    G = gpu_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    ref = _oracle_ref(L, x)
    for rows, path in ((1, None), (4, None), (7, "prefill")):   # decode, few-row (h' read from L2), prefill
        err = assert_parity(run_calls(G, x, rows, force_path=path), ref, f"maximum sizes rows={rows}")
        _say(f"rows={rows}: max abs err {err[0]:.3g}, max err/tolerance {err[1]:.3g}")


@pytest.mark.parametrize("mode", [0, 1])
def test_cache_aware_routing_bias(mode):
    """The opt-in cache-aware routing variant: logits z + lambda * Delta *
    cached_e (Research notes page, section 4, the cache-aware routing row),
    given as the per-expert router bias with MOE_BIAS_SELECT_ONLY (the bias
    picks the experts, the weights come from the unbiased logits), and the
    same bias in the selection and the weights (mode 0). Parity with the
    oracle's variant on decode, few-row and prefill calls; the bias moves
    selections toward the cached experts; both modes select the same experts."""
    _say(f"case: cache-aware routing bias, bias_mode {mode}")
    rng = np.random.default_rng(2412)
    a = _random_arrays(rng, 256, 64, 6, 64, 64, rstd=0.1)
    cached = (rng.random(64) < 0.25).astype(np.float32)
    x = rng.standard_normal((24, 256)).astype(np.float32)
    base = _oracle_ref(oracle_layer_from_arrays(a), x)
    hits0 = cached[base[0]].sum()
    for lam_delta in (0.25, 1.0):
        b = dict(a, router_bias=(lam_delta * cached).astype(np.float32), bias_mode=mode)
        L = oracle_layer_from_arrays(b)
        G = gpu_layer_from_arrays(b)
        ref = _oracle_ref(L, x)
        other = _oracle_ref(oracle_layer_from_arrays(dict(b, bias_mode=1 - mode)), x)
        np.testing.assert_array_equal(ref[0], other[0])
        for rows in (1, 3, 24):
            assert_parity(run_calls(G, x, rows), ref, f"cache bias {lam_delta} mode {mode} rows={rows}")
        assert_parity(run_calls(G, x, 24, force_path="prefill"), ref, f"cache bias {lam_delta} mode {mode} prefill")
        hits = cached[ref[0]].sum()
        assert hits >= hits0, (lam_delta, hits, hits0)
        hits0 = hits
    assert hits0 > cached[base[0]].sum()


@pytest.mark.parametrize("name", ["hand_bias_select_only.json", "hand_norm_residual.json"])
def test_hand_fixtures_bias_norm_residual(name):
    """The hand-derived fixtures of the selection-only bias and of the norm
    with the residual, on the decode and the prefill path."""
    _say(f"case: hand fixture {name}")
    a, exp = load_hand_fixture(name)
    G = gpu_layer_from_arrays(a)
    for path in (None, "prefill"):
        ids, wts, gate, y = run_calls(G, a["x"], 1, force_path=path)
        np.testing.assert_array_equal(ids[0], exp["ids"])
        assert tolerance_ok(wts[0], exp["wts"]).all()
        assert tolerance_ok(gate[0], exp["gate"]).all()
        assert tolerance_ok(y[0], exp["y"]).all(), (path, y[0][:8], exp["y"][:8])


@pytest.mark.parametrize("fmt", ["f32", "bf16", "q2", "q4"])
def test_norm_and_residual_layers(fmt):
    """Layers with the pre-MoE RMS norm (random gamma) and the residual, with
    a selection-only bias, on decode, few-row (3 and 12 rows) and prefill
    calls, against the oracle."""
    _say(f"case: norm + residual layer, {fmt} experts")
    import oracle
    rng = np.random.default_rng(4242)
    H, E, K, I, Is = 256, 48, 6, 96, 64
    a = _random_arrays(rng, H, E, K, I, Is, rstd=0.05, estd=0.05)
    a.update(norm_w=rng.uniform(0.5, 1.5, H).astype(np.float32), norm_eps=1e-6, residual=1,
             router_bias=(0.5 * (rng.random(E) < 0.3)).astype(np.float32), bias_mode=1)
    x = (rng.standard_normal((37, H)) * 3.0).astype(np.float32)
    rt = st = "f32" if fmt == "f32" else "bf16"
    b = dict(a)
    if fmt != "f32":
        for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
            b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    if fmt in oracle.BITS:
        src = {k: mi.bf16_bits_to_f32(b[k]).reshape(a[k].shape) for k in ("exp_gate", "exp_up", "exp_down")}
        qo = dict(b)
        for k in src:
            qo[k] = [oracle.qb_quantize(m, oracle.BITS[fmt]) for m in src[k]]
        L = oracle_layer_from_arrays(qo, router_t=rt, expert_t=fmt, shared_t=st)
        G = gpu_layer_from_arrays(dict(b, **src), router_t=rt, expert_t=fmt, shared_t=st)
    else:
        L = oracle_layer_from_arrays(b, router_t=rt, expert_t=fmt, shared_t=st)
        G = gpu_layer_from_arrays(b, router_t=rt, expert_t=fmt, shared_t=st)
    ref = _oracle_ref(L, x)
    for rows in (1, 3, 12):
        assert_parity(run_calls(G, x, rows), ref, f"norm {fmt} rows={rows}")
    assert_parity(run_calls(G, x, 37), ref, f"norm {fmt} prefill")
    ids, wts, gate = G.route(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref[0])


def test_given_routing_entry():
    """moe_forward with ids_in/wts_in/gate_in uses the routing as given."""
    _say("case: caller-supplied routing")
    rng = np.random.default_rng(51)
    a = _random_arrays(rng, 128, 16, 3, 64, 64)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    L = oracle_layer_from_arrays(a)
    ri, rw, rg, y, y64 = L.forward(x)
    G = gpu_layer_from_arrays(a)
    import sparse_moe_decode_amd as moe
    xt = torch.from_numpy(x).cuda()
    ids = torch.from_numpy(ri).cuda()
    wts = torch.from_numpy(rw.astype(np.float32)).cuda()
    gate = torch.from_numpy(rg.astype(np.float32)).cuda()
    for rows in (1, 2, 4):
        out = torch.empty((4, 128), dtype=torch.float32, device="cuda")
        ws = G.workspace(rows)
        for t in range(0, 4, rows):
            moe.forward(G.desc, xt[t:t + rows], out[t:t + rows], ws, ids_in=ids[t:t + rows],
                        wts_in=wts[t:t + rows], gate_in=gate[t:t + rows])
        torch.cuda.synchronize()
        assert tolerance_ok(out.cpu().numpy(), y64).all()


def test_given_routing_with_ids_outside_range():
    """Given ids outside [0, E) contribute nothing: each row's second choice
    is replaced by -1 or E; the reference is the oracle on the layer whose
    dropped expert has a zero down matrix (same routing, that expert adding
    zero), row by row. Decode, few-row and prefill calls."""
    _say("case: caller-supplied routing with ids outside [0, E)")
    rng = np.random.default_rng(53)
    a = _random_arrays(rng, 128, 16, 3, 64, 64)
    T = 6
    x = rng.standard_normal((T, 128)).astype(np.float32)
    ri, rw, rg, _, _ = oracle_layer_from_arrays(a).forward(x)
    ref = np.zeros((T, 128))
    for t in range(T):
        b = dict(a, exp_down=a["exp_down"].copy())
        b["exp_down"][ri[t, 1]] = 0.0
        ref[t] = oracle_layer_from_arrays(b).forward(x[t:t + 1])[4][0]
    ids = ri.copy()
    ids[:, 1] = np.where(np.arange(T) % 2 == 0, -1, 16)
    G = gpu_layer_from_arrays(a)
    import sparse_moe_decode_amd as moe
    xt = torch.from_numpy(x).cuda()
    for rows, path in ((1, None), (2, None), (3, None), (6, "prefill")):
        out = torch.empty((T, 128), dtype=torch.float32, device="cuda")
        old = os.environ.get("MOE_FORCE_PATH")
        if path:
            os.environ["MOE_FORCE_PATH"] = path
        try:
            ws = G.workspace(rows)   # sized for the forced path
            for t in range(0, T, rows):
                moe.forward(G.desc, xt[t:t + rows], out[t:t + rows], ws,
                            ids_in=torch.from_numpy(ids[t:t + rows].copy()).cuda(),
                            wts_in=torch.from_numpy(rw[t:t + rows].astype(np.float32)).cuda(),
                            gate_in=torch.from_numpy(rg[t:t + rows].astype(np.float32)).cuda())
            torch.cuda.synchronize()
        finally:
            if path:
                if old is None:
                    os.environ.pop("MOE_FORCE_PATH", None)
                else:
                    os.environ["MOE_FORCE_PATH"] = old
        assert tolerance_ok(out.cpu().numpy(), ref).all(), rows


# --------------------------------------------------------- graph capture

@pytest.mark.parametrize("rows", [1, 3, 300])   # decode, few-row, prefill
def test_graph_replay_matches_eager(rows):
    """Calls captured into a HIP graph (as bench.py runs them) give the eager
    results bit for bit on every replay, with other eager work on the same
    layer and synchronizations between the replays."""
    _say(f"case: graph replay rows={rows}")
    import torch
    import sparse_moe_decode_amd as moe
    rng = np.random.default_rng(77 + rows)
    a = _random_arrays(rng, 256, 32, 4, 96, 64, rstd=0.05)
    a["router_bias"] = rng.standard_normal(32).astype(np.float32) * 0.5
    G = gpu_layer_from_arrays(a)
    T = 600 if rows == 300 else 12
    x = torch.from_numpy(rng.standard_normal((T, 256)).astype(np.float32)).cuda()
    other = torch.from_numpy(rng.standard_normal((T, 256)).astype(np.float32)).cuda()
    ws = G.workspace(rows)

    def run(src, y, ids):
        for t in range(0, T, rows):
            moe.forward(G.desc, src[t:t + rows], y[t:t + rows], ws, ids_out=ids[t:t + rows])

    y_eager = torch.empty((T, 256), dtype=torch.float32, device="cuda")
    ids_eager = torch.empty((T, 4), dtype=torch.int32, device="cuda")
    run(x, y_eager, ids_eager)
    torch.cuda.synchronize()
    y_g = torch.full((T, 256), float("nan"), dtype=torch.float32, device="cuda")
    ids_g = torch.full((T, 4), -1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(x, y_g, ids_g)
    torch.cuda.synchronize()
    y_o = torch.empty_like(y_eager)
    ids_o = torch.empty_like(ids_eager)
    for rep in range(3):
        y_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids_g.cpu().numpy(), ids_eager.cpu().numpy())
        np.testing.assert_array_equal(y_g.cpu().numpy().view(np.uint32), y_eager.cpu().numpy().view(np.uint32))
        run(other, y_o, ids_o)   # eager work between the replays
        torch.cuda.synchronize()


def test_two_streams_two_workspaces():
    """Calls on two streams with two workspaces are independent: prefill and
    decode calls interleaved on two streams (no ordering between them) both
    match the oracle."""
    _say("case: two streams, two workspaces (prefill and decode interleaved)")
    import sparse_moe_decode_amd as moe
    rng = np.random.default_rng(303)
    a = _random_arrays(rng, 256, 32, 4, 96, 64, rstd=0.05)
    a["router_bias"] = rng.standard_normal(32).astype(np.float32) * 0.5
    G = gpu_layer_from_arrays(a)
    L = oracle_layer_from_arrays(a)
    xs = [rng.standard_normal((300, 256)).astype(np.float32) for _ in range(2)]
    refs = [_oracle_ref(L, x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for i in range(2):
        T = 300
        outs.append(dict(x=torch.from_numpy(xs[i]).cuda(), y=torch.empty((T, 256), device="cuda"),
                         yd=torch.empty((T, 256), device="cuda"),
                         ids=torch.empty((T, 4), dtype=torch.int32, device="cuda"),
                         wts=torch.empty((T, 4), device="cuda"), gate=torch.empty((T,), device="cuda"),
                         ws=G.workspace(300), wsd=G.workspace(1)))
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            o = outs[i]
            moe.forward(G.desc, o["x"], o["y"], o["ws"], ids_out=o["ids"], wts_out=o["wts"], gate_out=o["gate"],
                        stream=streams[i])
        for t in range(0, 40):   # decode calls on both streams, alternating
            for i in range(2):
                o = outs[i]
                moe.forward(G.desc, o["x"][t:t + 1], o["yd"][t:t + 1], o["wsd"], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        o = outs[i]
        got = (o["ids"].cpu().numpy(), o["wts"].cpu().numpy(), o["gate"].cpu().numpy(), o["y"].cpu().numpy())
        assert_parity(got, refs[i], f"stream {i} prefill")
        yd = o["yd"].cpu().numpy()[:40]
        assert tolerance_ok(yd, refs[i][3][:40]).all(), f"stream {i} decode"


def test_prefill_in_chunks():
    """A prefill call longer than the chunk runs as consecutive chunks on one
    workspace (MOE_PREFILL_CHUNK lowers the chunk here): 600 rows as 256,
    256 and 88, against the oracle, for moe_forward and moe_route."""
    _say("case: prefill in chunks of 256 rows (600 rows)")
    rng = np.random.default_rng(606)
    a = _random_arrays(rng, 256, 32, 4, 96, 64, rstd=0.05)
    a["router_bias"] = rng.standard_normal(32).astype(np.float32) * 0.5
    G = gpu_layer_from_arrays(a)
    L = oracle_layer_from_arrays(a)
    x = rng.standard_normal((600, 256)).astype(np.float32)
    ref = _oracle_ref(L, x)
    old = os.environ.get("MOE_PREFILL_CHUNK")
    os.environ["MOE_PREFILL_CHUNK"] = "256"
    try:
        assert G.workspace(600).numel() < G.workspace(300).numel() + 16
        assert_parity(run_calls(G, x, 600), ref, "prefill chunks")
        ids, wts, gate = G.route(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy(), ref[0])
        assert tolerance_ok(wts.cpu().numpy(), ref[1]).all()
    finally:
        if old is None:
            os.environ.pop("MOE_PREFILL_CHUNK", None)
        else:
            os.environ["MOE_PREFILL_CHUNK"] = old


# ------------------------------------------------------------- prefill

@pytest.mark.parametrize("fmt", ["f32", "bf16", "q2", "q3", "q4"])
@pytest.mark.parametrize("T", [5, 37, 300])
def test_prefill_small(fmt, T):
    """Grouped-GEMM path at small sizes: ragged expert groups (not multiples
    of the 64-row tile), intermediate 96 (not a multiple of the 64-channel
    block), all weight formats."""
    _say(f"case: prefill {fmt} T={T}")
    import oracle
    rng = np.random.default_rng(1000 + T)
    a = _random_arrays(rng, 256, 16, 4, 96, 64, rstd=0.05, estd=0.05)
    a["router_bias"] = rng.standard_normal(16).astype(np.float32) * 0.5
    x = rng.standard_normal((T, 256)).astype(np.float32)
    rt = st = "f32" if fmt == "f32" else "bf16"
    b = dict(a)
    if fmt != "f32":
        for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
            b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    if fmt in oracle.BITS:
        src = {k: mi.bf16_bits_to_f32(b[k]).reshape(a[k].shape) for k in ("exp_gate", "exp_up", "exp_down")}
        qo = dict(b)
        for k in src:
            qo[k] = [oracle.qb_quantize(m, oracle.BITS[fmt]) for m in src[k]]
        L = oracle_layer_from_arrays(qo, router_t=rt, expert_t=fmt, shared_t=st)
        G = gpu_layer_from_arrays(dict(b, **src), router_t=rt, expert_t=fmt, shared_t=st)
    else:
        L = oracle_layer_from_arrays(b, router_t=rt, expert_t=fmt, shared_t=st)
        G = gpu_layer_from_arrays(b, router_t=rt, expert_t=fmt, shared_t=st)
    ref = _oracle_ref(L, x)
    assert_parity(run_calls(G, x, T, force_path="prefill"), ref, f"prefill {fmt} T={T}")


@pytest.mark.parametrize("T", [8192, 16384])
def test_prefill_router_slices_large_T(T):
    """Large chunks on a 16-expert layer: the router GEMM already fills the
    chip with few K slices, so it runs with 2 (8192 rows) and 1 (16384 rows)
    slices; every row is compared with the oracle."""
    _say(f"case: prefill bf16 router slices T={T}")
    rng = np.random.default_rng(2000 + T)
    a = _random_arrays(rng, 256, 16, 4, 96, 64, rstd=0.05, estd=0.05)
    a["router_bias"] = rng.standard_normal(16).astype(np.float32) * 0.5
    x = rng.standard_normal((T, 256)).astype(np.float32)
    b = dict(a)
    for k in ("router_w", "gate_vec", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"):
        b[k] = mi.f32_to_bf16_bits(a[k]).reshape(a[k].shape)
    L = oracle_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    G = gpu_layer_from_arrays(b, router_t="bf16", expert_t="bf16", shared_t="bf16")
    ref = _oracle_ref(L, x)
    assert_parity(run_calls(G, x, T), ref, f"prefill router slices T={T}")


def test_prefill_forced_on_small_calls():
    """MOE_FORCE_PATH=prefill runs the grouped path for 1..3 rows per call."""
    _say("case: prefill forced for small calls")
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    stacks = mi.expert_stacks(cfg)
    G = gpu_layer_from_config(cfg, dense, stacks)
    L = oracle_layer_from_config(cfg, dense=dense, stacks=stacks)
    x = mi.activations(cfg, T=7)
    ref = _oracle_ref(L, x)
    for rows in (1, 3):
        assert_parity(run_calls(G, x, rows, force_path="prefill"), ref, f"forced prefill rows={rows}")


def test_prefill_given_routing():
    _say("case: prefill with caller-supplied routing")
    rng = np.random.default_rng(52)
    a = _random_arrays(rng, 128, 16, 3, 64, 64)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    L = oracle_layer_from_arrays(a)
    ri, rw, rg, y, y64 = L.forward(x)
    G = gpu_layer_from_arrays(a)
    import sparse_moe_decode_amd as moe
    out = torch.empty((40, 128), dtype=torch.float32, device="cuda")
    moe.forward(G.desc, torch.from_numpy(x).cuda(), out, G.workspace(40), ids_in=torch.from_numpy(ri).cuda(),
                wts_in=torch.from_numpy(rw.astype(np.float32)).cuda(),
                gate_in=torch.from_numpy(rg.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    assert tolerance_ok(out.cpu().numpy(), y64).all()


# ------------------------------------------------------------ 2-bit format

@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_qb_unpack_bit_exact_random_bytes(nbits):
    """Random codes and random finite fp16 scale/min patterns (subnormals
    included): the device unpack equals the oracle's dequantizer bit for bit."""
    _say(f"case: {nbits}-bit unpack random bytes")
    import oracle
    import sparse_moe_decode_amd as moe
    rng = np.random.default_rng(61 + nbits)
    rows, cols = 96, 1024
    nb = cols // 32
    ncode = rows * cols * nbits // 8
    codes = rng.integers(0, 256, (rows, cols * nbits // 8), dtype=np.uint8)
    bits = rng.integers(0, 0x7c00, (rows, nb, 2), dtype=np.uint16)     # finite magnitudes
    bits |= (rng.integers(0, 2, (rows, nb, 2), dtype=np.uint16) << 15)
    packed = np.zeros(moe.qb_packed_bytes(nbits, rows, cols), np.uint8)
    packed[:ncode] = codes.reshape(-1)
    packed[ncode: ncode + rows * cols // 8] = bits.reshape(-1).view(np.uint8)
    ref = oracle.qb_dequantize(oracle.Q2(codes, bits[..., 0].copy(), bits[..., 1].copy(), rows, cols, nbits))
    dev = torch.from_numpy(packed).cuda()
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    moe.qb_unpack(nbits, dev, rows, cols, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["q2", "q3", "q4"])
def test_qb_unpack_of_packed_expert_weights(fmt):
    _say(f"case: {fmt} unpack of packed expert matrices")
    import oracle
    import sparse_moe_decode_amd as moe
    nbits = oracle.BITS[fmt]
    cfg = mi.CONFIGS[2].with_(expert_t=fmt)
    for e, m in [(0, mi.MAT_GATE), (7, mi.MAT_DOWN)]:
        w = mi.expert_matrix_f32(cfg, e, m)
        rows, cols = w.shape
        dev = torch.from_numpy(moe.qb_pack(nbits, w)).cuda()
        out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        moe.qb_unpack(nbits, dev, rows, cols, out)
        torch.cuda.synchronize()
        ref = oracle.qb_dequantize(oracle.qb_quantize(w, nbits))
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,K,E,skew,invalid", [(2048, 10, 512, True, False), (5, 3, 8, False, False),
                                                (1, 1, 1, False, False), (3000, 16, 1024, True, False),
                                                (777, 10, 512, False, False), (300, 4, 16, False, True)])
def test_sort_by_expert(T, K, E, skew, invalid):
    _say(f"case: sort T={T} K={K} E={E} invalid={invalid}")
    import sparse_moe_decode_amd as moe
    rng = np.random.default_rng(T * 31 + K)
    p = rng.dirichlet(np.full(E, 0.3 if skew else 5.0))
    ids = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    if invalid:   # ids outside [0, E) are skipped
        flat_ids = ids.reshape(-1)
        flat_ids[rng.choice(flat_ids.size, size=flat_ids.size // 7, replace=False)] = -1
        flat_ids[rng.choice(flat_ids.size, size=flat_ids.size // 11, replace=False)] = E
    dev = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * K, dtype=torch.int32, device="cuda")
    # the workspace needs no initialization: start from arbitrary bytes
    ws = torch.full((moe.sort_workspace_bytes(T, K, E),), 0xA5, dtype=torch.uint8, device="cuda")
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    ref_perm = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    ref_counts = np.bincount(flat[valid], minlength=E)
    for _ in range(2):   # the second call reuses the workspace as the first left it
        moe.sort_by_expert(dev, E, counts, offsets, perm, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)
        np.testing.assert_array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(ref_counts)]))
        np.testing.assert_array_equal(perm.cpu().numpy()[:ref_perm.size], ref_perm)


# ------------------------------------------------------- full-size workloads

@pytest.fixture(scope="module")
def decode_bf16():
    cfg = mi.CONFIGS[1]
    dense = mi.dense_weights(cfg)
    stacks = mi.expert_stacks(cfg)
    return cfg, dense, stacks, gpu_layer_from_config(cfg, dense, stacks)


@pytest.fixture(scope="module")
def decode_q2():
    cfg = mi.CONFIGS[2]
    dense = mi.dense_weights(cfg)
    return cfg, dense, gpu_layer_from_config(cfg, dense)


def _oracle_rows(cfg, dense, x, ids_gpu, rows, stacks=None):
    """Oracle on a sample of rows, with only the experts those rows need."""
    need = set(np.unique(ids_gpu[rows]).tolist())
    L = oracle_layer_from_config(cfg, dense=dense, experts=need, stacks=stacks)
    return _oracle_ref(L, x[rows])


def test_decode_bf16_full(decode_bf16):
    cfg, dense, stacks, G = decode_bf16
    _say(f"case: {cfg.name} T={cfg.T} one row per call")
    x = mi.activations(cfg)
    got = run_calls(G, x, 1)
    Lr = oracle_layer_from_config(cfg, dense=dense, experts=[], stacks=stacks)
    ri, rw, rg, _ = Lr.route(x)
    np.testing.assert_array_equal(got[0], ri)
    rows = np.arange(0, cfg.T, 4)
    ref = _oracle_rows(cfg, dense, x, got[0], rows, stacks)
    err = assert_parity(got, ref, cfg.name, rows)
    _say(f"{cfg.name}: max abs err {err[0]:.3g}, max err/tolerance {err[1]:.3g}")


def test_decode_q2_full(decode_q2):
    cfg, dense, G = decode_q2
    _say(f"case: {cfg.name} T={cfg.T} one row per call")
    x = mi.activations(cfg)
    got = run_calls(G, x, 1)
    Lr = oracle_layer_from_config(cfg, dense=dense, experts=[])
    ri, rw, rg, _ = Lr.route(x)
    np.testing.assert_array_equal(got[0], ri)
    rows = np.arange(0, cfg.T, 5)
    ref = _oracle_rows(cfg, dense, x, got[0], rows)
    err = assert_parity(got, ref, cfg.name, rows)
    _say(f"{cfg.name}: max abs err {err[0]:.3g}, max err/tolerance {err[1]:.3g}")


@pytest.mark.parametrize("R", [2, 3, 5, 8])
def test_fewrow_q2_full(R):
    cfg = mi.CONFIGS[3].with_(rows_per_call=R)
    _say(f"case: {cfg.name} R={R}")
    dense = mi.dense_weights(cfg)
    G = gpu_layer_from_config(cfg, dense)
    calls = {2: 500, 3: 333, 5: 100, 8: 125}[R]
    x = mi.activations(cfg, T=calls * R, instance=R)
    got = run_calls(G, x, R)
    Lr = oracle_layer_from_config(cfg, dense=dense, experts=[])
    ri, _, _, _ = Lr.route(x)
    np.testing.assert_array_equal(got[0], ri)
    rows = np.arange(0, x.shape[0], 6)
    ref = _oracle_rows(cfg, dense, x, got[0], rows)
    assert_parity(got, ref, f"{cfg.name} R={R}", rows)
    # rows of a few-row call equal the same rows decoded one at a time
    single = run_calls(G, x[:60], 1)
    np.testing.assert_array_equal(single[0], got[0][:60])
    assert tolerance_ok(got[3][:60], single[3]).all()


def test_prefill_q2_full():
    cfg = mi.CONFIGS[4]
    _say(f"case: {cfg.name} T={cfg.T}")
    dense = mi.dense_weights(cfg)
    G = gpu_layer_from_config(cfg, dense)
    x = mi.activations(cfg)
    got = run_calls(G, x, cfg.T)
    Lr = oracle_layer_from_config(cfg, dense=dense, experts=[])
    ri, _, _, _ = Lr.route(x)
    np.testing.assert_array_equal(got[0], ri)
    rows = np.arange(0, cfg.T, 8)
    ref = _oracle_rows(cfg, dense, x, got[0], rows)
    err = assert_parity(got, ref, cfg.name, rows)
    _say(f"{cfg.name}: max abs err {err[0]:.3g}, max err/tolerance {err[1]:.3g}")


@pytest.mark.parametrize("fmt", ["q3", "q4"])
def test_block_formats_full(fmt):
    """The full-shape decode layer with 3- and 4-bit experts quantized from
    the same fp32 source as the 2-bit workload: 200 tokens one per call,
    120 tokens as 3-row calls and a 256-row prefill call; every routing
    decision and every fourth row's output against the oracle."""
    cfg = mi.CONFIGS[2].with_(expert_t=fmt, name=f"decode_{fmt}")
    _say(f"case: {cfg.name} full shape")
    dense = mi.dense_weights(cfg)
    G = gpu_layer_from_config(cfg, dense)
    Lr = oracle_layer_from_config(cfg, dense=dense, experts=[])
    runs = []
    for what, T, rows, inst in (("decode", 200, 1, 0), ("few-row", 120, 3, 3), ("prefill", 256, 256, 7)):
        x = mi.activations(cfg, T=T, instance=inst)
        got = run_calls(G, x, rows)
        ri, _, _, _ = Lr.route(x)
        np.testing.assert_array_equal(got[0], ri)
        runs.append((what, x, got, np.arange(0, T, 4)))
    # one oracle layer holding every expert the sampled rows use
    need = set()
    for _, _, got, sample in runs:
        need |= set(np.unique(got[0][sample]).tolist())
    L = oracle_layer_from_config(cfg, dense=dense, experts=need)
    for what, x, got, sample in runs:
        ref = _oracle_ref(L, x[sample])
        err = assert_parity(got, ref, f"{cfg.name} {what}", sample)
        _say(f"{cfg.name} {what}: max abs err {err[0]:.3g}, max err/tolerance {err[1]:.3g}")


def test_determinism(decode_q2):
    cfg, dense, G = decode_q2
    _say("case: run-to-run determinism")
    x = mi.activations(cfg, T=64)
    a = run_calls(G, x, 1)
    b = run_calls(G, x, 1)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ------------------------------------------------ 48-layer decode stack

def _rotated(mats, off, E):
    """Expert e of a rotated stack is expert (e + off) % E of the base stack."""
    return [mats[(e + off) % E] for e in range(E)]


def test_stack_48_layers(decode_bf16):
    """48 MoE layers in a row (the model's MoE layers, Architecture page,
    "Qwen3-Next shape"): each with its own router, gate vector, shared
    expert and pre-MoE norm gamma, the RMS norm and the residual, its routed
    experts a rotation of one bf16 stack (layer l's expert e is base expert
    (e + 97 l) mod 512, through a doubled stack on the GPU). Three tokens one
    per call, three in one few-row call and sixteen in one prefill call run
    through all 48 layers; at every layer the output is compared with the
    oracle given the same layer input (ids identical, the rest within the
    tolerance)."""
    cfg, dense, stacks, G0 = decode_bf16
    import sparse_moe_decode_amd as moe
    E, L_layers = cfg.E, 48
    _say(f"case: 48-layer stack, {cfg.name} shapes")
    dbl = [torch.cat([t, t]) for t in (G0.exp_gate, G0.exp_up, G0.exp_down)]
    strides = [t.shape[1] * t.shape[2] * 2 for t in (G0.exp_gate, G0.exp_up, G0.exp_down)]
    offs = [(97 * l) % E for l in range(L_layers)]
    layers, dense_l, gam = [], [], []
    for l in range(L_layers):
        d = dense if l == 0 else mi.dense_weights(mi.layer_instance(cfg, l))
        g = mi.norm_weights(cfg, l)
        Gl = moe.Layer(H=cfg.H, E=E, K=cfg.K, I=cfg.I, Is=cfg.Is, router_t=cfg.router_t, expert_t=cfg.expert_t,
                       shared_t=cfg.shared_t, router_w=d["router_w"], gate_vec=d["gate_vec"], router_bias=None,
                       sh_gate=d["sh_gate"], sh_up=d["sh_up"], sh_down=d["sh_down"], exp_gate=np.zeros((1, 8, 8), np.uint16),
                       exp_up=np.zeros((1, 8, 8), np.uint16), exp_down=np.zeros((1, 8, 8), np.uint16), norm_w=g,
                       norm_eps=1e-6, residual=1)
        Gl.desc.exp_gate, Gl.desc.exp_up, Gl.desc.exp_down = (t.data_ptr() + offs[l] * st for t, st in zip(dbl, strides))
        layers.append(Gl)
        dense_l.append(d)
        gam.append(g)
    import oracle

    def oracle_layer(l, need):
        d = dense_l[l]
        mats = [_rotated(m, offs[l], E) for m in stacks]
        keep = set(int(e) for e in need)
        pick = [[m[e] if e in keep else None for e in range(E)] for m in mats]
        return oracle.Layer(H=cfg.H, E=E, K=cfg.K, I=cfg.I, Is=cfg.Is, router_t=cfg.router_t, expert_t=cfg.expert_t,
                            shared_t=cfg.shared_t, router_w=d["router_w"], gate_vec=d["gate_vec"], router_bias=None,
                            exp_gate=pick[0], exp_up=pick[1], exp_down=pick[2], sh_gate=d["sh_gate"],
                            sh_up=d["sh_up"], sh_down=d["sh_down"], norm_w=gam[l], norm_eps=float(np.float32(1e-6)),
                            residual=1)

    x0 = mi.activations(cfg, T=22, instance=48)
    for what, rows, T in (("decode", 1, 3), ("few-row", 3, 3), ("prefill", 16, 16)):
        x = x0[:T].copy()
        worst = 0.0
        for l in range(L_layers):
            got = run_calls(layers[l], x, rows)
            Lo = oracle_layer(l, np.unique(got[0]))
            ref = _oracle_ref(Lo, x)
            err = assert_parity(got, ref, f"stack {what} layer {l}")
            worst = max(worst, err[1])
            x = got[3]
        assert np.isfinite(x).all()
        _say(f"stack {what}: 48 layers, worst error / tolerance {worst:.3g}")
