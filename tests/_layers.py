"""Test helpers: build the same seeded layer for the oracle and for the GPU path.

Only the seeded generator (``moe_inputs``) is shared; the oracle receives its
own quantization of 2-bit experts (``oracle.q2_quantize``), the GPU path gets
the library packer's bytes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def sig(a):
    return 1.0 / (1.0 + math.exp(-a))


def silu(a):
    return a * sig(a)


def eval_closed_form(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"sig": sig, "silu": silu, "exp": math.exp,
                                                   "log": math.log}))


def load_hand_fixture(name="hand_layer_f32.json"):
    """Dense fp32 arrays of the hand fixture plus its expected closed forms."""
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    H, E, I, Is = g["H"], g["E"], g["I"], g["Is"]
    x = np.zeros((1, H), np.float32)
    for h, v in g["x"]:
        x[0, h] = v
    rw = np.zeros((E, H), np.float32)
    for e, h, v in g["router_w"]:
        rw[e, h] = v
    gv = np.zeros((H,), np.float32)
    for h, v in g["gate_vec"]:
        gv[h] = v
    eg = np.zeros((E, I, H), np.float32)
    eu = np.zeros((E, I, H), np.float32)
    ed = np.zeros((E, H, I), np.float32)
    for e, i, h, v in g["exp_gate"]:
        eg[e, i, h] = v
    for e, i, h, v in g["exp_up"]:
        eu[e, i, h] = v
    for e, j, i, v in g["exp_down"]:
        ed[e, j, i] = v
    sg = np.zeros((Is, H), np.float32)
    su = np.zeros((Is, H), np.float32)
    sd = np.zeros((H, Is), np.float32)
    for i, h, v in g["sh_gate"]:
        sg[i, h] = v
    for i, h, v in g["sh_up"]:
        su[i, h] = v
    for j, i, v in g["sh_down"]:
        sd[j, i] = v
    def expected_of(exp):
        y = np.zeros((H,), np.float64)
        for j, expr in exp["y_nonzero"].items():
            y[int(j)] = eval_closed_form(expr)
        return dict(ids=np.array(exp["ids"], np.int32), wts=np.array([eval_closed_form(s) for s in exp["wts"]]),
                    gate=eval_closed_form(exp["gate"]), y=y)

    expected = expected_of(g["expected"])
    for k in g:   # further expectations of the same layer under other settings
        if k.startswith("expected_"):
            expected[k[len("expected_"):]] = expected_of(g[k])
    bias = None
    if "router_bias" in g:
        bias = np.zeros((E,), np.float32)
        for e, v in g["router_bias"]:
            bias[e] = v
    norm_w = None
    if "norm_w" in g:
        norm_w = np.ones((H,), np.float32)   # unlisted entries of gamma are 1
        for h, v in g["norm_w"]:
            norm_w[h] = v
    arrays = dict(H=H, E=E, K=g["K"], I=I, Is=Is, x=x, router_w=rw, gate_vec=gv, router_bias=bias,
                  exp_gate=eg, exp_up=eu, exp_down=ed, sh_gate=sg, sh_up=su, sh_down=sd,
                  bias_mode=g.get("bias_mode", 0), norm_w=norm_w, norm_eps=g.get("norm_eps", 1e-6),
                  residual=g.get("residual", 0))
    return arrays, expected


def oracle_layer_from_arrays(a: dict, *, router_t="f32", expert_t="f32", shared_t="f32", renormalize=1):
    """Oracle layer from dense arrays (f32 values or bf16 bits; experts may be
    a list of ``oracle.Q2``); optional bias_mode, norm_w / norm_eps, residual."""
    import oracle
    E = a["E"]
    return oracle.Layer(H=a["H"], E=E, K=a["K"], I=a["I"], Is=a["Is"], router_t=router_t,
                        expert_t=expert_t, shared_t=shared_t, router_w=a["router_w"],
                        gate_vec=a["gate_vec"], router_bias=a.get("router_bias"),
                        exp_gate=[a["exp_gate"][e] for e in range(E)],
                        exp_up=[a["exp_up"][e] for e in range(E)],
                        exp_down=[a["exp_down"][e] for e in range(E)],
                        sh_gate=a["sh_gate"], sh_up=a["sh_up"], sh_down=a["sh_down"],
                        renormalize=renormalize, bias_mode=a.get("bias_mode", 0), norm_w=a.get("norm_w"),
                        norm_eps=float(np.float32(a.get("norm_eps", 1e-6))), residual=a.get("residual", 0))


def oracle_layer_from_config(cfg: mi.LayerConfig, dense=None, experts=None, stacks=None):
    """Oracle layer for a seeded workload.

    ``experts``: restrict routed experts to this set (others absent; the oracle
    fails loudly if it selects one). Block-format experts (2, 3 or 4 bits) are
    quantized here with the oracle's own quantizer from the generator's fp32
    source.
    """
    import oracle
    dense = dense if dense is not None else mi.dense_weights(cfg)
    todo = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))
    G = [None] * cfg.E
    U = [None] * cfg.E
    D = [None] * cfg.E
    if cfg.expert_t in oracle.BITS:
        bits = oracle.BITS[cfg.expert_t]

        def quantize(e):   # experts are independent: quantized on a thread pool
            G[e] = oracle.qb_quantize(mi.expert_matrix_f32(cfg, e, mi.MAT_GATE), bits)
            U[e] = oracle.qb_quantize(mi.expert_matrix_f32(cfg, e, mi.MAT_UP), bits)
            D[e] = oracle.qb_quantize(mi.expert_matrix_f32(cfg, e, mi.MAT_DOWN), bits)

        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(mi._threads()) as ex:
            list(ex.map(quantize, todo))
    else:
        if stacks is None:
            stacks = mi.expert_stacks(cfg, experts)
        g, u, d = stacks
        for e in todo:
            G[e], U[e], D[e] = g[e], u[e], d[e]
    return oracle.Layer(H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, router_t=cfg.router_t,
                        expert_t=cfg.expert_t, shared_t=cfg.shared_t, router_w=dense["router_w"],
                        gate_vec=dense["gate_vec"], router_bias=dense["router_bias"],
                        exp_gate=G, exp_up=U, exp_down=D, sh_gate=dense["sh_gate"],
                        sh_up=dense["sh_up"], sh_down=dense["sh_down"])


def tolerance_ok(got, ref, atol=1e-4, rtol=2e-3):
    """Elementwise |got - ref| <= atol + rtol*|ref| (the stated output bound)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref) <= atol + rtol * np.abs(ref)


# ------------------------------------------------------------- GPU side

def gpu_layer_from_config(cfg: mi.LayerConfig, dense=None, stacks=None, renormalize=1):
    """The same seeded layer on the GPU (library packer for block-format experts)."""
    import sparse_moe_decode_amd as moe
    dense = dense if dense is not None else mi.dense_weights(cfg)
    kw = dict(H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, router_t=cfg.router_t, expert_t=cfg.expert_t,
              shared_t=cfg.shared_t, router_w=dense["router_w"], gate_vec=dense["gate_vec"],
              router_bias=dense["router_bias"], sh_gate=dense["sh_gate"], sh_up=dense["sh_up"],
              sh_down=dense["sh_down"], renormalize=renormalize)
    if cfg.expert_t in moe.BITS:
        return moe.Layer(**kw, expert_source=lambda e, m: mi.expert_matrix_f32(cfg, e, m))
    g, u, d = stacks if stacks is not None else mi.expert_stacks(cfg)
    return moe.Layer(**kw, exp_gate=g, exp_up=u, exp_down=d)


def gpu_layer_from_arrays(a: dict, *, router_t="f32", expert_t="f32", shared_t="f32", renormalize=1):
    import sparse_moe_decode_amd as moe
    kw = dict(H=a["H"], E=a["E"], K=a["K"], I=a["I"], Is=a["Is"], router_t=router_t, expert_t=expert_t,
              shared_t=shared_t, router_w=a["router_w"], gate_vec=a["gate_vec"], router_bias=a.get("router_bias"),
              sh_gate=a["sh_gate"], sh_up=a["sh_up"], sh_down=a["sh_down"], renormalize=renormalize,
              bias_mode=a.get("bias_mode", 0), norm_w=a.get("norm_w"), norm_eps=float(np.float32(a.get("norm_eps", 1e-6))),
              residual=a.get("residual", 0))
    if expert_t in moe.BITS:
        src = {0: a["exp_gate"], 1: a["exp_up"], 2: a["exp_down"]}
        return moe.Layer(**kw, expert_source=lambda e, m: np.asarray(src[m][e], np.float32))
    return moe.Layer(**kw, exp_gate=a["exp_gate"], exp_up=a["exp_up"], exp_down=a["exp_down"])


def run_calls(layer, x_host: np.ndarray, rows_per_call: int, force_path: str | None = None):
    """Run x through the layer in back-to-back calls of `rows_per_call` rows on
    one stream; returns host ids, wts, gate, y."""
    import torch
    import sparse_moe_decode_amd as moe
    T = x_host.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_host, np.float32)).cuda()
    y = torch.empty((T, layer.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, layer.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, layer.K), dtype=torch.float32, device="cuda")
    gate = torch.empty((T,), dtype=torch.float32, device="cuda")
    old = os.environ.get("MOE_FORCE_PATH")
    if force_path:
        os.environ["MOE_FORCE_PATH"] = force_path
    try:
        ws = layer.workspace(min(T, rows_per_call))
        for t in range(0, T, rows_per_call):
            r = min(rows_per_call, T - t)
            moe.forward(layer.desc, x[t:t + r], y[t:t + r], ws, ids_out=ids[t:t + r], wts_out=wts[t:t + r],
                        gate_out=gate[t:t + r])
        torch.cuda.synchronize()
    finally:
        if force_path:
            if old is None:
                os.environ.pop("MOE_FORCE_PATH", None)
            else:
                os.environ["MOE_FORCE_PATH"] = old
    return ids.cpu().numpy(), wts.cpu().numpy(), gate.cpu().numpy(), y.cpu().numpy()


def assert_parity(got, ref, what, sample_rows=None):
    """ids bit-identical; wts, gate, y within |d| <= 1e-4 + 2e-3 |ref|."""
    gi, gw, gg, gy = got
    ri, rw, rg, ry = ref
    rows = np.arange(len(ri)) if sample_rows is None else np.asarray(sample_rows)
    bad = np.nonzero(np.any(gi[rows] != ri, axis=1))[0]
    assert bad.size == 0, f"{what}: router selection differs on rows {rows[bad][:10]}: gpu {gi[rows[bad[0]]]} oracle {ri[bad[0]]}"
    ok_w = tolerance_ok(gw[rows], rw)
    assert ok_w.all(), f"{what}: wts out of tolerance, max err {np.abs(gw[rows] - rw).max():.3g}"
    ok_g = tolerance_ok(gg[rows], rg)
    assert ok_g.all(), f"{what}: gate out of tolerance, max err {np.abs(gg[rows] - rg).max():.3g}"
    ok_y = tolerance_ok(gy[rows], ry)
    err = np.abs(gy[rows].astype(np.float64) - ry)
    assert ok_y.all(), (f"{what}: {np.count_nonzero(~ok_y)} y values out of tolerance; max abs err "
                        f"{err.max():.3g}, worst row {rows[np.argmax(err.max(axis=1))]}")
    return float(err.max()), float((err / (1e-4 + 2e-3 * np.abs(ry))).max())
