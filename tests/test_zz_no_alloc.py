"""moe_forward_noalloc (the entry point that runs on the library's own
per-GPU scratch) against moe_forward on a caller workspace and against the
oracle: two calls in a row, the second smaller, for decode, few-row and
prefill row counts; and the rejection of a call whose workspace exceeds the
scratch."""
import sys

import numpy as np
import pytest

import moe_inputs as mi
from _layers import (assert_parity, gpu_layer_from_arrays, gpu_layer_from_config, oracle_layer_from_arrays,
                     oracle_layer_from_config, tolerance_ok)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_decode_amd as moe
    moe.lib()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(T, H, K):
    return (torch.full((T, H), float("nan"), device="cuda"), torch.full((T, K), -1, dtype=torch.int32, device="cuda"),
            torch.full((T, K), float("nan"), device="cuda"), torch.full((T,), float("nan"), device="cuda"))


def _run_pair(G, L, x_host, sizes, what):
    import sparse_moe_decode_amd as moe
    H, K = G.H, G.K
    for T in sizes:   # consecutive calls on the shared scratch, the later ones smaller
        _say(f"{what}: noalloc call of {T} rows")
        x = torch.from_numpy(np.ascontiguousarray(x_host[:T])).cuda()
        y, ids, wts, gate = _outputs(T, H, K)
        moe.forward_noalloc(G.desc, x, y, ids_out=ids, wts_out=wts, gate_out=gate)
        y2, ids2, wts2, gate2 = _outputs(T, H, K)
        moe.forward(G.desc, x, y2, G.workspace(T), ids_out=ids2, wts_out=wts2, gate_out=gate2)
        torch.cuda.synchronize()
        # same kernels on the same inputs: identical to the workspace entry point
        np.testing.assert_array_equal(ids.cpu().numpy(), ids2.cpu().numpy())
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(wts.cpu().numpy().view(np.uint32), wts2.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(gate.cpu().numpy().view(np.uint32), gate2.cpu().numpy().view(np.uint32))
        # and within the layer's tolerance of the oracle
        ri, rw, rg, _, y64 = L.forward(x_host[:T])
        got = (ids.cpu().numpy(), wts.cpu().numpy(), gate.cpu().numpy(), y.cpu().numpy())
        assert_parity(got, (ri, rw, rg, y64), f"{what} T={T}")


def test_noalloc_tiny_layer_decode_and_fewrow():
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    stacks = mi.expert_stacks(cfg)
    G = gpu_layer_from_config(cfg, dense, stacks)
    L = oracle_layer_from_config(cfg, dense=dense, stacks=stacks)
    x = mi.activations(cfg, T=16)
    _run_pair(G, L, x, (3, 1), "tiny fp32")
    _run_pair(G, L, x, (12, 2), "tiny fp32")


def test_noalloc_bf16_and_q2_layers_with_prefill_sizes():
    rng = np.random.default_rng(9)
    H, E, K, I, Is = 512, 64, 6, 128, 128
    a = dict(H=H, E=E, K=K, I=I, Is=Is, router_bias=None)
    for k, shp, sd in (("router_w", (E, H), 0.05), ("gate_vec", (H,), 0.05), ("exp_gate", (E, I, H), 0.03),
                       ("exp_up", (E, I, H), 0.03), ("exp_down", (E, H, I), 0.03), ("sh_gate", (Is, H), 0.03),
                       ("sh_up", (Is, H), 0.03), ("sh_down", (H, Is), 0.03)):
        a[k] = mi.f32_to_bf16_bits((rng.standard_normal(shp) * sd).astype(np.float32)).reshape(shp)
    x = rng.standard_normal((20, H)).astype(np.float32)
    L = oracle_layer_from_arrays(a, router_t="bf16", expert_t="bf16", shared_t="bf16")
    G = gpu_layer_from_arrays(a, router_t="bf16", expert_t="bf16", shared_t="bf16")
    _run_pair(G, L, x, (20, 13, 4, 1), "bf16")
    import oracle
    ef = {k: np.stack([mi.bf16_bits_to_f32(m) for m in a[k]]) for k in ("exp_gate", "exp_up", "exp_down")}
    q = dict(a)
    for k in ef:
        q[k] = [oracle.q2_quantize(m) for m in ef[k]]
    Lq = oracle_layer_from_arrays(q, router_t="bf16", expert_t="q2", shared_t="bf16")
    Gq = gpu_layer_from_arrays(dict(a, **ef), router_t="bf16", expert_t="q2", shared_t="bf16")
    _run_pair(Gq, Lq, x, (16, 3, 1), "q2")


def test_noalloc_rejects_calls_beyond_the_scratch():
    import sparse_moe_decode_amd as moe
    cfg = mi.CONFIGS[0]
    dense = mi.dense_weights(cfg)
    G = gpu_layer_from_config(cfg, dense, mi.expert_stacks(cfg))
    T = 4096
    assert moe.workspace_bytes(G.desc, T) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, cfg.H), device="cuda")
    y = torch.full((T, cfg.H), 7.0, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.forward_noalloc(G.desc, x, y)
    assert e.value.status == moe.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())   # nothing was enqueued
