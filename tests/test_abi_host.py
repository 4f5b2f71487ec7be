"""Host-only checks of the C ABI: the library loads and exports every entry
point of include/moe.h, validation returns the documented codes before any
launch, and the host packer equals the oracle's own quantizer byte for byte.
No GPU work is issued here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import sparse_moe_decode_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_header_function():
    names = _header_functions()
    assert set(names) == set(moe.EXPORTS)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strerror():
    assert moe.abi_version() == 3
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert moe.strerror(code) and moe.strerror(code) != "unknown status"
    assert moe.strerror(-99) == "unknown status"


def _fake_desc(**kw):
    a = 0x10000  # aligned placeholders: never dereferenced by these host-only calls
    d = dict(hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512, renormalize=1,
             router_t=moe.MOE_BF16, expert_t=moe.MOE_BF16, shared_t=moe.MOE_BF16, reserved=0,
             router_w=a, router_bias=None, shared_gate_w=a, exp_gate=a, exp_up=a, exp_down=a,
             sh_gate=a, sh_up=a, sh_down=a)
    d.update(kw)
    return moe.LayerDesc(**d)


def _fwd(desc, x=0x20000, T=1, y=0x30000, ws=0x40000, ws_bytes=1 << 30, ids_in=None, wts_in=None, gate_in=None):
    return moe.lib().moe_forward(C.byref(desc), x, T, y, ids_in, wts_in, gate_in, None, None, None, ws,
                                 ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=0), moe.MOE_EINVAL),
    (dict(hidden=2050), moe.MOE_EINVAL),            # not a multiple of 32
    (dict(inter=500), moe.MOE_EINVAL),
    (dict(top_k=0), moe.MOE_EINVAL),
    (dict(top_k=513), moe.MOE_EINVAL),              # K > E
    (dict(top_k=17), moe.MOE_EINVAL),               # K > 16
    (dict(renormalize=2), moe.MOE_EINVAL),
    (dict(router_t=moe.MOE_Q2B32), moe.MOE_EINVAL),
    (dict(router_t=moe.MOE_Q4B32), moe.MOE_EINVAL),
    (dict(shared_t=moe.MOE_Q3B32), moe.MOE_EINVAL),
    (dict(expert_t=5), moe.MOE_EINVAL),
    (dict(expert_t=-1), moe.MOE_EINVAL),
    (dict(shared_t=7), moe.MOE_EINVAL),
    (dict(reserved=1), moe.MOE_EINVAL),
    (dict(bias_mode=2), moe.MOE_EINVAL),
    (dict(residual=2), moe.MOE_EINVAL),
    (dict(norm_w=0x10000, norm_eps=-1.0), moe.MOE_EINVAL),
    (dict(norm_w=0x10004), moe.MOE_EALIGN),
    (dict(router_w=None), moe.MOE_EINVAL),
    (dict(exp_down=None), moe.MOE_EINVAL),
    (dict(exp_up=0x10008), moe.MOE_EALIGN),
    (dict(router_bias=0x10002), moe.MOE_EALIGN),
    (dict(n_experts=2048), moe.MOE_EUNSUPPORTED),
    (dict(hidden=16384), moe.MOE_EUNSUPPORTED),
])
def test_descriptor_validation(kw, code):
    d = _fake_desc(**kw)
    assert _fwd(d) == code
    assert moe.lib().moe_route(C.byref(d), 0x20000, 1, 0x50000, 0x60000, 0x70000, 0x40000, 1 << 30, None) == code
    assert moe.lib().moe_workspace_bytes(C.byref(d), 1) == 0


@pytest.mark.parametrize("et", [moe.MOE_Q2B32, moe.MOE_Q3B32, moe.MOE_Q4B32])
def test_block_formats_accepted(et):
    d = _fake_desc(expert_t=et)
    assert moe.lib().moe_workspace_bytes(C.byref(d), 1) > 0
    assert moe.lib().moe_workspace_bytes(C.byref(d), 2048) > 0


def test_call_validation():
    d = _fake_desc()
    assert _fwd(d, T=-1) == moe.MOE_EINVAL
    assert _fwd(d, T=0) == moe.MOE_OK                       # no-op
    assert _fwd(d, x=None) == moe.MOE_EINVAL
    assert _fwd(d, y=None) == moe.MOE_EINVAL
    assert _fwd(d, ws=None) == moe.MOE_EINVAL
    assert _fwd(d, x=0x20004) == moe.MOE_EALIGN
    assert _fwd(d, y=0x30008) == moe.MOE_EALIGN
    assert _fwd(d, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _fwd(d, ids_in=0x50000) == moe.MOE_EINVAL         # routing given without weights
    need = moe.lib().moe_workspace_bytes(C.byref(d), 1)
    assert need > 0
    assert _fwd(d, ws_bytes=need - 1) == moe.MOE_EWORKSPACE
    assert moe.lib().moe_workspace_bytes(C.byref(d), 2048) >= need


def test_prefill_chunks_keep_workspace_bounded(monkeypatch):
    """Long prefill calls run as chunks whose workspace stays below 1.5 GiB
    (the prefill kernels address it with 32-bit offsets): the workspace of a
    call of any length is that of its largest chunk, also at the largest
    shapes the ABI accepts."""
    limit = 3 << 29
    for kw in (dict(), dict(hidden=8192, inter=4096, shared_inter=4096, top_k=16, n_experts=1024,
                           expert_t=moe.MOE_Q2B32)):
        d = _fake_desc(**kw)
        big = moe.lib().moe_workspace_bytes(C.byref(d), 2 ** 31 - 1)
        assert 0 < big <= limit
        assert moe.lib().moe_workspace_bytes(C.byref(d), 10 ** 6) <= big
    d = _fake_desc()
    monkeypatch.setenv("MOE_PREFILL_CHUNK", "100")
    assert moe.lib().moe_workspace_bytes(C.byref(d), 1000) == moe.lib().moe_workspace_bytes(C.byref(d), 100)
    assert moe.lib().moe_workspace_bytes(C.byref(d), 250) == moe.lib().moe_workspace_bytes(C.byref(d), 100)
    monkeypatch.delenv("MOE_PREFILL_CHUNK")
    assert moe.lib().moe_workspace_bytes(C.byref(d), 1000) > moe.lib().moe_workspace_bytes(C.byref(d), 100)


def test_binding_rejects_bad_tensors():
    """The Python binding checks dtype, shape, contiguity and device before
    handing raw pointers to the library."""
    torch = pytest.importorskip("torch")
    d = _fake_desc(hidden=64, n_experts=8, top_k=2, inter=32, shared_inter=32)
    x = torch.zeros((3, 64), dtype=torch.float32)
    y = torch.zeros((3, 64), dtype=torch.float32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(TypeError):
        moe.forward(d, x.double(), y, ws)
    with pytest.raises(ValueError):
        moe.forward(d, x[:, :32], y, ws)                      # hidden mismatch
    with pytest.raises(ValueError):
        moe.forward(d, x, y[:2], ws)                          # row count mismatch
    with pytest.raises(ValueError):
        moe.forward(d, torch.zeros((64, 3)).t(), y, ws)       # strided
    with pytest.raises(TypeError):
        moe.forward(d, x, y, ws, ids_out=torch.zeros((3, 2), dtype=torch.int64))
    with pytest.raises(ValueError):
        moe.forward(d, x, y, ws, ids_out=torch.zeros((3, 3), dtype=torch.int32))
    with pytest.raises(ValueError):
        moe.forward(d, x, y, ws)                              # host tensors
    with pytest.raises(ValueError):
        moe.route(d, x, torch.zeros((3, 2), dtype=torch.int32), torch.zeros((3, 2)), None, ws)


def test_sort_and_unpack_validation():
    L = moe.lib()
    assert L.moe_sort_by_expert(0x1000, 4, 0, 8, 0x2000, 0x3000, 0x4000, 0x5000, 1 << 20, None) == moe.MOE_EINVAL
    assert L.moe_sort_by_expert(0x1000, 4, 2, 2048, 0x2000, 0x3000, 0x4000, 0x5000, 1 << 20, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_sort_by_expert(0x1002, 4, 2, 8, 0x2000, 0x3000, 0x4000, 0x5000, 1 << 20, None) == moe.MOE_EALIGN
    assert L.moe_sort_by_expert(0x1000, 4, 2, 8, 0x2000, 0x3000, 0x4000, 0x5000, 1, None) == moe.MOE_EWORKSPACE
    assert L.moe_sort_by_expert(0x1000, 0, 2, 8, 0x2000, 0x3000, 0x4000, 0x5000, 1 << 20, None) == moe.MOE_OK
    assert L.moe_sort_workspace_bytes(2048, 10, 512) > 0
    assert L.moe_q2_unpack(0x1000, 4, 48, 0x2000, None) == moe.MOE_EINVAL
    assert L.moe_q2_unpack(0x1008, 4, 64, 0x2000, None) == moe.MOE_EALIGN
    assert L.moe_q2_unpack(None, 4, 64, 0x2000, None) == moe.MOE_EINVAL
    for bits in (1, 5, 0, -2):
        assert L.moe_qb_unpack(bits, 0x1000, 4, 64, 0x2000, None) == moe.MOE_EINVAL
    assert L.moe_qb_unpack(3, 0x1000, 4, 48, 0x2000, None) == moe.MOE_EINVAL
    assert L.moe_qb_unpack(4, 0x1000, 4, 64, 0x2008, None) == moe.MOE_EALIGN


# ---------------------------------------------------------------- packer

def _decode_physical(packed, rows, cols, bits=2):
    """Split a packed matrix by the layout documented in include/moe.h."""
    nc = rows * cols * bits // 8
    codes = packed[:nc].reshape(rows, cols * bits // 8)
    sm = packed[nc:nc + rows * cols // 8].view(np.uint16).reshape(rows, cols // 32, 2)
    return codes, sm[..., 0], sm[..., 1]


def test_packed_bytes_formula():
    assert moe.q2_packed_bytes(512, 2048) == 393216
    assert moe.q2_packed_bytes(2048, 512) == 393216
    assert moe.q2_packed_bytes(1, 32) == 256
    assert moe.q2_packed_bytes(3, 64) == 256
    assert moe.q2_packed_bytes(1, 48) == 0
    assert moe.q2_packed_bytes(0, 64) == 0
    # (b + 1) / 8 bytes per weight, rounded up to 256
    assert moe.qb_packed_bytes(3, 512, 2048) == 524288
    assert moe.qb_packed_bytes(4, 2048, 512) == 655360
    assert moe.qb_packed_bytes(3, 1, 32) == 256
    assert moe.qb_packed_bytes(4, 7, 64) == 512
    assert moe.qb_packed_bytes(2, 3, 64) == moe.q2_packed_bytes(3, 64)
    for bits in (0, 1, 5, 8):
        assert moe.qb_packed_bytes(bits, 4, 64) == 0
    assert moe.qb_packed_bytes(4, 1, 48) == 0


def _adversarial_blocks(rng):
    blocks = []
    blocks.append(np.full(32, 0.0123, np.float32))                       # constant, not fp16-exact
    blocks.append(np.full(32, 0.5, np.float32))                          # constant, fp16-exact
    blocks.append(np.full(32, 0.99999, np.float32))                      # min rounds up -> negative step
    blocks.append((np.arange(32) % 4 * 2.0 ** -6 - 2.0 ** -5).astype(np.float32))   # exact codes
    b = np.zeros(32, np.float32)
    b[0] = 1e-7                                                          # subnormal fp16 step
    blocks.append(b)
    blocks.append((rng.standard_normal(32) * 1e-6).astype(np.float32))   # tiny range
    blocks.append((rng.standard_normal(32) * 100).astype(np.float32))    # large range
    # values landing exactly half-way between codes
    s, m = 2.0 ** -7, -0.25
    b = (m + s * np.array([0, 3] + [0.5, 1.5, 2.5] * 10)).astype(np.float32)
    blocks.append(b)
    blocks.append(np.linspace(-3e4, 3e4, 32, dtype=np.float32))         # near the fp16 range
    return np.stack(blocks)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_packer_equals_oracle_quantizer(bits):
    rng = np.random.default_rng(21 + bits)
    mats = [
        (rng.standard_normal((64, 512)) * 0.02).astype(np.float32),
        (rng.standard_normal((16, 2048)) * 0.02).astype(np.float32),
        _adversarial_blocks(rng).reshape(-1, 32),
        _adversarial_blocks(rng).reshape(3, 96),
        (rng.uniform(-1, 1, (8, 256)) * 2.0 ** rng.integers(-20, 10, (8, 1))).astype(np.float32),
    ]
    for w in mats:
        rows, cols = w.shape
        packed = moe.qb_pack(bits, w)
        assert packed.nbytes == moe.qb_packed_bytes(bits, rows, cols)
        codes, scale, minv = _decode_physical(packed, rows, cols, bits)
        q = oracle.qb_quantize(w, bits)
        np.testing.assert_array_equal(codes, q.codes)
        np.testing.assert_array_equal(scale, q.scale)
        np.testing.assert_array_equal(minv, q.minv)
        used = rows * cols * (bits + 1) // 8
        assert np.all(packed[used:] == 0)
    if bits == 2:
        w = mats[0]
        np.testing.assert_array_equal(moe.q2_pack(w), moe.qb_pack(2, w))


def test_packer_rejects_bad_input():
    w = np.zeros((2, 64), np.float32)
    w[1, 3] = np.nan
    with pytest.raises(moe.MoEError) as e:
        moe.q2_pack(w)
    assert e.value.status == moe.MOE_ENONFINITE
    w[1, 3] = 1e6                                                # min/scale out of fp16 range
    with pytest.raises(moe.MoEError) as e:
        moe.q2_pack(w)
    assert e.value.status == moe.MOE_ENONFINITE
    L = moe.lib()
    src = np.zeros((2, 64), np.float32)
    dst = np.zeros(16, np.uint8)
    assert L.moe_q2_pack(src.ctypes.data, 2, 64, dst.ctypes.data, 16) == moe.MOE_EWORKSPACE
    assert L.moe_q2_pack(src.ctypes.data, 2, 48, dst.ctypes.data, 1 << 20) == moe.MOE_EINVAL
    big = np.zeros(1 << 12, np.uint8)
    for bits in (1, 5):
        assert L.moe_qb_pack(bits, src.ctypes.data, 2, 64, big.ctypes.data, big.nbytes) == moe.MOE_EINVAL
    assert L.moe_qb_pack(4, src.ctypes.data, 2, 64, dst.ctypes.data, 16) == moe.MOE_EWORKSPACE
    assert L.moe_qb_pack(3, None, 2, 64, big.ctypes.data, big.nbytes) == moe.MOE_EINVAL
    with pytest.raises(ValueError):
        moe.qb_pack(3, np.zeros(64, np.float32))


def _bf16_rne(v: np.ndarray) -> np.ndarray:
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def test_router_candidate_bound():
    """The prefill routing takes candidates from approximate logits: x as a
    bf16 hi + lo pair times bf16 router weights, summed in fp32 in any order.
    Its bound |L' - L| <= c_H ||x|| ||w_e|| (c_H as the kernel computes it)
    must hold, here with sequential fp32 sums in a shuffled order and a large
    common offset in x (cancellation)."""
    rng = np.random.default_rng(5)
    H, E = 2048, 64
    c_h = 1.01 * (3 * 2.0 ** -16 + (3 * H + 64) * 2.0 ** -23)
    w = _bf16_rne((rng.standard_normal((E, H)) * 0.03).astype(np.float32)).astype(np.float64)
    for shift in (0.0, 50.0):
        x = (rng.standard_normal(H) + shift).astype(np.float32)
        hi = _bf16_rne(x)
        lo = _bf16_rne(x - hi)
        assert np.all(np.abs(x.astype(np.float64) - hi - lo) <= 2.0 ** -16 * np.abs(x))
        terms = np.concatenate([w * hi.astype(np.float64)[None, :], w * lo.astype(np.float64)[None, :]], axis=1)
        terms = terms[:, rng.permutation(2 * H)].astype(np.float32)   # each product exact in fp32
        acc = np.zeros(E, np.float32)
        for k in range(terms.shape[1]):
            acc += terms[:, k]
        exact = w @ x.astype(np.float64)
        bound = c_h * np.linalg.norm(x.astype(np.float64)) * np.linalg.norm(w, axis=1)
        assert np.all(np.abs(acc.astype(np.float64) - exact) <= bound)
