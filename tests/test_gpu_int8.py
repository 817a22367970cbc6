"""GPU parity of int8 expert tables with one scale per row (the multi-token
prediction head's format) against the CPU oracle.

Bar: routing and dispatch bit-exact, outputs within 2e-3 element-wise
(floored at the row RMS), as for the int4 GEMV path.  Covered: one token
(planes in registers), 2 to 4 tokens (the verify shapes), larger batches
(groups of tokens through the small-batch launches, then the whole batch's
routing), every byte including -128 with random row scales, no shared
expert, routing limits, and the GLM-like MTP layer.
"""
import dataclasses

import numpy as np
import pytest

import routed_expert_ffn_f32_amd as cm
import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err, row_rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(layer, x, dev):
    out = layer.moe(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(layer, x, dev, what):
    T = x.shape[0]
    out = run(layer, x, dev)
    assert_routing_matches(layer, x, T)
    ref, _, _ = layer.oracle_forward(x)
    err = rel_err(out, ref)
    log(f"  {what}: rel err {err:.3e} (per-token {row_rel_err(out, ref):.3e})")
    assert err <= TOL_GEMV, (what, err)
    return out


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 16])
def test_tiny_int8(dev, T):
    L = DeviceLayer(synth.TINY_I8, 41, 0, dev, max_tokens=16, keep_host=True)
    try:
        check(L, synth.hidden(synth.TINY_I8, 41, T, batch=T), dev, f"tiny int8 T={T}")
    finally:
        L.close()


@pytest.mark.parametrize("h,I,E,k,shared,T", [(2048, 1024, 64, 8, 0, 1), (2048, 1024, 64, 8, 0, 4),
                                              (1024, 4096, 16, 4, 1, 2), (4096, 512, 32, 6, 1, 3),
                                              (8192, 256, 8, 2, 1, 1), (6144, 2048, 16, 8, 1, 9)])
def test_int8_shapes(dev, h, I, E, k, shared, T):
    """Row widths that change the chunks per lane of both launches (gate/up
    h / 1024, down I / 1024), with and without a shared expert; T = 9 runs
    groups of 4, 4 and 1 tokens."""
    shape = synth.LayerShape(hidden=h, n_experts=E, top_k=k, inter=I, n_shared=shared, rsf=2.5, bias_sigma=0.05,
                             weight_format=synth.WEIGHTS_INT8_ROW)
    L = DeviceLayer(shape, 43, 0, dev, max_tokens=16, keep_host=True)
    try:
        check(L, synth.hidden(shape, 43, T), dev, f"int8 h={h} I={I} E={E} k={k} shared={shared} T={T}")
    finally:
        L.close()


def test_int8_every_byte_random_row_scales(dev):
    """Uniform random bytes (every code, -128 included) and row scales
    log-uniform over two decades."""
    rng = np.random.default_rng(44)
    shape = synth.LayerShape(hidden=1024, n_experts=8, top_k=2, inter=512, n_shared=1, rsf=1.0, bias_sigma=0.05,
                             weight_format=synth.WEIGHTS_INT8_ROW)
    h, I, E = shape.hidden, shape.inter, shape.n_experts

    def tables(n):
        sc = lambda m: np.exp(rng.uniform(np.log(1e-5), np.log(1e-3), m)).astype(np.float32)
        return dict(gate_q=rng.integers(0, 256, (n, I, h), dtype=np.uint8), gate_s=sc((n, I)),
                    up_q=rng.integers(0, 256, (n, I, h), dtype=np.uint8), up_s=sc((n, I)),
                    down_q=rng.integers(0, 256, (n, h, I), dtype=np.uint8), down_s=sc((n, h)))
    routed = tables(E)
    sh = {kk: v[0] for kk, v in tables(1).items()}
    L = DeviceLayer(shape, 44, 0, dev, max_tokens=8, keep_host=True, routed=routed, shared=sh)
    try:
        for T in (1, 4, 8):
            check(L, synth.hidden(shape, 44, T, batch=T), dev, f"random bytes T={T}")
    finally:
        L.close()


def test_int8_routing_limits_and_repeat(dev):
    """Routing limits on an int8 layer; a repeated call is bitwise equal."""
    shape = dataclasses.replace(synth.OLMOE, hidden=1024, inter=1024, weight_format=synth.WEIGHTS_INT8_ROW)
    L = DeviceLayer(shape, 45, 0, dev, max_tokens=12, keep_host=True)
    try:
        L.set_routing(8, 0.6)
        for T in (1, 4, 12):
            x = synth.hidden(shape, 45, T, batch=T)
            a = check(L, x, dev, f"int8 top-p 0.6 T={T}")
            b = run(L, x, dev)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    finally:
        L.close()


def test_int8_config_checks(dev):
    lib = cm.load_library()
    import ctypes
    base = dict(hidden=1024, n_experts=8, top_k=2, inter=512, n_shared=0, routed_scaling_factor=1.0, max_tokens=4,
                weight_format=cm.COLI_MOE_WEIGHTS_INT8_ROW)
    assert cm.coli_moe_workspace_bytes(cm.make_config(**base)) > 0
    assert cm.coli_moe_workspace_bytes(cm.make_config(**base, group_size=64)) == 0   # int8: a scale per row
    assert cm.coli_moe_workspace_bytes(cm.make_config(**dict(base, inter=8192))) == 0  # down rows too wide
    assert cm.coli_moe_workspace_bytes(cm.make_config(**dict(base, weight_format=2))) == 0
    assert lib.coli_moe_cache_slot_bytes(ctypes.byref(cm.make_config(**base)), 4) == 0  # no expert cache
    L = DeviceLayer(synth.TINY_I8, 46, 0, dev, max_tokens=4)
    try:
        e = torch.tensor([0, 1], dtype=torch.int32, device=dev)
        assert lib.coli_moe_probe_read(L.moe.handle, ctypes.c_void_p(e.data_ptr()), 2, None) == -4
        assert lib.coli_moe_probe_read_down(L.moe.handle, ctypes.c_void_p(e.data_ptr()), 2, None) == -4
    finally:
        L.close()


@pytest.fixture(scope="module")
def mtp(dev):
    log("building the GLM-like int8 MTP layer (9.7 GB of experts)")
    L = DeviceLayer(synth.GLM_MTP_I8, 1, 0, dev, max_tokens=8)
    yield L
    L.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 2, 3, 4, 6])
def test_glm_mtp_int8(dev, mtp, T):
    """The GLM-like layer with int8 tables: draft (T = 1) and verify
    (T = 2..4) shapes, and T = 6 (groups of 4 and 2)."""
    check(mtp, synth.hidden(synth.GLM_MTP_I8, 1, T, batch=700 + T), dev, f"GLM-like int8 MTP layer T={T}")
