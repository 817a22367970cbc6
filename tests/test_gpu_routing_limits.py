"""GPU parity of the run-time routing limits (explicit smaller k, adaptive
expert top-p: lossy routing overrides from the knob table of the Colibri
tuning and runtime knobs guide) against the CPU oracle's
coli_oracle_select_limited / coli_oracle_forward_limited.

Bar as for the plain routing: expert indices (-1 in dropped slots), weights
and every dispatch array bit-exact; outputs within 2e-3 (GEMV paths) or
2e-2 (fp16 MFMA path) element-wise, floored at the row RMS.  Every launch
structure the library picks by T is covered: one token, the small-batch
launches (T <= 4), the token-row launches (T up to 64) and the MFMA path.
"""
import dataclasses
import warnings

import numpy as np
import pytest

import oracle
import routed_expert_ffn_f32_amd as cm
import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err, row_rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3
TOL_MFMA_ELEM = 2e-2
MID = synth.LayerShape(hidden=256, n_experts=16, top_k=4, inter=512, n_shared=1, rsf=2.5, bias_sigma=0.05)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(layer, x, dev):
    out = layer.moe(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(layer, x, dev, tol, what):
    T = x.shape[0]
    out = run(layer, x, dev)
    idx, _ = assert_routing_matches(layer, x, T)
    ref, _, _ = layer.oracle_forward(x)
    err = rel_err(out, ref)
    kept = (idx >= 0).sum(axis=1)
    log(f"  {what}: kept slots per token {kept.min()}..{kept.max()} of {layer.shape.top_k}, "
        f"rel err {err:.3e} (per-token {row_rel_err(out, ref):.3e})")
    assert err <= tol, (what, err)
    return idx, out


def test_dispatch_kernel_with_dropped_slots(dev):
    """The dispatch kernel on ids with dropped slots (-1, a suffix of each
    token's slots, as the limits produce; also scattered ones) against the
    oracle, bit-exact, up to T*k = 131072."""
    rng = np.random.default_rng(5)
    for T, k, E, scattered in ((1, 8, 256, False), (4, 2, 8, False), (64, 8, 256, False), (4096, 8, 256, False),
                               (16384, 8, 256, False), (300, 4, 16, True), (7, 8, 64, True)):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        if scattered:
            idx[rng.random(idx.shape) < 0.4] = -1
        else:
            m = rng.integers(1, k + 1, size=T)
            idx[np.arange(k)[None, :] >= m[:, None]] = -1
        log(f"dispatch with dropped slots T={T} k={k} E={E} scattered={scattered}")
        n = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        d_idx = torch.from_numpy(idx.reshape(-1).copy()).to(dev)
        o = dict(offsets=torch.full((E + 1,), -7, **i32), sorted_ids=torch.full((n,), -7, **i32),
                 inv=torch.full((n,), -7, **i32), active=torch.full((E,), -7, **i32),
                 n_active=torch.full((1,), -7, **i32))
        cm.coli_moe_test_dispatch(d_idx.data_ptr(), T, k, E, *(o[key].data_ptr() for key in
                                  ("offsets", "sorted_ids", "inv", "active", "n_active")),
                                  torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = {key: v.cpu().numpy() for key, v in o.items()}
        d = oracle.dispatch(idx, E)
        na = int(g["n_active"][0])
        assert na == d["n_active"]
        assert np.array_equal(g["offsets"], d["offsets"])
        assert np.array_equal(g["sorted_ids"], d["sorted_ids"])
        assert np.array_equal(g["inv"], d["inv"])
        assert np.array_equal(g["active"][:na], d["active"])


@pytest.mark.parametrize("shape_name,T,k_use,top_p", [
    ("tiny", 1, 1, 1.0), ("tiny", 4, 2, 0.6), ("tiny", 3, 1, 0.3),
    ("olmoe", 1, 8, 0.7), ("olmoe", 2, 4, 1.0), ("olmoe", 4, 6, 0.5),
    ("olmoe", 16, 8, 0.7), ("olmoe", 64, 5, 0.9), ("olmoe", 33, 1, 1.0)])
def test_small_layers_with_limits(dev, shape_name, T, k_use, top_p):
    shape = {"tiny": synth.TINY, "olmoe": synth.OLMOE}[shape_name]
    log(f"{shape_name} T={T} k_use={k_use} top_p={top_p}")
    L = DeviceLayer(shape, 31, 0, dev, max_tokens=64, keep_host=True)
    try:
        L.set_routing(k_use, top_p)
        x = synth.hidden(shape, 31, T, batch=T)
        check(L, x, dev, TOL_GEMV, f"{shape_name} T={T}")
    finally:
        L.close()


@pytest.mark.parametrize("k_use,top_p", [(4, 0.5), (2, 1.0), (3, 0.8)])
def test_mfma_path_with_limits(dev, k_use, top_p):
    """T = 300 on the fp16 MFMA path (threshold 64): fewer assignments per
    token change every expert's tile count; the dropped assignments must
    neither be computed nor reach the combine."""
    log(f"MFMA path T=300 k_use={k_use} top_p={top_p}")
    L = DeviceLayer(MID, 33, 0, dev, max_tokens=300, prefill_threshold=64, keep_host=True)
    try:
        L.set_routing(k_use, top_p)
        x = synth.hidden(MID, 33, 300)
        out = run(L, x, dev)
        idx, _ = assert_routing_matches(L, x, 300)
        ref, _, _ = L.oracle_forward(x)
        err = rel_err(out, ref)
        log(f"  kept {(idx >= 0).sum()} of {idx.size} assignments, element-wise rel err {err:.3e}, "
            f"per-token {row_rel_err(out, ref):.3e}")
        assert err <= TOL_MFMA_ELEM
    finally:
        L.close()


def test_limits_set_and_cleared_on_one_handle(dev):
    """Limits on, then off again: the plain routing's output comes back bit
    for bit; every call in between matches the oracle."""
    shape = dataclasses.replace(synth.OLMOE, hidden=1024, inter=512)
    L = DeviceLayer(shape, 35, 0, dev, max_tokens=64, keep_host=True)
    try:
        x = synth.hidden(shape, 35, 4)
        plain = run(L, x, dev)
        for k_use, top_p in ((8, 0.6), (3, 1.0), (8, 1.0)):
            L.set_routing(k_use, top_p)
            for T in (1, 4, 20):
                check(L, synth.hidden(shape, 35, T, batch=T), dev, TOL_GEMV, f"k_use={k_use} top_p={top_p} T={T}")
        again = run(L, x, dev)
        assert np.array_equal(plain.view(np.uint32), again.view(np.uint32))
    finally:
        L.close()


def test_set_routing_checks_and_warns(dev):
    L = DeviceLayer(synth.TINY, 36, 0, dev, max_tokens=4)
    try:
        lib = cm.load_library()
        import ctypes
        for k_use, top_p in ((0, 1.0), (3, 1.0), (2, 0.0), (2, 1.5), (2, -0.5)):
            assert lib.coli_moe_set_routing(L.moe.handle, k_use, ctypes.c_float(top_p)) == -2, (k_use, top_p)
        with pytest.warns(UserWarning, match="lossy"):
            L.moe.set_routing(1, 1.0)
        with pytest.warns(UserWarning, match="lossy"):
            L.moe.set_routing(None, 0.8)
        with warnings.catch_warnings():
            warnings.simplefilter("error")
            L.moe.set_routing()  # the plain routing: no warning
    finally:
        L.close()


@pytest.fixture(scope="module")
def glm(dev):
    log("building GLM-like layer 0 (5.46 GB of experts)")
    L = DeviceLayer(synth.GLM, 1, 0, dev, max_tokens=64)
    yield L
    L.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k_use,top_p", [(8, 0.7), (6, 1.0), (4, 0.5)])
def test_glm_decode_with_limits(dev, glm, k_use, top_p):
    """GLM-like layer at T = 1, 2, 4 and 64 with the limits: routing bit-exact,
    outputs at the GEMV bar, and fewer distinct experts than the plain
    routing of the same tokens."""
    glm.set_routing(k_use, top_p)
    try:
        for T in (1, 2, 4, 64):
            x = synth.hidden(synth.GLM, 1, T, batch=500 + T)
            idx, _ = check(glm, x, dev, TOL_GEMV, f"GLM-like T={T} k_use={k_use} top_p={top_p}")
            plain, _ = oracle.route(synth.GLM, glm.wr, glm.bias, x)
            n_lim = len(set(idx[idx >= 0].tolist()))
            n_plain = len(set(plain.reshape(-1).tolist()))
            log(f"    distinct experts {n_lim} (plain routing {n_plain})")
            assert n_lim <= n_plain
    finally:
        glm.set_routing()
