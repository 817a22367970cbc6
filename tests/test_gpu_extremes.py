"""The largest routing shapes the boundary accepts, on every launch structure
the library picks by batch size: E = 512 experts (the most the dispatch
keeps histograms for), top_k = 32 (the most it accepts), top_k = E (every
expert selected: the forced dense mixture), top_k = 1, and E = 33 (a second
64-lane block of keys with one key).

Bar: routing and dispatch bit-exact against the oracle; outputs within 2e-3
element-wise floored at the row RMS on the GEMV paths, 2e-2 on the fp16 MFMA
path.  Small rows (h = I = 256) keep the oracle fast.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err, row_rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3
TOL_MFMA_ELEM = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def shape_of(E, k, shared=1):
    return synth.LayerShape(hidden=256, n_experts=E, top_k=k, inter=256, n_shared=shared, rsf=2.5,
                            bias_sigma=0.05)


def check(E, k, T, seed, dev, threshold=0, shared=1):
    shape = shape_of(E, k, shared)
    L = DeviceLayer(shape, seed, 0, dev, max_tokens=T, prefill_threshold=threshold, keep_host=True)
    try:
        x = synth.hidden(shape, seed, T, batch=T)
        out = L.moe(torch.from_numpy(x).to(dev))
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        idx, _ = assert_routing_matches(L, x, T)
        ref, _, _ = L.oracle_forward(x)
        err = rel_err(out, ref)
        tol = TOL_MFMA_ELEM if threshold and T >= threshold else TOL_GEMV
        log(f"  E={E} k={k} T={T}: {len(np.unique(idx))} distinct experts, rel err {err:.3e} "
            f"(per-token {row_rel_err(out, ref):.3e}, bar {tol:.0e})")
        assert err <= tol, err
        return idx
    finally:
        L.close()


@pytest.mark.parametrize("E,k,T", [
    (512, 8, 1), (512, 8, 4), (512, 8, 17), (512, 8, 40),   # one token, small batch, fused select+sort, sort launch
    (512, 32, 1), (512, 32, 2), (512, 32, 3), (512, 32, 33),  # the most experts per token
    (33, 32, 2), (33, 32, 5),                                  # a second block of keys holding one key
    (512, 1, 1), (512, 1, 70)])
def test_extreme_routing_gemv(dev, E, k, T):
    log(f"GEMV paths E={E} k={k} T={T}")
    check(E, k, T, 61 + E + k + T, dev)


@pytest.mark.parametrize("k,T", [(32, 1), (32, 4), (32, 50)])
def test_every_expert_selected(dev, k, T):
    """k = E = 32: every token selects every expert (the order of the slots is
    still the selection's), so each expert sees every token."""
    log(f"k = E = {k}, T={T}")
    idx = check(k, k, T, 71 + T, dev)
    assert np.all(np.sort(idx, axis=1) == np.arange(k)[None, :])


@pytest.mark.parametrize("E,k,T", [(512, 8, 300), (512, 32, 96), (64, 32, 128)])
def test_extreme_routing_mfma(dev, E, k, T):
    """The fp16 MFMA path with the most experts (tile list of up to 512
    active experts) and the most selections per token (T k = 3072 and 4096:
    the many-workgroup sort)."""
    log(f"MFMA path E={E} k={k} T={T}")
    check(E, k, T, 81 + E + k, dev, threshold=64)
