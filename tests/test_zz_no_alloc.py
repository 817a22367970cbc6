"""The forward entry point that allocates nothing (coli_moe_forward_noalloc,
whose workspace is the library's own device array) against the handle-based
coli_moe_forward on the same layer and inputs: two calls in a row, the second
with fewer tokens, both within the GEMV bar of 2e-3 of the handle's output
(they run the same kernels, so the outputs are expected bit for bit), and the
OLMoE-like calls also against the oracle."""
import numpy as np
import pytest

import synth
from tests.gpu_util import DeviceLayer, log, rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def noalloc(L: DeviceLayer, x: np.ndarray, dev) -> np.ndarray:
    import routed_expert_ffn_f32_amd as cm
    xd = torch.from_numpy(x).to(dev)
    out = torch.full_like(xd, float("nan"))
    cm.coli_moe_forward_noalloc(L.moe.cfg, L.moe.weights, xd.data_ptr(), out.data_ptr(), x.shape[0], L.moe.stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def handle(L: DeviceLayer, x: np.ndarray, dev) -> np.ndarray:
    out = L.moe(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,calls", [("olmoe", (16, 3)), ("glm", (64, 1))])
def test_noalloc_matches_handle_forward(dev, name, calls):
    shape = {"olmoe": synth.OLMOE, "glm": synth.GLM}[name]
    L = DeviceLayer(shape, 7, 0, dev, max_tokens=calls[0], keep_host=(name == "olmoe"))
    try:
        for b, T in enumerate(calls):
            log(f"no-alloc forward, {name} T={T} (call {b})")
            x = synth.hidden(shape, 7, T, batch=900 + b)
            want = handle(L, x, dev)
            got = noalloc(L, x, dev)
            assert np.all(np.isfinite(got))
            err = rel_err(got, want)
            same = bool(np.array_equal(got.view(np.uint32), want.view(np.uint32)))
            log(f"  against coli_moe_forward: rel err {err:.3e}, bitwise equal {same}")
            assert err <= TOL_GEMV, (T, err)
            if name == "olmoe":
                ref, _, _ = L.oracle_forward(x)
                e2 = rel_err(got, ref)
                log(f"  against the oracle: rel err {e2:.3e}")
                assert e2 <= TOL_GEMV, (T, e2)
    finally:
        L.close()
