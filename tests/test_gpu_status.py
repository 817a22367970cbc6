"""The device error word of the one-token gate/up launch.

Its waves wait for the routing through an LDS flag set by wave 0, a wait
bounded in polls.  A wave that gives up computes none of its routed rows and
stores 1 in the handle's error word, which coli_moe_status reports and
clears.  The bound is forced to zero polls from the host
(coli_moe_test_spin_limit), so that every waiting wave gives up at once: every
kernel still runs to its end, and no wait is left open.
"""
import ctypes

import numpy as np
import pytest

import routed_expert_ffn_f32_amd as cm
import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(layer, x, dev):
    out = layer.moe(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("shape_name", ["olmoe", "glm_small"])
def test_given_up_wait_is_reported_and_cleared(dev, shape_name):
    shape = {"olmoe": synth.OLMOE,
             "glm_small": synth.LayerShape(hidden=6144, n_experts=16, top_k=4, inter=512, n_shared=1, rsf=2.5,
                                           bias_sigma=0.05)}[shape_name]
    lib = cm.load_library()
    L = DeviceLayer(shape, 51, 0, dev, max_tokens=4, keep_host=True)
    try:
        x = synth.hidden(shape, 51, 1, batch=1)
        ref, _, _ = L.oracle_forward(x)
        out = run(L, x, dev)
        assert L.moe.status() == cm.COLI_MOE_OK
        log(f"  {shape_name}: plain call rel err {rel_err(out, ref):.3e}, status ok")
        assert lib.coli_moe_test_spin_limit(L.moe.handle, 0) == 0
        run(L, x, dev)
        assert L.moe.status() == cm.COLI_MOE_EDEVICE
        assert L.moe.status() == cm.COLI_MOE_OK  # read clears it
        assert lib.coli_moe_test_spin_limit(L.moe.handle, cm.COLI_MOE_DEFAULT_SPIN_LIMIT) == 0
        for b in range(3):
            xb = synth.hidden(shape, 51, 1, batch=10 + b)
            out = run(L, xb, dev)
            assert_routing_matches(L, xb, 1)
            refb, _, _ = L.oracle_forward(xb)
            assert rel_err(out, refb) <= 2e-3
        assert L.moe.status() == cm.COLI_MOE_OK
        assert lib.coli_moe_test_spin_limit(L.moe.handle, -1) == -4
    finally:
        L.close()
