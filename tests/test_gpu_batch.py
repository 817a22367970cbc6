"""GPU parity of the larger-batch decode kernels (int4 tables, batches above
the small-batch limits and below the prefill threshold) against the CPU
oracle, for both kernel families: the int8 matrix-core kernels (the
default: byte-plane activations, exact int32 products per 64-column group)
and the v_dot8 GEMV kernels, each forced with coli_moe_test_batch_kernels
(by default the library picks the GEMV kernels below 16 tokens).

Bar: routing and dispatch bit-exact, outputs within 2e-3 element-wise
(floored at the row RMS), as for every GEMV-class path.  Covered: token
counts that leave a ragged last pass of 4 tokens in the shared expert and in
the routed experts, one expert holding every token (passes of 4 in a row),
rows narrower than a column chunk (one weight group), widths whose row
blocks per workgroup are 4, 2 and 1, no shared expert, calls of decreasing
size in a row on one handle, and wide hidden rows.  The gate/up kernel runs
one token tile (4 tokens a pass) or two (8 a pass, from 2.5 assignments per
expert, or from 48 tokens with a shared expert): T = 5 and 7 of
h1024_I512_shared, T = 9 of the one-group rows, OLMoE-like T = 16 and the
wide rows take one, the other cases two, with ragged last passes both ways.
"""
import dataclasses

import numpy as np
import pytest

import routed_expert_ffn_f32_amd as cm
import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 2e-3
KERNELS = {"mfma": 1, "gemv": 0}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def forward_check(L, x, dev, what):
    T = x.shape[0]
    out = L.moe(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert_routing_matches(L, x, T)
    ref, _, _ = L.oracle_forward(x)
    err = rel_err(out, ref)
    log(f"  {what}: rel err {err:.3e}")
    assert np.isfinite(err) and err <= TOL, (what, err)
    return out


def layer(shape, seed, dev, max_tokens, kernels, **kw):
    L = DeviceLayer(shape, seed, 0, dev, max_tokens=max_tokens, keep_host=True, **kw)
    assert cm.load_library().coli_moe_test_batch_kernels(L.moe.handle, KERNELS[kernels]) == 0
    return L


SHAPES = {
    # name: (shape, T list)
    "h1024_I512_shared": (synth.LayerShape(hidden=1024, n_experts=16, top_k=4, inter=512, n_shared=1, rsf=2.0,
                                           bias_sigma=0.05), (5, 7, 13, 64)),
    "one_group_rows": (synth.TINY, (9, 30)),
    "h192_I320": (synth.LayerShape(hidden=192, n_experts=12, top_k=3, inter=320, n_shared=1, rsf=1.0,
                                   bias_sigma=0.02), (11,)),
    "olmoe_like": (synth.OLMOE, (16, 33)),
    "wide_h8192": (synth.LayerShape(hidden=8192, n_experts=8, top_k=2, inter=256, n_shared=1, rsf=1.5,
                                    bias_sigma=0.02), (6,)),
}


@pytest.mark.parametrize("kernels", list(KERNELS))
@pytest.mark.parametrize("name", list(SHAPES))
def test_batch_shapes(dev, name, kernels):
    shape, Ts = SHAPES[name]
    L = layer(shape, 21, dev, max(Ts), kernels)
    try:
        for T in Ts:
            forward_check(L, synth.hidden(shape, 21, T, batch=T), dev, f"{name} {kernels} T={T}")
    finally:
        L.close()


@pytest.mark.parametrize("kernels", list(KERNELS))
def test_batch_one_expert_takes_every_token(dev, kernels):
    """A huge bias sends every token to expert 3 first: T = 41 tokens in one
    routed expert (ten passes of 4 and one of 1 over its rows), the others
    ragged."""
    shape = synth.LayerShape(hidden=512, n_experts=10, top_k=2, inter=256, n_shared=1, rsf=1.0, bias_sigma=0.05)
    wr, b = synth.router(shape, 22)
    b = b.copy()
    b[3] = 6.0
    L = layer(shape, 22, dev, 41, kernels, wr=wr, bias=b)
    try:
        x = synth.hidden(shape, 22, 41)
        forward_check(L, x, dev, f"one expert, {kernels}")
        idx, _ = assert_routing_matches(L, x, 41)
        assert np.all(idx[:, 0] == 3)
    finally:
        L.close()


def test_batch_kernel_families_agree_and_repeat(dev):
    """Both families on one handle, calls of 64, 5 and 64 tokens in a row
    (stale planes of a larger call in the workspace); a repeated call is
    bitwise equal, and the two families agree within the bar."""
    shape = dataclasses.replace(synth.OLMOE, n_shared=1)
    L = layer(shape, 23, dev, 64, "mfma")
    lib = cm.load_library()
    try:
        outs = {}
        for kern in ("mfma", "gemv"):
            assert lib.coli_moe_test_batch_kernels(L.moe.handle, KERNELS[kern]) == 0
            for b, T in enumerate((64, 5, 64)):
                x = synth.hidden(shape, 23, T, batch=b % 2)  # calls 0 and 2: the same input
                outs[(kern, b)] = forward_check(L, x, dev, f"{kern} call {b} T={T}")
            assert np.array_equal(outs[(kern, 0)].view(np.uint32), outs[(kern, 2)].view(np.uint32))
        diff = rel_err(outs[("mfma", 0)], outs[("gemv", 0)])
        log(f"  families: rel diff {diff:.3e}")
        assert diff <= 2 * TOL
        assert lib.coli_moe_test_batch_kernels(L.moe.handle, 3) == -4
        assert lib.coli_moe_test_batch_kernels(L.moe.handle, 2) == 0
    finally:
        L.close()
