"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bar: expert indices, routing weights and every dispatch array bit-exact;
layer outputs, max relative error element-wise (floored at the row RMS,
tests/gpu_util.rel_err):
 - float32-accumulate GEMV path: 2e-3;
 - fp16 MFMA (prefill) path: 2e-2.  The per-token relative error
   ||out_t - ref_t|| / ||ref_t|| is logged beside it.  Half precision rounds
   the hidden rows, the weights (q * s) and the intermediate to 11
   significant bits, about 6e-4 RMS error relative to the row RMS, so the
   element-wise maximum over a 4096 x 6144 output is near 3.5e-3.
"""
import json
import os

import numpy as np
import pytest

import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err, row_rel_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3
TOL_MFMA_ELEM = 2e-2   # element-wise, floored at the row RMS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def assert_mfma_close(out, ref, what=""):
    nw, ew = row_rel_err(out, ref), rel_err(out, ref)
    log(f"  {what}element-wise rel err {ew:.3e} (bar {TOL_MFMA_ELEM:.0e}), per-token {nw:.3e}, "
        f"rows {len(out)}")
    assert ew <= TOL_MFMA_ELEM, (what, ew)


def run(layer: DeviceLayer, x: np.ndarray, dev):
    xd = torch.from_numpy(x).to(dev)
    out = layer.moe(xd)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---------------------------------------------------------------------------
# Dispatch kernel alone.
# ---------------------------------------------------------------------------

def gpu_dispatch(idx: np.ndarray, E: int, dev):
    import routed_expert_ffn_f32_amd as cm
    T, k = idx.shape
    n = T * k
    i32 = dict(dtype=torch.int32, device=dev)
    d_idx = torch.from_numpy(np.ascontiguousarray(idx.reshape(-1), np.int32)).to(dev) if n else torch.empty(1, **i32)
    o = dict(offsets=torch.full((E + 1,), -7, **i32), sorted_ids=torch.full((max(n, 1),), -7, **i32),
             inv=torch.full((max(n, 1),), -7, **i32), active=torch.full((E,), -7, **i32),
             n_active=torch.full((1,), -7, **i32))
    cm.coli_moe_test_dispatch(d_idx.data_ptr(), T, k, E, o["offsets"].data_ptr(), o["sorted_ids"].data_ptr(),
                              o["inv"].data_ptr(), o["active"].data_ptr(), o["n_active"].data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    h = {k2: v.cpu().numpy() for k2, v in o.items()}
    na = int(h["n_active"][0])
    return dict(offsets=h["offsets"], sorted_ids=h["sorted_ids"][:n], inv=h["inv"][:n], active=h["active"][:na],
                n_active=na)


def test_dispatch_worked_examples_from_pages(dev):
    import oracle
    for case in json.load(open(os.path.join(GOLDEN, "dispatch_worked_examples.json")))["examples"]:
        log(f"dispatch page example {case['name']}")
        g = gpu_dispatch(np.array(case["idx"], np.int32), case["E"], dev)
        for key in ("offsets", "sorted_ids", "inv", "active"):
            assert g[key].tolist() == case[key], (case["name"], key)
        d = oracle.dispatch(np.array(case["idx"], np.int32), case["E"])
        assert g["n_active"] == d["n_active"]


@pytest.mark.parametrize("T,k,E,skew", [(1, 8, 256, 0), (4, 2, 8, 0), (64, 8, 256, 0), (16, 8, 64, 0),
                                        (4096, 8, 256, 1), (333, 3, 17, 0), (1000, 1, 1, 0),
                                        (8192, 16, 512, 1), (0, 4, 8, 0), (1, 32, 32, 0),
                                        (1025, 1, 5, 0), (1024, 1, 7, 0), (2049, 2, 300, 1), (4000, 8, 512, 0)])
def test_dispatch_kernel_matches_oracle(dev, T, k, E, skew):
    import oracle
    log(f"dispatch T={T} k={k} E={E} skew={skew}")
    rng = np.random.default_rng(T * 7 + k * 3 + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]) if T else np.zeros((0, k))
    else:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else np.zeros((0, k))
    idx = idx.astype(np.int32).reshape(T, k)
    g = gpu_dispatch(idx, E, dev)
    d = oracle.dispatch(idx, E)
    for key in ("offsets", "sorted_ids", "inv", "active"):
        assert np.array_equal(g[key], d[key]), key
    assert g["n_active"] == d["n_active"]


# ---------------------------------------------------------------------------
# Small layers: full outputs against the oracle.
# ---------------------------------------------------------------------------

def check_full(shape, seed, T, dev, tol=TOL_GEMV, max_tokens=None, layer=0, batch=0):
    L = DeviceLayer(shape, seed, layer, dev, max_tokens=max_tokens or T, keep_host=True)
    x = synth.hidden(shape, seed, T, layer=layer, batch=batch)
    out = run(L, x, dev)
    assert_routing_matches(L, x, T)
    ref, _, _ = L.oracle_forward(x)
    err = rel_err(out, ref)
    log(f"  rel err {err:.3e}")
    assert err <= tol, err
    return L, x, out


def test_tiny_layer(dev):
    log("tiny layer T=4")
    check_full(synth.TINY, 1, 4, dev)


def test_tiny_layer_forced_all_experts(dev):
    """k = E = 8 selects every expert for every token (pattern of the pages'
    all-keys check of the sparse attention, applied to experts)."""
    log("tiny layer k=E=8")
    import dataclasses
    check_full(dataclasses.replace(synth.TINY, top_k=8), 2, 4, dev)


def test_olmoe_like_layer(dev):
    log("OLMoE-like layer T=16, no shared expert")
    check_full(synth.OLMOE, 1, 16, dev)


def test_single_expert_layer(dev):
    log("E=1 k=1 layer")
    shape = synth.LayerShape(hidden=128, n_experts=1, top_k=1, inter=192, n_shared=1, rsf=2.5, bias_sigma=0.0)
    check_full(shape, 3, 5, dev)


def test_skewed_routing_many_tokens_per_expert(dev):
    """A huge bias sends every token to expert 5 first: one expert holds all
    T = 37 tokens (token loops of 4, 2 and 1), ragged everywhere."""
    log("skewed routing T=37")
    shape = synth.LayerShape(hidden=256, n_experts=16, top_k=3, inter=128, n_shared=1, rsf=1.5, bias_sigma=0.05)
    wr, b = synth.router(shape, 8)
    b = b.copy()
    b[5] = 5.0
    L = DeviceLayer(shape, 8, 0, dev, max_tokens=64, keep_host=True, wr=wr, bias=b)
    x = synth.hidden(shape, 8, 37)
    out = run(L, x, dev)
    idx, _ = assert_routing_matches(L, x, 37)
    assert np.all(idx[:, 0] == 5)
    ref, _, _ = L.oracle_forward(x)
    assert rel_err(out, ref) <= TOL_GEMV


@pytest.mark.parametrize("h,I", [(3072, 4096), (1024, 6144), (2048, 8192), (8192, 512), (512, 10240)])
def test_larger_batch_row_widths(dev, h, I):
    """T = 12 (above the small-batch path) at the widths that pick each
    register-resident row width of the larger-batch kernels: gate/up rows of
    2 and 1 chunks of 2048 columns per lane, down rows of 2, 3 and 4 chunks
    (8, 4 and 4 rows a wave); and the streaming kernels past them (h = 8192
    for gate/up, I = 10240 for down)."""
    log(f"larger batch h={h} I={I} T=12")
    shape = synth.LayerShape(hidden=h, n_experts=6, top_k=2, inter=I, n_shared=1, rsf=1.5, bias_sigma=0.02)
    check_full(shape, 11, 12, dev)


@pytest.mark.parametrize("h,E", [(320, 20), (192, 20), (768, 36)])
def test_router_wide_tiles_ragged(dev, h, E):
    """T = 300 takes the router's wide tiles (32 tokens x 16 experts per
    block) with every edge ragged: T not a multiple of 32, E not a multiple
    of 16, and the chain blocks of 4 steps per lane (h / 256 of them, the
    last partial when h / 64 is not a multiple of 4) in every arrangement
    the loop has: h = 320, two blocks (one pair, the second partial);
    h = 192, one partial block (no pair, the odd tail alone); h = 768,
    three full blocks (a pair and the odd tail).  Routing weights must match
    the oracle bit for bit, which needs each logit's fma chain and butterfly
    unchanged; h = 320 keeps the call on the GEMV path, so the digit-plane
    launch that follows runs too."""
    log(f"router wide tiles T=300 E={E} h={h}")
    shape = synth.LayerShape(hidden=h, n_experts=E, top_k=3, inter=128, n_shared=1, rsf=2.5, bias_sigma=0.05)
    check_full(shape, 31, 300, dev)


def test_measurement_probes(dev):
    """The probes bench.py measures the GPU's own rates with do their work:
    the stream probe's XOR of a 64 MiB + 48 B buffer (not a multiple of
    its grid stride) equals numpy's, so every word was read exactly once;
    every wave of the MFMA probe finds all its accumulators at 16 x iters."""
    import routed_expert_ffn_f32_amd as cm
    log("measurement probes")
    stream = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(5)
    words = (64 << 20) // 4 + 12
    host = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cm.coli_moe_probe_stream(buf.data_ptr(), words * 4, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host))
    sink.zero_()
    cm.coli_moe_probe_mfma(1000, 96, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert int(sink.item()) == 96 * 4
    # the read probes of the two decode launches run on a layer's tables,
    # out-of-range ids reading nothing
    shape = synth.LayerShape(hidden=6144, n_experts=16, top_k=4, inter=2048, n_shared=1, rsf=2.5, bias_sigma=0.05)
    L = DeviceLayer(shape, 9, 0, dev, max_tokens=1)
    try:
        e = torch.tensor([0, 15, -1, 16, -2], dtype=torch.int32, device=dev)
        cm.coli_moe_probe_read(L.moe.handle, e.data_ptr(), e.numel(), stream)
        cm.coli_moe_probe_read_down(L.moe.handle, e.data_ptr(), e.numel(), stream)
        torch.cuda.synchronize()
    finally:
        L.close()


def test_all_codes_including_minus_eight(dev):
    """Codes drawn uniformly over all 256 byte values (so -8 appears) with
    random positive scales: the unpacking of every code is exercised."""
    log("uniform byte codes")
    shape = synth.LayerShape(hidden=128, n_experts=4, top_k=2, inter=64, n_shared=1, rsf=1.0, bias_sigma=0.01)
    rng = np.random.default_rng(99)
    E, h, I = 4, 128, 64

    def tables(n):
        return dict(gate_q=rng.integers(0, 256, (n, I, h // 2), dtype=np.uint8),
                    gate_s=rng.uniform(0.001, 0.004, (n, I, h // 64)).astype(np.float32),
                    up_q=rng.integers(0, 256, (n, I, h // 2), dtype=np.uint8),
                    up_s=rng.uniform(0.001, 0.004, (n, I, h // 64)).astype(np.float32),
                    down_q=rng.integers(0, 256, (n, h, I // 2), dtype=np.uint8),
                    down_s=rng.uniform(0.001, 0.004, (n, h, I // 64)).astype(np.float32))
    routed = tables(E)
    shared = {k: v[0] for k, v in tables(1).items()}
    assert np.any((routed["gate_q"] & 0xF) == 8)
    L = DeviceLayer(shape, 5, 0, dev, max_tokens=8, keep_host=True, routed=routed, shared=shared)
    x = synth.hidden(shape, 5, 8)
    out = run(L, x, dev)
    assert_routing_matches(L, x, 8)
    ref, _, _ = L.oracle_forward(x)
    assert rel_err(out, ref) <= TOL_GEMV


def test_token_counts_on_one_handle(dev):
    """One handle, T = max_tokens, smaller T, a dry run and an over-capacity
    call; outputs of each call match the oracle."""
    import routed_expert_ffn_f32_amd as cm
    log("token counts on one handle")
    shape = synth.TINY
    L = DeviceLayer(shape, 6, 0, dev, max_tokens=24, keep_host=True)
    for T in (24, 1, 7, 24, 2):
        x = synth.hidden(shape, 6, T, batch=T)
        out = run(L, x, dev)
        assert_routing_matches(L, x, T)
        ref, _, _ = L.oracle_forward(x)
        assert rel_err(out, ref) <= TOL_GEMV, T
    xd = torch.zeros((1, shape.hidden), dtype=torch.float32, device=dev)
    od = torch.full((1, shape.hidden), 3.0, dtype=torch.float32, device=dev)
    assert cm.coli_moe_forward(L.moe.handle, xd.data_ptr(), od.data_ptr(), 0, L.moe.stream) == 0
    torch.cuda.synchronize()
    assert torch.all(od == 3.0)
    with pytest.raises(cm.ColiMoeError) as ei:
        cm.coli_moe_forward(L.moe.handle, xd.data_ptr(), od.data_ptr(), 25, L.moe.stream)
    assert ei.value.code == -1


def test_kernel_choice_boundaries_on_one_handle(dev):
    """One GEMV-path handle (h = 320 is not a multiple of 256, so no MFMA
    path at any T) at the batch sizes on both sides of every switch between
    kernels: the small-batch kernels (T <= 4), the router's tile sizes (12,
    24, 48, 256), selection and sort in one workgroup (T <= 16).  Routing
    bit-exact and outputs against the oracle at each."""
    log("kernel choice boundaries")
    shape = synth.LayerShape(hidden=320, n_experts=24, top_k=4, inter=192, n_shared=1, rsf=2.5, bias_sigma=0.05)
    L = DeviceLayer(shape, 41, 0, dev, max_tokens=300, keep_host=True)
    for T in (4, 5, 11, 12, 16, 17, 23, 24, 47, 48, 255, 256, 300):
        x = synth.hidden(shape, 41, T, batch=T)
        out = run(L, x, dev)
        assert_routing_matches(L, x, T)
        ref, _, _ = L.oracle_forward(x)
        assert rel_err(out, ref) <= TOL_GEMV, T


@pytest.mark.parametrize("path", ["small_batch", "token_rows", "mfma"])
def test_outlier_channels_and_zero_rows(dev, path):
    """Hidden rows of three kinds in one batch: N(0,1); all zeros (every
    logit 0, so the selection falls to the bias, and the output must be
    exactly 0); N(0,1) with four massive-activation channels at +-300 (one
    32-column block of the digit-plane format then spans five orders of
    magnitude).  Routing bit-exact for every row, zero rows exactly zero,
    the rest against the oracle at the path's bound."""
    log(f"outlier channels and zero rows, {path}")
    if path == "mfma":
        shape, T, thr = MID, 300, 64
    else:
        shape = synth.LayerShape(hidden=320, n_experts=24, top_k=4, inter=192, n_shared=1, rsf=2.5, bias_sigma=0.05)
        T, thr = (3, 0) if path == "small_batch" else (20, 0)
    L = DeviceLayer(shape, 51, 0, dev, max_tokens=T, prefill_threshold=thr, keep_host=True)
    x = synth.hidden(shape, 51, T, batch=77)
    x[1::3] = 0.0
    ch = [3, 77, 150, shape.hidden - 1]
    x[2::3, ch] = np.where(x[2::3, ch] < 0, -300.0, 300.0).astype(np.float32)
    out = run(L, x, dev)
    assert_routing_matches(L, x, T)
    zero = np.all(x == 0.0, axis=1)
    assert zero.sum() == len(range(1, T, 3))
    assert np.all(out[zero] == 0.0)
    ref, _, _ = L.oracle_forward(x[~zero])
    if path == "mfma":
        assert_mfma_close(out[~zero], ref, "outliers: ")
    else:
        err = rel_err(out[~zero], ref)
        log(f"  rel err {err:.3e}")
        assert err <= TOL_GEMV, err


def test_two_runs_bitwise_identical(dev):
    log("determinism")
    shape = synth.OLMOE
    L = DeviceLayer(shape, 11, 0, dev, max_tokens=16)
    x = synth.hidden(shape, 11, 16)
    a = run(L, x, dev)
    _, ra = L.moe.last_routing()
    ra = {k: v.cpu().numpy().copy() for k, v in ra.items()}
    b = run(L, x, dev)
    _, rb = L.moe.last_routing()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for k, v in rb.items():
        assert np.array_equal(v.cpu().numpy().view(np.uint32), ra[k].view(np.uint32)), k


# ---------------------------------------------------------------------------
# Calls in a row on one handle: the gate/up launch hands rows out through
# atomic queues that the down launch clears for the next call.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny_all", 1), ("olmoe", 1), ("single", 1), ("olmoe", 3),
                                    ("tiny", 4)])
def test_small_batch_calls_in_a_row(dev, name, T):
    """Five calls on one handle, each with its own input: routing bit-exact
    and outputs at the GEMV bar every time."""
    import dataclasses
    shapes = {"tiny": synth.TINY, "tiny_all": dataclasses.replace(synth.TINY, top_k=8), "olmoe": synth.OLMOE,
              "single": synth.LayerShape(hidden=128, n_experts=1, top_k=1, inter=192, n_shared=1, rsf=2.5,
                                         bias_sigma=0.0)}
    shape = shapes[name]
    log(f"small-batch calls in a row: {name} T={T}")
    L = DeviceLayer(shape, 31, 0, dev, max_tokens=4, keep_host=True)
    for b in range(5):
        x = synth.hidden(shape, 31, T, batch=200 + b)
        out = run(L, x, dev)
        assert_routing_matches(L, x, T)
        ref, _, _ = L.oracle_forward(x)
        err = rel_err(out, ref)
        log(f"  call {b}: rel err {err:.3e}")
        assert err <= TOL_GEMV, (b, err)
    L.close()


# ---------------------------------------------------------------------------
# The fp16 MFMA (prefill) path on small layers: full outputs.
# ---------------------------------------------------------------------------

MID = synth.LayerShape(hidden=256, n_experts=16, top_k=4, inter=512, n_shared=1, rsf=2.5, bias_sigma=0.05)


def check_mfma(shape, seed, T, dev, threshold, max_tokens=None, wr=None, bias=None, rows=None):
    L = DeviceLayer(shape, seed, 0, dev, max_tokens=max_tokens or T, prefill_threshold=threshold,
                    keep_host=True, wr=wr, bias=bias)
    x = synth.hidden(shape, seed, T)
    out = run(L, x, dev)
    idx, _ = assert_routing_matches(L, x, T)
    sel = slice(None) if rows is None else rows
    ref, _, _ = L.oracle_forward(x[sel])
    assert_mfma_close(out[sel], ref)
    return L, x, out, idx


def test_mfma_path_several_tiles_ragged(dev):
    """T = 300 tokens, 16 experts, k = 4: about 75 tokens per expert, the
    shared expert in 2 tiles (256 + 44 rows), every N tile count > 1."""
    log("MFMA path T=300 h=256 I=512 E=16 k=4")
    check_mfma(MID, 21, 300, dev, threshold=64)


def test_mfma_path_one_expert_takes_all(dev):
    """Bias 5.0 on expert 3: all 300 tokens in its first slot, so one expert
    spans three M tiles and the rest are small or empty."""
    log("MFMA path, one expert holds every token")
    wr, b = synth.router(MID, 22)
    b = b.copy()
    b[3] = 5.0
    _, _, _, idx = check_mfma(MID, 22, 300, dev, threshold=64, wr=wr, bias=b)
    assert np.all(idx[:, 0] == 3)


def test_mfma_path_few_tokens(dev):
    """Threshold 1: T = 5 tokens on the MFMA path (tiles almost all padding)."""
    log("MFMA path T=5 (threshold 1)")
    check_mfma(MID, 23, 5, dev, threshold=1)


def random_tables(rng, n, h, I, lo, hi):
    """n experts of uniform random code bytes (every code, -8 included) and
    scales log-uniform in [lo, hi) (each group its own)."""
    def sc(shape):
        return np.exp(rng.uniform(np.log(lo), np.log(hi), shape)).astype(np.float32)
    return dict(gate_q=rng.integers(0, 256, (n, I, h // 2), dtype=np.uint8), gate_s=sc((n, I, h // 64)),
                up_q=rng.integers(0, 256, (n, I, h // 2), dtype=np.uint8), up_s=sc((n, I, h // 64)),
                down_q=rng.integers(0, 256, (n, h, I // 2), dtype=np.uint8), down_s=sc((n, h, I // 64)))


def test_mfma_path_all_codes_wide_scales(dev):
    """MFMA path on uniform random code bytes (all 16 codes, -8 included)
    with group scales log-uniform over five decades, 1e-6 .. 1e-1: the
    per-matrix power-of-two prescale keeps every weight a normal half."""
    log("MFMA path, all codes, scales 1e-6 .. 1e-1")
    rng = np.random.default_rng(123)
    h, I, E = MID.hidden, MID.inter, MID.n_experts
    routed = random_tables(rng, E, h, I, 1e-6, 1e-1)
    shared = {k: v[0] for k, v in random_tables(rng, 1, h, I, 1e-6, 1e-1).items()}
    L = DeviceLayer(MID, 61, 0, dev, max_tokens=200, prefill_threshold=64, keep_host=True, routed=routed,
                    shared=shared)
    x = synth.hidden(MID, 61, 200)
    out = run(L, x, dev)
    assert_routing_matches(L, x, 200)
    ref, _, _ = L.oracle_forward(x)
    assert_mfma_close(out, ref, "all codes: ")


def test_mfma_path_hidden_and_weight_ranges(dev):
    """MFMA path with hidden rows scaled by 10^-4 .. 10^4 (row by row) and
    experts whose scales sit near 1e-7 or near 10: every per-token,
    per-matrix and intermediate power-of-two factor is exercised, far outside
    half precision's own range."""
    log("MFMA path, hidden rows 1e-4 .. 1e4, scales near 1e-7 and 10")
    rng = np.random.default_rng(321)
    h, I, E = MID.hidden, MID.inter, MID.n_experts
    routed = synth.routed_tables(MID, 62)
    for name in ("gate_s", "up_s", "down_s"):
        routed[name] = routed[name].copy()
        routed[name][: E // 2] *= np.float32(1e-5)
        routed[name][E // 2:] *= np.float32(1e3)
    shared = synth.shared_tables(MID, 62)
    L = DeviceLayer(MID, 62, 0, dev, max_tokens=160, prefill_threshold=64, keep_host=True, routed=routed,
                    shared=shared)
    x = synth.hidden(MID, 62, 160)
    x = (x * (10.0 ** rng.integers(-4, 5, size=(160, 1)))).astype(np.float32)
    out = run(L, x, dev)
    assert_routing_matches(L, x, 160)
    ref, _, _ = L.oracle_forward(x)
    assert np.all(np.isfinite(out))
    assert_mfma_close(out, ref, "ranges: ")


def test_mfma_path_no_shared_expert_olmoe(dev):
    """OLMoE-like layer (h 2048, E 64, k 8, I 1024, no shared expert) at
    T = 512 on the MFMA path, outputs of 96 tokens (every 8th, plus the
    last)."""
    log("MFMA path OLMoE-like T=512")
    rows = list(range(0, 512, 8))[:95] + [511]
    check_mfma(synth.OLMOE, 24, 512, dev, threshold=256, rows=rows)


def test_threshold_switch_on_one_handle(dev):
    """One handle: T just below the threshold (GEMV path), at it (MFMA path),
    decode again; each call against the oracle at its own bar."""
    log("GEMV / MFMA switch on one handle")
    L = DeviceLayer(MID, 25, 0, dev, max_tokens=200, prefill_threshold=100, keep_host=True)
    for T in (99, 100, 3, 200):
        x = synth.hidden(MID, 25, T, batch=T)
        out = run(L, x, dev)
        assert_routing_matches(L, x, T)
        ref, _, _ = L.oracle_forward(x)
        if T >= 100:
            assert_mfma_close(out, ref, f"T={T} ")
        else:
            err = rel_err(out, ref)
            log(f"  T={T} rel err {err:.3e}")
            assert err <= TOL_GEMV, (T, err)


# ---------------------------------------------------------------------------
# GLM-5.2-like layer (h=6144, E=256, k=8, I=2048, 1 shared) at full size.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def glm(dev):
    log("building GLM-like layer 0 (5.46 GB of experts)")
    L = DeviceLayer(synth.GLM, 1, 0, dev, max_tokens=4096)
    yield L
    L.close()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T", [1, 2, 4])
def test_glm_decode_full(dev, glm, T):
    log(f"GLM-like decode T={T}")
    x = synth.hidden(synth.GLM, 1, T, batch=100 + T)
    out = run(glm, x, dev)
    assert_routing_matches(glm, x, T)
    ref, _, _ = glm.oracle_forward(x)
    err = rel_err(out, ref)
    log(f"  rel err {err:.3e}")
    assert err <= TOL_GEMV


@pytest.mark.timeout(300)
def test_glm_decode_calls_in_a_row(dev, glm):
    """Single-token and four-token calls alternating on the GLM-like layer,
    each against the oracle."""
    for b, T in enumerate((1, 4, 1)):
        log(f"GLM-like decode T={T}, call {b}")
        x = synth.hidden(synth.GLM, 1, T, batch=300 + b)
        out = run(glm, x, dev)
        assert_routing_matches(glm, x, T)
        ref, _, _ = glm.oracle_forward(x)
        err = rel_err(out, ref)
        log(f"  rel err {err:.3e}")
        assert err <= TOL_GEMV


@pytest.mark.timeout(600)
def test_glm_decode_T64_all_rows(dev, glm):
    T = 64
    log("GLM-like decode T=64, every row against the oracle")
    x = synth.hidden(synth.GLM, 1, T, batch=164)
    out = run(glm, x, dev)
    assert_routing_matches(glm, x, T)
    ref, _, _ = glm.oracle_forward(x)
    err = rel_err(out, ref)
    log(f"  rel err {err:.3e} over {T} rows")
    assert err <= TOL_GEMV


@pytest.mark.timeout(600)
def test_two_resident_glm_layers_on_separate_handles(dev, glm):
    """Layers 0 and 1 of the stack resident at once, each on its own handle:
    single-token and four-token calls alternate between them, each against
    the oracle of its own layer (the benchmark cycles 8 such layers)."""
    log("building GLM-like layer 1 beside layer 0")
    L1 = DeviceLayer(synth.GLM, 1, 1, dev, max_tokens=64)
    try:
        for b, (lay, T) in enumerate(((glm, 1), (L1, 1), (glm, 4), (L1, 4), (L1, 1))):
            log(f"  layer {lay.layer} T={T}")
            x = synth.hidden(synth.GLM, 1, T, layer=lay.layer, batch=500 + b)
            out = run(lay, x, dev)
            assert_routing_matches(lay, x, T)
            ref, _, _ = lay.oracle_forward(x)
            err = rel_err(out, ref)
            log(f"  rel err {err:.3e}")
            assert err <= TOL_GEMV, (lay.layer, T, err)
    finally:
        L1.close()


def prefill_sample_rows(idx: np.ndarray, E: int, n_rows: int, seed: int) -> list:
    """Tokens whose outputs cover every kind of GEMM tile of a prefill call:
    the first and last token of every 128-token tile of the most loaded
    expert, one token of each expert holding at most 32 tokens (one-block
    tiles), the shared expert's last tile (the last tokens), then random
    tokens up to n_rows."""
    T = idx.shape[0]
    counts = np.bincount(idx.reshape(-1), minlength=E)
    head = int(np.argmax(counts))
    on_head = np.nonzero((idx == head).any(axis=1))[0]
    rows = set(int(on_head[i]) for i in range(0, len(on_head), 128))
    rows |= set(int(on_head[min(i + 127, len(on_head) - 1)]) for i in range(0, len(on_head), 128))
    for e in np.nonzero((counts > 0) & (counts <= 32))[0]:
        rows.add(int(np.nonzero((idx == e).any(axis=1))[0][0]))
    rows |= set(range(max(0, T - 8), T)) | {0, 1, T // 2}
    rest = np.random.default_rng(seed).permutation(T)
    for r in rest:
        if len(rows) >= n_rows:
            break
        rows.add(int(r))
    return sorted(rows)


@pytest.mark.timeout(900)
def test_glm_prefill_routing_and_sampled_outputs(dev):
    """T = 4096 on the prefill workload (Zipf-biased selection): routing and
    dispatch bit-exact for every token, outputs of 256 tokens covering every
    tile of the head expert, the one-block tail tiles and the shared
    expert's last tile, element-wise at the MFMA bar."""
    T = 4096
    log("GLM-like prefill T=4096 (Zipf selection bias)")
    L = DeviceLayer(synth.GLM_PREFILL, 1, 0, dev, max_tokens=T)
    x = synth.hidden(synth.GLM_PREFILL, 1, T)
    out = run(L, x, dev)
    idx, _ = assert_routing_matches(L, x, T)
    counts = np.bincount(idx.reshape(-1), minlength=256)
    log(f"  distinct experts {int((counts > 0).sum())}, head load {int(counts.max())}, "
        f"experts with <= 32 tokens {int(((counts > 0) & (counts <= 32)).sum())}")
    rows = prefill_sample_rows(idx, 256, 256, 4096)
    log(f"  oracle on {len(rows)} rows")
    ref, _, _ = L.oracle_forward(x[rows])
    assert_mfma_close(out[rows], ref)
    L.close()
