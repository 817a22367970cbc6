"""GPU: the HBM expert cache with host-RAM backing (coli_moe_cache_*).

A cached layer keeps its routed experts in pinned host memory and copies the
ones a call routes to into a few HBM slots.  It must compute exactly what the
fully resident layer computes: every output bit for bit equal to
coli_moe_forward on the same layer and input, routing bit-exact against the
oracle, and outputs within the GEMV bar (2e-3) of the oracle, through calls
that miss, hit, evict and prefetch.  The counters must add up.

Router look-ahead prefetch (PILOT) is exercised on two layers whose inputs
are correlated the way consecutive layers of a residual stream are (the
second input is the first plus a small update): the second layer's router
applied to the first input predicts most of its experts."""
import numpy as np
import pytest

import synth
from tests.gpu_util import DeviceLayer, assert_routing_matches, log, rel_err, routing_from_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL_GEMV = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make_cache(L: DeviceLayer, n_slots: int, repin_every: int = 0):
    """A cache over the same tables as DeviceLayer L (its routed experts
    copied to pinned host memory)."""
    import routed_expert_ffn_f32_amd as cm
    host = {k: torch.from_numpy(np.ascontiguousarray(v)).pin_memory() for k, v in L.host_routed.items()}
    resident = {k: v for k, v in L.tensors.items() if k in ("router_w", "sel_bias") or k.startswith("sh_")}
    return cm.ExpertCache(L.moe.cfg, resident, host, n_slots, repin_every=repin_every)


def run_both(L: DeviceLayer, C, x: np.ndarray, dev):
    xd = torch.from_numpy(x).to(dev)
    a = L.moe(xd)
    b = C(xd)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def check_cache_routing(C, L: DeviceLayer, x: np.ndarray):
    import oracle
    T, r = C.last_routing()
    torch.cuda.synchronize()
    g = routing_from_device(r, T, L.shape.top_k)
    idx, w = oracle.route(L.shape, L.wr, L.bias, x)
    assert np.array_equal(g["idx"], idx) and np.array_equal(g["w"].view(np.uint32), w.view(np.uint32))
    d = oracle.dispatch(idx, L.shape.n_experts)
    for key in ("offsets", "sorted_ids", "inv", "active"):
        assert np.array_equal(g[key], d[key]), key


SMALL = synth.LayerShape(hidden=256, n_experts=32, top_k=2, inter=128, n_shared=1, rsf=2.5, bias_sigma=0.05)
# calls of 16 tokens and more take the matrix-core batch kernels, here on
# cache slots.  A cache holds at least max_tokens * top_k slots (40 here);
# these six calls route to 8 to 25 distinct experts each and 48 in all, so
# the 40 slots fill and then evict
BATCH = synth.LayerShape(hidden=512, n_experts=64, top_k=2, inter=256, n_shared=1, rsf=2.5, bias_sigma=0.05)


@pytest.mark.parametrize("name,shape,max_t,n_slots,Ts", [
    ("olmoe", synth.OLMOE, 2, 20, (1, 2, 1, 1, 2, 1, 2, 2, 1, 1, 2, 1)),
    ("small_shared", SMALL, 6, 14, (3, 6, 1, 4, 5, 6, 2, 1, 3, 6)),
    ("batch_mfma", BATCH, 20, 40, (16, 20, 17, 5, 18, 16))])
def test_cache_matches_resident_layer(dev, name, shape, max_t, n_slots, Ts):
    """Every call bit-identical to the resident layer (small-batch and
    larger-batch launch structures both run, the latter on the GEMV and on
    the matrix-core kernels), routing bit-exact, outputs against the oracle,
    counters consistent."""
    log(f"expert cache {name}: {shape.n_experts} experts in host memory, {n_slots} HBM slots")
    L = DeviceLayer(shape, 17, 0, dev, max_tokens=max_t, keep_host=True)
    C = make_cache(L, n_slots)
    try:
        needed = 0
        for b, T in enumerate(Ts):
            x = synth.hidden(shape, 17, T, batch=700 + b)
            want, got = run_both(L, C, x, dev)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (b, T)
            check_cache_routing(C, L, x)
            needed += len(np.unique(L.oracle_route(x)))
            if b % 3 == 0:
                ref, _, _ = L.oracle_forward(x)
                err = rel_err(got, ref)
                log(f"  call {b} T={T}: rel err {err:.3e}")
                assert err <= TOL_GEMV
        st = C.stats()
        log(f"  stats {st}")
        assert st["calls"] == len(Ts) and st["needed"] == needed
        assert st["hits"] + st["misses"] == st["needed"]
        assert 0 < st["misses"] < st["needed"] and st["resident"] == n_slots
        eb = shape.expert_bytes
        assert st["bytes_copied"] == st["misses"] * eb
        assert sum(C.usage()) == sum(T * shape.top_k for T in Ts)
        slots = C.slot_map()
        used = [s for s in slots if s >= 0]
        assert len(used) == n_slots and len(set(used)) == n_slots
    finally:
        C.close()
        L.close()


def test_cache_pins_and_repin(dev):
    """Pinned experts stay resident through calls that miss; re-pinning
    (every 2 calls) swaps pins towards the hot experts and never loses
    residency of a pinned one; outputs stay bit-identical."""
    shape = SMALL
    L = DeviceLayer(shape, 18, 0, dev, max_tokens=2, keep_host=True)
    C = make_cache(L, 8, repin_every=2)
    try:
        assert C.pin([5, 6, 7, 8]) == 4  # budget 8 - min(32, 2 * 2) = 4
        assert C.pin([9]) == 0
        for b in range(12):
            T = 1 + b % 2
            x = synth.hidden(shape, 18, T, batch=800 + b)
            want, got = run_both(L, C, x, dev)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), b
        st = C.stats()
        log(f"  stats {st}")
        assert st["pinned"] == 4 and st["resident"] == 8
    finally:
        C.close()
        L.close()


def test_cache_router_lookahead_prefetch(dev):
    """PILOT on two OLMoE-like layers: before layer 0 runs on x0, layer 1's
    experts are predicted with layer 1's router on x0 and copied ahead;
    layer 1 then runs on x1 = x0 + 0.2 N(0,1).  Outputs bit-identical to the
    resident layers, and most of layer 1's experts found prefetched."""
    shape = synth.OLMOE
    L0 = DeviceLayer(shape, 19, 0, dev, max_tokens=1, keep_host=True)
    L1 = DeviceLayer(shape, 19, 1, dev, max_tokens=1, keep_host=True)
    C0, C1 = make_cache(L0, 16), make_cache(L1, 16)
    rng = np.random.default_rng(19)
    try:
        for b in range(16):
            x0 = synth.hidden(shape, 19, 1, batch=900 + b)
            x1 = (x0 + 0.2 * rng.standard_normal(x0.shape)).astype(np.float32)
            d0 = torch.from_numpy(x0).to(dev)
            C1.prefetch(d0, 8)
            want0, got0 = run_both(L0, C0, x0, dev)
            want1, got1 = run_both(L1, C1, x1, dev)
            assert np.array_equal(got0.view(np.uint32), want0.view(np.uint32))
            assert np.array_equal(got1.view(np.uint32), want1.view(np.uint32))
        st = C1.stats()
        log(f"  layer 1 stats {st}; prefetch recall {st['prefetch_hits'] / st['needed']:.3f}")
        assert st["prefetched"] > 0 and st["prefetch_hits"] > 0
        assert st["prefetch_hits"] <= st["prefetched"] and st["hits"] + st["misses"] == st["needed"]
    finally:
        C0.close()
        C1.close()
        L0.close()
        L1.close()
