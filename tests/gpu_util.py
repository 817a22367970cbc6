"""Helpers of the GPU tests: build a layer on the device from the seeded
generator, and compute oracle references for all or some tokens.

The oracle reads only host arrays that the generator wrote (or regenerates
single experts from their seeds); nothing it reads comes from the GPU."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import routed_expert_ffn_f32_amd as cm
import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arrays: dict, dev, prefix: str = "") -> dict:
    import torch
    return {prefix + k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in arrays.items()}


class DeviceLayer:
    """Layer `layer` of `shape` from seed `seed`, resident on `dev`.

    Keeps the router and bias on the host (small); routed experts are
    regenerated from their seeds when the oracle needs them, unless
    keep_host=True."""

    def __init__(self, shape: synth.LayerShape, seed: int, layer: int, dev, max_tokens: int,
                 prefill_threshold: int = 0, keep_host: bool = False, routed=None, shared=None,
                 wr=None, bias=None):
        import torch
        self.shape, self.seed, self.layer = shape, seed, layer
        if wr is None:
            wr, bias = synth.router(shape, seed, layer)
        self.wr, self.bias = wr, bias
        if routed is None:
            routed = synth.routed_tables(shape, seed, layer)
        if shared is None and shape.n_shared:
            shared = synth.shared_tables(shape, seed, layer)
        self.host_routed = routed if keep_host else None
        self.host_shared = shared
        t = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(bias).to(dev)}
        t.update(to_device(routed, dev))
        if shared is not None:
            t.update(to_device(shared, dev, "sh_"))
        self.tensors = t
        cfg = cm.make_config(hidden=shape.hidden, n_experts=shape.n_experts, top_k=shape.top_k,
                             inter=shape.inter, n_shared=shape.n_shared,
                             routed_scaling_factor=shape.rsf, max_tokens=max_tokens,
                             prefill_threshold=prefill_threshold, weight_format=shape.weight_format)
        self.moe = cm.MoELayer(cfg, t)
        self.limits = {}  # run-time routing limits of the oracle calls (k_use, top_p)

    def set_routing(self, k_use: int | None = None, top_p: float = 1.0):
        """Routing limits on the device layer and in the oracle calls."""
        import warnings
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            self.moe.set_routing(k_use, top_p)
        self.limits = {} if (k_use in (None, self.shape.top_k) and top_p == 1.0) else dict(k_use=k_use, top_p=top_p)

    def routed_for(self, experts) -> list:
        E = self.shape.n_experts
        if self.host_routed is not None:
            return [{k: v[e] for k, v in self.host_routed.items()} if e in experts else None for e in range(E)]
        return [synth.expert(self.shape, self.seed, e, self.layer) if e in experts else None for e in range(E)]

    def oracle_route(self, x_rows: np.ndarray) -> np.ndarray:
        idx, _ = oracle.route(self.shape, self.wr, self.bias, x_rows, **self.limits)
        return idx

    def oracle_forward(self, x_rows: np.ndarray):
        idx, _ = oracle.route(self.shape, self.wr, self.bias, x_rows, **self.limits)
        needed = set(int(e) for e in np.unique(idx) if e >= 0)
        return oracle.forward(self.shape, self.wr, self.bias, self.routed_for(needed), self.host_shared, x_rows,
                              **self.limits)

    def close(self):
        self.moe.close()
        self.tensors = None


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over (t, i) of |got - ref| / max(|ref|, rms(ref[t])): element-wise
    relative error, floored at the row RMS so near-zero outputs cannot blow
    it up."""
    ref64 = np.asarray(ref, np.float64)
    got64 = np.asarray(got, np.float64)
    rms = np.sqrt((ref64 ** 2).mean(axis=-1, keepdims=True))
    den = np.maximum(np.abs(ref64), rms)
    return float((np.abs(got64 - ref64) / den).max())


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over tokens t of ||got[t] - ref[t]||_2 / ||ref[t]||_2."""
    ref64 = np.asarray(ref, np.float64)
    got64 = np.asarray(got, np.float64)
    return float((np.linalg.norm(got64 - ref64, axis=-1) / np.linalg.norm(ref64, axis=-1)).max())


def routing_from_device(r: dict, T: int, k: int):
    f = {key: v.cpu().numpy() for key, v in r.items()}
    n_active = int(f["n_active"][0])
    return dict(idx=f["idx"].reshape(T, k), w=f["w"].reshape(T, k), offsets=f["offsets"],
                sorted_ids=f["sorted_ids"], inv=f["inv"], active=f["active"][:n_active], n_active=n_active)


def assert_routing_matches(layer: DeviceLayer, x: np.ndarray, T: int):
    """idx, w, offsets, sorted_ids, inv, active bit-exact against the oracle."""
    import torch
    torch.cuda.synchronize()
    Tr, r = layer.moe.last_routing()
    torch.cuda.synchronize()
    assert Tr == T
    g = routing_from_device(r, T, layer.shape.top_k)
    idx_o, w_o = oracle.route(layer.shape, layer.wr, layer.bias, x, **layer.limits)
    assert np.array_equal(g["idx"], idx_o), "expert indices differ"
    assert np.array_equal(g["w"].view(np.uint32), w_o.view(np.uint32)), "routing weights differ"
    d = oracle.dispatch(idx_o, layer.shape.n_experts)
    for key in ("offsets", "sorted_ids", "inv", "active"):
        assert np.array_equal(g[key], d[key]), key
    assert g["n_active"] == d["n_active"]
    return idx_o, w_o
