"""Python binding of libcoli_moe, the gfx950 routed-MoE layer library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels (include/coli_moe.h documents the C ABI).  The functions keep the C
names; pointers are passed as integers (device addresses, e.g. a torch
tensor's data_ptr()) and streams as integer hipStream_t handles (e.g.
torch.cuda.current_stream().cuda_stream).  Non-zero return codes raise
ColiMoeError.

`MoELayer` is a convenience wrapper that uses PyTorch for what PyTorch is
here for: device memory (weights, workspace, outputs) and streams.

There is no fallback: if the library is not built, importing works but the
first call raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build (routed_expert_ffn_f32_amd/build.py), and only that.
LIB_PATH = os.path.join(_HERE, "_lib", "libcoli_moe.so")

COLI_MOE_OK = 0
COLI_MOE_ECAPACITY = -1
COLI_MOE_EROUTING = -2
COLI_MOE_EDEVICE = -3
COLI_MOE_EARG = -4
COLI_MOE_N_KERNELS = 10
COLI_MOE_STATIC_SCRATCH_BYTES = 64 << 20
COLI_MOE_DEFAULT_SPIN_LIMIT = 1 << 22


class ColiMoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: error {code} ({coli_moe_error_string(code)})")


class coli_moe_config_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("prefill_threshold", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("weight_format", ctypes.c_int32)]


class coli_moe_weights_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "sel_bias", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
        "sh_gate_q", "sh_gate_s", "sh_up_q", "sh_up_s", "sh_down_q", "sh_down_s")]


class coli_moe_host_experts_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


class coli_moe_cache_config_t(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("repin_every", ctypes.c_int32), ("decay", ctypes.c_float)]


class coli_moe_cache_stats_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("calls", "needed", "hits", "misses", "prefetched", "prefetch_hits",
                                               "evictions", "repin_swaps", "bytes_copied")] + \
               [("pinned", ctypes.c_int32), ("resident", ctypes.c_int32)]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


def load_library():
    """Load the built library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m routed_expert_ffn_f32_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp, wp = ctypes.POINTER(coli_moe_config_t), ctypes.POINTER(coli_moe_weights_t)
        L.coli_moe_workspace_bytes.argtypes = [cfgp]
        L.coli_moe_workspace_bytes.restype = sz
        L.coli_moe_init.argtypes = [ctypes.POINTER(vp), cfgp, wp, vp, sz, vp]
        L.coli_moe_init.restype = ctypes.c_int
        L.coli_moe_forward.argtypes = [vp, vp, vp, i32, vp]
        L.coli_moe_forward.restype = ctypes.c_int
        L.coli_moe_forward_noalloc.argtypes = [cfgp, wp, vp, vp, i32, vp]
        L.coli_moe_forward_noalloc.restype = ctypes.c_int
        L.coli_moe_free.argtypes = [vp]
        L.coli_moe_free.restype = None
        L.coli_moe_set_routing.argtypes = [vp, i32, ctypes.c_float]
        L.coli_moe_set_routing.restype = ctypes.c_int
        L.coli_moe_last_routing.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.coli_moe_last_routing.restype = ctypes.c_int
        L.coli_moe_status.argtypes = [vp, vp]
        L.coli_moe_status.restype = ctypes.c_int
        L.coli_moe_test_spin_limit.argtypes = [vp, i32]
        L.coli_moe_test_spin_limit.restype = ctypes.c_int
        L.coli_moe_test_batch_kernels.argtypes = [vp, i32]
        L.coli_moe_test_batch_kernels.restype = ctypes.c_int
        L.coli_moe_test_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.coli_moe_test_dispatch.restype = ctypes.c_int
        L.coli_moe_probe_read.argtypes = [vp, vp, i32, vp]
        L.coli_moe_probe_read.restype = ctypes.c_int
        L.coli_moe_probe_read_down.argtypes = [vp, vp, i32, vp]
        L.coli_moe_probe_read_down.restype = ctypes.c_int
        L.coli_moe_probe_stream.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.coli_moe_probe_stream.restype = ctypes.c_int
        L.coli_moe_probe_mfma.argtypes = [i32, i32, vp, vp]
        L.coli_moe_probe_mfma.restype = ctypes.c_int
        L.coli_moe_probe_mfma_f16.argtypes = [i32, i32, ctypes.c_uint32, vp, vp]
        L.coli_moe_probe_mfma_f16.restype = ctypes.c_int
        L.coli_moe_profile_begin.argtypes = [vp, i32]
        L.coli_moe_profile_begin.restype = ctypes.c_int
        L.coli_moe_profile_end.argtypes = [vp, vp, vp]
        L.coli_moe_profile_end.restype = ctypes.c_int
        L.coli_moe_kernel_name.argtypes = [i32]
        L.coli_moe_kernel_name.restype = ctypes.c_char_p
        L.coli_moe_error_string.argtypes = [i32]
        L.coli_moe_error_string.restype = ctypes.c_char_p
        hp, ccp = ctypes.POINTER(coli_moe_host_experts_t), ctypes.POINTER(coli_moe_cache_config_t)
        L.coli_moe_cache_slot_bytes.argtypes = [cfgp, i32]
        L.coli_moe_cache_slot_bytes.restype = sz
        L.coli_moe_cache_init.argtypes = [ctypes.POINTER(vp), cfgp, ccp, wp, hp, vp, sz, vp, sz, vp]
        L.coli_moe_cache_init.restype = ctypes.c_int
        L.coli_moe_cache_forward.argtypes = [vp, vp, vp, i32, vp]
        L.coli_moe_cache_forward.restype = ctypes.c_int
        L.coli_moe_cache_prefetch.argtypes = [vp, vp, i32, i32, vp]
        L.coli_moe_cache_prefetch.restype = ctypes.c_int
        L.coli_moe_cache_pin.argtypes = [vp, vp, i32, vp]
        L.coli_moe_cache_pin.restype = ctypes.c_int
        L.coli_moe_cache_stats.argtypes = [vp, ctypes.POINTER(coli_moe_cache_stats_t)]
        L.coli_moe_cache_stats.restype = ctypes.c_int
        L.coli_moe_cache_usage.argtypes = [vp, vp]
        L.coli_moe_cache_usage.restype = ctypes.c_int
        L.coli_moe_cache_slots.argtypes = [vp, vp]
        L.coli_moe_cache_slots.restype = ctypes.c_int
        L.coli_moe_cache_layer.argtypes = [vp]
        L.coli_moe_cache_layer.restype = vp
        L.coli_moe_cache_free.argtypes = [vp]
        L.coli_moe_cache_free.restype = None
        L.coli_moe_usage_engine_id.argtypes = []
        L.coli_moe_usage_engine_id.restype = ctypes.c_uint32
        L.coli_moe_usage_write.argtypes = [ctypes.c_char_p, i32, i32, vp]
        L.coli_moe_usage_write.restype = ctypes.c_int
        L.coli_moe_usage_read.argtypes = [ctypes.c_char_p, i32, i32, vp]
        L.coli_moe_usage_read.restype = ctypes.c_int
        L.coli_moe_test_cache_policy.argtypes = [i32, i32, i32, ctypes.c_float, i32, vp, i32, vp, vp, i32, vp, vp]
        L.coli_moe_test_cache_policy.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise ColiMoeError(rc, where)
    return rc


def coli_moe_error_string(code: int) -> str:
    return load_library().coli_moe_error_string(int(code)).decode()


def coli_moe_kernel_name(i: int) -> str:
    return load_library().coli_moe_kernel_name(int(i)).decode()


def coli_moe_workspace_bytes(cfg: coli_moe_config_t) -> int:
    return int(load_library().coli_moe_workspace_bytes(ctypes.byref(cfg)))


def coli_moe_init(cfg: coli_moe_config_t, weights: coli_moe_weights_t, workspace: int,
                  workspace_bytes: int, stream: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().coli_moe_init(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(weights),
                                        workspace, workspace_bytes, stream), "coli_moe_init")
    return h


def coli_moe_forward(handle, hidden: int, out: int, T: int, stream: int = 0) -> int:
    return _check(load_library().coli_moe_forward(handle, hidden, out, int(T), stream), "coli_moe_forward")


def coli_moe_forward_noalloc(cfg: coli_moe_config_t, weights: coli_moe_weights_t, hidden: int, out: int, T: int,
                             stream: int = 0) -> int:
    """The forward without handle or workspace: the library's own device
    array (COLI_MOE_STATIC_SCRATCH_BYTES per device) is the workspace."""
    return _check(load_library().coli_moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), hidden, out,
                                                          int(T), stream), "coli_moe_forward_noalloc")


def coli_moe_free(handle) -> None:
    load_library().coli_moe_free(handle)


def coli_moe_set_routing(handle, k_use: int, top_p: float = 1.0) -> int:
    """Run-time routing limits (explicit smaller k, adaptive expert top-p) of
    the handle's later forwards; (top_k, 1.0) is the plain routing."""
    return _check(load_library().coli_moe_set_routing(handle, int(k_use), float(top_p)), "coli_moe_set_routing")


def _warn_lossy(k_use: int, top_k: int, top_p: float) -> None:
    if k_use < top_k or top_p < 1.0:
        import warnings
        warnings.warn(f"lossy routing override: k {k_use} of {top_k}, expert top-p {top_p}: outputs differ from the "
                      f"layer's plain routing", stacklevel=3)


def coli_moe_last_routing(handle, idx=None, w=None, offsets=None, sorted_ids=None, inv=None,
                          active=None, n_active=None, stream: int = 0) -> int:
    return _check(load_library().coli_moe_last_routing(handle, idx, w, offsets, sorted_ids, inv, active,
                                                       n_active, stream), "coli_moe_last_routing")


def coli_moe_test_dispatch(idx: int, T: int, k: int, E: int, offsets: int, sorted_ids: int, inv: int,
                           active: int, n_active: int, stream: int = 0) -> int:
    return _check(load_library().coli_moe_test_dispatch(idx, int(T), int(k), int(E), offsets, sorted_ids,
                                                        inv, active, n_active, stream),
                  "coli_moe_test_dispatch")


def coli_moe_probe_read(handle, experts: int, n: int, stream: int = 0) -> int:
    """Pure-load probe of the gate/up rows of n experts (device int32 ids, -1
    = shared): the read ceiling of the gate/up access pattern."""
    return _check(load_library().coli_moe_probe_read(handle, experts, int(n), stream), "coli_moe_probe_read")


def coli_moe_probe_read_down(handle, experts: int, n: int, stream: int = 0) -> int:
    """Pure-load probe of the down rows of n experts with the one-token down +
    combine launch's grid: the read ceiling of that access pattern."""
    return _check(load_library().coli_moe_probe_read_down(handle, experts, int(n), stream),
                  "coli_moe_probe_read_down")


def coli_moe_probe_stream(buf: int, nbytes: int, sink: int, stream: int = 0) -> int:
    """XOR of every 32-bit word of a device buffer into the device word at
    sink, each byte read once (the HBM read rate of this GPU)."""
    return _check(load_library().coli_moe_probe_stream(buf, int(nbytes), sink, stream), "coli_moe_probe_stream")


MFMA_PROBE_MFMAS_PER_ROUND = 8


def coli_moe_probe_mfma(iters: int, blocks: int, sink: int, stream: int = 0) -> int:
    """blocks x 4 waves of iters x 8 back-to-back bf16 MFMAs (32768 flops
    each); each wave whose results check adds 1 to the device word at sink."""
    return _check(load_library().coli_moe_probe_mfma(int(iters), int(blocks), sink, stream), "coli_moe_probe_mfma")


MFMA_F16_PROBE_MFMAS_PER_ROUND = 16


def coli_moe_probe_mfma_f16(iters: int, blocks: int, seed: int, sink: int, stream: int = 0) -> int:
    """blocks x 4 waves of iters x 16 back-to-back f16 MFMAs on operands that
    change from one MFMA to the next; each wave whose accumulators are all
    finite adds 1 to the device word at sink."""
    return _check(load_library().coli_moe_probe_mfma_f16(int(iters), int(blocks), int(seed) & 0xFFFFFFFF, sink, stream),
                  "coli_moe_probe_mfma_f16")


def coli_moe_profile_begin(handle, max_calls: int) -> int:
    return _check(load_library().coli_moe_profile_begin(handle, int(max_calls)), "coli_moe_profile_begin")


def coli_moe_profile_end(handle):
    """Returns (calls, {kernel name: (total ms, launches)})."""
    ms = (ctypes.c_float * COLI_MOE_N_KERNELS)()
    n = (ctypes.c_int32 * COLI_MOE_N_KERNELS)()
    calls = _check(load_library().coli_moe_profile_end(handle, ms, n), "coli_moe_profile_end")
    return calls, {coli_moe_kernel_name(i): (float(ms[i]), int(n[i])) for i in range(COLI_MOE_N_KERNELS)}


def coli_moe_cache_slot_bytes(cfg: coli_moe_config_t, n_slots: int) -> int:
    return int(load_library().coli_moe_cache_slot_bytes(ctypes.byref(cfg), int(n_slots)))


def coli_moe_cache_init(cfg, cache_cfg, resident, host, slots: int, slot_bytes: int, workspace: int,
                        workspace_bytes: int, stream: int = 0):
    h = ctypes.c_void_p()
    _check(load_library().coli_moe_cache_init(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(cache_cfg),
                                              ctypes.byref(resident), ctypes.byref(host), slots, slot_bytes,
                                              workspace, workspace_bytes, stream), "coli_moe_cache_init")
    return h


def coli_moe_cache_forward(cache, hidden: int, out: int, T: int, stream: int = 0) -> int:
    return _check(load_library().coli_moe_cache_forward(cache, hidden, out, int(T), stream), "coli_moe_cache_forward")


def coli_moe_cache_prefetch(cache, hidden: int, T: int, n_predict: int, stream: int = 0) -> int:
    return _check(load_library().coli_moe_cache_prefetch(cache, hidden, int(T), int(n_predict), stream),
                  "coli_moe_cache_prefetch")


def coli_moe_cache_pin(cache, experts, stream: int = 0) -> int:
    arr = (ctypes.c_int32 * len(experts))(*[int(e) for e in experts])
    return _check(load_library().coli_moe_cache_pin(cache, arr, len(experts), stream), "coli_moe_cache_pin")


def coli_moe_cache_stats(cache) -> dict:
    st = coli_moe_cache_stats_t()
    _check(load_library().coli_moe_cache_stats(cache, ctypes.byref(st)), "coli_moe_cache_stats")
    return st.as_dict()


def coli_moe_cache_usage(cache, n_experts: int):
    arr = (ctypes.c_int64 * n_experts)()
    _check(load_library().coli_moe_cache_usage(cache, arr), "coli_moe_cache_usage")
    return [int(v) for v in arr]


def coli_moe_cache_slots(cache, n_experts: int):
    arr = (ctypes.c_int32 * n_experts)()
    _check(load_library().coli_moe_cache_slots(cache, arr), "coli_moe_cache_slots")
    return [int(v) for v in arr]


def coli_moe_cache_layer(cache):
    return load_library().coli_moe_cache_layer(cache)


def coli_moe_cache_free(cache) -> None:
    load_library().coli_moe_cache_free(cache)


def coli_moe_usage_engine_id() -> int:
    return int(load_library().coli_moe_usage_engine_id())


def coli_moe_usage_write(path: str, counts) -> int:
    """counts: int64 array [n_layers][n_experts] (numpy)."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.int64)
    return _check(load_library().coli_moe_usage_write(path.encode(), c.shape[0], c.shape[1], c.ctypes.data),
                  "coli_moe_usage_write")


def coli_moe_usage_read(path: str, n_layers: int, n_experts: int):
    """Returns (records, counts int64 [n_layers][n_experts])."""
    import numpy as np
    c = np.zeros((n_layers, n_experts), np.int64)
    n = _check(load_library().coli_moe_usage_read(path.encode(), n_layers, n_experts, c.ctypes.data),
               "coli_moe_usage_read")
    return n, c


def coli_moe_test_cache_policy(n_experts, n_slots, reserve, decay, repin_every, pins, calls):
    """The residency policy alone; `calls` is a list of expert lists.
    Returns (repin swaps, misses per call, final slot per expert)."""
    flat = [int(e) for c in calls for e in c]
    lens = [len(c) for c in calls]
    pa = (ctypes.c_int32 * max(1, len(pins)))(*[int(e) for e in pins])
    ca = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    la = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    miss = (ctypes.c_int32 * max(1, len(calls)))()
    slots = (ctypes.c_int32 * n_experts)()
    rc = _check(load_library().coli_moe_test_cache_policy(n_experts, n_slots, reserve, decay, repin_every, pa,
                                                          len(pins), ca, la, len(calls), miss, slots),
                "coli_moe_test_cache_policy")
    return rc, [int(miss[i]) for i in range(len(calls))], [int(v) for v in slots]


# ---------------------------------------------------------------------------
# Convenience wrapper over torch device tensors.
# ---------------------------------------------------------------------------

_WEIGHT_KEYS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


COLI_MOE_WEIGHTS_INT4_GS64 = 0
COLI_MOE_WEIGHTS_INT8_ROW = 1


def make_config(hidden, n_experts, top_k, inter, n_shared, routed_scaling_factor, max_tokens,
                prefill_threshold=0, group_size=None, n_group=1,
                weight_format=COLI_MOE_WEIGHTS_INT4_GS64) -> coli_moe_config_t:
    if group_size is None:
        group_size = 0 if weight_format == COLI_MOE_WEIGHTS_INT8_ROW else 64
    return coli_moe_config_t(hidden=hidden, n_experts=n_experts, top_k=top_k, inter=inter, n_shared=n_shared,
                             group_size=group_size, n_group=n_group, max_tokens=max_tokens,
                             prefill_threshold=prefill_threshold,
                             routed_scaling_factor=routed_scaling_factor, weight_format=weight_format)


class MoELayer:
    """One layer on the current torch device.

    `tensors` maps names to device tensors: router_w [h,E] f32, sel_bias [E]
    f32 (optional), gate_q/up_q [E,I,h/2] u8, gate_s/up_s [E,I,h/64] f32,
    down_q [E,h,I/2] u8, down_s [E,h,I/64] f32, and sh_* for the shared
    expert.  The tensors are borrowed: keep them alive with the layer.
    """

    def __init__(self, cfg: coli_moe_config_t, tensors: dict, stream: int | None = None):
        import torch
        self.cfg = cfg
        self.tensors = tensors
        w = coli_moe_weights_t()
        for name, _ in coli_moe_weights_t._fields_:
            t = tensors.get(name)
            setattr(w, name, None if t is None else t.data_ptr())
        self.weights = w
        nbytes = coli_moe_workspace_bytes(cfg)
        if nbytes == 0:
            raise ColiMoeError(COLI_MOE_EARG, "coli_moe_workspace_bytes")
        dev = tensors["router_w"].device
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
        self.handle = coli_moe_init(cfg, w, self.workspace.data_ptr(), nbytes, self.stream)

    def forward(self, hidden, out=None):
        import torch
        T = hidden.shape[0]
        if out is None:
            out = torch.empty_like(hidden)
        coli_moe_forward(self.handle, hidden.data_ptr(), out.data_ptr(), T, self.stream)
        return out

    __call__ = forward

    def set_routing(self, k_use: int | None = None, top_p: float = 1.0):
        """Lossy run-time routing limits for later forwards (warns when they
        change the routing); no arguments restore the plain routing."""
        k_use = self.cfg.top_k if k_use is None else int(k_use)
        coli_moe_set_routing(self.handle, k_use, top_p)
        _warn_lossy(k_use, self.cfg.top_k, top_p)

    def status(self) -> int:
        """Waits for the layer's stream; COLI_MOE_OK unless a launch since the
        last check gave up its bounded wait (COLI_MOE_EDEVICE).  Clears the
        error word."""
        return int(load_library().coli_moe_status(self.handle, ctypes.c_void_p(self.stream)))

    def last_routing(self):
        """Device tensors of the last forward's routing and dispatch."""
        import torch
        dev = self.workspace.device
        T, k, E = None, self.cfg.top_k, self.cfg.n_experts
        T = coli_moe_last_routing(self.handle, stream=self.stream)
        n = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        r = dict(idx=torch.empty(n, **i32), w=torch.empty(n, dtype=torch.float32, device=dev),
                 offsets=torch.empty(E + 1, **i32), sorted_ids=torch.empty(n, **i32),
                 inv=torch.empty(n, **i32), active=torch.empty(E, **i32), n_active=torch.empty(1, **i32))
        coli_moe_last_routing(self.handle, *(r[key].data_ptr() for key in
                                             ("idx", "w", "offsets", "sorted_ids", "inv", "active",
                                              "n_active")), stream=self.stream)
        return T, r

    def close(self):
        if getattr(self, "handle", None) is not None:
            coli_moe_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """One layer whose routed experts live in pinned host memory, copied on
    demand into `n_slots` HBM slots (torch device tensors hold the slots and
    the workspace).  `resident` maps router_w, sel_bias and sh_* to device
    tensors; `host` maps gate_q ... down_s to pinned host tensors."""

    def __init__(self, cfg: coli_moe_config_t, resident: dict, host: dict, n_slots: int, repin_every: int = 0,
                 decay: float = 0.0, stream: int | None = None):
        import torch
        self.cfg, self.resident, self.host = cfg, resident, host
        dev = resident["router_w"].device
        w = coli_moe_weights_t()
        for name, _ in coli_moe_weights_t._fields_:
            t = resident.get(name)
            setattr(w, name, None if t is None else t.data_ptr())
        hx = coli_moe_host_experts_t()
        for name, _ in coli_moe_host_experts_t._fields_:
            setattr(hx, name, host[name].data_ptr())
        self.weights, self.hx = w, hx
        sb = coli_moe_cache_slot_bytes(cfg, n_slots)
        wb = coli_moe_workspace_bytes(cfg)
        if sb == 0 or wb == 0:
            raise ColiMoeError(COLI_MOE_EARG, "coli_moe_cache_slot_bytes")
        self.slots = torch.empty(sb, dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
        cc = coli_moe_cache_config_t(n_slots=n_slots, repin_every=repin_every, decay=decay)
        self.handle = coli_moe_cache_init(cfg, cc, w, hx, self.slots.data_ptr(), sb, self.workspace.data_ptr(), wb,
                                          self.stream)

    def forward(self, hidden, out=None):
        import torch
        if out is None:
            out = torch.empty_like(hidden)
        coli_moe_cache_forward(self.handle, hidden.data_ptr(), out.data_ptr(), hidden.shape[0], self.stream)
        return out

    __call__ = forward

    def prefetch(self, hidden, n_predict: int):
        return coli_moe_cache_prefetch(self.handle, hidden.data_ptr(), hidden.shape[0], n_predict, self.stream)

    def pin(self, experts):
        return coli_moe_cache_pin(self.handle, experts, self.stream)

    def stats(self) -> dict:
        return coli_moe_cache_stats(self.handle)

    def usage(self):
        return coli_moe_cache_usage(self.handle, self.cfg.n_experts)

    def slot_map(self):
        return coli_moe_cache_slots(self.handle, self.cfg.n_experts)

    def set_routing(self, k_use: int | None = None, top_p: float = 1.0):
        """Lossy run-time routing limits of the cached layer (see
        MoELayer.set_routing)."""
        k_use = self.cfg.top_k if k_use is None else int(k_use)
        coli_moe_set_routing(coli_moe_cache_layer(self.handle), k_use, top_p)
        _warn_lossy(k_use, self.cfg.top_k, top_p)

    def last_routing(self):
        """Device tensors of the last forward's routing and dispatch."""
        import torch
        layer = coli_moe_cache_layer(self.handle)
        dev = self.workspace.device
        k, E = self.cfg.top_k, self.cfg.n_experts
        T = coli_moe_last_routing(layer, stream=self.stream)
        n = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        r = dict(idx=torch.empty(n, **i32), w=torch.empty(n, dtype=torch.float32, device=dev),
                 offsets=torch.empty(E + 1, **i32), sorted_ids=torch.empty(n, **i32),
                 inv=torch.empty(n, **i32), active=torch.empty(E, **i32), n_active=torch.empty(1, **i32))
        coli_moe_last_routing(layer, *(r[key].data_ptr() for key in
                                       ("idx", "w", "offsets", "sorted_ids", "inv", "active", "n_active")),
                              stream=self.stream)
        return T, r

    def close(self):
        if getattr(self, "handle", None) is not None:
            coli_moe_cache_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
