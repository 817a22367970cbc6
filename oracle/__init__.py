"""CPU ORACLE for the routed Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import this package.  The product library
(routed_expert_ffn_f32_amd) never imports it, links it or falls back to it.

This module is argument marshalling around coli_oracle.c, which holds the
oracle's arithmetic (plain C, float32 exact routing program, float64 FFN and
combine; the page citations and readings are in that file's header).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")


def build(force: bool = True) -> str:
    """Compile coli_oracle.c into _oracle.so with gcc (no contraction, no
    fast-math, OpenMP over independent tokens and assignments)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-math-errno", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Expert(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("router_w", ctypes.c_void_p), ("sel_bias", ctypes.c_void_p),
                ("experts", ctypes.POINTER(Expert)), ("weight_format", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i32, f32, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.coli_oracle_exp_spec.argtypes = [f32]
        L.coli_oracle_exp_spec.restype = f32
        L.coli_oracle_sigmoid_spec.argtypes = [f32]
        L.coli_oracle_sigmoid_spec.restype = f32
        L.coli_oracle_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
        L.coli_oracle_router_logits.restype = i32
        L.coli_oracle_select.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp]
        L.coli_oracle_select.restype = i32
        L.coli_oracle_select_limited.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, vp, vp]
        L.coli_oracle_select_limited.restype = i32
        L.coli_oracle_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.coli_oracle_dispatch.restype = i32
        L.coli_oracle_unpack_code.argtypes = [vp, i32]
        L.coli_oracle_unpack_code.restype = i32
        L.coli_oracle_expert_ffn.argtypes = [ctypes.POINTER(Expert), i32, i32, vp, vp]
        L.coli_oracle_expert_ffn.restype = None
        L.coli_oracle_expert_ffn_fmt.argtypes = [ctypes.POINTER(Expert), i32, i32, i32, vp, vp]
        L.coli_oracle_expert_ffn_fmt.restype = None
        L.coli_oracle_int8_code.argtypes = [vp, i32]
        L.coli_oracle_int8_code.restype = i32
        L.coli_oracle_forward.argtypes = [ctypes.POINTER(Layer), vp, i32, vp, vp, vp]
        L.coli_oracle_forward.restype = i32
        L.coli_oracle_forward_limited.argtypes = [ctypes.POINTER(Layer), vp, i32, i32, f32, vp, vp, vp]
        L.coli_oracle_forward_limited.restype = i32
        L.coli_oracle_threads.argtypes = []
        L.coli_oracle_threads.restype = i32
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().coli_oracle_threads())


def exp_spec(y: float) -> float:
    return float(_load().coli_oracle_exp_spec(float(y)))


def sigmoid_spec(z: float) -> float:
    return float(_load().coli_oracle_sigmoid_spec(float(z)))


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x, wr = _f32(x), _f32(wr)
    T, h = x.shape
    E = wr.shape[1]
    out = np.empty((T, E), np.float32)
    rc = _load().coli_oracle_router_logits(x.ctypes.data, wr.ctypes.data, T, h, E, out.ctypes.data)
    if rc:
        raise ValueError(f"coli_oracle_router_logits: {rc}")
    return out


def select(logits: np.ndarray, bias, k: int, rsf: float, k_use: int | None = None, top_p: float = 1.0):
    """Returns (idx [T,k] int32, w [T,k] float32).  k_use / top_p: the
    run-time routing limits (dropped slots: idx -1, w 0)."""
    logits = _f32(logits)
    T, E = logits.shape
    b = None if bias is None else _f32(bias)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    if k_use is None and top_p == 1.0:
        rc = _load().coli_oracle_select(logits.ctypes.data, None if b is None else b.ctypes.data,
                                        T, E, k, rsf, idx.ctypes.data, w.ctypes.data)
    else:
        rc = _load().coli_oracle_select_limited(logits.ctypes.data, None if b is None else b.ctypes.data,
                                                T, E, k, k if k_use is None else k_use, top_p, rsf,
                                                idx.ctypes.data, w.ctypes.data)
    if rc:
        raise ValueError(f"coli_oracle_select: {rc}")
    return idx, w


def dispatch(idx: np.ndarray, E: int) -> dict:
    idx = _i32(idx)
    T, k = idx.shape
    n = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ids = np.empty(n, np.int32)
    inv = np.empty(n, np.int32)
    active = np.empty(E, np.int32)
    n_active = ctypes.c_int32(0)
    rc = _load().coli_oracle_dispatch(idx.ctypes.data, T, k, E, counts.ctypes.data, offsets.ctypes.data,
                                      sorted_ids.ctypes.data, inv.ctypes.data, active.ctypes.data,
                                      ctypes.addressof(n_active))
    if rc:
        raise ValueError(f"coli_oracle_dispatch: {rc}")
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids, inv=inv,
                active=active[: n_active.value].copy(), n_active=n_active.value)


def unpack_code(row: np.ndarray, c: int) -> int:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return int(_load().coli_oracle_unpack_code(row.ctypes.data, c))


def int8_code(row: np.ndarray, c: int) -> int:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return int(_load().coli_oracle_int8_code(row.ctypes.data, c))


def _expert_struct(t: dict | None, keep: list) -> Expert:
    if t is None:
        return Expert()
    arrs = {}
    for name, dt in (("gate_q", np.uint8), ("gate_s", np.float32), ("up_q", np.uint8),
                     ("up_s", np.float32), ("down_q", np.uint8), ("down_s", np.float32)):
        a = np.ascontiguousarray(t[name], dtype=dt)
        keep.append(a)
        arrs[name] = a.ctypes.data
    return Expert(**arrs)


def expert_ffn(tables: dict, x: np.ndarray, weight_format: int = 0) -> np.ndarray:
    """One expert on one token, float64 output [h] (tables in storage format
    weight_format: 0 int4 gs64, 1 int8 per row)."""
    keep = []
    ex = _expert_struct(tables, keep)
    x = _f32(x)
    h = x.shape[0]
    I = tables["gate_q"].shape[0]
    y = np.empty(h, np.float64)
    _load().coli_oracle_expert_ffn_fmt(ctypes.byref(ex), int(weight_format), h, I, x.ctypes.data, y.ctypes.data)
    return y


def forward(shape, wr, bias, routed: dict | list, shared: dict | None, x: np.ndarray,
            k_use: int | None = None, top_p: float = 1.0):
    """The layer forward on tokens x [T, h].

    `routed` is either stacked tables (dict of [E, ...] arrays) or a list of E
    per-expert dicts (None for experts no token selects).  k_use / top_p: the
    run-time routing limits.  Returns (out [T, h] float32, idx [T, k] int32,
    w [T, k] float32)."""
    x = _f32(x)
    T, h = x.shape
    E, k = shape.n_experts, shape.top_k
    keep = [x]
    arr = (Expert * (E + shape.n_shared))()
    for e in range(E):
        if isinstance(routed, dict):
            t = {name: routed[name][e] for name in routed}
        else:
            t = routed[e]
        arr[e] = _expert_struct(t, keep)
    if shape.n_shared:
        arr[E] = _expert_struct(shared, keep)
    wr_c, b_c = _f32(wr), None if bias is None else _f32(bias)
    keep += [wr_c, b_c]
    L = Layer(hidden=h, n_experts=E, top_k=k, inter=shape.inter, n_shared=shape.n_shared,
              routed_scaling_factor=shape.rsf, router_w=wr_c.ctypes.data,
              sel_bias=None if b_c is None else b_c.ctypes.data,
              experts=ctypes.cast(arr, ctypes.POINTER(Expert)),
              weight_format=getattr(shape, "weight_format", 0))
    out = np.empty((T, h), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    if k_use is None and top_p == 1.0:
        rc = _load().coli_oracle_forward(ctypes.byref(L), x.ctypes.data, T, out.ctypes.data,
                                         idx.ctypes.data, w.ctypes.data)
    else:
        rc = _load().coli_oracle_forward_limited(ctypes.byref(L), x.ctypes.data, T, k if k_use is None else k_use,
                                                 top_p, out.ctypes.data, idx.ctypes.data, w.ctypes.data)
    if rc:
        raise ValueError(f"coli_oracle_forward: {rc}")
    return out, idx, w


def route(shape, wr, bias, x, k_use: int | None = None, top_p: float = 1.0):
    """Routing only: (idx, w) for tokens x."""
    return select(router_logits(x, wr), bias, shape.top_k, shape.rsf, k_use, top_p)
