"""Seeded synthetic inputs for the routed-MoE layer.

Test and benchmark infrastructure shared by the oracle side and the GPU side.
It holds none of the layer's arithmetic: it draws numbers (SplitMix64 counter
streams, Box-Muller normals; see gen.c) and writes them in the layer's storage
format (int4 codes, two per byte, low nibble = even column, plus one float32
scale per 64 consecutive input elements; or int8 codes with one float32 scale
per row).

Every tensor is its own stream, named by (seed, tag) with
tag = layer << 40 | kind << 32 | index, so any tensor (say one expert of one
layer) can be regenerated alone, in any order, on any host.

The workloads are five synthetic layer configurations:
weights N(0, 0.02) before int4 gs64 quantisation, router N(0, 0.02), hidden
states N(0, 1); selection bias N(0, sigma_b) (0.01 tiny, 0 for the OLMoE-like
layer with uniform selection, 0.05 GLM-like), plus for the prefill workload a
Zipf term -1.1 * beta * ln(rank_e) over a seeded rank permutation.
"""
from __future__ import annotations

import ctypes
import dataclasses

import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_synth.so")

KIND_ROUTER = 1
KIND_BIAS = 2
KIND_GATE = 3
KIND_UP = 4
KIND_DOWN = 5
KIND_HIDDEN = 6
KIND_ZIPF_PERM = 7

WEIGHT_SIGMA = 0.02

WEIGHTS_INT4_GS64 = 0   # storage formats of the expert tables
WEIGHTS_INT8_ROW = 1
ROUTER_SIGMA = 0.02
HIDDEN_SIGMA = 1.0


def build(force: bool = True) -> str:
    """Compile gen.c into _synth.so (gcc, OpenMP, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-math-errno", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i32, f32, vp, sz = (ctypes.c_uint64, ctypes.c_int, ctypes.c_float,
                                 ctypes.c_void_p, ctypes.c_size_t)
        L.synth_stream_key.argtypes = [u64, u64]
        L.synth_stream_key.restype = u64
        L.synth_bits.argtypes = [u64, u64, u64]
        L.synth_bits.restype = u64
        L.synth_normal_f32.argtypes = [u64, u64, u64, sz, f32, vp]
        L.synth_normal_f32.restype = None
        L.synth_uniform_f32.argtypes = [u64, u64, u64, sz, vp]
        L.synth_uniform_f32.restype = None
        L.synth_quant_matrix.argtypes = [u64, u64, i32, i32, f32, vp, vp]
        L.synth_quant_matrix.restype = i32
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_permutation.restype = None
        L.synth_quantize_rows.argtypes = [vp, i32, i32, vp, vp]
        L.synth_quantize_rows.restype = i32
        L.synth_quant_matrix_i8.argtypes = [u64, u64, i32, i32, f32, vp, vp]
        L.synth_quant_matrix_i8.restype = i32
        L.synth_quantize_rows_i8.argtypes = [vp, i32, i32, vp, vp]
        L.synth_quantize_rows_i8.restype = i32
        _lib = L
    return _lib


def tag(layer: int, kind: int, index: int = 0) -> int:
    return (int(layer) << 40) | (int(kind) << 32) | int(index)


def normal(seed: int, tg: int, n: int, sigma: float, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    _load().synth_normal_f32(seed, tg, start, out.size, sigma, out.ctypes.data)
    return out


def uniform(seed: int, tg: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    _load().synth_uniform_f32(seed, tg, start, out.size, out.ctypes.data)
    return out


def bits(seed: int, tg: int, j: int) -> int:
    return int(_load().synth_bits(seed, tg, j))


def permutation(seed: int, tg: int, n: int) -> np.ndarray:
    out = np.empty(int(n), np.int32)
    _load().synth_permutation(seed, tg, out.size, out.ctypes.data)
    return out


def quant_matrix_into(seed: int, tg: int, rows: int, cols: int, sigma: float,
                      codes: np.ndarray, scales: np.ndarray) -> None:
    """Draw w[r][c] = sigma * N_{r*cols+c} and quantise into caller arrays
    (C-contiguous uint8 [rows, cols/2] and float32 [rows, cols/64] views)."""
    assert cols % 64 == 0
    assert codes.dtype == np.uint8 and codes.flags.c_contiguous and codes.size == rows * cols // 2
    assert scales.dtype == np.float32 and scales.flags.c_contiguous and scales.size == rows * cols // 64
    rc = _load().synth_quant_matrix(seed, tg, rows, cols, sigma, codes.ctypes.data, scales.ctypes.data)
    if rc != 0:
        raise ValueError("synth_quant_matrix failed")


def quantize_rows(w: np.ndarray):
    """Quantise a caller-given float32 matrix [rows, cols] with the generator's
    rule; returns (codes [rows, cols/2] uint8, scales [rows, cols/64])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 64), np.float32)
    if _load().synth_quantize_rows(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data):
        raise ValueError("synth_quantize_rows: cols must be a positive multiple of 64")
    return codes, scales


def quant_matrix(seed: int, tg: int, rows: int, cols: int, sigma: float, weight_format: int = 0):
    """The matrix of stream (seed, tg) in storage format weight_format (0:
    int4 gs64, codes [rows, cols/2] and scales [rows, cols/64]; 1: int8 with
    a scale per row, codes [rows, cols] and scales [rows])."""
    if weight_format == WEIGHTS_INT8_ROW:
        codes = np.empty((rows, cols), np.uint8)
        scales = np.empty(rows, np.float32)
        quant_matrix_i8_into(seed, tg, rows, cols, sigma, codes, scales)
        return codes, scales
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 64), np.float32)
    quant_matrix_into(seed, tg, rows, cols, sigma, codes, scales)
    return codes, scales


def quant_matrix_i8_into(seed: int, tg: int, rows: int, cols: int, sigma: float,
                         codes: np.ndarray, scales: np.ndarray) -> None:
    """Draw w[r][c] = sigma * N_{r*cols+c} and quantise to int8 with one scale
    per row (s = absmax / 127, q = clamp(rne(w / s), -127, 127)) into caller
    arrays (uint8 [rows, cols], float32 [rows])."""
    assert cols % 64 == 0
    assert codes.dtype == np.uint8 and codes.flags.c_contiguous and codes.size == rows * cols
    assert scales.dtype == np.float32 and scales.flags.c_contiguous and scales.size == rows
    if _load().synth_quant_matrix_i8(seed, tg, rows, cols, sigma, codes.ctypes.data, scales.ctypes.data) != 0:
        raise ValueError("synth_quant_matrix_i8 failed")


def quantize_rows_i8(w: np.ndarray):
    """Quantise a caller-given float32 matrix [rows, cols] to int8 with one
    scale per row; returns (codes [rows, cols] uint8, scales [rows])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty(rows, np.float32)
    if _load().synth_quantize_rows_i8(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data):
        raise ValueError("synth_quantize_rows_i8 failed")
    return codes, scales


def normal_matrix(seed: int, tg: int, rows: int, cols: int, sigma: float) -> np.ndarray:
    """The unquantised draws behind quant_matrix (for quantiser tests)."""
    return normal(seed, tg, rows * cols, sigma).reshape(rows, cols)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One routed-MoE layer: hidden size h, E routed experts, top-k, expert
    intermediate size I, n_shared in {0, 1}, routed_scaling_factor, the sigma
    of the selection bias and the Zipf strength beta (0 = no Zipf term)."""
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int
    rsf: float
    bias_sigma: float
    zipf_beta: float = 0.0
    weight_format: int = WEIGHTS_INT4_GS64

    @property
    def expert_bytes(self) -> int:
        """Codes + float32 scales of one expert (gate + up + down)."""
        w = 3 * self.hidden * self.inter
        if self.weight_format == WEIGHTS_INT8_ROW:
            return w + 4 * (2 * self.inter + self.hidden)
        return w // 2 + 4 * (w // 64)


# The five synthetic workloads (tokens per call in `tokens`).
TINY = LayerShape(hidden=64, n_experts=8, top_k=2, inter=128, n_shared=1, rsf=1.0, bias_sigma=0.01)
OLMOE = LayerShape(hidden=2048, n_experts=64, top_k=8, inter=1024, n_shared=0, rsf=1.0, bias_sigma=0.0)
GLM = LayerShape(hidden=6144, n_experts=256, top_k=8, inter=2048, n_shared=1, rsf=2.5, bias_sigma=0.05)
# Zipf(s=1.1) expert load for the prefill workload: beta fixed once by
# tests/golden/zipf_calibration.py (bisection on the realised load slope).
GLM_PREFILL_ZIPF_BETA = 0.054741911590099335
GLM_PREFILL = dataclasses.replace(GLM, zipf_beta=GLM_PREFILL_ZIPF_BETA)
# The same layer shape with int8 tables (one scale per row): the multi-token
# prediction head's MoE layer, which must be int8.
GLM_MTP_I8 = dataclasses.replace(GLM, weight_format=WEIGHTS_INT8_ROW)
TINY_I8 = dataclasses.replace(TINY, weight_format=WEIGHTS_INT8_ROW)

WORKLOADS = {
    "tiny": dict(shape=TINY, tokens=(4,), layers=1),
    "olmoe_like": dict(shape=OLMOE, tokens=(16,), layers=1),
    "glm_decode": dict(shape=GLM, tokens=(1,), layers=1),
    "glm_stack": dict(shape=GLM, tokens=(1, 2, 4, 64), layers=8),
    "glm_prefill": dict(shape=GLM_PREFILL, tokens=(4096,), layers=1),
}


def router(shape: LayerShape, seed: int, layer: int = 0):
    """Router weight [h, E] float32 and selection bias [E] float32."""
    h, E = shape.hidden, shape.n_experts
    wr = normal(seed, tag(layer, KIND_ROUTER), h * E, ROUTER_SIGMA).reshape(h, E)
    if shape.bias_sigma > 0:
        b = normal(seed, tag(layer, KIND_BIAS), E, shape.bias_sigma)
    else:
        b = np.zeros(E, np.float32)
    if shape.zipf_beta > 0:
        b = (b + zipf_term(shape, seed, layer)).astype(np.float32)
    return wr, b


def zipf_term(shape: LayerShape, seed: int, layer: int = 0) -> np.ndarray:
    """-1.1 * beta * ln(rank_e) (float64, rounded to float32), rank_e = 1 +
    position of expert e in a seeded permutation."""
    perm = permutation(seed, tag(layer, KIND_ZIPF_PERM), shape.n_experts)
    rank = np.empty(shape.n_experts, np.float64)
    rank[perm] = np.arange(1, shape.n_experts + 1, dtype=np.float64)
    return (-1.1 * shape.zipf_beta * np.log(rank)).astype(np.float32)


def hidden(shape: LayerShape, seed: int, T: int, layer: int = 0, batch: int = 0) -> np.ndarray:
    """Hidden states [T, h] float32, N(0, 1), stream (layer, batch)."""
    return normal(seed, tag(layer, KIND_HIDDEN, batch), T * shape.hidden, HIDDEN_SIGMA).reshape(T, shape.hidden)


def expert(shape: LayerShape, seed: int, e: int, layer: int = 0) -> dict:
    """Tables of expert e (e == n_experts is the shared expert), in the
    shape's storage format."""
    h, I, f = shape.hidden, shape.inter, shape.weight_format
    gq, gs = quant_matrix(seed, tag(layer, KIND_GATE, e), I, h, WEIGHT_SIGMA, f)
    uq, us = quant_matrix(seed, tag(layer, KIND_UP, e), I, h, WEIGHT_SIGMA, f)
    dq, ds = quant_matrix(seed, tag(layer, KIND_DOWN, e), h, I, WEIGHT_SIGMA, f)
    return dict(gate_q=gq, gate_s=gs, up_q=uq, up_s=us, down_q=dq, down_s=ds)


def routed_tables(shape: LayerShape, seed: int, layer: int = 0, experts=None) -> dict:
    """Stacked tables of the routed experts: gate_q/up_q [E][I][h/2],
    gate_s/up_s [E][I][h/64], down_q [E][h][I/2], down_s [E][h][I/64] (int8
    tables: gate_q/up_q [E][I][h], gate_s/up_s [E][I], down_q [E][h][I],
    down_s [E][h]).
    `experts` restricts generation to a subset (others stay zero)."""
    h, I, E = shape.hidden, shape.inter, shape.n_experts
    if shape.weight_format == WEIGHTS_INT8_ROW:
        t = dict(gate_q=np.zeros((E, I, h), np.uint8), gate_s=np.zeros((E, I), np.float32),
                 up_q=np.zeros((E, I, h), np.uint8), up_s=np.zeros((E, I), np.float32),
                 down_q=np.zeros((E, h, I), np.uint8), down_s=np.zeros((E, h), np.float32))
        for e in (range(E) if experts is None else experts):
            quant_matrix_i8_into(seed, tag(layer, KIND_GATE, e), I, h, WEIGHT_SIGMA, t["gate_q"][e], t["gate_s"][e])
            quant_matrix_i8_into(seed, tag(layer, KIND_UP, e), I, h, WEIGHT_SIGMA, t["up_q"][e], t["up_s"][e])
            quant_matrix_i8_into(seed, tag(layer, KIND_DOWN, e), h, I, WEIGHT_SIGMA, t["down_q"][e], t["down_s"][e])
        return t
    t = dict(gate_q=np.zeros((E, I, h // 2), np.uint8), gate_s=np.zeros((E, I, h // 64), np.float32),
             up_q=np.zeros((E, I, h // 2), np.uint8), up_s=np.zeros((E, I, h // 64), np.float32),
             down_q=np.zeros((E, h, I // 2), np.uint8), down_s=np.zeros((E, h, I // 64), np.float32))
    for e in (range(E) if experts is None else experts):
        quant_matrix_into(seed, tag(layer, KIND_GATE, e), I, h, WEIGHT_SIGMA, t["gate_q"][e], t["gate_s"][e])
        quant_matrix_into(seed, tag(layer, KIND_UP, e), I, h, WEIGHT_SIGMA, t["up_q"][e], t["up_s"][e])
        quant_matrix_into(seed, tag(layer, KIND_DOWN, e), h, I, WEIGHT_SIGMA, t["down_q"][e], t["down_s"][e])
    return t


def shared_tables(shape: LayerShape, seed: int, layer: int = 0):
    return expert(shape, seed, shape.n_experts, layer) if shape.n_shared else None


def expected_distinct(E: int, k: int, T: int) -> float:
    """Expected number of distinct experts hit by T tokens choosing k of E
    uniformly (a planning figure; measured runs count the real ones)."""
    return E * (1.0 - (1.0 - k / E) ** T)


