"""The C-ABI library without a GPU: it loads, exports every function that
include/*.h declares, and its host-side argument checks return the documented
error codes before any HIP call is made."""
import ctypes
import glob
import os
import re

import pytest

import routed_expert_ffn_f32_amd as cm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(coli_moe_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    lib = cm.load_library()
    declared = _declared_functions()
    assert {"coli_moe_init", "coli_moe_forward", "coli_moe_free", "coli_moe_workspace_bytes",
            "coli_moe_last_routing", "coli_moe_test_dispatch"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(hidden=6144, n_experts=256, top_k=8, inter=2048, n_shared=1, routed_scaling_factor=2.5,
                max_tokens=64)
    base.update(kw)
    return cm.make_config(**base)


def test_workspace_bytes_valid_and_invalid():
    n = cm.coli_moe_workspace_bytes(_cfg())
    E, h, I, T, k = 256, 6144, 2048, 64, 8
    rows = T * k + T
    assert n >= E * h * 4 + rows * (I + h) * 4
    assert n % 256 == 0
    assert cm.coli_moe_workspace_bytes(_cfg(max_tokens=128)) > n
    for bad in (dict(hidden=100), dict(inter=96 + 1), dict(n_experts=0), dict(n_experts=513),
                dict(top_k=0), dict(top_k=9, n_experts=8), dict(top_k=33, n_experts=64),
                dict(max_tokens=0), dict(n_shared=2), dict(group_size=32), dict(n_group=2),
                dict(prefill_threshold=-1)):
        assert cm.coli_moe_workspace_bytes(_cfg(**bad)) == 0, bad


def _weights(addr=0x100000):
    w = cm.coli_moe_weights_t()
    for i, (name, _) in enumerate(cm.coli_moe_weights_t._fields_):
        setattr(w, name, addr + 0x1000 * (i + 1))
    return w


def _init_rc(cfg, w, ws=0x7f0000000000, nbytes=None):
    lib = cm.load_library()
    h = ctypes.c_void_p()
    if nbytes is None:
        nbytes = cm.coli_moe_workspace_bytes(cfg)
    return lib.coli_moe_init(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), ws, nbytes, None)


def test_init_argument_errors():
    lib = cm.load_library()
    cfg, w = _cfg(), _weights()
    assert lib.coli_moe_init(None, ctypes.byref(cfg), ctypes.byref(w), 0x7f0000000000, 1 << 30, None) == -4
    assert _init_rc(cfg, w, ws=0) == -4
    assert _init_rc(_cfg(top_k=300), w) == -2
    assert _init_rc(_cfg(n_group=2), w) == -2
    assert _init_rc(_cfg(group_size=128), w) == -2
    assert _init_rc(_cfg(hidden=96), w) == -4
    assert _init_rc(cfg, w, nbytes=1024) == -1          # workspace too small
    assert _init_rc(cfg, w, ws=0x7f0000000010) == -4    # workspace not 256-byte aligned
    bad = _weights()
    bad.gate_q = None
    assert _init_rc(cfg, bad) == -4
    bad = _weights()
    bad.down_s = 0x100008                                 # not 16-byte aligned
    assert _init_rc(cfg, bad) == -4
    bad = _weights()
    bad.sh_up_q = None                                    # shared expert configured but missing
    assert _init_rc(cfg, bad) == -4


def test_forward_and_dispatch_argument_errors():
    lib = cm.load_library()
    assert lib.coli_moe_forward(None, 0x1000, 0x2000, 1, None) == -4
    assert lib.coli_moe_last_routing(None, None, None, None, None, None, None, None, None) == -4
    assert lib.coli_moe_test_dispatch(0x1000, 4, 0, 8, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == -4
    assert lib.coli_moe_test_dispatch(0x1000, 4, 2, 513, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == -4
    assert lib.coli_moe_probe_read(None, 0x1000, 9, None) == -4
    # measurement probes: every bad argument is refused before any launch
    assert lib.coli_moe_probe_stream(None, 1024, 0x2000, None) == -4
    assert lib.coli_moe_probe_stream(0x1000, 1000, 0x2000, None) == -4   # not a multiple of 16
    assert lib.coli_moe_probe_stream(0x1008, 1024, 0x2000, None) == -4   # buffer not 16-byte aligned
    assert lib.coli_moe_probe_stream(0x1000, 0, 0x2000, None) == -4
    assert lib.coli_moe_probe_stream(0x1000, 1024, None, None) == -4
    assert lib.coli_moe_probe_mfma(0, 4, 0x2000, None) == -4
    assert lib.coli_moe_probe_mfma(1 << 20, 4, 0x2000, None) == -4
    assert lib.coli_moe_probe_mfma(10, 0, 0x2000, None) == -4
    assert lib.coli_moe_probe_mfma(10, 4, None, None) == -4
    assert lib.coli_moe_probe_mfma_f16(0, 4, 1, 0x2000, None) == -4
    assert lib.coli_moe_probe_mfma_f16(10, 1 << 21, 1, 0x2000, None) == -4
    assert lib.coli_moe_probe_mfma_f16(10, 4, 1, 0x2002, None) == -4
    assert lib.coli_moe_set_routing(None, 4, ctypes.c_float(0.7)) == -4
    assert lib.coli_moe_status(None, None) == -4
    assert lib.coli_moe_probe_read_down(None, 0x1000, 2, None) == -4
    assert lib.coli_moe_test_spin_limit(None, 5) == -4
    assert lib.coli_moe_test_batch_kernels(None, 1) == -4
    assert lib.coli_moe_test_dispatch(0x1000, -1, 2, 8, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == -4
    assert lib.coli_moe_test_dispatch(None, 4, 2, 8, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == -4
    lib.coli_moe_free(None)  # no-op
    assert lib.coli_moe_profile_begin(None, 4) == -4
    assert lib.coli_moe_profile_end(None, None, None) == -4


def test_error_strings_and_kernel_names():
    for code in (0, -1, -2, -3, -4):
        assert cm.coli_moe_error_string(code)
    assert cm.coli_moe_error_string(-99) == "unknown error code"
    names = [cm.coli_moe_kernel_name(i) for i in range(cm.COLI_MOE_N_KERNELS)]
    assert len(set(names)) == cm.COLI_MOE_N_KERNELS and all(names)
    assert cm.coli_moe_kernel_name(cm.COLI_MOE_N_KERNELS) == ""


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(cm, "_lib", None)
    monkeypatch.setattr(cm, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="build it"):
        cm.load_library()


def test_forward_noalloc_host_checks():
    """The allocation-free forward rejects bad arguments, over-capacity
    calls and configurations whose workspace exceeds the library's static
    device array before any HIP call; a zero-token call is a dry run."""
    lib = cm.load_library()
    w = _weights()
    limit = cm.COLI_MOE_STATIC_SCRATCH_BYTES
    assert 0 < cm.coli_moe_workspace_bytes(_cfg(max_tokens=64)) <= limit
    assert cm.coli_moe_workspace_bytes(_cfg(max_tokens=163)) <= limit < cm.coli_moe_workspace_bytes(_cfg(max_tokens=164))
    f = lib.coli_moe_forward_noalloc
    assert f(None, ctypes.byref(w), 0x1000, 0x2000, 1, None) == -4
    assert f(ctypes.byref(_cfg()), None, 0x1000, 0x2000, 1, None) == -4
    assert f(ctypes.byref(_cfg(n_group=2)), ctypes.byref(w), 0x1000, 0x2000, 1, None) == -2
    assert f(ctypes.byref(_cfg(max_tokens=64)), ctypes.byref(w), 0x1000, 0x2000, 65, None) == -1
    assert f(ctypes.byref(_cfg(max_tokens=164)), ctypes.byref(w), 0x1000, 0x2000, 1, None) == -1
    assert f(ctypes.byref(_cfg(max_tokens=64)), ctypes.byref(w), 0x1000, 0x2000, -1, None) == -4
    assert f(ctypes.byref(_cfg(max_tokens=64)), ctypes.byref(w), 0x1000, 0x2000, 0, None) == 0
    assert f(ctypes.byref(_cfg(max_tokens=64)), ctypes.byref(w), 0x1001, 0x2000, 1, None) == -4
    with pytest.raises(cm.ColiMoeError) as ei:
        cm.coli_moe_forward_noalloc(_cfg(max_tokens=164), w, 0x1000, 0x2000, 1)
    assert ei.value.code == -1
