"""CPU-side checks of the C-ABI library: it loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

from sparse_moe_routing_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_create", "moe_destroy", "moe_workspace_bytes", "moe_route",
                     "moe_bucket", "moe_forward", "moe_status_str"):
        assert required in names
    assert set(names) == set(binding.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_oracle_code_in_the_library():
    # the product library must not contain the oracle's entry points
    data = open(binding.LIB_PATH, "rb").read()
    assert b"oracle_" not in data


def test_read_probe_is_a_library_of_its_own(lib):
    """The benchmark's streaming-read calibration kernel is built as libmoe_probe.so, exports
    moe_probe_read and rejects a misaligned size on the host; libmoe.so carries no such symbol."""
    path = os.path.join(ROOT, "sparse_moe_routing_amd", "libmoe_probe.so")
    probe = ctypes.CDLL(path)
    probe.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    probe.moe_probe_read.restype = ctypes.c_int
    assert probe.moe_probe_read(ctypes.c_void_p(16), 17, 1, ctypes.c_void_p(16), None) != 0
    assert probe.moe_probe_read(None, 16, 1, ctypes.c_void_p(16), None) != 0
    assert not hasattr(lib, "moe_probe_read")


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.moe_status_str(st)
    assert lib.moe_status_str(12345) == b"unknown status"


def good_config():
    return binding.moe_config(2048, 256, 8, 512, 512, 64, binding.MOE_BF16)


def fake_weights(shared=True):
    # host addresses that are never dereferenced: validation runs before any device access
    base = 0x10000000
    return binding.moe_weights(base, None, base + 0x1000000, base + 0x2000000,
                               base + 0x3000000 if shared else None,
                               base + 0x4000000 if shared else None)


def create(lib, cfg, w):
    ctx = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(cfg) if cfg is not None else None,
                        ctypes.byref(w) if w is not None else None, ctypes.byref(ctx))
    return st, ctx


@pytest.mark.parametrize("field,value,want", [
    ("top_k", 4, binding.MOE_ERR_UNSUPPORTED),
    ("top_k", 16, binding.MOE_ERR_UNSUPPORTED),
    ("num_experts", 7, binding.MOE_ERR_UNSUPPORTED),
    ("num_experts", 257, binding.MOE_ERR_UNSUPPORTED),
    ("hidden", 100, binding.MOE_ERR_UNSUPPORTED),
    ("hidden", 0, binding.MOE_ERR_UNSUPPORTED),
    ("inter", 48, binding.MOE_ERR_UNSUPPORTED),     # bf16 needs a multiple of 32
    ("shared_inter", 8, binding.MOE_ERR_UNSUPPORTED),
    ("max_tokens", 0, binding.MOE_ERR_INVALID_ARG),
    ("max_tokens", 70000, binding.MOE_ERR_UNSUPPORTED),
    ("dtype", 7, binding.MOE_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config(lib, field, value, want):
    cfg = good_config()
    setattr(cfg, field, value)
    st, ctx = create(lib, cfg, fake_weights())
    assert st == want
    assert not ctx.value


def test_create_rejects_bad_weights(lib):
    cfg = good_config()
    assert create(lib, None, fake_weights())[0] == binding.MOE_ERR_INVALID_ARG
    assert create(lib, cfg, None)[0] == binding.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.router_w = None
    assert create(lib, cfg, w)[0] == binding.MOE_ERR_INVALID_ARG
    w = fake_weights(shared=False)  # shared_inter > 0 but no shared weights
    assert create(lib, cfg, w)[0] == binding.MOE_ERR_INVALID_ARG
    cfg0 = good_config()
    cfg0.shared_inter = 0
    assert create(lib, cfg0, fake_weights(shared=True))[0] == binding.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.gate_up = 0x10000008  # not 16-byte aligned
    assert create(lib, cfg, w)[0] == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_create(ctypes.byref(cfg), ctypes.byref(fake_weights()), None) == \
        binding.MOE_ERR_INVALID_ARG


def test_create_checks_fp8_weights(lib):
    """FP8 E4M3 expert weights need every row-scale array (16-byte aligned) and 128-element
    multiples for I and I_s; other dtypes must not pass scales."""
    cfg = good_config()
    cfg.dtype = binding.MOE_FP8_E4M3
    base = 0x20000000

    def fp8_weights(shared=True):
        w = fake_weights(shared)
        w.gate_up_scale = base
        w.down_scale = base + 0x100000
        w.shared_gate_up_scale = base + 0x200000 if shared else None
        w.shared_down_scale = base + 0x300000 if shared else None
        return w

    for name in ("gate_up_scale", "down_scale", "shared_gate_up_scale", "shared_down_scale"):
        w = fp8_weights()
        setattr(w, name, None)
        assert create(lib, cfg, w)[0] == binding.MOE_ERR_INVALID_ARG, name
        w = fp8_weights()
        setattr(w, name, getattr(w, name) + 4)  # 4-byte but not 16-byte aligned
        assert create(lib, cfg, w)[0] == binding.MOE_ERR_INVALID_ARG, name
    cfg0 = good_config()
    cfg0.dtype = binding.MOE_FP8_E4M3
    cfg0.shared_inter = 0  # no shared expert: no shared scales either
    w = fp8_weights(shared=False)
    w.shared_down_scale = base + 0x300000
    assert create(lib, cfg0, w)[0] == binding.MOE_ERR_INVALID_ARG
    bf = good_config()  # bf16 weights take no scales
    assert create(lib, bf, fp8_weights())[0] == binding.MOE_ERR_INVALID_ARG
    for field, value in (("inter", 96), ("shared_inter", 160), ("hidden", 192)):
        c = good_config()
        c.dtype = binding.MOE_FP8_E4M3
        setattr(c, field, value)
        assert create(lib, c, fp8_weights())[0] == binding.MOE_ERR_UNSUPPORTED, field


def test_create_checks_mxfp4_weights(lib):
    """MXFP4 expert weights need every scale-byte array (at any address) and 256-weight
    multiples for H, I and I_s."""
    base = 0x20000000

    def mx_cfg():
        c = good_config()
        c.dtype = binding.MOE_MXFP4
        return c

    def mx_weights():
        w = fake_weights(True)
        w.gate_up_scale = base + 1  # byte arrays: no alignment asked for
        w.down_scale = base + 0x100003
        w.shared_gate_up_scale = base + 0x200005
        w.shared_down_scale = base + 0x300007
        return w

    for name in ("gate_up_scale", "down_scale", "shared_gate_up_scale", "shared_down_scale"):
        w = mx_weights()
        setattr(w, name, None)
        assert create(lib, mx_cfg(), w)[0] == binding.MOE_ERR_INVALID_ARG, name
    st, ctx = create(lib, mx_cfg(), mx_weights())  # valid: fails only for want of a GPU here
    assert st in (binding.MOE_OK, binding.MOE_ERR_HIP, binding.MOE_ERR_UNSUPPORTED)
    if st == binding.MOE_OK:
        lib.moe_destroy(ctx)
    for field, value in (("inter", 384), ("shared_inter", 128), ("hidden", 384)):
        c = mx_cfg()
        setattr(c, field, value)
        assert create(lib, c, mx_weights())[0] == binding.MOE_ERR_UNSUPPORTED, field


def test_calls_reject_null_context(lib):
    assert lib.moe_workspace_bytes(None, 4) == 0
    assert lib.moe_route(None, None, None, 4, None, None, None, None, None, 0, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert lib.moe_bucket(None, None, 4, None, None, None, None, 0, None) == \
        binding.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(None, None, 4, None, None, None, None, None, 0, None) == \
        binding.MOE_ERR_INVALID_ARG
    n = ctypes.c_int32()
    assert lib.moe_forward_plan(None, 4, 0, ctypes.byref(n), None, 0) == binding.MOE_ERR_INVALID_ARG
    lib.moe_destroy(None)


def test_create_without_gpu_reports_hip_error(lib):
    """A valid config on a machine without a usable gfx950 device fails cleanly."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, ctx = create(lib, good_config(), fake_weights())
    assert st in (binding.MOE_ERR_HIP, binding.MOE_ERR_UNSUPPORTED)
    assert not ctx.value


@pytest.mark.slow
def test_no_kernel_spills_to_scratch(tmp_path):
    """Every gfx950 kernel of the library keeps its state in registers: the device code of each
    source, compiled with the library's flags, declares no private (scratch) segment. A spill in a
    streaming kernel has cost 2x at large T (the wait-state barrier case), so it is a build check."""
    import glob
    import shutil
    import subprocess
    from sparse_moe_routing_amd import build as lib_build
    try:
        cc = lib_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    # -Werror off here only: hipcc adds a link flag that a device-only compile leaves unused
    flags = [f for f in lib_build.compile_flags() if f not in ("-fPIC", "-Werror")]
    srcs = sorted(glob.glob(os.path.join(lib_build.CSRC, "*.hip")))
    assert srcs
    bad = []
    for src in srcs:
        out = tmp_path / (os.path.basename(src) + ".s")
        cmd = [cc, *flags, "--cuda-device-only", "-S", src, "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = out.read_text()
        for name, size in re.findall(r"\.name:\s+(\S+)\n(?:(?!\.name:).)*?\.private_segment_fixed_size:\s+(\d+)",
                                     text, re.S):
            if int(size) > 0:
                bad.append((os.path.basename(src), name, int(size)))
    assert not bad, bad
