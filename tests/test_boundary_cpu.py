"""CPU-side checks of the C-ABI library: it loads, exports what include/gptq_mi355x.h declares,
and its host validation agrees with the rules the pages state (no GPU, no kernel launch)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as o
import weight_only_quantized_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq_mi355x.h")
CODES = {"ok": 0, "shape": 2, "gidx": 3, "unsupported": 4}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(wq.symbols)


def test_library_exports_every_declared_symbol():
    lib = wq.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings():
    lib = wq.load_library()
    for s in range(10):
        assert lib.gptq_status_str(s)
    assert lib.gptq_status_str(0) == b"ok"


def test_null_handle_calls_fail_cleanly():
    lib = wq.load_library()
    assert lib.gptq_destroy(None) == 0
    assert lib.gptq_gemm(None, None, 1, 0, None, None, 0, 0, None) == 1
    assert lib.gptq_info(None, None) == 1
    assert lib.gptq_decode_runtime(None, None, None, None, None) == 1
    n = ctypes.c_size_t()
    assert lib.gptq_workspace_size(None, 1, 0, 0, ctypes.byref(n)) == 1
    # repack with a NULL out pointer must fail before touching the device
    assert lib.gptq_repack(None, None, None, None, None, None, None) == 1


def _desc(K, N, bits, gs, qw=None, qz=None, sc=None, glen=None, fmt="gptq", sdt=wq.F16):
    G = o.num_groups(K, gs) if gs == -1 or gs > 0 else 1
    qw = qw if qw is not None else (K // 32 * bits, N)
    qz = qz if qz is not None else (G, N // 32 * bits)
    sc = sc if sc is not None else (G, N)
    return wq.make_desc(K, N, bits, gs, sdt, qw, qz, sc, K if glen is None else glen, checkpoint_format=fmt)


def test_example_header_rules_match_the_oracle():
    import json
    h = json.load(open(os.path.join(ROOT, "tests", "golden", "small_gptq_header.json")))["tensors"]
    K, N, bits, gs = 256, 32, 4, 32
    qw, qz, sc = h["gptq.qweight"]["shape"], h["gptq.qzeros"]["shape"], h["gptq.scales"]["shape"]
    g = (np.arange(K) // gs).astype(np.int32)
    cases = [
        (dict(), g, "ok"),
        (dict(bits=5), g, "unsupported"),
        (dict(qw=(31, 32)), g, "shape"),
        (dict(qz=(8, 5)), g, "shape"),
        (dict(sc=(8, 31)), g, "shape"),
        (dict(fmt="marlin"), g, "unsupported"),
        (dict(fmt="gptq_v2"), g, "ok"),
        (dict(fmt="gptq_p"), g, "ok"),
        (dict(fmt="gptq_p", bits=5), g, "ok"),
        (dict(fmt="gptq_p", bits=9), g, "unsupported"),
        (dict(fmt="gptq_v2", bits=6), g, "unsupported"),
        (dict(gs=48), None, "unsupported"),
    ]
    for kw, gi_, want in cases:
        b = kw.get("bits", bits)
        gsz = kw.get("gs", gs)
        d = _desc(K, N, b, gsz, qw=kw.get("qw", qw if b == bits else None), qz=kw.get("qz", qz if gsz == gs and b == bits else None),
                  sc=kw.get("sc", sc if gsz == gs else None), glen=None if gi_ is not None else 0, fmt=kw.get("fmt", "gptq"))
        got = wq.validate(d, gi_)
        ref = o.validate_layer(K, N, b, gsz, tuple(d.qweight_shape), tuple(d.qzeros_shape), tuple(d.scales_shape), gi_,
                               checkpoint_format=kw.get("fmt", "gptq"))
        assert got == CODES[want] == CODES[ref], (kw, got, ref)
    bad = g.copy(); bad[7] = 8
    assert wq.validate(_desc(K, N, bits, gs), bad) == CODES["gidx"]
    bad[7] = -3
    assert wq.validate(_desc(K, N, bits, gs), bad) == CODES["gidx"]
    assert wq.validate(_desc(K, N, bits, gs, glen=255)) == CODES["gidx"]


def test_validation_agrees_with_oracle_on_random_mutations():
    rng = np.random.default_rng(0)
    for trial in range(400):
        K = int(rng.choice([64, 96, 256, 288, 4096]))
        N = int(rng.choice([32, 64, 96, 128]))
        bits = int(rng.choice([2, 3, 4, 8, 5, 6, 7, 1, 9]))
        fmt = str(rng.choice(["gptq", "gptq", "gptq_v2", "gptq_p", "awq_gemm", "marlin"]))
        gs = int(rng.choice([-1, 32, 64, 128, 96, 48, 0]))
        G = o.num_groups(K, gs) if (gs == -1 or gs > 0) else 1
        qw = [K, N // 8] if fmt == "awq_gemm" else [K // 32 * bits, N]
        qz = [G, N // 8] if fmt == "awq_gemm" else [G, N // 32 * bits]
        sc = [G, N]
        which = rng.integers(0, 6)
        if which == 1: qw[0] += int(rng.choice([-1, 1]))
        if which == 2: qz[1] += int(rng.choice([-1, 1]))
        if which == 3: sc[0] += 1
        gsz = K if gs == -1 else (gs if gs > 0 else 32)
        if rng.random() < 0.5:
            g = (np.arange(K) // gsz).astype(np.int32)
        else:
            g = (rng.permutation(K) // gsz).astype(np.int32)
        if which == 4: g[rng.integers(0, K)] = G
        if which == 5 and G > 1:
            g[0], g[-1] = g[-1], 0
            g[1] = g[-1]
        if fmt == "awq_gemm" and rng.random() < 0.7:
            g = None                                 # an AWQ layer has no g_idx
        d = wq.make_desc(K, N, bits, gs, wq.F16, qw, qz, sc, K if g is not None else 0, checkpoint_format=fmt)
        ref = o.validate_layer(K, N, bits, gs, qw, qz, sc, g, checkpoint_format=fmt)
        assert wq.validate(d, g) == CODES[ref], (K, N, bits, gs, fmt, which, ref)


def test_runtime_layout_map_is_a_bijection():
    exe = os.path.join("/tmp", f"gq_layout_check_{os.getpid()}")
    src = os.path.join(ROOT, "tests", "layout_check.cpp")
    inc = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, src, "-o", exe], check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
    finally:
        os.remove(exe)


def test_dispatch_plans_fit_their_kernels():
    """Every form the skinny dispatch rules pick fits its kernel's LDS, wave bound, copy pieces and
    instantiated chunk and part counts (tests/plan_check.cpp over rows 0..64, chunks 1..160 and a
    spread of column-tile counts)."""
    exe = os.path.join("/tmp", f"gq_plan_check_{os.getpid()}")
    src = os.path.join(ROOT, "tests", "plan_check.cpp")
    inc = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, src, "-o", exe], check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
    finally:
        os.remove(exe)


def test_act_order_bank_spread():
    """The within-group order of act-order layers (csrc/bank_spread.h): for seeded act-order maps
    over K = 128 .. 8192 and groups of 128 / 256 / 512 / all inputs it succeeds and gives a
    permutation that keeps every group on its positions with distinct LDS banks per staging write
    instruction (tests/spread_check.cpp, checked independently of the function's own check)."""
    exe = os.path.join("/tmp", f"gq_spread_check_{os.getpid()}")
    src = os.path.join(ROOT, "tests", "spread_check.cpp")
    inc = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", inc, src, "-o", exe], check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
    finally:
        os.remove(exe)


def test_bias_patterns_are_the_stated_values():
    # dequant.h feeds -bias as raw 16-bit patterns; check them against numpy's conversions
    text = open(os.path.join(ROOT, "weight_only_quantized_amd", "csrc", "dequant.h")).read()
    assert "0xC310C310u" in text and "0xE400u" in text
    assert (np.float32(-144.0).view(np.uint32) >> 16) == 0xC310            # -bias, bf16
    assert np.float16(-1024.0).view(np.uint16) == 0xE400                   # -(1024 + z) = 0xE400 + z
    for z in range(1, 257):
        assert np.float16(-(1024.0 + z)).view(np.uint16) == 0xE400 + z
    for v in range(0, 256):
        assert np.uint16(0x6400 + v).view(np.float16) == 1024 + v          # fp16 magic: 0x64vv
    for v in range(0, 128):
        assert np.float32(np.uint32((0x4300 + v) << 16).view(np.float32)) == 128 + v   # bf16 magic: 0x43vv


def test_runtime_perm_checker_rejects_wrong_orders():
    """The GPU tests' check of the decoded load-time order (gpu_util.check_runtime_perm) fails a
    permutation that breaks a group, and, for an act-order layer staged whole in LDS, the stable
    order (whose scatter instructions hit repeated banks); it passes the stable order where the
    library keeps it."""
    import numpy as np
    import oracle as o
    from gpu_util import check_runtime_perm
    rng = np.random.default_rng(5)
    K, gs = 1024, 128
    g = np.empty(K, np.int64)
    g[rng.permutation(K)] = np.arange(K) // gs
    stable = o.runtime_perm(g)
    with pytest.raises(AssertionError):
        check_runtime_perm(stable, g, gs)          # the staged act-order layer must spread banks
    broken = stable.copy()
    broken[[0, gs]] = broken[[gs, 0]]              # two inputs of different groups swapped
    with pytest.raises(AssertionError):
        check_runtime_perm(broken, g, 32)
    check_runtime_perm(stable, g, 32)              # 32-input groups keep the stable order
    check_runtime_perm(np.arange(K), np.arange(K) // gs, gs)   # identity order
