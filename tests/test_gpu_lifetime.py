"""Lifetime, stream and graph cases of the C ABI ("Kernel Backends Reference", "Kernel implementation
and validation checklist" item 6: repeated forwards, mutation and lifetime cases, not one call; its
section "Marlin and caller-owned scratch": a graph caller preallocates the scratch and owns it for
the graph's lifetime).

- every PATH_AUTO route (skinny with staged x, skinny with x from L2, the skinny copy form whole and
  in two halves, the mid kernel's split K and its reduction launch, the tiled family's prep + tiles
  + split-K reduction, act-order staging and act-order prep) captured in a HIP graph and replayed
  several times, with the program's own eager work and new inputs between replays: every replay
  bitwise equal to the eager call;
- two handles on two streams, and one handle on two streams, each call with its own workspace:
  bitwise equal to the eager single-stream results;
- a destroyed handle is refused (no use of freed memory); a device allocation failure during repack
  returns GPTQ_E_OOM and leaves the library usable."""
import sys

import numpy as np
import pytest

import gptq_inputs as gi
import oracle as o
from gpu_util import bits_to_device, check, device_to_bits, repack_layer, run_gemm, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_amd as wq
    wq.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# (label, K, N, bits, gs, desc_act, x dtype, M, path, needs workspace or None): one case per route of the
# dispatcher (PATH_AUTO where it takes that route, else the family forced; 1 = SKINNY, 2 = TILED)
ROUTES = [
    ("skinny staged x", 4096, 2048, 4, 128, False, "f16", 1, 0, False),
    ("skinny staged x bf16 offset form", 8192, 2048, 4, 128, False, "bf16", 1, 0, False),
    ("skinny x from L2", 4096, 2048, 4, 128, False, "f16", 3, 1, False),
    ("skinny copy of x", 4096, 2048, 4, 128, False, "f16", 16, 1, False),
    ("skinny copy of x in two halves, offset form", 8192, 2048, 4, 128, False, "bf16", 12, 1, False),
    ("mid split K + reduction", 8192, 2048, 8, 128, False, "bf16", 12, 1, True),
    ("tiled prep + split K + reduction", 4096, 2048, 4, 128, False, "bf16", 64, 2, True),
    ("tiled large M", 2048, 1024, 3, 64, False, "f16", 300, 0, None),
    ("act-order staged", 2048, 1024, 4, 128, True, "f16", 3, 0, False),
    ("act-order prep + tiled", 2048, 1024, 2, 64, True, "bf16", 48, 2, True),
]


@pytest.mark.parametrize("route", ROUTES, ids=[r[0] for r in ROUTES])
def test_graph_replays_equal_eager(route):
    import torch
    label, K, N, bits, gs, act, xdt, M, path, needs_ws = route
    say("graph", label)
    L = gi.make_layer(K, N, bits, gs, desc_act=act, scales_dtype="f16", seed=gi.seed_for(9, bits))
    h = repack_layer(L)
    tdt = torch_dtype(xdt)
    xs = [bits_to_device(gi.make_x(M, K, xdt, seed=gi.seed_for(9, 10 + i)), xdt) for i in range(3)]
    need = h.workspace_size(M, tdt, path)
    assert needs_ws is None or (need > 0) == needs_ws, (label, need)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    eager = []
    for x in xs:
        eager.append(device_to_bits(h.gemm(x, workspace=ws, path=path)))
    x_in = xs[0].clone()
    y = torch.empty((M, N), dtype=tdt, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # one warm-up call on the capture stream
        h.gemm(x_in, out=y, workspace=ws, path=path)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.gemm(x_in, out=y, workspace=ws, path=path)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 3
        x_in.copy_(xs[i])                 # the program's own eager work between replays
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(device_to_bits(y), eager[i]), (label, rep)
    del g
    h.close()


def test_two_handles_on_two_streams():
    import torch
    say("two handles, two streams")
    specs = [(4096, 2048, 4, 128, False, "bf16"), (2048, 3072, 3, 64, True, "f16")]
    hs, xs, refs, wss, tdts = [], [], [], [], []
    for j, (K, N, bits, gs, act, xdt) in enumerate(specs):
        L = gi.make_layer(K, N, bits, gs, desc_act=act, scales_dtype="f16", seed=gi.seed_for(9, 20 + j))
        h = repack_layer(L)
        tdt = torch_dtype(xdt)
        per = []
        for M in (1, 12, 64):
            x = bits_to_device(gi.make_x(M, K, xdt, seed=gi.seed_for(9, 30 + M + j)), xdt)
            per.append((x, device_to_bits(h.gemm(x))))
        hs.append(h)
        xs.append(per)
        tdts.append(tdt)
        wss.append([torch.empty(max(h.workspace_size(x.shape[0], tdt), 256), dtype=torch.uint8, device="cuda")
                    for x, _ in per])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * 3 for _ in range(2)]
    for rnd in range(3):                   # interleave the two streams' launches
        for i in range(3):
            for j in range(2):
                x, _ = xs[j][i]
                outs[j][i] = hs[j].gemm(x, workspace=wss[j][i], stream=streams[j])
        torch.cuda.synchronize()
        for j in range(2):
            for i in range(3):
                assert np.array_equal(device_to_bits(outs[j][i]), xs[j][i][1]), (rnd, j, i)
    for h in hs:
        h.close()


def test_one_handle_on_two_streams():
    import torch
    say("one handle, two streams")
    K, N = 8192, 2048      # 8-bit codes: the mid kernel's split K at 12 rows, the tiled split K at 64
    L = gi.make_layer(K, N, 8, 128, desc_act=False, scales_dtype="f16", seed=gi.seed_for(9, 40))
    h = repack_layer(L)
    cases = []
    for M, xdt in ((12, "bf16"), (64, "f16")):     # both need workspace (split K / prep)
        tdt = torch_dtype(xdt)
        x = bits_to_device(gi.make_x(M, K, xdt, seed=gi.seed_for(9, 41 + M)), xdt)
        ref = device_to_bits(h.gemm(x))
        ws = torch.empty(max(h.workspace_size(M, tdt), 256), dtype=torch.uint8, device="cuda")
        assert h.workspace_size(M, tdt) > 0
        cases.append((x, ref, ws))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(4):
        ys = [h.gemm(cases[j][0], workspace=cases[j][2], stream=streams[j]) for j in range(2)]
        torch.cuda.synchronize()
        for j in range(2):
            assert np.array_equal(device_to_bits(ys[j]), cases[j][1]), (rnd, j)
    h.close()


def test_destroyed_handle_is_refused():
    import ctypes
    import torch
    import weight_only_quantized_amd as wq
    lib = wq.load_library()
    L = gi.make_layer(256, 256, 4, 128, desc_act=False, scales_dtype="f16", seed=gi.seed_for(9, 50))
    h = repack_layer(L)
    ptr = h.ptr
    x = torch.zeros((1, 256), dtype=torch.float16, device="cuda")
    y = torch.empty((1, 256), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.gptq_gemm(ptr, x.data_ptr(), 1, wq.F16, y.data_ptr(), None, 0, 0, s) == 0
    assert lib.gptq_destroy(ptr) == 0
    h._ptr = None                              # the Python wrapper must not destroy it again
    assert wq.STATUS[lib.gptq_gemm(ptr, x.data_ptr(), 1, wq.F16, y.data_ptr(), None, 0, 0, s)] == "E_INVALID_ARG"
    n = ctypes.c_size_t(0)
    assert wq.STATUS[lib.gptq_workspace_size(ptr, 1, wq.F16, 0, ctypes.byref(n))] == "E_INVALID_ARG"
    info = wq.Info()
    assert wq.STATUS[lib.gptq_info(ptr, ctypes.byref(info))] == "E_INVALID_ARG"
    assert wq.STATUS[lib.gptq_destroy(ptr)] == "E_INVALID_ARG"
    assert lib.gptq_destroy(None) == 0
    # a pointer never issued by the library
    assert wq.STATUS[lib.gptq_info(ctypes.c_void_p(x.data_ptr()), ctypes.byref(info))] == "E_INVALID_ARG"


def test_hip_runtime_error_is_reported_with_its_code():
    """A HIP runtime failure surfaces as GPTQ_E_HIP, with the runtime's own error code behind it in
    gptq_last_hip_error: gptq_repack reads g_idx back to the host and synchronises its stream, which
    a stream under graph capture refuses.  No kernel is launched.  The library works as before
    once the capture has ended."""
    import ctypes
    import torch
    import weight_only_quantized_amd as wq
    say("HIP error")
    hip = ctypes.CDLL("libamdhip64.so")
    lib = wq.load_library()
    K, N = 256, 64
    L = gi.make_layer(K, N, 4, 128, desc_act=True, scales_dtype="f16", seed=gi.seed_for(9, 61))
    qw = torch.from_numpy(L.qweight).cuda()
    qz = torch.from_numpy(L.qzeros).cuda()
    sc = bits_to_device(L.scales, "f16")
    gx = torch.from_numpy(L.g_idx).cuda()
    d = wq.make_desc(K, N, 4, 128, wq.F16, qw.shape, qz.shape, sc.shape, K, True)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    sp = ctypes.c_void_p(s.cuda_stream)
    assert hip.hipStreamBeginCapture(sp, 2) == 0          # hipStreamCaptureModeRelaxed
    out = ctypes.c_void_p()
    try:
        st = lib.gptq_repack(ctypes.byref(d), qw.data_ptr(), qz.data_ptr(), sc.data_ptr(), gx.data_ptr(), sp,
                             ctypes.byref(out))
        code = lib.gptq_last_hip_error()
    finally:
        graph = ctypes.c_void_p()
        hip.hipStreamEndCapture(sp, ctypes.byref(graph))    # the capture is invalidated
        if graph.value:
            hip.hipGraphDestroy(graph)
        hip.hipGetLastError()
    assert wq.STATUS[st] == "E_HIP", st
    assert code != 0
    assert not out.value
    h = wq.repack(qw, qz, sc, gx, bits=4, group_size=128, desc_act=True)
    x = gi.make_x(3, K, "f16", seed=7)
    y_ref = o.gemm(x, "f16", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 4)
    check(run_gemm(h, x, "f16"), "f16", y_ref, label="after a HIP error")
    h.close()


def test_out_of_device_memory_is_reported():
    """Fill the device's free memory from the host, leaving less than the runtime layout needs:
    gptq_repack returns GPTQ_E_OOM and frees what it had taken; after the memory is released the
    same repack succeeds."""
    import torch
    import weight_only_quantized_amd as wq
    say("out of memory")
    # runtime layout 256 MiB + metadata: far above the headroom left below, and above what the
    # HIP runtime can still find by releasing memory it holds for itself (a 64 MiB layer was
    # placed there once the library's code objects had grown)
    K, N = 16384, 32768
    L = gi.make_layer(K, N, 4, 128, desc_act=False, scales_dtype="f16", seed=gi.seed_for(9, 60))
    qw = torch.from_numpy(L.qweight).cuda()
    qz = torch.from_numpy(L.qzeros).cuda()
    sc = bits_to_device(L.scales, "f16")
    torch.cuda.synchronize()
    filler = []
    headroom = 24 << 20                        # leave a little for the runtime itself
    try:
        while True:
            free, _ = torch.cuda.mem_get_info()
            if free <= headroom + (1 << 20):
                break
            chunk = min(free - headroom, 8 << 30)
            try:
                filler.append(torch.empty(chunk, dtype=torch.uint8, device="cuda"))
            except torch.OutOfMemoryError:
                if chunk <= (64 << 20):
                    break
                headroom += 64 << 20
        free, _ = torch.cuda.mem_get_info()
        say("free after fill:", free)
        assert free < (K * N // 2) // 4
        with pytest.raises(wq.GPTQError) as e:
            wq.repack(qw, qz, sc, None, bits=4, group_size=128)
        assert e.value.name == "E_OOM"
    finally:
        del filler
        torch.cuda.empty_cache()
    h = wq.repack(qw, qz, sc, None, bits=4, group_size=128)
    assert h.info()["runtime_bytes"] >= K * N // 2
    h.close()
