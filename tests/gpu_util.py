"""Shared helpers of the GPU tests: move seeded numpy inputs to the device and call the library.
Nothing here computes the method: expected values come from oracle/ only."""
import numpy as np

import oracle as o
import gptq_inputs as gi

TOL = {"f16": dict(rel_l2=1e-3, max_abs_over_rms=2e-2), "bf16": dict(rel_l2=4e-3, max_abs_over_rms=2e-2)}


def torch_dtype(tag):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[tag]


def bits_to_device(a, tag):
    """uint16 bit patterns (or float32) -> torch tensor of that float dtype on cuda:0."""
    import torch
    if tag == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).cuda()
    return t.view(torch_dtype(tag))


def device_to_bits(t):
    import torch
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def repack_layer(L: gi.Layer, use_gidx=True):
    import torch
    import weight_only_quantized_amd as wq
    qw = torch.from_numpy(np.ascontiguousarray(L.qweight)).cuda()
    qz = torch.from_numpy(np.ascontiguousarray(L.qzeros)).cuda()
    sc = bits_to_device(L.scales, L.scales_dtype)
    g = torch.from_numpy(np.ascontiguousarray(L.g_idx, dtype=np.int32)).cuda() if use_gidx else None
    h = wq.repack(qw, qz, sc, g, bits=L.bits, group_size=L.group_size, desc_act=L.desc_act)
    return h


def repack_awq_layer(L: gi.AwqLayer):
    import torch
    import weight_only_quantized_amd as wq
    qw = torch.from_numpy(np.ascontiguousarray(L.qweight)).cuda()
    qz = torch.from_numpy(np.ascontiguousarray(L.qzeros)).cuda()
    sc = bits_to_device(L.scales, L.scales_dtype)
    return wq.repack(qw, qz, sc, None, bits=4, group_size=L.group_size, checkpoint_format="awq_gemm")


def run_gemm(h, x_bits, x_tag, path=0, bias=None, bias_tag=None):
    """One gemm call (gptq_gemm_bias when `bias`, bit patterns in `bias_tag`, is given)."""
    x = bits_to_device(x_bits, x_tag)
    b = bits_to_device(bias, bias_tag) if bias is not None else None
    y = h.gemm(x, path=path, bias=b)
    import torch
    torch.cuda.synchronize()
    return device_to_bits(y)


def out_ulp(y_ref, x_tag):
    """One unit in the last place of the output dtype (fp16: 10 fraction bits, bf16: 7) at |y_ref|
    (the subnormal step below the normal range)."""
    frac, emin = (10, -14) if x_tag == "f16" else (7, -126)
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(y_ref, dtype=np.float64)), 2.0 ** emin)))
    return np.ldexp(1.0, (e - frac).astype(np.int64))


def check(y_bits, x_tag, y_ref, label=""):
    """rel-L2 and max-abs bars of the layer (rel-L2 1e-3 for fp16 outputs, 4e-3 for bf16; max-abs
    2e-2 * rms(y_ref)).  The max-abs bar sits below the output dtype's own rounding for outputs far
    above the rms (bf16 carries 8 significant bits, so beyond ~10 rms half a unit in the last place
    exceeds 2e-2 * rms): only for those elements, where half an ulp of y_ref is larger than the bar,
    the bound is half an ulp plus the bar (the correctly rounded result is within half an ulp of the
    fp32 sum, and the fp32 sum within far less than the bar of y_ref).  Every other element keeps
    the bar itself."""
    m = o.compare(y_bits, x_tag, y_ref)
    tol = TOL[x_tag]
    assert m["nonfinite"] == 0, (label, m)
    assert m["rel_l2"] <= tol["rel_l2"], (label, m)
    if m["max_abs_over_rms"] > tol["max_abs_over_rms"]:
        y = o.decode_float_bits(y_bits, x_tag)
        ref = np.asarray(y_ref, dtype=np.float64)
        bar = tol["max_abs_over_rms"] * m["rms_ref"]
        half_ulp = 0.5 * out_ulp(ref, x_tag)
        wide = half_ulp > bar
        err = np.abs(y - ref)
        assert np.all(err[~wide] <= bar), (label, m, float(err[~wide].max()) / m["rms_ref"])
        assert np.all(err[wide] <= half_ulp[wide] + bar), (label, m)
        print(f"half-ulp bar used: {label} ({int(np.count_nonzero(wide & (err > bar)))} outputs past "
              f"2e-2 rms, {int(np.count_nonzero(wide))} where half an ulp exceeds it)", flush=True)
    return m


def check_runtime_perm(perm, g_idx, group_size):
    """The decoded load-time order against what the sort by g_idx fixes: a permutation of the inputs
    under which every group is contiguous, groups ascending (oracle runtime_perm gives one such
    order, the stable one).  The order within a group is free (a group shares one scale and one zero
    per output).  The library keeps the stable order except for act-order layers that the skinny
    kernel stages whole in LDS (padded K <= 8192, every group a multiple of 128 inputs): there the
    inputs 512 b + 8 L + e (lanes L = 0..63 of one 2-byte LDS write instruction) must land on 64
    distinct LDS banks (4-byte words mod 64), and on 32 distinct banks mod 32 within each half-wave.
    Checked from the decoded order alone."""
    g = np.asarray(g_idx, dtype=np.int64)
    K = g.shape[0]
    perm = np.asarray(perm, dtype=np.int64)
    stable = o.runtime_perm(g)
    assert np.array_equal(np.sort(perm), np.arange(K)), "not a permutation"
    assert np.array_equal(g[perm], g[stable]), "groups not contiguous in ascending order"
    gse = K if group_size == -1 else group_size
    Kp = -(-K // 128) * 128
    spread = not np.array_equal(stable, np.arange(K)) and Kp <= 8192 and K % 128 == 0 and gse % 128 == 0
    if not spread:
        assert np.array_equal(perm, stable)
        return
    pos = np.empty(K, np.int64)
    pos[perm] = np.arange(K)
    lanes = np.arange(64)
    for blk in range(-(-K // 512)):
        for e in range(8):
            ks = blk * 512 + lanes * 8 + e
            real = ks < K
            banks = (pos[ks[real]] >> 1) & 63
            assert len(np.unique(banks)) == banks.size, (blk, e)
            for half in (0, 1):
                b = banks[(lanes[real] >> 5) == half] & 31
                assert len(np.unique(b)) == b.size, (blk, e, half)
