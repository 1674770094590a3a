"""Helpers shared by the GPU tests: move generator output to the device and to fp64."""
import numpy as np

from oracle.formats import bf16_bits_to_f64

# Tolerances of the bf16 path against the fp64 oracle.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def to_device(x, dtype):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def to_f64(x, dtype):
    """Exact fp64 values of what the GPU consumes."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    return bf16_bits_to_f64(x)


def out_to_f64(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.cpu().numpy().astype(np.float64)


def compare(o, lse, o_ref, lse_ref, max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS, lse_abs=LSE_ABS, what=""):
    """Element-wise comparison; -inf LSE (rows that see no key) must match exactly."""
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    assert err.max() <= max_abs, f"{what}: max |O err| {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{what}: mean |O err| {err.mean():.3e} > {mean_abs}"
    inf_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), inf_ref, err_msg=f"{what}: -inf LSE rows differ")
    if (~inf_ref).any():
        le = np.abs(lse[~inf_ref] - lse_ref[~inf_ref])
        assert le.max() <= lse_abs, f"{what}: max |LSE err| {le.max():.3e} > {lse_abs}"
    return float(err.max()), float(err.mean())
