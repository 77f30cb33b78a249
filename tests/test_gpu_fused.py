"""GPU: the fused search (AWQ_SEARCH_FUSED) against the two-pass search.

The fused search forms each candidate's error weights inside the search
GEMM, from W and the per-(candidate, row, group) step, zero point and
reciprocal of a parameter pass, with the transform kernel's arithmetic
operation for operation ("05 — AWQ: Activation-Aware Weight Scaling",
section 4: scale, quantise, measure the output error). Its operand is
therefore the two-pass path's bit for bit, and the MFMAs accumulate in the
same order, so every per-row output error, the curve, α*, the clip ratios
and mse_clip must be identical (the two-pass path itself is held to the
oracle by test_gpu_parity and test_gpu_fullsize).
"""
import numpy as np
import pytest
import torch

from post_weight_quantization_26_amd import synth
from test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    from post_weight_quantization_26_amd import api as A
    return A


def log(msg):
    print(msg, flush=True)


CASES = [
    # T (ragged), N (multiple of 256), K, group, bits, zero point, dtype
    (300, 512, 384, 128, 4, True, "bf16"),
    (520, 256, 512, 64, 4, False, "f16"),
    (257, 768, 256, 32, 3, True, "bf16"),
    (700, 1024, 640, 32, 4, True, "f16"),
    (4096, 4096, 4096, 128, 4, True, "bf16"),
    (129, 256, 128, 32, 4, True, "bf16"),     # K = 128: two k-tiles
    (64, 512, 128, 128, 3, False, "f16"),
]


@pytest.mark.parametrize("T,N,K,group,bits,zp,dtype", CASES)
def test_fused_equals_two_pass(api, T, N, K, group, bits, zp, dtype):
    log(f"fused T={T} N={N} K={K} g={group} b={bits} zp={zp} {dtype}")
    X, W = synth.make_custom(T, N, K, dtype, seed=T + N + K)
    Xd, Wd = to_dev(X, dtype), to_dev(W, dtype)
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(20)
    ref = api.search_scale(Xd, Wd, abar, alphas, bits=bits, group=group, zero_point=zp,
                           want_row_sums=True)
    fus = api.search_scale(Xd, Wd, abar, alphas, bits=bits, group=group, zero_point=zp,
                           want_row_sums=True, fused=True)
    assert np.array_equal(ref["mse"], fus["mse"]), (ref["mse"], fus["mse"])
    assert ref["index"] == fus["index"]
    assert torch.equal(ref["row_sums"], fus["row_sums"])
    ratios = synth.ratio_grid(20)
    rc = api.search_clip(Xd, Wd, ref["s_best"], ratios, bits=bits, group=group, zero_point=zp,
                         want_row_sums=True)
    fc = api.search_clip(Xd, Wd, ref["s_best"], ratios, bits=bits, group=group, zero_point=zp,
                         want_row_sums=True, fused=True)
    assert rc["mse_clip"] == fc["mse_clip"]
    assert torch.equal(rc["ratio_best"], fc["ratio_best"])
    assert torch.equal(rc["row_sums"], fc["row_sums"])


def test_fused_batches(api):
    # fused workspaces for 3 candidates (α) and 1 candidate (ratios) at a
    # time: the candidate offsets of later batches (scale rows and ratios)
    # must line up
    T, N, K = 520, 512, 512
    X, W = synth.make_custom(T, N, K, "bf16", seed=5)
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(11)
    ws = torch.empty(api.workspace_bytes_batch(api.L.AWQ_OP_SEARCH_SCALE_FUSED, T, N, K,
                                               len(alphas), 3, Xd.dtype),
                     dtype=torch.uint8, device="cuda:0")
    ref = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True)
    fus = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, ws=ws, fused=True)
    assert np.array_equal(ref["mse"], fus["mse"])
    assert torch.equal(ref["row_sums"], fus["row_sums"])
    ratios = synth.ratio_grid(7)
    wsc = torch.empty(api.workspace_bytes_batch(api.L.AWQ_OP_SEARCH_CLIP_FUSED, T, N, K,
                                                len(ratios), 1, Xd.dtype),
                      dtype=torch.uint8, device="cuda:0")
    rc = api.search_clip(Xd, Wd, ref["s_best"], ratios, want_row_sums=True)
    fc = api.search_clip(Xd, Wd, ref["s_best"], ratios, want_row_sums=True, ws=wsc, fused=True)
    assert torch.equal(rc["row_sums"], fc["row_sums"])
    assert torch.equal(rc["ratio_best"], fc["ratio_best"])
