"""Torch-facing wrappers of the C ABI: AWQ per-layer search on one MI355X.

PyTorch provides device memory and the current HIP stream; every computation
runs in the HIP library through the C ABI. Tensors must live on the GPU and be
contiguous. Defaults follow the AutoAWQ configuration the roadmap page prints
in section 9 (zero point on, group 128, 4 bits).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.AWQ_F32, torch.bfloat16: L.AWQ_BF16, torch.float16: L.AWQ_F16}

DEFAULT_BITS = 4
DEFAULT_GROUP = 128
DEFAULT_ZERO_POINT = True


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def workspace_bytes(op: int, T: int, N: int, K: int, n_grid: int, dtype: torch.dtype) -> int:
    return int(L.lib().awq_workspace_bytes(op, T, N, K, n_grid, _DT[dtype]))


def workspace_bytes_batch(op: int, T: int, N: int, K: int, n_grid: int, batch: int,
                          dtype: torch.dtype) -> int:
    return int(L.lib().awq_workspace_bytes_batch(op, T, N, K, n_grid, batch, _DT[dtype]))


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is not None:
        return ws
    return torch.empty(max(need, 256), dtype=torch.uint8, device=device)


def qconfig(bits=DEFAULT_BITS, group=DEFAULT_GROUP, zero_point=DEFAULT_ZERO_POINT,
            split_e=False, fused=False) -> L.QConfig:
    return L.QConfig(int(bits), int(group), int(bool(zero_point)),
                     (L.AWQ_SEARCH_SPLIT_E if split_e else 0) |
                     (L.AWQ_SEARCH_FUSED if fused else 0))


def _direct_op(op: int, split_e: bool, fused: bool = False) -> int:
    """The workspace op of a direct search, in its split or fused form when asked."""
    if fused:
        return {L.AWQ_OP_SEARCH_SCALE: L.AWQ_OP_SEARCH_SCALE_FUSED,
                L.AWQ_OP_SEARCH_CLIP: L.AWQ_OP_SEARCH_CLIP_FUSED}.get(op, op)
    if not split_e:
        return op
    return {L.AWQ_OP_SEARCH_SCALE: L.AWQ_OP_SEARCH_SCALE_SPLIT_E,
            L.AWQ_OP_SEARCH_CLIP: L.AWQ_OP_SEARCH_CLIP_SPLIT_E}.get(op, op)


def act_stats(X: torch.Tensor, ws: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-input-channel mean |x| over tokens: X [T, K] -> abar [K] float32."""
    _dev(X, "X")
    T, K = X.shape
    abar = out if out is not None else torch.empty(K, dtype=torch.float32, device=X.device)
    ws = _workspace(ws, workspace_bytes(L.AWQ_OP_STATS, T, 1, K, 1, X.dtype), X.device)
    L.check(L.lib().awq_act_stats(_ptr(X), _dtype(X), T, K, _ptr(abar), _ptr(ws), ws.numel(),
                                  _stream()))
    return abar


def act_stats_noalloc(X: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act_stats through the entry point that allocates nothing (its partials
    live in a static device array shared by all such calls on a GPU; calls
    that overlap on one GPU race). ``out`` lets the caller avoid torch's
    allocation too."""
    _dev(X, "X")
    T, K = X.shape
    abar = out if out is not None else torch.empty(K, dtype=torch.float32, device=X.device)
    L.check(L.lib().awq_act_stats_noalloc(_ptr(X), _dtype(X), T, K, _ptr(abar), _stream()))
    return abar


def act_stats_accumulate(X: torch.Tensor, sums: torch.Tensor,
                         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sums[j] += Σ_t |x_tj| for one calibration batch X [T, K]; sums is a
    float64 [K] device tensor the caller zeroes before the first batch."""
    _dev(X, "X")
    _dev(sums, "sums")
    T, K = X.shape
    if sums.dtype != torch.float64 or sums.numel() != K:
        raise ValueError("sums must be a float64 tensor of K elements")
    ws = _workspace(ws, workspace_bytes(L.AWQ_OP_STATS, T, 1, K, 1, X.dtype), X.device)
    L.check(L.lib().awq_act_stats_accumulate(_ptr(X), _dtype(X), T, K, _ptr(sums), _ptr(ws),
                                             ws.numel(), _stream()))
    return sums


def act_stats_finalize(sums: torch.Tensor, count: int,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """abar_j = fl32(sums_j / count), count = all calibration tokens."""
    _dev(sums, "sums")
    K = sums.numel()
    abar = out if out is not None else torch.empty(K, dtype=torch.float32, device=sums.device)
    L.check(L.lib().awq_act_stats_finalize(_ptr(sums), count, K, _ptr(abar), _stream()))
    return abar


def scale_table(abar: torch.Tensor, alphas: Sequence[float]) -> torch.Tensor:
    """s[a][j] = abar_j^alpha_a / sqrt(max abar^alpha_a * min abar^alpha_a), float32."""
    _dev(abar, "abar")
    n = len(alphas)
    out = torch.empty((n, abar.numel()), dtype=torch.float32, device=abar.device)
    L.check(L.lib().awq_scale_table(_ptr(abar), abar.numel(), L.float_array(alphas), n, _ptr(out),
                                    _stream()))
    return out


_METHODS = ("direct", "gram")


def _method(method: str, G: Optional[torch.Tensor] = None) -> bool:
    if method not in _METHODS:
        raise ValueError(f"method must be one of {_METHODS}")
    if G is not None:
        if method != "gram":
            raise ValueError("a prepared Gram matrix G goes with method='gram'")
        _dev(G, "G")
    return method == "gram"


def gram_bytes(K: int) -> int:
    return int(L.lib().awq_gram_bytes(K))


def gram_build(X: torch.Tensor, ws: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """G = XᵀX of a bf16 layer input [T, K], in the layout the Gram searches
    read (a uint8 device buffer of gram_bytes(K) bytes). Pass it as ``G=`` to
    search_scale, search_clip and search_scale_group (method "gram") of every
    layer that reads X, instead of building it in each search."""
    _dev(X, "X")
    T, K = X.shape
    nbytes = gram_bytes(K)
    G = out if out is not None else torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    ws = _workspace(ws, workspace_bytes(L.AWQ_OP_GRAM_BUILD, T, 1, K, 1, X.dtype), X.device)
    L.check(L.lib().awq_gram_build(_ptr(X), _dtype(X), T, K, _ptr(G), G.numel() * G.element_size(),
                                   _ptr(ws), ws.numel(), _stream()))
    return G


def search_scale(X: torch.Tensor, W: torch.Tensor, abar: torch.Tensor, alphas: Sequence[float],
                 bits: int = DEFAULT_BITS, group: int = DEFAULT_GROUP,
                 zero_point: bool = DEFAULT_ZERO_POINT, want_row_sums: bool = False,
                 ws: Optional[torch.Tensor] = None, method: str = "direct",
                 G: Optional[torch.Tensor] = None, split_e: bool = False,
                 fused: bool = False) -> dict:
    """Grid search over alpha. Returns alpha_best, index, s_best [K], mse (numpy
    [n_alpha]) and, if asked, row_sums [n_alpha, N] float64 on the GPU.
    method "direct" measures X·Eᵀ per candidate; "gram" (bf16 only) uses the
    activations' Gram matrix, E·G·Eᵀ per candidate row, built in the call or
    taken from ``G`` (gram_build(X)). split_e (direct method): candidates go
    to the matrix cores as hi + lo 16-bit halves (twice the GEMM work).
    fused (direct method, 16-bit, N a multiple of 256): the search GEMM forms
    the candidates itself from W and per-group parameters; same results."""
    gram = _method(method, G)
    _dev(X, "X"), _dev(W, "W"), _dev(abar, "abar")
    if X.dtype != W.dtype:
        raise ValueError("X and W must share a dtype")
    T, K = X.shape
    N = W.shape[0]
    n = len(alphas)
    op = (L.AWQ_OP_SEARCH_SCALE_GRAM_G if G is not None else
          L.AWQ_OP_SEARCH_SCALE_GRAM if gram else
          _direct_op(L.AWQ_OP_SEARCH_SCALE, split_e, fused))
    ws = _workspace(ws, workspace_bytes(op, T, N, K, n, X.dtype), X.device)
    s_best = torch.empty(K, dtype=torch.float32, device=X.device)
    rows = torch.empty((n, N), dtype=torch.float64, device=X.device) if want_row_sums else None
    a_best = ctypes.c_float(0.0)
    mse = (ctypes.c_double * n)()
    grid = L.float_array(alphas)
    fn = (L.lib().awq_search_scale_gram_g if G is not None else
          L.lib().awq_search_scale_gram if gram else L.lib().awq_search_scale)
    L.check(fn(_ptr(G if G is not None else X), _ptr(W), _dtype(X), T, N, K, _ptr(abar), grid, n,
               qconfig(bits, group, zero_point, split_e, fused), _ptr(s_best),
               ctypes.byref(a_best), mse, _ptr(rows), _ptr(ws), ws.numel(), _stream()))
    mse_np = np.array(mse[:], dtype=np.float64)
    g32 = np.asarray(alphas, dtype=np.float32)
    idx = int(np.flatnonzero(g32 == np.float32(a_best.value))[0])
    return dict(alpha_best=np.float32(a_best.value), index=idx, s_best=s_best, mse=mse_np,
                row_sums=rows)


def search_scale_group(X: torch.Tensor, Ws: Sequence[torch.Tensor], abar: torch.Tensor,
                       alphas: Sequence[float], bits: int = DEFAULT_BITS,
                       group: int = DEFAULT_GROUP, zero_point: bool = DEFAULT_ZERO_POINT,
                       want_row_sums: bool = False, ws: Optional[torch.Tensor] = None,
                       method: str = "direct", G: Optional[torch.Tensor] = None,
                       split_e: bool = False) -> dict:
    """One alpha search for linears that read the same X (one shared s): the
    error is averaged over all their outputs. Same result dict as
    ``search_scale``; row_sums [n_alpha, sum N] keeps the layers in order.
    method "gram" (bf16) scores all layers through one G = XᵀX (or ``G``)."""
    gram = _method(method, G)
    _dev(X, "X"), _dev(abar, "abar")
    if not 1 <= len(Ws) <= 16:
        raise ValueError("a group holds 1 to 16 layers")
    for i, W in enumerate(Ws):
        _dev(W, f"Ws[{i}]")
        if W.dtype != X.dtype or W.shape[1] != X.shape[1]:
            raise ValueError(f"Ws[{i}] must be [N, K] with X's dtype and K")
    T, K = X.shape
    Ns = [int(W.shape[0]) for W in Ws]
    N = sum(Ns)
    n = len(alphas)
    op = (L.AWQ_OP_SEARCH_SCALE_GRAM_G if G is not None else
          L.AWQ_OP_SEARCH_SCALE_GRAM if gram else _direct_op(L.AWQ_OP_SEARCH_SCALE, split_e))
    ws = _workspace(ws, workspace_bytes(op, T, N, K, n, X.dtype), X.device)
    s_best = torch.empty(K, dtype=torch.float32, device=X.device)
    rows = torch.empty((n, N), dtype=torch.float64, device=X.device) if want_row_sums else None
    a_best = ctypes.c_float(0.0)
    mse = (ctypes.c_double * n)()
    wptrs = (ctypes.c_void_p * len(Ws))(*[W.data_ptr() for W in Ws])
    nvals = (ctypes.c_int64 * len(Ws))(*Ns)
    fn = (L.lib().awq_search_scale_group_gram_g if G is not None else
          L.lib().awq_search_scale_group_gram if gram else L.lib().awq_search_scale_group)
    L.check(fn(_ptr(G if G is not None else X), wptrs, nvals, len(Ws), _dtype(X), T, K, _ptr(abar), L.float_array(alphas),
               n, qconfig(bits, group, zero_point, split_e), _ptr(s_best), ctypes.byref(a_best),
               mse,
               _ptr(rows), _ptr(ws), ws.numel(), _stream()))
    mse_np = np.array(mse[:], dtype=np.float64)
    g32 = np.asarray(alphas, dtype=np.float32)
    idx = int(np.flatnonzero(g32 == np.float32(a_best.value))[0])
    return dict(alpha_best=np.float32(a_best.value), index=idx, s_best=s_best, mse=mse_np,
                row_sums=rows)


def fold_norm(gamma: torch.Tensor, s: torch.Tensor, beta: Optional[torch.Tensor] = None) -> None:
    """In place: gamma /= s (and beta /= s) per channel, for the normalisation
    that produces the searched layer's input."""
    _dev(gamma, "gamma"), _dev(s, "s")
    if beta is not None:
        _dev(beta, "beta")
        if beta.dtype != gamma.dtype or beta.numel() != gamma.numel():
            raise ValueError("beta must match gamma")
    if s.dtype != torch.float32 or s.numel() != gamma.numel():
        raise ValueError("s must be float32 with one value per channel")
    L.check(L.lib().awq_fold_norm(_ptr(gamma), _ptr(beta), _dtype(gamma), gamma.numel(), _ptr(s),
                                  _stream()))


def fold_linear(W_prev: torch.Tensor, s: torch.Tensor, bias: Optional[torch.Tensor] = None) -> None:
    """In place: row j of W_prev [K, K_prev] (and bias[j]) /= s[j], for the
    linear whose outputs are the searched layer's inputs."""
    _dev(W_prev, "W_prev"), _dev(s, "s")
    K, K_prev = W_prev.shape
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != W_prev.dtype or bias.numel() != K:
            raise ValueError("bias must be [K] with W_prev's dtype")
    if s.dtype != torch.float32 or s.numel() != K:
        raise ValueError("s must be float32 with one value per output channel of W_prev")
    L.check(L.lib().awq_fold_linear(_ptr(W_prev), _ptr(bias), _dtype(W_prev), K, K_prev, _ptr(s),
                                    _stream()))


def search_clip(X: torch.Tensor, W: torch.Tensor, s: torch.Tensor, ratios: Sequence[float],
                bits: int = DEFAULT_BITS, group: int = DEFAULT_GROUP,
                zero_point: bool = DEFAULT_ZERO_POINT, want_row_sums: bool = False,
                ws: Optional[torch.Tensor] = None, method: str = "direct",
                G: Optional[torch.Tensor] = None, split_e: bool = False,
                fused: bool = False) -> dict:
    """Per-output-channel clip-ratio search with s fixed. Returns ratio_best [N]
    (GPU), mse_clip (float) and optionally row_sums [n_ratio, N]. method, G,
    split_e and fused as in search_scale."""
    gram = _method(method, G)
    _dev(X, "X"), _dev(W, "W"), _dev(s, "s")
    if X.dtype != W.dtype:
        raise ValueError("X and W must share a dtype")
    T, K = X.shape
    N = W.shape[0]
    n = len(ratios)
    op = (L.AWQ_OP_SEARCH_CLIP_GRAM_G if G is not None else
          L.AWQ_OP_SEARCH_CLIP_GRAM if gram else
          _direct_op(L.AWQ_OP_SEARCH_CLIP, split_e, fused))
    ws = _workspace(ws, workspace_bytes(op, T, N, K, n, X.dtype), X.device)
    r_best = torch.empty(N, dtype=torch.float32, device=X.device)
    rows = torch.empty((n, N), dtype=torch.float64, device=X.device) if want_row_sums else None
    mse_clip = ctypes.c_double(0.0)
    fn = (L.lib().awq_search_clip_gram_g if G is not None else
          L.lib().awq_search_clip_gram if gram else L.lib().awq_search_clip)
    L.check(fn(_ptr(G if G is not None else X), _ptr(W), _dtype(X), T, N, K, _ptr(s), L.float_array(ratios), n,
               qconfig(bits, group, zero_point, split_e, fused), _ptr(r_best),
               ctypes.byref(mse_clip),
               _ptr(rows),
               _ptr(ws), ws.numel(), _stream()))
    return dict(ratio_best=r_best, mse_clip=float(mse_clip.value), row_sums=rows)


def quantize_pack(W: torch.Tensor, s: torch.Tensor, ratio: Optional[torch.Tensor] = None,
                  bits: int = DEFAULT_BITS, group: int = DEFAULT_GROUP,
                  zero_point: bool = DEFAULT_ZERO_POINT, ws: Optional[torch.Tensor] = None,
                  out=None):
    """Packed layer: qweight [K, N·b/32] int32, qzeros [K/g, N·b/32] int32,
    scales [K/g, N] float16 (b = bits, 4 or 3; codes packed densely along the
    output dim, lowest bits first)."""
    _dev(W, "W"), _dev(s, "s")
    if ratio is not None:
        _dev(ratio, "ratio")
    N, K = W.shape
    if out is None:
        nw = N * int(bits) // 32
        qweight = torch.empty((K, nw), dtype=torch.int32, device=W.device)
        qzeros = torch.empty((K // group, nw), dtype=torch.int32, device=W.device)
        scales = torch.empty((K // group, N), dtype=torch.float16, device=W.device)
    else:
        qweight, qzeros, scales = out
    ws = _workspace(ws, workspace_bytes(L.AWQ_OP_PACK, 1, N, K, 1, W.dtype), W.device)
    L.check(L.lib().awq_quantize_pack(_ptr(W), _dtype(W), N, K, _ptr(s), _ptr(ratio),
                                      qconfig(bits, group, zero_point), _ptr(qweight),
                                      _ptr(qzeros), _ptr(scales), _ptr(ws), ws.numel(), _stream()))
    return qweight, qzeros, scales


def w4a16_workspace_bytes(T: int, N: int, K: int, dtype: torch.dtype) -> int:
    return int(L.lib().awq_w4a16_workspace_bytes(T, N, K, _DT[dtype]))


def w3a16_workspace_bytes(T: int, N: int, K: int, dtype) -> int:
    return int(L.lib().awq_w3a16_workspace_bytes(T, N, K, _DT[dtype]))


def w4a16_matmul(X: torch.Tensor, qweight: torch.Tensor, qzeros: torch.Tensor,
                 scales: torch.Tensor, group: int = DEFAULT_GROUP,
                 ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 bits: int = 4, on_the_fly: bool = False):
    """Y = X·Ŵᵀ for a packed layer (bits 4: qweight [K, N/8], qzeros
    [K/g, N/8]; bits 3: [K, 3N/32] and [K/g, 3N/32]; scales [K/g, N] float16)
    and activations X [T, K] (bf16 or float16, already divided by s). Returns
    Y [T, N] in X's dtype. on_the_fly (4 bits, T > 16): the GEMM dequantises
    as it goes and takes no workspace (same result, slower)."""
    _dev(X, "X"), _dev(qweight, "qweight"), _dev(qzeros, "qzeros"), _dev(scales, "scales")
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    T, K = X.shape
    N = scales.shape[1]
    cols = N * bits // 32
    if qweight.shape != (K, cols) or qzeros.shape != (K // group, cols) or \
            scales.shape != (K // group, N):
        raise ValueError("packed layer shapes do not match X and the group size")
    Y = out if out is not None else torch.empty((T, N), dtype=X.dtype, device=X.device)
    if bits == 4:
        fn, need = L.lib().awq_w4a16_matmul, w4a16_workspace_bytes(T, N, K, X.dtype)
    else:
        fn, need = L.lib().awq_w3a16_matmul, w3a16_workspace_bytes(T, N, K, X.dtype)
    if on_the_fly and bits == 4 and T > 16:
        L.check(fn(_ptr(X), _dtype(X), T, N, K, _ptr(qweight), _ptr(qzeros), _ptr(scales),
                   int(group), _ptr(Y), None, 0, _stream()))
        return Y
    ws = _workspace(ws, need, X.device)
    L.check(fn(_ptr(X), _dtype(X), T, N, K, _ptr(qweight), _ptr(qzeros), _ptr(scales), int(group),
               _ptr(Y), _ptr(ws), ws.numel(), _stream()))
    return Y


def profile_enable(on: bool = True) -> None:
    L.lib().awq_profile_enable(1 if on else 0)


def profile_reset() -> None:
    L.lib().awq_profile_reset()


def profile_read(kind: str):
    """(total milliseconds, launches) of one kernel kind since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    L.check(L.lib().awq_profile_read(L.KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
