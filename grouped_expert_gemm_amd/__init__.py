"""MoE expert feed-forward hot path on AMD MI355X (gfx950): Python binding.

Thin argument marshalling over the C ABI of include/moe.h: every step runs in
the HIP kernels of libmoe.so; torch only provides device memory and the
current stream. The functions carry the C entry points' names.

Path (per "Efficient MoE Training for Biological Foundation Models",
Challenges 1-3): moe_route_topk -> moe_permute -> moe_grouped_mlp_fwd
(gate_up grouped GEMM + ScaledSwiGLU, down grouped GEMM) ->
moe_unpermute_combine; moe_grouped_mlp_bwd for the backward; mxfp8_quantize
for MXFP8 block quantisation.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, MOE_FP8, MOE_MXFP8, MlpDesc, MoeError, check, lib, ptr_table

__all__ = [
    "moe_route_topk", "moe_router_logits", "moe_route_topk_bwd", "moe_router_bwd", "moe_permute", "moe_unpermute_combine", "mxfp8_quantize",
    "fp8_tensor_quantize", "mxfp8_quantize_colwise", "fp8_tensor_quantize_colwise", "mxfp8_pack_weight_bwd",
    "fp8_tensor_pack_weight_bwd", "mxfp8_quantize_weights", "fp8_tensor_quantize_weights",
    "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd", "moe_grouped_linear", "moe_grouped_gate_up_swiglu", "gemm_workspace",
    "workspace_size", "MoeError", "lib",
    "MOE_F32", "MOE_BF16", "MOE_MXFP8", "MOE_FP8",
]

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_MXFP8}


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def workspace_size(op, desc=None, R=0, T=0, E=1, k=1):
    n = ctypes.c_size_t(0)
    check("moe_workspace_size", lib().moe_workspace_size(op, ctypes.byref(desc) if desc is not None else None,
                                                         R, T, E, k, ctypes.byref(n)))
    return n.value


def moe_route_topk(logits: torch.Tensor, k: int, renormalize: bool = True):
    """logits [T, E] float32 -> (topk_idx int32 [T, k], topk_prob float32 [T, k])."""
    _need_cuda(logits)
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    prob = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    check("moe_route_topk", lib().moe_route_topk(_p(logits), T, E, k, int(renormalize), _p(idx), _p(prob),
                                                 _stream(logits.device)))
    return idx, prob


def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor) -> torch.Tensor:
    """x [T, H] bf16, w_router [E, H] bf16 -> logits [T, E] float32."""
    _need_cuda(x, w_router)
    T, H = x.shape
    E = w_router.shape[0]
    if x.dtype != torch.bfloat16 or w_router.dtype != torch.bfloat16 or w_router.shape[1] != H:
        raise ValueError("moe_router_logits: x [T, H] and w_router [E, H] must be bfloat16")
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    check("moe_router_logits", lib().moe_router_logits(_p(x), _p(w_router), T, H, E, _p(logits),
                                                       _stream(x.device)))
    return logits


def moe_route_topk_bwd(topk_idx: torch.Tensor, topk_prob: torch.Tensor, d_topk_prob: torch.Tensor, E: int,
                       renormalize: bool = True, logits: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient of moe_route_topk's probabilities -> d_logits [T, E] float32
    (``logits`` is needed only without renormalisation)."""
    _need_cuda(topk_idx, topk_prob, d_topk_prob, logits)
    T, k = topk_idx.shape
    d = torch.empty((T, E), dtype=torch.float32, device=topk_idx.device)
    check("moe_route_topk_bwd", lib().moe_route_topk_bwd(_p(logits), _p(topk_idx), _p(topk_prob), _p(d_topk_prob),
                                                         T, E, k, int(renormalize), _p(d),
                                                         _stream(topk_idx.device)))
    return d


def moe_router_bwd(x: torch.Tensor, w_router: torch.Tensor, d_logits: torch.Tensor,
                   dx_in: torch.Tensor | None = None, dx: torch.Tensor | None = None):
    """Backward of moe_router_logits -> (dx [T, H] bf16 = dx_in + d_logits w_router,
    dw_router [E, H] float32 = d_logits^T x)."""
    _need_cuda(x, w_router, d_logits, dx_in, dx)
    T, H = x.shape
    E = w_router.shape[0]
    if dx is None:
        dx = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    dw = torch.empty((E, H), dtype=torch.float32, device=x.device)
    desc = MlpDesc(E, H, 1, 0, MOE_BF16, MOE_BF16, 0)
    ws = _workspace(workspace_size(_lib.MOE_OP_ROUTER_BWD, desc, 0, T), x.device)
    check("moe_router_bwd", lib().moe_router_bwd(_p(x), _p(w_router), _p(d_logits), _p(dx_in), T, H, E, _p(dx),
                                                 _p(dw), _p(ws), ws.numel(), _stream(x.device)))
    return dx, dw


def moe_permute(x: torch.Tensor, topk_idx: torch.Tensor, topk_prob: torch.Tensor | None, E: int,
                x_scale: torch.Tensor | None = None, row_id_map: torch.Tensor | None = None):
    """Group the (token, slot) pairs by expert.

    Returns a dict with x_perm [R, H], x_perm_scale (MXFP8 only), prob_perm [R],
    split_sizes [E], offsets [E+1], row_id_map [T*k], src_token [R].
    With ``row_id_map`` given, only x is gathered with that map (topk_idx gives k).
    """
    _need_cuda(x, topk_idx, topk_prob, x_scale, row_id_map)
    T, H = x.shape
    k = topk_idx.shape[1]
    R = T * k
    dt = _DT[x.dtype]
    dev = x.device
    x_perm = torch.empty((R, H), dtype=x.dtype, device=dev)
    xps = torch.empty((R, H // 32), dtype=torch.uint8, device=dev) if dt == MOE_MXFP8 else None
    if row_id_map is not None:
        check("moe_permute", lib().moe_permute(_p(x), _p(x_scale), dt, T, H, E, k, None, None, 1, _p(x_perm),
                                               _p(xps), None, None, None, _p(row_id_map), None, None, 0,
                                               _stream(dev)))
        return dict(x_perm=x_perm, x_perm_scale=xps)
    prob_perm = torch.empty(R, dtype=torch.float32, device=dev) if topk_prob is not None else None
    split = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rmap = torch.empty(R, dtype=torch.int32, device=dev)
    src = torch.empty(R, dtype=torch.int32, device=dev)
    ws = _workspace(workspace_size(_lib.MOE_OP_PERMUTE, None, 0, T, E, k), dev)
    check("moe_permute", lib().moe_permute(_p(x), _p(x_scale), dt, T, H, E, k, _p(topk_idx), _p(topk_prob), 0,
                                           _p(x_perm), _p(xps), _p(prob_perm), _p(split), _p(offsets), _p(rmap),
                                           _p(src), _p(ws), ws.numel(), _stream(dev)))
    return dict(x_perm=x_perm, x_perm_scale=xps, prob_perm=prob_perm, split_sizes=split, offsets=offsets,
                row_id_map=rmap, src_token=src)


def moe_unpermute_combine(y_perm: torch.Tensor, row_id_map: torch.Tensor, T: int, k: int,
                          weights: torch.Tensor | None = None):
    """out[t] = sum_j w[t, j] * y_perm[row_id_map[t*k + j]] (w = 1 without weights)."""
    _need_cuda(y_perm, row_id_map, weights)
    H = y_perm.shape[1]
    out = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device)
    check("moe_unpermute_combine", lib().moe_unpermute_combine(_p(y_perm), _DT[y_perm.dtype], _p(row_id_map),
                                                               _p(weights), T, H, k, _p(out),
                                                               _stream(y_perm.device)))
    return out


def mxfp8_quantize(x: torch.Tensor):
    """bf16 [rows, cols] -> (E4M3 codes uint8 [rows, cols], E8M0 scales uint8 [rows, cols/32])."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16:
        raise ValueError("mxfp8_quantize takes bfloat16")
    x2 = x.reshape(-1, x.shape[-1])
    rows, cols = x2.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    check("mxfp8_quantize", lib().mxfp8_quantize(_p(x2), rows, cols, _p(codes), _p(scales), _stream(x.device)))
    return codes.reshape(x.shape), scales.reshape(*x.shape[:-1], cols // 32)


def fp8_tensor_quantize(x: torch.Tensor):
    """bf16 tensor -> (E4M3 codes uint8 of x's shape, float32 scale tensor of shape [1])."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16:
        raise ValueError("fp8_tensor_quantize takes bfloat16")
    x = x.contiguous()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    check("fp8_tensor_quantize", lib().fp8_tensor_quantize(_p(x), x.numel(), _p(codes), _p(scale),
                                                           _stream(x.device)))
    return codes, scale


def mxfp8_quantize_colwise(x: torch.Tensor, offsets: torch.Tensor, pad: int = 32):
    """bf16 [R, C] with expert row offsets [E+1] -> (E4M3 codes [C, kcap], E8M0 scales
    [C, kcap/32], padded offsets kofs [E+1]) with kcap = R + E * (pad - 1) rounded up to
    128 (whole cache lines per output row): each expert's rows, zero-padded to a
    multiple of pad, quantised along the token axis as columns [kofs[e], kofs[e+1])."""
    _need_cuda(x, offsets)
    if x.dtype != torch.bfloat16:
        raise ValueError("mxfp8_quantize_colwise takes bfloat16")
    x = x.contiguous()
    R, C = x.shape
    E = offsets.numel() - 1
    kcap = (R + E * (pad - 1) + 127) // 128 * 128
    codes = torch.zeros((C, kcap), dtype=torch.uint8, device=x.device)
    scales = torch.zeros((C, kcap // 32), dtype=torch.uint8, device=x.device)
    kofs = torch.empty(E + 1, dtype=torch.int32, device=x.device)
    check("mxfp8_quantize_colwise", lib().mxfp8_quantize_colwise(_p(x), R, C, E, _p(offsets), pad, kcap, _p(codes),
                                                                 _p(scales), _p(kofs), _stream(x.device)))
    return codes, scales, kofs


def fp8_tensor_quantize_colwise(x: torch.Tensor, offsets: torch.Tensor, pad: int = 256):
    """bf16 [R, C] with expert row offsets [E+1] -> (E4M3 codes [C, kcap], float32 scale
    [1], padded offsets kofs [E+1]) with kcap = R + E * (pad - 1) rounded up to 128: the
    per-tensor FP8 codes of x, each expert's rows zero-padded to a multiple of pad and
    transposed to columns [kofs[e], kofs[e+1])."""
    _need_cuda(x, offsets)
    if x.dtype != torch.bfloat16:
        raise ValueError("fp8_tensor_quantize_colwise takes bfloat16")
    x = x.contiguous()
    R, C = x.shape
    E = offsets.numel() - 1
    kcap = (R + E * (pad - 1) + 127) // 128 * 128
    codes = torch.zeros((C, kcap), dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    kofs = torch.empty(E + 1, dtype=torch.int32, device=x.device)
    check("fp8_tensor_quantize_colwise", lib().fp8_tensor_quantize_colwise(
        _p(x), R, C, E, _p(offsets), pad, kcap, _p(codes), _p(scale), _p(kofs), _stream(x.device)))
    return codes, scale, kofs


def fp8_tensor_pack_weight_bwd(w: torch.Tensor) -> torch.Tensor:
    """bf16 weight [rows, cols] -> packed per-tensor FP8 for moe_grouped_mlp_bwd (uint8,
    rows * cols + 4 bytes: the codes of w^T, then the float32 factor)."""
    _need_cuda(w)
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("fp8_tensor_pack_weight_bwd takes a 2-D bfloat16 weight")
    w = w.contiguous()
    rows, cols = w.shape
    packed = torch.empty(rows * cols + 16, dtype=torch.uint8, device=w.device)
    check("fp8_tensor_pack_weight_bwd", lib().fp8_tensor_pack_weight_bwd(_p(w), rows, cols, _p(packed),
                                                                         _stream(w.device)))
    return packed


def mxfp8_pack_weight_bwd(w: torch.Tensor) -> torch.Tensor:
    """bf16 weight [rows, cols] -> packed MXFP8 for moe_grouped_mlp_bwd (uint8, rows * cols
    * 33 / 32 bytes: the codes of w^T quantised along rows, then the step-major scales)."""
    _need_cuda(w)
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("mxfp8_pack_weight_bwd takes a 2-D bfloat16 weight")
    rows, cols = w.shape
    packed = torch.empty(rows * cols + rows * cols // 32, dtype=torch.uint8, device=w.device)
    check("mxfp8_pack_weight_bwd", lib().mxfp8_pack_weight_bwd(_p(w), rows, cols, _p(packed), _stream(w.device)))
    return packed


def _weight_stack(w, fn):
    _need_cuda(w)
    if w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError(f"{fn} takes bfloat16 weights [n, rows, cols]")
    return w.contiguous()


def mxfp8_quantize_weights(w: torch.Tensor):
    """bf16 weights [n, rows, cols] -> (E4M3 codes uint8 [n, rows, cols], E8M0 scales uint8
    [n, rows, cols/32], packed uint8 [n, rows * cols * 33 / 32]): for each weight the
    outputs of mxfp8_quantize and of mxfp8_pack_weight_bwd, from one read of it."""
    w = _weight_stack(w, "mxfp8_quantize_weights")
    n, rows, cols = w.shape
    codes = torch.empty((n, rows, cols), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, rows, cols // 32), dtype=torch.uint8, device=w.device)
    packed = torch.empty((n, rows * cols + rows * cols // 32), dtype=torch.uint8, device=w.device)
    tw, kw = _lib.ptr_table([w[i].data_ptr() for i in range(n)])
    tc, kc = _lib.ptr_table([codes[i].data_ptr() for i in range(n)])
    ts, ks = _lib.ptr_table([scales[i].data_ptr() for i in range(n)])
    tp, kp = _lib.ptr_table([packed[i].data_ptr() for i in range(n)])
    check("mxfp8_quantize_weights", lib().mxfp8_quantize_weights(n, tw, rows, cols, tc, ts, tp, _stream(w.device)))
    return codes, scales, packed


def fp8_tensor_quantize_weights(w: torch.Tensor):
    """bf16 weights [n, rows, cols] -> (E4M3 codes uint8 [n, rows, cols], float32 scales [n],
    packed uint8 [n, rows * cols + 16]): for each weight the outputs of
    fp8_tensor_quantize and of fp8_tensor_pack_weight_bwd (in the first rows * cols + 4
    bytes of its packed row), from one pass for the maxima and one for the codes."""
    w = _weight_stack(w, "fp8_tensor_quantize_weights")
    n, rows, cols = w.shape
    codes = torch.empty((n, rows, cols), dtype=torch.uint8, device=w.device)
    scale = torch.empty(n, dtype=torch.float32, device=w.device)
    packed = torch.empty((n, rows * cols + 16), dtype=torch.uint8, device=w.device)
    tw, kw = _lib.ptr_table([w[i].data_ptr() for i in range(n)])
    tc, kc = _lib.ptr_table([codes[i].data_ptr() for i in range(n)])
    tp, kp = _lib.ptr_table([packed[i].data_ptr() for i in range(n)])
    check("fp8_tensor_quantize_weights", lib().fp8_tensor_quantize_weights(n, tw, rows, cols, tc, _p(scale), tp,
                                                                           _stream(w.device)))
    return codes, scale, packed


def _experts(w):
    """A [E, ...] tensor or a list of per-expert tensors -> list of per-expert tensors."""
    if isinstance(w, torch.Tensor):
        return [w[e] for e in range(w.shape[0])]
    return list(w)


_COMPUTE = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8, "fp8": MOE_FP8}


def moe_grouped_mlp_fwd(x_perm: torch.Tensor, w_gate_up, w_down, offsets: torch.Tensor, prob_perm: torch.Tensor,
                        compute: str = "bf16", save_for_bwd: bool = False, x_perm_scale=None,
                        w_gate_up_scale=None, w_down_scale=None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None):
    """Grouped MLP forward on permuted rows. Returns y_perm, or (y_perm, z, h) with save_for_bwd.

    compute: "f32", "bf16", "mxfp8" or "fp8" (per-tensor scales). For mxfp8 and fp8,
    x_perm may be bf16 (quantised in the call) or uint8 codes with x_perm_scale; weights
    may be bf16 master weights (quantised in the call) or uint8 codes with per-expert
    scale tensors (fp8: one float32 scale tensor per expert weight).
    """
    w1 = _experts(w_gate_up)
    w2 = _experts(w_down)
    E = len(w1)
    twoI, H = w1[0].shape
    I = twoI // 2
    R = x_perm.shape[0]
    dev = x_perm.device
    _need_cuda(x_perm, offsets, prob_perm, x_perm_scale, *w1, *w2)
    c = _COMPUTE[compute]
    act = c if x_perm.dtype == torch.uint8 else _DT[x_perm.dtype]
    wt = c if w1[0].dtype == torch.uint8 else _DT[w1[0].dtype]
    desc = MlpDesc(E, H, I, c, act, wt, int(save_for_bwd))
    out_dtype = torch.float32 if c == MOE_F32 else torch.bfloat16
    y = out if out is not None else torch.empty((R, H), dtype=out_dtype, device=dev)
    z = torch.empty((R, 2 * I), dtype=out_dtype, device=dev) if save_for_bwd else None
    h = torch.empty((R, I), dtype=out_dtype, device=dev) if save_for_bwd else None
    need = workspace_size(_lib.MOE_OP_MLP_FWD, desc, R)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, dev)
    t1, k1 = ptr_table([t.data_ptr() for t in w1])
    t2, k2 = ptr_table([t.data_ptr() for t in w2])
    s1 = s2 = None
    keep = []
    if w_gate_up_scale is not None:
        s1, a = ptr_table([t.data_ptr() for t in _experts(w_gate_up_scale)])
        keep.append(a)
        s2, a = ptr_table([t.data_ptr() for t in _experts(w_down_scale)])
        keep.append(a)
    check("moe_grouped_mlp_fwd", lib().moe_grouped_mlp_fwd(
        ctypes.byref(desc), R, _p(x_perm), _p(x_perm_scale), t1, t2, s1, s2, _p(offsets), _p(prob_perm), _p(y),
        _p(z), _p(h), _p(ws), ws.numel(), _stream(dev)))
    del k1, k2, keep
    return (y, z, h) if save_for_bwd else y


def moe_grouped_mlp_bwd(dy_perm, x_perm, z, h, prob_perm, w_gate_up, w_down, offsets, compute: str = "bf16",
                        dw_gate_up=None, dw_down=None, workspace: torch.Tensor | None = None):
    """Grouped MLP backward. Returns (dx_perm, dw_gate_up [E, 2I, H], dw_down [E, H, I], dprob_perm [R]).

    With compute="mxfp8" the weights may be bf16 or packed by mxfp8_pack_weight_bwd (uint8); with
    compute="fp8", bf16 or packed by fp8_tensor_pack_weight_bwd (uint8)."""
    w1 = _experts(w_gate_up)
    w2 = _experts(w_down)
    E = len(w1)
    H = x_perm.shape[1]
    I = z.shape[1] // 2
    twoI = 2 * I
    R = x_perm.shape[0]
    dev = x_perm.device
    _need_cuda(dy_perm, x_perm, z, h, prob_perm, offsets, *w1, *w2)
    c = _COMPUTE[compute]
    dt = torch.float32 if c == MOE_F32 else torch.bfloat16
    wt = c if w1[0].dtype == torch.uint8 else _DT[w1[0].dtype]    # uint8: the compute dtype's packs
    desc = MlpDesc(E, H, I, c, _DT[x_perm.dtype], wt, 1)
    dx = torch.empty((R, H), dtype=dt, device=dev)
    dw1 = dw_gate_up if dw_gate_up is not None else torch.empty((E, twoI, H), dtype=dt, device=dev)
    dw2 = dw_down if dw_down is not None else torch.empty((E, H, I), dtype=dt, device=dev)
    dprob = torch.empty(R, dtype=torch.float32, device=dev)
    need = workspace_size(_lib.MOE_OP_MLP_BWD, desc, R)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, dev)
    t1, k1 = ptr_table([t.data_ptr() for t in w1])
    t2, k2 = ptr_table([t.data_ptr() for t in w2])
    d1, k3 = ptr_table([t.data_ptr() for t in _experts(dw1)])
    d2, k4 = ptr_table([t.data_ptr() for t in _experts(dw2)])
    check("moe_grouped_mlp_bwd", lib().moe_grouped_mlp_bwd(
        ctypes.byref(desc), R, _p(dy_perm), _p(x_perm), _p(z), _p(h), _p(prob_perm), t1, t2, _p(offsets), _p(dx),
        d1, d2, _p(dprob), _p(ws), ws.numel(), _stream(dev)))
    del k1, k2, k3, k4
    return dx, dw1, dw2, dprob


def gemm_workspace(device) -> torch.Tensor:
    """A workspace for moe_grouped_linear / moe_grouped_gate_up_swiglu (split-K tail area)."""
    return _workspace(workspace_size(_lib.MOE_OP_GROUPED_GEMM, None, 0), device)


def moe_grouped_linear(x: torch.Tensor, w, offsets: torch.Tensor, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """GroupedLinear: y[r] = x[r] W_e^T for the rows of expert e. x [R, K], W_e [N, K] -> y [R, N].

    workspace: optional (see gemm_workspace); without it no tile is split along K.
    """
    ws = _experts(w)
    E = len(ws)
    N, K = ws[0].shape
    R = x.shape[0]
    _need_cuda(x, offsets, *ws)
    y = out if out is not None else torch.empty((R, N), dtype=x.dtype, device=x.device)
    t, keep = ptr_table([t.data_ptr() for t in ws])
    nws = workspace.numel() if workspace is not None else 0
    check("moe_grouped_linear", lib().moe_grouped_linear(E, R, K, N, _DT[x.dtype], _p(x), t, _p(offsets), _p(y),
                                                         _p(workspace), nws, _stream(x.device)))
    del keep
    return y


def moe_grouped_gate_up_swiglu(x: torch.Tensor, w_gate_up, offsets: torch.Tensor, prob: torch.Tensor,
                               save_z: bool = False, x_scale=None, w_scale=None, out: torch.Tensor | None = None,
                               out_scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """GroupedLinear(gate_up) fused with ScaledSwiGLU: h = silu(x W_e[:I]^T) * (x W_e[I:]^T) * prob.

    bf16/f32: returns h [R, I] (and z [R, 2I] with save_z). MXFP8 (x given as uint8 codes
    with x_scale, weights as codes with w_scale): returns (h codes [R, I], h scales [R, I/32]).
    """
    ws = _experts(w_gate_up)
    E = len(ws)
    twoI, H = ws[0].shape
    I = twoI // 2
    R = x.shape[0]
    dev = x.device
    _need_cuda(x, offsets, prob, x_scale, *ws)
    dt = _DT[x.dtype]
    t, keep = ptr_table([t.data_ptr() for t in ws])
    st = None
    if dt == MOE_MXFP8:
        st, keep2 = ptr_table([t.data_ptr() for t in _experts(w_scale)])
        h = out if out is not None else torch.empty((R, I), dtype=torch.uint8, device=dev)
        hs = out_scale if out_scale is not None else torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
        z = None
    else:
        h = out if out is not None else torch.empty((R, I), dtype=x.dtype, device=dev)
        hs = None
        z = torch.empty((R, twoI), dtype=x.dtype, device=dev) if save_z else None
    check("moe_grouped_gate_up_swiglu", lib().moe_grouped_gate_up_swiglu(
        E, R, H, I, dt, _p(x), _p(x_scale), t, st, _p(offsets), _p(prob), _p(h), _p(hs), _p(z), _p(workspace),
        workspace.numel() if workspace is not None else 0, _stream(dev)))
    del keep
    if dt == MOE_MXFP8:
        return h, hs
    return (h, z) if save_z else h
