"""The C-ABI library (CPU only, no compute calls): it loads, exports every entry
point include/moe.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from grouped_expert_gemm_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from grouped_expert_gemm_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:moe_status|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_permute", "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd",
              "moe_unpermute_combine", "mxfp8_quantize"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from grouped_expert_gemm_amd import _lib
    names = declared_functions()
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(5):
        assert L.moe_status_str(s)


def test_argument_errors_before_launch(L):
    from grouped_expert_gemm_amd import _lib
    INV, UNS, WS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
    assert L.moe_route_topk(None, 10, 0, 1, 1, None, None, None) == INV        # E = 0
    assert L.moe_route_topk(None, 10, 8, 9, 1, None, None, None) == INV        # k > E
    assert L.moe_route_topk(None, 10, 32, 17, 1, None, None, None) == UNS      # k > 16
    assert L.moe_route_topk(None, 0, 8, 2, 1, None, None, None) == 0           # T = 0: nothing to do
    assert L.moe_route_topk(None, 5, 8, 2, 1, None, None, None) == INV         # NULL
    assert b"NULL" in L.moe_last_error()
    assert L.mxfp8_quantize(None, 4, 33, None, None, None) == INV              # cols % 32
    assert L.moe_unpermute_combine(None, 2, None, None, 4, 8, 2, None, None) == UNS  # MXFP8 rows
    assert L.moe_unpermute_combine(None, 1, None, None, 1 << 34, 8, 2, None, None) == UNS  # grid past 2^31 blocks
    assert L.moe_unpermute_combine(None, 1, None, None, 4, 8, 2, None, None) == INV  # NULL
    # permute: undersized workspace is reported before any launch
    dummy = ctypes.c_void_p(256)
    assert L.moe_permute(dummy, None, 1, 1000, 64, 8, 2, dummy, dummy, 0, dummy, None, dummy, dummy, dummy,
                         dummy, dummy, dummy, 16, None) == WS
    assert L.moe_permute(dummy, None, 1, 10, 64, 300, 2, dummy, dummy, 0, dummy, None, dummy, dummy, dummy,
                         dummy, dummy, dummy, 1 << 20, None) == INV             # E > 256


def test_mlp_descriptor_checks(L):
    from grouped_expert_gemm_amd import _lib
    n = ctypes.c_size_t()
    D = _lib.MlpDesc
    ok = D(8, 4096, 14336, 1, 1, 1, 0)
    assert L.moe_workspace_size(1, ctypes.byref(ok), 16384, 0, 0, 0, ctypes.byref(n)) == 0
    assert n.value >= 16384 * 14336 * 2
    assert L.moe_workspace_size(2, ctypes.byref(ok), 8192, 0, 0, 0, ctypes.byref(n)) == 0
    assert L.moe_workspace_size(1, ctypes.byref(D(8, 100, 14336, 1, 1, 1, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, 2, 1, 1, 0)), 8192, 0, 0, 0,
                                ctypes.byref(n)) == 0                           # MXFP8 backward
    assert n.value >= 8192 * (4096 + 2 * 14336 + 14336 * 2 + 2 * 14336 * 2)     # its quantised operands
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, 2, 2, 1, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG    # MXFP8 backward: bf16 activations
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, 3, 1, 1, 0)), 8192, 0, 0, 0,
                                ctypes.byref(n)) == 0                           # per-tensor FP8 backward
    assert n.value >= 8192 * (4096 + 2 * 14336 + 14336 * 2 + 2 * 14336 * 2)     # its quantised operands
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, 3, 3, 1, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG    # FP8 backward: bf16 activations
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, 3, 1, 3, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == 0                           # ... packed FP8 weights
    assert L.moe_workspace_size(1, ctypes.byref(D(0, 256, 128, 1, 1, 1, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_size(1, ctypes.byref(D(8, 256, 128, 1, 0, 1, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == _lib.MOE_ERR_INVALID_ARG    # f32 storage, bf16 compute
    assert L.moe_grouped_mlp_fwd(None, 1, None, None, None, None, None, None, None, None, None, None, None,
                                 None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    # a NULL expert pointer is caught before launch
    ptrs = (ctypes.c_void_p * 8)(*([4096] * 7 + [0]))
    pp = ctypes.cast(ptrs, _lib.PP)
    d = D(8, 256, 128, 1, 1, 1, 0)
    st = L.moe_grouped_mlp_fwd(ctypes.byref(d), 64, ctypes.c_void_p(4096), None, pp, pp, None, None,
                               ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096), None, None,
                               ctypes.c_void_p(4096), 1 << 30, None)
    assert st == _lib.MOE_ERR_INVALID_ARG and b"expert 7" in L.moe_last_error()


def test_fp8_tensor_argument_checks(L):
    """Per-tensor FP8: size and pointer checks before any launch; descriptor rules of the
    FP8 forward (storage matching the compute dtype, both saved tensors when saving) and
    backward (bf16 activations and weights)."""
    from grouped_expert_gemm_amd import _lib
    INV, UNS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED
    scale = ctypes.c_void_p(4096)
    assert L.fp8_tensor_quantize(None, 12, None, scale, None) == INV                  # n % 8
    assert L.fp8_tensor_quantize(None, -8, None, scale, None) == INV                  # negative
    assert L.fp8_tensor_quantize(None, 16, None, None, None) == INV                   # NULL scale
    assert L.fp8_tensor_quantize(None, 16, None, ctypes.c_void_p(4098), None) == INV  # scale misaligned
    assert L.fp8_tensor_quantize(None, 16, None, scale, None) == INV                  # NULL input
    n = ctypes.c_size_t()
    D = _lib.MlpDesc
    FP8, BF16, MX = _lib.MOE_FP8, _lib.MOE_BF16, _lib.MOE_MXFP8
    assert L.moe_workspace_size(1, ctypes.byref(D(8, 4096, 14336, FP8, BF16, BF16, 0)), 16384, 0, 0, 0,
                                ctypes.byref(n)) == 0
    # scale words, x codes, both weights' codes of 8 experts, h in bf16 and its codes
    assert n.value >= 16384 * 4096 + 8 * 3 * 14336 * 4096 + 16384 * 14336 * 3
    assert L.moe_workspace_size(1, ctypes.byref(D(8, 4096, 14336, FP8, MX, BF16, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == INV                                # MXFP8 storage, FP8 compute
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, FP8, BF16, BF16, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == 0                                  # FP8 backward
    assert L.moe_workspace_size(2, ctypes.byref(D(8, 4096, 14336, FP8, FP8, BF16, 0)), 1, 0, 0, 0,
                                ctypes.byref(n)) == INV                                # ... on bf16 activations
    ptrs = (ctypes.c_void_p * 8)(*([4096] * 8))
    pp = ctypes.cast(ptrs, _lib.PP)
    # FP8 saves z and h for the backward too, and needs both buffers to do it
    d = D(8, 256, 256, FP8, BF16, BF16, 1)
    st = L.moe_grouped_mlp_fwd(ctypes.byref(d), 64, ctypes.c_void_p(4096), None, pp, pp, None, None,
                               ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                               None, ctypes.c_void_p(4096), ctypes.c_void_p(4096), 1 << 40, None)
    assert st == INV and b"save_for_bwd" in L.moe_last_error()
    # MXFP8 saves z and h for the backward, and needs both buffers to do it
    d = D(8, 256, 256, MX, BF16, BF16, 1)
    st = L.moe_grouped_mlp_fwd(ctypes.byref(d), 64, ctypes.c_void_p(4096), None, pp, pp, None, None,
                               ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                               None, None, ctypes.c_void_p(4096), 1 << 40, None)
    assert st == INV and b"z_save" in L.moe_last_error()


def test_mxfp8_colwise_argument_checks(L):
    from grouped_expert_gemm_amd import _lib
    INV, UNS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED
    d = ctypes.c_void_p(4096)
    assert L.mxfp8_quantize_colwise(d, 100, 96, 4, d, 32, 256, d, d, d, None) == UNS     # C % 64
    assert L.mxfp8_quantize_colwise(d, 100, 64, 4, d, 48, 256, d, d, d, None) == INV     # pad % 32
    assert L.mxfp8_quantize_colwise(d, 100, 64, 4, d, 32, 192, d, d, d, None) == INV     # kcap < R + E (pad - 1)
    assert L.mxfp8_quantize_colwise(d, 100, 64, 0, d, 32, 256, d, d, d, None) == INV     # E = 0
    assert L.mxfp8_quantize_colwise(d, 100, 64, 4, None, 32, 256, d, d, d, None) == INV  # NULL offsets
    assert b"kcap" in L.moe_last_error() or b"NULL" in L.moe_last_error()
    f = L.fp8_tensor_quantize_colwise
    assert f(d, 100, 96, 4, d, 32, 256, d, d, d, None) == UNS      # C % 64
    assert f(d, 100, 64, 4, d, 48, 256, d, d, d, None) == INV      # pad % 32
    assert f(d, 100, 64, 4, d, 32, 192, d, d, d, None) == INV      # kcap < R + E (pad - 1)
    assert f(d, 100, 64, 0, d, 32, 256, d, d, d, None) == INV      # E = 0
    assert f(d, 100, 64, 4, d, 32, 256, d, None, d, None) == INV   # NULL scale
    assert f(d, -1, 64, 4, d, 32, 256, d, d, d, None) == INV       # negative R


def test_noalloc_permute_rejects_sizes_beyond_its_scratch(L):
    """moe_permute_noalloc checks its fixed 8 MiB scratch against the request before it
    touches any device: a size that would need more is refused with UNSUPPORTED."""
    from grouped_expert_gemm_amd import _lib
    dummy = ctypes.c_void_p(256)
    T, E, k = 1 << 20, 8, 4          # rank table alone: T * k * 4 = 16 MiB
    assert L.moe_permute_noalloc(dummy, None, 1, T, 64, E, k, dummy, dummy, 0, dummy, None, dummy, dummy, dummy,
                                 dummy, dummy, None) == _lib.MOE_ERR_UNSUPPORTED
    assert b"8 MiB" in L.moe_last_error()
    assert L.moe_permute_noalloc(dummy, None, 1, 10, 64, 0, 1, dummy, dummy, 0, dummy, None, dummy, dummy, dummy,
                                 dummy, dummy, None) == _lib.MOE_ERR_INVALID_ARG     # E = 0


def test_pack_weight_argument_checks(L):
    from grouped_expert_gemm_amd import _lib
    dummy = ctypes.c_void_p(256)
    assert L.mxfp8_pack_weight_bwd(dummy, 100, 64, dummy, None) == _lib.MOE_ERR_UNSUPPORTED   # rows % 128
    assert L.mxfp8_pack_weight_bwd(dummy, 128, 96, dummy, None) == _lib.MOE_ERR_UNSUPPORTED   # cols % 64
    assert L.mxfp8_pack_weight_bwd(None, 128, 64, dummy, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.mxfp8_pack_weight_bwd(None, 0, 64, None, None) == 0                             # empty: no-op
    f = L.fp8_tensor_pack_weight_bwd
    assert f(dummy, 100, 64, dummy, None) == _lib.MOE_ERR_UNSUPPORTED    # rows % 32
    assert f(dummy, 128, 96, dummy, None) == _lib.MOE_ERR_UNSUPPORTED    # cols % 64
    assert f(None, 128, 64, dummy, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(dummy, 128, 64, ctypes.c_void_p(264), None) == _lib.MOE_ERR_INVALID_ARG  # packed misaligned
    assert f(None, 0, 64, None, None) == 0                               # empty: no-op


def test_weight_quantisers_argument_checks(L):
    """mxfp8_quantize_weights / fp8_tensor_quantize_weights reject bad counts, shapes,
    NULL tables and entries, and misaligned pointers before any GPU work."""
    from grouped_expert_gemm_amd import _lib
    d = ctypes.c_void_p(256)
    one = _lib.ptr_table([256])[0]
    odd = _lib.ptr_table([264])[0]
    nul = _lib.ptr_table([None])[0]
    INV, UNS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED
    m = L.mxfp8_quantize_weights
    assert m(0, one, 128, 64, one, one, one, None) == INV          # n < 1
    assert m(257, one, 128, 64, one, one, one, None) == INV        # n > 256
    assert m(1, one, 100, 64, one, one, one, None) == UNS          # rows % 128
    assert m(1, one, 128, 96, one, one, one, None) == UNS          # cols % 64
    assert m(1, None, 128, 64, one, one, one, None) == INV         # NULL table
    assert m(1, nul, 128, 64, one, one, one, None) == INV          # NULL entry
    assert m(1, one, 128, 64, one, one, odd, None) == INV          # packed misaligned
    assert m(1, None, 0, 64, None, None, None, None) == 0          # empty: no-op
    f = L.fp8_tensor_quantize_weights
    assert f(0, one, 32, 64, one, d, one, None) == INV             # n < 1
    assert f(1, one, 48, 64, one, d, one, None) == UNS             # rows % 32
    assert f(1, one, 32, 96, one, d, one, None) == UNS             # cols % 64
    assert f(1, one, 32, 64, one, None, one, None) == INV          # NULL scale
    assert f(1, one, 32, 64, one, ctypes.c_void_p(258), one, None) == INV   # scale misaligned
    assert f(1, None, 32, 64, one, d, one, None) == INV            # NULL table
    assert f(1, one, 32, 64, nul, d, one, None) == INV             # NULL entry
    assert f(1, one, 32, 64, _lib.ptr_table([260])[0], d, one, None) == INV   # codes not 8-byte aligned


def test_mx_and_fp8_reject_more_than_128_experts(L):
    """The MXFP8 and per-tensor FP8 kernels take at most 128 experts per call (their
    pointer tables travel in the kernel arguments): more is refused before any launch."""
    from grouped_expert_gemm_amd import _lib
    E = 129
    D = _lib.MlpDesc
    ptrs = (ctypes.c_void_p * E)(*([4096] * E))
    pp = ctypes.cast(ptrs, _lib.PP)
    p = ctypes.c_void_p(4096)
    for compute in (_lib.MOE_MXFP8, _lib.MOE_FP8):
        d = D(E, 256, 256, compute, 1, 1, 0)   # bf16 activations and weights, quantised inside
        st = L.moe_grouped_mlp_fwd(ctypes.byref(d), 64, p, None, pp, pp, None, None, p, p, p, None, None,
                                   p, 1 << 40, None)
        assert st == _lib.MOE_ERR_UNSUPPORTED and b"128" in L.moe_last_error(), (compute, st, L.moe_last_error())
        st = L.moe_grouped_mlp_bwd(ctypes.byref(d), 64, p, p, p, p, p, pp, pp, p, p, pp, pp, p, p, 1 << 40, None)
        assert st == _lib.MOE_ERR_UNSUPPORTED and b"128" in L.moe_last_error(), (compute, st, L.moe_last_error())
