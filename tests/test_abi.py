"""The C-ABI library loads, exports every function include/fp4moe.h declares,
and rejects bad arguments on the host (no GPU needed: these return before any
HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4moe.h")


def _declared_functions(header=HEADER):
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from block_scaled_fp4_nvfp4_amd import _lib
    return _lib.lib()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("fp4_quantize", "fp4_dequantize", "moe_fp4_forward", "moe_fp4_workspace_size",
              "moe_fp4_workspace_layout", "fp4_status_string", "fp4_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    import glob
    headers = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert HEADER in headers and len(headers) == 2  # the library ABI and its ceiling probes
    for h in headers:
        for n in _declared_functions(h):
            assert hasattr(L, n), (h, n)
    assert _declared_functions(os.path.join(ROOT, "include", "fp4moe_probe.h")) == \
        ["fp4_probe_combine", "fp4_probe_mfma", "fp4_probe_read"]
    from block_scaled_fp4_nvfp4_amd import _lib
    assert sorted(_lib.EXPORTED) == _declared_functions()


def test_status_strings(L):
    from block_scaled_fp4_nvfp4_amd import status_string
    assert status_string(0) == "FP4_OK"
    assert status_string(-2) == "FP4_ERR_SHAPE"
    assert status_string(-4) == "FP4_ERR_WORKSPACE"


def test_host_validation_errors(L):
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    # cols not a multiple of 16 for NVFP4
    assert L.fp4_quantize(0, 1, 0, fake, 0, 1, 4, 24, fake, fake, fake, None, None) == -2
    assert b"multiple of 16" in L.fp4_last_error()
    # MXFP4 needs cols % 32
    assert L.fp4_quantize(1, 1, 0, fake, 0, 1, 4, 48, fake, fake, None, None, None) == -2
    # unknown format / rule / dtype
    assert L.fp4_quantize(9, 1, 0, fake, 0, 1, 4, 32, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize(0, 7, 0, fake, 0, 1, 4, 32, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize(0, 1, 0, fake, 5, 1, 4, 32, fake, fake, fake, None, None) == -1
    # null pointers
    assert L.fp4_quantize(0, 1, 0, None, 0, 1, 4, 32, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize(0, 1, 0, fake, 0, 1, 4, 32, fake, fake, None, None, None) == -1
    # empty problem is a no-op
    assert L.fp4_quantize(0, 1, 0, None, 0, 0, 4, 32, None, None, None, None, None) == 0
    # FP8 block weights need rows % 128
    assert L.fp4_quantize(3, 0, 0, fake, 0, 1, 64, 128, fake, fake, None, None, None) == -2
    assert L.fp4_dequantize(0, fake, fake, None, 1, 4, 32, fake, 1, None) == -1
    # block errors: NVFP4 / MXFP4 only, cols % block, null and misaligned pointers, empty is a no-op
    odd = ctypes.c_void_p(0x1004)
    assert L.fp4_block_error(2, fake, 0, 1, 4, 64, fake, fake, None, fake, None) == -3
    assert L.fp4_block_error(0, fake, 0, 1, 4, 40, fake, fake, fake, fake, None) == -2
    assert L.fp4_block_error(1, fake, 0, 1, 4, 48, fake, fake, None, fake, None) == -2
    assert L.fp4_block_error(0, fake, 0, 1, 4, 64, fake, fake, None, fake, None) == -1  # NVFP4 needs S
    assert L.fp4_block_error(1, odd, 0, 1, 4, 64, fake, fake, None, fake, None) == -1
    assert L.fp4_block_error(1, fake, 7, 1, 4, 64, fake, fake, None, fake, None) == -1
    assert L.fp4_block_error(1, None, 0, 0, 4, 64, None, None, None, None, None) == 0
    # Hessian-weighted search: cols % 16, dtype, null and misaligned pointers; empty is a no-op
    assert L.fp4_quantize_hessian(fake, 0, 2, 4, 24, fake, fake, fake, fake, fake, None, None) == -2
    assert L.fp4_quantize_hessian(fake, 3, 2, 4, 32, fake, fake, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize_hessian(fake, 0, 2, 4, 32, None, fake, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize_hessian(fake, 0, 2, 4, 32, fake, None, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize_hessian(odd, 0, 2, 4, 32, fake, fake, fake, fake, fake, None, None) == -1
    assert L.fp4_quantize_hessian(fake, 0, 2, 4, 32, fake, fake, odd, fake, fake, None, None) == -1
    assert L.fp4_quantize_hessian(None, 0, 0, 4, 32, None, None, None, None, None, None, None) == 0
    # routing: k outside [1, min(E, 32)], too many experts, empty batch, null outputs
    assert L.moe_fp4_route(fake, None, 4, 8, 0, fake, fake, None) == -1
    assert L.moe_fp4_route(fake, None, 4, 8, 9, fake, fake, None) == -1
    assert L.moe_fp4_route(fake, None, 4, 64, 33, fake, fake, None) == -1
    assert L.moe_fp4_route(fake, None, 4, 2048, 8, fake, fake, None) == -3
    assert L.moe_fp4_route(None, None, 0, 8, 2, None, None, None) == 0
    assert L.moe_fp4_route(fake, None, 4, 8, 2, None, fake, None) == -1


def _layer(**kw):
    from block_scaled_fp4_nvfp4_amd import _lib
    base = dict(w_fmt=0, a_fmt=5, num_experts=8, hidden=256, inter=128, top_k=2)
    base.update(kw)
    s = _lib.LayerStruct()
    for k, v in base.items():
        setattr(s, k, v)
    for k in ("w13", "w13_scale", "w13_scale_2", "w2", "w2_scale", "w2_scale_2"):
        setattr(s, k, 0x1000)
    return s


def test_moe_validation_and_workspace(L):
    sz = ctypes.c_size_t()
    s = _layer()
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0 and sz.value > 0
    # workspace grows with tokens
    sz2 = ctypes.c_size_t()
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 128, ctypes.byref(sz2)) == 0 and sz2.value > sz.value
    assert L.moe_fp4_workspace_size(ctypes.byref(_layer(top_k=9)), 64, ctypes.byref(sz)) == -1
    assert L.moe_fp4_workspace_size(ctypes.byref(_layer(top_k=0)), 64, ctypes.byref(sz)) == -1
    assert L.moe_fp4_workspace_size(ctypes.byref(_layer(hidden=250)), 64, ctypes.byref(sz)) == -2
    assert L.moe_fp4_workspace_size(ctypes.byref(_layer(w_fmt=0, a_fmt=2)), 64, ctypes.byref(sz)) == -3
    fake = ctypes.c_void_p(0x1000)
    # too-small workspace is refused before any launch
    assert L.moe_fp4_forward(ctypes.byref(s), fake, 64, fake, fake, fake, fake, 16, None) == -4
    # T == 0 is a no-op
    assert L.moe_fp4_forward(ctypes.byref(s), None, 0, None, None, None, None, 0, None) == 0
    # the allocation-free forward validates the layer, then refuses (before any HIP call) a
    # problem whose workspace exceeds its scratch; T == 0 is a no-op
    from block_scaled_fp4_nvfp4_amd import _lib
    big = _layer(num_experts=512, hidden=2560, inter=640, top_k=10)
    assert L.moe_fp4_workspace_size(ctypes.byref(big), 8192, ctypes.byref(sz)) == 0
    assert sz.value > _lib.NOALLOC_SCRATCH_BYTES
    assert L.moe_fp4_forward_noalloc(ctypes.byref(big), fake, 8192, fake, fake, fake, None) == -4
    assert b"scratch" in L.fp4_last_error()
    assert L.moe_fp4_forward_noalloc(ctypes.byref(_layer(top_k=0)), fake, 64, fake, fake, fake, None) == -1
    assert L.moe_fp4_forward_noalloc(ctypes.byref(s), None, 0, None, None, None, None) == 0
    # the header's limit and the binding's agree
    hdr = open(HEADER).read()
    assert "#define FP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr and _lib.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_tile_weights_and_tiled_layer_validation(L):
    fake, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1004)
    # weight formats only (not MXFP8 / FP8 rows); rows % 16 and cols % 128; null and misaligned
    # pointers; empty is a no-op.  Every call here fails (or does nothing) before any launch.
    assert L.moe_fp4_tile_weights(2, fake, fake, 2, 32, 256, fake, fake, None) == -3
    assert L.moe_fp4_tile_weights(4, fake, fake, 2, 32, 256, fake, fake, None) == -3
    assert L.moe_fp4_tile_weights(0, fake, odd, 2, 32, 256, fake, fake, None) == -1  # NVFP4 scales: 8 bytes
    assert L.moe_fp4_tile_weights(3, fake, None, 2, 32, 256, None, None, None) == -1  # null tiled codes
    assert L.moe_fp4_tile_weights(1, fake, fake, 2, 24, 256, fake, fake, None) == -2
    assert L.moe_fp4_tile_weights(1, fake, fake, 2, 32, 192, fake, fake, None) == -2
    assert L.moe_fp4_tile_weights(1, fake, None, 2, 32, 256, fake, fake, None) == -1
    assert L.moe_fp4_tile_weights(1, odd, fake, 2, 32, 256, fake, fake, None) == -1
    assert L.moe_fp4_tile_weights(1, None, None, 0, 32, 256, None, None, None) == 0
    sz = ctypes.c_size_t()
    # tiled W13: both pointers or neither, MXFP4 weights only
    s = _layer(w_fmt=1, a_fmt=2)
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0
    s.w13_tiled = 0x2000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == -1
    s.w13_scale_tiled = 0x3000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0
    s.w2_scale_tiled = 0x4000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == -1
    s.w2_tiled = 0x5000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0
    s = _layer(w_fmt=0, a_fmt=0)
    s.w13_tiled = 0x2000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == -1
    s.w13_scale_tiled = 0x3000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0
    # block FP8: tiled codes without tiled scales
    s = _layer(w_fmt=3, a_fmt=4)
    s.w13_tiled = 0x2000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == 0
    s.w13_scale_tiled = 0x3000
    assert L.moe_fp4_workspace_size(ctypes.byref(s), 64, ctypes.byref(sz)) == -1
