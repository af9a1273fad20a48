"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, reports sizes, and rejects bad arguments on the host before
anything is enqueued.  No compute call reaches the device here."""

import ctypes
import os
import re

import numpy as np
import pytest

import nf4_bit_quantized_amd as q
from oracle import nf4 as onf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.LIB_PATH), reason="library not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_what_binding_lists():
    assert _declared() == sorted(q.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = q.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {q.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert isinstance(q.qlora_status_string(code), str) and q.qlora_status_string(code)
    assert q.qlora_status_string(-99) == "unknown status"


def test_library_table_is_bit_identical_to_oracle_table():
    levels, thr = q.qlora_nf4_levels()
    np.testing.assert_array_equal(levels.view(np.uint32), onf4.nf4_levels().view(np.uint32))


def test_library_thresholds_reproduce_oracle_nearest_level():
    levels, thr = q.qlora_nf4_levels()
    T = onf4.nf4_levels()
    for k in range(15):
        at = np.array([thr[k]], np.float32)
        above = np.nextafter(at, np.float32(np.inf))
        assert onf4._nearest_level(at, T)[0] == k
        assert onf4._nearest_level(above, T)[0] == k + 1


def test_uniform_table_is_the_oracles():
    levels, thr = q.qlora_table_levels(q.TABLE_UNIFORM)
    U = onf4.uniform_levels()
    np.testing.assert_array_equal(levels.view(np.uint32), U.view(np.uint32))
    for k in range(15):
        at = np.array([thr[k]], np.float32)
        above = np.nextafter(at, np.float32(np.inf))
        assert onf4._nearest_level(at, U)[0] == k
        assert onf4._nearest_level(above, U)[0] == k + 1
    # the NF4 table through the same call
    levels, _ = q.qlora_table_levels(q.TABLE_NF4)
    np.testing.assert_array_equal(levels.view(np.uint32), onf4.nf4_levels().view(np.uint32))


def test_unknown_table_rejected():
    L = q.lib()
    assert L.qlora_table_levels(2, None, None) == q.QLORA_ERR_UNSUPPORTED
    d = q._desc(64, 64, table=2)
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qlora_nf4_sizes(ctypes.byref(d), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == \
        q.QLORA_ERR_UNSUPPORTED


def test_sizes():
    p, c, k = q.qlora_nf4_sizes(4096, 4096)
    assert p == 4096 * 4096 // 2 and c == 4096 * 4096 // 64 and k == 4 * (4096 * 4096 // 64 // 256)
    p, c, k = q.qlora_nf4_sizes(64, 320)          # 320 blocks -> 2 groups (partial last group)
    assert (p, c, k) == (64 * 160, 320, 8)
    bits = (8 * p + 8 * c + 8 * k) / (64 * 320)
    assert abs(bits - onf4.storage_bits_per_weight(64 * 320)) < 1e-12


def _err(fn, *a):
    with pytest.raises(q.QloraError) as e:
        fn(*a)
    return e.value.status


def test_bad_descriptor_rejected():
    assert _err(q.qlora_nf4_sizes, 100, 64) == q.QLORA_ERR_SHAPE
    assert _err(q.qlora_nf4_sizes, 64, 0) == q.QLORA_ERR_SHAPE
    assert _err(q.qlora_nf4_sizes, 64, 64, 32) == q.QLORA_ERR_UNSUPPORTED
    assert _err(q.qlora_nf4_sizes, 64, 64, 512) == q.QLORA_ERR_UNSUPPORTED
    # blocks of 128 and 256 weights: one code per block, one constant per 256 codes
    assert q.qlora_nf4_sizes(4096, 4096, 128) == (4096 * 2048, 4096 * 4096 // 128, 4 * 4096 * 4096 // 128 // 256)
    assert q.qlora_nf4_sizes(64, 192, 256) == (64 * 96, 48, 4)
    assert _err(q.qlora_nf4_sizes, 64, 64, 64, 64) == q.QLORA_ERR_UNSUPPORTED
    assert _err(q.qlora_fwd_workspace_bytes, 64, 64, 4, 129) == q.QLORA_ERR_SHAPE
    assert _err(q.qlora_fwd_workspace_bytes, 64, 64, -1, 4) == q.QLORA_ERR_SHAPE


def _raw_fwd(desc, packed, codes, consts, T, X, r, A, B, Y, ws, wsb):
    L = q.lib()
    return L.qlora_linear_fwd(ctypes.byref(desc), packed, codes, consts, T, X, r, ctypes.c_float(2.0), A, B, Y,
                              None, ws, wsb, None)


def test_validation_happens_before_any_launch():
    # fake, aligned, never-dereferenced addresses: every call below must fail on the host
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    assert L.qlora_quantize_nf4(None, fake, fake, fake, fake, None) == q.QLORA_ERR_NULL
    assert L.qlora_quantize_nf4(ctypes.byref(d), None, fake, fake, fake, None) == q.QLORA_ERR_NULL
    assert L.qlora_quantize_nf4(ctypes.byref(d), fake + 4, fake, fake, fake, None) == q.QLORA_ERR_UNSUPPORTED
    bad = q._desc(64, 96)
    assert L.qlora_quantize_nf4(ctypes.byref(bad), fake, fake, fake, fake, None) == q.QLORA_ERR_SHAPE
    # forward: missing adapter, missing output, missing / short workspace
    assert _raw_fwd(d, fake, fake, fake, 8, fake, 4, None, fake, fake, fake, 1 << 20) == q.QLORA_ERR_NULL
    assert _raw_fwd(d, fake, fake, fake, 8, fake, 4, fake, fake, None, fake, 1 << 20) == q.QLORA_ERR_NULL
    need = q.qlora_fwd_workspace_bytes(64, 64, 8, 4)
    assert need > 0
    assert _raw_fwd(d, fake, fake, fake, 8, fake, 4, fake, fake, fake, None, need) == q.QLORA_ERR_WORKSPACE
    assert _raw_fwd(d, fake, fake, fake, 8, fake, 4, fake, fake, fake, fake, need - 1) == q.QLORA_ERR_WORKSPACE
    assert _raw_fwd(d, fake, fake, fake, 8, fake + 8, 4, fake, fake, fake, fake, need) == q.QLORA_ERR_UNSUPPORTED
    # backward: dA / dB required when r > 0
    nb = q.qlora_bwd_workspace_bytes(64, 64, 8, 4)
    r = L.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, 8, fake, 4, ctypes.c_float(1.0), fake, fake, None,
                           fake, fake, None, fake, fake, nb, None)
    assert r == q.QLORA_ERR_NULL
    r = L.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, 8, fake, 4, ctypes.c_float(1.0), fake, fake, None,
                           fake, fake, fake, fake, None, nb, None)
    assert r == q.QLORA_ERR_WORKSPACE


def test_export_validation_happens_before_any_launch():
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    f = ctypes.c_float(2.0)
    assert L.qlora_dequantize_nf4(None, fake, fake, fake, fake, None) == q.QLORA_ERR_NULL
    assert L.qlora_dequantize_nf4(ctypes.byref(d), fake, fake, fake, None, None) == q.QLORA_ERR_NULL
    assert L.qlora_dequantize_nf4(ctypes.byref(d), fake, fake, fake, fake + 2, None) == q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_dequantize_nf4(ctypes.byref(q._desc(64, 96)), fake, fake, fake, fake, None) == q.QLORA_ERR_SHAPE
    assert L.qlora_merge_lora(ctypes.byref(d), fake, fake, fake, 4, f, None, fake, fake, None) == q.QLORA_ERR_NULL
    assert L.qlora_merge_lora(ctypes.byref(d), fake, fake, fake, 4, f, fake, None, fake, None) == q.QLORA_ERR_NULL
    assert L.qlora_merge_lora(ctypes.byref(d), fake, fake, fake, 129, f, fake, fake, fake, None) == q.QLORA_ERR_SHAPE
    assert L.qlora_merge_lora(ctypes.byref(d), fake, fake, fake, 4, f, fake + 8, fake, fake, None) == \
        q.QLORA_ERR_UNSUPPORTED


def test_typed_quantize_validation_happens_before_any_launch():
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    assert L.qlora_quantize_nf4_typed(ctypes.byref(d), fake, 3, fake, fake, fake, None) == q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_quantize_nf4_typed(ctypes.byref(d), fake, -1, fake, fake, fake, None) == q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_quantize_nf4_typed(ctypes.byref(d), None, q.QLORA_W_BF16, fake, fake, fake, None) == \
        q.QLORA_ERR_NULL
    assert L.qlora_quantize_nf4_typed(ctypes.byref(d), fake + 2, q.QLORA_W_F16, fake, fake, fake, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_quantize_nf4_typed(ctypes.byref(q._desc(64, 96)), fake, q.QLORA_W_BF16, fake, fake, fake,
                                      None) == q.QLORA_ERR_SHAPE


def test_adamw_validation_happens_before_any_launch():
    fake = 0x10000
    L = q.lib()
    ok = q.AdamwHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    assert L.qlora_adamw_step(None, 8, fake, fake, fake, fake, None, None) == q.QLORA_ERR_NULL
    assert L.qlora_adamw_step(ctypes.byref(ok), 8, fake, None, fake, fake, None, None) == q.QLORA_ERR_NULL
    assert L.qlora_adamw_step(ctypes.byref(ok), 0, None, None, None, None, None, None) == q.QLORA_OK
    assert L.qlora_adamw_step(ctypes.byref(ok), -1, fake, fake, fake, fake, None, None) == q.QLORA_ERR_SHAPE
    for bad in (q.AdamwHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 0),        # step 0
                q.AdamwHparams(1e-3, 1.0, 0.999, 1e-8, 0.01, 1.0, 1),        # beta1 = 1
                q.AdamwHparams(1e-3, 0.9, -0.1, 1e-8, 0.01, 1.0, 1),         # beta2 < 0
                q.AdamwHparams(1e-3, 0.9, 0.999, -1.0, 0.01, 1.0, 1),        # eps < 0
                q.AdamwHparams(float("nan"), 0.9, 0.999, 1e-8, 0.01, 1.0, 1)):
        assert L.qlora_adamw_step(ctypes.byref(bad), 8, fake, fake, fake, fake, None, None) == \
            q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_adamw_step(ctypes.byref(ok), 8, fake + 4, fake, fake, fake, None, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_adamw_step(ctypes.byref(ok), 8, fake, fake, fake, fake, fake + 2, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert ctypes.sizeof(q.AdamwHparams) == 32


def test_fp32_scale_format_sizes():
    """No second level ("7、QLoRA 量化微调" §7.1, extended calculation: 64 weights
    sharing one fp32 scale cost 4.5 bits each): no codes, one fp32 scale per block."""
    n_p, n_c, n_k = q.qlora_nf4_sizes(4096, 4096, 64, 0)
    assert n_c == 0 and n_k == 4 * 4096 * 4096 // 64
    assert (n_p + n_c + n_k) * 8 / (4096 * 4096) == 4.5
    assert q.qlora_nf4_sizes(64, 320, 256, 0) == (64 * 160, 0, 4 * 64 * 320 // 256)
    assert _err(q.qlora_nf4_sizes, 64, 64, 64, 128) == q.QLORA_ERR_UNSUPPORTED


def test_dropout_validation_happens_before_any_launch():
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    f = ctypes.c_float
    big = 1 << 30
    # p outside [0, 1)
    for p in (-0.1, 1.0, float("nan")):
        assert L.qlora_linear_fwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, fake,
                                          f(p), fake, None, fake, big, None) == q.QLORA_ERR_UNSUPPORTED
    # no mask
    assert L.qlora_linear_fwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, None,
                                      f(0.1), fake, None, fake, big, None) == q.QLORA_ERR_NULL
    assert L.qlora_linear_bwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, None, fake,
                                      None, f(0.1), fake, fake, fake, 0, fake, big, None) == q.QLORA_ERR_NULL
    # workspace below the query
    n = ctypes.c_size_t()
    assert L.qlora_dropout_workspace_bytes(ctypes.byref(d), 4, 8, 1, ctypes.byref(n)) == q.QLORA_OK
    assert n.value >= 4 * 64 * 2
    assert L.qlora_linear_bwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, None, fake,
                                      fake, f(0.1), fake, fake, fake, 0, fake, n.value - 1, None) == \
        q.QLORA_ERR_WORKSPACE


def test_multi_forward_validation():
    L = q.lib()
    n = ctypes.c_size_t()
    d3 = (q.Nf4Desc * 3)(q._desc(512, 512), q._desc(128, 512), q._desc(128, 512))
    assert L.qlora_multi_fwd_workspace_bytes(3, d3, 4, 8, ctypes.byref(n)) == q.QLORA_OK and n.value > 0
    assert L.qlora_multi_fwd_workspace_bytes(0, d3, 4, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    d5 = (q.Nf4Desc * 5)(*[q._desc(64, 64)] * 5)
    assert L.qlora_multi_fwd_workspace_bytes(5, d5, 4, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    dk = (q.Nf4Desc * 2)(q._desc(64, 64), q._desc(64, 128))
    assert L.qlora_multi_fwd_workspace_bytes(2, dk, 4, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    db = (q.Nf4Desc * 2)(q._desc(64, 256), q._desc(64, 256, 128))
    assert L.qlora_multi_fwd_workspace_bytes(2, db, 4, 8, ctypes.byref(n)) == q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_multi_bwd_workspace_bytes(3, d3, 40, 8, ctypes.byref(n)) == q.QLORA_OK and n.value > 0
    assert L.qlora_multi_bwd_workspace_bytes(2, dk, 40, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE


def test_caller_outputs_are_checked_on_the_host():
    """A caller-given output must have the shape and dtype the call writes and
    be contiguous: the C entry points see only its pointer."""
    import torch
    q._check_out(None, (4, 8), torch.bfloat16, "Y")
    q._check_out(torch.empty(4, 8, dtype=torch.bfloat16), (4, 8), torch.bfloat16, "Y")
    for bad in (torch.empty(4, 9, dtype=torch.bfloat16), torch.empty(4, 8, dtype=torch.float32),
                torch.empty(8, 4, dtype=torch.bfloat16).t()):
        with pytest.raises(ValueError, match="Y must be"):
            q._check_out(bad, (4, 8), torch.bfloat16, "Y")


def test_trace_api_on_the_host():
    """The kernel-timing switches and read-out need no GPU: names of every
    timed kernel, an empty read, selection by name."""
    names = []
    k = 0
    while q.qlora_trace_kernel_name(k) is not None:
        names.append(q.qlora_trace_kernel_name(k))
        k += 1
    for n in ("nf4_quantize", "fwd_gemm", "dx_gemm", "decode", "export", "adamw", "dropout"):
        assert n in names
    assert len(set(names)) == len(names)
    assert q.qlora_trace_kernel_name(-1) is None
    q.qlora_trace_enable(False)
    assert q.qlora_trace_read(reset=True) == {}
    q.qlora_trace_select({"fwd_gemm", "dx_gemm"})
    q.qlora_trace_enable(False)
    assert q.qlora_trace_read(reset=True) == {}


def test_workspace_sizes_grow_with_tokens_and_rank():
    a = q.qlora_bwd_workspace_bytes(4096, 4096, 2048, 16)
    b = q.qlora_bwd_workspace_bytes(4096, 4096, 4096, 64)
    assert 0 < a < b
    assert q.qlora_fwd_workspace_bytes(4096, 4096, 2048, 0) == 0          # base-only, no decode: nothing
    assert q.qlora_bwd_workspace_bytes(4096, 4096, 0, 16) == 0


def _no_gpu_here():
    """The fake-pointer tests below must never reach a device: on a machine
    with a GPU a call that passed validation would launch on them."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")


def test_operand_size_limits_rejected_before_any_launch():
    """Every dense operand is addressed with 32-bit byte offsets: a packed
    weight, X, Y, dY or dX of 2 GiB or more is a shape error on the host (the
    query functions agree), never a launch failure."""
    _no_gpu_here()
    fake = 0x10000
    L = q.lib()
    n = ctypes.c_size_t()
    big_w = q._desc(65536, 65536)                  # packed weight 2 GiB
    assert L.qlora_fwd_workspace_bytes(ctypes.byref(big_w), 16, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    assert _raw_fwd(big_w, fake, fake, fake, 16, fake, 8, fake, fake, fake, fake, 1 << 30) == q.QLORA_ERR_SHAPE
    d = q._desc(8192, 8192)
    T = 131072                                     # X = T x 8192 bf16 = 2 GiB
    assert L.qlora_fwd_workspace_bytes(ctypes.byref(d), T, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    assert L.qlora_bwd_workspace_bytes(ctypes.byref(d), T, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    assert _raw_fwd(d, fake, fake, fake, T, fake, 8, fake, fake, fake, fake, 1 << 30) == q.QLORA_ERR_SHAPE
    wide = q._desc(262144, 64)                     # Y = T x 262144 bf16 = 2 GiB at T = 4096
    assert L.qlora_fwd_workspace_bytes(ctypes.byref(wide), 4096, 8, ctypes.byref(n)) == q.QLORA_ERR_SHAPE
    assert L.qlora_fwd_workspace_bytes(ctypes.byref(wide), 4095, 8, ctypes.byref(n)) == q.QLORA_OK
    assert L.qlora_merge_lora(ctypes.byref(big_w), fake, fake, fake, 4, ctypes.c_float(1.0), fake, fake, fake,
                              None) == q.QLORA_ERR_SHAPE


def test_output_alignment_rejected_before_any_launch():
    """Y and dX are written with 16-byte stores, U and the gradients need it
    too: a misaligned output is UNSUPPORTED on the host."""
    _no_gpu_here()
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    need = q.qlora_fwd_workspace_bytes(64, 64, 8, 4)
    assert _raw_fwd(d, fake, fake, fake, 8, fake, 4, fake, fake, fake + 2, fake, need) == q.QLORA_ERR_UNSUPPORTED
    nb = q.qlora_bwd_workspace_bytes(64, 64, 8, 4)
    f1 = ctypes.c_float(1.0)
    for dX, dA, dB in ((fake + 2, fake, fake), (fake, fake + 4, fake), (fake, fake, fake + 8)):
        assert L.qlora_linear_bwd(ctypes.byref(d), fake, fake, fake, 8, fake, 4, f1, fake, fake, None, fake, dX, dA,
                                  dB, fake, nb, None) == q.QLORA_ERR_UNSUPPORTED


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_multi_calls_validate_every_layer_before_the_first_launch():
    """A bad second layer makes the whole call fail on the host: the status
    is the validation error, not a launch failure from layer 0 (which, with
    no GPU here, is what a launch would report)."""
    _no_gpu_here()
    fake = 0x10000
    L = q.lib()
    f = ctypes.c_float(16.0)
    T, r = 40, 8
    d2 = (q.Nf4Desc * 2)(q._desc(128, 256), q._desc(64, 256))
    n = ctypes.c_size_t()
    assert L.qlora_multi_fwd_workspace_bytes(2, d2, T, r, ctypes.byref(n)) == q.QLORA_OK
    wsf = n.value
    assert L.qlora_multi_bwd_workspace_bytes(2, d2, T, r, ctypes.byref(n)) == q.QLORA_OK
    wsb = n.value
    P = _ptrs(fake, fake)
    for bad_packed, bad_A, bad_Y in (((fake, fake + 8), (fake, fake), (fake, fake)),
                                     ((fake, fake), (fake, fake + 2), (fake, fake)),
                                     ((fake, fake), (fake, fake), (fake, fake + 2))):
        st = L.qlora_linear_fwd_multi(2, d2, _ptrs(*bad_packed), P, P, T, fake, r, f, _ptrs(*bad_A), P,
                                      _ptrs(*bad_Y), None, fake, wsf, None)
        assert st == q.QLORA_ERR_UNSUPPORTED
    # a NULL B in the second layer
    st = L.qlora_linear_fwd_multi(2, d2, P, P, P, T, fake, r, f, P, _ptrs(fake, None), P, None, fake, wsf, None)
    assert st == q.QLORA_ERR_NULL
    # backward: misaligned A, dY or dA of the second layer; a short workspace
    for bad_A, bad_dY, bad_dA in (((fake, fake + 2), (fake, fake), (fake, fake)),
                                  ((fake, fake), (fake, fake + 2), (fake, fake)),
                                  ((fake, fake), (fake, fake), (fake, fake + 4))):
        st = L.qlora_linear_bwd_multi(2, d2, P, P, P, T, fake, r, f, _ptrs(*bad_A), P, None, _ptrs(*bad_dY), fake,
                                      _ptrs(*bad_dA), P, fake, wsb, None)
        assert st == q.QLORA_ERR_UNSUPPORTED
    st = L.qlora_linear_bwd_multi(2, d2, P, P, P, T, fake, r, f, P, P, None, P, fake, P, P, fake, wsb - 1, None)
    assert st == q.QLORA_ERR_WORKSPACE


def test_dropout_calls_validate_before_the_dropout_launch():
    """The dropout calls apply the mask in a launch of their own before the
    layer: everything is validated before that first launch."""
    _no_gpu_here()
    fake = 0x10000
    d = q._desc(64, 64)
    L = q.lib()
    f = ctypes.c_float
    big = 1 << 30
    # misaligned Y / misaligned dX: rejected, not a launch failure
    assert L.qlora_linear_fwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, fake,
                                      f(0.1), fake + 2, None, fake, big, None) == q.QLORA_ERR_UNSUPPORTED
    assert L.qlora_linear_bwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, None, fake,
                                      fake, f(0.1), fake + 2, fake, fake, 0, fake, big, None) == \
        q.QLORA_ERR_UNSUPPORTED
    # workspace that holds X_d but not the layer's own part
    n = ctypes.c_size_t()
    assert L.qlora_dropout_workspace_bytes(ctypes.byref(d), 4, 8, 0, ctypes.byref(n)) == q.QLORA_OK
    assert L.qlora_linear_fwd_dropout(ctypes.byref(d), fake, fake, fake, 4, fake, 8, f(16.0), fake, fake, fake,
                                      f(0.1), fake, None, fake, n.value - 1, None) == q.QLORA_ERR_WORKSPACE


def test_binding_checks_inputs_against_the_stored_weight():
    """The binding compares X, A, B and dY with the weight's shape and the
    rank before any call: too narrow a tensor would otherwise be read past its
    end by kernels that size their reads from the weight."""
    import torch
    bf = torch.bfloat16
    packed = torch.zeros(128, 128, dtype=torch.uint8)            # d_out 128, d_in 256
    codes = torch.zeros(128 * 256 // 64, dtype=torch.uint8)
    consts = torch.zeros(2, dtype=torch.float32)
    X = torch.zeros(8, 256, dtype=bf)
    A = torch.zeros(4, 256, dtype=bf)
    B = torch.zeros(128, 4, dtype=bf)
    dY = torch.zeros(8, 128, dtype=bf)
    bad_cases = [
        ("X must be", dict(X=torch.zeros(8, 192, dtype=bf))),
        ("X must be", dict(X=torch.zeros(8, 256, dtype=torch.float32))),
        ("A must be", dict(A=torch.zeros(4, 192, dtype=bf))),
        ("B must be", dict(B=torch.zeros(64, 4, dtype=bf))),
        ("B must be", dict(B=torch.zeros(128, 8, dtype=bf))),
        ("A and B", dict(B=None)),
    ]
    for msg, kw in bad_cases:
        a = dict(X=X, A=A, B=B)
        a.update(kw)
        with pytest.raises(ValueError, match=msg):
            q.qlora_linear_fwd(packed, codes, consts, a["X"], a["A"], a["B"], 16.0)
        with pytest.raises(ValueError, match=msg):
            q.qlora_linear_bwd(packed, codes, consts, a["X"], a["A"], a["B"], 16.0, dY)
    with pytest.raises(ValueError, match="dY must be"):
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, 16.0, torch.zeros(8, 64, dtype=bf))
    with pytest.raises(ValueError, match="dY must be"):
        q.qlora_linear_bwd(packed, codes, consts, X, A, B, 16.0, torch.zeros(4, 128, dtype=bf))
    with pytest.raises(ValueError, match="packed must be"):
        q.qlora_linear_fwd(packed.view(torch.int8), codes, consts, X, A, B, 16.0)
    with pytest.raises(ValueError, match="consts must be"):
        q.qlora_linear_fwd(packed, codes, consts.double(), X, A, B, 16.0)
    # correct shapes get as far as the device check
    with pytest.raises(ValueError, match="on the GPU"):
        q.qlora_linear_fwd(packed, codes, consts, X, A, B, 16.0)
    # several layers: each layer's adapter against its own weight, one rank for all
    small = torch.zeros(64, 128, dtype=torch.uint8)               # d_out 64
    scodes = torch.zeros(64 * 256 // 64, dtype=torch.uint8)
    sconsts = torch.zeros(1, dtype=torch.float32)
    layers = [(packed, codes, consts, A, B), (small, scodes, sconsts, A, torch.zeros(128, 4, dtype=bf))]
    with pytest.raises(ValueError, match=r"layers\[1\] B must be"):
        q.qlora_linear_fwd_multi(layers, X, 16.0)
    layers = [(packed, codes, consts, A, B), (small, scodes, sconsts, torch.zeros(8, 256, dtype=bf),
                                              torch.zeros(64, 8, dtype=bf))]
    with pytest.raises(ValueError, match=r"layers\[1\] A must be"):
        q.qlora_linear_fwd_multi(layers, X, 16.0)
    layers = [(packed, codes, consts, A, B), (small, scodes, sconsts, A, torch.zeros(64, 4, dtype=bf))]
    with pytest.raises(ValueError, match=r"dYs\[1\] must be"):
        q.qlora_linear_bwd_multi(layers, X, 16.0, [dY, dY])
    with pytest.raises(ValueError, match="A must be"):
        q.qlora_merge_lora(packed, codes, consts, torch.zeros(4, 128, dtype=bf), B, 16.0)


def test_noalloc_forward_validation_happens_before_any_launch():
    """The allocation-free forward validates like the plain one and refuses a
    call whose scratch exceeds the static array before looking it up."""
    _no_gpu_here()
    fake = 0x10000
    L = q.lib()
    f = ctypes.c_float(16.0)
    d = q._desc(64, 64)
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, fake, fake, 8, fake, 4, f, fake, fake, None, None,
                                      None) == q.QLORA_ERR_NULL
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, fake, fake, 8, fake, 4, f, fake, fake, fake + 2, None,
                                      None) == q.QLORA_ERR_UNSUPPORTED
    T = 40000
    assert q.qlora_fwd_workspace_bytes(64, 64, T, 64) > q.QLORA_STATIC_SCRATCH_BYTES
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, fake, fake, T, fake, 64, f, fake, fake, fake, None,
                                      None) == q.QLORA_ERR_SCRATCH_LIMIT
    assert q.qlora_fwd_workspace_bytes(64, 64, 32768, 64) <= q.QLORA_STATIC_SCRATCH_BYTES
