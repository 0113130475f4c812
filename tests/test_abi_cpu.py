"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/mnb.h declares, and rejects every invalid call on the host
before any HIP call (so no call here reaches a kernel)."""

import ctypes
import os
import re

import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from weight_only_int4_matmulnbits_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mnb.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mnb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_probe_library_exports_its_header():
    """The benchmark's control-arm library (not part of libmnb) exports
    exactly what include/mnb_probe.h declares, and refuses bad arguments on
    the host."""
    import torch  # noqa: F401
    hdr = os.path.join(os.path.dirname(HEADER), "mnb_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mnb_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mnb_probe_stream_read"]
    L = ctypes.CDLL(os.path.join(os.path.dirname(_lib.LIB_PATH), "libmnb_probe.so"))
    f = L.mnb_probe_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 16, P16, None) == -1
    assert f(P16, 17, P16, None) == -1
    assert f(P16 + 8, 16, P16, None) == -1
    assert f(P16, 16, None, None) == -1


def test_library_exports_every_declared_symbol():
    L = mnb.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert mnb.version().startswith("mnb")


def test_sizes():
    d = mnb.make_desc(1024, 3072, 32)
    assert mnb.packed_weight_bytes(d) == 3072 * 1024 // 2
    assert mnb.scale_bytes(d) == 3072 * 32 * 4
    assert mnb.zero_point_bytes(d) == 0
    d = mnb.make_desc(2560, 151936, 128, has_zero_points=True)
    assert mnb.packed_weight_bytes(d) == 151936 * 20 * 64
    assert mnb.zero_point_bytes(d) == 151936 * 10
    d = mnb.make_desc(20, 3, 16, has_zero_points=True)   # partial block, odd nb
    assert mnb.packed_weight_bytes(d) == 3 * 2 * 8
    assert mnb.zero_point_bytes(d) == 3 * 1
    d = mnb.make_desc(100, 5, 64, act_dtype=__import__("torch").bfloat16)
    assert mnb.scale_bytes(d) == 5 * 2 * 2
    # the memory gate on the page "Qwen3 CPU Inference Critical Path"
    # ("Benchmark gates", INT4 memory: packed <= 1.25x serialized): the packed
    # layout IS the serialized MatMulNBits layout, i.e. exactly 1.00x
    for K, N, bs in [(1024, 3072, 32), (9728, 2560, 128), (1000, 7, 16)]:
        d = mnb.make_desc(K, N, bs, has_zero_points=True)
        nb = -(-K // bs)
        serialized = N * nb * bs // 2 + N * nb * 4 + N * (-(-nb // 2))
        got = mnb.packed_weight_bytes(d) + mnb.scale_bytes(d) + mnb.zero_point_bytes(d)
        assert got == serialized


def _status(desc, M=1):
    return mnb.lib().mnb_validate(ctypes.byref(desc), M)


@pytest.mark.parametrize("field,value,status", [
    ("bits", 8, -2), ("bits", 2, -2), ("block_size", 24, -2), ("block_size", 8, -2),
    ("block_size", 512, -2), ("act_dtype", 2, -2), ("reserved", 1, -2),
    ("K", 0, -1), ("N", 0, -1), ("K", -5, -1), ("has_zero_points", 2, -1),
    ("accuracy_level", 5, -1), ("K", 1 << 31, -4), ("N", 1 << 40, -4),
])
def test_validate_rejects(field, value, status):
    d = mnb.make_desc(64, 8, 32)
    setattr(d, field, value)
    assert _status(d) == status
    assert mnb.lib().mnb_last_error().decode()


def test_validate_accepts_contract():
    for bs in (16, 32, 64, 128, 256):
        for al in range(5):
            assert _status(mnb.make_desc(1, 1, bs, accuracy_level=al)) == 0
    assert _status(mnb.make_desc(64, 8, 32), M=0) == -1


def test_sizes_of_invalid_desc_are_zero():
    d = mnb.make_desc(64, 8, 24)
    assert mnb.packed_weight_bytes(d) == 0 and mnb.scale_bytes(d) == 0


P16 = 0x10000          # fake, never dereferenced: each call below fails validation
P_MIS = 0x10008        # 8-byte aligned only


def _gemv(d, M=1, a=P16, b=P16, s=P16, zp=None, bias=None, y=P16, fn="mnb_gemv", ws=None, ws_bytes=0):
    f = getattr(mnb.lib(), fn)
    if fn == "mnb_gemm":
        return f(ctypes.byref(d), M, a, b, s, zp, bias, y, ws, ws_bytes, None)
    return f(ctypes.byref(d), M, a, b, s, zp, bias, y, None)


@pytest.mark.parametrize("fn", ["mnb_gemv", "mnb_gemm"])
def test_matmul_argument_errors(fn):
    d = mnb.make_desc(64, 8, 32)
    dz = mnb.make_desc(64, 8, 32, has_zero_points=True)
    assert _gemv(d, a=None, fn=fn) == -1
    assert _gemv(d, y=None, fn=fn) == -1
    assert _gemv(d, s=None, fn=fn) == -1
    assert _gemv(d, zp=P16, fn=fn) == -1          # zp given without has_zero_points
    assert _gemv(dz, zp=None, fn=fn) == -1        # has_zero_points without zp
    assert _gemv(d, a=P_MIS, fn=fn) == -3
    assert _gemv(d, b=P_MIS, fn=fn) == -3
    assert _gemv(d, y=0x10002, fn=fn) == -3       # f32 output needs 4-byte alignment
    assert _gemv(d, bias=0x10002, fn=fn) == -3
    assert _gemv(d, M=0, fn=fn) == -1
    bad = mnb.make_desc(64, 8, 32)
    bad.bits = 3
    assert _gemv(bad, fn=fn) == -2
    assert "bits" in mnb.lib().mnb_last_error().decode()


def test_gemv_requires_single_row():
    d = mnb.make_desc(64, 8, 32)
    assert _gemv(d, M=2) == -1
    assert "M == 1" in mnb.lib().mnb_last_error().decode()
    assert _gemv(d, M=(65535 * 128) + 1, fn="mnb_gemm") == -4


def test_pack_and_dequant_argument_errors():
    L = mnb.lib()
    d = mnb.make_desc(64, 8, 32)
    dz = mnb.make_desc(64, 8, 32, has_zero_points=True)
    assert L.mnb_pack(ctypes.byref(d), None, None, P16, None, None) == -1
    assert L.mnb_pack(ctypes.byref(d), P16, None, P_MIS, None, None) == -3
    assert L.mnb_pack(ctypes.byref(dz), P16, None, P16, None, None) == -1
    assert L.mnb_pack(ctypes.byref(d), P16, P16, P16, P16, None) == -1
    assert L.mnb_dequant(ctypes.byref(d), P16, P16, None, 3, P16, None) == -1
    assert L.mnb_dequant(ctypes.byref(d), P16, None, None, 0, P16, None) == -1
    assert L.mnb_dequant(ctypes.byref(d), P16, P16, None, 0, 0x10002, None) == -3


def test_sequence_validates_every_entry_before_launching():
    L = mnb.lib()
    good = _lib.MatmulArgs(desc=mnb.make_desc(64, 8, 32), M=1, a=P16, b_packed=P16,
                           scales=P16, zp_packed=None, bias=None, y=P16)
    bad = _lib.MatmulArgs(desc=mnb.make_desc(64, 8, 24), M=1, a=P16, b_packed=P16,
                          scales=P16, zp_packed=None, bias=None, y=P16)
    arr = (_lib.MatmulArgs * 2)(good, bad)
    # the invalid second entry stops the call before the first is launched
    assert L.mnb_matmul_sequence(arr, 2, None, 0, None) == -2
    assert "entry 1" in L.mnb_last_error().decode()
    g = ctypes.c_void_p()
    assert L.mnb_graph_create(arr, 2, None, 0, ctypes.byref(g)) == -2
    assert not g.value
    assert L.mnb_graph_create(arr, 2, None, 0, None) == -1
    assert L.mnb_graph_launch(None, None) == -1
    assert L.mnb_graph_destroy(None) == 0
    assert L.mnb_matmul_sequence(arr, -1, None, 0, None) == -1
    assert L.mnb_sequence_workspace_bytes(arr, 2) == 0          # invalid entry


def test_status_strings():
    L = mnb.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.mnb_status_string(s).decode().startswith("MNB_")
    assert b"unknown" in L.mnb_status_string(42)


def test_import_qdq_argument_errors():
    L = mnb.lib()
    dz = mnb.make_desc(64, 8, 32, has_zero_points=True)
    d = mnb.make_desc(64, 8, 32)

    def imp(desc, axis=0, w=P16, s=0x20000, z=None, b=0x30000, so=0x40000, zo=0x50000):
        return L.mnb_import_qdq(ctypes.byref(desc), axis, w, s, z, b, so, zo, None)

    assert imp(dz, axis=2) == -1
    assert imp(d) == -1                              # the result always has zero points
    assert "has_zero_points" in L.mnb_last_error().decode()
    assert imp(dz, w=None) == -1
    assert imp(dz, zo=None) == -1
    assert imp(dz, b=0x30008) == -3                  # b_packed needs 16-byte alignment
    assert imp(dz, s=0x20002) == -3                  # float32 scales need 4
    assert imp(dz, b=P16 + 16) == -1                 # b_packed overlaps w_q (256 bytes)
    assert "overlap" in L.mnb_last_error().decode()


def test_qdq_native_storage_rule():
    # axis 1, whole blocks, even block count per row, zero points present
    assert mnb.qdq_is_native(1024, 151936, 32, axis=1)
    assert mnb.qdq_is_native(2560, 151936, 128, axis=1)
    assert not mnb.qdq_is_native(1024, 151936, 32, axis=0)      # needs the transpose
    assert not mnb.qdq_is_native(96, 10, 32, axis=1)            # 3 blocks: zero-point rows straddle
    assert not mnb.qdq_is_native(100, 10, 32, axis=1)           # partial block: rows straddle
    assert not mnb.qdq_is_native(1024, 10, 32, axis=1, has_zero_points=False)


def test_gather_argmax_silu_argument_errors():
    L = mnb.lib()
    d = mnb.make_desc(64, 8, 32)
    assert L.mnb_gather_rows(ctypes.byref(d), P16, -1, P16, P16, None, P16, None) == -1
    assert L.mnb_gather_rows(ctypes.byref(d), P16, 0, None, None, None, None, None) == 0   # nothing to do
    assert L.mnb_gather_rows(ctypes.byref(d), 0x10004, 2, P16, P16, None, P16, None) == -3
    assert L.mnb_gather_rows(ctypes.byref(d), P16, 2, P16, P16, P16, P16, None) == -1      # zp without flag
    assert L.mnb_argmax(2, 1, 8, P16, P16, None, 0, None) == -2
    assert L.mnb_argmax(0, 0, 8, P16, P16, None, 0, None) == -1
    assert L.mnb_argmax(0, 1, 0, P16, P16, None, 0, None) == -1
    assert L.mnb_argmax(0, 1, 8, P16, 0x10004, None, 0, None) == -3
    odd = mnb.make_desc(64, 7, 32)
    assert _gemv(odd, fn="mnb_gemv_silu_mul") == -1
    assert "even" in L.mnb_last_error().decode()
    assert _gemv(d, M=2, fn="mnb_gemv_silu_mul") == -1


# ---- caller-provided workspace ("Prepared weight-only plan": a bounded
# workspace is part of the plan) ---------------------------------------------

def _ws(K, N, M, bs, dt="f32", zp=True):
    import torch
    adt = torch.float32 if dt == "f32" else torch.bfloat16
    return mnb.workspace_bytes(mnb.make_desc(K, N, bs, adt, zp), M)


def test_workspace_sizes_are_a_function_of_the_shape():
    """The K split (and so the workspace) follows from the shape alone, sized
    for 256 CUs: float32 partial slices of M x N for split products, of the
    last round's 256 x 256 tiles for a split tail, none for the decode,
    row and small-M kernels."""
    MB = 2048 * 2560 * 4
    # Qwen3-4B prefill, 2048 bf16 rows, block 128: o and down (80 tiles of
    # 256 x 256) split K three ways; gate||up (608 tiles) splits its last
    # 96 tiles two ways; qkv (192 tiles) and the LM head run unsplit
    assert _ws(4096, 2560, 2048, 128, "bf16") == 3 * MB
    assert _ws(9728, 2560, 2048, 128, "bf16") == 3 * MB
    assert _ws(2560, 19456, 2048, 128, "bf16") == 2 * 96 * 256 * 256 * 4
    assert _ws(2560, 6144, 2048, 128, "bf16") == 0
    assert _ws(2560, 151936, 2048, 128, "bf16") == 0
    # Qwen3-0.6B prefill, 512 float32 rows, block 32: o and down (128 tiles
    # of 64 x 64) take four splits; qkv, gate||up and the LM head none
    assert _ws(2048, 1024, 512, 32) == 4 * 512 * 1024 * 4
    assert _ws(3072, 1024, 512, 32) == 4 * 512 * 1024 * 4
    assert _ws(1024, 4096, 512, 32) == 0
    assert _ws(1024, 6144, 512, 32) == 0
    assert _ws(1024, 151936, 512, 32) == 0
    # decode, 2-4 rows, small M: no workspace
    for M in (1, 2, 3, 4, 8, 16):
        assert _ws(2560, 151936, M, 128) == 0
    # invalid descriptor or M
    assert mnb.workspace_bytes(mnb.make_desc(64, 8, 24), 600) == 0
    assert mnb.workspace_bytes(mnb.make_desc(64, 8, 32), 0) == 0


def test_gemm_refuses_a_missing_or_short_workspace():
    d = mnb.make_desc(2048, 1024, 32, has_zero_points=True)
    need = mnb.workspace_bytes(d, 512)
    assert need > 0
    L = mnb.lib()
    assert _gemv(d, M=512, zp=P16, fn="mnb_gemm") == -1
    assert "workspace" in L.mnb_last_error().decode()
    assert _gemv(d, M=512, zp=P16, fn="mnb_gemm", ws=0x100000, ws_bytes=need - 1) == -1
    assert _gemv(d, M=512, zp=P16, fn="mnb_gemm", ws=0x100010, ws_bytes=need) == -3   # 256-byte aligned
    # a product that needs none ignores what is offered
    d1 = mnb.make_desc(1024, 4096, 32, has_zero_points=True)
    assert mnb.workspace_bytes(d1, 512) == 0


def test_bf16_block16_scales_need_word_alignment_in_gemm():
    import torch
    d = mnb.make_desc(64, 8, 16, torch.bfloat16)
    assert _gemv(d, M=300, s=0x10002, fn="mnb_gemm") == -3
    assert "4-byte" in mnb.lib().mnb_last_error().decode()


def test_gemv_refuses_k_beyond_the_register_kernel():
    d = mnb.make_desc(20000, 8, 32)
    assert 20000 > mnb.gemv_max_k(d)
    assert _gemv(d) == -2
    assert "mnb_gemm" in mnb.lib().mnb_last_error().decode()


def test_argmax_workspace_rule():
    assert mnb.argmax_workspace_bytes(1, 2048) == 0          # one segment: one workgroup per row
    one = mnb.argmax_workspace_bytes(1, 151936)
    assert one > 0 and mnb.argmax_workspace_bytes(3, 151936) == 3 * one
    assert mnb.argmax_workspace_bytes(70000, 151936) == 0    # beyond grid.y: one workgroup per row
    assert mnb.argmax_workspace_bytes(0, 10) == 0
    L = mnb.lib()
    assert L.mnb_argmax(0, 1, 151936, P16, P16, None, 0, None) == -1
    assert L.mnb_argmax(0, 1, 151936, P16, P16, 0x100000, one - 1, None) == -1


def test_sequence_workspace_is_the_largest_entry():
    L = mnb.lib()
    mk = lambda K, N, M: _lib.MatmulArgs(desc=mnb.make_desc(K, N, 32, has_zero_points=True), M=M,  # noqa: E731
                                         a=P16, b_packed=P16, scales=P16, zp_packed=P16, bias=None, y=P16)
    arr = (_lib.MatmulArgs * 3)(mk(1024, 4096, 512), mk(2048, 1024, 512), mk(1024, 4096, 1))
    assert L.mnb_sequence_workspace_bytes(arr, 3) == 4 * 512 * 1024 * 4
    assert L.mnb_matmul_sequence(arr, 3, None, 0, None) == -1
    assert L.mnb_matmul_sequence(arr, 3, 0x100000, 4 * 512 * 1024 * 4 - 4, None) == -1
    g = ctypes.c_void_p()
    assert L.mnb_graph_create(arr, 3, None, 0, ctypes.byref(g)) == -1
    assert not g.value


def test_gated_gemm_workspace_and_arguments():
    import torch
    # Qwen3-4B prefill gate||up: the wide kernel's split last round only
    d = mnb.make_desc(2560, 19456, 128, torch.bfloat16, True)
    assert mnb.gemm_silu_workspace_bytes(d, 2048) == 2 * 96 * 256 * 256 * 4
    # one row: the gated decode GEMV, no workspace
    assert mnb.gemm_silu_workspace_bytes(d, 1) == 0
    # float32 activations: the unfused path keeps y [M][N] (after the
    # product's own workspace, 256-byte aligned)
    d32 = mnb.make_desc(1024, 6144, 32, has_zero_points=True)
    assert mnb.gemm_silu_workspace_bytes(d32, 512) == 512 * 6144 * 4
    # odd N is no gated weight
    assert mnb.gemm_silu_workspace_bytes(mnb.make_desc(64, 7, 32), 4) == 0
    L = mnb.lib()
    odd = mnb.make_desc(64, 7, 32)
    assert L.mnb_gemm_silu_mul(ctypes.byref(odd), 4, P16, P16, P16, None, None, P16, None, 0, None) == -1
    assert "even" in L.mnb_last_error().decode()
    assert L.mnb_gemm_silu_mul(ctypes.byref(d32), 512, P16, P16, P16, P16, None, P16, None, 0, None) == -1
    assert "workspace" in L.mnb_last_error().decode()


def test_gemv_rmsnorm_argument_errors():
    L = mnb.lib()
    d = mnb.make_desc(64, 8, 32)

    def call(desc, M=1, x=P16, gamma=0x20000, eps=1e-6, b=P16, s=P16, zp=None, y=P16):
        return L.mnb_gemv_rmsnorm(ctypes.byref(desc), M, x, gamma, eps, b, s, zp, None, y, None)

    assert call(d, gamma=None) == -1
    assert call(d, gamma=0x20008) == -3              # gamma needs 16-byte alignment
    assert call(d, eps=-1.0) == -1
    assert call(d, eps=float("nan")) == -1
    assert call(d, M=2) == -1
    assert call(mnb.make_desc(66, 8, 32)) == -2      # K * 4 not a multiple of 16
    assert call(mnb.make_desc(20000, 8, 32)) == -2   # past the decode kernel


def test_persistent_step_workspace_and_refusals():
    """mnb_step_*: the workspace is the counter header (2304 bytes) plus the
    entry table (112 bytes an entry, rounded up to 256), and entries the step
    kernel does not take are refused before any HIP call."""
    L = mnb.lib()

    def mk(K, N, M=1, bs=128, dt=torch.float32, zp=False):
        return _lib.MatmulArgs(desc=mnb.make_desc(K, N, bs, act_dtype=dt, has_zero_points=zp), M=M, a=P16,
                               b_packed=P16, scales=P16, zp_packed=P16 if zp else None, bias=None, y=P16)

    # the Qwen3-4B decode step's 145 entries
    layer = [mk(2560, 6144), mk(4096, 2560), mk(2560, 19456), mk(9728, 2560)]
    ents = layer * 36 + [mk(2560, 151936)]
    arr = (_lib.MatmulArgs * len(ents))(*ents)
    assert L.mnb_step_workspace_bytes(arr, len(ents)) == 2304 + ((145 * 112 + 255) // 256) * 256
    one = (_lib.MatmulArgs * 1)(mk(1024, 3072, bs=32, zp=True))
    assert L.mnb_step_workspace_bytes(one, 1) == 2304 + 256
    h = ctypes.c_void_p()
    # refusals: status, and nothing launched (no GPU here)
    cases = [
        ((mk(1024, 64, M=2),), -2),                  # M != 1
        ((mk(1024, 64, bs=16),), -2),                # 16-value blocks
        ((mk(1022, 64),), -2),                       # K * 4 not a multiple of 16
        ((mk(12288, 64),), -2),                      # needs split-K wavefront teams
        ((mk(1024, 64), mk(1024, 64, dt=torch.bfloat16)), -2),    # mixed activation types
    ]
    for ents, st in cases:
        arr = (_lib.MatmulArgs * len(ents))(*ents)
        assert L.mnb_step_workspace_bytes(arr, len(ents)) == 0, ents
        assert L.mnb_step_create(arr, len(ents), 0x100000, 1 << 20, ctypes.byref(h)) == st
        assert not h.value
    assert L.mnb_step_create(one, 0, 0x100000, 1 << 20, ctypes.byref(h)) == -1          # n_ops 0
    assert L.mnb_step_create(one, 1, None, 0, ctypes.byref(h)) == -1                     # no workspace
    assert L.mnb_step_create(one, 1, 0x100000, 2304 + 255, ctypes.byref(h)) == -1       # too small
    assert L.mnb_step_create(one, 1, 0x100010, 1 << 20, ctypes.byref(h)) == -3          # misaligned
    assert L.mnb_step_create(one, 1, 0x100000, 1 << 20, None) == -1
    # y inside the workspace
    bad = (_lib.MatmulArgs * 1)(_lib.MatmulArgs(desc=mnb.make_desc(1024, 64, 32), M=1, a=P16, b_packed=P16,
                                                scales=P16, zp_packed=None, bias=None, y=0x100100))
    assert L.mnb_step_create(bad, 1, 0x100000, 1 << 20, ctypes.byref(h)) == -1
    assert L.mnb_step_launch(None, None) == -1
    assert L.mnb_step_check(None, None) == -1
    assert L.mnb_step_destroy(None) == 0
    assert L.mnb_step_trace_bytes(None) == 0
    assert L.mnb_step_set_trace(None, None, 0) == -1
