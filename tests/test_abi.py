"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/fa.h declares, and
reject bad arguments with the documented status codes before any HIP call.
Only argument-validation paths are exercised here: none of them reaches the
HIP runtime, so they run on a machine without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import exact_tiled_attention_29_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULLPTR, SHAPE, DTYPE, HEADDIM, SCALE, WORKSPACE, HIP, CAUSAL, SCRATCH, ALIGN = range(11)
BF16, F32 = 0, 1
REJECTED = (1 << 64) - 1   # fa_bwd_workspace_bytes for arguments fa_bwd rejects (SIZE_MAX)
P = 0x1000  # a non-null dummy pointer; never dereferenced on the validation paths


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.skip("libfa.so not built")
    return fa.load_library()


def test_header_declares_the_boundary():
    assert header_functions() == sorted(
        ["fa_fwd", "fa_fwd_ws", "fa_fwd_workspace_bytes", "fa_bwd", "fa_bwd_timed", "fa_bwd_noalloc",
         "fa_bwd_workspace_bytes", "fa_row_softmax", "fa_status_str", "fa_abi_version"])


def test_library_exports_every_header_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(fa_[a-z_0-9]+)$", out, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    assert lib.fa_abi_version() == 5
    for code in range(11):
        s = fa.fa_status_str(code)
        assert s and s != "unknown status"
    assert fa.fa_status_str(99) == "unknown status"


def fwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, o_dtype=BF16, lse=P, batch=1, heads=1, n_q=8, n_k=8, d=64,
                dtype=BF16, causal=0, scale=0.125, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


def fwd_ws(**kw):
    args = dict(q=P, k=P, v=P, o=P, o_dtype=BF16, lse=P, batch=1, heads=1, n_q=8, n_k=8, d=64,
                dtype=BF16, causal=0, scale=0.125, workspace=P, workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return fa.fa_fwd_ws(**args)


def bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, o_dtype=BF16, lse=P, d_o=P, dq=P, dk=P, dv=P, batch=1, heads=1,
                n_q=8, n_k=8, d=64, dtype=BF16, causal=0, scale=0.125, workspace=P,
                workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("call", [fwd, fwd_ws, bwd])
def test_validation_codes(lib, call):
    assert call(dtype=7) == DTYPE
    assert call(o_dtype=5) == DTYPE
    assert call(dtype=F32, o_dtype=BF16, d=32) == DTYPE
    assert call(batch=-1) == SHAPE
    assert call(n_q=-3) == SHAPE
    assert call(n_k=0) == SHAPE
    assert call(heads=1 << 20, batch=1 << 12) == SHAPE
    for d in (0, 16, 48, 80, 112, 160, 192, 512):   # bf16: 32, 64, 96, 128, 256
        assert call(d=d) == HEADDIM, d
    for d in (32, 64, 96, 128, 256):
        assert call(d=d, q=None) == NULLPTR, d
    for d in (8, 48, 256):                          # f32: 16, 32, 64, 96, 128
        assert call(dtype=F32, o_dtype=F32, d=d) == HEADDIM, d
    for d in (16, 32, 64, 96, 128):
        assert call(dtype=F32, o_dtype=F32, d=d, q=None) == NULLPTR, d
    assert call(scale=0.0) == SCALE
    assert call(scale=-1.0) == SCALE
    assert call(scale=float("inf")) == SCALE
    assert call(scale=float("nan")) == SCALE
    assert call(q=None) == NULLPTR
    assert call(v=None) == NULLPTR
    assert call(lse=None) == NULLPTR
    # causal: 0 none, 1 top-left, 2 bottom-right; anything else is refused
    for bad in (3, -1, 255):
        assert call(causal=bad) == CAUSAL
    for good in (1, 2):
        assert call(causal=good, q=None) == NULLPTR   # accepted, then the pointer check
    # one head's Q, K or V must stay under 2 GiB (32-bit byte offsets)
    assert call(n_q=1 << 23, n_k=8, d=128) == SHAPE
    assert call(n_k=1 << 23, d=128) == SHAPE
    assert call(n_k=(1 << 23) - 1, d=128, q=None) == NULLPTR
    assert call(dtype=F32, o_dtype=F32, n_k=1 << 22, d=128) == SHAPE


@pytest.mark.parametrize("call", [fwd, fwd_ws, bwd])
def test_tensor_pointers_must_be_16_byte_aligned(lib, call):
    names = ["q", "k", "v", "o"] + (["d_o", "dq", "dk", "dv"] if call is bwd else [])
    for name in names:
        for off in (2, 4, 8):
            assert call(**{name: P + off}) == ALIGN, (name, off)
        assert call(**{name: P + 16}) != ALIGN, name
    # null pointers are reported first; L (fp32, read and written per row)
    # needs only its natural alignment
    assert call(q=P + 2, k=None) == NULLPTR
    assert call(lse=P + 4) != ALIGN
    # an empty backward still writes dK, dV: they are checked too
    if call is bwd:
        assert call(n_q=0, dk=P + 8) == ALIGN
        assert call(n_q=0, q=P + 8) != ALIGN
    for name in ("q", "dq", "dv"):
        assert noalloc(**{name: P + 2}) == ALIGN, name


def test_backward_specific_codes(lib):
    assert bwd(d_o=None) == NULLPTR
    assert bwd(dq=None) == NULLPTR
    assert bwd(workspace=None) == WORKSPACE
    need = fa.fa_bwd_workspace_bytes(1, 1, 8, 8, 64, BF16, 0)
    assert bwd(workspace_bytes=need - 1) == WORKSPACE
    assert bwd(workspace=P + 4) == WORKSPACE  # not 256-byte aligned


def noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, o_dtype=BF16, lse=P, d_o=P, dq=P, dk=P, dv=P, batch=1, heads=1,
                n_q=8, n_k=8, d=64, dtype=BF16, causal=0, scale=0.125, stream=None)
    args.update(kw)
    return fa.fa_bwd_noalloc(**args)


def test_noalloc_validation_codes(lib):
    # the same host checks as fa_bwd, all before any HIP call
    assert noalloc(dtype=7) == DTYPE
    assert noalloc(n_k=0) == SHAPE
    assert noalloc(d=80) == HEADDIM
    assert noalloc(scale=0.0) == SCALE
    assert noalloc(causal=3) == CAUSAL
    assert noalloc(q=None) == NULLPTR
    assert noalloc(d_o=None) == NULLPTR
    assert noalloc(dq=None) == NULLPTR
    assert noalloc(dtype=F32, o_dtype=F32, d=32, dv=None) == NULLPTR
    # beyond the static scratch: refused with nothing launched
    cap = fa.FA_BWD_NOALLOC_SCRATCH_BYTES
    rows = 1 << 21                       # bf16 needs 8 bytes per padded query row
    assert fa.fa_bwd_workspace_bytes(1, 64, rows // 64, 8, 64, BF16, 0) == cap
    assert fa.fa_bwd_workspace_bytes(1, 64, rows // 64 + 32, 8, 64, BF16, 0) > cap
    assert noalloc(heads=64, n_q=rows // 64 + 32) == SCRATCH
    assert noalloc(heads=64, n_q=rows // 64 + 32, q=None) == NULLPTR   # pointers checked first
    assert noalloc(batch=2, heads=64, n_q=rows // 64 + 1, dtype=F32, o_dtype=F32, d=32) == SCRATCH
    # empty: nothing to compute, no scratch needed
    assert noalloc(batch=0, q=None, dq=None) == OK


def test_empty_forward_is_a_noop(lib):
    # Nothing to compute: returns before any HIP call, pointers untouched.
    for call in (fwd, fwd_ws):
        assert call(n_q=0, q=None, o=None, lse=None) == OK
        assert call(batch=0, q=None, k=None, v=None, o=None, lse=None) == OK
        assert call(heads=0, n_k=0) == OK
    assert fwd_ws(n_q=0, workspace=None, workspace_bytes=0) == OK


def test_forward_workspace_bytes(lib):
    # SIZE_MAX for what fa_fwd rejects; 0 for empty calls and for the paths
    # that never split (float32, head dims other than 64 and 128, few keys)
    assert fa.fa_fwd_workspace_bytes(1, 1, 8, 8, 80, BF16, 0) == REJECTED
    assert fa.fa_fwd_workspace_bytes(1, 1, 8, 0, 64, BF16, 0) == REJECTED
    assert fa.fa_fwd_workspace_bytes(1, 1, 8, 8, 64, BF16, 3) == REJECTED
    assert fa.fa_fwd_workspace_bytes(1, 1, 8, 8, 64, 9, 0) == REJECTED
    assert fa.fa_fwd_workspace_bytes(0, 1, 8, 8, 64, BF16, 0) == 0
    assert fa.fa_fwd_workspace_bytes(1, 1, 4096, 4096, 32, F32, 0) == 0
    assert fa.fa_fwd_workspace_bytes(1, 1, 4096, 4096, 96, BF16, 0) == 0
    assert fa.fa_fwd_workspace_bytes(1, 1, 4096, 511, 128, BF16, 0) == 0


def test_workspace_bytes(lib):
    def up(x):
        return (x + 255) // 256 * 256
    B, H, n_q, n_k, d = 2, 3, 100, 77, 128
    rows = B * H * n_q
    pad = (n_q + 31) // 32 * 32
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, d, BF16, 1) == 2 * up(B * H * pad * 4)
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, 32, F32, 0) == up(rows * 4)
    assert fa.fa_bwd_workspace_bytes(B, H, 0, n_k, d, BF16, 0) == 0
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, 80, BF16, 0) == REJECTED
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, 96, BF16, 0) == 2 * up(B * H * pad * 4)
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, 0, d, BF16, 0) == REJECTED
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, d, BF16, 2) == 2 * up(B * H * pad * 4)
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, d, BF16, 3) == REJECTED
    assert fa.fa_bwd_workspace_bytes(B, H, n_q, n_k, d, 5, 0) == REJECTED
    assert fa.fa_bwd_workspace_bytes(B, H, -1, n_k, d, BF16, 0) == REJECTED


def test_mask_codes_of_the_binding():
    assert fa._mask_code(False) == fa.FA_NO_MASK == 0
    assert fa._mask_code(True) == fa.FA_CAUSAL_TOP_LEFT == 1
    assert fa._mask_code("top_left") == 1
    assert fa._mask_code("bottom_right") == fa.FA_CAUSAL_BOTTOM_RIGHT == 2
    assert fa._mask_code("none") == 0
    with pytest.raises(ValueError):
        fa._mask_code("lower_right")


def rows_call(**kw):
    args = dict(x=P, dtype=BF16, rows=4, cols=8, scale=1.0, lse=P, y=P, y_dtype=BF16, stream=None)
    args.update(kw)
    return fa.fa_row_softmax(**args)


def test_row_softmax_validation_codes(lib):
    assert rows_call(dtype=2) == DTYPE
    assert rows_call(y_dtype=-1) == DTYPE
    assert rows_call(rows=-1) == SHAPE
    assert rows_call(cols=-2) == SHAPE
    assert rows_call(cols=0) == SHAPE
    assert rows_call(rows=1 << 40, cols=2) == SHAPE
    assert rows_call(scale=0.0) == SCALE
    assert rows_call(scale=float("nan")) == SCALE
    assert rows_call(x=None) == NULLPTR
    assert rows_call(lse=None) == NULLPTR
    # nothing to compute: returns before any HIP call
    assert rows_call(rows=0, x=None, lse=None, y=None) == OK
    assert rows_call(rows=0, cols=0) == OK


@pytest.mark.parametrize("call", [fwd, fwd_ws, bwd])
def test_binding_refuses_sizes_past_32_bits(lib, call):
    # ctypes would hand 2**32 + 100 to the library as 100: the binding stops
    # such values before the call (with null pointers, a call that got
    # through would return NULLPTR instead of raising)
    for name in ("batch", "heads", "n_q", "n_k", "d"):
        for bad in ((1 << 32) + 100, 1 << 31, -(1 << 31) - 1):
            with pytest.raises(ValueError, match=name):
                call(**{name: bad, "q": None})
    with pytest.raises(ValueError, match="causal"):
        call(causal=(1 << 32) + 1, q=None)
    assert call(n_q=(1 << 31) - 1, q=None) == SHAPE   # fits, and the library refuses it
    for size_fn in (fa.fa_fwd_workspace_bytes, fa.fa_bwd_workspace_bytes):
        with pytest.raises(ValueError, match="heads"):
            size_fn(1, (1 << 32) + 1, 8, 8, 64, BF16, 0)
    with pytest.raises(ValueError, match="cols"):
        rows_call(cols=(1 << 32) + 8)


def test_python_helpers_refuse_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q)
    with pytest.raises(TypeError):
        fa.forward(q.half(), q.half(), q.half())
    with pytest.raises(ValueError, match="GPU"):
        fa.row_softmax(q)
