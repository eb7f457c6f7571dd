"""Every kernel writes its own outputs and nothing else.

Each output (O in the input dtype and in fp32, L, dQ, dK, dV) is a view
into a larger buffer whose head and tail hold a NaN bit pattern. After the
forward and backward calls the guard regions must be unchanged bit for bit
and the outputs finite. The shapes are ragged (no size a multiple of any
tile or of the 32-row output blocks), cover every head dim, both causal
masks, and grids that take the forward's and dQ's key split and the dK/dV
query split, so every store path runs: the staged whole-row stores with
partial blocks, the split partials and their merge / reduce passes, and
the fp32 kernels.
"""
import pytest
import torch

import exact_tiled_attention_29_amd as fa
import workloads

PAD = 4096                                # guard elements on each side (keeps 16-byte alignment)
SENTINEL = {2: 0x7FC1, 4: 0x7FC00001}     # NaN bit patterns for 16- and 32-bit elements

SHAPES = [
    # B, H, n_q, n_k, d, dtype, causal
    (1, 3, 100, 77, 64, "bf16", True),
    (2, 2, 257, 129, 128, "bf16", False),
    (1, 2, 300, 517, 96, "bf16", "bottom_right"),
    (1, 2, 129, 200, 32, "bf16", True),
    (1, 1, 70, 90, 256, "bf16", False),
    (1, 1, 1000, 4100, 128, "bf16", False),        # forward and dQ split the keys
    (1, 1, 4100, 300, 64, "bf16", True),           # dK/dV splits the queries
    (1, 1, 1000, 4100, 64, "bf16", "bottom_right"),
    (1, 2, 100, 100, 32, "f32", True),
    (1, 1, 33, 65, 128, "f32", False),
]


def _bits(buf):
    return buf.view(torch.int16 if buf.element_size() == 2 else torch.int32)


def guarded(shape, dtype, device="cuda"):
    """A view of `shape` in the middle of a buffer with guard regions."""
    n = 1
    for s in shape:
        n *= s
    buf = torch.empty(n + 2 * PAD, dtype=dtype, device=device)
    _bits(buf).fill_(SENTINEL[buf.element_size()])
    return buf, buf[PAD:PAD + n].view(shape)


def guards_intact(buf):
    bits, s = _bits(buf), SENTINEL[buf.element_size()]
    return bool((bits[:PAD] == s).all()) and bool((bits[-PAD:] == s).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_guards_catch_a_write_next_to_the_view(dtype):
    # the check itself, on the CPU: one element written just before or just
    # after the view (or the NaN pattern replaced by another NaN) is seen
    for where in (-1, 0):
        buf, view = guarded((2, 3, 5, 8), dtype, device="cpu")
        view.fill_(1.0)
        assert guards_intact(buf)
        buf[PAD - 1 if where == -1 else PAD + view.numel()] = 0.0
        assert not guards_intact(buf)
    buf, view = guarded((4, 8), dtype, device="cpu")
    _bits(buf)[-1] = SENTINEL[buf.element_size()] + 1
    assert not guards_intact(buf)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,n_q,n_k,d,dtype,causal", SHAPES)
def test_outputs_stay_in_bounds(B, H, n_q, n_k, d, dtype, causal):
    w = workloads.custom(B, H, n_q, n_k, d, dtype, causal)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(w, seed=11))
    tag = f"{B}x{H}x{n_q}x{n_k} d={d} {dtype} causal={causal}"
    bufs = {}
    o_dtypes = [q.dtype] + ([torch.float32] if q.dtype == torch.bfloat16 else [])
    for o_dtype in o_dtypes:
        ob, o = guarded((B, H, n_q, d), o_dtype)
        lb, l = guarded((B, H, n_q), torch.float32)
        fa.forward(q, k, v, causal, o_dtype=o_dtype, out=o, lse=l)
        bufs[f"O ({o_dtype})"], bufs[f"L ({o_dtype})"] = (ob, o), (lb, l)
    o, l = bufs[f"O ({q.dtype})"][1], bufs[f"L ({q.dtype})"][1]
    grads = {}
    for name, shape in (("dQ", q.shape), ("dK", k.shape), ("dV", v.shape)):
        grads[name] = guarded(tuple(shape), q.dtype)
    fa.backward(q, k, v, o, l, do, causal, grads=tuple(grads[n][1] for n in ("dQ", "dK", "dV")))
    bufs.update(grads)
    torch.cuda.synchronize()
    for name, (buf, view) in bufs.items():
        assert guards_intact(buf), f"{tag}: a kernel wrote outside {name}"
        if name.startswith("L"):
            # rows that see no key (bottom-right, n_q > n_k) have L = -inf
            assert not torch.isnan(view).any(), f"{tag}: NaN in {name}"
        else:
            assert torch.isfinite(view.float()).all(), f"{tag}: non-finite {name}"
