"""fa_bwd_noalloc (the backward with the library's static per-GPU scratch)
against fa_bwd with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the gradients must agree
bit for bit. Two calls in a row, the second smaller, check that a call does
not depend on what the previous one left in the shared scratch."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_tiled_attention_29_amd as fa


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    yield
    torch.cuda.empty_cache()


def _grads_both_ways(w):
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(w, seed=3))
    o, lse = fa.forward(q, k, v, w.causal)
    ref = fa.backward(q, k, v, o, lse, do, w.causal)
    dt = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    got = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
           torch.full_like(v, float("nan")))
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dt,
                           lse.data_ptr(), do.data_ptr(), got[0].data_ptr(), got[1].data_ptr(),
                           got[2].data_ptr(), w.batch, w.heads, w.n_q, w.n_k, w.d, dt,
                           fa._mask_code(w.causal), 1.0 / w.d ** 0.5,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_status_str(st)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    (workloads.custom(2, 8, 1000, 1000, 128, "bf16", True), workloads.custom(1, 3, 77, 300, 64, "bf16", False)),
    (workloads.custom(1, 4, 513, 200, 64, "bf16", "bottom_right"), workloads.custom(1, 1, 100, 100, 32, "f32", True)),
])
def test_noalloc_matches_workspace_path(first, second):
    for w in (first, second):
        ref, got = _grads_both_ways(w)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), f"{w}: {name} differs from fa_bwd"


def test_noalloc_with_the_dq_key_split():
    # few query tiles and 4096 keys: fa_bwd splits dQ's keys. Small partials
    # fit in the scratch and noalloc splits the same way (bitwise equal);
    # 33 MB of partials (dQ's, and dK/dV's from the query split) do not, and
    # noalloc runs both kernels unsplit (the same gradients up to rounding).
    small = workloads.custom(1, 2, 128, 4096, 64, "bf16", "bottom_right")
    ref, got = _grads_both_ways(small)
    for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(a, b), f"{small}: {name} differs from fa_bwd"
    big = workloads.custom(1, 2, 4096, 4096, 128, "bf16", True)
    need = fa.fa_bwd_workspace_bytes(1, 2, 4096, 4096, 128, fa.FA_BF16, 1)
    assert need > fa.FA_BWD_NOALLOC_SCRATCH_BYTES
    ref, got = _grads_both_ways(big)
    for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
        err = float((a.float() - b.float()).abs().max() / a.float().abs().max())
        assert err <= 1e-2, f"{name}: {err}"


def test_noalloc_refuses_beyond_scratch():
    # needs 2 * 64 * 32800 * 4 bytes > 16 MiB of scratch: refused, nothing launched
    q = torch.zeros(1, 64, 32800, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 64, 8, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 64, 32800, dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 7.0)
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), q.data_ptr(), fa.FA_BF16,
                           lse.data_ptr(), q.data_ptr(), dq.data_ptr(), k.data_ptr(), k.data_ptr(),
                           1, 64, 32800, 8, 64, fa.FA_BF16, 0, 0.125,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 9 and fa.fa_status_str(st).startswith("problem needs more")
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all())


def test_noalloc_under_graph_capture():
    # The callers fa_bwd_noalloc is for: a forward (fa_fwd, no workspace) and
    # the no-alloc backward captured in one HIP graph, replayed three times
    # with eager work and synchronisations between the replays; every replay
    # must give the eager results bit for bit.
    w = workloads.custom(2, 4, 300, 300, 128, "bf16", True)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(w, seed=5))
    dt, mask, scale = fa.FA_BF16, fa._mask_code(w.causal), 1.0 / w.d ** 0.5
    o = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads, w.n_q, device="cuda")
    grads = tuple(torch.empty_like(t) for t in (q, k, v))

    def step(stream):
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dt, lse.data_ptr(),
                       w.batch, w.heads, w.n_q, w.n_k, w.d, dt, mask, scale, stream)
        assert st == 0
        st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dt, lse.data_ptr(),
                               do.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                               w.batch, w.heads, w.n_q, w.n_k, w.d, dt, mask, scale, stream)
        assert st == 0

    step(torch.cuda.current_stream().cuda_stream)      # eager (also looks the scratch up)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse) + grads]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse) + grads:
            t.fill_(float("nan"))                         # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "L", "dQ", "dK", "dV"), ref, (o, lse) + grads):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
