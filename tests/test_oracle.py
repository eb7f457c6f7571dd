"""Pins for the fp64 oracle, checked against facts other than the oracle itself.

Each pin names the passage or the mathematical fact it rests on. The pages
print no run outputs, so there are no printed worked-example values; the pins
are closed forms, invariants, finite differences, independent library
routines (scipy / torch CPU) and a negative control. The last group plants
mistakes in the oracle (on the CPU) and checks that some pin catches each.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as oracle_mod

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# online (m, l) == three-pass softmax / logsumexp
# (page 1 "05_flash_attention.py", section 1; page 3 "Flash Attention", 1.1,
#  including its induction argument that (m, l) is exact after every element)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 10, 33, 100])
@pytest.mark.parametrize("block", [1, 3, 4, 16, 1000])
def test_online_stats_match_logsumexp(n, block):
    x = rng(n * 31 + block).normal(size=n) * 5.0
    m, l = oracle.online_softmax_stats(x, block)
    assert m == x.max()
    assert abs((m + math.log(l)) - scipy.special.logsumexp(x)) <= 1e-12 * max(1.0, abs(m))
    np.testing.assert_allclose(np.exp(x - m) / l, scipy.special.softmax(x), rtol=1e-12, atol=1e-15)


def test_online_stats_with_neg_inf_entries():
    x = np.array([-np.inf, -np.inf, -np.inf, 2.0, -np.inf, 0.5, -1.0])
    for block in (1, 2, 3, 4):
        m, l = oracle.online_softmax_stats(x, block)
        assert m == 2.0
        assert abs(m + math.log(l) - scipy.special.logsumexp(x)) < 1e-14


def test_online_stats_page1_demo_input():
    # Page 1, section 1 demo: seed 0, x = randn(10) * 5, blocks of 3.
    torch.manual_seed(0)
    x = (torch.randn(10) * 5).double().numpy()
    m, l = oracle.online_softmax_stats(x, 3)
    ref = torch.logsumexp(torch.from_numpy(x), 0).item()
    assert abs(m + math.log(l) - ref) < 1e-12
    np.testing.assert_allclose(np.exp(x - m) / l, torch.softmax(torch.from_numpy(x), 0).numpy(),
                               rtol=1e-12)


def test_three_pass_softmax_matches_scipy():
    S = rng(1).normal(size=(9, 17)) * 10
    S[2, 3:] = -np.inf
    P, m, l = oracle.softmax_three_pass(S)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(m + np.log(l), scipy.special.logsumexp(S, axis=1), rtol=1e-14)


# --------------------------------------------------------------------------
# forward closed forms and invariants
# --------------------------------------------------------------------------

def _rand_head(n_q, n_k, d, seed=0, q_std=1.0):
    r = rng(seed)
    return (r.normal(size=(n_q, d)) * q_std, r.normal(size=(n_k, d)),
            r.normal(size=(n_k, d)), r.normal(size=(n_q, d)))


@pytest.mark.parametrize("n_q,n_k", [(37, 37), (50, 130), (130, 50), (1, 9), (9, 1)])
@pytest.mark.parametrize("chunk", [5, 256])
def test_zero_query_gives_row_means(n_q, n_k, chunk):
    # Q = 0 makes every visible score 0: O_i is the mean of the visible V
    # rows and L_i = ln(#visible). Non-causal: all n_k keys. Top-left causal
    # (page 1, section 2, standard_attention: triu(1) masked): keys 0..i.
    d = 6
    _, K, V, _ = _rand_head(n_q, n_k, d, seed=n_q + n_k)
    Q = np.zeros((n_q, d))
    r = oracle.attention_head(Q, K, V, causal=False, row_chunk=chunk)
    np.testing.assert_allclose(r["O"], np.broadcast_to(V.mean(0), (n_q, d)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["L"], np.full(n_q, math.log(n_k)), rtol=0, atol=1e-13)
    r = oracle.attention_head(Q, K, V, causal=True, row_chunk=chunk)
    cnt = np.minimum(np.arange(n_q), n_k - 1) + 1
    means = np.cumsum(V, axis=0)[cnt - 1] / cnt[:, None]
    np.testing.assert_allclose(r["O"], means, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["L"], np.log(cnt), rtol=0, atol=1e-13)


def test_first_causal_row_sees_only_key0():
    # Page 1, section 2 (boundary note): under the causal mask query 0 sees
    # key 0 only, so O_0 = V_0 and L_0 = scale * q_0 . k_0.
    Q, K, V, _ = _rand_head(20, 20, 8, seed=3)
    scale = 1 / math.sqrt(8)
    r = oracle.attention_head(Q, K, V, causal=True)
    np.testing.assert_allclose(r["O"][0], V[0], rtol=0, atol=1e-15)
    assert abs(r["L"][0] - scale * Q[0] @ K[0]) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # Softmax is invariant to a per-row shift (page 2, safe softmax; page 3,
    # 1.1). K -> K + 1 c^T adds scale * q_i . c to row i: O unchanged,
    # L_i -> L_i + scale * q_i . c.
    Q, K, V, _ = _rand_head(23, 31, 8, seed=4)
    c = rng(5).normal(size=8)
    scale = 0.3
    a = oracle.attention_head(Q, K, V, causal=causal, scale=scale)
    b = oracle.attention_head(Q, K + c, V, causal=causal, scale=scale)
    np.testing.assert_allclose(b["O"], a["O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["L"], a["L"] + scale * Q @ c, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(causal):
    Q, K, _, _ = _rand_head(19, 25, 8, seed=6, q_std=4.0)
    V = np.tile(np.arange(8.0) - 3.0, (25, 1))
    r = oracle.attention_head(Q, K, V, causal=causal)
    np.testing.assert_allclose(r["O"], V[: 19], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_torch_sdpa_page1_demo(causal):
    # Page 1, section 2, demo_forward: seed 0, n = 100, d = 32, float64,
    # Q, K, V = randn in order; torch's own sdpa is an independent routine.
    torch.manual_seed(0)
    Q, K, V = (torch.randn(100, 32, dtype=torch.float64) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None],
                                                           is_causal=causal)[0]
    r = oracle.attention_head(Q.numpy(), K.numpy(), V.numpy(), causal=causal)
    np.testing.assert_allclose(r["O"], ref.numpy(), rtol=0, atol=1e-13)
    s = (Q @ K.T) / math.sqrt(32)
    if causal:
        s = s.masked_fill(torch.ones(100, 100, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(r["L"], torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-13)


def _torch_grads(Q, K, V, dO, causal, scale):
    """Autograd of the materialising formula in torch fp64 (independent of
    the oracle's hand-written backward)."""
    Qt, Kt, Vt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V))
    s = (Qt @ Kt.T) * scale
    if causal:
        n, m = s.shape
        s = s.masked_fill(torch.ones(n, m, dtype=torch.bool).triu(1), float("-inf"))
    O = torch.softmax(s, -1) @ Vt
    O.backward(torch.tensor(dO))
    return O.detach().numpy(), Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_page1_demo(causal):
    # Page 1, section 3, demo_backward: seed 0, n = 70, d = 16, float64,
    # loss = sum(O^2), so dO = 2 O.
    torch.manual_seed(0)
    Q, K, V = (torch.randn(70, 16, dtype=torch.float64).numpy() for _ in range(3))
    scale = 1 / math.sqrt(16)
    O = oracle.attention_head(Q, K, V, causal=causal)["O"]
    dO = 2 * O
    r = oracle.attention_head(Q, K, V, dO, causal=causal)
    _, gq, gk, gv = _torch_grads(Q, K, V, dO, causal, scale)
    for name, ref in (("dQ", gq), ("dK", gk), ("dV", gv)):
        np.testing.assert_allclose(r[name], ref, rtol=0, atol=1e-12 * max(1, np.abs(ref).max()))


# --------------------------------------------------------------------------
# backward: finite differences and invariants
# --------------------------------------------------------------------------

def _fd_grads(Q, K, V, dO, causal, scale, h=1e-6):
    def loss(Q_, K_, V_):
        return float((oracle.attention_head(Q_, K_, V_, causal=causal, scale=scale)["O"] * dO).sum())
    grads = []
    for which in range(3):
        args = [Q.copy(), K.copy(), V.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[which][idx] += h
            m[which][idx] -= h
            g[idx] = (loss(*p) - loss(*m)) / (2 * h)
        grads.append(g)
    return grads


def _fd_check(fn, n_q, n_k, d, causal, seed):
    Q, K, V, dO = _rand_head(n_q, n_k, d, seed=seed)
    scale = 1 / math.sqrt(d)
    r = fn(Q, K, V, dO, causal=causal, scale=scale)
    fq, fk, fv = _fd_grads(Q, K, V, dO, causal, scale)
    errs = []
    for got, ref in ((r["dQ"], fq), (r["dK"], fk), (r["dV"], fv)):
        errs.append(np.abs(got - ref).max() / max(1e-300, np.abs(ref).max()))
    return max(errs)


FD_SHAPES = [(8, 8, 4), (5, 8, 3), (8, 5, 4), (1, 6, 2), (6, 1, 2), (7, 7, 1)]


@pytest.mark.parametrize("n_q,n_k,d", FD_SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(n_q, n_k, d, causal):
    # The backward formulas (page 3, section 1.5) against central finite
    # differences of the loss <dO, O> on n <= 8, h = 1e-6.
    err = _fd_check(oracle.attention_head, n_q, n_k, d, causal, seed=n_q * 10 + n_k + d)
    assert err < 1e-7, err


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    Q, K, V, dO = _rand_head(40, 57, 8, seed=11)
    r = oracle.attention_head(Q, K, V, dO, causal=causal)
    # Rows of dS sum to zero, so the dK rows sum to zero.
    np.testing.assert_allclose(r["dK"].sum(0), 0, atol=1e-12)
    # Rows of P sum to one, so the dV rows sum to the dO rows.
    np.testing.assert_allclose(r["dV"].sum(0), dO.sum(0), atol=1e-12)
    # The loss depends on Q K^T only: scaling Q up and K down leaves it
    # unchanged, hence <dQ, Q> = <dK, K>.
    assert abs((r["dQ"] * Q).sum() - (r["dK"] * K).sum()) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_row_term_identity(causal):
    # Page 3, 1.5 defines D = rowsum(P * dP); page 1, section 3 computes it as
    # rowsum(dO * O). Same thing, because dP = dO V^T and O = P V.
    Q, K, V, dO = _rand_head(33, 45, 8, seed=12)
    scale = 1 / math.sqrt(8)
    S = scale * Q @ K.T
    if causal:
        S[np.triu(np.ones_like(S, dtype=bool), 1)] = -np.inf
    P = scipy.special.softmax(S, axis=1)
    O = oracle.attention_head(Q, K, V, causal=causal)["O"]
    np.testing.assert_allclose((P * (dO @ V.T)).sum(1), (dO * O).sum(1), atol=1e-13)


# --------------------------------------------------------------------------
# chunking / sampling consistency (the oracle's own bookkeeping)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_chunking_and_sampling_are_exact(causal):
    Q, K, V, dO = _rand_head(70, 90, 8, seed=13)
    full = oracle.attention_head(Q, K, V, dO, causal=causal, row_chunk=1000)
    for chunk in (1, 7, 64):
        r = oracle.attention_head(Q, K, V, dO, causal=causal, row_chunk=chunk)
        for key in full:
            np.testing.assert_allclose(r[key], full[key], rtol=0, atol=1e-13)
    rows = np.array([0, 5, 69, 33])
    cols = np.array([89, 0, 40])
    s = oracle.attention_head(Q, K, V, dO, causal=causal, rows=rows, cols=cols, row_chunk=16)
    for key, idx in (("O", rows), ("L", rows), ("dQ", rows), ("dK", cols), ("dV", cols)):
        np.testing.assert_allclose(s[key], full[key][idx], rtol=0, atol=1e-13)
    f = oracle.attention_head(Q, K, V, causal=causal, rows=rows)
    np.testing.assert_allclose(f["O"], full["O"][rows], rtol=0, atol=1e-13)
    # no key columns requested: only the requested rows are visited
    q = oracle.attention_head(Q, K, V, dO, causal=causal, rows=rows, cols=np.array([], dtype=np.int64),
                              row_chunk=3)
    for key in ("O", "L", "dQ"):
        np.testing.assert_allclose(q[key], full[key][rows], rtol=0, atol=1e-13)
    assert q["dK"].shape == (0, 8) and q["dV"].shape == (0, 8)


@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
def test_partial_row_sets_add_up(causal):
    # A partition of the query rows into visited sets: O, L, dQ of each set
    # are the full result's rows, and the partial dK, dV sum to the full ones
    # (both are sums over query rows). Parallel timing of the oracle relies
    # on this.
    Q, K, V, dO = _rand_head(75, 60, 8, seed=21)
    full = oracle.attention_head(Q, K, V, dO, causal=causal)
    dK = np.zeros_like(full["dK"])
    dV = np.zeros_like(full["dV"])
    for part in (np.arange(0, 30), np.arange(30, 31), np.arange(31, 75)):
        r = oracle.attention_head(Q, K, V, dO, causal=causal, rows=part, visit=part, row_chunk=16)
        for key in ("O", "L", "dQ"):
            np.testing.assert_allclose(r[key], full[key][part], rtol=0, atol=1e-13)
        dK += r["dK"]
        dV += r["dV"]
    np.testing.assert_allclose(dK, full["dK"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, full["dV"], rtol=0, atol=1e-12)
    # a proper subset alone is not the full gradient
    r = oracle.attention_head(Q, K, V, dO, causal=causal, rows=np.arange(30), visit=np.arange(30))
    assert np.abs(r["dV"] - full["dV"]).max() > 1e-3


def test_batched_wrappers_match_heads():
    r = rng(14)
    Q, K, V, dO = (r.normal(size=(2, 3, 20, 8)) for _ in range(4))
    out = oracle.attention_backward(Q, K, V, dO, causal=True)
    h = oracle.attention_head(Q[1, 2], K[1, 2], V[1, 2], dO[1, 2], causal=True)
    for key in h:
        np.testing.assert_allclose(out[key][1, 2], h[key], rtol=0, atol=0)
    O, L = oracle.attention_forward(Q, K, V, causal=True)
    np.testing.assert_allclose(O, out["O"], rtol=0, atol=0)


# --------------------------------------------------------------------------
# negative control: page 2's block-diagonal sketch is not exact attention
# --------------------------------------------------------------------------

def _block_diagonal(Q, K, V, block):
    # Page 2 (代码实现): query block i attends to key block i only.
    O = np.zeros_like(Q)
    for s in range(0, Q.shape[0], block):
        e = min(s + block, Q.shape[0])
        S = Q[s:e] @ K[s:e].T / math.sqrt(Q.shape[1])
        O[s:e] = scipy.special.softmax(S, axis=1) @ V[s:e]
    return O


def test_block_diagonal_sketch_differs_from_exact():
    Q, K, V, _ = _rand_head(10, 10, 4, seed=15)
    exact = oracle.attention_head(Q, K, V)["O"]
    np.testing.assert_allclose(_block_diagonal(Q, K, V, 16), exact, atol=1e-13)
    assert np.abs(_block_diagonal(Q, K, V, 4) - exact).max() > 1e-2


# --------------------------------------------------------------------------
# bottom-right aligned causal mask (a variant the pages leave open: key j is
# visible to query i iff j <= i + n_k - n_q; rows that see no key give
# O = 0, L = -inf, dQ = 0 and add nothing to dK, dV)
# --------------------------------------------------------------------------

def _visible_counts(n_q, n_k, off):
    return np.clip(np.arange(n_q) + off + 1, 0, n_k)


BR_SHAPES = [(37, 37), (50, 130), (130, 50), (1, 9), (9, 1), (12, 9)]


@pytest.mark.parametrize("n_q,n_k", BR_SHAPES)
def test_causal_offsets(n_q, n_k):
    assert oracle.causal_offset(False, n_q, n_k) is None
    assert oracle.causal_offset(0, n_q, n_k) is None
    assert oracle.causal_offset(True, n_q, n_k) == 0
    assert oracle.causal_offset("top_left", n_q, n_k) == 0
    assert oracle.causal_offset("bottom_right", n_q, n_k) == n_k - n_q
    assert oracle.causal_offset(2, n_q, n_k) == n_k - n_q
    with pytest.raises(ValueError):
        oracle.causal_offset("diagonal", n_q, n_k)


@pytest.mark.parametrize("n_q,n_k", BR_SHAPES)
@pytest.mark.parametrize("chunk", [5, 256])
def test_bottom_right_zero_query_gives_suffix_means(n_q, n_k, chunk):
    # Q = 0: O_i is the mean of the first c_i = clip(i + n_k - n_q + 1, 0, n_k)
    # V rows and L_i = ln c_i; a row with c_i = 0 gives O = 0, L = -inf.
    d = 5
    _, K, V, _ = _rand_head(n_q, n_k, d, seed=n_q * 3 + n_k)
    r = oracle.attention_head(np.zeros((n_q, d)), K, V, causal="bottom_right", row_chunk=chunk)
    cnt = _visible_counts(n_q, n_k, n_k - n_q)
    live = cnt > 0
    means = np.zeros((n_q, d))
    means[live] = np.cumsum(V, axis=0)[cnt[live] - 1] / cnt[live, None]
    np.testing.assert_allclose(r["O"], means, rtol=0, atol=1e-13)
    assert np.all(np.isneginf(r["L"][~live]))
    np.testing.assert_allclose(r["L"][live], np.log(cnt[live]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_q,n_k", [(1, 9), (5, 40), (33, 70), (70, 70)])
def test_bottom_right_is_the_tail_of_a_square_causal_problem(n_q, n_k):
    # n_q <= n_k: the queries are the last n_q of an n_k-long sequence, so the
    # result equals the last n_q rows of the square top-left causal problem
    # (itself pinned to torch's sdpa above); with dO zero on the earlier rows
    # the square problem's dK, dV are the bottom-right ones.
    d = 6
    Qf, K, V, dOf = _rand_head(n_k, n_k, d, seed=n_q + 2 * n_k)
    dOf[: n_k - n_q] = 0.0
    sq = oracle.attention_head(Qf, K, V, dOf, causal=True)
    br = oracle.attention_head(Qf[n_k - n_q:], K, V, dOf[n_k - n_q:], causal="bottom_right")
    tail = slice(n_k - n_q, None)
    for key, want in (("O", sq["O"][tail]), ("L", sq["L"][tail]), ("dQ", sq["dQ"][tail]),
                      ("dK", sq["dK"]), ("dV", sq["dV"])):
        np.testing.assert_allclose(br[key], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_q,n_k", [(5, 40), (33, 70), (16, 16), (1, 7)])
def test_bottom_right_matches_torch_lower_right_bias(n_q, n_k):
    # torch's causal_lower_right bias is an independent implementation of the
    # same alignment (defined there for n_q <= n_k, where no row is empty).
    from torch.nn.attention.bias import causal_lower_right
    Q, K, V, dO = (torch.from_numpy(a) for a in _rand_head(n_q, n_k, 8, seed=n_q + n_k))
    Qt, Kt, Vt = (a.clone().requires_grad_(True) for a in (Q, K, V))
    bias = causal_lower_right(n_q, n_k)
    ref = torch.nn.functional.scaled_dot_product_attention(Qt[None], Kt[None], Vt[None],
                                                           attn_mask=bias)[0]
    ref.backward(dO)
    r = oracle.attention_head(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal="bottom_right")
    np.testing.assert_allclose(r["O"], ref.detach().numpy(), rtol=0, atol=1e-13)
    for name, t in (("dQ", Qt), ("dK", Kt), ("dV", Vt)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_q,n_k,d", [(8, 5, 4), (6, 1, 2), (5, 8, 3), (8, 8, 4)])
def test_bottom_right_finite_differences(n_q, n_k, d):
    err = _fd_check(oracle.attention_head, n_q, n_k, d, "bottom_right", seed=n_q * 13 + n_k + d)
    assert err < 1e-7, err


def test_bottom_right_dead_rows():
    # n_q > n_k: rows 0 .. n_q - n_k - 1 see no key. They give O = 0,
    # L = -inf, dQ = 0, and the live rows are those of the problem without
    # them (the dead rows add nothing to dK, dV).
    n_q, n_k, d = 11, 4, 3
    Q, K, V, dO = _rand_head(n_q, n_k, d, seed=31)
    r = oracle.attention_head(Q, K, V, dO, causal="bottom_right")
    dead = n_q - n_k
    assert np.all(r["O"][:dead] == 0) and np.all(np.isneginf(r["L"][:dead]))
    assert np.all(r["dQ"][:dead] == 0)
    live = oracle.attention_head(Q[dead:], K, V, dO[dead:], causal="bottom_right")
    for key in ("O", "L", "dQ"):
        np.testing.assert_allclose(r[key][dead:], live[key], rtol=0, atol=1e-13)
    for key in ("dK", "dV"):
        np.testing.assert_allclose(r[key], live[key], rtol=0, atol=1e-13)


def _bottom_right_pins_pass(fn):
    """Compact bottom-right pins against an attention_head-like fn."""
    ok = True
    d = 4
    for n_q, n_k in ((12, 9), (9, 12)):
        _, K, V, _ = _rand_head(n_q, n_k, d, seed=41 + n_q)
        r = fn(np.zeros((n_q, d)), K, V, causal="bottom_right", row_chunk=5)
        cnt = _visible_counts(n_q, n_k, n_k - n_q)
        live = cnt > 0
        means = np.zeros((n_q, d))
        means[live] = np.cumsum(V, 0)[cnt[live] - 1] / cnt[live, None]
        with np.errstate(divide="ignore"):
            want_l = np.where(live, np.log(np.maximum(cnt, 1)), -np.inf)
        ok &= np.allclose(r["O"], means, atol=1e-12)
        ok &= bool(np.array_equal(np.isneginf(r["L"]), ~live))
        ok &= np.allclose(r["L"][live], want_l[live], atol=1e-12)
    # tail of the square top-left problem (forward and backward)
    Qf, K, V, dOf = _rand_head(10, 10, 3, seed=43)
    dOf[:4] = 0.0
    sq = oracle.attention_head(Qf, K, V, dOf, causal=True)
    br = fn(Qf[4:], K, V, dOf[4:], causal="bottom_right")
    for key, want in (("O", sq["O"][4:]), ("dQ", sq["dQ"][4:]), ("dK", sq["dK"]), ("dV", sq["dV"])):
        ok &= np.allclose(br[key], want, atol=1e-10)
    # torch's lower-right causal bias (independent), n_q < n_k
    from torch.nn.attention.bias import causal_lower_right
    Q, K, V, dO = (torch.from_numpy(a) for a in _rand_head(6, 11, 4, seed=45))
    Qt, Kt, Vt = (a.clone().requires_grad_(True) for a in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Qt[None], Kt[None], Vt[None], attn_mask=causal_lower_right(6, 11))[0]
    ref.backward(dO)
    r = fn(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal="bottom_right")
    for got, want in ((r["O"], ref.detach()), (r["dQ"], Qt.grad), (r["dK"], Kt.grad), (r["dV"], Vt.grad)):
        ok &= np.allclose(got, want.numpy(), atol=1e-10)
    # dead rows in the backward: zero dQ, finite everything
    Q, K, V, dO = _rand_head(7, 3, 3, seed=44)
    r = fn(Q, K, V, dO, causal="bottom_right")
    ok &= bool(np.all(np.isfinite(r["dK"])) and np.all(np.isfinite(r["dV"])))
    ok &= bool(np.all(r["dQ"][:4] == 0) and np.all(r["O"][:4] == 0))
    return bool(ok)


def test_bottom_right_pins_pass_on_the_oracle():
    assert _bottom_right_pins_pass(oracle.attention_head)


# --------------------------------------------------------------------------
# planted mistakes: each one must trip at least one pin above
# --------------------------------------------------------------------------

def _pins_pass(fn):
    """Run a compact version of the pins against an attention_head-like fn."""
    ok = True
    # closed forms (causal, chunked so the causal offset matters)
    d = 4
    _, K, V, _ = _rand_head(12, 9, d, seed=21)
    r = fn(np.zeros((12, d)), K, V, causal=True, row_chunk=5)
    cnt = np.minimum(np.arange(12), 8) + 1
    ok &= np.allclose(r["O"], np.cumsum(V, 0)[cnt - 1] / cnt[:, None], atol=1e-12)
    ok &= np.allclose(r["L"], np.log(cnt), atol=1e-12)
    # first causal row
    Q, K, V, dO = _rand_head(6, 7, 3, seed=22)
    r = fn(Q, K, V, causal=True)
    ok &= np.allclose(r["L"][0], Q[0] @ K[0] / math.sqrt(3), atol=1e-12)
    # torch autograd of the materialising formula, both masks, n_q != n_k
    for causal in (False, True):
        r = fn(Q, K, V, dO, causal=causal, scale=1 / math.sqrt(3))
        o, gq, gk, gv = _torch_grads(Q, K, V, dO, causal, 1 / math.sqrt(3))
        for got, ref in ((r["O"], o), (r["dQ"], gq), (r["dK"], gk), (r["dV"], gv)):
            ok &= np.allclose(got, ref, atol=1e-10)
    return bool(ok)


def test_pins_pass_on_the_oracle():
    assert _pins_pass(oracle.attention_head)


def _mutant_scores(kind):
    orig = oracle_mod._scores

    def scores(Qr, K, row_ids, off, scale):
        if kind == "mask_local_rows":      # causal mask indexed by chunk-local row
            return orig(Qr, K, np.arange(len(row_ids)), off, scale)
        if kind == "mask_diagonal":        # hides the diagonal too (j >= i + off)
            S = orig(Qr, K, row_ids, off, scale)
            if off is not None:
                S[np.arange(K.shape[0])[None, :] == row_ids[:, None] + off] = -np.inf
            return S
        if kind == "no_scale":
            return orig(Qr, K, row_ids, off, 1.0)
        if kind == "offset_ignored":       # bottom-right treated as top-left
            return orig(Qr, K, row_ids, None if off is None else 0, scale)
        if kind == "offset_sign":          # diagonal shifted the wrong way
            return orig(Qr, K, row_ids, None if off is None else -off, scale)
        if kind == "offset_plus_one":      # one key too many (j <= i + off + 1)
            return orig(Qr, K, row_ids, None if off is None else off + 1, scale)
        raise ValueError(kind)
    return scores


@pytest.mark.parametrize("kind", ["mask_local_rows", "mask_diagonal", "no_scale"])
def test_planted_score_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle_mod, "_scores", _mutant_scores(kind))
    assert not _pins_pass(oracle_mod.attention_head)


@pytest.mark.parametrize("kind", ["mask_local_rows", "mask_diagonal", "no_scale",
                                  "offset_ignored", "offset_sign", "offset_plus_one"])
def test_planted_bottom_right_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle_mod, "_scores", _mutant_scores(kind))
    assert not _bottom_right_pins_pass(oracle_mod.attention_head)


def test_planted_dead_row_mistakes_are_caught(monkeypatch):
    # A row with no visible key must come out as O = 0, L = -inf, dQ = 0;
    # plain three-pass softmax of such a row gives NaN instead.
    def naive(X, scale=1.0):
        P, m, l = oracle_mod.softmax_three_pass(np.asarray(X, dtype=np.float64) * scale)
        return P, m + np.log(l)
    monkeypatch.setattr(oracle_mod, "row_softmax", naive)
    assert not _bottom_right_pins_pass(oracle_mod.attention_head)


@pytest.mark.parametrize("kind", ["log2_L", "dQ_no_scale", "dK_no_scale", "D_dropped",
                                  "dV_unnormalised_P", "K_for_V"])
def test_planted_output_mistakes_are_caught(kind):
    def fn(Q, K, V, dO=None, causal=False, scale=None, row_chunk=256):
        if kind == "K_for_V":
            return oracle.attention_head(Q, K, K if K.shape == V.shape else V, dO, causal, scale,
                                         row_chunk=row_chunk)
        r = oracle.attention_head(Q, K, V, dO, causal, scale, row_chunk=row_chunk)
        sc = scale if scale is not None else 1 / math.sqrt(Q.shape[1])
        if kind == "log2_L":
            r["L"] = r["L"] / math.log(2)
        if dO is None:
            return r
        if kind == "dQ_no_scale":
            r["dQ"] = r["dQ"] / sc
        if kind == "dK_no_scale":
            r["dK"] = r["dK"] / sc
        if kind in ("D_dropped", "dV_unnormalised_P"):
            S = sc * Q @ K.T
            if causal:
                S[np.triu(np.ones_like(S, dtype=bool), 1)] = -np.inf
            P = scipy.special.softmax(S, axis=1)
            if kind == "D_dropped":
                dS = P * (dO @ V.T)
                r["dQ"] = sc * dS @ K
            else:                           # exp(S - m) without the 1/l
                E = np.exp(S - S.max(1, keepdims=True))
                r["dV"] = E.T @ dO
        return r
    assert not _pins_pass(fn)


# --------------------------------------------------------- row softmax / logsumexp
# oracle.row_softmax is the definition the standalone row kernel follows
# (page 1, section 1). Pins: SciPy's logsumexp / softmax, closed forms,
# masked entries, overflow-prone magnitudes and the one-pass statistics.

def _row_pins(fn):
    rng = np.random.default_rng(11)
    X = rng.standard_normal((37, 301)) * 3.0
    for scale in (1.0, 0.125, 2.5):
        P, L = fn(X, scale)
        assert np.allclose(L, scipy.special.logsumexp(X * scale, axis=1), rtol=0, atol=1e-12)
        assert np.allclose(P, scipy.special.softmax(X * scale, axis=1), rtol=0, atol=1e-14)
    # constant rows: P = 1/n, L = ln n + scale * c
    n = 64
    C = np.tile(np.arange(5, dtype=np.float64)[:, None], (1, n))
    P, L = fn(C, 0.5)
    assert np.allclose(P, 1.0 / n, atol=1e-15)
    assert np.allclose(L, math.log(n) + 0.5 * np.arange(5), atol=1e-12)
    # -inf entries drop out; an all -inf row gives P = 0, L = -inf
    Y = rng.standard_normal((3, 10))
    Y[0, ::2] = -np.inf
    Y[2, :] = -np.inf
    P, L = fn(Y, 1.0)
    assert np.allclose(P[0, 1::2], scipy.special.softmax(Y[0, 1::2]), atol=1e-14)
    assert (P[0, ::2] == 0).all()
    assert (P[2] == 0).all() and L[2] == -math.inf
    assert np.isclose(L[1], scipy.special.logsumexp(Y[1]), atol=1e-12)
    # magnitudes that overflow exp without the max shift
    Z = np.array([[1000.0, 999.0, 998.0], [-1000.0, -1001.0, -1002.0]])
    P, L = fn(Z, 1.0)
    ref = np.log(1 + math.exp(-1) + math.exp(-2))
    assert np.allclose(L, [1000 + ref, -1000 + ref], atol=1e-9)
    assert np.allclose(P[0], P[1], atol=1e-15)


def test_row_softmax_pins():
    _row_pins(oracle.row_softmax)


@pytest.mark.parametrize("block", [1, 7, 64, 301])
def test_row_softmax_matches_one_pass_stats(block):
    rng = np.random.default_rng(12)
    X = rng.standard_normal((5, 301)) * 4.0
    _, L = oracle.row_softmax(X, 0.25)
    for i in range(5):
        m, l = oracle.online_softmax_stats(X[i] * 0.25, block)
        assert abs(L[i] - (m + math.log(l))) < 1e-12


@pytest.mark.parametrize("kind", ["no_scale", "log2", "no_shift_sum", "unnormalised"])
def test_planted_row_softmax_mistakes_are_caught(kind):
    def mutant(X, scale=1.0):
        P, L = oracle.row_softmax(X, 1.0 if kind == "no_scale" else scale)
        if kind == "log2":
            L = L / math.log(2)
        if kind == "no_shift_sum":
            L = L + 1.0
        if kind == "unnormalised":
            P = P * 1.01
        return P, L
    with pytest.raises(AssertionError):
        _row_pins(mutant)
