"""fp64 CPU oracle for exact scaled-dot-product attention (test infrastructure).

Only the test suite, the smoke check and the CPU-baseline leg of the bench may
import this module. The product path (the HIP library and its Python binding)
never does, and this module imports nothing from it.

What is computed, and where the pages define it:

* Attention is softmax(Q K^T / sqrt(d)) V, the formula on page 2 ("FlashAttention：
  深度学习中的高效注意力机制", section 公式推导 / 传统注意力机制). The scale is an
  argument; every workload uses 1/sqrt(d).
* The causal mask is top-left aligned: key j is visible to query i iff j <= i,
  also when n_q != n_k (page 1, "05_flash_attention.py", section 2,
  standard_attention masks triu(1) of the n x m score matrix).
* The bottom-right aligned causal mask is a variant the pages do not define:
  key j is visible to query i iff j <= i + (n_k - n_q), i.e. the last query
  sees every key, as when the queries are the newest n_q positions of an
  n_k-long sequence. For n_q == n_k it is the top-left mask. When n_q > n_k
  the first n_q - n_k queries see no key; a softmax over no entries is
  undefined, and here such a row gets O = 0, L = -inf and adds nothing to
  any gradient (its dQ is 0), the same convention as row_softmax.
* Softmax is the three-pass safe softmax: row max, exponentials of the
  shifted scores and their sum, then normalisation (page 2, section
  块内归一化; page 3, "Flash Attention", section 1.1).
* L is the natural-log logsumexp of each masked, scaled score row, L = m +
  ln(l) (page 1, section 1, compared there against torch.logsumexp).
* The backward follows the matrix-calculus rules of page 3, section 1.5:
  for O = P V, dP = dO V^T and dV = P^T dO; for P = softmax(S),
  dS = P * (dP - rowsum(P * dP)). With S = scale * Q K^T,
  dQ = scale * dS K and dK = scale * dS^T Q (page 1, section 3 docstring).
  The row term D is taken in its defining form rowsum(P * dP), not in the
  rowsum(dO * O) form the tiled method uses; their equality is a test.

Nothing here is tiled, fused or reordered beyond the definition: for each
head the full score rows are materialised, in chunks of query rows taken at
full key width (a softmax row never spans two chunks; dK and dV are sums over
rows, so chunking them is exact).

Also here: the one-pass running (m, l) statistics of page 1, section 1
(online_softmax_stats) and page 3, section 1.1, and the row softmax /
logsumexp of a plain matrix (row_softmax) that the standalone row kernel
computes.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "online_softmax_stats",
    "softmax_three_pass",
    "row_softmax",
    "causal_offset",
    "attention_head",
    "attention_forward",
    "attention_backward",
]

ROW_CHUNK = 256


def online_softmax_stats(x, block):
    """One pass over x in blocks, keeping the running max m and the sum l of
    exp(x - m) rebased to the current max (page 1, section 1; page 3, section
    1.1). Returns (m, l); softmax(x) = exp(x - m) / l and logsumexp = m + ln l.

    A block whose entries are all -inf (and every block before it) leaves
    (m, l) = (-inf, 0), so (-inf) - (-inf) is never formed.
    """
    x = np.asarray(x, dtype=np.float64)
    m = -math.inf
    l = 0.0
    for s in range(0, len(x), block):
        chunk = x[s:s + block]
        m_new = max(m, float(chunk.max()))
        if m_new == -math.inf:
            continue
        l = l * math.exp(m - m_new) + float(np.exp(chunk - m_new).sum())
        m = m_new
    return m, l


def softmax_three_pass(S):
    """Row-wise safe softmax of a 2-D array: max, exp-sum, normalise.
    Returns (P, m, l) with l the row sum of exp(S - m)."""
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    return E / l[:, None], m, l


def row_softmax(X, scale=1.0):
    """Softmax and natural-log logsumexp of each row of scale * X (page 1,
    section 1: the softmax of a score row and its logsumexp, compared there
    against torch.softmax / torch.logsumexp), by the three-pass definition.

    A row whose entries are all -inf has no defined softmax; here it gets
    P = 0 and L = -inf (the pages leave it open; the row kernel does the
    same). Returns (P, L) as float64 arrays.
    """
    S = np.asarray(X, dtype=np.float64) * float(scale)
    if S.ndim != 2 or S.shape[1] == 0:
        raise ValueError("X must be 2-D with at least one column")
    P = np.zeros_like(S)
    L = np.full(S.shape[0], -math.inf)
    live = np.isfinite(S.max(axis=1)) if S.shape[0] else np.zeros(0, bool)
    if live.any():
        Pl, m, l = softmax_three_pass(S[live])
        P[live] = Pl
        L[live] = m + np.log(l)
    return P, L


def causal_offset(causal, n_q, n_k):
    """Diagonal offset of the causal mask: key j is visible to query i iff
    j <= i + offset. None for no mask; 0 for the top-left mask (causal True,
    1 or "top_left"); n_k - n_q for the bottom-right mask (2 or
    "bottom_right")."""
    if causal is False or causal is None or (not isinstance(causal, str) and causal == 0):
        return None
    if causal is True or causal == "top_left" or (not isinstance(causal, str) and causal == 1):
        return 0
    if causal == "bottom_right" or (not isinstance(causal, str) and causal == 2):
        return n_k - n_q
    raise ValueError(f"unknown causal mode {causal!r}")


def _scores(Qr, K, row_ids, off, scale):
    """S = scale * Qr K^T for the query rows row_ids (global indices), with
    keys j > i + off masked as -inf (off None: no mask)."""
    S = scale * (Qr @ K.T)
    if off is not None:
        key_ids = np.arange(K.shape[0])
        S[key_ids[None, :] > row_ids[:, None] + off] = -np.inf
    return S


def attention_head(Q, K, V, dO=None, causal=False, scale=None, rows=None, cols=None,
                   row_chunk=ROW_CHUNK, visit=None):
    """Exact attention for one head, in float64.

    Q: (n_q, d); K, V: (n_k, d); dO: (n_q, d) or None for forward only.
    causal: False (no mask), True / "top_left", or "bottom_right" (see
    causal_offset).
    rows: query indices whose O, L (and dQ) are returned (default: all).
    cols: key indices whose dK, dV are returned (default: all).

    Returns a dict with "O" (len(rows), d), "L" (len(rows),) and, when dO is
    given, "dQ" (len(rows), d), "dK", "dV" (len(cols), d).

    With a subset of rows only those rows are computed when dO is None. The
    backward needs every query row for dK and dV, so with dO given all rows
    are visited and only the requested ones are kept, unless cols is empty:
    then only the requested rows are visited (their O, L and dQ need no
    other row).

    visit: optionally, exactly the query rows whose score rows are formed
    (global indices, containing rows). dK and dV are then the sums over
    these rows only; over any partition of the rows such partial sums add up
    to the full gradients (dK and dV are sums over query rows), which lets a
    caller spread one head over several workers.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_q, d = Q.shape
    n_k = K.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_k) if cols is None else np.asarray(cols, dtype=np.int64)
    visit_given = visit
    want_bwd = dO is not None
    if want_bwd:
        dO = np.asarray(dO, dtype=np.float64)

    out_pos = {int(r): i for i, r in enumerate(rows)}
    O = np.zeros((len(rows), d))
    L = np.zeros(len(rows))
    if want_bwd:
        dQ = np.zeros((len(rows), d))
        dK = np.zeros((len(cols), d))
        dV = np.zeros((len(cols), d))
        # every row contributes to dK, dV; only the requested ones to dQ
        visit = np.arange(n_q) if len(cols) else np.unique(rows)
    else:
        visit = np.unique(rows)
    if visit_given is not None:
        visit = np.unique(np.asarray(visit_given, dtype=np.int64))

    off = causal_offset(causal, n_q, n_k)
    for c0 in range(0, len(visit), row_chunk):
        ids = visit[c0:c0 + row_chunk]
        S = _scores(Q[ids], K, ids, off, scale)
        # rows that see no key (bottom-right mask, n_q > n_k): P = 0, L = -inf
        P, Lc = row_softmax(S)
        keep = np.array([int(r) in out_pos for r in ids])
        if keep.any():
            pos = np.array([out_pos[int(r)] for r in ids[keep]])
            O[pos] = P[keep] @ V
            L[pos] = Lc[keep]
        if want_bwd:
            dOc = dO[ids]
            dP = dOc @ V.T
            Drow = (P * dP).sum(axis=1)
            dS = P * (dP - Drow[:, None])
            if keep.any():
                dQ[pos] = scale * (dS[keep] @ K)
            dK += scale * (dS[:, cols].T @ Q[ids])
            dV += P[:, cols].T @ dOc
    res = {"O": O, "L": L}
    if want_bwd:
        res.update(dQ=dQ, dK=dK, dV=dV)
    return res


def _as_f64(t):
    """Accept numpy arrays or CPU torch tensors (any float dtype)."""
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def attention_forward(Q, K, V, causal=False, scale=None, heads=None):
    """Batched forward over [B, H, n, d] inputs. heads: optional list of
    (b, h) pairs to compute (others are left as NaN). Returns (O, L)."""
    Q, K, V = _as_f64(Q), _as_f64(K), _as_f64(V)
    B, H, n_q, d = Q.shape
    O = np.full((B, H, n_q, d), np.nan)
    L = np.full((B, H, n_q), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        r = attention_head(Q[b, h], K[b, h], V[b, h], None, causal, scale)
        O[b, h], L[b, h] = r["O"], r["L"]
    return O, L


def attention_backward(Q, K, V, dO, causal=False, scale=None, heads=None):
    """Batched forward + backward over [B, H, n, d] inputs. Returns a dict of
    O, L, dQ, dK, dV (heads not requested are NaN)."""
    Q, K, V, dO = _as_f64(Q), _as_f64(K), _as_f64(V), _as_f64(dO)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    out = {
        "O": np.full((B, H, n_q, d), np.nan), "L": np.full((B, H, n_q), np.nan),
        "dQ": np.full((B, H, n_q, d), np.nan), "dK": np.full((B, H, n_k, d), np.nan),
        "dV": np.full((B, H, n_k, d), np.nan),
    }
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        r = attention_head(Q[b, h], K[b, h], V[b, h], dO[b, h], causal, scale)
        for key in out:
            out[key][b, h] = r[key]
    return out
