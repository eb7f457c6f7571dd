"""Shared helpers of the GPU parity tests: run the HIP path through the
binding and compare with the fp64 oracle on the same seeded inputs.

Tolerances (max absolute error against the fp64 oracle):
  bf16 inputs: O (the kernel's unrounded fp32 output) <= 1e-2, L <= 1e-3,
               each gradient <= 2e-2 * max|reference gradient|; the bf16 O
               must equal the round-to-nearest-even rounding of the fp32 O.
  fp32 inputs: O, L <= 1e-5, each gradient <= 1e-5 * max|reference|.
When an exact gradient is identically zero (a single key: every softmax row
is the constant 1, so dQ = dK = 0), "max|reference|" is floored at 1e-3 of
the largest reference gradient of the three, so the bar stays relative to
the gradients' scale instead of collapsing to 0.
A query row that sees no key (bottom-right mask, n_q > n_k) must come out
exactly as the oracle defines it: O = 0, L = -inf, dQ = 0.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import exact_tiled_attention_29_amd as fa
import oracle

TOL = {
    "bf16": {"O": 1e-2, "L": 1e-3, "grad": 2e-2},
    "f32": {"O": 1e-5, "L": 1e-5, "grad": 1e-5},
}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def to_gpu(*ts):
    return [t.to("cuda").contiguous() for t in ts]


def run(q, k, v, do, causal, scale=None, backward=True):
    """Run the HIP forward (fp32 O and input-dtype O) and, optionally, the
    backward fed with the input-dtype O and L. Returns a dict of CPU float64
    numpy arrays plus the raw bf16 / fp32 outputs."""
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    o32, l32 = fa.forward(qg, kg, vg, causal, scale, o_dtype=torch.float32)
    o, l = fa.forward(qg, kg, vg, causal, scale)
    res = {"O32": o32.cpu(), "O": o.cpu(), "L": l.cpu(), "L32": l32.cpu()}
    # every head, also those the oracle does not see: O is finite (a row
    # that sees no key gives 0)
    assert torch.isfinite(res["O32"]).all() and torch.isfinite(res["O"]).all(), "non-finite O"
    if backward:
        dq, dk, dv = fa.backward(qg, kg, vg, o, l, dog, causal, scale)
        torch.cuda.synchronize()
        res.update(dQ=dq.cpu(), dK=dk.cpu(), dV=dv.cpu())
        assert all(torch.isfinite(res[n]).all() for n in ("dQ", "dK", "dV")), "non-finite gradient"
    del qg, kg, vg, dog
    return res


def oracle_heads(Q, K, V, dO, causal, heads, scale=None, rows=None, cols=None):
    """oracle.attention_head for several (b, h) heads at once, on a thread
    pool (numpy releases the GIL in its kernels; one BLAS thread per worker)
    over the heads and, when every key row is wanted, over chunks of query
    rows whose partial dK, dV are summed. Returns {(b, h): result}."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    n_q = Q.shape[2]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    chunk = 512
    split = dO is not None and (cols is None or len(cols)) and rows is None
    tasks = []
    for hd in heads:
        if split:
            for r0 in range(0, n_q, chunk):
                tasks.append((hd, np.arange(r0, min(n_q, r0 + chunk))))
        else:
            tasks.append((hd, None))

    def one(t):
        (b, h), part = t
        if part is None:
            return oracle.attention_head(Q[b, h], K[b, h], V[b, h], None if dO is None else dO[b, h],
                                         causal, scale, rows=rows, cols=cols)
        return oracle.attention_head(Q[b, h], K[b, h], V[b, h], dO[b, h], causal, scale, rows=part,
                                     cols=cols, visit=part)

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(one, tasks))
    out = {}
    for (hd, part), r in zip(tasks, parts):
        if part is None:
            out[hd] = r
            continue
        acc = out.setdefault(hd, {"O": [], "L": [], "dQ": [], "dK": 0.0, "dV": 0.0})
        for key in ("O", "L", "dQ"):
            acc[key].append(r[key])
        acc["dK"] = acc["dK"] + r["dK"]
        acc["dV"] = acc["dV"] + r["dV"]
    for hd, acc in out.items():
        if isinstance(acc["O"], list):
            for key in ("O", "L", "dQ"):
                acc[key] = np.concatenate(acc[key])
    return out


def rounding_floor(res, refs, heads, rows=None):
    """max|O_bf16 - O_ref| of the kernel's bf16 O beside max|RNE(O_ref) -
    O_ref|, the error that rounding the exact result to bf16 leaves by
    itself, over the given heads."""
    got = f64(res["O"])
    e_bf16 = floor = 0.0
    for b, h in heads:
        ref = refs[(b, h)]["O"]
        g = got[b, h] if rows is None else got[b, h][rows]
        rne = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        e_bf16 = max(e_bf16, float(np.abs(g - ref).max()))
        floor = max(floor, float(np.abs(rne - ref).max()))
    return {"max_err_bf16_O": e_bf16, "max_err_RNE_of_exact_O": floor}


def report(tag, values):
    """Print a parity figure and append it to $PARITY_REPORT (JSON lines)."""
    import json
    line = {"case": tag, **{k: (float(v) if isinstance(v, (float, np.floating)) else v)
                            for k, v in values.items()}}
    print("[parity]", json.dumps(line))
    path = os.environ.get("PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(line) + "\n")


def check_heads(res, q, k, v, do, causal, dtype, heads, scale=None, grads=True, rows=None,
                cols=None, tag="", refs=None):
    """Compare the given (b, h) heads of a run with the oracle. rows / cols
    optionally restrict the compared query rows (O, L, dQ) and key rows
    (dK, dV). refs: oracle results by head, computed here when not given.
    Returns a dict of the worst errors."""
    tol = TOL[dtype]
    worst = {}
    Q, K, V, dO = f64(q), f64(k), f64(v), f64(do)
    if refs is None:
        refs = oracle_heads(Q, K, V, dO if grads else None, causal, heads, scale, rows, cols)
    for b, h in heads:
        ref = refs[(b, h)]
        ridx = slice(None) if rows is None else rows
        cidx = slice(None) if cols is None else cols
        o_key = "O32" if dtype == "bf16" else "O"
        got_o = f64(res[o_key][b, h])[ridx]
        got_l = f64(res["L"][b, h])[ridx]
        dead = np.isneginf(ref["L"])
        if dead.any():
            assert np.all(np.isneginf(got_l[dead])), f"{tag} head {(b, h)}: L of an empty row != -inf"
            assert np.all(got_o[dead] == 0), f"{tag} head {(b, h)}: O of an empty row != 0"
            if grads:
                assert np.all(f64(res["dQ"][b, h])[ridx][dead] == 0), \
                    f"{tag} head {(b, h)}: dQ of an empty row != 0"
        e_o = np.abs(got_o - ref["O"]).max()
        e_l = np.abs(got_l[~dead] - ref["L"][~dead]).max() if (~dead).any() else 0.0
        worst["O"] = max(worst.get("O", 0.0), e_o)
        worst["L"] = max(worst.get("L", 0.0), e_l)
        assert e_o <= tol["O"], f"{tag} head {(b, h)}: max|dO| {e_o:.3e} > {tol['O']}"
        assert e_l <= tol["L"], f"{tag} head {(b, h)}: max|dL| {e_l:.3e} > {tol['L']}"
        if grads:
            gmax = max(np.abs(ref[n]).max() for n in ("dQ", "dK", "dV") if ref[n].size)
            for name, idx in (("dQ", ridx), ("dK", cidx), ("dV", cidx)):
                want = ref[name]
                if want.size == 0:          # no rows / columns requested
                    continue
                got = f64(res[name][b, h])[idx]
                scale_ = max(np.abs(want).max(), 1e-3 * gmax, 1e-30)
                err = np.abs(got - want).max() / scale_
                worst[name] = max(worst.get(name, 0.0), err)
                assert err <= tol["grad"], \
                    f"{tag} head {(b, h)}: {name} rel err {err:.3e} > {tol['grad']}"
    if dtype == "bf16":
        # the bf16 O is the RNE rounding of the fp32 O, bit for bit
        assert torch.equal(res["O"], res["O32"].to(torch.bfloat16)), f"{tag}: bf16 O != RNE(fp32 O)"
        assert torch.equal(res["L"], res["L32"]), f"{tag}: L depends on o_dtype"
    return worst


def check_sum_invariants(res, do, dtype, tag=""):
    """Properties that hold at any size, for every head: the dK rows sum to
    zero and the dV rows sum to the dO rows (a softmax row sums to one)."""
    dK, dV = f64(res["dK"]), f64(res["dV"])
    dO = f64(do)
    tol = 5e-2 if dtype == "bf16" else 1e-5
    sum_dk = np.abs(dK.sum(axis=2))                       # [B, H, d]
    mag_dk = np.abs(dK).sum(axis=2) + 1e-30
    assert (sum_dk / mag_dk).max() < tol, f"{tag}: sum_j dK_j not ~0"
    err_dv = np.abs(dV.sum(axis=2) - dO.sum(axis=2))
    mag_dv = np.abs(dV).sum(axis=2) + 1e-30
    assert (err_dv / mag_dv).max() < tol, f"{tag}: sum_j dV_j != sum_i dO_i"
    for name in ("O", "L", "dQ", "dK", "dV"):
        if name in res:
            assert torch.isfinite(res[name].float()).all(), f"{tag}: non-finite {name}"
