"""The MoE layer, written out plainly: routing, schedule, gather, SwiGLU experts, combine, backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The grouped, fused GPU execution reaches exactly the plain MoE result, so the oracle is that plain
definition. The exceptions are the roundings the method itself performs: MX quantisation of the
expert GEMM operands (done here, step by step) and the bfloat16 storage of intermediates (covered by
the tolerance, not replayed).

Notation: T tokens, hidden h, expert width m, E experts (E_loc local), top-k k, R = T*k routed rows,
assignment a = t*k + j for token t and slot j.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, bf16_to_f64, mx_roundtrip

# ----------------------------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------------------------


def router_logits_fixed_order(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """Router logits l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e] in float32, in one written order.

    The pages name token routing as part of the fused layer ("Merged summary" of the MoK news
    digest; the Mixture-of-Kittens page's TL;DR) but print no formula; the workloads define the
    logits as x times the router matrix, plus a per-expert bias where they give one.

    Reading: routing must be reproducible bit for bit, so the sum has one fixed order, the plain
    left-to-right one: acc = +0.0; acc = acc + x[t, i] * W_r[e, i] for i = 0 .. h-1, in float32;
    then l = acc + b[e]. A product of two bfloat16 values is exact in float32, so each step rounds
    once, exactly as a fused multiply-add would.

    x: [T, h] bf16 bits; w_router: [E, h] bf16 bits (row e = expert e); bias: [E] float32 or None.
    Returns float32 [T, E].
    """
    xf = bf16_to_f32(x)
    wf = bf16_to_f32(w_router)
    T, h = xf.shape
    E = wf.shape[0]
    acc = np.zeros((T, E), dtype=np.float32)
    for i in range(h):
        acc += np.multiply.outer(xf[:, i], wf[:, i])  # exact float32 product, one rounding in +=
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32)[None, :]
    return acc


def router_logits_f64(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """The same logits in float64 (used to measure the float32 order's rounding, and for margins)."""
    l = bf16_to_f64(x) @ bf16_to_f64(w_router).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, in rank order.

    Order: logit descending, then expert index ascending (the lowest index wins a tie). -0.0 is
    first made +0.0 so the two zeros tie. Selection is on logits, not on softmax probabilities:
    softmax is strictly increasing, so the selected set is the same mathematically, but float
    exponentials can merge distinct logits.
    Returns int32 [T, k].
    """
    l = np.asarray(logits, dtype=np.float64) + 0.0  # -0.0 + 0.0 == +0.0
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    experts = np.broadcast_to(np.arange(E), l.shape)
    order = np.lexsort((experts, -l), axis=-1)  # last key is primary
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights of the selected experts: softmax over all logits, renormalised over the k.

    The full softmax denominator cancels, so this equals the softmax of the k selected logits:
    w[t, j] = exp(l_j - l_max) / sum over selected i of exp(l_i - l_max), with l_max the first
    (largest) selected logit. Slot j keeps the top-k rank order. float64.
    """
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k):
    """Router logits (fixed float32 order), top-k indices and renormalised softmax weights."""
    logits = router_logits_fixed_order(x, w_router, bias)
    idx = topk(logits, k)
    return logits, idx, topk_weights(logits, idx)


# ----------------------------------------------------------------------------------------------
# Device-side schedule (its result), gather
# ----------------------------------------------------------------------------------------------


def schedule(assign: np.ndarray, n_experts: int, drop: bool = False):
    """Group the assignments by expert, keeping their order inside each expert.

    The Mixture-of-Kittens page's flowchart and Key claims describe a device-side schedule that
    absorbs dynamic per-expert token counts without a host synchronisation and without dropping
    tokens; its result is a stable counting sort of the R = T*k assignments by expert:
      counts[e]  = number of assignments to e,
      offsets    = exclusive prefix sum of counts (length n_experts + 1),
      perm[r]    = the assignment held in routed row r (rows of e are offsets[e] .. offsets[e+1]-1,
                   assignments ascending inside each expert),
      inv[a]     = the row that holds assignment a (inv[perm[r]] == r).

    Reading (the pages say nothing of expert ids outside the local range): with drop=True an
    assignment whose expert id is outside [0, n_experts) gets no row and inv = -1, so perm holds
    offsets[-1] <= R entries; with drop=False such an id is an error.
    """
    a = np.asarray(assign, dtype=np.int64).reshape(-1)
    valid = (a >= 0) & (a < n_experts)
    if not drop and not valid.all():
        raise ValueError("expert id out of range")
    counts = np.bincount(a[valid], minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    np.cumsum(counts, out=offsets[1:])
    kept = np.nonzero(valid)[0]
    perm = kept[np.argsort(a[kept], kind="stable")].astype(np.int32)
    inv = np.full(a.size, -1, dtype=np.int32)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv


def gather_rows(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """A[r] = x[t] for the token t = perm[r] div k that assignment perm[r] belongs to."""
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) // k]


# ----------------------------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(a: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               mx: bool = False, keep: bool = False):
    """One SwiGLU expert on the rows a: H = silu(a W_gate) * (a W_up), O = H W_down. float64.

    The Mixture-of-Kittens Key claims name expert grouped GEMMs with SwiGLU fused, MXFP8 by
    default, with activation quantisation fused into the dispatch, the grouped GEMMs and the
    SwiGLU. With mx=True every GEMM operand is MX-quantised along that GEMM's reduction axis
    before the product: a and W_gate / W_up along h, H and W_down along m. H is quantised from its
    unrounded value (Reading: not via bfloat16).

    a: [n, h] float64; w_gate, w_up: [h, m]; w_down: [m, h] (float64 values).
    Returns O [n, h] (and, with keep=True, a dict of the intermediates G, U, H and the quantised
    operands actually multiplied).
    """
    if mx:
        a = mx_roundtrip(a, axis=1)
        w_gate = mx_roundtrip(w_gate, axis=0)
        w_up = mx_roundtrip(w_up, axis=0)
        w_down = mx_roundtrip(w_down, axis=0)
    g = a @ w_gate
    u = a @ w_up
    hdn = silu(g) * u
    hq = mx_roundtrip(hdn, axis=1) if mx else hdn
    o = hq @ w_down
    if keep:
        return o, {"A": a, "G": g, "U": u, "H": hdn, "Hq": hq, "Wg": w_gate, "Wu": w_up,
                   "Wd": w_down}
    return o


def expert_outputs(A_rows: np.ndarray, offsets: np.ndarray, weights_of, mx: bool) -> np.ndarray:
    """O[r] for every routed row, one expert at a time (weights_of(e) -> bf16 bits triple)."""
    R, h = A_rows.shape
    O = np.zeros((R, h), dtype=np.float64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        wg, wu, wd = (bf16_to_f64(w) for w in weights_of(e))
        O[r0:r1] = swiglu_ffn(A_rows[r0:r1], wg, wu, wd, mx=mx)
    return O


# ----------------------------------------------------------------------------------------------
# Combine
# ----------------------------------------------------------------------------------------------


def combine(O: np.ndarray, inv: np.ndarray, w: np.ndarray, k: int, shared=None) -> np.ndarray:
    """y[t] = S[t] + sum over j = 0..k-1 of w[t, j] * O[inv[t*k + j]] (S = 0 without a shared expert),
    skipping dropped assignments (inv = -1, see schedule).

    The Mixture-of-Kittens page stresses bitwise determinism through a fixed floating-point order;
    the result here is the plain weighted sum in float64, the GPU's fixed j-ascending float32 order
    is compared against it within tolerance.
    """
    inv = np.asarray(inv, dtype=np.int64).reshape(-1, k)
    w = np.asarray(w, dtype=np.float64).reshape(-1, k)
    y = np.zeros((inv.shape[0], O.shape[1]), dtype=np.float64) if shared is None else \
        np.array(shared, dtype=np.float64, copy=True)
    for j in range(k):
        sel = inv[:, j] >= 0  # a dropped assignment (inv = -1) contributes nothing
        y[sel] += w[sel, j:j + 1] * O[inv[sel, j]]
    return y


# ----------------------------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------------------------


def layer_forward(wl, inp: dict, weights_of, shared_weights=None, keep: bool = False) -> dict:
    """The whole forward of one workload on its inputs (moe_inputs.make_inputs).

    weights_of(e) returns local expert e's (W_gate, W_up, W_down) as bf16 bits; shared_weights is
    the shared expert's triple (a BF16 expert over the T source tokens, kept in BF16 as the
    Mixture-of-Kittens Key claims say) or None.
    """
    out = {}
    if wl.mode == "router":
        logits, idx, w = route(inp["x"], inp["w_router"], inp["bias"], wl.k)
        out.update(logits=logits, idx=idx, w=w)
        assign = idx.reshape(-1)
        wflat = w.reshape(-1)
    else:
        assign = inp["assign"]
        wflat = inp["assign_w"].astype(np.float64)
    counts, offsets, perm, inv = schedule(assign, wl.E_loc, drop=True)
    out.update(counts=counts, offsets=offsets, perm=perm, inv=inv)
    x64 = bf16_to_f64(inp["x"])
    A = gather_rows(x64, perm, wl.k)
    O = expert_outputs(A, offsets, weights_of, mx=(wl.dtype == "mxfp8"))
    S = None
    if shared_weights is not None:
        wg, wu, wd = (bf16_to_f64(v) for v in shared_weights)
        S = swiglu_ffn(x64, wg, wu, wd, mx=False)
        out["S"] = S
    out["y"] = combine(O, inv, wflat, wl.k, S)
    if keep:
        out["A"], out["O"] = A, O
    return out


def token_outputs(wl, inp: dict, tokens, weights_of, shared_weights=None, workers: int = 1) -> dict:
    """y[t] for a few tokens only. Each routed row depends only on its own token and expert, so a
    token's output needs no other token's rows; used to check full-size runs on sampled tokens.

    Experts are visited in ascending id order and their contributions added in that order;
    workers > 1 computes the per-expert FFNs in a thread pool (the same values, added in the same
    order). Expert ids outside [0, E_loc) contribute nothing (schedule's drop reading)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x64 = bf16_to_f64(inp["x"][tokens])
    res = {"tokens": tokens}
    if wl.mode == "router":
        logits, idx, w = route(inp["x"][tokens], inp["w_router"], inp["bias"], wl.k)
        res.update(logits=logits, idx=idx, w=w)
    else:
        idx = inp["assign"].reshape(-1, wl.k)[tokens]
        w = inp["assign_w"].reshape(-1, wl.k)[tokens].astype(np.float64)
        res.update(idx=idx, w=w)
    mx = wl.dtype == "mxfp8"
    y = np.zeros((len(tokens), wl.h), dtype=np.float64)
    if shared_weights is not None:
        wg, wu, wd = (bf16_to_f64(v) for v in shared_weights)
        y += swiglu_ffn(x64, wg, wu, wd, mx=False)
    experts = [int(e) for e in np.unique(idx) if 0 <= e < wl.E_loc]

    def expert_rows(e):
        wg, wu, wd = (bf16_to_f64(v) for v in weights_of(e))
        ti, jj = np.nonzero(idx == e)
        return ti, jj, swiglu_ffn(x64[ti], wg, wu, wd, mx=mx)

    if workers > 1 and len(experts) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            parts = ex.map(expert_rows, experts)  # results come back in submission order
            for ti, jj, o in parts:
                # a token can hold the same expert in two slots (expert shares): unbuffered add
                np.add.at(y, ti, w[ti, jj][:, None] * o)
    else:
        for e in experts:
            ti, jj, o = expert_rows(e)
            np.add.at(y, ti, w[ti, jj][:, None] * o)
    res["y"] = y
    return res


# ----------------------------------------------------------------------------------------------
# Backward of the expert path (routing weights held fixed)
# ----------------------------------------------------------------------------------------------


def dsilu(z: np.ndarray) -> np.ndarray:
    """d/dz silu(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _mx_rows(v: np.ndarray) -> np.ndarray:
    """MX round trip along axis 0 (the routed rows of one expert): blocks of 32 rows counted from
    the expert's first row, the last block zero-padded (Reading: the wgrad GEMMs reduce over an
    expert's rows, so their MX blocks run along those rows)."""
    n = v.shape[0]
    if n == 0:
        return v.copy()
    pad = (-n) % 32
    if pad:
        v = np.concatenate([v, np.zeros((pad,) + v.shape[1:], dtype=v.dtype)], axis=0)
    return mx_roundtrip(v, axis=0)[:n]


def expert_backward(a: np.ndarray, dO: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                    w_down: np.ndarray, mx: bool = False):
    """Backward of one SwiGLU expert with respect to its input rows and its three weights.

    a: [n, h] the expert's routed rows before any quantisation; dO: [n, h] the gradient of its
    output rows; w_gate, w_up: [h, m]; w_down: [m, h]. Returns (dA, dW_gate, dW_up, dW_down).

    With G = a W_gate, U = a W_up (the forward's values, from its MX operands when mx) and
    H = silu(G) * U:
      dH = dO W_down^T;  dG = dH * U * dsilu(G);  dU = dH * silu(G)
      dA = dG W_gate^T + dU W_up^T
      dW_gate = a^T dG;  dW_up = a^T dU;  dW_down = H^T dO
    With mx=True every operand of these five GEMMs is MX-quantised along that GEMM's reduction
    axis (Reading: as in the forward, which quantises each GEMM's operands along its reduction
    axis): dO and W_down along h for dH; dG, dU, W_gate and W_up along m for dA; a, dG, dU, H and
    dO along the expert's rows for the weight gradients. The quantised values are those of the
    unrounded float64 quantities (a: the bf16 input itself).
    """
    if mx:
        aq, wgq, wuq = mx_roundtrip(a, axis=1), mx_roundtrip(w_gate, axis=0), \
            mx_roundtrip(w_up, axis=0)
    else:
        aq, wgq, wuq = a, w_gate, w_up
    g, u = aq @ wgq, aq @ wuq
    hdn = silu(g) * u

    def q(v, axis):
        if not mx:
            return v
        return _mx_rows(v) if axis == "rows" else mx_roundtrip(v, axis=axis)

    dh = q(dO, 1) @ q(w_down, 1).T
    dg = dh * u * dsilu(g)
    du = dh * silu(g)
    dA = q(dg, 1) @ q(w_gate, 1).T + q(du, 1) @ q(w_up, 1).T
    ar = q(a, "rows")
    return dA, ar.T @ q(dg, "rows"), ar.T @ q(du, "rows"), q(hdn, "rows").T @ q(dO, "rows")


def layer_backward(wl, inp: dict, fwd: dict, weights_of, dy_f64=None, mx=None):
    """Gradients of the expert path: dX and per-expert (dW_gate, dW_up, dW_down), in float64.

    Reading: the gate weights w are held fixed (the router's own gradient is not part of the
    expert path), so with a = perm[r] and t = a div k the gradient of routed row r's output is
    dO[r] = w[a] * dY[t]; each expert then runs expert_backward on its rows, and
      dX[t] = sum over j ascending of dA[inv[t*k + j]]
    (the un-permute). mx defaults to the workload's dtype being MXFP8.
    """
    if mx is None:
        mx = wl.dtype == "mxfp8"
    k = wl.k
    perm, inv, offsets = fwd["perm"], fwd["inv"], fwd["offsets"]
    dy = bf16_to_f64(inp["dy"]) if dy_f64 is None else dy_f64
    wflat = fwd["w"].reshape(-1) if wl.mode == "router" else inp["assign_w"].astype(np.float64)
    tok = perm.astype(np.int64) // k
    dO = wflat[perm][:, None] * dy[tok]
    A = fwd["A"]
    dA = np.zeros_like(A)
    dW = []
    for e in range(wl.E_loc):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        wg, wu, wd = (bf16_to_f64(v) for v in weights_of(e))
        dA[r0:r1], dwg, dwu, dwd = expert_backward(A[r0:r1], dO[r0:r1], wg, wu, wd, mx=mx)
        dW.append((dwg, dwu, dwd))
    dX = np.zeros_like(dy)
    invk = inv.astype(np.int64).reshape(-1, k)
    for j in range(k):
        sel = invk[:, j] >= 0
        dX[sel] += dA[invk[sel, j]]
    return dX, dW


def token_input_grads(wl, inp: dict, tokens, weights_of, dy_f64=None, mx=None) -> np.ndarray:
    """dX[t] for a few tokens only. The input gradient of a routed row depends only on that row
    (its dgrad GEMMs reduce along h and m, never across rows), so a token's dX needs only its own
    k rows: for each slot j, expert_backward of the single row x[t] with dO = w[t, j] dY[t]."""
    if mx is None:
        mx = wl.dtype == "mxfp8"
    tokens = np.asarray(tokens, dtype=np.int64)
    dy = bf16_to_f64(inp["dy"]) if dy_f64 is None else dy_f64
    x64 = bf16_to_f64(inp["x"][tokens])
    if wl.mode == "router":
        _, idx, w = route(inp["x"][tokens], inp["w_router"], inp["bias"], wl.k)
    else:
        idx = inp["assign"].reshape(-1, wl.k)[tokens]
        w = inp["assign_w"].reshape(-1, wl.k)[tokens].astype(np.float64)
    out = np.zeros((len(tokens), wl.h), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(wl.k):
            e = int(idx[i, j])
            if not 0 <= e < wl.E_loc:
                continue
            wg, wu, wd = (bf16_to_f64(v) for v in weights_of(e))
            dA = expert_backward(x64[i:i + 1], w[i, j] * dy[t][None, :], wg, wu, wd, mx=mx)[0]
            out[i] += dA[0]
    return out


def expert_weight_grads(wl, inp: dict, assign: np.ndarray, assign_w: np.ndarray, e: int,
                        weights_of, dy_f64=None, mx=None):
    """(dW_gate, dW_up, dW_down) of one expert only. They reduce over the expert's routed rows,
    in the schedule's order (its assignments ascending), so only those rows are needed.
    assign / assign_w: the local expert and gate weight of every assignment (length T*k)."""
    if mx is None:
        mx = wl.dtype == "mxfp8"
    dy = bf16_to_f64(inp["dy"]) if dy_f64 is None else dy_f64
    a_idx = np.nonzero(np.asarray(assign) == e)[0]  # ascending: the stable schedule's row order
    tok = a_idx // wl.k
    a = bf16_to_f64(inp["x"][tok])
    dO = np.asarray(assign_w, dtype=np.float64)[a_idx][:, None] * dy[tok]
    wg, wu, wd = (bf16_to_f64(v) for v in weights_of(e))
    _, dwg, dwu, dwd = expert_backward(a, dO, wg, wu, wd, mx=mx)
    return dwg, dwu, dwd


# ----------------------------------------------------------------------------------------------
# Backward through the gate weights and the router
# ----------------------------------------------------------------------------------------------


def gate_grads(dy: np.ndarray, O: np.ndarray, inv: np.ndarray, k: int) -> np.ndarray:
    """dL/dw[t, j] = <dY[t], O[inv[t*k + j]]>: the combine y[t] = S[t] + sum_j w[t, j] O_row is
    linear in each gate weight. O are the expert outputs the forward combined. A dropped
    assignment (inv = -1) has no output row and gets 0. float64, shape [T, k]."""
    inv = np.asarray(inv, dtype=np.int64).reshape(-1, k)
    g = np.zeros(inv.shape, dtype=np.float64)
    for j in range(k):
        sel = inv[:, j] >= 0
        g[sel, j] = np.einsum("th,th->t", dy[sel], O[inv[sel, j]])
    return g


def selected_logit_grads(w: np.ndarray, dgate: np.ndarray) -> np.ndarray:
    """Gradient of the loss with respect to the k selected logits of each token, through the
    renormalised softmax w_j = exp(l_j) / sum over selected i of exp(l_i):
      dl_j = w_j * (dgate_j - sum_i w_i dgate_i).
    The top-k selection itself is piecewise constant in the logits, so the other logits get 0
    (Reading: the gradient of the selection is taken as zero almost everywhere). [T, k]."""
    w = np.asarray(w, dtype=np.float64)
    s = np.sum(w * dgate, axis=1, keepdims=True)
    return w * (dgate - s)


def router_backward(x: np.ndarray, w_router: np.ndarray, idx: np.ndarray, dl: np.ndarray):
    """The router's own gradients from the selected-logit gradients dl [T, k] of the experts idx
    [T, k], with logits l[t, e] = sum_i x[t, i] W_r[e, i] + b[e]:
      dlogits[t, e] = dl[t, j] where idx[t, j] = e, else 0      [T, E]
      dW_r = dlogits^T x   [E, h];   db = sum_t dlogits[t]   [E];   dX_router = dlogits W_r   [T, h]
    x, w_router: bf16 bits. float64. Returns (dW_r, db, dX_router, dlogits)."""
    xf = bf16_to_f64(x)
    wf = bf16_to_f64(w_router)
    T, k = idx.shape
    E = wf.shape[0]
    dlogits = np.zeros((T, E), dtype=np.float64)
    for j in range(k):
        e = np.asarray(idx[:, j], dtype=np.int64)
        ok = (e >= 0) & (e < E)
        np.add.at(dlogits, (np.nonzero(ok)[0], e[ok]), dl[ok, j])
    return dlogits.T @ xf, dlogits.sum(axis=0), dlogits @ wf, dlogits


def layer_backward_full(wl, inp: dict, fwd: dict, weights_of, dy_f64=None, mx=None):
    """The whole layer's backward: the expert path (layer_backward, gate weights fixed) plus the
    gradients through the gate weights. Returns a dict with dX (expert path + router part for a
    router layer), dW (per expert), dgate [T, k] and, for a router layer, dW_r, db, dlogits.
    fwd: layer_forward(..., keep=True) of the same inputs (its O are the expert outputs)."""
    dy = bf16_to_f64(inp["dy"]) if dy_f64 is None else dy_f64
    dX, dW = layer_backward(wl, inp, fwd, weights_of, dy_f64=dy, mx=mx)
    dgate = gate_grads(dy, fwd["O"], fwd["inv"], wl.k)
    out = {"dX": dX, "dW": dW, "dgate": dgate}
    if wl.mode == "router":
        dl = selected_logit_grads(fwd["w"], dgate)
        dWr, db, dXr, dlogits = router_backward(inp["x"], inp["w_router"], fwd["idx"], dl)
        out.update(dX=dX + dXr, dW_r=dWr, db=db, dlogits=dlogits, dl=dl)
    return out
