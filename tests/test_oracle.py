"""Pins of the CPU oracle against things other than itself.

Each check compares the oracle with brute force, a library routine, a closed
form, finite differences or an exact identity, so that a plausible slip in the
oracle (dropped term, wrong sign or index, transposed operand, wrong tie rule)
fails at least one of them.  ``tests/test_oracle_mutants.py`` plants such
slips in a copy of the oracle and checks that they are caught.

The check functions are plain callables (``PINS``) so that the mutant test can
run them against a modified library.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _random_layer(T, D, I, E, K, score, seed):
    r = _rng(seed)
    x = r.standard_normal((T, D))
    wg = r.standard_normal((E, I, D)) / math.sqrt(D)
    wu = r.standard_normal((E, I, D)) / math.sqrt(D)
    wd = r.standard_normal((E, D, I)) / math.sqrt(I)
    dy = r.standard_normal((T, D))
    logits = r.standard_normal((T, E)).astype(np.float32)
    return oracle.Layer(x, wg, wu, wd, K, score, dy), logits


def _dense_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU MLP with numpy matmuls: (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    return (_silu(x @ wg.T) * (x @ wu.T)) @ wd.T


# --------------------------------------------------------------------------- routing

def pin_route_bruteforce():
    """Top-K indices equal a lexsort by (-logit, expert id) for every row,
    including rows with exact ties, all-equal rows and signed zeros."""
    r = _rng(11)
    T, E = 300, 16
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[0] = 0.0
    logits[1] = np.float32(1.5)
    logits[2, :] = r.integers(-2, 3, E).astype(np.float32)   # many ties
    logits[3, ::2] = -0.0
    logits[3, 1::2] = 0.0
    logits[4] = np.linspace(1, -1, E, dtype=np.float32)
    logits[5] = np.linspace(-1, 1, E, dtype=np.float32)
    logits[6:40] = np.round(logits[6:40])                     # coarse values: frequent ties
    for K in (1, 2, 5, E):
        idx, _ = oracle.route(logits, K, synth.SOFTMAX_TOPK)
        for t in range(T):
            order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
            assert list(idx[t]) == list(order[:K]), (K, t)


def pin_route_hand_example():
    """Hand-worked routing case.  E=4, K=2; ties go to the lower expert id and
    -0.0 ties with +0.0.  Derivation:
      t0 [0.5, 2, 2, -1]  -> experts 1, 2 (tie at 2)      w = 1/2, 1/2
      t1 [0, 0, 0, 0]     -> experts 0, 1                 w = 1/2, 1/2
      t2 [-3, 1, -0, 0]   -> experts 1, 2 (-0 ties +0)    w = 1/(1+e^-1), 1/(1+e)
      t3 [4, 1, 4, 2]     -> experts 0, 2                 w = 1/2, 1/2
    flat slots f = 2t + k carry experts 1,2,0,1,1,2,0,2, so counts = 2,3,3,0,
    offsets = 0,2,5,8,8, sorted_to_flat = 2,6 | 0,3,4 | 1,5,7 and
    flat_to_sorted is its inverse 2,5,0,3,4,6,1,7.  Sigmoid score, K=1:
    experts 1,0,1,0 with w = s(2), s(0), s(1), s(4), s(z)=1/(1+e^-z)."""
    logits = np.array([[0.5, 2.0, 2.0, -1.0], [0.0, 0.0, 0.0, 0.0],
                       [-3.0, 1.0, -0.0, 0.0], [4.0, 1.0, 4.0, 2.0]], dtype=np.float32)
    idx, w = oracle.route(logits, 2, synth.SOFTMAX_TOPK)
    assert idx.tolist() == [[1, 2], [0, 1], [1, 2], [0, 2]]
    e1 = math.exp(-1.0)
    np.testing.assert_allclose(w, [[0.5, 0.5], [0.5, 0.5], [1 / (1 + e1), 1 / (1 + math.e)],
                                   [0.5, 0.5]], rtol=1e-15, atol=0)
    counts, offsets, s2f, f2s = oracle.sort(idx, 4)
    assert counts.tolist() == [2, 3, 3, 0]
    assert offsets.tolist() == [0, 2, 5, 8, 8]
    assert s2f.tolist() == [2, 6, 0, 3, 4, 1, 5, 7]
    assert f2s.tolist() == [2, 5, 0, 3, 4, 6, 1, 7]
    idx1, w1 = oracle.route(logits, 1, synth.SIGMOID)
    assert idx1.ravel().tolist() == [1, 0, 1, 0]
    sig = [1 / (1 + math.exp(-z)) for z in (2.0, 0.0, 1.0, 4.0)]
    np.testing.assert_allclose(w1.ravel(), sig, rtol=1e-15, atol=0)


def pin_route_softmax_weights():
    """Renormalised weights equal the full softmax over all E experts (computed
    with numpy) restricted to the selected experts and divided by their sum;
    they sum to one; K=1 gives exactly 1."""
    r = _rng(12)
    T, E = 200, 32
    logits = (3 * r.standard_normal((T, E))).astype(np.float32)
    for K in (1, 3, 8, E):
        idx, w = oracle.route(logits, K, synth.SOFTMAX_TOPK)
        l64 = logits.astype(np.float64)
        p = np.exp(l64 - l64.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        sel = np.take_along_axis(p, idx.astype(np.int64), 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
        assert np.all(np.diff(w, axis=1) <= 0)               # slot order = rank order
        if K == 1:
            assert np.all(w == 1.0)


def pin_route_sigmoid_weights():
    """Sigmoid score: w = scipy's expit of the selected logit, no renormalisation."""
    from scipy.special import expit
    r = _rng(13)
    logits = (2 * r.standard_normal((100, 16))).astype(np.float32)
    for K in (1, 4):
        idx, w = oracle.route(logits, K, synth.SIGMOID)
        sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), 1)
        np.testing.assert_allclose(w, expit(sel), rtol=1e-14)


# --------------------------------------------------------------------------- sort

def pin_sort_library():
    """counts = bincount; offsets = exclusive cumsum; sorted_to_flat equals
    numpy's stable argsort of the flat expert ids; flat_to_sorted is its inverse."""
    r = _rng(14)
    for (T, K, E) in [(300, 4, 16), (1, 1, 1), (50, 3, 64), (0, 2, 8), (129, 8, 128)]:
        logits = r.standard_normal((T, E)).astype(np.float32)
        if T > 3:
            logits[: T // 3, 0] += 4.0       # skew: one hot expert, some empty ones
        idx, _ = oracle.route(logits, K, synth.SOFTMAX_TOPK)
        counts, offsets, s2f, f2s = oracle.sort(idx, E)
        flat = idx.ravel()
        assert counts.tolist() == np.bincount(flat, minlength=E).tolist()
        assert int(counts.sum()) == T * K
        assert offsets.tolist() == [0] + np.cumsum(counts).tolist()
        assert s2f.tolist() == np.argsort(flat, kind="stable").tolist()
        assert np.array_equal(f2s[s2f], np.arange(T * K))


# --------------------------------------------------------------------------- forward

def pin_forward_dense_mlp():
    """One expert, K=1 (renormalised weight 1): y equals the dense SwiGLU MLP."""
    L, logits = _random_layer(T=40, D=24, I=12, E=1, K=1, score=synth.SOFTMAX_TOPK, seed=21)
    idx, w = oracle.route(logits, 1, synth.SOFTMAX_TOPK)
    y = oracle.forward(L, idx, w)
    ref = _dense_swiglu(L.x, L.w_gate[0], L.w_up[0], L.w_down[0])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def pin_forward_dense_mixture():
    """K=E with softmax routing: y is the dense softmax mixture of all experts."""
    E = 5
    L, logits = _random_layer(T=30, D=16, I=8, E=E, K=E, score=synth.SOFTMAX_TOPK, seed=22)
    idx, w = oracle.route(logits, E, synth.SOFTMAX_TOPK)
    y = oracle.forward(L, idx, w)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    outs = np.stack([_dense_swiglu(L.x, L.w_gate[e], L.w_up[e], L.w_down[e]) for e in range(E)], 1)
    ref = np.einsum("te,ted->td", p, outs)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def pin_forward_top1_sigmoid():
    """K=1 with the sigmoid score: y = sigmoid(max logit) * MLP_argmax(x)."""
    E = 6
    L, logits = _random_layer(T=25, D=16, I=8, E=E, K=1, score=synth.SIGMOID, seed=23)
    idx, w = oracle.route(logits, 1, synth.SIGMOID)
    y = oracle.forward(L, idx, w)
    am = np.argmax(logits, 1)
    ref = np.stack([_dense_swiglu(L.x[t:t + 1], L.w_gate[am[t]], L.w_up[am[t]], L.w_down[am[t]])[0]
                    / (1 + np.exp(-float(logits[t, am[t]]))) for t in range(L.T)])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def pin_forward_token_subset():
    """Forward on a token list equals the matching rows of the full forward,
    and the unweighted expert outputs combine back into y."""
    L, logits = _random_layer(T=40, D=16, I=8, E=6, K=3, score=synth.SOFTMAX_TOPK, seed=24)
    idx, w = oracle.route(logits, 3, synth.SOFTMAX_TOPK)
    y_all = oracle.forward(L, idx, w)
    tok = np.array([39, 0, 17, 17, 5])
    y_sub, o = oracle.forward(L, idx, w, tokens=tok, want_o=True)
    np.testing.assert_array_equal(y_sub, y_all[tok])
    np.testing.assert_allclose(np.einsum("nk,nkd->nd", w[tok], o), y_sub, rtol=1e-13, atol=1e-14)
    for n, t in enumerate(tok):
        for k in range(3):
            e = idx[t, k]
            ref = _dense_swiglu(L.x[t:t + 1], L.w_gate[e], L.w_up[e], L.w_down[e])[0]
            np.testing.assert_allclose(o[n, k], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- backward

def _loss(L, idx, w):
    return float(np.sum(L.dy * oracle.forward(L, idx, w)))


def pin_backward_finite_differences():
    """Central finite differences of L = <dY, y> in float64 with routing held
    fixed: every entry of dX, dW_gate, dW_up, dW_down and dRouterWeights of a
    small layer, plus random directions."""
    L, logits = _random_layer(T=10, D=8, I=6, E=4, K=2, score=synth.SOFTMAX_TOPK, seed=31)
    idx, w = oracle.route(logits, 2, synth.SOFTMAX_TOPK)
    dx, drw = oracle.backward_tokens(L, idx, w)
    dwg, dwu, dwd = oracle.backward_dw(L, idx, w)
    h = 1e-5

    def fd(arr_name, grad):
        flat = getattr(L, arr_name).reshape(-1)          # a view: edits reach the oracle
        num = np.empty(flat.size)
        for j in range(flat.size):
            keep = flat[j]
            flat[j] = keep + h
            lp = _loss(L, idx, w_cur[0])
            flat[j] = keep - h
            lm = _loss(L, idx, w_cur[0])
            flat[j] = keep
            num[j] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad.reshape(-1), num, rtol=1e-6, atol=1e-8, err_msg=arr_name)

    w_cur = [w.copy()]
    fd("x", dx)
    fd("w_gate", dwg)
    fd("w_up", dwu)
    fd("w_down", dwd)
    # router weights
    wf = w_cur[0].reshape(-1)
    num = np.empty(wf.size)
    for j in range(wf.size):
        keep = wf[j]
        wf[j] = keep + h
        lp = _loss(L, idx, w_cur[0])
        wf[j] = keep - h
        lm = _loss(L, idx, w_cur[0])
        wf[j] = keep
        num[j] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(drw.reshape(-1), num, rtol=1e-6, atol=1e-8, err_msg="w")
    # random directions through all parameters at once
    r = _rng(32)
    for _ in range(4):
        dirs = {n: r.standard_normal(getattr(L, n).shape) for n in ("x", "w_gate", "w_up", "w_down")}
        dw_dir = r.standard_normal(w.shape)
        pred = (np.sum(dirs["x"] * dx) + np.sum(dirs["w_gate"] * dwg) + np.sum(dirs["w_up"] * dwu)
                + np.sum(dirs["w_down"] * dwd) + np.sum(dw_dir * drw))
        base = {n: getattr(L, n).copy() for n in dirs}

        def at(s):
            for n in dirs:
                getattr(L, n)[...] = base[n] + s * dirs[n]
            return _loss(L, idx, w + s * dw_dir)
        num = (at(h) - at(-h)) / (2 * h)
        at(0.0)
        assert abs(num - pred) <= 1e-6 * max(1.0, abs(pred)), (num, pred)


def pin_backward_euler_identities():
    """y is linear in W_down, in W_up and in the router weights, so
    <W_down, dW_down> = <W_up, dW_up> = sum w * dRW = <dY, y> exactly (up to
    rounding), on the tiny workload's real shape."""
    d = synth.generate(synth.TINY)
    f = synth.bf16_bits_to_f64
    L = oracle.Layer(f(d["x"]), f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]), synth.TINY.K,
                     synth.TINY.score, f(d["dy"]))
    idx, w = oracle.route(d["logits"], L.K, L.score)
    y = oracle.forward(L, idx, w)
    dx, drw = oracle.backward_tokens(L, idx, w)
    dwg, dwu, dwd = oracle.backward_dw(L, idx, w)
    ref = float(np.sum(L.dy * y))
    for val in (np.sum(L.w_down * dwd), np.sum(L.w_up * dwu), np.sum(w * drw)):
        assert abs(val - ref) <= 1e-10 * max(1.0, abs(ref)), (val, ref)


def pin_backward_empty_expert_and_entries():
    """An expert that receives no rows gets exact-zero weight gradients; single
    entries agree with the full gradient; token-subset backward rows agree with
    the full backward."""
    L, logits = _random_layer(T=30, D=16, I=8, E=6, K=2, score=synth.SOFTMAX_TOPK, seed=33)
    logits[:, 4] = -50.0                                   # expert 4 never selected
    idx, w = oracle.route(logits, 2, synth.SOFTMAX_TOPK)
    assert not np.any(idx == 4)
    dwg, dwu, dwd = oracle.backward_dw(L, idx, w)
    assert not dwg[4].any() and not dwu[4].any() and not dwd[4].any()
    r = _rng(34)
    which = r.integers(0, 3, 60)
    e = r.integers(0, 6, 60)
    rr = np.where(which == 2, r.integers(0, 16, 60), r.integers(0, 8, 60))
    cc = np.where(which == 2, r.integers(0, 8, 60), r.integers(0, 16, 60))
    vals = oracle.dw_entries(L, idx, w, which, e, rr, cc)
    full = [dwg, dwu, dwd]
    ref = np.array([full[q][a, b, c] for q, a, b, c in zip(which, e, rr, cc)])
    np.testing.assert_allclose(vals, ref, rtol=1e-12, atol=1e-14)
    dx_all, drw_all = oracle.backward_tokens(L, idx, w)
    tok = np.array([3, 29, 0])
    dx_s, drw_s = oracle.backward_tokens(L, idx, w, tokens=tok)
    np.testing.assert_array_equal(dx_s, dx_all[tok])
    np.testing.assert_array_equal(drw_s, drw_all[tok])


def pin_backward_dw_token_subset():
    """Weight gradients over a token subset equal those of a layer holding only
    those tokens."""
    L, logits = _random_layer(T=20, D=8, I=4, E=3, K=2, score=synth.SOFTMAX_TOPK, seed=35)
    idx, w = oracle.route(logits, 2, synth.SOFTMAX_TOPK)
    tok = np.array([2, 3, 11, 19])
    sub = oracle.Layer(L.x[tok], L.w_gate, L.w_up, L.w_down, 2, L.score, L.dy[tok])
    a = oracle.backward_dw(L, idx, w, tokens=tok)
    b = oracle.backward_dw(sub, idx[tok], w[tok])
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-13, atol=1e-15)


def pin_expert_dw_finite_differences():
    """One expert's weight gradients (the matrix-product form) against central
    finite differences of L = <dY, y> in that expert's W_gate, W_up and W_down,
    for every expert of a small layer (one of them receives no rows)."""
    L, logits = _random_layer(T=9, D=5, I=4, E=4, K=2, score=synth.SOFTMAX_TOPK, seed=36)
    logits[:, 3] = -50.0                                   # expert 3 never selected
    idx, w = oracle.route(logits, 2, synth.SOFTMAX_TOPK)
    h = 1e-5
    for e in range(4):
        grads = oracle.expert_dw(L, idx, w, e)
        for name, grad in zip(("w_gate", "w_up", "w_down"), grads):
            flat = getattr(L, name)[e].reshape(-1)         # a view: edits reach the oracle
            num = np.empty(flat.size)
            for j in range(flat.size):
                keep = flat[j]
                flat[j] = keep + h
                lp = _loss(L, idx, w)
                flat[j] = keep - h
                lm = _loss(L, idx, w)
                flat[j] = keep
                num[j] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(grad.reshape(-1), num, rtol=1e-6, atol=1e-8,
                                       err_msg=f"{name}[{e}]")
        if e == 3:
            assert not any(g.any() for g in grads)


def pin_expert_dw_matches_row_loop():
    """The matrix-product form equals the per-row loop of backward_dw for every
    expert, with either score function."""
    for score, seed in ((synth.SOFTMAX_TOPK, 37), (synth.SIGMOID, 38)):
        L, logits = _random_layer(T=40, D=16, I=8, E=5, K=2, score=score, seed=seed)
        idx, w = oracle.route(logits, 2, score)
        full = oracle.backward_dw(L, idx, w)
        for e in range(5):
            for a, b in zip(oracle.expert_dw(L, idx, w, e), full):
                np.testing.assert_allclose(a, b[e], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- router side

def pin_router_logits_library():
    """The router projection equals a numpy matmul x @ W_r."""
    r = _rng(41)
    x = r.standard_normal((37, 24))
    w_r = r.standard_normal((24, 9)) / math.sqrt(24)
    np.testing.assert_allclose(oracle.router_logits(x, w_r), x @ w_r, rtol=1e-13, atol=1e-13)


def _router_weights(l, idx, score):
    """Router weights of the selected experts as a function of the logits (numpy)."""
    ls = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if score == synth.SOFTMAX_TOPK:
        z = np.exp(ls - ls.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-ls))


def pin_router_backward_finite_differences():
    """With the selection fixed, L(x, W_r) = sum drw * w(x W_r); central
    differences of L against every entry of dl = dL/dlogits, dW_r and the
    router's dX, for both scores."""
    h = 1e-6
    for score, K in ((synth.SOFTMAX_TOPK, 3), (synth.SIGMOID, 1), (synth.SOFTMAX_TOPK, 5)):
        r = _rng(42 + K)
        T, D, E = 7, 6, 5
        x = r.standard_normal((T, D))
        w_r = r.standard_normal((D, E))
        drw = r.standard_normal((T, K))
        l0 = x @ w_r
        idx, w = oracle.route(l0.astype(np.float32), K, score)
        dl, dw_r, dx_r = oracle.router_backward(x, w_r, idx, _router_weights(l0, idx, score), drw,
                                                score)

        def loss_l(l):
            return float(np.sum(drw * _router_weights(l, idx, score)))

        def fd(arr, f):
            out = np.empty(arr.size)
            flat = arr.reshape(-1)
            for j in range(flat.size):
                keep = flat[j]
                flat[j] = keep + h
                lp = f()
                flat[j] = keep - h
                lm = f()
                flat[j] = keep
                out[j] = (lp - lm) / (2 * h)
            return out.reshape(arr.shape)

        l = l0.copy()
        np.testing.assert_allclose(dl, fd(l, lambda: loss_l(l)), rtol=1e-6, atol=1e-8, err_msg="dl")
        np.testing.assert_allclose(dw_r, fd(w_r, lambda: loss_l(x @ w_r)), rtol=1e-6, atol=1e-8,
                                   err_msg="dW_r")
        np.testing.assert_allclose(dx_r, fd(x, lambda: loss_l(x @ w_r)), rtol=1e-6, atol=1e-8,
                                   err_msg="dx_r")


def pin_router_backward_invariants():
    """Renormalised weights are invariant to a common shift of the selected
    logits, so each token's dl sums to 0 over its experts; K = 1 renormalised
    (w = 1 always) gives dl = 0 exactly; unselected experts get dl = 0."""
    r = _rng(45)
    T, D, E, K = 40, 8, 6, 3
    x = r.standard_normal((T, D))
    w_r = r.standard_normal((D, E))
    l = (x @ w_r).astype(np.float32)
    idx, w = oracle.route(l, K, synth.SOFTMAX_TOPK)
    dl, _, _ = oracle.router_backward(x, w_r, idx, w, r.standard_normal((T, K)), synth.SOFTMAX_TOPK)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-13)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert not dl[~sel].any()
    idx1, w1 = oracle.route(l, 1, synth.SOFTMAX_TOPK)
    assert np.all(w1 == 1.0)
    dl1, dw1, dx1 = oracle.router_backward(x, w_r, idx1, w1, r.standard_normal((T, 1)),
                                           synth.SOFTMAX_TOPK)
    assert not dl1.any() and not dw1.any() and not dx1.any()


def pin_router_full_layer_input_gradient():
    """Through the whole layer with the selection fixed, L = <dY, y> depends on
    x along two paths (the experts' inputs and the router logits x W_r); the
    expert-path dX plus the router's dX (fed with the layer's dRouterWeights)
    matches central differences of L in x, and dW_r matches them in W_r."""
    L, _ = _random_layer(T=6, D=5, I=4, E=4, K=2, score=synth.SOFTMAX_TOPK, seed=46)
    r = _rng(47)
    w_r = r.standard_normal((L.D, L.E))
    l0 = L.x @ w_r
    idx, _ = oracle.route(l0.astype(np.float32), 2, synth.SOFTMAX_TOPK)

    def loss():
        w = _router_weights(L.x @ w_r, idx, synth.SOFTMAX_TOPK)
        return float(np.sum(L.dy * oracle.forward(L, idx, w)))

    w = _router_weights(l0, idx, synth.SOFTMAX_TOPK)
    dx_e, drw = oracle.backward_tokens(L, idx, w)
    _, dw_r, dx_r = oracle.router_backward(L.x, w_r, idx, w, drw, synth.SOFTMAX_TOPK)
    h = 1e-6
    for arr, grad, name in ((L.x, dx_e + dx_r, "dx"), (w_r, dw_r, "dW_r")):
        flat = arr.reshape(-1)
        num = np.empty(flat.size)
        for j in range(flat.size):
            keep = flat[j]
            flat[j] = keep + h
            lp = loss()
            flat[j] = keep - h
            lm = loss()
            flat[j] = keep
            num[j] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad.reshape(-1), num, rtol=1e-6, atol=1e-8, err_msg=name)


PINS = [
    pin_route_bruteforce,
    pin_route_hand_example,
    pin_route_softmax_weights,
    pin_route_sigmoid_weights,
    pin_sort_library,
    pin_forward_dense_mlp,
    pin_forward_dense_mixture,
    pin_forward_top1_sigmoid,
    pin_forward_token_subset,
    pin_backward_finite_differences,
    pin_backward_euler_identities,
    pin_backward_empty_expert_and_entries,
    pin_backward_dw_token_subset,
    pin_expert_dw_finite_differences,
    pin_expert_dw_matches_row_loop,
    pin_router_logits_library,
    pin_router_backward_finite_differences,
    pin_router_backward_invariants,
    pin_router_full_layer_input_gradient,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()


def test_oracle_bad_args():
    with pytest.raises(RuntimeError):
        oracle.route(np.zeros((4, 3), np.float32), 4, synth.SOFTMAX_TOPK)   # K > E
    with pytest.raises(RuntimeError):
        oracle.sort(np.array([[0, 5]], np.int32), 4)                         # id >= E
