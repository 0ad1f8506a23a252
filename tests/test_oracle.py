"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test compares the oracle with something other than itself: the page's
worked example (tests/golden/worked_example_p3.json), hand-derived special
cases, library routines (scipy's softmax, torch's silu and matmul), brute
force over all k-subsets, a dense sum over all experts, and invariants.
``test_planted_mistakes`` plants plausible bugs in the oracle and checks that
at least one pin fails for each.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_p3.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


def worked_example_inputs():
    """Logits designed to give the page's routing: Wr = I, x[t] = ln(w) on the chosen experts, -10 elsewhere."""
    g = _golden()["page_facts"]
    E = len(g["experts"])
    x = np.full((len(g["tokens"]), E), -10.0)
    for t, tok in enumerate(g["tokens"]):
        for ename, wt in g["routing"][tok]:
            x[t, g["experts"].index(ename)] = np.log(wt)
    return x, np.eye(E), None, g["k"]


# ----------------------------------------------------------------- checks --
def check_worked_example_routing():
    g = _golden()
    x, Wr, b, k = worked_example_inputs()
    r = oracle.route(x, Wr, b, k)
    d = oracle.dispatch(r.ids, r.keep, Wr.shape[1])
    exp = g["derived"]
    assert np.array_equal(r.ids, exp["topk_ids"])
    assert np.allclose(r.w, exp["topk_w"], atol=1e-6, rtol=0)
    assert np.array_equal(d.counts, exp["counts"]) and list(d.counts) == g["page_facts"]["group_rows"]
    assert np.array_equal(d.offsets, exp["offsets"])
    assert np.array_equal(d.row_token, exp["row_token"])
    assert np.array_equal(d.inv, exp["inv"])
    # the page's groups, read back from the dispatch
    toks, exps = g["page_facts"]["tokens"], g["page_facts"]["experts"]
    for e, name in enumerate(exps):
        rows = d.row_token[d.offsets[e]:d.offsets[e + 1]]
        assert [toks[t] for t in rows] == g["page_facts"]["groups"][name]


def check_worked_example_combine():
    """Unit-vector y_perm rows make the combine's output spell out (row, weight) pairs."""
    g = _golden()
    x, Wr, b, k = worked_example_inputs()
    r = oracle.route(x, Wr, b, k)
    d = oracle.dispatch(r.ids, r.keep, Wr.shape[1])
    A = int(d.offsets[-1])
    y = oracle.combine(np.eye(A), d.inv, r.w)
    want = np.zeros((4, A))
    for t, (ra, rb) in enumerate(g["derived"]["inv"]):
        wa, wb = g["derived"]["topk_w"][t]
        want[t, ra] += wa
        want[t, rb] += wb
    assert np.allclose(y, want, atol=1e-6, rtol=0)
    # T1 = 0.7 * E1(x1) + 0.3 * E3(x1), as printed on the page
    e1_row = d.offsets[0] + list(d.row_token[d.offsets[0]:d.offsets[1]]).index(0)
    e3_row = d.offsets[2] + list(d.row_token[d.offsets[2]:d.offsets[3]]).index(0)
    assert abs(y[0, e1_row] - 0.7) < 1e-6 and abs(y[0, e3_row] - 0.3) < 1e-6


def check_drop_case():
    g = _golden()["drop_case"]
    x, Wr, b, k = worked_example_inputs()
    r = oracle.route(x, Wr, b, k, drop_thresh=g["drop_thresh"])
    d = oracle.dispatch(r.ids, r.keep, Wr.shape[1])
    assert np.allclose(r.w, g["topk_w"], atol=1e-6, rtol=0)
    assert np.array_equal(d.counts, g["counts"])
    assert np.array_equal(d.offsets, g["offsets"])
    assert np.array_equal(d.row_token, g["row_token"])
    assert np.array_equal(d.inv, g["inv"])


def check_tie_break():
    logits = np.array([[1.0, 2.0, 2.0, 0.5], [3.0, 3.0, 3.0, 3.0]])
    ids, _ = oracle.select_topk(logits, 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    ids, _ = oracle.select_topk(np.array([[0.0, 1.0, 1.0, 1.0]]), 1)
    assert ids.tolist() == [[1]]


def check_single_expert_mlp(seed=3):
    """E = 1, k = 1: the layer is a plain two-layer MLP (torch silu + matmul, float64)."""
    import torch

    rng = np.random.default_rng(seed)
    T, H, F = 7, 12, 20
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((H, 1))
    W1 = rng.standard_normal((1, H, F)) / np.sqrt(H)
    W2 = rng.standard_normal((1, F, H)) / np.sqrt(F)
    y = oracle.forward(x, Wr, None, W1, W2, 1).y
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.silu(xt @ torch.from_numpy(W1[0])) @ torch.from_numpy(W2[0])
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def check_k_equals_E_softmax(seed=4):
    from scipy.special import softmax

    rng = np.random.default_rng(seed)
    T, H, E = 9, 6, 5
    x, Wr, b = rng.standard_normal((T, H)), rng.standard_normal((H, E)), rng.standard_normal(E)
    r = oracle.route(x, Wr, b, E)
    assert np.array_equal(r.ids, np.tile(np.arange(E), (T, 1)))
    assert np.allclose(r.w, softmax(x @ Wr + b, axis=1), rtol=1e-13, atol=1e-15)


def check_dense_bruteforce(seed=5, drop=0.0, shared=False):
    rng = np.random.default_rng(seed)
    T, H, F, E, k, Fs = 11, 16, 24, 6, 3, 10
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((H, E))
    b = rng.standard_normal(E) * 0.5
    W1 = rng.standard_normal((E, H, F)) / np.sqrt(H)
    W2 = rng.standard_normal((E, F, H)) / np.sqrt(F)
    W1s = rng.standard_normal((H, Fs)) / np.sqrt(H) if shared else None
    W2s = rng.standard_normal((Fs, H)) / np.sqrt(Fs) if shared else None
    res = oracle.forward(x, Wr, b, W1, W2, k, drop, W1s, W2s)
    yd = oracle.dense_bruteforce(x, Wr, b, W1, W2, k, drop, W1s, W2s)
    scale = np.abs(yd).max()
    assert np.abs(res.y - yd).max() <= 1e-12 * scale
    # and every routed term, one token at a time, straight from the equation
    for t in range(T):
        acc = np.zeros(H) if not shared else oracle.shared_ffn(x[t:t + 1], W1s, W2s)[0]
        for j in range(k):
            e = res.route.ids[t, j]
            h = x[t] @ W1[e]
            acc = acc + res.route.w[t, j] * ((h / (1 + np.exp(-h))) @ W2[e])
        assert np.allclose(res.y[t], acc, rtol=1e-12, atol=1e-12 * scale)


def check_softmax_all_then_restrict(seed=6):
    """Softmax over all E, keep the top-k, renormalise == softmax over the top-k logits."""
    from scipy.special import softmax

    rng = np.random.default_rng(seed)
    T, H, E, k = 20, 8, 10, 3
    x, Wr = rng.standard_normal((T, H)), rng.standard_normal((H, E))
    r = oracle.route(x, Wr, None, k)
    p = softmax(x @ Wr, axis=1)
    for t in range(T):
        top = np.argsort(-p[t])[:k]
        q = p[t, np.sort(top)]
        assert np.allclose(r.w[t], q / q.sum(), rtol=1e-14, atol=1e-15)


def check_topk_subsets(seed=7):
    """Top-k == the k-subset with the largest logit sum (no ties), by enumeration."""
    rng = np.random.default_rng(seed)
    T, E = 30, 7
    for k in range(1, E + 1):
        logits = rng.standard_normal((T, E))
        ids, _ = oracle.select_topk(logits, k)
        for t in range(T):
            best = max(itertools.combinations(range(E), k), key=lambda s: logits[t, list(s)].sum())
            assert list(ids[t]) == sorted(best)


ALL_CHECKS = [
    check_worked_example_routing, check_worked_example_combine, check_drop_case, check_tie_break,
    check_single_expert_mlp, check_k_equals_E_softmax, check_dense_bruteforce, check_softmax_all_then_restrict,
    check_topk_subsets,
]


# ------------------------------------------------------------------ tests --
@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


def test_dense_bruteforce_with_drop_and_shared():
    check_dense_bruteforce(seed=11, drop=0.2, shared=True)
    check_dense_bruteforce(seed=12, drop=0.0, shared=True)


def test_drop_005_changes_nothing_on_worked_example():
    x, Wr, b, k = worked_example_inputs()
    r0 = oracle.route(x, Wr, b, k)
    r1 = oracle.route(x, Wr, b, k, drop_thresh=0.05)
    assert np.array_equal(r0.keep, r1.keep) and np.allclose(r0.w, r1.w, rtol=0, atol=1e-15)


def _random_case(rng, T, H, F, E, k, drop):
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((H, E))
    W1 = rng.standard_normal((E, H, F)) / np.sqrt(H)
    W2 = rng.standard_normal((E, F, H)) / np.sqrt(F)
    return x, Wr, W1, W2


def check_invariants(res, T, E, k):
    w, keep, d = res.route.w, res.route.keep, res.dispatch
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w[~keep] == 0.0) and np.all(w[keep] > 0)
    assert int(d.counts.sum()) == T * k - int((~keep).sum())
    assert np.all(np.diff(d.offsets) >= 0) and d.offsets[0] == 0
    A = int(d.offsets[-1])
    flat = d.inv[keep]
    assert sorted(flat.tolist()) == list(range(A))          # bijection onto [0, A)
    assert np.all(d.inv[~keep] == -1)
    tt = np.nonzero(keep)[0]
    assert np.array_equal(d.row_token[d.inv[keep]], tt)      # row_token[inv[t, j]] == t
    for e in range(E):                                      # rows of e: ascending tokens, all chose e
        rows = d.row_token[d.offsets[e]:d.offsets[e + 1]]
        assert np.all(np.diff(rows) > 0)
        for t in rows:
            j = list(res.route.ids[t]).index(e)
            assert keep[t, j]
    assert np.array_equal(res.x_perm, np.asarray(res.x_perm))


def test_invariants_random():
    rng = np.random.default_rng(21)
    for (T, H, F, E, k, drop) in [(13, 8, 8, 5, 2, 0.0), (40, 8, 16, 9, 4, 0.1), (1, 8, 8, 3, 3, 0.0),
                                  (25, 16, 8, 16, 1, 0.0), (30, 8, 8, 6, 6, 1 / 6)]:
        x, Wr, W1, W2 = _random_case(rng, T, H, F, E, k, drop)
        res = oracle.forward(x, Wr, None, W1, W2, k, drop)
        check_invariants(res, T, E, k)


def test_forward_tokens_matches_forward():
    rng = np.random.default_rng(22)
    T, H, F, E, k = 17, 8, 12, 6, 2
    x, Wr, W1, W2 = _random_case(rng, T, H, F, E, k, 0.1)
    full = oracle.forward(x, Wr, None, W1, W2, k, 0.1)
    toks = [0, 3, 16, 5]
    ids, w, keep, y = oracle.forward_tokens(toks, x, Wr, None, W1, W2, k, 0.1)
    assert np.array_equal(ids, full.route.ids[toks]) and np.array_equal(keep, full.route.keep[toks])
    assert np.allclose(y, full.y[toks], rtol=1e-12, atol=1e-12)


def test_property_random_shapes():
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies

    @hyp.settings(max_examples=40, deadline=None, derandomize=True)
    @hyp.given(T=st.integers(1, 24), H=st.integers(1, 9), F=st.integers(1, 9), E=st.integers(1, 8),
               kf=st.floats(0.0, 1.0), seed=st.integers(0, 10_000), use_drop=st.booleans())
    def run(T, H, F, E, kf, seed, use_drop):
        k = 1 + int(kf * (E - 1))
        drop = (0.5 / k) if use_drop else 0.0
        rng = np.random.default_rng(seed)
        x, Wr, W1, W2 = _random_case(rng, T, H, F, E, k, drop)
        res = oracle.forward(x, Wr, None, W1, W2, k, drop)
        check_invariants(res, T, E, k)
        yd = oracle.dense_bruteforce(x, Wr, None, W1, W2, k, drop)
        assert np.abs(res.y - yd).max() <= 1e-12 * max(1.0, np.abs(yd).max())

    run()


# ------------------------------------------------------ planted mistakes --
def _mut_silu_identity(mp):
    mp.setattr(mo, "silu", lambda u: u)


def _mut_silu_sign(mp):
    mp.setattr(mo, "silu", lambda u: u / (1.0 + np.exp(u)))


def _mut_reverse_rows(mp):
    orig = mo.dispatch

    def bad(ids, keep, E):
        d = orig(ids, keep, E)
        rt, inv = d.row_token.copy(), d.inv.copy()
        for e in range(E):
            a, b = d.offsets[e], d.offsets[e + 1]
            rt[a:b] = d.row_token[a:b][::-1]
        for t in range(inv.shape[0]):
            for j in range(inv.shape[1]):
                if d.inv[t, j] >= 0:
                    e = ids[t, j]
                    a, b = d.offsets[e], d.offsets[e + 1]
                    inv[t, j] = a + (b - 1 - d.inv[t, j])
        return mo.DispatchResult(d.counts, d.offsets, rt, inv)

    mp.setattr(mo, "dispatch", bad)
    mp.setattr(oracle, "dispatch", bad)


def _mut_combine_slot_swap(mp):
    orig = mo.combine

    def bad(y_perm, inv, w, y_shared=None, T=None):
        return orig(y_perm, inv, w[:, ::-1], y_shared, T)

    mp.setattr(mo, "combine", bad)
    mp.setattr(oracle, "combine", bad)


def _mut_tie_high(mp):
    def bad(logits, k):
        T, E = logits.shape
        ids = np.broadcast_to(-np.arange(E), (T, E))
        order = np.lexsort((ids, -logits), axis=1)
        ranked = np.take_along_axis(logits, order, axis=1)
        gap = ranked[:, k - 1] - ranked[:, k] if k < E else np.full(T, np.inf)
        return np.sort(order[:, :k], axis=1), gap

    mp.setattr(mo, "select_topk", bad)
    mp.setattr(oracle, "select_topk", bad)


def _mut_softmax_over_all(mp):
    def bad(x, Wr, b, k, drop_thresh=0.0):
        logits = mo.router_logits(x, Wr, b)
        ids, gap = mo.select_topk(logits, k)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
        keep = np.ones_like(w, dtype=bool)
        return mo.RouteResult(ids, w, keep, logits, gap)

    mp.setattr(mo, "route", bad)
    mp.setattr(oracle, "route", bad)


def _mut_drop_no_renorm(mp):
    orig = mo.route

    def bad(x, Wr, b, k, drop_thresh=0.0):
        r = orig(x, Wr, b, k, 0.0)
        if drop_thresh > 0:
            keep = r.w >= drop_thresh
            r = mo.RouteResult(r.ids, np.where(keep, r.w, 0.0), keep, r.logits, r.gap)
        return r

    mp.setattr(mo, "route", bad)
    mp.setattr(oracle, "route", bad)


def _mut_w2_transposed_square(mp):
    orig = mo.expert_ffn

    def bad(rows, W1e, W2e):
        W2e = np.asarray(W2e)
        if W2e.shape[0] == W2e.shape[1]:
            W2e = W2e.T
        else:
            W2e = W2e.T.reshape(W2e.shape)
        return orig(rows, W1e, W2e)

    mp.setattr(mo, "expert_ffn", bad)


def _mut_bias_sign(mp):
    orig = mo.router_logits

    def bad(x, Wr, b=None):
        return orig(x, Wr, None if b is None else -np.asarray(b))

    mp.setattr(mo, "router_logits", bad)


def _mut_shared_dropped(mp):
    mp.setattr(mo, "shared_ffn", lambda x, W1s, W2s: 0.0 * mo.expert_ffn(x, W1s, W2s))


MUTATIONS = [_mut_silu_identity, _mut_silu_sign, _mut_reverse_rows, _mut_combine_slot_swap, _mut_tie_high,
             _mut_softmax_over_all, _mut_drop_no_renorm, _mut_w2_transposed_square, _mut_bias_sign,
             _mut_shared_dropped]


def _check_bias_k_equals_E():
    from scipy.special import softmax

    rng = np.random.default_rng(8)
    x, Wr, b = rng.standard_normal((5, 4)), rng.standard_normal((4, 3)), rng.standard_normal(3) * 3
    r = oracle.route(x, Wr, b, 3)
    assert np.allclose(r.w, softmax(x @ Wr + b, axis=1), rtol=1e-12)


def _check_shared_mlp():
    """Shared expert alone (all routed weights zero via W2 = 0) equals the plain MLP."""
    import torch

    rng = np.random.default_rng(9)
    T, H, F, E, Fs = 6, 10, 8, 3, 14
    x, Wr = rng.standard_normal((T, H)), rng.standard_normal((H, E))
    W1, W2 = rng.standard_normal((E, H, F)), np.zeros((E, F, H))
    W1s, W2s = rng.standard_normal((H, Fs)), rng.standard_normal((Fs, H))
    y = oracle.forward(x, Wr, None, W1, W2, 2, 0.0, W1s, W2s).y
    ref = torch.nn.functional.silu(torch.from_numpy(x) @ torch.from_numpy(W1s)) @ torch.from_numpy(W2s)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_shared_expert_pin():
    _check_shared_mlp()
    _check_bias_k_equals_E()


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda m: m.__name__)
def test_planted_mistakes(mutation, monkeypatch):
    """Every planted bug in the oracle must make at least one pin fail."""
    checks = ALL_CHECKS + [_check_shared_mlp, _check_bias_k_equals_E,
                           lambda: check_dense_bruteforce(seed=13, drop=0.2, shared=True)]
    with monkeypatch.context() as mp:
        mutation(mp)
        failures = 0
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError):
                failures += 1
        assert failures > 0, f"no pin caught {mutation.__name__}"
