"""Pins of the oracle's capacity-limited routing (CPU only).

Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 3.2, second
routing pitfall: each expert accepts at most tokens*k/experts*1.2 selections;
an over-capacity expert is set to -inf for the excess tokens, which choose
again. The oracle reads this as serial priority by token id. These pins check
it against things fixed independently of its own loop:

* the capacity formula on the page's example shapes;
* a never-binding capacity reduces to plain top-k routing;
* hand-derived cases;
* a certificate every correct answer satisfies (capacity respected, and every
  selected expert beats every unselected expert that still had room);
* two different algorithms with the same unique answer: deferred acceptance
  (tokens propose to their best experts, experts keep the lowest token ids up
  to capacity, rejected tokens propose again) and a fixed-point iteration on
  the token index at which each expert fills;
* planted mistakes in the oracle, each caught by at least one of the above.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import moe_oracle  # noqa: E402


# ----------------------------------------------------- independent algorithms --
def deferred_acceptance(logits, k, cap):
    """Tokens propose to their best not-yet-rejecting experts; every expert keeps
    the cap lowest token ids among its proposers and rejects the rest; repeat."""
    T, E = logits.shape
    pref = [sorted(range(E), key=lambda e: (-logits[t, e], e)) for t in range(T)]
    nxt = [0] * T
    held = [set() for _ in range(T)]
    pool = [set() for _ in range(E)]
    while True:
        changed = False
        for t in range(T):
            while len(held[t]) < k:
                e = pref[t][nxt[t]]
                nxt[t] += 1
                held[t].add(e)
                pool[e].add(t)
                changed = True
        for e in range(E):
            if len(pool[e]) > cap:
                for t in sorted(pool[e])[cap:]:
                    pool[e].discard(t)
                    held[t].discard(e)
                changed = True
        if not changed:
            break
    return np.array([sorted(h) for h in held], dtype=np.int64)


def fixed_point_cutoffs(logits, k, cap):
    """tau[e] = first token index for which expert e is no longer available;
    start at T, select with t < tau, recompute where each expert reaches cap,
    repeat until tau stops moving."""
    T, E = logits.shape
    tau = np.full(E, T)
    while True:
        avail = np.arange(T)[:, None] < tau[None, :]
        L = np.where(avail, logits, -np.inf)
        order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -L), axis=1)[:, :k]
        sel = np.sort(order, axis=1)
        new = tau.copy()
        for e in range(E):
            toks = np.nonzero((sel == e).any(axis=1))[0]
            if len(toks) > cap:
                new[e] = min(new[e], toks[cap - 1] + 1)
        if np.array_equal(new, tau):
            return sel
        tau = new


def certificate_ok(logits, ids, k, cap):
    T, E = logits.shape
    count = np.zeros(E, dtype=np.int64)
    for t in range(T):
        row = ids[t]
        if len(set(row.tolist())) != k or not np.all(np.diff(row) > 0):
            return False
        room = count < cap
        if not room[row].all():
            return False
        sel = np.zeros(E, dtype=bool)
        sel[row] = True
        for e in np.nonzero(room & ~sel)[0]:
            for s in row:  # s must be preferred to e: larger logit, or equal with a lower id
                if logits[t, s] < logits[t, e] or (logits[t, s] == logits[t, e] and s > e):
                    return False
        count[row] += 1
    return bool((count <= cap).all())


def skewed_logits(rng, T, E, hot=3, boost=2.0):
    lg = rng.standard_normal((T, E))
    lg[:, :hot] += boost  # a few experts everybody wants
    return lg


# ------------------------------------------------------------------- pins --
def check_capacity_formula():
    # tokens*k/experts*1.2 rounded up: 8192*8/128*1.2 = 614.4 -> 615; 32*8/128*1.2 = 2.4 -> 3
    assert oracle.capacity_slots(8192, 8, 128, 1.2) == 615
    assert oracle.capacity_slots(32, 8, 128, 1.2) == 3
    assert oracle.capacity_slots(2048, 2, 64, 1.2) == 77
    assert oracle.capacity_slots(10, 2, 4, 1.0) == 5
    assert oracle.capacity_feasible(64, 2, 4, 39) is False   # at most 3 experts can fill: 1 < k left
    assert oracle.capacity_feasible(2048, 2, 64, 77) is True


def check_never_binding_is_plain_topk(seed=11):
    rng = np.random.default_rng(seed)
    T, E, k = 50, 8, 3
    lg = rng.standard_normal((T, E))
    ids = oracle.select_capacity(lg, k, T)  # an expert can take every token
    ref, _ = oracle.select_topk(lg, k)
    assert np.array_equal(ids, ref)
    x = rng.standard_normal((T, 16))
    Wr = rng.standard_normal((16, E))
    a = oracle.route_capacity(x, Wr, None, k, 0.1, E / k)  # factor E/k: capacity T
    b = oracle.route(x, Wr, None, k, 0.1)
    assert np.array_equal(a.ids, b.ids) and np.allclose(a.w, b.w, rtol=0, atol=1e-15)


def check_hand_cases():
    lg = np.array([[3.0, 2.0, 1.0]] * 4)
    assert oracle.select_capacity(lg, 1, 2).ravel().tolist() == [0, 0, 1, 1]
    lg = np.array([[4.0, 3.0, 2.0, 1.0]] * 3)
    assert oracle.select_capacity(lg, 2, 2).tolist() == [[0, 1], [0, 1], [2, 3]]
    # priority by token id: token 0 keeps its first choice even though token 1 wants it more
    lg = np.array([[1.0, 0.0], [9.0, 0.0]])
    assert oracle.select_capacity(lg, 1, 1).ravel().tolist() == [0, 1]
    # equal logits among the experts with room: the lower id wins
    lg = np.array([[5.0, 2.0, 2.0, 2.0], [5.0, 2.0, 2.0, 2.0]])
    assert oracle.select_capacity(lg, 2, 1).tolist() == [[0, 1], [2, 3]]


def check_certificate_random(seed=12):
    rng = np.random.default_rng(seed)
    for T, E, k, f in [(40, 6, 2, 1.2), (100, 16, 4, 1.1), (64, 8, 1, 1.0), (30, 10, 3, 1.5)]:
        lg = skewed_logits(rng, T, E)
        cap = oracle.capacity_slots(T, k, E, f)
        ids = oracle.select_capacity(lg, k, cap)
        assert certificate_ok(lg, ids, k, cap), (T, E, k, f)


def check_equals_deferred_acceptance(seed=13):
    rng = np.random.default_rng(seed)
    for T, E, k, f in [(40, 6, 2, 1.2), (60, 8, 3, 1.2), (25, 5, 1, 1.0), (80, 16, 4, 1.1)]:
        lg = skewed_logits(rng, T, E, hot=2, boost=3.0)
        cap = oracle.capacity_slots(T, k, E, f)
        assert np.array_equal(oracle.select_capacity(lg, k, cap), deferred_acceptance(lg, k, cap)), (T, E, k, f)


def check_equals_fixed_point(seed=14):
    rng = np.random.default_rng(seed)
    for T, E, k, f in [(200, 16, 2, 1.2), (120, 12, 4, 1.2), (300, 8, 1, 1.05)]:
        lg = skewed_logits(rng, T, E, hot=4, boost=1.5)
        cap = oracle.capacity_slots(T, k, E, f)
        assert np.array_equal(oracle.select_capacity(lg, k, cap), fixed_point_cutoffs(lg, k, cap)), (T, E, k, f)


def check_capacity_gaps():
    lg = np.array([[3.0, 2.0, 1.0]] * 4)
    ids = oracle.select_capacity(lg, 1, 2)
    g = oracle.capacity_gaps(lg, ids, 2)
    assert g.tolist() == [1.0, 1.0, 1.0, np.inf] or g.tolist() == [1.0, 1.0, 1.0, 1.0]
    # tokens 2 and 3 choose between experts 1 and 2 (expert 0 is full): gap 2 - 1 = 1
    assert g[2] == 1.0 and g[3] == 1.0


PINS = [check_capacity_formula, check_never_binding_is_plain_topk, check_hand_cases, check_certificate_random,
        check_equals_deferred_acceptance, check_equals_fixed_point, check_capacity_gaps]


@pytest.mark.parametrize("check", PINS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


# --------------------------------------------------------- planted mistakes --
_orig = moe_oracle.select_capacity


def _mut_off_by_one(logits, k, cap):
    return _orig(logits, k, cap + 1)  # lets an expert take cap + 1


def _mut_reverse_priority(logits, k, cap):
    return _orig(logits[::-1], k, cap)[::-1]  # the highest token id chooses first


def _mut_no_capacity(logits, k, cap):
    return _orig(logits, k, logits.shape[0])


def _mut_tie_high(logits, k, cap):
    E = logits.shape[1]
    return (E - 1 - _orig(logits[:, ::-1], k, cap))[:, ::-1]  # ties to the higher id


@pytest.mark.parametrize("mutation", [_mut_off_by_one, _mut_reverse_priority, _mut_no_capacity, _mut_tie_high],
                         ids=lambda f: f.__name__)
def test_planted_mistakes(mutation, monkeypatch):
    """Every planted bug in the oracle's capacity routing makes at least one pin fail."""
    failed = []
    with monkeypatch.context() as mp:
        mp.setattr(moe_oracle, "select_capacity", mutation)
        mp.setattr(oracle, "select_capacity", mutation)
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"{mutation.__name__} survived every pin"
