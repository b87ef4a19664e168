"""Plant plausible mistakes in the oracle (CPU only) and check that at least
one pin in test_oracle_pins.py fails for each: the pins are strong enough
to catch a dropped term, a wrong sign or index, or a transposed operand."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ra_oracle as ro
import tests.test_oracle_pins as pins


_REAL_SCORES = ro.scores
_REAL_TOPK = ro.topk


def _scores_no_scale(q, K):
    return _REAL_SCORES(q, K) * math.sqrt(ro.HEAD_DIM)


def _scores_wrong_group(q, K):
    qf = ro.as_f64(q)
    Kf = ro.as_f64(K)
    H_q = qf.shape[0]
    H_kv = Kf.shape[1]
    z = np.empty((H_q, Kf.shape[0]))
    for h in range(H_q):
        z[h] = Kf[:, h % H_kv, :] @ qf[h] / math.sqrt(ro.HEAD_DIM)
    return z


def _topk_smallest(z_h, M, k):
    return _REAL_TOPK(-z_h, M, k)


def _topk_ties_high(z_h, M, k):
    M = np.asarray(M, dtype=np.int64)
    k_eff = min(k, M.size)
    if k_eff == 0:
        return np.zeros(0, dtype=np.int64)
    zM = z_h[M]
    t = np.partition(zM, M.size - k_eff)[M.size - k_eff]
    above = M[zM > t]
    equal = M[zM == t][::-1]
    return np.sort(np.concatenate([above, equal[:k_eff - above.size]]))


def _static_off_by_one(N, n_sink, window):
    first = np.arange(0, min(n_sink, N))
    last = np.arange(max(N - window - 1, 0), N)
    return np.union1d(first, last).astype(np.int64)


def _merge_no_rescale(parts):
    parts = [p for p in parts if p[1] > 0.0]
    if not parts:
        return np.zeros(ro.HEAD_DIM), -math.inf
    num = sum(p[2] for p in parts)
    den = sum(p[1] for p in parts)
    m = max(p[0] for p in parts)
    return num / den, m + math.log(den)


def _attend_no_renorm(z_h, V_g, S):
    S = np.asarray(S, dtype=np.int64)
    if S.size == 0:
        return np.zeros(np.asarray(V_g).shape[-1]), -math.inf
    e = np.exp(z_h[S])
    return e @ ro.as_f64(V_g[S]), float(np.log(e.sum()))


_REAL_ATTEND = ro.attend


def _attend_transposed_v(z_h, V_g, S):
    o, l = _REAL_ATTEND(z_h, V_g, S)
    return o[::-1].copy(), l


_REAL_PREFILL = ro.prefill_topk


def _prefill_rows_reversed(Q, K, k, n_sink, window):
    return _REAL_PREFILL(np.asarray(Q)[::-1].copy(), K, k, n_sink, window)


def _prefill_whole_range(Q, K, k, n_sink, window):
    # searches all of [0, N) instead of M
    return _REAL_PREFILL(Q, K, k, 0, 0)


_REAL_BUDGETS = ro.layer_budgets


def _budgets_rising(L, k, slope):
    # more keys for the upper layers instead of the lower ones
    return _REAL_BUDGETS(L, k, slope)[::-1]


def _budgets_floor_only(L, k, slope):
    # the rounding that restores the total is dropped
    if L == 1:
        return [k]
    s = Fraction(slope, 1000)
    return [math.floor(Fraction(k) * (1 + s * Fraction(L - 1 - 2 * l, L - 1))) for l in range(L)]


def _budgets_ties_high(L, k, slope):
    # extra units go to the higher layer on equal fractional parts
    if L == 1:
        return [k]
    s = Fraction(slope, 1000)
    exact = [Fraction(k) * (1 + s * Fraction(L - 1 - 2 * l, L - 1)) for l in range(L)]
    ks = [math.floor(x) for x in exact]
    order = sorted(range(L), key=lambda l: (-(exact[l] - ks[l]), -l))
    for l in order[:L * k - sum(ks)]:
        ks[l] += 1
    return ks


_REAL_BUILD = ro.graph_build
_REAL_SEARCH = ro.graph_search
_REAL_F32 = ro.score_f32_ordered


def _build_one_way(hubs, lists, N, D):
    # only hub -> key links, no way back
    nbr = [[] for _ in range(N)]
    for t, a in enumerate(np.asarray(hubs).tolist()):
        if a < 0:
            continue
        for b in sorted(x for x in np.asarray(lists[t]).tolist() if x >= 0):
            if b != a and len(nbr[a]) < D and b not in nbr[a]:
                nbr[a].append(b)
    out = np.full((N, D), -1, dtype=np.int64)
    for a in range(N):
        out[a, :len(nbr[a])] = nbr[a]
    return out, _REAL_BUILD(hubs, lists, N, D)[1]


def _search_worst_first(q, K, nbr, entry, ef, k, batch=1, scoring="f32", trace=None):
    # ranks the keys upside down (the worst first)
    return _REAL_SEARCH(np.asarray(q) ^ np.uint16(0x8000), K, nbr, entry, ef, k, batch,
                        scoring, trace)


def _search_one_per_round(q, K, nbr, entry, ef, k, batch=1, scoring="f32", trace=None):
    # ignores the batch: one key expanded per round
    return _REAL_SEARCH(q, K, nbr, entry, ef, k, 1, scoring, trace)


def _score_fn(q, K, scoring):
    if scoring == "f64":
        return lambda pos: [float(x) for x in ro.as_f64(np.asarray(K)[np.asarray(pos)]) @ ro.as_f64(q)]
    return lambda pos: [float(x) for x in ro.score_f32_ordered(q, K, pos)]


def _search_merge_before_marking(q, K, nbr, entry, ef, k, batch=1, scoring="f32", trace=None):
    # picks a round's keys one at a time, each after the previous key's new
    # neighbours were merged into R (so a new key can join the same round)
    if entry < 0:
        return np.zeros(0, dtype=np.int64), 0
    score = _score_fn(q, K, scoring)
    visited = {int(entry)}
    R = [(score([entry])[0], int(entry), False)]
    while True:
        took = 0
        for _ in range(batch):
            R.sort(key=lambda e: (-e[0], e[1]))
            i = next((i for i, e in enumerate(R) if not e[2]), None)
            if i is None:
                break
            took += 1
            R[i] = (R[i][0], R[i][1], True)
            new = [int(u) for u in nbr[R[i][1]] if u >= 0 and int(u) not in visited]
            visited.update(new)
            if new:
                R.extend((x, u, False) for x, u in zip(score(new), new))
                R.sort(key=lambda e: (-e[0], e[1]))
                del R[ef:]
        if not took:
            break
        if trace is not None:
            trace.append(([(e[1], e[2]) for e in R], sorted(visited)))
    return np.asarray(sorted(e[1] for e in R[:k]), dtype=np.int64), len(visited)


def _search_resort_mid_round(q, K, nbr, entry, ef, k, batch=1, scoring="f32", trace=None):
    # re-sorts R after each expansion while the round's remaining keys are
    # still addressed by their positions from before
    if entry < 0:
        return np.zeros(0, dtype=np.int64), 0
    score = _score_fn(q, K, scoring)
    visited = {int(entry)}
    R = [(score([entry])[0], int(entry), False)]
    while True:
        R.sort(key=lambda e: (-e[0], e[1]))
        todo = [i for i, e in enumerate(R) if not e[2]][:batch]
        if not todo:
            break
        for i in todo:
            if i >= len(R):
                continue
            R[i] = (R[i][0], R[i][1], True)
            new = [int(u) for u in nbr[R[i][1]] if u >= 0 and int(u) not in visited]
            visited.update(new)
            R.extend((x, u, False) for x, u in zip(score(new), new))
            R.sort(key=lambda e: (-e[0], e[1]))
            del R[ef:]
        if trace is not None:
            trace.append(([(e[1], e[2]) for e in R], sorted(visited)))
    return np.asarray(sorted(e[1] for e in R[:k]), dtype=np.int64), len(visited)


def _f32_reversed(q, K, positions):
    # adds the dimensions in the opposite order
    return _REAL_F32(np.asarray(q)[::-1].copy(), np.asarray(K)[:, ::-1].copy(), positions)


MUTANTS = {
    "graph_build_one_way": ("graph_build", _build_one_way),
    "graph_search_worst_first": ("graph_search", _search_worst_first),
    "graph_search_one_key_per_round": ("graph_search", _search_one_per_round),
    "graph_search_merge_before_marking": ("graph_search", _search_merge_before_marking),
    "graph_search_resort_mid_round": ("graph_search", _search_resort_mid_round),
    "score_f32_reversed_order": ("score_f32_ordered", _f32_reversed),
    "budgets_rising": ("layer_budgets", _budgets_rising),
    "budgets_floor_only": ("layer_budgets", _budgets_floor_only),
    "budgets_ties_high": ("layer_budgets", _budgets_ties_high),
    "prefill_rows_reversed": ("prefill_topk", _prefill_rows_reversed),
    "prefill_whole_range": ("prefill_topk", _prefill_whole_range),
    "scores_no_scale": ("scores", _scores_no_scale),
    "scores_wrong_group": ("scores", _scores_wrong_group),
    "topk_smallest": ("topk", _topk_smallest),
    "topk_ties_high": ("topk", _topk_ties_high),
    "static_off_by_one": ("static_set", _static_off_by_one),
    "merge_no_rescale": ("merge", _merge_no_rescale),
    "attend_no_renorm": ("attend", _attend_no_renorm),
    "attend_transposed_v": ("attend", _attend_transposed_v),
}

PIN_FUNCS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _run_pins():
    """Run every parameter-free pin; return the number that fail."""
    failed = 0
    for f in PIN_FUNCS:
        params = getattr(f, "pytestmark", [])
        cases = [()]
        for m in params:
            if m.name == "parametrize":
                names = m.args[0]
                cases = [c if isinstance(c, tuple) else (c,) for c in m.args[1]]
        for c in cases:
            try:
                f(*c)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed += 1
    return failed


def test_pins_pass_on_the_real_oracle():
    assert _run_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ro, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    with np.errstate(all="ignore"):
        assert _run_pins() > 0, f"mutant {name} survived every pin"
