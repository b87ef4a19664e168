"""Plain, slow, obviously correct fp64 definition of one RetrievalAttention
decode step with an exact top-k retrieval. TEST INFRASTRUCTURE ONLY: the
product path never imports this module.

Source pages (cited by title and slide/equation, never by line):

* RetrievalAttention slides (arXiv:2409.10516v3 discussion deck)
  - frame "Sparse attention renormalizes selected tokens": Eq. (1) scores and
    softmax, Eq. (2) renormalised attention over a selected set, and the
    fixed retrieval budget (top-k) used instead of a threshold.
  - frame "The GPU keeps 640 fixed positions": static set W = first 128 +
    last 512 tokens, W and the retrieved set are disjoint, GQA query heads get
    their own indices over shared KV storage.
  - frame "Two local softmax outputs need global weights": the stable partial
    form (m_S, Z_S, o_S) and the merge weights gamma_S, Eqs. (3)-(5).
  - backup frame "the normalization identity": N_S, Z_S, and that merging
    disjoint partials gives the exact softmax on their union.
  - frame "The bottleneck is both storage and KV access": Table 1, KV capacity.
  - frame "Extra experiments show where budget matters": a PyramidKV-style
    per-layer budget (more keys for the lower layers).
  - frame "Prefill queries teach the key graph what matters": prefill
    queries' exact top-k keys, query-key links projected into a key-only
    graph (the RoarGraph idea), searched with each decode query.

Readings of points the pages leave open:

* d in 1/sqrt(d) is the head dimension (128).
* The retrieved set is searched over M = [0, N) minus W, so it never holds a
  W position; k_eff = min(k, |M|).
* Ties at the k-th score go to the lower position; the retrieved indices are
  returned in ascending position order.
* GQA groups are contiguous: query head h reads KV head floor(h / G),
  G = H_q / H_kv. Selection is per query head.
* An empty attended set gives out = 0 and lse = -inf.

Every quantity is float64 after exact widening of the bf16 inputs.
"""

from __future__ import annotations

from fractions import Fraction

import math

import numpy as np

HEAD_DIM = 128

# Token tile for score computation: bounds the fp64 working set (a 1M-token
# layer is 8 GiB as fp64, so K is widened one tile at a time).
_SCORE_TILE = 65536


def as_f64(x) -> np.ndarray:
    """Widen an input array to float64 exactly.

    ``uint16`` arrays are taken as raw bfloat16 bit patterns (the top 16 bits
    of an IEEE binary32), so the widening is exact. Any float array is cast.
    """
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# Sets: RetrievalAttention slides, frame "The GPU keeps 640 fixed positions".
# --------------------------------------------------------------------------

def static_set(N: int, n_sink: int, window: int) -> np.ndarray:
    """W: the first ``n_sink`` and the last ``window`` positions of [0, N).

    The slides fix W as the first 128 plus the last 512 tokens; the two counts
    are parameters here. Returned sorted, without duplicates.
    """
    if N < 0 or n_sink < 0 or window < 0:
        raise ValueError("N, n_sink and window must be non-negative")
    first = np.arange(0, min(n_sink, N), dtype=np.int64)
    last = np.arange(max(N - window, 0), N, dtype=np.int64)
    return np.union1d(first, last)


def selection_domain(N: int, n_sink: int, window: int) -> np.ndarray:
    """M = [0, N) minus W: the positions retrieval may choose from.

    W and the retrieved set are disjoint on the slides, and only retrieved
    KV outside W enters the second partial.
    """
    return np.setdiff1d(np.arange(N, dtype=np.int64), static_set(N, n_sink, window))


# --------------------------------------------------------------------------
# Scores: RetrievalAttention slides, "Sparse attention renormalizes selected
# tokens", Eq. (1): z_i = q_t k_i^T / sqrt(d).
# --------------------------------------------------------------------------

def scores(q, K) -> np.ndarray:
    """z[h, n] = (q[h] . K[n, g(h)]) / sqrt(d) for every cached position n.

    q: [H_q, d]; K: [N, H_kv, d] (logical token order). g(h) = h // G with
    G = H_q / H_kv: GQA query heads share their group's KV storage.
    Returns float64 [H_q, N].
    """
    qf = as_f64(q)
    H_q, d = qf.shape
    Kn = np.asarray(K)
    N, H_kv, d2 = Kn.shape
    if d2 != d:
        raise ValueError("head_dim mismatch between q and K")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    inv_sqrt_d = 1.0 / math.sqrt(d)
    z = np.empty((H_q, N), dtype=np.float64)
    for t0 in range(0, N, _SCORE_TILE):
        t1 = min(N, t0 + _SCORE_TILE)
        Kt = as_f64(Kn[t0:t1])  # [T, H_kv, d]
        for g in range(H_kv):
            qg = qf[g * G:(g + 1) * G]          # the G query heads of group g
            z[g * G:(g + 1) * G, t0:t1] = (qg @ Kt[:, g, :].T) * inv_sqrt_d
    return z


# --------------------------------------------------------------------------
# Exact top-k: the fixed retrieval budget ("usually top-100") of the slides'
# Eq. (2) frame, searched over M ("The GPU keeps 640 fixed positions").
# --------------------------------------------------------------------------

def topk(z_h: np.ndarray, M: np.ndarray, k: int) -> np.ndarray:
    """Omega: the k_eff = min(k, |M|) positions of M with the largest score.

    Ties at the k-th score go to the lower position. Returned ascending.
    """
    if k < 0:
        raise ValueError("k must be non-negative")
    M = np.asarray(M, dtype=np.int64)
    k_eff = min(k, M.size)
    if k_eff == 0:
        return np.zeros(0, dtype=np.int64)
    zM = z_h[M]
    # the k_eff-th largest score over M
    t = np.partition(zM, M.size - k_eff)[M.size - k_eff]
    above = M[zM > t]
    equal = M[zM == t]                    # ascending, because M is
    take = k_eff - above.size
    return np.sort(np.concatenate([above, equal[:take]]))


# --------------------------------------------------------------------------
# Partials and merge: "Two local softmax outputs need global weights",
# Eqs. (3)-(5), and the backup frame "the normalization identity".
# --------------------------------------------------------------------------

def partial(z_h: np.ndarray, V_g, S) -> tuple[float, float, np.ndarray]:
    """(m_S, Z_S, N_S) for one head over the index set S.

    m_S = max_{i in S} z_i; Z_S = sum e^{z_i - m_S};
    N_S = sum e^{z_i - m_S} v_i (so o_S = N_S / Z_S).
    V_g: [N, d] values of the head's KV group. Empty S gives (-inf, 0, 0).
    """
    S = np.asarray(S, dtype=np.int64)
    Vf = as_f64(V_g[S]) if S.size else np.zeros((0, np.asarray(V_g).shape[-1]))
    if S.size == 0:
        return -math.inf, 0.0, np.zeros(Vf.shape[-1], dtype=np.float64)
    zs = z_h[S]
    m = float(zs.max())
    e = np.exp(zs - m)
    return m, float(e.sum()), e @ Vf


def merge(parts) -> tuple[np.ndarray, float]:
    """Combine disjoint partials: m = max_S m_S, weights e^{m_S - m}.

    o = sum_S e^{m_S-m} N_S / sum_S e^{m_S-m} Z_S, which equals
    sum_S gamma_S o_S with gamma_S = e^{m_S-m} Z_S / sum_T e^{m_T-m} Z_T.
    Returns (o, lse) with lse = m + ln sum_S e^{m_S-m} Z_S. No non-empty
    partial gives (0, -inf).
    """
    parts = list(parts)
    d = parts[0][2].shape[-1] if parts else HEAD_DIM
    parts = [p for p in parts if p[1] > 0.0]
    if not parts:
        return np.zeros(d, dtype=np.float64), -math.inf
    m = max(p[0] for p in parts)
    num = sum(math.exp(p[0] - m) * p[2] for p in parts)
    den = sum(math.exp(p[0] - m) * p[1] for p in parts)
    return num / den, m + math.log(den)


def attend(z_h: np.ndarray, V_g, S) -> tuple[np.ndarray, float]:
    """Eq. (2): softmax over the selected set S, renormalised on S, times V.

    o = sum_{i in S} e^{z_i} / sum_{j in S} e^{z_j} * v_i, computed with the
    max subtracted. Returns (o [d], lse). Empty S gives (zeros, -inf).
    """
    d = np.asarray(V_g).shape[-1]
    S = np.asarray(S, dtype=np.int64)
    if S.size == 0:
        return np.zeros(d, dtype=np.float64), -math.inf
    zs = z_h[S]
    m = float(zs.max())
    e = np.exp(zs - m)
    den = float(e.sum())
    p = e / den
    return p @ as_f64(V_g[S]), m + math.log(den)


def dense(z_h: np.ndarray, V_g) -> tuple[np.ndarray, float]:
    """Eq. (1): full softmax attention over every cached position."""
    return attend(z_h, V_g, np.arange(z_h.shape[0], dtype=np.int64))


# --------------------------------------------------------------------------
# One decode step.
# --------------------------------------------------------------------------

def decode_head(z_h: np.ndarray, V_g, W: np.ndarray, M: np.ndarray, k: int):
    """One query head: Omega = top-k over M, then attention over W u Omega.

    Also returns the two-partial merge (W, Omega) of Eqs. (3)-(5), which must
    equal the direct softmax over the union.
    """
    omega = topk(z_h, M, k)
    S = np.union1d(W, omega)
    o, lse = attend(z_h, V_g, S)
    o_m, lse_m = merge([partial(z_h, V_g, W), partial(z_h, V_g, omega)])
    return omega, o, lse, o_m, lse_m


def decode(q, K, V, k: int, n_sink: int, window: int, with_dense: bool = False):
    """One decode step for one sequence (all query heads).

    q: [H_q, d]; K, V: [N, H_kv, d] in logical order (N = length after the
    new token was appended, so the recent window includes it).
    Returns a dict with float64 ``z`` [H_q, N], ``out`` [H_q, d], ``lse``
    [H_q], the merged-partials ``out_merge``/``lse_merge``, and ``idx``: a
    list of ascending int64 arrays (one per head, length k_eff). With
    ``with_dense`` also the dense output and the attention mass recovered
    (sum of full-softmax weights over W u Omega, the Fig. 2 metric).
    """
    Kn = np.asarray(K)
    Vn = np.asarray(V)
    N, H_kv, d = Kn.shape
    qf = as_f64(q)
    H_q = qf.shape[0]
    G = H_q // H_kv
    z = scores(qf, Kn)
    W = static_set(N, n_sink, window)
    M = selection_domain(N, n_sink, window)
    out = np.zeros((H_q, d))
    out_m = np.zeros((H_q, d))
    lse = np.zeros(H_q)
    lse_m = np.zeros(H_q)
    idx = []
    dense_out = np.zeros((H_q, d)) if with_dense else None
    mass = np.zeros(H_q) if with_dense else None
    for h in range(H_q):
        Vg = Vn[:, h // G, :]
        om, o, l, o2, l2 = decode_head(z[h], Vg, W, M, k)
        idx.append(om)
        out[h], lse[h] = o, l
        out_m[h] = o2
        lse_m[h] = l2
        if with_dense:
            dense_out[h], l_all = dense(z[h], Vg)
            S = np.union1d(W, om)
            mass[h] = float(np.exp(z[h][S] - l_all).sum()) if S.size else 0.0
    res = dict(z=z, out=out, lse=lse, out_merge=out_m, lse_merge=lse_m, idx=idx,
               W=W, M=M)
    if with_dense:
        res["dense_out"] = dense_out
        res["mass_recovered"] = mass
    return res


# --------------------------------------------------------------------------
# Prefill: "Prefill queries teach the key graph what matters", step 1: the
# prefill queries find their exact top-k keys on the GPU, and each query is
# then linked to those keys to build the key graph. The keys the graph
# indexes are the members of M (W stays on the GPU), and a query is linked to
# the best keys of the whole domain (no causal cut: the links describe which
# keys a query finds important, not an attention step).
# --------------------------------------------------------------------------

def prefill_topk(Q, K, k: int, n_sink: int, window: int) -> np.ndarray:
    """Exact top-k keys of every prefill query row and query head.

    Q: [T, H_q, d]; K: [N, H_kv, d] in logical order. For row t and head h
    the scores are Eq. (1) against every key (``scores`` of that row), and
    the selection is ``topk`` over M. Returns int64 [T, H_q, k] with each
    row's k_eff positions ascending, padded with -1.
    """
    Qn = np.asarray(Q)
    T, H_q, _ = Qn.shape
    N = np.asarray(K).shape[0]
    M = selection_domain(N, n_sink, window)
    out = np.full((T, H_q, k), -1, dtype=np.int64)
    for t in range(T):
        z = scores(Qn[t], K)
        for h in range(H_q):
            sel = topk(z[h], M, k)
            out[t, h, :sel.size] = sel
    return out


# --------------------------------------------------------------------------
# KV sizing: "The bottleneck is both storage and KV access", Table 1.
# --------------------------------------------------------------------------

def kv_bytes_per_token(n_layers: int, H_kv: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V per cached token across all layers: 2*L*H_kv*d*b."""
    return 2 * n_layers * H_kv * head_dim * elem_bytes


# --------------------------------------------------------------------------
# Per-layer budgets: "Extra experiments show where budget matters" (a
# PyramidKV-style layer budget). The slides give no formula; the reading
# here is a budget falling linearly with depth that keeps the total of the
# uniform budget.
# --------------------------------------------------------------------------

def layer_budgets(n_layers: int, k_mean: int, slope_permille: int) -> list:
    """Integer budgets k_0 >= ... >= k_{L-1} summing to L * k_mean.

    The exact budget of layer l is k_mean * (1 + s * (L-1-2l) / (L-1)),
    s = slope_permille / 1000 (a straight line through k_mean at the middle
    layer; s = 0 is uniform). Each layer gets its floor; the layers with
    the largest fractional parts get one more until the total is reached,
    ties to the lower layer.
    """
    L = int(n_layers)
    if L == 1:
        return [int(k_mean)]
    s = Fraction(int(slope_permille), 1000)
    exact = [Fraction(int(k_mean)) * (1 + s * Fraction(L - 1 - 2 * l, L - 1)) for l in range(L)]
    ks = [math.floor(x) for x in exact]
    short = L * int(k_mean) - sum(ks)
    by_fraction = sorted(range(L), key=lambda l: (-(exact[l] - ks[l]), l))
    for l in by_fraction[:short]:
        ks[l] += 1
    return ks


# --------------------------------------------------------------------------
# Query-aware key graph: "Prefill queries teach the key graph what matters"
# (steps 2-4: link each prefill query to its exact top keys, project the
# links into a key-only graph, search it with each decode query). The
# slides give the steps, not their parameters; the readings here are the
# plainest deterministic ones.
# --------------------------------------------------------------------------

def score_f32_ordered(q, K, positions) -> np.ndarray:
    """Scores of one query against the keys at ``positions`` as a graph
    search compares them: q . k in fp32, the (exact) products of the bf16
    inputs added one dimension after another, 0 to d-1, each sum rounded to
    fp32. The search only ranks keys, so the positive factor 1/sqrt(d) is
    left out. q: [d] raw bf16 bits; K: [N, d] raw bf16 bits (one KV head)."""
    qf = (np.asarray(q).astype(np.uint32) << np.uint32(16)).view(np.float32)
    P = np.asarray(positions, dtype=np.int64)
    Kf = (np.asarray(K)[P].astype(np.uint32) << np.uint32(16)).view(np.float32)
    s = np.zeros(P.size, dtype=np.float32)
    for i in range(qf.size):
        s = (s + Kf[:, i] * qf[i]).astype(np.float32)
    return s


def graph_build(hubs, lists, N: int, D: int):
    """Key-only graph from prefill query-key links.

    hubs[t]: the best key of prefill query t (-1: none); lists[t]: its top
    keys (-1 padded). For t = 0, 1, ... and each other key b of lists[t] in
    ascending position, the hub and b are linked both ways. A key keeps its
    first D distinct neighbours. The entry point is the key that is the hub
    of the most queries (ties to the lower position), -1 if there is none.
    Returns (nbr int64 [N, D] padded with -1, entry).
    """
    nbr = [[] for _ in range(N)]

    def link(a, b):
        if a != b and len(nbr[a]) < D and b not in nbr[a]:
            nbr[a].append(b)

    hub_count = {}
    for t, a in enumerate(np.asarray(hubs).tolist()):
        if a < 0:
            continue
        hub_count[a] = hub_count.get(a, 0) + 1
        for b in sorted(x for x in np.asarray(lists[t]).tolist() if x >= 0):
            if b != a:
                link(a, b)
                link(b, a)
    out = np.full((N, D), -1, dtype=np.int64)
    for a in range(N):
        out[a, :len(nbr[a])] = nbr[a]
    entry = min(hub_count, key=lambda a: (-hub_count[a], a)) if hub_count else -1
    return out, entry


def graph_search(q, K, nbr, entry: int, ef: int, k: int, batch: int = 1,
                 scoring: str = "f32", trace=None):
    """Best-first search of the key graph with one decode query.

    A result list R keeps the ef best visited keys by (score, lower
    position). Starting from the entry point, each round expands the
    ``batch`` best keys of R not yet expanded (fewer if fewer are left):
    every neighbour of theirs not visited before is visited, scored and
    offered to R. The search ends when every key in R has been expanded.
    Returns (the best min(k, |R|) keys of R in ascending position, the
    number of keys visited).

    ``scoring``: "f32" ranks by ``score_f32_ordered`` (the dimension-by-
    dimension fp32 sum); "f64" by the plain definition, q . k summed in
    float64 after exact widening (Eq. (1) without the 1/sqrt(d), which does
    not change the order). ``trace``: a list that receives, after every
    round, (R as [(key, expanded)] in rank order, the sorted visited keys).
    The batch size and the fp32 order are readings of this build: the frame
    names a best-first search and no parameters.
    """
    if entry < 0:
        return np.zeros(0, dtype=np.int64), 0
    nbr = np.asarray(nbr)
    if scoring == "f32":
        def score(pos):
            return [float(x) for x in score_f32_ordered(q, K, pos)]
    elif scoring == "f64":
        qf = as_f64(q)
        Kf = np.asarray(K)

        def score(pos):
            return [float(x) for x in as_f64(Kf[np.asarray(pos, dtype=np.int64)]) @ qf]
    else:
        raise ValueError(f"unknown scoring {scoring!r}")
    visited = {int(entry)}
    R = [(score([entry])[0], int(entry), False)]
    while True:
        R.sort(key=lambda e: (-e[0], e[1]))
        todo = [i for i, e in enumerate(R) if not e[2]][:batch]
        if not todo:
            break
        new = []
        for i in todo:
            R[i] = (R[i][0], R[i][1], True)
            for u in nbr[R[i][1]]:
                u = int(u)
                if u >= 0 and u not in visited:
                    visited.add(u)
                    new.append(u)
        if new:
            R.extend((x, u, False) for x, u in zip(score(new), new))
            R.sort(key=lambda e: (-e[0], e[1]))
            del R[ef:]
        if trace is not None:
            trace.append(([(e[1], e[2]) for e in R], sorted(visited)))
    best = sorted(e[1] for e in R[:k])
    return np.asarray(best, dtype=np.int64), len(visited)
