"""Shared helpers for the GPU parity tests: run the HIP path through the C
ABI binding, run the fp64 oracle on the same seeded inputs, and compare with
the stated tolerances.

Tolerances:
* scores: |z_gpu - z| <= gamma_130 * sum_j |q_j k_j| / sqrt(128) + 2^-23 |z|,
  the fp32 dot-product bound (bf16 products are exact in fp32; 128 terms,
  plus the scale multiply), gamma_n = n u / (1 - n u), u = 2^-24.
* indices: exact, except positions whose oracle score lies within
  1e-3 |z_(k)| + eps_h of the oracle's k-th score z_(k); eps_h is the score
  bound above for the head's largest |q| . |k| (an added floor that matters
  only when z_(k) is near 0). Inside that band the GPU set must still be a
  valid top-k: right size, inside M, no duplicates, ascending.
* outputs: |o_gpu - o| <= 2e-3 + 1e-2 |o| elementwise, same for lse.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth
import top_sparse_attention_gqa_amd as ra

U32 = 2.0 ** -24


def gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class Run:
    """Outputs of one decode step on the GPU, as host arrays."""

    def __init__(self, out, lse, idx, scores=None, rescanned=0):
        self.out, self.lse, self.idx, self.scores = out, lse, idx, scores
        self.rescanned = rescanned  # heads decided by the full rescan


def gpu_decode(L: synth.LayerInputs, max_seq_len: int | None = None, k_max: int | None = None,
               with_scores: bool = False, ks=None, n_sink=None, window=None) -> Run:
    dev = L.q.device
    B, H_q = L.q.shape[0], L.q.shape[1]
    max_seq_len = max_seq_len or max(L.seq_lens)
    ks = list(L.ks if ks is None else ks)
    k_max = max(ks) if k_max is None else k_max
    n_sink = L.n_sink if n_sink is None else n_sink
    window = L.window if window is None else window
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor(L.seq_lens, dtype=torch.int32, device=dev)
    kt = torch.tensor(ks, dtype=torch.int32, device=dev)
    out = torch.full((B, H_q, 128), float("nan"), device=dev)
    lse = torch.full((B, H_q), float("nan"), device=dev)
    idx = torch.full((B, H_q, max(k_max, 1)), -7, dtype=torch.int32, device=dev)
    ws = ra.alloc_workspace(B, H_q, L.H_kv, max_seq_len, k_max, device=dev)
    ws.fill_(0xA5)  # no initial contents are required
    ra.decode_step_ex(L.q, kv, seq, max_seq_len, kt, k_max, n_sink, window, out, lse,
                   idx if k_max else None, ws, keep_scores=with_scores)
    # the score rows hold W and (kept) the retrieved positions after the step
    sc = ra.scores_view(ws, B, H_q, L.H_kv, max_seq_len, k_max).clone() if with_scores else None
    torch.cuda.synchronize()
    return Run(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
               idx.cpu().numpy()[:, :, :k_max],
               sc.cpu().numpy() if sc is not None else None,
               ra.rescan_count(ws, B, H_q, L.H_kv, max_seq_len, k_max))


def host_seq(L: synth.LayerInputs, b: int, kv_heads=None, appended=None):
    """q bits [H_q][128], K and V bits [N][H_kv][128] of sequence b (only the
    KV heads listed in kv_heads, if given). appended = (N0, k_rows, v_rows):
    the rows at N0 and past it were appended by decode steps on the GPU; the
    oracle takes them from the generator's streams instead of the pools."""
    n = L.seq_lens[b]
    if appended is not None:
        N0, kr, vr = appended
        return (synth.bf16_bits(L.q[b]),
                synth.history(L.k_pool, L.block_table, b, N0, kr, n, heads=kv_heads),
                synth.history(L.v_pool, L.block_table, b, N0, vr, n, heads=kv_heads))
    return (synth.bf16_bits(L.q[b]), synth.depage(L.k_pool, L.block_table, b, n, heads=kv_heads),
            synth.depage(L.v_pool, L.block_table, b, n, heads=kv_heads))


def score_bound(q_bits, K_bits) -> np.ndarray:
    """Per (h, n) fp32 error bound of the GPU score: [H_q][N]."""
    qa = np.abs(oracle.as_f64(q_bits))
    Ka = np.abs(oracle.as_f64(K_bits))
    H_q, H_kv = qa.shape[0], Ka.shape[1]
    G = H_q // H_kv
    s = np.empty((H_q, Ka.shape[0]))
    for g in range(H_kv):
        s[g * G:(g + 1) * G] = qa[g * G:(g + 1) * G] @ Ka[:, g, :].T
    s /= math.sqrt(128)
    return s


def check_scores(z_gpu_row, z64, bound, positions) -> None:
    """Scores the GPU kept (W and the retrieved set) within the fp32 bound."""
    pos = np.asarray(positions, dtype=np.int64)
    if pos.size == 0:
        return
    err = np.abs(z_gpu_row[pos].astype(np.float64) - z64[pos])
    lim = gamma(130) * bound[pos] + 2.0 ** -23 * np.abs(z64[pos])
    bad = err > lim
    assert not bad.any(), f"{bad.sum()} scores outside the fp32 bound, worst {err.max():.3e}"


def check_indices(gpu_row: np.ndarray, res: dict, h: int, k: int, eps_h: float) -> int:
    """Compare one head's GPU index row with the oracle; returns the number
    of band differences (0 when the sets are equal)."""
    M = res["M"]
    ref = res["idx"][h]
    k_eff = min(k, M.size)
    assert ref.size == k_eff
    sel = gpu_row[:k_eff]
    assert np.all(gpu_row[k_eff:] == -1), "padding after k_eff must be -1"
    assert np.all(np.diff(sel) > 0), "indices must be ascending and unique"
    if k_eff == 0:
        return 0
    assert np.all(np.isin(sel, M)), "indices must lie in M"
    if np.array_equal(sel, ref):
        return 0
    z = res["z"][h]
    zk = z[ref].min()
    band = np.abs(z - zk) <= 1e-3 * abs(zk) + eps_h
    out_g = sel[~band[sel]]
    out_r = ref[~band[ref]]
    assert np.array_equal(out_g, out_r), (
        f"head {h}: sets differ outside the tie band ({np.setdiff1d(sel, ref)[:8]} vs "
        f"{np.setdiff1d(ref, sel)[:8]})")
    return int(np.setdiff1d(sel, ref).size)


def check_out(o_gpu, o_ref, what="out") -> None:
    err = np.abs(o_gpu - o_ref)
    lim = 2e-3 + 1e-2 * np.abs(o_ref)
    both_inf = np.isinf(o_ref) & (o_gpu == o_ref)
    bad = (err > lim) & ~both_inf
    assert not bad.any(), f"{what}: {bad.sum()} elements outside tolerance, worst abs {np.nanmax(err[~both_inf]) if (~both_inf).any() else 0:.3e}"


def compare_sequence(L: synth.LayerInputs, run: Run, b: int, heads=None, ks=None,
                     n_sink=None, window=None, check_score_rows=True, appended=None) -> dict:
    """Oracle for sequence b and full comparison (appended: see host_seq).
    Returns stats."""
    k = (L.ks if ks is None else ks)[b]
    n_sink = L.n_sink if n_sink is None else n_sink
    window = L.window if window is None else window
    if heads is not None:
        G = L.H_q // L.H_kv
        grp = sorted({h // G for h in heads})
        assert len(grp) == 1, "sampled heads must share one KV head"
        q, K, V = host_seq(L, b, kv_heads=grp, appended=appended)
        q = q[heads]
    else:
        q, K, V = host_seq(L, b, appended=appended)
        heads = list(range(L.H_q))
    res = oracle.decode(q, K, V, k=k, n_sink=n_sink, window=window)
    bound = score_bound(q, K)
    eps = gamma(130) * bound.max(axis=1)
    band_diffs = 0
    for i, h in enumerate(heads):
        band_diffs += check_indices(run.idx[b, h], res, i, k, eps[i])
        if run.scores is not None and check_score_rows:
            sel = run.idx[b, h]
            check_scores(run.scores[b, h], res["z"][i], bound[i],
                         np.union1d(res["W"], sel[sel >= 0]))
        check_out(run.out[b, h], res["out"][i], f"out[b={b},h={h}]")
        check_out(np.array([run.lse[b, h]]), np.array([res["lse"][i]]), f"lse[b={b},h={h}]")
    return {"band_diffs": band_diffs, "res": res}
