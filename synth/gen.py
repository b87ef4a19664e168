"""Seeded generator of one layer's decode-step inputs, in the paged layout.

Distribution (the workloads' description, read plainly):

* u: one random unit vector per layer (d = 128), shared by all heads.
* keys   K ~ N(0, 1) + 0.5 u   (every KV head, every position);
* queries q ~ N(0, 1) - 0.5 u  (so queries are out of distribution with
  respect to keys, the Q-to-K gap of the RetrievalAttention slides, frames
  "Ordinary ANN indices miss Q-to-K neighbors" and "Query and key vectors
  occupy different regions");
* values V ~ N(0, 1).
* Needles: positions drawn uniformly without replacement from the
  selection domain (outside the sink prefix and the recent window), each
  owned by one query head h. A needle key is aligned to its query:
  0.5 u + 0.1 x + (6 / |q_h|) q_h, where x is the N(0, 1) draw the key had.
  Over keys drawn as above, q_h . k / sqrt(d) has mean mu_h = 0.5 q_h . u /
  sqrt(d) and standard deviation sigma_h = |q_h| / sqrt(d), so the needle
  scores mu_h + 6 sigma_h up to a tenth of sigma_h of noise. No score is
  computed here, only the norm |q_h|.
* Sinks: the keys at positions 0..3 are multiplied by 4, after the offset
  and the needles.
* Everything is drawn in fp32 and rounded to bf16 (round to nearest even)
  last.

Structural draws (lengths, page permutation, needle positions) come from a
CPU generator, so they are the same whatever device draws the values.

Paged layout: K and V pools are bf16 [num_pages][H_kv][64][128]; the block
table (int32 [B][max_pages]) maps sequence b's logical page j to a physical
page. Unused table entries are 0.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

PAGE = 64
HEAD_DIM = 128
_CHUNK_TOKENS = 65536  # generation chunk (fixed, so the random stream is too)
_STRUCT_SALT = 0x5EED5EED


@dataclass
class LayerInputs:
    q: torch.Tensor            # bf16 [B][H_q][128]
    k_pool: torch.Tensor       # bf16 [P][H_kv][64][128]
    v_pool: torch.Tensor       # bf16 [P][H_kv][64][128]
    block_table: torch.Tensor  # int32 [B][max_pages]
    seq_lens: list             # per sequence, after the current token
    ks: list                   # per-sequence budget k_b
    n_sink: int
    window: int
    H_q: int
    H_kv: int
    needles: list              # per sequence: int64 [n, 2] rows (position, query head)
    u: torch.Tensor            # fp32 [128], the layer's offset direction

    @property
    def B(self) -> int:
        return len(self.seq_lens)


def draw_lengths(B: int, lo: int, hi: int, seed: int) -> list:
    """B integer lengths uniform in [lo, hi] (inclusive), from a CPU generator."""
    g = torch.Generator().manual_seed(seed ^ _STRUCT_SALT)
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]


def _domain(N: int, n_sink: int, window: int) -> tuple:
    """[lo, hi): the positions outside the first n_sink and last window."""
    lo = min(n_sink, N)
    hi = max(N - window, lo)
    return lo, hi


def make_layer(H_q: int, H_kv: int, seq_lens, ks, n_sink: int, window: int,
               needles_per_head: int, seed: int, device,
               shuffle_pages: bool = False, reserve_tokens: int = 0,
               sink_tokens: int = 4, sink_scale: float = 4.0,
               tail_fill: float = 0.0) -> LayerInputs:
    """Draw one layer's q, K, V for B sequences and lay K, V out in pages.

    ``reserve_tokens`` extra positions per sequence get pages too (for later
    appends); they are zero. ``tail_fill`` is written to the unused slots of
    each sequence's last page.
    """
    d = HEAD_DIM
    B = len(seq_lens)
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    device = torch.device(device)
    dev_gen = torch.Generator(device=device).manual_seed(seed)
    cpu_gen = torch.Generator().manual_seed(seed ^ _STRUCT_SALT)

    # direction u and the queries
    u = torch.randn(d, generator=dev_gen, device=device, dtype=torch.float32)
    u = u / u.norm()
    q32 = torch.randn(B, H_q, d, generator=dev_gen, device=device) - 0.5 * u

    # pages: sequence b owns ceil((N_b + reserve) / 64) logical pages
    pages = [-(-(n + reserve_tokens) // PAGE) for n in seq_lens]
    total = sum(pages)
    max_pages = max(pages)
    phys = (torch.randperm(total, generator=cpu_gen) if shuffle_pages
            else torch.arange(total)).to(torch.int32)
    table = torch.zeros(B, max_pages, dtype=torch.int32)
    off = 0
    for b, p in enumerate(pages):
        table[b, :p] = phys[off:off + p]
        off += p

    # needles: positions and owning query head, per sequence
    needles = []
    for b, n in enumerate(seq_lens):
        lo, hi = _domain(n, n_sink, window)
        cnt = min(needles_per_head * H_q, hi - lo)
        pos = torch.randperm(hi - lo, generator=cpu_gen)[:cnt] + lo
        head = torch.arange(cnt) // max(needles_per_head, 1)
        needles.append(torch.stack([pos, head], 1).numpy().astype(np.int64))

    k_pool = torch.empty(total, H_kv, PAGE, d, dtype=torch.bfloat16, device=device)
    v_pool = torch.empty_like(k_pool)
    table_dev = table.to(device)

    for b, n in enumerate(seq_lens):
        nd = torch.as_tensor(needles[b], device=device)
        coef = 6.0 / q32[b].norm(dim=-1)                 # [H_q]
        for t0 in range(0, n, _CHUNK_TOKENS):
            t1 = min(n, t0 + _CHUNK_TOKENS)
            kc = torch.randn(t1 - t0, H_kv, d, generator=dev_gen, device=device) + 0.5 * u
            if nd.numel():
                sel = (nd[:, 0] >= t0) & (nd[:, 0] < t1)
                if bool(sel.any()):
                    npos = nd[sel, 0] - t0
                    nh = nd[sel, 1]
                    noise = kc[npos, nh // G] - 0.5 * u
                    kc[npos, nh // G] = 0.5 * u + 0.1 * noise + coef[nh, None] * q32[b, nh]
            if t0 == 0 and sink_tokens > 0:
                kc[:min(sink_tokens, t1)] *= sink_scale
            _store(k_pool, table_dev[b], t0, kc, tail_fill)
        for t0 in range(0, n, _CHUNK_TOKENS):
            t1 = min(n, t0 + _CHUNK_TOKENS)
            vc = torch.randn(t1 - t0, H_kv, d, generator=dev_gen, device=device)
            _store(v_pool, table_dev[b], t0, vc, tail_fill)
        # reserve pages for later appends start out zero
        first_free = -(-n // PAGE)
        if pages[b] > first_free:
            ids = table_dev[b, first_free:pages[b]].long()
            k_pool[ids] = 0
            v_pool[ids] = 0

    ks = [int(x) for x in ks]
    return LayerInputs(q=q32.to(torch.bfloat16), k_pool=k_pool, v_pool=v_pool,
                       block_table=table_dev, seq_lens=[int(x) for x in seq_lens],
                       ks=ks, n_sink=n_sink, window=window, H_q=H_q, H_kv=H_kv,
                       needles=needles, u=u)


def _store(pool: torch.Tensor, table_row: torch.Tensor, t0: int, x: torch.Tensor,
           tail_fill: float) -> None:
    """Round x ([T][H_kv][d] fp32, logical positions t0..) to bf16 and write
    it into its pages; the unused slots of a partial last page get tail_fill."""
    T, H_kv, d = x.shape
    np_ = -(-T // PAGE)
    if np_ * PAGE != T:
        pad = torch.full((np_ * PAGE - T, H_kv, d), tail_fill, device=x.device)
        x = torch.cat([x, pad], 0)
    xb = x.to(torch.bfloat16).view(np_, PAGE, H_kv, d).permute(0, 2, 1, 3)
    ids = table_row[t0 // PAGE: t0 // PAGE + np_].long()
    pool[ids] = xb


def make_new_tokens(B: int, H_kv: int, u: torch.Tensor, seed: int, device):
    """One new K row (N(0,1) + 0.5 u) and V row (N(0,1)) per (sequence, KV
    head), bf16 [B][H_kv][128]."""
    g = torch.Generator(device=torch.device(device)).manual_seed(seed)
    k = torch.randn(B, H_kv, HEAD_DIM, generator=g, device=device) + 0.5 * u.to(device)
    v = torch.randn(B, H_kv, HEAD_DIM, generator=g, device=device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def history(pool: torch.Tensor, block_table: torch.Tensor, b: int, N0: int,
            new_rows: torch.Tensor, n: int, heads=None) -> np.ndarray:
    """Logical rows [0, n) of sequence b as raw bf16 bits, from the generator
    alone: rows below N0 from the pool as the generator filled it (the rows
    that decode steps appended sit at N0 and above and are not read back),
    rows N0 .. n - 1 from new_rows ([steps][B][H_kv][128], the stream those
    steps appended). Pure data movement."""
    base = depage(pool, block_table, b, min(n, N0), heads=heads)
    if n <= N0:
        return base
    new = new_rows[:n - N0, b]
    if heads is not None:
        new = new[:, list(heads)]
    return np.concatenate([base, bf16_bits(new)], axis=0)


def make_decode_stream(B: int, H_q: int, H_kv: int, u: torch.Tensor, steps: int, seed: int,
                       device):
    """Inputs of `steps` consecutive decode steps of one layer, drawn like the
    layer's own: per step a query (N(0,1) - 0.5 u, bf16 [B][H_q][128]) and
    one new K row (N(0,1) + 0.5 u) and V row (N(0,1)) per (sequence, KV head).
    Returns (q [steps][B][H_q][128], k_new, v_new [steps][B][H_kv][128])."""
    g = torch.Generator(device=torch.device(device)).manual_seed(seed)
    u = u.to(device)
    q = torch.randn(steps, B, H_q, HEAD_DIM, generator=g, device=device) - 0.5 * u
    k = torch.randn(steps, B, H_kv, HEAD_DIM, generator=g, device=device) + 0.5 * u
    v = torch.randn(steps, B, H_kv, HEAD_DIM, generator=g, device=device)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_prefill_queries(T: int, H_q: int, u: torch.Tensor, seed: int, device) -> torch.Tensor:
    """T prefill query rows of a layer, drawn like its decode queries
    (N(0,1) - 0.5 u): bf16 [T][H_q][128]."""
    g = torch.Generator(device=torch.device(device)).manual_seed(seed)
    q = torch.randn(T, H_q, HEAD_DIM, generator=g, device=device) - 0.5 * u.to(device)
    return q.to(torch.bfloat16)


def make_topic_queries(T: int, H_q: int, u: torch.Tensor, topics_seed: int, n_topics: int,
                       spread: float, seed: int, device) -> torch.Tensor:
    """T query rows drawn around a few shared directions per head: row t of
    head h is topic[h][c] + spread * N(0,1) - 0.5 u with c uniform over
    n_topics and topic ~ N(0,1) drawn from topics_seed, so rows drawn with
    the same topics_seed (prefill rows, later decode queries) resemble each
    other. bf16 [T][H_q][128]."""
    dev = torch.device(device)
    gt = torch.Generator(device=dev).manual_seed(topics_seed)
    topics = torch.randn(H_q, n_topics, HEAD_DIM, generator=gt, device=dev)
    g = torch.Generator(device=dev).manual_seed(seed)
    c = torch.randint(0, n_topics, (T, H_q), generator=g, device=dev)
    base = topics[torch.arange(H_q, device=dev).view(1, H_q), c]        # [T][H_q][128]
    q = base + spread * torch.randn(T, H_q, HEAD_DIM, generator=g, device=dev) - 0.5 * u.to(dev)
    return q.to(torch.bfloat16)


def copy_pages(pool: torch.Tensor, block_table: torch.Tensor, b: int, positions, device):
    """A small pool holding only the pages of sequence b that contain the
    given positions, and a block table [1][max_pages] mapping those pages
    into it (the other entries point at its page 0). Pure data movement."""
    pages = sorted({int(n) // PAGE for n in positions})
    src = block_table[b, pages].long().to(pool.device)
    small = pool[src].to(device).contiguous()
    table = torch.zeros(1, block_table.shape[1], dtype=torch.int32)
    table[0, pages] = torch.arange(len(pages), dtype=torch.int32)
    return small, table.to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor, as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def depage(pool: torch.Tensor, block_table: torch.Tensor, b: int, N: int,
           t0: int = 0, t1: int | None = None, heads=None) -> np.ndarray:
    """Logical rows [t0, t1) of sequence b from a paged pool, as raw bf16
    bits: host uint16 [t1 - t0][H_kv][128] (or only the KV heads listed in
    ``heads``). Pure data movement."""
    t1 = N if t1 is None else t1
    p0, p1 = t0 // PAGE, -(-t1 // PAGE)
    ids = block_table[b, p0:p1].long().to(pool.device)
    x = pool[ids]
    if heads is not None:
        x = x[:, list(heads)]
    x = x.permute(0, 2, 1, 3).reshape((p1 - p0) * PAGE, x.shape[1], pool.shape[3])
    x = x[t0 - p0 * PAGE: t1 - p0 * PAGE]
    return bf16_bits(x)

