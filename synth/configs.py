"""The five workloads, by shape.

C1  tiny: one sequence, H_q=4, H_kv=1, N=4096, k=64, n_sink=16, window=64,
    8 planted needles in total (2 per query head).
C2  one Llama-3-8B layer (H_q=32, H_kv=8, d=128), N=131072, k=2048.
C3  the same layer at N=1048576 with k = 1 %, 2 % or 3 % of N.
C4  16 sequences of that layer shape, lengths uniform in [32768, 131072],
    64-token pages in shuffled physical order, k = 2 % of each length.
C5  32 such layers at N=1048576, k = 1 %, one seed per layer, plus 1000
    decode steps that each append one token per layer.

C2-C5 use n_sink=128, window=512 (the 128 + 512 static positions of the
RetrievalAttention slides, frame "The GPU keeps 640 fixed positions") and 64
needles per query head.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    H_q: int
    H_kv: int
    # Fixed per-sequence lengths, or None when they are drawn (C4).
    seq_lens: tuple | None
    # Budget: an absolute k, or a percentage of each sequence's length.
    k_abs: int | None = None
    k_pct: int | None = None
    n_sink: int = 128
    window: int = 512
    needles_per_head: int = 64
    shuffle_pages: bool = False
    seed: int = 0
    len_range: tuple | None = None  # (lo, hi) inclusive, when lengths are drawn
    n_layers: int = 1
    extra: dict = field(default_factory=dict)

    def k_for(self, n: int) -> int:
        """Per-sequence budget: k_abs, or floor(k_pct * n / 100)."""
        if self.k_abs is not None:
            return self.k_abs
        return (self.k_pct * n) // 100


CONFIGS = {
    "C1": LayerConfig("C1", B=1, H_q=4, H_kv=1, seq_lens=(4096,), k_abs=64,
                      n_sink=16, window=64, needles_per_head=2),
    "C2": LayerConfig("C2", B=1, H_q=32, H_kv=8, seq_lens=(131072,), k_abs=2048),
    "C3_1": LayerConfig("C3_1", B=1, H_q=32, H_kv=8, seq_lens=(1048576,), k_pct=1),
    "C3_2": LayerConfig("C3_2", B=1, H_q=32, H_kv=8, seq_lens=(1048576,), k_pct=2),
    "C3_3": LayerConfig("C3_3", B=1, H_q=32, H_kv=8, seq_lens=(1048576,), k_pct=3),
    "C4": LayerConfig("C4", B=16, H_q=32, H_kv=8, seq_lens=None, k_pct=2,
                      shuffle_pages=True, len_range=(32768, 131072)),
    "C5": LayerConfig("C5", B=1, H_q=32, H_kv=8, seq_lens=(1048576,), k_pct=1,
                      n_layers=32, extra={"steps": 1000}),
}


def config(name: str) -> LayerConfig:
    return CONFIGS[name]
