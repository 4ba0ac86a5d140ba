"""The five synthetic LSA workloads, as plain data.

Each workload fixes shapes, value ranges and selection budgets. Nothing here
computes anything of the method; tests and the benchmark read these records to
size inputs and to pass parameters to the kernels and to the oracle.

Selection budget names follow the LongCat-2.0 release article (techsir.com),
section "LongCat 稀疏注意力": sink tokens, the streaming-aware (SI) window, the
dynamic top-k, hierarchical (HI) block recall and cross-layer (CLI) reuse.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "hier_decode"
    B: int                    # sequences
    L: int                    # prefill rows == keys; decode: cached context n_k
    H_I: int                  # indexer heads
    d_I: int                  # indexer head dim
    qk_lo: int                # int8 indexer q/k drawn uniform in [qk_lo, qk_hi]
    qk_hi: int
    w_lo: int                 # per-head indexer weights uniform in [w_lo, w_hi]
    w_hi: int
    n_sink: int
    n_window: int
    k_dyn: int                # dynamic top-k on top of sinks + window
    H: int                    # attention query heads (one shared KV head)
    D: int = 128
    n_q: int = 1              # decode: query rows per sequence (target + drafts)
    n_split: int = 1          # decode: split-KV chunks merged by log-sum-exp
    n_layers: int = 1         # CLI: layers sharing one index
    blk: int = 0              # HI block size (0: HI off)
    n_blk_recall: int = 0     # HI coarse recall
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def K_tot(self) -> int:
        return self.n_sink + self.n_window + self.k_dyn

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# C1: tiny prefill, L=4096; total budget 256 = 4 sinks + 64 window + 188 top-k.
C1 = Workload("c1_prefill_4k", "prefill", B=1, L=4096, H_I=4, d_I=64,
              qk_lo=-8, qk_hi=7, w_lo=1, w_hi=4,
              n_sink=4, n_window=64, k_dyn=256 - 4 - 64, H=16)

# C2: prefill L=32768; total budget 2048 = 4 + 512 + 1532.
C2 = Workload("c2_prefill_32k", "prefill", B=1, L=32768, H_I=64, d_I=128,
              qk_lo=-16, qk_hi=15, w_lo=1, w_hi=8,
              n_sink=4, n_window=512, k_dyn=2048 - 4 - 512, H=64)

# C3: decode with 3-step MTP, B=64 at 128K context; 4 query rows share the
# target row's index; top-k 2048 on top of 4 sinks + 512 window; 8 KV splits.
C3 = Workload("c3_mtp_decode_128k", "decode", B=64, L=131072, H_I=64, d_I=128,
              qk_lo=-16, qk_hi=15, w_lo=1, w_hi=8,
              n_sink=4, n_window=512, k_dyn=2048, H=64, n_q=4, n_split=8)

# C4: hierarchical decode, B=4 at 1M context; block 64, recall 256 blocks,
# fine top-k 2048 + 4 sinks + 512 window; 8 KV splits.
C4 = Workload("c4_hi_decode_1m", "hier_decode", B=4, L=1 << 20, H_I=64, d_I=128,
              qk_lo=-16, qk_hi=15, w_lo=1, w_hi=8,
              n_sink=4, n_window=512, k_dyn=2048, H=64, n_q=1, n_split=8,
              blk=64, n_blk_recall=256)

# C5: CLI prefill L=131072, two layers sharing the layer-1 index;
# total budget 2048 = 4 + 1024 + 1020.
C5 = Workload("c5_cli_prefill_128k", "prefill", B=1, L=131072, H_I=64, d_I=128,
              qk_lo=-16, qk_hi=15, w_lo=1, w_hi=8,
              n_sink=4, n_window=1024, k_dyn=2048 - 4 - 1024, H=64, n_layers=2)

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}
BY_ID = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}
