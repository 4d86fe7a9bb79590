"""Workload shapes for one pipeline cell's training step.

A cell is a run of identical pre-LN Transformer layers (LayerNorm, multi-head
attention, GeLU FFN); the mini-batch of N sequences is split into M equal
micro-batches (GPipe technical review, "GPipe algorithm in detail / pipeline
execution flow / phase 1: forward").  The shapes below are the synthetic
stand-ins for the pages' Transformer workloads (the multilingual NMT models of
the "Experiment 5" table, whose corpus is private); the convolutional cell
stands in for the pages' AmoebaNet experiments.

Plain data only: no arithmetic of the method lives here.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class CellConfig:
    name: str
    layers: int        # layers in the cell (L/K)
    d_model: int
    heads: int
    d_ff: int
    seq: int
    batch: int         # N, sequences per mini-batch
    micro: int         # M, micro-batches per mini-batch
    causal: bool
    precision: str     # "fp32" or "bf16"
    # RMSProp hyper-parameters (ms_0 = 0, epsilon outside the square root)
    lr: float = 1e-3
    decay: float = 0.9
    eps: float = 1e-8
    ln_eps: float = 1e-5
    seed: int = 0

    @property
    def head_dim(self) -> int:
        return self.d_model // self.heads

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def with_(self, **kw) -> "CellConfig":
        return replace(self, **kw)

    def param_count(self) -> int:
        d, f = self.d_model, self.d_ff
        per_layer = 4 * d * d + 2 * d * f + 9 * d + f
        return self.layers * per_layer


@dataclass(frozen=True)
class ConvCellConfig:
    name: str
    blocks: int
    channels: int
    height: int
    width: int
    batch: int
    micro: int
    precision: str
    bn_momentum: float = 0.9   # retention of the running statistics
    bn_eps: float = 1e-5
    lr: float = 1e-3
    decay: float = 0.9
    eps: float = 1e-8
    seed: int = 0

    def param_count(self) -> int:
        c = self.channels
        return self.blocks * (2 * 9 * c * c + 4 * c)

    def pixels(self) -> int:
        return self.batch * self.height * self.width

    def with_(self, **kw) -> "ConvCellConfig":
        return replace(self, **kw)


# Tiny fp32 cell: the small case every oracle check runs in seconds.
TINY = CellConfig("tiny_fp32", layers=2, d_model=64, heads=4, d_ff=256, seq=32,
                  batch=8, micro=4, causal=False, precision="fp32")

# Small bf16 cell (also run with M=1 to compare with the full-batch step).
SMALL = CellConfig("small_bf16", layers=6, d_model=512, heads=8, d_ff=2048, seq=128,
                   batch=64, micro=8, causal=False, precision="bf16")

# One cell of a 128-layer stack split into 16 cells, causal attention.  The
# layer width is the T(.,8192,16) family of the NMT table; this is the
# throughput workload.
CELL_2048 = CellConfig("cell_d2048_L8_causal", layers=8, d_model=2048, heads=16,
                       d_ff=8192, seq=512, batch=64, micro=32, causal=True,
                       precision="bf16")

# Memory-scaling cell (48 layers of d_model 4096): its parameter state is
# ~9.7 B params; only the planner and reduced-N runs are practical.
MEMORY_4096 = CellConfig("cell_d4096_L48", layers=48, d_model=4096, heads=32,
                         d_ff=16384, seq=1024, batch=32, micro=32, causal=False,
                         precision="bf16")

# Convolutional cells with micro-batch BatchNorm: a tiny fp32 case, a small
# bf16 case whose GEMMs take the tiled MFMA path, and the throughput workload.
CONV_TINY = ConvCellConfig("conv_tiny_fp32", blocks=2, channels=16, height=8, width=8,
                           batch=8, micro=4, precision="fp32")
CONV_SMALL = ConvCellConfig("conv_small_bf16", blocks=2, channels=64, height=16, width=16,
                            batch=16, micro=4, precision="bf16")
CONV_CELL = ConvCellConfig("conv_c256_b8", blocks=8, channels=256, height=32, width=32,
                           batch=256, micro=16, precision="bf16")

ALL = {c.name: c for c in (TINY, SMALL, CELL_2048, MEMORY_4096)}
CONV_ALL = {c.name: c for c in (CONV_TINY, CONV_SMALL, CONV_CELL)}
