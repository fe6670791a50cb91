"""The five synthetic workloads, as plain data.

Each workload takes its shapes from a looped model named by the pages:
Ouro-1.4B (24 layers, T=4 loops, d=2048, 16 heads x 128) for workloads 2-4 and
a Huginn-3.5B-like recurrent block (4 layers, T=32, d=5280, 55 heads x 96) for
workload 5.  Workload 1 is a tiny fp32 case small enough for exhaustive checks.

A "set" is one latent set of one layer: the loops it serves, its groups G
(1 = shared by all heads, H = one latent per head), and its key/value widths.
Hybrid Latent Attention has two sets per layer (loop 1, and loops 2..T);
Looped Latent Attention has one set serving loops 1..T.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional


@dataclass(frozen=True)
class SetSpec:
    loop_first: int          # 1-based, inclusive
    loop_last: int
    groups: int              # G
    r_k: int                 # key latent width per group
    r_v: int                 # value latent width per group
    d_in: int                # writer input width per loop and group

    @property
    def n_loops(self) -> int:
        return self.loop_last - self.loop_first + 1


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    layers: int
    loops: int               # T
    d_model: int
    heads: int               # H
    head_dim: int            # d_h
    batch: int               # B
    context: int             # N = tokens attended including the current one
    window: int              # W
    dtype: str               # "f32" or "bf16"
    rope_base: float         # 0 = no rotary embedding
    rope_baked: int
    sets: List[SetSpec] = field(default_factory=list)
    page_size: int = 64
    family: str = "hla"      # "hla" (absorbed + window) or "lla" (one set, loops 1..T)
    value_scale: str = "unit"
    # "iid": latents, maps and exact K/V drawn directly; "trajectory": per-head
    # loop trajectories of rank 8 plus noise, decoders fit to a calibration
    # sample, latents written through the writer (gen.trajectory_codec)
    inputs: str = "iid"

    @property
    def pos(self) -> int:
        return self.context - 1

    def set_for_loop(self, t: int) -> int:
        for k, s in enumerate(self.sets):
            if s.loop_first <= t <= s.loop_last:
                return k
        raise ValueError(t)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# 1: tiny fp32 looped decode (both HLA sets; RoPE off)
W1 = Workload(
    key=1, name="tiny-fp32", layers=1, loops=4, d_model=128, heads=2, head_dim=64,
    batch=1, context=256, window=16, dtype="f32", rope_base=0.0, rope_baked=0,
    sets=[SetSpec(1, 1, 1, 32, 32, 128), SetSpec(2, 4, 1, 128, 128, 128)],
    family="hla")

# 2: per-head LLA reconstruct, Ouro-1.4B shape, rank 32 per head (16x)
W2 = Workload(
    key=2, name="lla-per-head-ouro1.4b", layers=24, loops=4, d_model=2048, heads=16,
    head_dim=128, batch=32, context=4096, window=0, dtype="bf16", rope_base=0.0,
    rope_baked=0, sets=[SetSpec(1, 4, 16, 32, 32, 256)], family="lla", inputs="trajectory")

# 3: HLA absorbed + exact window, Ouro-1.4B shape, 72 KiB/token
W3 = Workload(
    key=3, name="hla-absorbed-ouro1.4b-b128-ctx4k", layers=24, loops=4, d_model=2048,
    heads=16, head_dim=128, batch=128, context=4096, window=128, dtype="bf16",
    rope_base=10000.0, rope_baked=1,
    sets=[SetSpec(1, 1, 1, 256, 256, 2048), SetSpec(2, 4, 1, 512, 512, 2048)],
    family="hla")

# 4: HLA long context
W4 = W3.with_(key=4, name="hla-absorbed-ouro1.4b-b32-ctx16k", batch=32, context=16384)

# 5: LLA-2D head-folded, Huginn-3.5B-like
W5 = Workload(
    key=5, name="lla2d-huginn-like", layers=4, loops=32, d_model=5280, heads=55,
    head_dim=96, batch=64, context=4096, window=0, dtype="bf16", rope_base=0.0,
    rope_baked=0, sets=[SetSpec(1, 32, 1, 5280, 5280, 10560)], family="lla")

WORKLOADS = {1: W1, 2: W2, 3: W3, 4: W4, 5: W5}


def get(key: int) -> Workload:
    return WORKLOADS[key]
