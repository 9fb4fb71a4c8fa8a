"""The synthetic workloads of the selective scan (S6), by shape and input recipe.

Each workload is named by what it is.  c0..c4 restate the benchmark configurations this
library is measured on; d1 is a decode step (one token per sequence, the state carried in
and out) at the D=5120 width with a serving-size batch; p2 is the block around the scan
(input projection, selection projections, gated scan) at the D=5120 width with an input
twice as narrow (the block's usual expansion by 2).  Nothing here computes any part of the
scan.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str          # short handle used by tests and the bench
    label: str         # human description (shape + precision)
    batch: int
    seqlen: int
    dim: int           # D, number of channels per batch row
    dstate: int        # N, state size per channel
    dtype: str         # "f32" or "bf16": dtype of x, dt_raw, z, B, C
    gate: bool         # silu(z) gate on the output
    a_perturb: bool    # A[d,n] = -(n+1)*exp(eps), eps ~ N(0, 0.1^2)
    backward: bool     # workload also exercises the backward pass
    h_final: bool      # final state is an output of the workload
    decode: bool = False  # one token per (batch row, channel) through ss_step, state in place
    d_in: int = 0         # > 0: the block (projections + gated scan) on input width d_in

    @property
    def elems(self) -> int:
        """B*L*D: the element count the throughput metric divides by."""
        return self.batch * self.seqlen * self.dim

    @property
    def channels(self) -> int:
        return self.batch * self.dim


WORKLOADS = (
    Workload("c0", "S6 fwd fp32 B=1 L=256 D=64 N=16 no gate",
             1, 256, 64, 16, "f32", False, False, False, False),
    Workload("c1", "S6 fwd+gate fp32 B=2 L=2048 D=1536 N=16",
             2, 2048, 1536, 16, "f32", True, False, False, False),
    Workload("c2", "S6 fwd+gate bf16-in B=8 L=2048 D=5120 N=16 A=-(n+1)exp(eps)",
             8, 2048, 5120, 16, "bf16", True, True, False, False),
    Workload("c3", "S6 fwd bf16-in long sequence B=1 L=1048576 D=256 N=16 with final state",
             1, 1048576, 256, 16, "bf16", False, False, False, True),
    Workload("c4", "S6 fwd+bwd+gate bf16-in B=4 L=4096 D=2048 N=16",
             4, 4096, 2048, 16, "bf16", True, False, True, False),
    Workload("d1", "S6 decode step (one token, state in place) bf16-in B=256 D=5120 N=16 gate",
             256, 1, 5120, 16, "bf16", True, True, False, True, decode=True),
    Workload("p2", "S6 block fwd: bf16 u [8, 2048, 2560] x W_in [10240, 2560] on the matrix "
             "cores, fp32 selection projections, gated scan D=5120 N=16",
             8, 2048, 5120, 16, "bf16", True, True, False, False, d_in=2560),
)

BY_NAME = {w.name: w for w in WORKLOADS}


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    return BY_NAME[name_or_index]


def seed_of(w: Workload) -> int:
    """Seed of a workload = its index in WORKLOADS."""
    return WORKLOADS.index(w)
