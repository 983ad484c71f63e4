"""The five synthetic shard-step workloads (sizes, distributions, settings).

"GPT-2-sized", "1.5B", "7B" and "13B" are buffer sizes only: no model,
weights or dataset.  Each workload is one flat Psi-element buffer split over
N data-parallel ranks; the measured rank is the last one (r = N-1) except for
the toy, whose 32 shards all run.  Contribution rows are padded to a stride
that is a multiple of 64 elements.
"""
from __future__ import annotations

from dataclasses import dataclass, field

F16 = 1
BF16 = 2


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclass(frozen=True)
class Workload:
    name: str
    psi: int                  # flat parameter count
    nranks: int               # data-parallel degree N = number of contributions
    ranks: tuple              # ranks whose shard step runs
    dtype: int                # 16-bit format of contributions and of the gathered parameters
    steps: int
    contrib_sigma: float = 1e-3
    contrib_scale: float = 1.0    # contributions are drawn already multiplied by this
    outlier_p: float = 0.0        # Bernoulli probability per contribution element
    outlier_mult: float = 100.0
    master_sigma: float = 0.02
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_grad_norm: float = 0.0    # > 0 turns clipping on (two-pass path)
    scaler: int = 0               # 0 none (S = 1), 1 static, 2 dynamic
    loss_scale: float = 1.0
    min_scale: float = 1.0
    growth_interval: int = 1000
    inject_inf: tuple = ()        # (step, k, element-in-shard) triples set to +inf
    seed: int = 0
    gather_dtype: int = 0         # 16-bit format of the gathered parameters; 0: as dtype
    note: str = field(default="", compare=False)

    @property
    def slot_dtype(self) -> int:
        return self.gather_dtype or self.dtype

    @property
    def shard(self) -> int:
        return -(-self.psi // self.nranks)

    @property
    def stride(self) -> int:
        return round_up(self.shard, 64)

    @property
    def variant(self) -> str:
        return "two_pass" if self.max_grad_norm > 0 else "fused"

    @property
    def bytes_per_elem(self) -> int:
        """Algorithmic HBM bytes per shard element of one step."""
        return 2 * self.nranks + (34 if self.variant == "two_pass" else 26)


TOY = Workload(
    name="toy_psi637824_n32", psi=637_824, nranks=32, ranks=tuple(range(32)), dtype=F16, steps=3,
    note="toy flat buffer, all 32 shards, fp16, no loss scale")

GPT2 = Workload(
    name="gpt2_psi124439808_n8", psi=124_439_808, nranks=8, ranks=(7,), dtype=F16, steps=20,
    contrib_scale=2.0 ** 16, scaler=1, loss_scale=2.0 ** 16, weight_decay=0.01,
    note="GPT-2-small-sized buffer, fp16, static loss scale 2^16, AdamW wd 0.01")

P1_5B = Workload(
    name="psi1.5e9_n64", psi=1_500_000_000, nranks=64, ranks=(63,), dtype=BF16, steps=10,
    lr=3e-4, note="1.5B buffer, 64 bf16 contributions, small-shard regime")

P7B = Workload(
    name="psi7e9_n8_clip", psi=7_000_000_000, nranks=8, ranks=(7,), dtype=BF16, steps=5,
    outlier_p=1e-3, max_grad_norm=1.0,
    note="7B buffer, bf16, 0.1% outliers x100, global-norm clip 1.0 (two-pass)")

P13B = Workload(
    name="psi1.3e10_n8_dynscale", psi=13_000_000_000, nranks=8, ranks=(7,), dtype=F16, steps=5,
    contrib_scale=2.0 ** 15, scaler=2, loss_scale=2.0 ** 15,
    inject_inf=((2, 3, 1_625_000_000 // 2),),
    note="13B buffer, fp16, dynamic loss scale 2^15, +inf in contribution 3 at step 2")

ALL = (TOY, GPT2, P1_5B, P7B, P13B)
BY_NAME = {w.name: w for w in ALL}
