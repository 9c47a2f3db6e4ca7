"""The five synthetic workloads, by shape.

Shapes follow the pages: the mere.run transfer report ("Shared architecture
and implemented paths"; "Exact verification kernels and benchmark admission")
for the 5,120-wide dense projections and the MoE of 256 experts (hidden
2,048, intermediate 512) with 8 routed per row;
the Flash-Next plan ("2.1 Gated DeltaNet", "2.3 MoE") for the 48-layer
hybrid with 16/48 GDN heads of dimension 128 and the 512-expert top-10 MoE
with intermediate 640 and one shared expert.
"""

from dataclasses import dataclass, field

# config ids used in seeds
TINY, DENSE, ORNITH, GDN36, FLASH = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class MoeShape:
    hidden: int
    experts: int
    inter: int
    topk: int
    mode: str          # "softmax" or "sigmoid"
    renorm: bool
    shared: bool       # one always-on shared expert, sigmoid-gated per row


@dataclass(frozen=True)
class GdnShape:
    hv: int
    hk: int
    dk: int
    dv: int

    @property
    def state_elems(self):
        return self.hv * self.dv * self.dk


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    widths: tuple
    dense: tuple = None            # (N, K) of one dense projection
    moe: MoeShape = None
    gdn: GdnShape = None
    layers: int = 1                # MoE layers (or dense weights) streamed per step
    gdn_layers: tuple = ()         # layer indices that carry a GDN state
    notes: str = ""
    extra: dict = field(default_factory=dict)


C0 = Config(TINY, "tiny", widths=(2,), dense=(1024, 1024),
            gdn=GdnShape(hv=4, hk=4, dk=64, dv=64), layers=1, gdn_layers=(0,),
            extra={"rollback_prefix": 1})

C1 = Config(DENSE, "dense5120", widths=(1, 4, 8, 9), dense=(5120, 5120), layers=64)

C2 = Config(ORNITH, "ornith_moe", widths=tuple(range(2, 10)),
            moe=MoeShape(hidden=2048, experts=256, inter=512, topk=8, mode="softmax",
                         renorm=False, shared=False),
            layers=40)

C3 = Config(GDN36, "gdn36", widths=tuple(range(1, 10)),
            gdn=GdnShape(hv=48, hk=16, dk=128, dv=128), layers=36,
            gdn_layers=tuple(range(36)))

C4 = Config(FLASH, "flashnext_k9", widths=(9,),
            moe=MoeShape(hidden=2560, experts=512, inter=640, topk=10, mode="sigmoid",
                         renorm=True, shared=True),
            gdn=GdnShape(hv=48, hk=16, dk=128, dv=128), layers=48,
            gdn_layers=tuple(l for l in range(48) if l % 4 != 3),
            # Flash-Next plan, "1. Target model and identity": vocab 248,320 (padded)
            extra={"vocab": 248320})

ALL = (C0, C1, C2, C3, C4)


def q4_bytes(n, k):
    """Bytes of one affine-Q4/g64 matrix: nibbles plus bf16 scale and bias per group."""
    return n * k // 2 + n * (k // 64) * 4
