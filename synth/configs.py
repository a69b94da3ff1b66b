"""The five workloads, by shape."""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    num_experts: int
    hidden: int
    inter: int
    topk: int
    tokens: tuple            # live token counts exercised
    t_cap: int               # token capacity (workspace size); None -> tokens
    align_rows: int          # per-expert row alignment
    row_cap: int             # rows of the aligned workspace (0 -> minimum bound)
    scale_fmts: tuple        # activation scale formats exercised
    acts: tuple = ("swiglu",)
    clamp_limit: float = float("inf")
    routing: str = "softmax"  # "softmax" or "zipf"
    zipf_s: float = 1.1
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "tiny": Workload(
        name="tiny", index=0, num_experts=4, hidden=256, inter=128, topk=2,
        tokens=(8,), t_cap=8, align_rows=16, row_cap=64,
        scale_fmts=("fp32",)),
    "decode": Workload(
        name="decode", index=1, num_experts=288, hidden=4096, inter=512,
        topk=8, tokens=(1, 4), t_cap=0, align_rows=16, row_cap=0,
        scale_fmts=("fp32",), acts=("swiglu", "swiglu_clamp"),
        clamp_limit=7.0),
    "padded": Workload(
        name="padded", index=2, num_experts=32, hidden=7168, inter=2048,
        topk=8, tokens=(16,), t_cap=512, align_rows=16, row_cap=0,
        scale_fmts=("ue8m0", "fp32")),
    "full": Workload(
        name="full", index=3, num_experts=32, hidden=7168, inter=2048,
        topk=8, tokens=(4096,), t_cap=4096, align_rows=16, row_cap=0,
        scale_fmts=("fp32", "ue8m0")),
    "sweep": Workload(
        name="sweep", index=4, num_experts=256, hidden=6144, inter=256,
        topk=8, tokens=(1, 8, 64, 256, 1024, 4096), t_cap=0, align_rows=16,
        row_cap=0, scale_fmts=("fp32", "pow2"), routing="zipf"),
}


def get(name):
    return CONFIGS[name]

