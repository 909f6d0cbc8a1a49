"""The synthetic workloads, named by what they are.

Shapes follow the Flash-MoE pages for Qwen3.5-397B-A17B ("Flash-MoE: Running
a 397B Parameter Model on a Laptop", hysenlabs.com, section "How the SSD
expert streaming pipeline works": 60 layers, 512 experts, K=4 plus a shared
expert, hidden 4096, ~6.75 MB 4-bit experts, which with groups of 64 and bf16
scale and bias pins the intermediate size at 1024).  Value distributions:
codes uniform, scale ~ U(0.005, 0.02), bias ~ U(-0.08, 0.08), router
~ N(0, 0.02^2), activations ~ N(0, 1) then RMS-normalised.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    K: int
    bits: int
    layers: int
    T: int             # tokens per call (batch)
    tokens: int        # consecutive decode tokens (1 for single-call workloads)
    seed: int          # seed of router and activations
    blob_seed: int     # seed of the expert blobs
    rho: float = 0.0   # AR(1) token-to-token correlation of activations (0: i.i.d.)
    has_shared: int = 1
    group: int = 64
    description: str = ""


# AR(1) correlation giving about 70% expert reuse between consecutive tokens
# (the page-cache hit rate the pages report, "How the SSD expert streaming
# pipeline works"); calibrated with the float64 router on the stack's own
# routers, the benchmark reports the reuse it actually sees.
STACK_RHO = 0.97

WORKLOADS = {
    "tiny": Workload("tiny", 4096, 1024, 16, 4, 4, 1, 1, 1, 1000, 1000,
                     description="one layer, 16 experts, 1 token"),
    "layer": Workload("layer", 4096, 1024, 512, 4, 4, 1, 1, 1, 1001, 1001,
                      description="one full layer, 512 experts, 1 token"),
    "stack60": Workload("stack60", 4096, 1024, 512, 4, 4, 60, 1, 128, 1002, 1002, rho=STACK_RHO,
                        description="60 HBM-resident layers x 512 4-bit experts, "
                                    "128 consecutive decode tokens"),
    "batch64": Workload("batch64", 4096, 1024, 512, 4, 4, 1, 64, 1, 1003, 1003,
                        description="one full layer, 64 tokens routed independently"),
    "stack60_2bit": Workload("stack60_2bit", 4096, 1024, 512, 4, 2, 60, 1, 128, 1002, 1004,
                             rho=STACK_RHO,
                             description="the 60-layer stack with 2-bit codes, same routers "
                                         "and activations"),
}
