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
    chain: bool = False  # layers chained through the residual stream (x = norm(r), r += y)
    z_lo: float = -0.08  # bias range of the expert blobs
    z_hi: float = 0.08
    tier_slots: int = 0  # > 0: experts in host memory behind this many device slots
    resid_scale: float = 1.0  # chained stacks: the initial residual is residual(...) times this
    description: str = ""


# AR(1) correlation giving about 70% expert reuse between consecutive tokens
# (the page-cache hit rate the pages report, "How the SSD expert streaming
# pipeline works"); calibrated with the float64 router on the stack's own
# routers, the benchmark reports the reuse it actually sees.
STACK_RHO = 0.97

# Scale of the chained stack's initial residual.  With unit channels every
# layer's output is as large as the residual it is added to, so the routing
# of consecutive tokens decorrelates after a few layers (reuse 0.08 over the
# stack); in a trained model each layer adds a small update to a large
# residual stream.  At 1024 the reuse between consecutive tokens is ~0.69 in
# every layer (measured on the stack's own weights with the multi-layer
# kernel: 0.70 in layers 1-9, 0.69 in layers 10-59), the ~70% that the
# per-layer stack gets from its AR(1) activations.  The norm makes x
# independent of the scale.
CHAIN_RESID_SCALE = 1024.0

# Bias range centred on -(2^4 - 1)/2 * mean scale (7.5 * 0.0125), so that each
# 4-bit weight matrix has zero mean, as a trained model's do.  With the
# uncentred range every weight has mean ~0.094: the first layer's output is
# then a near-constant vector that dominates the residual, and from the second
# layer on every gate sum is ~ -0.094 * 4096 and SwiGLU underflows -- the
# chained stack degenerates.  Per-layer (teacher-forced) workloads keep the
# uncentred range.
CENTRED_Z = (-0.08 - 7.5 * 0.0125, 0.08 - 7.5 * 0.0125)

WORKLOADS = {
    "tiny": Workload("tiny", 4096, 1024, 16, 4, 4, 1, 1, 1, 1000, 1000,
                     description="one layer, 16 experts, 1 token"),
    "layer": Workload("layer", 4096, 1024, 512, 4, 4, 1, 1, 128, 1001, 1001,
                      description="one full layer, 512 experts, 1 token per call, 128 "
                                  "distinct tokens"),
    "stack60": Workload("stack60", 4096, 1024, 512, 4, 4, 60, 1, 128, 1002, 1002, rho=STACK_RHO,
                        description="60 HBM-resident layers x 512 4-bit experts, "
                                    "128 consecutive decode tokens"),
    "stack60_chain": Workload("stack60_chain", 4096, 1024, 512, 4, 4, 60, 1, 128, 1002, 1002,
                              rho=STACK_RHO, chain=True, z_lo=CENTRED_Z[0], z_hi=CENTRED_Z[1],
                              resid_scale=CHAIN_RESID_SCALE,
                              description="the 60-layer stack chained through the residual "
                                          "stream: per layer x = norm(r), the MoE layer, "
                                          "r += y; 128 consecutive decode tokens"),
    "stack8_tier": Workload("stack8_tier", 4096, 1024, 512, 4, 4, 8, 1, 128, 1002, 1002,
                            rho=STACK_RHO, tier_slots=1024,
                            description="8 layers x 512 4-bit experts in pinned host memory "
                                        "behind 1024 device expert slots (LRU), 128 "
                                        "consecutive decode tokens"),
    "batch64": Workload("batch64", 4096, 1024, 512, 4, 4, 1, 64, 1, 1003, 1003,
                        description="one full layer, 64 tokens routed independently"),
    "prefill4096": Workload("prefill4096", 4096, 1024, 512, 4, 4, 1, 4096, 1, 1006, 1006,
                            description="one full layer, a prefill chunk of 4096 tokens "
                                        "routed independently"),
    "stack60_2bit": Workload("stack60_2bit", 4096, 1024, 512, 4, 2, 60, 1, 128, 1002, 1004,
                             rho=STACK_RHO,
                             description="the 60-layer stack with 2-bit codes, same routers "
                                         "and activations"),
}
