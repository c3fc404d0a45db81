"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package holds no arithmetic of the attention method itself: it only draws
random document contents, queries, request compositions and lengths, with the
shapes and structure of the workloads described on the LazyAttention pages
(retrieval-augmented requests built from cached documents in per-request
orders, GQA/MQA head layouts, Zipf-skewed document popularity).  Both the HIP
path and the fp64 oracle consume exactly these arrays.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Geometry,
    PosSpec,
    PrefillRequest,
    DecodeRequest,
    Workload,
    make_workload,
    round_to_bf16,
    sharpened,
    zipf_accesses,
    zipf_trace,
)
