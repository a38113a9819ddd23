"""CPU fp64 oracle for the routed MoE expert-FFN layer — TEST INFRASTRUCTURE.

Only the test suite, the smoke check of ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import or run anything in this package. The
product path (the HIP library and its Python binding) never does, and the
oracle imports nothing from it: the two share no code. Both consume the same
seeded inputs from the ``workloads`` package.

What the oracle computes is the plain definition of the layer, in float64:

1. route alignment (group valid routes by expert in route-ID order, pad each
   expert to a multiple of b, emit the expert-block vector);
2. AWQ-style int4 dequantisation ``(q - z) * s`` per group (and, for the
   MXFP8 variant, E4M3 code times 2^(E8M0 - 127) per 32 elements);
3. per route: gate/up projection, ``silu(gate) * up``, down projection;
4. the router-weighted top-k combine.

Pins (tests run with ``-m "not gpu"``): hand-worked alignment fixtures under
``tests/golden``, a sort-based brute-force alignment, the b = 1 case against
``numpy.argsort(kind="stable")``, the padded-count identity and other
alignment invariants, dequantisation on hand-built words and on all 16 x 16
(q, z) pairs, a pure-Python loop FFN on tiny shapes, the identical-experts
case against a dense SwiGLU built from torch's float64 ``matmul`` and
``silu``, zero input giving exact zeros, linearity in the combine weights,
W2 scale doubling, invalid-ID skipping, and all 256 E4M3 codes against
``torch.float8_e4m3fn``. The expert-range form (only experts [expert_base,
expert_base + E) held here) is pinned by hand-worked range fixtures, the
sort-based brute force with a range, disjoint shards partitioning the routes,
the loop FFN with a range, and shard outputs summing to the full layer. The
batched-layout GEMMs are pinned by a loop over elements on tiny shapes and
by the routed layer's own per-route surfaces when the batch is built from a
routing.
Every function below is pinned by at least one of these; none is "parity
unpinned".
"""
from .moe_oracle import (  # noqa: F401
    align,
    align_capacity,
    batched_down,
    batched_gate_up,
    bf16_to_f64,
    dequant_int4,
    dequant_mxfp8,
    e4m3_to_f64,
    e8m0_to_f64,
    ffn,
    ffn_stages,
    unpack_int4,
)
