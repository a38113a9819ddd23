"""Plain float64 definition of the routed MoE expert-FFN layer (test infrastructure).

Sources (the pages this layer is defined by):
  [P1] "Route-Block Membership Selects Packed-AWQ Arithmetic — A Controlled
       Single-Fixture Mechanism Study" (arXiv 2607.26316): first paragraph
       (route flattening and alignment), the paragraph defining A_e and the
       blocks B(e, j), and the paragraph on stable construction.
  [P2] "Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE"
       (arXiv 2610.02241): Section 2 (routed MoE layer, expert products),
       Section 3.3 with Eq. 4 (the gate coefficient weights each expert's
       output; gate-up-down expert block) and Section 3.4 (SwiGLU
       intermediate).
  [P3] "warp decode" (cursor.com blog): "Cómo funcionan los dos kernels"
       (gate/up with SiLU(gate) x up, down projection with the routing
       weight folded into one accumulator).

Readings taken where the pages leave a step open are listed in the module
docstrings of each function and collected in the design notes.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# 1. Route alignment  [P1, first paragraph; A_e / B(e, j) paragraph; stable
#    construction paragraph]
# ----------------------------------------------------------------------------

def align_capacity(M: int, k: int, E: int, b: int) -> int:
    """Upper bound on the aligned row count, rounded up to a multiple of b.

    Each touched expert adds at most b - 1 padding rows to its count, and at
    most min(E, M*k) experts are touched.
    """
    mk = M * k
    raw = mk + min(E, mk) * (b - 1)
    return ((raw + b - 1) // b) * b


def align(topk_ids: np.ndarray, E: int, b: int, capacity: int | None = None,
          expert_base: int = 0):
    """Stable route alignment.

    Route IDs r are the row-major flattening of the M x k expert-ID array
    (r = t*k + j) [P1, first paragraph]. A route is valid when its expert ID
    lies in [expert_base, expert_base + E) — the E experts held here, all of
    them when expert_base is 0; invalid routes are skipped. For each expert e
    in ascending order, its valid routes are listed in ascending route ID
    (ordering by (expert ID, flattened route ID) [P1, stable construction]),
    then padded with the sentinel M*k up to ceil(c_e / b) * b rows; each
    group of b rows is one block whose entry in the expert-block vector is
    the expert's local index e - expert_base [P1, first paragraph; A_e /
    B(e, j) paragraph]. Experts with no routes get no rows.

    Returns (sorted_route_ids int32 [C], expert_block_ids int32 [C / b],
    num_padded int) with C = ``capacity`` (default ``align_capacity``).
    Positions from num_padded to C hold the sentinel in sorted_route_ids and
    -1 in expert_block_ids.
    """
    arr = np.asarray(topk_ids)
    if arr.ndim != 2:
        raise ValueError("topk_ids must be [M, k]")
    M, k = arr.shape
    ids = arr.reshape(-1).astype(np.int64)
    mk = ids.size
    C = align_capacity(M, k, E, b) if capacity is None else int(capacity)
    sentinel = mk
    sorted_ids = np.full(C, sentinel, dtype=np.int32)
    blocks = np.full(C // b, -1, dtype=np.int32)
    off = 0
    for e in range(E):
        routes = np.nonzero(ids == expert_base + e)[0]    # ascending route IDs
        c = routes.size
        if c == 0:
            continue
        padded = -(-c // b) * b
        sorted_ids[off:off + c] = routes
        blocks[off // b:(off + padded) // b] = e
        off += padded
    return sorted_ids, blocks, off


# ----------------------------------------------------------------------------
# 2. Dequantisation
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# AWQ's interleaved packing: nibble slot i (bits 4i..4i+3) of a word holds
# element AWQ_ORDER[i] of that word's eight elements.
AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def unpack_int4(qwords: np.ndarray) -> np.ndarray:
    """uint32 words [..., K/8] -> unsigned 4-bit values [..., K].

    Word kk // 8 holds elements 8*(kk // 8) .. +7; element AWQ_ORDER[i] sits in
    nibble slot i (bits 4i..4i+3).
    """
    w = np.asarray(qwords, dtype=np.uint32)
    slots = (w[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & np.uint32(15)
    out = np.empty_like(slots)
    out[..., list(AWQ_ORDER)] = slots
    return out.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.int64)


def dequant_int4(qwords: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 g: int) -> np.ndarray:
    """AWQ-style group dequantisation W[n, kk] = (q[n, kk] - z[n, kk//g]) * s[n, kk//g].

    4-bit weight-only quantisation with group size g along the reduction
    dimension [P1, fixture paragraph: 4-bit AWQ, group size 128].
    """
    q = unpack_int4(qwords).astype(np.float64)
    K = q.shape[-1]
    grp = np.arange(K) // g
    s = np.asarray(scales).astype(np.float64)[..., grp]
    z = np.asarray(zeros).astype(np.float64)[..., grp]
    return (q - z) * s


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    is subnormal (m/8 * 2^-6); code 0x7F / 0xFF is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6,
                   (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7))
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return sign * val


def e8m0_to_f64(exps: np.ndarray) -> np.ndarray:
    """E8M0 shared-exponent bytes -> 2^(e - 127); 0xFF is NaN."""
    e = np.asarray(exps, dtype=np.uint8).astype(np.float64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def dequant_mxfp8(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """MXFP8 weights: E4M3 element times the E8M0 scale of its 32-element block.

    The warp-decode kernels read MXFP8 weights and convert them to FP32 on
    the fly [P3, "Cómo funcionan los dos kernels"]; the MX block format is the
    OCP microscaling one [P2, Section 2].
    """
    v = e4m3_to_f64(codes)
    K = v.shape[-1]
    sc = e8m0_to_f64(exps)[..., np.arange(K) // 32]
    return v * sc


def _dequant(pw, e: int) -> np.ndarray:
    if pw.fmt == "int4":
        return dequant_int4(pw.q[e], pw.s[e], pw.z[e], pw.g)
    if pw.fmt == "mxfp8":
        return dequant_mxfp8(pw.q[e], pw.s[e])
    raise ValueError(pw.fmt)


# ----------------------------------------------------------------------------
# 3-4. Expert FFN and combine
# ----------------------------------------------------------------------------

def _silu(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def ffn_stages(x_bits: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
               w13, w2, E: int, expert_base: int = 0) -> dict:
    """All intermediate surfaces of the layer in float64.

    A route is valid when its expert ID lies in [expert_base, expert_base +
    E); the weights hold those E experts, expert ID e at index e -
    expert_base (expert_base = 0: all experts).
    For each valid route r (token t = r // k, expert e = ids[r]):
      gate = W13[e, 0:I, :] x_t,  up = W13[e, I:2I, :] x_t   (W13 rows 0..I-1
      are the gate projection, I..2I-1 the up projection),
      a_r  = silu(gate) * up with silu(v) = v / (1 + e^-v)
      yhat_r = W2[e] a_r
    [P2, Sections 3.3-3.4: gate-up-down expert block with SwiGLU
    intermediate; P3, "Cómo funcionan los dos kernels": SiLU(gate) x up].
    Then y_t = sum over j = 0..k-1 of w[t, j] * yhat_{t*k+j}, skipping
    invalid routes [P2, Eq. 4: the gate coefficient weights the expert
    output; P3: routing weight folded into the down accumulator]. The
    weights are used as given (no renormalisation inside the layer).

    Returns dict with gate, up, a [Mk, I], yhat [Mk, H] (zero rows for
    invalid routes) and y [M, H].
    """
    x = bf16_to_f64(x_bits)
    ids = np.asarray(topk_ids).astype(np.int64)
    wts = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    M, k = ids.shape
    H = x.shape[1]
    I = w13.N // 2
    flat = ids.reshape(-1)
    gate = np.zeros((M * k, I))
    up = np.zeros((M * k, I))
    a = np.zeros((M * k, I))
    yhat = np.zeros((M * k, H))
    for e in np.unique(flat):
        if e < expert_base or e >= expert_base + E:
            continue
        routes = np.nonzero(flat == e)[0]
        W13 = _dequant(w13, int(e - expert_base))          # [2I, H]
        W2 = _dequant(w2, int(e - expert_base))            # [H, I]
        X = x[routes // k]                   # [n, H]
        G = X @ W13[:I].T
        U = X @ W13[I:].T
        A = _silu(G) * U
        gate[routes] = G
        up[routes] = U
        a[routes] = A
        yhat[routes] = A @ W2.T
    y = np.zeros((M, H))
    for t in range(M):
        for j in range(k):
            e = ids[t, j]
            if expert_base <= e < expert_base + E:
                y[t] += wts[t, j] * yhat[t * k + j]
    return {"gate": gate, "up": up, "a": a, "yhat": yhat, "y": y}


def ffn(x_bits, topk_ids, topk_w, w13, w2, E: int, expert_base: int = 0) -> np.ndarray:
    """Layer output y [M, H] in float64 (see ``ffn_stages``)."""
    return ffn_stages(x_bits, topk_ids, topk_w, w13, w2, E, expert_base)["y"]


# ----------------------------------------------------------------------------
# 5. The two grouped GEMMs on a fixed-capacity batched layout  [P2, App. D.1:
#    operands of expert e at a fixed stride with a per-expert capacity, token
#    counts kept on the device; the GEMM shapes of App. D.2, Table 8]
# ----------------------------------------------------------------------------

def _valid_rows(counts, cap: int) -> np.ndarray:
    return np.clip(np.asarray(counts, dtype=np.int64), 0, cap)


def batched_gate_up(xb_bits: np.ndarray, counts: np.ndarray, w13) -> np.ndarray:
    """a [E, cap, I] float64: for expert e and row n < clamp(counts[e], 0, cap),
    a[e, n] = silu(W13[e, 0:I] x[e, n]) * (W13[e, I:2I] x[e, n]) with x the
    bf16 rows of ``xb_bits`` [E, cap, H] (the gate/up expert product of
    ``ffn_stages``); rows at or past the count are zero."""
    x = bf16_to_f64(xb_bits)
    E, cap, H = x.shape
    I = w13.N // 2
    n = _valid_rows(counts, cap)
    a = np.zeros((E, cap, I))
    for e in range(E):
        if n[e] == 0:
            continue
        W13 = _dequant(w13, e)
        X = x[e, :n[e]]
        a[e, :n[e]] = _silu(X @ W13[:I].T) * (X @ W13[I:].T)
    return a


def batched_down(a: np.ndarray, counts: np.ndarray, w2) -> np.ndarray:
    """yhat [E, cap, H] float64: yhat[e, n] = W2[e] a[e, n] for n <
    clamp(counts[e], 0, cap) (the down expert product of ``ffn_stages``,
    before any combine); rows at or past the count are zero."""
    E, cap, _ = a.shape
    H = w2.N
    n = _valid_rows(counts, cap)
    y = np.zeros((E, cap, H))
    for e in range(E):
        if n[e] == 0:
            continue
        y[e, :n[e]] = a[e, :n[e]] @ _dequant(w2, e).T
    return y
