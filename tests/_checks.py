"""Comparison helpers shared by the CPU and GPU tests.

The alignment is integer work and must match bit for bit, over whole
buffers (valid prefix, sentinel padding and tails). The FFN output is
floating point and must satisfy both
    rel-L2  = ||y - y_ref||_2 / ||y_ref||_2          <= 1e-3
    max-abs = max |y - y_ref|                         <= 1e-2 * rms(y_ref)
(the layer's stated tolerance); cosine similarity is reported alongside, as
the warp-decode write-up does ("Eficiencia de hardware").
"""
import hashlib

import numpy as np

REL_L2_TOL = 1e-3
MAX_ABS_REL_RMS = 1e-2

# Bounds for the intermediate a = silu(gate)*up as the library stores it
# (moe_ffn_intermediate): format 1 (bf16 hi + lo) is within 2^-17 relative of
# the kernel's fp32 value; format 2 (fp16 scaled per 64-element chunk) within
# 2^-11, fp16's unit roundoff. Both add the fp32 accumulation error (about
# 1e-5 at most on these layers).
INTERMEDIATE_REL_L2 = {1: 1e-4, 2: 2.0 ** -11 + 1e-5}


def decode_scaled_f16(a16, mult):
    """Format-2 intermediate as fp64: a16 [..., I] fp16 values and mult
    [..., ceil(I/128), 4] fp32, entries 0 and 1 of slab s multiplying the
    elements of chunks 2s and 2s+1 (64 elements each; the last chunk may be
    partial)."""
    # Rows the library leaves unspecified (invalid routes) and the unused
    # entries may hold any bits, signalling NaNs included.
    with np.errstate(invalid="ignore"):
        a = np.asarray(a16).astype(np.float64)
        m = np.asarray(mult)[..., :2].astype(np.float64)
        m = m.reshape(m.shape[:-2] + (2 * m.shape[-2],))
        return a * np.repeat(m, 64, axis=-1)[..., :a.shape[-1]]


def alignment_mismatch(got, ref):
    """None if (sorted, blocks, num_padded) are identical, else a reason."""
    gs, gb, gn = got
    rs, rb, rn = ref
    if int(gn) != int(rn):
        return f"num_padded {int(gn)} != {int(rn)}"
    gs = np.asarray(gs).reshape(-1)
    rs = np.asarray(rs).reshape(-1)
    if gs.shape != rs.shape:
        return f"sorted_route_ids shape {gs.shape} != {rs.shape}"
    bad = np.nonzero(gs != rs)[0]
    if bad.size:
        i = int(bad[0])
        return f"sorted_route_ids differ at {bad.size} positions, first {i}: {gs[i]} != {rs[i]}"
    gb = np.asarray(gb).reshape(-1)
    rb = np.asarray(rb).reshape(-1)
    if gb.shape != rb.shape:
        return f"expert_block_ids shape {gb.shape} != {rb.shape}"
    bad = np.nonzero(gb != rb)[0]
    if bad.size:
        i = int(bad[0])
        return f"expert_block_ids differ at {bad.size} positions, first {i}: {gb[i]} != {rb[i]}"
    return None


def ffn_errors(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    diff = y - r
    nref = np.linalg.norm(r)
    rel = np.linalg.norm(diff) / nref if nref > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    ny = np.linalg.norm(y)
    cos = float(np.dot(y.ravel(), r.ravel()) / (ny * nref)) if ny > 0 and nref > 0 else 1.0
    return {"rel_l2": float(rel), "max_abs": mx, "rms_ref": rms, "cosine": cos}


def ffn_mismatch(y, y_ref):
    """None if y is within the layer's tolerance of y_ref, else a reason."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return "non-finite output"
    e = ffn_errors(y, y_ref)
    if e["rel_l2"] > REL_L2_TOL:
        return f"rel-L2 {e['rel_l2']:.3e} > {REL_L2_TOL}"
    if e["max_abs"] > MAX_ABS_REL_RMS * e["rms_ref"]:
        return f"max-abs {e['max_abs']:.3e} > {MAX_ABS_REL_RMS} * rms {e['rms_ref']:.3e}"
    return None


def digest(a) -> str:
    """SHA-256 of an array's bytes (bitwise identity check)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
