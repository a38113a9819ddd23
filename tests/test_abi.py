"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and rejects bad arguments before enqueuing any GPU work.

Nothing here launches a kernel: every call either is a pure host helper or
fails validation, so the suite runs on machines without a GPU.
"""
import ctypes

import pytest

import mixture_experts_ffn_align_amd as moe
import oracle
from mixture_experts_ffn_align_amd import _binding as B

FAKE = 0x10000  # a 256-byte-aligned non-null address; never dereferenced on these paths


def test_library_exports_every_declared_symbol():
    names = moe.declared_symbols()
    assert len(names) >= 11
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe_ffn.h but not exported"


def test_measurement_library_exports_and_validates():
    names = B.declared_symbols(B.BENCH_HEADER_PATH, "MOE_BENCH_API")
    assert set(names) == {"moe_bench_stream_read", "moe_bench_copy", "moe_bench_mfma"}
    L = B.bench_lib()
    for n in names:
        assert hasattr(L, n)
    rd, cp, mf = L.moe_bench_stream_read, L.moe_bench_copy, L.moe_bench_mfma
    assert mf(0, 0, 64, 8, None, None, None, None, None) == 1
    assert mf(0, 0, 0, 8, FAKE, None, None, None, None) == 1
    assert mf(0, 0, 64, 0, FAKE, None, None, None, None) == 1
    assert mf(0, 0, 64, 8193, FAKE, None, None, None, None) == 1
    assert mf(1, 2, 64, 8, FAKE, None, None, None, None) == 1
    assert rd(None, 16, FAKE, 1, 4, None, None, None, None) == 1
    assert rd(FAKE, 17, FAKE, 1, 4, None, None, None, None) == 1
    assert rd(FAKE + 4, 16, FAKE, 1, 4, None, None, None, None) == 1
    assert rd(FAKE, 16, FAKE, 0, 4, None, None, None, None) == 1
    assert rd(FAKE, 16, FAKE, 1, 3, None, None, None, None) == 1
    assert cp(FAKE, None, 16, 4, None, None, None) == 1
    assert cp(FAKE, FAKE + 8, 16, 4, None, None, None) == 1
    assert cp(FAKE, FAKE, 16, 32, None, None, None) == 1


@pytest.mark.parametrize("M,k,E,b", [(4, 2, 8, 8), (1, 8, 128, 8), (21, 8, 128, 8),
                                     (256, 8, 128, 64), (3, 2, 4, 2), (0, 8, 128, 8),
                                     (5, 3, 2, 16), (100, 1, 1, 1)])
def test_align_capacity_matches_oracle(M, k, E, b):
    assert moe.moe_align_capacity(M, k, E, b) == oracle.align_capacity(M, k, E, b)


def test_align_capacity_rejects_bad_sizes():
    assert moe.moe_align_capacity(-1, 2, 8, 8) == 0
    assert moe.moe_align_capacity(4, 0, 8, 8) == 0
    assert moe.moe_align_capacity(4, 2, 0, 8) == 0
    assert moe.moe_align_capacity(4, 2, 8, 0) == 0


def _align(ids, M, k, E, b, s=FAKE, blk=FAKE, n=FAKE, cap=None):
    if cap is None:
        cap = moe.moe_align_capacity(max(M, 0), max(k, 1), max(E, 1), max(b, 1))
    return moe.lib().moe_align(ids, M, k, E, b, s, blk, n, cap, None)


def test_align_validation():
    L = moe.lib()
    assert _align(None, 4, 2, 8, 8) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, 4, 2, 8, 8, s=None) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, -1, 2, 8, 8) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, 4, 0, 8, 8) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, 4, 2, 0, 8) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, 4, 2, 8, 0) == B.MOE_ERR_INVALID_ARG
    assert _align(FAKE, 4, 2, 4096, 8) == B.MOE_ERR_UNSUPPORTED
    cap = moe.moe_align_capacity(4, 2, 8, 8)
    assert _align(FAKE, 4, 2, 8, 8, cap=cap - 1) == B.MOE_ERR_CAPACITY
    assert _align(FAKE, 0, 2, 8, 8) == B.MOE_OK  # M == 0 is a no-op
    assert L.moe_status_str(B.MOE_ERR_CAPACITY) == b"alignment capacity too small"


def test_align_ex_workspace_and_validation():
    L = moe.lib()
    assert moe.moe_align_ex_workspace_size(1024, 8, 128) == 0          # 8192 routes: one workgroup
    n = moe.moe_align_ex_workspace_size(1025, 8, 128)                  # 8200 routes: 3 workgroups
    assert n >= (3 * 128 + 128) * 4 and n % 256 == 0
    assert moe.moe_align_ex_workspace_size(2**21, 8, 2048) >= (4096 * 2048 + 2048) * 4
    size = ctypes.c_size_t(0)
    assert L.moe_align_ex_workspace_size(4, 0, 8, ctypes.byref(size)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_align_ex_workspace_size(4, 2, 4096, ctypes.byref(size)) == B.MOE_ERR_UNSUPPORTED
    cap = moe.moe_align_capacity(4096, 8, 16, 8)
    ex = L.moe_align_ex
    assert ex(FAKE, 4, 2, 8, -1, 8, FAKE, FAKE, FAKE, 64, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert ex(FAKE, 4, 2, 8, 2**31 - 4, 8, FAKE, FAKE, FAKE, 64, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert ex(FAKE, 4096, 8, 16, 32, 8, FAKE, FAKE, FAKE, cap - 8, None, 0, None) == B.MOE_ERR_CAPACITY
    need = moe.moe_align_ex_workspace_size(4096, 8, 16)
    assert need > 0
    assert ex(FAKE, 4096, 8, 16, 32, 8, FAKE, FAKE, FAKE, cap, FAKE, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert ex(FAKE, 4096, 8, 16, 32, 8, FAKE, FAKE, FAKE, cap, FAKE + 16, need, None) == B.MOE_ERR_INVALID_ARG
    assert ex(FAKE, 0, 8, 16, 32, 8, None, None, None, 0, None, 0, None) == B.MOE_OK


def _w(fmt=B.MOE_W_INT4_AWQ, g=128, q=FAKE, s=FAKE, z=FAKE):
    return B.moe_weights(fmt, g, q, s, z)


def _desc(M=1, H=2048, I=768, E=128, k=8, b=8, path=B.MOE_PATH_AUTO, g13=128, g2=128, expert_base=0, **kw):
    return B.make_desc(M, H, I, E, k, b, _w(g=g13, **kw), _w(g=g2, **kw), path, 0, expert_base)


def _ws_status(d):
    return moe.moe_ffn_workspace_size(d, check=False)[0]


def test_workspace_size_decode_and_grouped():
    d = _desc(M=1)
    assert moe.moe_ffn_kernel_count(d) == 2
    assert moe.moe_ffn_workspace_size(d) >= 8 * 768 * 4
    dg = _desc(M=256, b=64)
    assert moe.moe_ffn_kernel_count(dg) == 4
    cap = oracle.align_capacity(256, 8, 128, 64)
    need = cap * 4 + (cap // 64) * 4 + 2048 * 768 * 2 + 2048 * (768 // 128) * 16 + 2048 * 2048 * 4
    assert moe.moe_ffn_workspace_size(dg) >= need
    off, aux, fmt = moe.moe_ffn_intermediate(dg)
    assert fmt == 2 and aux >= off + 2048 * 768 * 2
    off, lo, fmt = moe.moe_ffn_intermediate(d)
    assert fmt == 1 and lo >= off + 8 * 768 * 2
    assert [moe.moe_ffn_kernel_name(dg, i) for i in range(4)] == [
        "align_kernel", "grouped_gemm (gate/up)", "grouped_gemm (down)", "combine_topk"]
    assert moe.moe_ffn_kernel_name(dg, 4) is None
    assert [moe.moe_ffn_kernel_name(d, i) for i in range(2)] == ["decode_gate_up", "decode_down"]


def test_auto_path_threshold():
    m = moe.moe_ffn_auto_decode_max_m()
    assert moe.moe_ffn_kernel_count(_desc(M=m)) == 2
    assert moe.moe_ffn_kernel_count(_desc(M=m + 1)) == 4
    assert moe.moe_ffn_kernel_count(_desc(M=1, path=B.MOE_PATH_GROUPED)) == 4
    assert moe.moe_ffn_kernel_count(_desc(M=500, path=B.MOE_PATH_DECODE)) == 2
    rp = moe.moe_ffn_resolved_path
    assert rp(_desc(M=m)) == B.MOE_PATH_DECODE
    assert rp(_desc(M=m + 1)) == B.MOE_PATH_GROUPED
    assert rp(_desc(M=256, b=64)) == B.MOE_PATH_GROUPED
    assert rp(_desc(M=1, path=B.MOE_PATH_GROUPED)) == B.MOE_PATH_GROUPED
    # A choice whose shape rules fail falls back to the grouped path.
    assert rp(_desc(M=1, k=20)) == B.MOE_PATH_GROUPED              # decode: at most 16 routes per token
    assert rp(_desc(M=1, g13=256, g2=256, I=768, H=2048)) == B.MOE_PATH_DECODE
    assert rp(_desc(M=1, k=20, path=B.MOE_PATH_DECODE)) == -1
    assert rp(_desc(M=64, b=2048)) == B.MOE_PATH_DECODE             # grouped: blocks of at most 1024 routes
    assert rp(_desc(M=64, b=2048, path=B.MOE_PATH_GROUPED)) == -1
    assert rp(_desc(M=64, b=128)) == B.MOE_PATH_GROUPED               # in two parts of 64 columns
    # Both paths take H and I that are multiples of 32 only.
    assert rp(_desc(M=64, I=448, g2=64)) == B.MOE_PATH_GROUPED
    assert rp(_desc(M=64, H=2080, I=160, g13=32, g2=32)) == B.MOE_PATH_GROUPED
    assert rp(_desc(M=64, H=2080, I=176, g13=32, g2=32, path=B.MOE_PATH_GROUPED)) == -1
    assert rp(_desc(M=-1)) == -1


def test_desc_validation():
    assert _ws_status(_desc(M=-1)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(k=0)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(k=200, path=B.MOE_PATH_DECODE)) == B.MOE_ERR_UNSUPPORTED   # at most 16 routes per token
    assert _ws_status(_desc(k=200)) == B.MOE_OK                     # automatic path: grouped
    assert _ws_status(_desc(M=64, E=4, k=8)) == B.MOE_OK            # a shard may hold fewer experts than k
    assert _ws_status(_desc(expert_base=-1)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(expert_base=2**31 - 100)) == B.MOE_ERR_INVALID_ARG   # base + E overflows
    assert _ws_status(_desc(expert_base=2**31 - 129)) == B.MOE_OK
    assert _ws_status(_desc(b=0)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(H=2000)) == B.MOE_ERR_INVALID_ARG      # not a multiple of 32
    assert _ws_status(_desc(g13=96)) == B.MOE_ERR_INVALID_ARG      # H % g != 0
    assert _ws_status(_desc(g13=48, H=1536)) == B.MOE_ERR_INVALID_ARG  # g % 32 != 0
    assert _ws_status(_desc(q=None)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(z=None)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(q=FAKE + 4)) == B.MOE_ERR_INVALID_ARG  # weights not 16-byte aligned
    assert _ws_status(_desc(path=7)) == B.MOE_ERR_INVALID_ARG
    assert _ws_status(_desc(E=4096, k=8)) == B.MOE_ERR_UNSUPPORTED
    assert _ws_status(_desc(M=256, b=2048, path=B.MOE_PATH_GROUPED)) == B.MOE_ERR_UNSUPPORTED
    # Layers whose kernels would exceed 2^30 tasks are refused, not truncated.
    assert _ws_status(_desc(M=2**21, path=B.MOE_PATH_DECODE)) == B.MOE_ERR_UNSUPPORTED
    assert _ws_status(_desc(M=2**21, H=2**14, I=2**14, g13=512, g2=512, b=1,
                            path=B.MOE_PATH_GROUPED)) == B.MOE_ERR_UNSUPPORTED   # 2^24 blocks x 256 tiles
    assert _ws_status(_desc(M=2**21)) == B.MOE_OK                   # automatic: grouped, 25M tasks
    d = _desc()
    d.w2.fmt = B.MOE_W_MXFP8
    assert _ws_status(d) == B.MOE_ERR_INVALID_ARG                 # formats differ


def test_forward_validation_enqueues_nothing():
    L = moe.lib()
    d = _desc(M=1)
    need = moe.moe_ffn_workspace_size(d)
    fwd = L.moe_ffn_forward
    assert fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, need, None) == B.MOE_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 8, FAKE, need, None) == B.MOE_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE + 64, need, None) == B.MOE_ERR_INVALID_ARG
    assert fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.MOE_ERR_INVALID_ARG
    d0 = _desc(M=0)
    assert fwd(ctypes.byref(d0), None, None, None, None, None, 0, None) == B.MOE_OK
    # aligned variant: capacity checks
    dg = _desc(M=4, H=256, I=128, E=8, k=2, b=8, g13=64, g2=64, path=B.MOE_PATH_GROUPED)
    need = moe.moe_ffn_workspace_size(dg)
    cap = moe.moe_align_capacity(4, 2, 8, 8)
    fa = L.moe_ffn_forward_aligned
    assert fa(ctypes.byref(dg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap - 8, FAKE, FAKE, need,
              None) == B.MOE_ERR_CAPACITY
    assert fa(ctypes.byref(dg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap + 1, FAKE, FAKE, need,
              None) == B.MOE_ERR_INVALID_ARG
    assert fa(ctypes.byref(dg), FAKE, FAKE, FAKE, None, FAKE, FAKE, cap, FAKE, FAKE, need,
              None) == B.MOE_ERR_INVALID_ARG
    # capture variant: the W13 output buffer is required and 16-byte aligned
    cap_fn = L.moe_ffn_forward_capture
    dd = ctypes.byref(_desc(M=1))
    assert cap_fn(dd, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, None, None) == B.MOE_ERR_INVALID_ARG
    assert cap_fn(dd, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, FAKE + 4, None) == B.MOE_ERR_INVALID_ARG
    # profiled variant: two events (start, end) per kernel
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.moe_ffn_forward_profiled(ctypes.byref(_desc(M=1)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                      10**9, None, ev, 2) == B.MOE_ERR_INVALID_ARG


def test_mxfp8_descriptor_rules():
    # MXFP8 weights: E4M3 codes with an E8M0 exponent per 32 elements, no zeros.
    mx = lambda g=32: _w(B.MOE_W_MXFP8, g, z=None)
    for path in (B.MOE_PATH_AUTO, B.MOE_PATH_DECODE, B.MOE_PATH_GROUPED):
        d = B.make_desc(64, 2048, 768, 128, 8, 16, mx(), mx(), path, 0)
        assert _ws_status(d) == B.MOE_OK
    d = B.make_desc(64, 2048, 768, 128, 8, 16, mx(64), mx(64), B.MOE_PATH_AUTO, 0)
    assert _ws_status(d) == B.MOE_ERR_INVALID_ARG               # blocks are 32 elements
