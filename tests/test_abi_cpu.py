"""C-ABI checks that run without a GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments on the host before any HIP
call.  No test here launches a kernel."""
import ctypes
import itertools
import os
import re

import pytest

from dropless_grouped_gemm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libmoe.so not built")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced (validation fails first)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    assert fns == sorted(B.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for fn in header_functions():
        assert hasattr(L, fn), fn


def test_debug_library_exports_every_declared_symbol():
    L = B.debug_lib()
    for fn in header_functions():
        assert hasattr(L, fn), fn


def test_debug_flags_on_release_and_debug_builds():
    """The release library has no debug word: moe_debug_flags reports MOE_ENOTSUP (and 0)
    without touching a device; both builds reject a NULL output."""
    v = ctypes.c_uint32(7)
    assert B.lib().moe_debug_flags(ctypes.byref(v), 1) == B.MOE_ENOTSUP
    assert v.value == 0
    assert B.lib().moe_debug_flags(None, 0) == B.MOE_EINVAL
    assert B.debug_lib().moe_debug_flags(None, 0) == B.MOE_EINVAL
    with B.debug_library():
        assert B.lib() is B.debug_lib()
    assert B.lib() is not B.debug_lib()


def test_debug_bits_match_the_header():
    text = open(HEADER).read()
    bits = dict((n, int(v, 16)) for n, v in re.findall(r"#define (MOE_DBG_[A-Z_]+)\s+(0x[0-9a-f]+)u", text))
    assert bits == {n: getattr(B, n) for n in bits} and len(bits) == 5
    assert len(set(bits.values())) == 5 and all(v & (v - 1) == 0 for v in bits.values())


def test_status_strings():
    assert B.status_str(B.MOE_OK) == "ok"
    assert "workspace" in B.status_str(B.MOE_EWORKSPACE)
    assert B.status_str(99) == "unknown status"


def good_shape(**kw):
    base = dict(T=64, d=256, E=8, k=2, d_e=512, block_m=128, dtype="bf16")
    base.update(kw)
    return B.make_shape(**base)


BAD_SHAPES = [
    (dict(k=1025), B.MOE_ENOTSUP),
    (dict(k=0), B.MOE_EINVAL),
    (dict(d=12), B.MOE_EINVAL),                # bf16 rows must be 16-byte multiples
    (dict(d_e=4), B.MOE_EINVAL),
    (dict(T=-1), B.MOE_EINVAL),
    (dict(E=1025, k=2), B.MOE_ENOTSUP),
    (dict(n_groups=3), B.MOE_EINVAL),          # E % n_groups
    (dict(n_groups=4, topk_groups=0), B.MOE_EINVAL),
    (dict(n_groups=4, topk_groups=5), B.MOE_EINVAL),
    (dict(n_groups=128, topk_groups=1, E=128), B.MOE_ENOTSUP),
    (dict(n_groups=0, topk_groups=2), B.MOE_EINVAL),
    (dict(block_m=0), B.MOE_EINVAL),
    (dict(block_m=32), B.MOE_ENOTSUP),         # bf16 grouped GEMM works in 128-row tiles
    (dict(d_e_shared=12), B.MOE_EINVAL),
    (dict(T=1 << 29, k=4), B.MOE_EINVAL),      # T*k >= 2^31
    # the padded bound fits 2^31 rows (2^31 - 128), the unpadded table's
    # (ceil(T*k / 128) + E - 1) * 128 does not
    (dict(T=16776199 * 128, k=1, E=1024, unpadded=1), B.MOE_EINVAL),
]


def test_routing_needs_k_at_most_E_but_routed_rows_may_repeat_experts():
    """k > E is a valid shape for rows that arrive already routed (duplicates within a
    token), but the router itself cannot pick k distinct experts out of E."""
    L = B.lib()
    s = good_shape(k=9)
    ps = ctypes.byref(s)
    assert L.moe_max_blocks(ps) > 0
    assert L.moe_route(ps, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 40, None) == B.MOE_EINVAL
    need = L.moe_workspace_bytes(ps)
    # without given routes the layer must route: rejected
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, FAKE, need, None) == B.MOE_EINVAL
    s2 = good_shape(n_groups=4, topk_groups=1, k=3)
    assert L.moe_route(ctypes.byref(s2), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 40,
                       None) == B.MOE_EINVAL
    assert L.moe_max_blocks(ctypes.byref(s2)) > 0


@pytest.mark.parametrize("kw,status", BAD_SHAPES)
def test_invalid_shapes_rejected_by_every_entry_point(kw, status):
    L = B.lib()
    s = good_shape(**kw)
    ps = ctypes.byref(s)
    assert L.moe_max_blocks(ps) == -1
    assert L.moe_max_rows(ps) == -1
    assert L.moe_workspace_bytes(ps) == 0
    assert L.moe_route(ps, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 40, None) == status
    assert L.moe_build_offsets(ps, *([FAKE] * 9), FAKE, 1 << 40, None) == status
    assert L.moe_permute(ps, FAKE, FAKE, FAKE, None) == status
    assert L.moe_grouped_gemm(ps, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == status
    assert L.moe_grouped_gemm_shared(ps, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                     FAKE, FAKE, FAKE, FAKE, None) == status
    assert L.moe_combine(ps, FAKE, FAKE, FAKE, None, FAKE, None) == status
    assert L.moe_layer_fwd(ps, *([FAKE] * 6), None, None, None, None, None, FAKE, FAKE,
                           1 << 40, None) == status
    assert L.moe_grouped_gemm_gather(ps, *([FAKE] * 6), 1, FAKE, None, None, None,
                                     None) == status


def test_null_and_misaligned_pointers_rejected():
    L = B.lib()
    s = good_shape()
    ps = ctypes.byref(s)
    odd = ctypes.c_void_p(0x10008)           # 8-byte aligned only
    assert L.moe_route(ps, None, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_route(ps, odd, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert L.moe_permute(ps, FAKE, FAKE, odd, None) == B.MOE_EINVAL
    assert L.moe_permute(ps, FAKE, None, FAKE, None) == B.MOE_EINVAL
    # op-specific operand rules of the grouped GEMM
    assert L.moe_grouped_gemm(ps, 0, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 7, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None) == B.MOE_EINVAL
    mb = L.moe_max_blocks(ps)
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, FAKE, FAKE, mb + 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 0, FAKE, None) == B.MOE_EINVAL
    # dense mode: block table and count both NULL, max_blocks 0; half of the pair is an error
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, None, FAKE, 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, FAKE, None, 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, None, None, 1, FAKE, None) == B.MOE_EINVAL
    assert L.moe_grouped_gemm(ps, 1, FAKE, FAKE, None, None, None, -1, FAKE, None) == B.MOE_EINVAL
    s0 = good_shape(T=0)
    assert L.moe_grouped_gemm(ctypes.byref(s0), 1, FAKE, FAKE, None, None, None, 0, FAKE,
                              None) == B.MOE_OK
    # layer: shared-expert pointers must match d_e_shared; routing pair all-or-nothing
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                           FAKE, FAKE, 1 << 40, None) == B.MOE_EINVAL
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                           FAKE, FAKE, 1 << 40, None) == B.MOE_EINVAL
    assert L.moe_layer_fwd(ps, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, FAKE, 1 << 40, None) == B.MOE_EINVAL
    s2 = good_shape(d_e_shared=256)
    assert L.moe_layer_fwd(ctypes.byref(s2), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None,
                           None, None, FAKE, FAKE, 1 << 40, None) == B.MOE_EINVAL


def test_grouped_gemm_shared_argument_rules():
    L = B.lib()
    s = good_shape(d_e_shared=256)
    ps = ctypes.byref(s)
    mb = L.moe_max_blocks(ps)
    g = L.moe_grouped_gemm_shared
    odd = ctypes.c_void_p(0x10008)
    # needs a shared expert in the shape
    s0 = good_shape()
    assert g(ctypes.byref(s0), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == B.MOE_EINVAL
    # op rules apply to both halves
    assert g(ps, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_EINVAL
    assert g(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_EINVAL
    assert g(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, odd, FAKE, None, FAKE, None) == B.MOE_EINVAL
    assert g(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, None, None) == B.MOE_EINVAL
    assert g(ps, 2, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_EINVAL
    # the routed half needs its block table
    assert g(ps, 1, FAKE, FAKE, None, None, None, 0, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_EINVAL
    assert g(ps, 1, FAKE, FAKE, None, FAKE, FAKE, mb + 1, FAKE, FAKE, FAKE, None, FAKE,
             None) == B.MOE_EINVAL
    assert g(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_EINVAL
    # T == 0: validated, nothing launched
    sT = good_shape(T=0, d_e_shared=256)
    assert g(ctypes.byref(sT), 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE,
             None) == B.MOE_EINVAL      # max_blocks must be <= moe_max_blocks = 0
    assert L.moe_max_blocks(ctypes.byref(sT)) == 0


def test_workspace_too_small_rejected_before_launch():
    L = B.lib()
    s = good_shape()
    ps = ctypes.byref(s)
    need = L.moe_workspace_bytes(ps)
    assert need > 0
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, FAKE, need - 1, None) == B.MOE_EWORKSPACE
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, None, need, None) == B.MOE_EWORKSPACE
    assert L.moe_route(ps, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0, None) == B.MOE_EWORKSPACE
    assert L.moe_build_offsets(ps, *([FAKE] * 9), FAKE, 16, None) == B.MOE_EWORKSPACE


def test_empty_batch_is_a_noop():
    """T == 0 validates and returns OK without touching the device."""
    L = B.lib()
    s = good_shape(T=0)
    ps = ctypes.byref(s)
    assert L.moe_max_blocks(ps) == 0 and L.moe_max_rows(ps) == 0
    need = L.moe_workspace_bytes(ps)
    assert L.moe_layer_fwd(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, FAKE, need, None) == B.MOE_OK
    assert L.moe_permute(ps, FAKE, FAKE, FAKE, None) == B.MOE_OK
    assert L.moe_combine(ps, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_OK
    assert L.moe_route(ps, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0, None) == B.MOE_OK


def _max_blocks_brute(M, E, bm):
    best = 0
    for c in itertools.product(range(M + 1), repeat=E):
        if sum(c) == M:
            best = max(best, sum(-(-x // bm) for x in c))
    return best


@pytest.mark.parametrize("M,E,bm", [(M, E, bm) for M in range(1, 7) for E in (1, 2, 3)
                                    for bm in (1, 2, 3, 4)])
def test_max_blocks_is_the_exact_worst_case(M, E, bm):
    """moe_max_blocks is the largest sum_e ceil(c_e / bm) over every way of splitting
    M assignments over E experts (brute force), so it bounds the real block count."""
    s = B.make_shape(T=M, d=4, E=E, k=1, d_e=4, block_m=bm, dtype="fp32")
    assert B.moe_max_blocks(s) == _max_blocks_brute(M, E, bm)
    assert B.moe_max_rows(s) == B.moe_max_blocks(s) * bm


def test_workspace_layout_is_disjoint_and_aligned():
    for kw in (dict(), dict(d_e_shared=256), dict(T=8192, d=7168, E=8, k=4, d_e=2048, d_e_shared=2048),
               dict(T=64, d=7168, E=256, k=8, d_e=2048, n_groups=8, topk_groups=4, d_e_shared=2048)):
        s = good_shape(**kw)
        L = B.moe_workspace_layout(s)
        assert L["total"] == B.moe_workspace_bytes(s)
        names = [n for n in L if n != "total"]
        offs = sorted(L[n] for n in names)
        assert all(o % 256 == 0 for o in offs)
        assert len(set(offs)) == len(offs) or True   # zero-sized fields may share an offset
        rows = B.moe_max_rows(s)
        # bf16 with d % 32 == 0: the permute is fused into the gate/up loads and x_perm
        # takes no room
        assert L["act"] - L["x_perm"] == 0
        assert L["y"] - L["act"] >= rows * s.d_e * 2
        assert L["total"] > L["scratch"]


def test_grouped_gemm_gather_argument_rules():
    """The fused-permute gate/up: bf16 with d % 32 == 0 only (else ENOTSUP), the block
    table as for moe_grouped_gemm, shared-expert operands matching d_e_shared."""
    L = B.lib()
    g = L.moe_grouped_gemm_gather
    odd = ctypes.c_void_p(0x10008)
    s32 = B.make_shape(T=8, d=64, E=2, k=1, d_e=32, block_m=16, dtype="fp32")
    s_k = good_shape(d=72)
    for s in (s32, s_k):
        assert not B.gather_supported(s)
        assert g(ctypes.byref(s), *([FAKE] * 6), 1, FAKE, None, None, None, None) == B.MOE_ENOTSUP
    s = good_shape()
    ps = ctypes.byref(s)
    assert B.gather_supported(s)
    mb = L.moe_max_blocks(ps)
    ok = lambda *a: g(ps, *a, None)
    assert ok(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, None, None) == B.MOE_EINVAL
    assert ok(odd, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, None, None) == B.MOE_EINVAL
    assert ok(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None, None, None) == B.MOE_EINVAL
    assert ok(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, FAKE, None, None, None) == B.MOE_EINVAL
    assert ok(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mb + 1, FAKE, None, None, None) == B.MOE_EINVAL
    assert ok(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None, None) == B.MOE_EINVAL
    # no shared expert in the shape: its operands must be NULL
    assert ok(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL
    s2 = good_shape(d_e_shared=256)
    ps2 = ctypes.byref(s2)
    assert g(ps2, *([FAKE] * 6), 1, FAKE, None, None, None, None) == B.MOE_EINVAL
    sT = good_shape(T=0)
    assert g(ctypes.byref(sT), *([FAKE] * 6), 0, FAKE, None, None, None, None) == B.MOE_EINVAL


def test_fp8_entry_point_argument_rules():
    """fp8 weights: bf16 activations with 128-row blocks only; codes/scales pairs per
    op; shared-expert operands all or nothing; bad sizes rejected before any launch."""
    L = B.lib()
    q = L.moe_quantize_fp8
    assert q(0, 128, 128, FAKE, FAKE, FAKE, None) == B.MOE_EINVAL
    assert q(1, 128, 12, FAKE, FAKE, FAKE, None) == B.MOE_EINVAL          # N % 8
    assert q(1, 128, 128, None, FAKE, FAKE, None) == B.MOE_EINVAL
    assert q(1, 128, 128, FAKE, ctypes.c_void_p(0x10004), FAKE, None) == B.MOE_EINVAL
    g = L.moe_grouped_gemm_fp8
    s = good_shape()
    ps = ctypes.byref(s)
    mb = L.moe_max_blocks(ps)
    n6 = [None] * 6
    # fp32 activations, or 256-row blocks: not supported
    for bad in (good_shape(dtype="fp32", block_m=128), good_shape(block_m=256), good_shape(d=272)):
        assert g(ctypes.byref(bad), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE,
                 *n6, None, 0, None) == B.MOE_ENOTSUP
    assert B.fp8_supported(s) and not B.fp8_supported(good_shape(d=272))
    ok = lambda op, *a: g(ps, op, *a, None, 0, None)
    assert ok(0, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1, None, FAKE, *n6) == B.MOE_EINVAL
    assert ok(1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, *n6) == B.MOE_EINVAL
    assert ok(0, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, *n6) == B.MOE_EINVAL
    assert ok(1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, mb + 1, None, FAKE, *n6) == B.MOE_EINVAL
    assert ok(1, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1, FAKE, FAKE, *n6) == B.MOE_EINVAL  # gather on down
    # shared operands with no shared expert in the shape
    assert ok(0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE,
              FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == B.MOE_EINVAL
    lf = L.moe_layer_fwd_fp8
    need = L.moe_fp8_workspace_bytes(ps)
    # no router weights and no given routes; and a shared-expert pointer without one
    assert lf(ps, FAKE, None, None, *([FAKE] * 6), *([None] * 6), None, None, FAKE, FAKE, need,
              None) == B.MOE_EINVAL
    assert lf(ps, FAKE, FAKE, None, *([FAKE] * 6), FAKE, *([None] * 5), None, None, FAKE, FAKE,
              need, None) == B.MOE_EINVAL
    least = L.moe_workspace_bytes(ps)
    assert lf(ps, FAKE, FAKE, None, *([FAKE] * 6), *([None] * 6), None, None, FAKE, FAKE,
              least - 1, None) == B.MOE_EWORKSPACE
    # the optional scratch of the GEMM: too small or misaligned is an error, NULL is none
    args = (0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, *n6)
    sk = L.moe_grouped_gemm_fp8_workspace_bytes(ps)
    assert sk == 256 + 2 * 256 * 64 * 1024 * 4
    assert g(ps, *args, FAKE, sk - 1, None) == B.MOE_EWORKSPACE
    assert g(ps, *args, ctypes.c_void_p(0x10004), sk, None) == B.MOE_EWORKSPACE


def test_fp8_layer_workspace_holds_the_streaming_scratch():
    """Where experts average at most 64 rows the fp8 layer's full workspace ends with the
    GEMM's last-round scratch; elsewhere it does not."""
    L = B.lib()
    dec = good_shape(T=64, d=256, E=64, k=4, d_e=256)          # 4 rows per expert
    pre = good_shape(T=4096, d=256, E=8, k=2, d_e=256)         # 1024 rows per expert
    mid = good_shape(T=1024, d=256, E=8, k=1, d_e=256)         # 128 rows per expert
    sk = L.moe_grouped_gemm_fp8_workspace_bytes(ctypes.byref(dec))
    for shp, extra in ((dec, True), (pre, False), (mid, False)):
        p = ctypes.byref(shp)
        base, full = L.moe_workspace_bytes(p), L.moe_fp8_workspace_bytes(p)
        if extra:
            assert full == base + sk
        else:
            assert full < base + sk


def test_forward_router_needs_a_16_byte_aligned_w_gate():
    """The forward router stages W_g slices with 16-byte copies: moe_route, moe_layer_fwd and
    moe_layer_fwd_fp8 reject a W_g that is only 4-byte aligned (EINVAL, nothing launched)
    and accept an aligned one."""
    L = B.lib()
    s = good_shape(T=64, d=256, E=8, k=2)
    ps = ctypes.byref(s)
    w4 = ctypes.c_void_p(0x10004)
    need = L.moe_workspace_bytes(ps)
    assert L.moe_route(ps, FAKE, w4, None, None, FAKE, FAKE, FAKE, need, None) == B.MOE_EINVAL
    assert L.moe_layer_fwd(ps, FAKE, w4, None, FAKE, FAKE, FAKE, None, None, None, None, None,
                           FAKE, FAKE, need, None) == B.MOE_EINVAL
    need8 = L.moe_fp8_workspace_bytes(ps)
    assert L.moe_layer_fwd_fp8(ps, FAKE, w4, None, *([FAKE] * 6), *([None] * 6), None, None, FAKE,
                               FAKE, need8, None) == B.MOE_EINVAL
    s0 = good_shape(T=0)                      # T == 0 enqueues nothing: validation only
    p0 = ctypes.byref(s0)
    assert L.moe_route(p0, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.MOE_OK
    assert L.moe_route(p0, FAKE, w4, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.MOE_EINVAL


def test_fp8_layer_accepts_the_minimal_workspace():
    """moe_layer_fwd_fp8 takes any workspace of at least moe_workspace_bytes (then the wide
    kernel dequantises in registers); moe_fp8_workspace_bytes adds the room for the
    dequantised weights (then they are dequantised once).  One byte short of the minimum
    is MOE_EWORKSPACE.  T = 0: validation only, nothing is launched."""
    L = B.lib()
    s = good_shape(T=0, d_e_shared=0)
    ps = ctypes.byref(s)
    lo = L.moe_workspace_bytes(ps)
    args = lambda n: (ps, FAKE, FAKE, None, *([FAKE] * 6), *([None] * 6), None, None, FAKE, FAKE, n,
                      None)
    assert L.moe_layer_fwd_fp8(*args(lo)) == B.MOE_OK
    assert L.moe_layer_fwd_fp8(*args(lo - 1)) == B.MOE_EWORKSPACE


def test_fp8_workspace_size_rule():
    """moe_fp8_workspace_bytes: moe_workspace_bytes's layout, plus room for the
    dequantised bf16 weights exactly where the layer takes the dequantised path (routed
    rows M = T * k at least 256 * min(E, M)), or for the streaming GEMM's last-round
    scratch exactly where experts average at most 64 rows."""
    L = B.lib()
    for kw in (dict(T=64), dict(T=1023), dict(T=1024), dict(T=4096, d_e_shared=512),
               dict(T=0), dict(T=70, E=1, k=4), dict(T=512, E=300, k=8)):
        s = good_shape(**kw)
        base, f8 = L.moe_workspace_bytes(ctypes.byref(s)), L.moe_fp8_workspace_bytes(ctypes.byref(s))
        M = s.T * s.k
        wide = M > 0 and M >= 256 * min(s.E, M)
        streaming = M > 0 and M <= 64 * min(s.E, M)
        assert B.fp8_dequantises(s) == wide, kw
        w = 2 * (3 * s.E * s.d * s.d_e + 3 * s.d * s.d_e_shared)
        if wide:
            assert w <= f8 - base <= w + 6 * 256, kw
        elif streaming:
            assert f8 - base == L.moe_grouped_gemm_fp8_workspace_bytes(ctypes.byref(s)), kw
        else:
            assert f8 == base, kw
    assert L.moe_fp8_workspace_bytes(ctypes.byref(good_shape(k=0))) == 0


def test_dequantize_fp8_argument_rules():
    """Sizes and pointers checked before any launch: N a multiple of 8, q 8-byte and w
    16-byte aligned, scales 4-byte aligned."""
    L = B.lib()
    dq = L.moe_dequantize_fp8
    F16 = ctypes.c_void_p(0x10000)
    assert dq(1, 128, 12, F16, F16, F16, None) == B.MOE_EINVAL
    assert dq(0, 128, 16, F16, F16, F16, None) == B.MOE_EINVAL
    assert dq(1, 0, 16, F16, F16, F16, None) == B.MOE_EINVAL
    assert dq(1, 128, 16, None, F16, F16, None) == B.MOE_EINVAL
    assert dq(1, 128, 16, F16, F16, None, None) == B.MOE_EINVAL
    assert dq(1, 128, 16, ctypes.c_void_p(0x10004), F16, F16, None) == B.MOE_EINVAL
    assert dq(1, 128, 16, F16, F16, ctypes.c_void_p(0x10008), None) == B.MOE_EINVAL
    assert dq(1, 128, 16, F16, ctypes.c_void_p(0x10002), F16, None) == B.MOE_EINVAL


def test_backward_entry_point_argument_rules():
    """Backward: bf16 with d, d_e, d_e_shared multiples of 32 (else ENOTSUP); operand
    pairs per op; the block table or the dense mode; workspaces checked before launch.
    Every call here fails validation, so nothing is launched."""
    L = B.lib()
    odd = ctypes.c_void_p(0x10008)
    s = good_shape()
    ps = ctypes.byref(s)
    mb = L.moe_max_blocks(ps)
    assert B.backward_supported(s)
    for bad in (good_shape(dtype="fp32"), good_shape(d=264), good_shape(d_e=520),
                good_shape(d_e_shared=40)):
        pb = ctypes.byref(bad)
        assert not B.backward_supported(bad)
        assert L.moe_combine_bwd(pb, *([FAKE] * 6), None) == B.MOE_ENOTSUP
        assert L.moe_swiglu_bwd(pb, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                *([None] * 5), None) == B.MOE_ENOTSUP
        assert L.moe_grouped_gemm_dgrad(pb, 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE,
                                        None, 0, None) == B.MOE_ENOTSUP
        assert L.moe_grouped_gemm_wgrad(pb, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                        None, 0, None) == B.MOE_ENOTSUP
        assert L.moe_router_bwd(pb, *([FAKE] * 10), FAKE, 1 << 40, None) == B.MOE_ENOTSUP
    assert L.moe_combine_bwd(ctypes.byref(good_shape(d=8224)), *([FAKE] * 6), None) == B.MOE_ENOTSUP
    # combine backward: every pointer required
    assert L.moe_combine_bwd(ps, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.MOE_EINVAL
    assert L.moe_combine_bwd(ps, odd, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MOE_EINVAL
    # SwiGLU backward: dact required, block table checked, shared operands all or none
    sb = L.moe_swiglu_bwd
    assert sb(ps, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, *([None] * 5), None) == B.MOE_EINVAL
    assert sb(ps, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, 1, FAKE, *([None] * 5), None) == B.MOE_EINVAL
    assert sb(ps, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, mb + 1, FAKE, *([None] * 5),
              None) == B.MOE_EINVAL
    assert sb(ps, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
              None) == B.MOE_EINVAL                        # no shared expert in the shape
    s2 = good_shape(d_e_shared=256)
    assert sb(ctypes.byref(s2), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
              None, FAKE, None) == B.MOE_EINVAL            # shared dact missing
    # dgrad: op rules, dense mode all-or-nothing
    dg = L.moe_grouped_gemm_dgrad
    assert dg(ps, 0, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None, 0, None) == B.MOE_EINVAL
    assert dg(ps, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 0, None) == B.MOE_EINVAL
    assert dg(ps, 3, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, None, 0, None) == B.MOE_EINVAL
    assert dg(ps, 1, FAKE, FAKE, None, None, FAKE, 1, FAKE, None, 0, None) == B.MOE_EINVAL
    assert dg(ps, 1, FAKE, FAKE, None, None, None, 1, FAKE, None, 0, None) == B.MOE_EINVAL
    assert dg(ps, 1, FAKE, FAKE, None, FAKE, FAKE, mb + 1, FAKE, None, 0, None) == B.MOE_EINVAL
    # a workspace selects the transposed-weight path and must hold the transposed weights
    need = L.moe_grouped_gemm_dgrad_workspace_bytes(ps, 0)
    assert need == -(-2 * s.E * s.d * s.d_e * 2 // 256) * 256
    assert dg(ps, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, need - 1, None) == B.MOE_EWORKSPACE
    assert dg(ps, 1, FAKE, FAKE, None, FAKE, FAKE, 1, FAKE, ctypes.c_void_p(0x10008),
              1 << 40, None) == B.MOE_EWORKSPACE
    # wgrad: dB1 exactly for gate/up; counts and offsets together
    wg = L.moe_grouped_gemm_wgrad
    assert wg(ps, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_EINVAL
    assert wg(ps, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.MOE_EINVAL
    assert wg(ps, 1, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == B.MOE_EINVAL
    assert wg(ps, 1, odd, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_EINVAL
    # the work-queue scratch: (E + 64) int32, 16-byte aligned, or NULL
    wneed = L.moe_grouped_gemm_wgrad_workspace_bytes(ps)
    assert wneed == -(-(s.E + 64) * 4 // 256) * 256
    assert wg(ps, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, (s.E + 64) * 4 - 1,
              None) == B.MOE_EWORKSPACE
    assert wg(ps, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, odd, wneed, None) == B.MOE_EWORKSPACE
    # router backward: dbias and dx_in optional, the rest required
    rb = L.moe_router_bwd
    big = 1 << 40
    assert rb(ps, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, big,
              None) == B.MOE_EINVAL
    assert rb(ps, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, big,
              None) == B.MOE_EINVAL
    # the token-chunk partial sums need their scratch once the tokens are split
    sw = good_shape(T=8192, d=7168, E=8, k=4)
    need = L.moe_router_bwd_workspace_bytes(ctypes.byref(sw))
    assert need > 0
    assert rb(ctypes.byref(sw), *([FAKE] * 10), FAKE, need - 1, None) == B.MOE_EWORKSPACE
    assert rb(ctypes.byref(sw), *([FAKE] * 10), None, need, None) == B.MOE_EWORKSPACE
    # layer backward: workspaces, routing pair, shared operands, router-only outputs
    lb = L.moe_layer_bwd
    fwd_need, bwd_need = L.moe_workspace_bytes(ps), L.moe_bwd_workspace_bytes(ps)
    assert bwd_need > 0
    args = lambda **o: [o.get(n, v) for n, v in (
        ("x", FAKE), ("w_gate", FAKE), ("w1", FAKE), ("w3", FAKE), ("w2", FAKE), ("ws1", None),
        ("ws3", None), ("ws2", None), ("idx", None), ("tw", None), ("dout", FAKE),
        ("fws", FAKE), ("fwb", fwd_need), ("dx", FAKE), ("dw1", FAKE), ("dw3", FAKE),
        ("dw2", FAKE), ("dws1", None), ("dws3", None), ("dws2", None), ("dwg", FAKE),
        ("db", None), ("dtw", None), ("ws", FAKE), ("wsb", bwd_need))]
    assert lb(ps, *args(fwb=fwd_need - 1), None) == B.MOE_EWORKSPACE
    assert lb(ps, *args(wsb=bwd_need - 1), None) == B.MOE_EWORKSPACE
    assert lb(ps, *args(ws=None), None) == B.MOE_EWORKSPACE
    assert lb(ps, *args(idx=FAKE), None) == B.MOE_EINVAL                  # half a routing pair
    assert lb(ps, *args(idx=FAKE, tw=FAKE), None) == B.MOE_EINVAL         # dW_g with given routes
    assert lb(ps, *args(w_gate=None), None) == B.MOE_EINVAL
    assert lb(ps, *args(dw2=None), None) == B.MOE_EINVAL
    assert lb(ps, *args(ws1=FAKE), None) == B.MOE_EINVAL                   # no shared expert
    assert lb(ctypes.byref(s2), *args(), None) == B.MOE_EINVAL            # shared expert missing


def test_backward_workspace_layout_is_disjoint_and_aligned():
    for kw in (dict(), dict(d_e_shared=256), dict(T=8192, d=7168, E=8, k=4, d_e=2048, d_e_shared=2048)):
        s = good_shape(**kw)
        L = B.moe_bwd_workspace_layout(s)
        assert L["total"] == B.moe_bwd_workspace_bytes(s)
        rows, T, d, de, ds = B.moe_max_rows(s), s.T, s.d, s.d_e, s.d_e_shared
        sizes = dict(dy=rows * d * 2, dact=rows * de * 2, dgu=rows * 2 * de * 2, x_perm=rows * d * 2,
                     dx_perm=rows * d * 2, dtopk_w=T * s.k * 4, dlogits=T * s.E * 4,
                     shared_dact=T * ds * 2, shared_dgu=T * 2 * ds * 2,
                     shared_dx=T * d * 2 if ds else 0, router_dx=T * d * 2,
                     router_scratch=B.moe_router_bwd_workspace_bytes(s),
                     wgrad_sched=(s.E + 64) * 4)
        tw = T * s.k >= 256 * min(s.E, T * s.k)           # data gradients on transposed weights
        sizes.update(w2_t=s.E * d * de * 2 if tw else 0, w13_t=2 * s.E * de * d * 2 if tw else 0,
                     ws2_t=d * ds * 2 if tw else 0, ws13_t=2 * ds * d * 2 if tw else 0)
        spans = sorted((L[n], L[n] + sz) for n, sz in sizes.items() if sz)
        assert all(o % 256 == 0 for o, _ in spans)
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[-1][1] <= L["total"]


@pytest.mark.parametrize("M,E,bm", [(M, E, bm) for M in range(1, 8) for E in (1, 2, 3)
                                    for bm in (1, 2, 3, 4)])
def test_unpadded_max_blocks_bounds_every_table(M, E, bm):
    """Unpadded layout: moe_max_blocks bounds the number of (tile, expert) entries of every
    way of splitting M rows over E experts (brute force over the oracle's table), is
    reached whenever tiles can hold every boundary, and the permuted buffers have M rows."""
    from oracle import moe_oracle as O
    s = B.make_shape(T=M, d=4, E=E, k=1, d_e=4, block_m=bm, dtype="fp32", unpadded=True)
    worst = 0
    for c in itertools.product(range(M + 1), repeat=E):
        if sum(c) == M:
            worst = max(worst, len(O.unpadded_tile_table(c, bm)))
    assert worst <= B.moe_max_blocks(s)
    if bm > 1 and M >= bm * min(E, M):
        assert worst == B.moe_max_blocks(s)
    assert B.moe_max_rows(s) == M
    L = B.moe_workspace_layout(s)
    assert L["act"] - L["x_perm"] >= M * s.d * 4


def test_workspace_has_no_x_perm_where_the_permute_is_fused():
    """bf16 with d % 32 == 0 gathers x's rows in the gate/up loads: the workspace holds
    no x_perm there (forward and fp8 forward), and shrinks by max_rows * d * 2 bytes
    against a shape that needs it (d % 32 != 0); the fp32 path keeps it."""
    kw = dict(T=600, E=8, k=4, d_e=256, block_m=128)
    fused = good_shape(d=512, **kw)
    assert B.gather_supported(fused)
    L = B.moe_workspace_layout(fused)
    assert L["act"] == L["x_perm"]
    rows = B.moe_max_rows(fused)
    need = L["act"] + rows * 256 * 2
    assert L["y"] >= need
    assert B.moe_fp8_workspace_bytes(fused) >= B.moe_workspace_bytes(fused)
    unfused = good_shape(d=520, **kw)                  # d % 32 != 0: permute, then GEMM
    assert not B.gather_supported(unfused)
    Lu = B.moe_workspace_layout(unfused)
    assert Lu["act"] - Lu["x_perm"] >= B.moe_max_rows(unfused) * 520 * 2
    f32 = B.make_shape(T=600, d=512, E=8, k=4, d_e=256, block_m=128, dtype="fp32")
    Lf = B.moe_workspace_layout(f32)
    assert Lf["act"] - Lf["x_perm"] >= B.moe_max_rows(f32) * 512 * 4


def test_unpadded_flag_is_validated():
    L = B.lib()
    s = good_shape()
    s.unpadded = 2
    assert L.moe_max_blocks(ctypes.byref(s)) == -1
