"""fp8 (e4m3) expert weights on the GPU, through the C ABI, against the fp8 oracle.

  * the quantiser's codes and scales are integers / fp32 values decided in fp32 on both
    sides: bit-exact;
  * a grouped-GEMM stage with fp8 weights is compared with the fp64 product by the
    exactly dequantised weights.  The device rounds each dequantised weight to bf16
    (<= 2^-9 relative) before the MFMA and rounds its output to bf16 (<= 2^-9), with
    fp32 accumulation in between; with random signs the weight roundings add up like
    a random walk, well inside 1e-2 * max|ref| (TOL_STAGE_FP8);
  * the layer output keeps the stated bound 2e-2 * max|ref|.
"""
import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B
from oracle import fp8_oracle as F
from oracle import moe_oracle as O
from workloads import get_config, make_inputs

from gpu_util import TOL_OUT, assert_close, f64, i64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_STAGE_FP8 = 1e-2


@pytest.mark.parametrize("E,K,N", [(2, 300, 200), (3, 256, 384), (1, 7168, 256), (4, 128, 8)])
def test_quantize_is_bit_exact(E, K, N):
    g = torch.Generator(device=DEV)
    g.manual_seed(E * 1000 + K + N)
    w = (torch.randn((E, K, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    if K >= 256 and N >= 128:
        w[0, 128:256, 0:128] = 0                       # an all-zero block
        w[-1, 3, 5] = 30.0                             # one large weight in a block
        w[-1, 4, 6] = -1e-30                           # a value that flushes to a zero code
    q, s = B.quantize_fp8(w)
    torch.cuda.synchronize()
    rq, rs = F.quantize(w.float().cpu().numpy())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("E,K,N", [(2, 300, 200), (1, 7168, 256), (3, 128, 8)])
def test_dequantize_is_bit_exact(E, K, N):
    """Every e4m3 code (NaNs aside) times fp32 block scales, rounded once to fp32 and
    then to bf16 (nearest even): the decode is the oracle's code table, the two
    roundings numpy's and torch's CPU casts."""
    rng = np.random.default_rng(E + K + N)
    codes = rng.integers(0, 256, size=(E, K, N)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    kb, nb = -(-K // 128), -(-N // 128)
    scales = (rng.uniform(0.5, 2.0, size=(E, kb, nb)) *
              2.0 ** rng.integers(-12, 4, size=(E, kb, nb))).astype(np.float32)
    w = B.dequantize_fp8(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    full = np.repeat(np.repeat(scales, 128, axis=1), 128, axis=2)[:, :K, :N]
    prod = F.e4m3_decode(codes).astype(np.float32) * full          # fp32 product, RNE
    ref = torch.from_numpy(prod).to(torch.bfloat16)
    assert torch.equal(w.cpu().view(torch.int16), ref.view(torch.int16))


def _routes(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, E, size=(T, k))


@pytest.mark.parametrize("T,d,E,k,d_e,d_es", [
    (200, 512, 8, 2, 256, 256),      # shared expert in the same launch
    (64, 1024, 16, 4, 128, 0),       # decode-like: few rows per expert
    (150, 256, 4, 2, 384, 128),      # shared expert in launches of its own; ragged n-blocks
    (40, 1280, 3, 3, 160, 0),        # partial 128-blocks in both k and n
    (300, 256, 2, 1, 1056, 96),      # blocks of 128 valid rows: both 64-row halves; N tails
    (64, 2048, 64, 8, 768, 768),     # decode-like: 512 rows over 64 experts + shared
])
@pytest.mark.parametrize("item_rows", ["64", "128", "384"])
def test_grouped_gemm_fp8_against_oracle(T, d, E, k, d_e, d_es, item_rows, monkeypatch):
    """Every fp8 kernel (64-row items with wide weight rows, 128-row items, the wide
    kernel's 384-row groups) on every shape, forced with MOE_FP8_ITEM_ROWS."""
    monkeypatch.setenv("MOE_FP8_ITEM_ROWS", item_rows)
    idx = _routes(T, E, k, T + d)
    g = torch.Generator(device=DEV)
    g.manual_seed(T + d_e)
    dt = torch.bfloat16
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    (q1, s1), (q3, s3), (q2, s2) = B.quantize_fp8(w1), B.quantize_fp8(w3), B.quantize_fp8(w2)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16", d_e_shared=d_es)
    assert B.fp8_supported(s)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    ws = B.alloc_workspace(s)
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err, ws)
    x_perm = torch.empty((rows, d), dtype=dt, device=DEV)
    B.moe_permute(s, x, pos, x_perm)
    e = lambda *sh: torch.empty(sh, dtype=dt, device=DEV)
    act, act_g, y = e(rows, d_e), e(rows, d_e), e(rows, d)
    sh = {}
    if d_es:
        ws1 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        ws3 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        ws2 = (torch.randn((d_es, d), generator=g, device=DEV) / d_es ** 0.5).to(dt)
        (qa, sa), (qb, sb), (qc, sc) = B.quantize_fp8(ws1), B.quantize_fp8(ws3), B.quantize_fp8(ws2)
        sact, sact_g, sout = e(T, d_es), e(T, d_es), e(T, d)
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, q1, s1, q3, s3, meta, nblk, mb,
                               None, act, x, qa, sa, qb, sb, sact)
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x, q1, s1, q3, s3, meta, nblk, mb,
                               row_src, act_g, x, qa, sa, qb, sb, sact_g)
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_DOWN, act, q2, s2, None, None, meta, nblk, mb, None, y,
                               sact, qc, sc, None, None, sout)
    else:
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, q1, s1, q3, s3, meta, nblk, mb,
                               None, act)
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x, q1, s1, q3, s3, meta, nblk, mb,
                               row_src, act_g)
        B.moe_grouped_gemm_fp8(s, B.MOE_OP_DOWN, act, q2, s2, None, None, meta, nblk, mb, None, y)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_pos, ref_src = O.permutation(idx, E, 128)
    valid = np.nonzero(ref_src >= 0)[0]
    dv = torch.from_numpy(valid).to(DEV)
    # the fused gather is the same arithmetic on the same rows: bit-exact
    assert torch.equal(act[dv].view(torch.int16), act_g[dv].view(torch.int16))
    c = O.expert_counts(idx, E)
    xp_ref = O.permute(f64(x), ref_pos, k, len(ref_src))
    def dq(qq, ss):
        qn, sn = qq.cpu().numpy(), ss.cpu().numpy()
        return F.dequantize(qn.reshape((-1,) + qn.shape[-2:]), sn.reshape((-1,) + sn.shape[-2:]))
    W1, W3, W2 = dq(q1, s1), dq(q3, s3), dq(q2, s2)
    act_ref, _ = O.grouped_ffn(xp_ref, c, 128, W1, W3, W2)
    assert_close(f64(act)[valid], act_ref[valid], TOL_STAGE_FP8, "act")
    # down on the device's own act
    act_dev = f64(act)
    P = O.padded_offsets(c, 128)
    y_ref = np.zeros((len(ref_src), d))
    for ex in range(E):
        lo, hi = P[ex], P[ex] + c[ex]
        y_ref[lo:hi] = act_dev[lo:hi] @ W2[ex]
    assert_close(f64(y)[valid], y_ref[valid], TOL_STAGE_FP8, "y")
    if item_rows == "384":
        # the same bf16 weights, the same tiles and the same order of the fp32 sums as the
        # wide bf16 kernel on moe_dequantize_fp8's weights: bit for bit
        monkeypatch.setenv("MOE_GG_TILE_ROWS", "384")
        dw1, dw3, dw2 = (B.dequantize_fp8(qq, ss) for qq, ss in ((q1, s1), (q3, s3), (q2, s2)))
        act16, y16 = e(rows, d_e), e(rows, d)
        B.moe_grouped_gemm(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, dw1, dw3, meta, nblk, mb, act16)
        B.moe_grouped_gemm(s, B.MOE_OP_DOWN, act, dw2, None, meta, nblk, mb, y16)
        torch.cuda.synchronize()
        assert torch.equal(act[dv].view(torch.int16), act16[dv].view(torch.int16))
        assert torch.equal(y[dv].view(torch.int16), y16[dv].view(torch.int16))
    if d_es:
        assert torch.equal(sact.view(torch.int16), sact_g.view(torch.int16))
        Ws1, Ws3, Ws2 = (dq(qa, sa)[0], dq(qb, sb)[0], dq(qc, sc)[0])
        assert_close(f64(sact), O.swiglu_act(f64(x), Ws1, Ws3), TOL_STAGE_FP8, "shared act")
        assert_close(f64(sout), f64(sact) @ Ws2, TOL_STAGE_FP8, "shared out")


@pytest.mark.parametrize("name,scale", [
    ("decode-256x2048", dict(name="decode-fp8-r", d=512, d_e=256, d_e_shared=256)),
    ("fusedmoe-8x2048", dict(name="fusedmoe-fp8-r", T=600, d=1024, d_e=384, d_e_shared=256)),
    ("ep-share-4x2048", dict(name="ep-share-fp8-r", T=512, d=1024, d_e=256,
                             fixed_counts=(1357, 938, 1124, 677))),
])
def test_layer_fwd_fp8(name, scale):
    """The layer with fp8 weights against the oracle layer evaluated with the exactly
    dequantised weights, at the stated output bound."""
    cfg = get_config(name).scaled(**scale)
    torch.manual_seed(0)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    qz = [B.quantize_fp8(w) for w in (inp.w1, inp.w3, inp.w2)]
    qs = [B.quantize_fp8(w) for w in (inp.ws1, inp.ws3, inp.ws2)] if cfg.d_e_shared else [(None, None)] * 3
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    ws = B.alloc_workspace(s, fp8=True)
    routed = inp.topk_idx is not None
    B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0], *qs[1],
                        *qs[2], inp.topk_idx if routed else None, inp.topk_w if routed else None,
                        out, ws)
    torch.cuda.synchronize()
    dq = lambda p: None if p[0] is None else F.dequantize(
        p[0].cpu().numpy().reshape((-1,) + tuple(p[0].shape[-2:])),
        p[1].cpu().numpy().reshape((-1,) + tuple(p[1].shape[-2:])))
    W1, W3, W2 = (dq(p) for p in qz)
    Ws = [dq(p) for p in qs]
    kw = dict(k=cfg.k, block_m=cfg.block_m)
    if cfg.d_e_shared:
        kw.update(ws1=Ws[0][0], ws3=Ws[1][0], ws2=Ws[2][0])
    xh = f64(inp.x)
    if routed:
        ref = O.moe_layer(xh, W1, W3, W2, topk_idx=i64(inp.topk_idx), topk_w=f64(inp.topk_w), **kw)
    else:
        logits = B.ws_view(ws, s, "logits", torch.float32, (cfg.T, cfg.E)).cpu().numpy()
        ref = O.moe_layer(xh, W1, W3, W2, w_gate=f64(inp.w_gate),
                          bias=None if inp.bias is None else f64(inp.bias),
                          n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                          renormalize=cfg.renormalize, decision_logits=logits, **kw)
    rel = assert_close(f64(out), ref.out, TOL_OUT["bf16"], "out")
    print(f"[fp8 parity] {cfg.name}: out max|d|/max|ref| = {rel:.2e}")


@pytest.mark.parametrize("name,scale,wide", [
    ("ep-share-4x2048", dict(name="ep-fp8-wide", T=512, d=512, d_e=256,
                             fixed_counts=(1357, 938, 1124, 677)), True),
    ("fusedmoe-8x2048", dict(name="fm-fp8-wide", T=600, d=512, d_e=256, d_e_shared=256), True),
    # a shared expert of another width: its own launches on both paths
    ("fusedmoe-8x2048", dict(name="fm-fp8-wide-s", T=600, d=512, d_e=256, d_e_shared=96), True),
    ("fusedmoe-8x2048", dict(name="fm-fp8-narrow-s", T=300, d=512, d_e=256, d_e_shared=96), False),
    ("fusedmoe-8x2048", dict(name="fm-fp8-narrow", T=400, d=512, d_e=256, d_e_shared=256), False),
    ("decode-256x2048", dict(name="decode-fp8-dq", d=512, d_e=256, d_e_shared=256), False),
])
def test_layer_fwd_fp8_against_bf16_layer_on_dequantised_weights(name, scale, wide):
    """Where experts average >= 256 rows the fp8 layer either dequantises its weights into
    the workspace and runs the bf16 layer's kernels (a workspace of
    moe_fp8_workspace_bytes) or runs the wide kernel with the fragments dequantised in
    registers (a workspace of moe_workspace_bytes only): both bitwise equal to
    moe_layer_fwd on moe_dequantize_fp8's weights (the same bf16 values, tiles and order
    of the sums).  Below that the fp8 kernels with other tiles build the same bf16
    weights: equal up to the order of the fp32 sums (5e-3 * max|out|)."""
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    M = cfg.T * cfg.k
    assert (M >= 256 * min(cfg.E, M)) == wide
    extra = B.moe_fp8_workspace_bytes(s) - B.moe_workspace_bytes(s)
    wbytes = 2 * 3 * cfg.E * cfg.d * cfg.d_e + 2 * 3 * cfg.d * cfg.d_e_shared
    # where experts average at most 64 rows the extra room is the streaming GEMM's scratch
    streaming = M <= 64 * min(cfg.E, M)
    sk = B.moe_grouped_gemm_fp8_workspace_bytes(s) if streaming else 0
    assert extra >= wbytes if wide else extra == sk
    qz = [B.quantize_fp8(w) for w in (inp.w1, inp.w3, inp.w2)]
    qs = [B.quantize_fp8(w) for w in (inp.ws1, inp.ws3, inp.ws2)] if cfg.d_e_shared else [(None, None)] * 3
    dqz = [B.dequantize_fp8(*p) for p in qz]
    dqs = [None if p[0] is None else B.dequantize_fp8(*p) for p in qs]
    routed = inp.topk_idx is not None
    ri, rw = (inp.topk_idx, inp.topk_w) if routed else (None, None)
    out8 = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    out16 = torch.empty_like(out8)
    ws8 = torch.full((B.moe_fp8_workspace_bytes(s),), 0xFF, dtype=torch.uint8, device=DEV)
    B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0], *qs[1],
                        *qs[2], ri, rw, out8, ws8)
    B.moe_layer_fwd(s, inp.x, inp.w_gate, inp.bias, *dqz, *dqs, ri, rw, out16,
                    B.alloc_workspace(s))
    torch.cuda.synchronize()
    assert torch.isfinite(out8.float()).all()
    if wide:
        assert torch.equal(out8.view(torch.int16), out16.view(torch.int16))
        out8m = torch.empty_like(out8)
        wsm = torch.full((B.moe_workspace_bytes(s),), 0xFF, dtype=torch.uint8, device=DEV)
        B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0],
                            *qs[1], *qs[2], ri, rw, out8m, wsm)
        torch.cuda.synchronize()
        assert torch.equal(out8m.view(torch.int16), out16.view(torch.int16))
    else:
        assert_close(f64(out8), f64(out16), 5e-3, "fp8 kernels vs bf16 kernels")


@pytest.mark.parametrize("name,scale", [
    ("decode-256x2048", dict(name="decode-fp8-det", d=512, d_e=256, d_e_shared=256)),
    ("fusedmoe-8x2048", dict(name="fm-fp8-det", T=600, d=512, d_e=256, d_e_shared=256)),
])
def test_layer_fwd_fp8_is_deterministic(name, scale):
    """Both fp8 layer paths (fp8 kernels; dequantise then bf16 kernels) give bitwise-equal
    outputs run to run."""
    cfg = get_config(name).scaled(**scale)
    inp = make_inputs(cfg, device=DEV)
    s = B.shape_of_config(cfg)
    qz = [B.quantize_fp8(w) for w in (inp.w1, inp.w3, inp.w2)]
    qs = [B.quantize_fp8(w) for w in (inp.ws1, inp.ws3, inp.ws2)]
    outs = []
    for _ in range(2):
        out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
        B.moe_layer_fwd_fp8(s, inp.x, inp.w_gate, inp.bias, *qz[0], *qz[1], *qz[2], *qs[0],
                            *qs[1], *qs[2], None, None, out, B.alloc_workspace(s, fp8=True))
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def _split_plan(nblocks, n_tiles, G):
    """Whether the 64-row kernel splits its last round (the rule of moe_fp8.hip)."""
    V = nblocks * n_tiles
    R = V % G
    return G <= 256 and R > 0 and 10 * R <= 9 * G


@pytest.mark.parametrize("T,d,E,k,d_e,d_es,skew", [
    (64, 1024, 64, 8, 512, 0, False),      # every item of both launches split (no full round)
    (64, 512, 40, 3, 256, 256, False),     # the shared expert's block in the same launch
    (96, 512, 40, 3, 256, 256, False),     # ... with 96 dense rows: whole items only
    (40, 1280, 24, 3, 160, 0, False),      # down with K = 160: five slices per item
    (64, 1024, 64, 8, 512, 0, True),       # a block of 100 rows: whole items only
])
def test_fp8_split_last_round(T, d, E, k, d_e, d_es, skew, monkeypatch):
    """The 64-row kernel given scratch: the items of its grid's last round split along K
    over every work group, then added in slice order by the tail kernel.  Against the
    oracle at the stage bound, within bf16 rounding of the whole-item run, and bitwise the
    same when repeated; a table with a block of more than 64 rows runs whole items,
    bitwise as without scratch."""
    _check_fp8_split(T, d, E, k, d_e, d_es, skew, monkeypatch, expect_split=not skew)


def _random_fp8_split_cases(n=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(8, 97))
        k = int(rng.integers(1, min(8, E) + 1))
        out.append((int(rng.integers(1, 65)), int(rng.choice([256, 512, 768, 1024])), E, k,
                    int(rng.choice([128, 256, 384])), int(rng.choice([0, 0, 128]))))
    return out


@pytest.mark.parametrize("T,d,E,k,d_e,d_es", _random_fp8_split_cases())
def test_fp8_split_last_round_random(T, d, E, k, d_e, d_es, monkeypatch):
    """Seeded random decode shapes through the 64-row kernel with and without scratch:
    whichever of whole and split items the plan picks, the same checks as above."""
    _check_fp8_split(T, d, E, k, d_e, d_es, False, monkeypatch, expect_split=None)


def _check_fp8_split(T, d, E, k, d_e, d_es, skew, monkeypatch, expect_split):
    monkeypatch.setenv("MOE_FP8_ITEM_ROWS", "64")
    rng = np.random.default_rng(T * 7 + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if skew:
        # expert 0 in slot 0 of every token and slot 1 of 40 (a repeat within a token is
        # a valid route): more than 100 rows in its block
        idx[:, 0] = 0
        idx[:40, 1] = 0
    g = torch.Generator(device=DEV)
    g.manual_seed(T + d_e)
    dt = torch.bfloat16
    x = torch.randn((T, d), generator=g, device=DEV).to(dt)
    w1 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w3 = (torch.randn((E, d, d_e), generator=g, device=DEV) / d ** 0.5).to(dt)
    w2 = (torch.randn((E, d_e, d), generator=g, device=DEV) / d_e ** 0.5).to(dt)
    (q1, s1), (q3, s3), (q2, s2) = B.quantize_fp8(w1), B.quantize_fp8(w3), B.quantize_fp8(w2)
    s = B.make_shape(T=T, d=d, E=E, k=k, d_e=d_e, block_m=128, dtype="bf16", d_e_shared=d_es)
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(DEV)
    counts, offs, pad, meta, nblk, pos, row_src, err = (i32(E), i32(E + 1), i32(E + 1), i32(3 * mb),
                                                         i32(1), i32(T * k), i32(rows), i32(1))
    B.moe_build_offsets(s, d_idx, counts, offs, pad, meta, nblk, pos, row_src, err,
                        B.alloc_workspace(s))
    x_perm = torch.zeros((rows, d), dtype=dt, device=DEV)
    B.moe_permute(s, x, pos, x_perm)
    sh = {}
    if d_es:
        ws1 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        ws3 = (torch.randn((d, d_es), generator=g, device=DEV) / d ** 0.5).to(dt)
        ws2 = (torch.randn((d_es, d), generator=g, device=DEV) / d_es ** 0.5).to(dt)
        sh = dict(q=[B.quantize_fp8(w) for w in (ws1, ws3, ws2)])
    scratch = B.alloc_fp8_gemm_workspace(s)
    e = lambda *shp: torch.full(shp, 7.0, dtype=dt, device=DEV)

    def run(ws):
        act, y = e(rows, d_e), e(rows, d)
        sact, sout = (e(T, d_es), e(T, d)) if d_es else (None, None)
        if d_es:
            (qa, sa), (qb, sb), (qc, sc) = sh["q"]
            B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, q1, s1, q3, s3, meta, nblk,
                                   mb, None, act, x, qa, sa, qb, sb, sact, ws=ws)
            B.moe_grouped_gemm_fp8(s, B.MOE_OP_DOWN, act, q2, s2, None, None, meta, nblk, mb,
                                   None, y, sact, qc, sc, None, None, sout, ws=ws)
        else:
            B.moe_grouped_gemm_fp8(s, B.MOE_OP_GATEUP_SWIGLU, x_perm, q1, s1, q3, s3, meta, nblk,
                                   mb, None, act, ws=ws)
            B.moe_grouped_gemm_fp8(s, B.MOE_OP_DOWN, act, q2, s2, None, None, meta, nblk, mb,
                                   None, y, ws=ws)
        torch.cuda.synchronize()
        return act, y, sact, sout

    print(f"[fp8 split] T={T} d={d} E={E} k={k} d_e={d_e} skew={skew}", flush=True)
    whole = run(None)
    split = run(scratch)
    again = run(scratch)
    assert int(err.item()) == 0
    ref_pos, ref_src = O.permutation(idx, E, 128)
    valid = np.nonzero(ref_src >= 0)[0]
    dv = torch.from_numpy(valid).to(DEV)
    for a, b in zip(split, again):
        if a is not None:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the plan the kernels follow: blocks of the table, column tiles, grid
    nb = int(nblk.item()) + (1 if d_es else 0)
    vm = i64(meta)[:3 * int(nblk.item())].reshape(-1, 3)[:, 2]
    fits = bool(np.all(vm <= 64)) and (not d_es or T <= 64)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for op, out_s, out_w, n_cols, N in ((0, split[0], whole[0], 512, d_e), (1, split[1], whole[1], 1024, d)):
        n_tiles = -(-N // n_cols)
        G = min((mb + (1 if d_es else 0)) * 2 * n_tiles, cus)
        on = fits and _split_plan(nb, n_tiles, G)
        if not fits:
            assert not on
            assert torch.equal(out_s[dv].view(torch.int16), out_w[dv].view(torch.int16))
        elif expect_split:
            assert on, (op, nb, n_tiles, G)
        # the split changes only the order of fp32 partial sums: bf16 rounding apart
        a, b = f64(out_s[dv]), f64(out_w[dv])
        assert np.abs(a - b).max() <= 2 ** -6 * np.abs(b).max()
    # against the oracle on the exactly dequantised weights
    c = O.expert_counts(idx, E)
    def dq(qq, ss):
        qn, sn = qq.cpu().numpy(), ss.cpu().numpy()
        return F.dequantize(qn.reshape((-1,) + qn.shape[-2:]), sn.reshape((-1,) + sn.shape[-2:]))
    W1, W3, W2 = dq(q1, s1), dq(q3, s3), dq(q2, s2)
    xp_ref = O.permute(f64(x), ref_pos, k, len(ref_src))
    act_ref, _ = O.grouped_ffn(xp_ref, c, 128, W1, W3, W2)
    assert_close(f64(split[0])[valid], act_ref[valid], TOL_STAGE_FP8, "act")
    act_dev = f64(split[0])
    P = O.padded_offsets(c, 128)
    y_ref = np.zeros((len(ref_src), d))
    for ex in range(E):
        lo, hi = P[ex], P[ex] + c[ex]
        y_ref[lo:hi] = act_dev[lo:hi] @ W2[ex]
    assert_close(f64(split[1])[valid], y_ref[valid], TOL_STAGE_FP8, "y")
    if d_es:
        Ws = [dq(qq, ss)[0] for qq, ss in sh["q"]]
        assert_close(f64(split[2]), O.swiglu_act(f64(x), Ws[0], Ws[1]), TOL_STAGE_FP8, "shared act")
        assert_close(f64(split[3]), f64(split[2]) @ Ws[2], TOL_STAGE_FP8, "shared out")
