"""Host-side models of the HIP kernels' index arithmetic (not tests by themselves).

Each model restates, in numpy, how one kernel addresses its operands: which global
bytes every lane's 16-byte global->LDS copy reads and where in the LDS ring they land,
which LDS bytes every fragment read takes, and which global elements the epilogue
writes.  The checks then hold the kernel to two properties on the CPU, before any GPU
run: every access stays inside its buffer, and every fragment read finds exactly the
logical element (row, column) that the matrix instruction expects there - so a swizzle
on the copy side and its inverse on the read side agree.  The models follow the
kernel sources line by line on purpose: a change to a kernel's addressing has to be
mirrored here, and the CPU suite then says whether it is still consistent.

Conventions: LDS content is tracked per 16-byte chunk as the global byte offset of the
chunk that was copied there (-1: never written).
"""
from __future__ import annotations

import numpy as np

LDS_BYTES = 160 * 1024
LANES = np.arange(64)


def _lds_map(size: int) -> np.ndarray:
    return np.full(size // 16, -1, dtype=np.int64)


# ---------------------------------------------------------------------------
# Fused router (moe_route.hip: RouteFused<TB, E8>, k_route_fused<TB, E8>)
# ---------------------------------------------------------------------------
def route_fused_params(TB: int, E8: int) -> dict:
    EP = 8 * E8
    NT = 1 if EP <= 16 else EP // 16
    SK0 = 20480 // (2 * (TB + EP))
    SKa = 256 if SK0 >= 256 else 128 if SK0 >= 128 else 64
    SK = SKa if TB * SKa * 2 >= 4096 else 4096 // (2 * TB)
    XB = TB * SK * 2
    CX = XB // 4096
    CW = (SK * EP * 2 + 4095) // 4096
    WB = CW * 4096
    slot = XB + WB + 256
    NS = min(LDS_BYTES // slot, 12)
    KS = SK // 32
    SWZ = min(SK // 8 - 1, 15)
    return dict(EP=EP, NT=NT, SK=SK, XB=XB, CX=CX, CW=CW, WB=WB, slot=slot, NS=NS, KS=KS,
                SWZ=SWZ, CPW=CX + CW)


def wg_swz(row):
    return 2 * ((row >> 3) & 3) + ((row >> 1) & 1)


def check_route_fused(TB: int, E8: int, E: int, T: int, d: int) -> dict:
    """One slice of the first and last block of a launch over x [T, d], W_g [d, E]."""
    P = route_fused_params(TB, E8)
    SK, XB, CX, CW, WB, KS, NT, SWZ = (P[k] for k in ("SK", "XB", "CX", "CW", "WB", "KS", "NT", "SWZ"))
    assert 8 * (E8 // 2 if E8 > 1 else 0) < E <= 8 * E8 and E % 8 == 0
    assert d % SK == 0 and T >= 1
    assert P["CX"] >= 1 and XB % 4096 == 0 and P["NS"] >= 3 and (P["NS"] - 2) * P["CPW"] <= 63
    assert KS in (2, 4, 8) and TB in (16, 32, 64)
    assert P["NS"] * P["slot"] <= LDS_BYTES
    kPitch = SK * 2
    wrow = E * 2
    nsl = d // SK
    NTT, KW = TB // 16, 4 // (TB // 16)
    EPT = 16 * NT
    # epilogue LDS: k-phase partials, then the waves' selection patches
    red_floats = 4 * 64 * NT * 4 if KW > 1 else 0
    assert (red_floats + 4 * 16 * EPT) * 4 <= P["NS"] * P["slot"]
    assert 4 * 64 * NT * 16 + 4 * 16 * 16 * NT * 4 <= P["NS"] * P["slot"]
    nblocks = -(-T // TB)
    for blk in sorted({0, nblocks - 1}):
        t0 = blk * TB
        rot = blk % nsl
        for j in sorted({0, nsl - 1}):
            js = min(j, nsl - 1) + rot
            if js >= nsl:
                js -= nsl
            lds = _lds_map(XB + WB + 256)      # + the read slack of the slot
            # x copies: 1 KB per copy, two or four rows of SK contiguous elements
            for wave in range(4):
                for c in range(CX):
                    p = (wave * CX + c) * 1024 + LANES * 16
                    row, pc = p // kPitch, (p % kPitch) // 16
                    lc = pc ^ (row & SWZ)
                    assert np.all(row < TB) and np.all(lc < SK // 8)
                    rowc = np.minimum(t0 + row, T - 1) - t0
                    xoff = rowc * d * 2 + lc * 16
                    assert xoff.max() < 2 ** 32
                    src = (t0 * d + js * SK) * 2 + xoff          # bytes from the start of x
                    assert src.min() >= 0 and (src + 16).max() <= T * d * 2
                    assert np.all(p + 16 <= XB)
                    lds[p // 16] = src
            # W_g copies
            wslice = SK * wrow
            for wave in range(4):
                for c in range(CW):
                    Pb = ((wave * CW + c) * 64 + LANES) * 16
                    if E8 == 8:
                        row = Pb >> 7
                        lc = ((Pb >> 4) & 7) ^ wg_swz(row)
                        woff = np.minimum(row, SK - 1) * wrow + np.where(lc * 8 < E, lc, 0) * 16
                    else:
                        woff = np.minimum(Pb, wslice - 16)
                    src = js * SK * E * 2 + woff                  # bytes from the start of W_g
                    assert src.min() >= 0 and (src + 16).max() <= d * E * 2
                    assert np.all(Pb + 16 <= WB)
                    lds[(XB + Pb) // 16] = src + (1 << 40)        # tag: W_g
            # fragment reads of every wave (its tile and k-phase)
            g, r16 = LANES >> 4, LANES & 15
            tr_r, tr_c = (LANES & 15) >> 2, LANES & 3
            for wave in range(4):
                tw, kw = wave % NTT, wave // NTT
                for q in range((KS + KW - 1) // KW):
                    kk = kw + KW * q
                    if kk >= KS:
                        break
                    for nt in range(NT):
                        for hh in (0, 1):
                            krow = kk * 32 + g * 8 + tr_r + 4 * hh    # row of W_g in the slice
                            col_b = nt * 32 + tr_c * 8                # byte column (4 experts)
                            if E8 == 8:
                                addr = XB + (kk * 32 + g * 8 + tr_r) * 128 + hh * 4 * 128 + \
                                    (((2 * nt + (tr_c >> 1)) ^ (2 * g + (tr_r >> 1))) * 16) + (tr_c & 1) * 8
                                assert np.all(wg_swz(krow) == 2 * g + (tr_r >> 1))
                            else:
                                addr = XB + krow * wrow + col_b
                            assert (addr + 8).max() <= XB + WB + 256
                            # experts < E: the 8 bytes are W_g[js*SK + krow][col_b / 2 ..]
                            live = col_b < wrow
                            if not np.any(live):
                                continue
                            want = js * SK * E * 2 + krow * wrow + col_b + (1 << 40)
                            got = lds[addr // 16] + addr % 16
                            assert np.all(got[live] == want[live]), (TB, E8, E, wave, nt, hh)
                    row = tw * 16 + r16
                    pc = (kk * 4 + g) ^ (row & SWZ)
                    addr = row * kPitch + pc * 16
                    assert (addr + 16).max() <= XB
                    rowc = np.minimum(t0 + row, T - 1) - t0
                    want = (t0 * d + js * SK) * 2 + rowc * d * 2 + (kk * 4 + g) * 16
                    assert np.all(lds[addr // 16] == want), (TB, E8, E, wave, kk)
    # selection patch: token tk of the tile, slot j < k <= E <= EPT
    assert E <= EPT
    return P


# ---------------------------------------------------------------------------
# Wide grouped GEMM (moe_gemm_wide.hip: wide_build_groups, wide_item, k_gg_wide<OP, 8, FP8>)
# ---------------------------------------------------------------------------
W_ROWS, W_BK = 384, 32
W_ABYTES = W_ROWS * W_BK * 2          # 24 KB
W_BBYTES = W_BK * 256 * 2             # 16 KB (bf16)
W_STAGE, W_STAGES = W_ABYTES + W_BBYTES, 4


def swz_a(row, c):
    return c ^ ((row >> 2) & 3)


def swz_b(k, c):
    return c ^ (4 * (k & 3))


def _block_ok(m, b, E, max_rows):
    e, ms, v = int(m[b, 0]), int(m[b, 1]), int(m[b, 2])
    return 0 <= e < E and ms >= 0 and 1 <= v <= 128 and ms + v <= max_rows


def _joins(m, b, E, max_rows):
    return (b > 0 and _block_ok(m, b - 1, E, max_rows) and m[b, 0] == m[b - 1, 0]
            and m[b, 1] == m[b - 1, 1] + m[b - 1, 2])


def wide_groups_kernel(meta, nb, E, max_rows, GB=3):
    """The group list as wide_build_groups forms it: 64 lanes over chunks of blocks, the
    run start and each lane's first output slot from two scans."""
    m = np.asarray(meta)
    ok = lambda b: _block_ok(m, b, E, max_rows)
    joins = lambda b: _joins(m, b, E, max_rows)
    per = (nb + 63) // 64
    lo = [min(l * per, nb) for l in range(64)]
    hi = [min(lo[l] + per, nb) for l in range(64)]
    last_rs = []
    for l in range(64):
        r = -1
        for b in range(lo[l], hi[l]):
            if ok(b) and not joins(b):
                r = b
        last_rs.append(r)
    incl = np.maximum.accumulate(last_rs)
    in_rs = [-1] + [int(v) for v in incl[:-1]]
    cnt = []
    for l in range(64):
        c, rs = 0, in_rs[l]
        for b in range(lo[l], hi[l]):
            if not ok(b):
                continue
            if not joins(b):
                rs = b
            if (b - rs) % GB == 0:
                c += 1
        cnt.append(c)
    inc = np.cumsum(cnt)
    out = [None] * int(inc[-1])
    for l in range(64):
        idx, rs = int(inc[l] - cnt[l]), in_rs[l]
        for b in range(lo[l], hi[l]):
            if not ok(b):
                continue
            if not joins(b):
                rs = b
            if (b - rs) % GB == 0:
                n = 1
                while n < GB and b + n < nb and ok(b + n) and joins(b + n):
                    n += 1
                out[idx] = (b, n)
                idx += 1
    assert all(o is not None for o in out)
    return out


def wide_groups_serial(meta, nb, E, max_rows, GB=3):
    """The same list from its definition: maximal runs of valid blocks of one expert with
    contiguous rows, cut into GB-block pieces from each run's start."""
    m = np.asarray(meta)
    out, run_len = [], 0
    for b in range(nb):
        if not _block_ok(m, b, E, max_rows):
            run_len = 0
            continue
        run_len = run_len + 1 if (run_len and _joins(m, b, E, max_rows)) else 1
        if (run_len - 1) % GB == 0:
            out.append([b, 1])
        else:
            out[-1][1] += 1
    return [tuple(x) for x in out]


def wide_split_tail(groups, ng_dense, n_tiles, G):
    """The group list after wide_build_groups' last-round split: trailing three-block
    groups become single blocks when that adds no round of the persistent grid (G work
    groups) and the last round then holds only single-block items."""
    groups = list(groups)
    ng = len(groups)
    total = (ng_dense + ng) * n_tiles
    F = total // G
    if total - F * G == 0:
        return groups, 0
    smax = ((F + 1) * G - total) // (2 * n_tiles)
    sp = 0
    while sp < smax and sp < ng and groups[ng - 1 - sp][1] == 3:
        sp += 1
    if sp == 0 or 3 * sp * n_tiles < total + 2 * sp * n_tiles - F * G:
        return groups, 0
    tail = [(b + j, 1) for b, _ in groups[ng - sp:] for j in range(3)]
    return groups[:ng - sp] + tail, sp


def check_wide_split_tail(groups, ng_dense, n_tiles, G):
    """The split keeps every block once, in order, adds no round, and (when it splits)
    leaves only split single-block items in the last round."""
    new, sp = wide_split_tail(groups, ng_dense, n_tiles, G)
    blocks = lambda gl: [b + j for b, n in gl for j in range(n)]
    assert blocks(new) == blocks(groups)
    total, total2 = (ng_dense + len(groups)) * n_tiles, (ng_dense + len(new)) * n_tiles
    assert -(-total2 // G) == -(-total // G)
    ngt = ng_dense + len(new)
    seen = set()
    for w in range(total2):                               # every (group, tile) once
        seen.add(wide_item_split(w, ngt, 3 * sp, n_tiles))
    assert len(seen) == total2
    if sp:
        first_split = ngt - 3 * sp                        # group index of the first single
        for w in range((total2 - 1) // G * G, total2):    # the last round
            g, _ = wide_item_split(w, ngt, 3 * sp, n_tiles)
            assert g >= first_split and new[g - ng_dense][1] == 1, (w, g, first_split)
    return new, sp


def wide_item_split(slot, ngt, nsingle, n_tiles):
    """wide_item with nsingle trailing single-block groups numbered last, group-major."""
    main = (ngt - nsingle) * n_tiles
    if slot < main:
        return wide_item(slot, ngt - nsingle, n_tiles)
    r = slot - main
    return ngt - nsingle + r // n_tiles, r % n_tiles


def wide_item(slot, ngt, n_tiles):
    Ts = min(n_tiles, 8)
    Gs = 32 // Ts
    row_items = Gs * n_tiles
    sr, rem = divmod(slot, row_items)
    gr = min(Gs, ngt - sr * Gs)
    sc, within = divmod(rem, gr * Ts)
    tc = min(Ts, n_tiles - sc * Ts)
    return sr * Gs + within // tc, sc * Ts + within % tc


def check_wide_item_order(ngt, n_tiles):
    seen = set(wide_item(s, ngt, n_tiles) for s in range(ngt * n_tiles))
    assert seen == {(g, t) for g in range(ngt) for t in range(n_tiles)}


def wide_subtile_row(wave, i, NW=8):
    """First tile row of 32-row subtile i of a wave of the wide kernel: wave pair p = wave // 2
    owns subtiles p, p + NW/2, p + NW, ... (interleaved), each with both column halves split
    between the pair's two waves."""
    return (i * (NW // 2) + (wave >> 1)) * 32


def wide_live_subtiles(wave, valid, NW=8):
    """Subtiles of the wave that hold a row below valid (the kernel multiplies only these)."""
    MI = W_ROWS * 2 // NW // 32
    return sum(1 for i in range(MI) if wide_subtile_row(wave, i, NW) < valid)


def check_wide_row_split(NW=8):
    """The waves' subtiles cover the tile's rows once per column half, and for every valid
    count the live subtiles of each wave are its first ones and hold every valid row."""
    MI = W_ROWS * 2 // NW // 32
    for ch in (0, 1):
        owned = np.zeros(W_ROWS, int)
        for wave in range(ch, NW, 2):
            for i in range(MI):
                r0 = wide_subtile_row(wave, i, NW)
                owned[r0:r0 + 32] += 1
        assert np.all(owned == 1)
    for valid in range(1, W_ROWS + 1):
        for wave in range(NW):
            n = wide_live_subtiles(wave, valid, NW)
            rows = [wide_subtile_row(wave, i, NW) for i in range(MI)]
            assert all(r < valid for r in rows[:n]) and all(r >= valid for r in rows[n:])
        # a group of b blocks (valid in (128 (b-1), 128 b]) gives every wave at most b live
        # subtiles, and b to the waves of every SIMD but the last rows'
        b = -(-valid // 128)
        assert max(wide_live_subtiles(w, valid, NW) for w in range(NW)) == b


def check_wide_item(op, fp8, K, N, e, m0, valid, a_rows, n_e, gather=None, n_tiles_check=None):
    """Every copy, fragment read and store of one row group (all column tiles, or the
    listed ones) of k_gg_wide<op, 8, fp8>; slices 0 and the last.  gather: per-row source
    rows of A (routed gate/up with the permutation fused) or None."""
    GU = op == 0
    NW = 8
    WR, MI = W_ROWS * 2 // NW, W_ROWS * 2 // NW // 32
    BB = W_BBYTES // 2 if fp8 else W_BBYTES
    stage = W_ABYTES + BB
    stages = 5 if fp8 else W_STAGES
    assert stages * stage <= W_STAGES * W_STAGE <= LDS_BYTES
    CPA, CPB = (W_ROWS // 16) // NW, BB // 1024 // NW
    eb = 1 if fp8 else 2
    pitch = (128 if GU else 256) * eb
    out_cols = 128 if GU else 256
    n_tiles = -(-N // out_cols)
    nk = K // W_BK
    assert 0 < valid <= W_ROWS and m0 >= 0 and m0 + valid <= a_rows and 0 <= e < n_e
    lane = LANES
    for nt in (n_tiles_check if n_tiles_check is not None else range(n_tiles)):
        n0 = nt * out_cols
        for ks in sorted({0, nk - 1}):
            lds = _lds_map(stage)
            # A: window t = wave*CPA + i, rows 16t .. 16t+15, four lanes per row
            for wave in range(NW):
                for i in range(CPA):
                    t = wave * CPA + i
                    row = t * 16 + (lane >> 2)
                    c = (lane & 3) ^ ((lane >> 4) & 3)
                    assert np.all(swz_a(row, c) == (lane & 3))
                    rr = np.where(row < valid, row, 0)
                    src_row = gather[m0 + rr] if gather is not None else m0 + rr
                    base_rows = a_rows if gather is None else int(np.max(gather)) + 1
                    elem = src_row * K + ks * W_BK + c * 8
                    voff = (np.where(gather is not None, src_row, rr) * K + c * 8) * 2 + (CPA - 1 - i) * 1024
                    assert voff.min() >= 0 and voff.max() < 2 ** 32
                    assert elem.min() >= 0 and (elem + 8).max() <= base_rows * K
                    lds[(t * 1024 + lane * 16) // 16] = elem * 2
            # B
            for wave in range(NW):
                u0 = wave * CPB
                for p in range(CPB):
                    u = u0 + p
                    if fp8:
                        rows_per = 8 if GU else 4
                        uu = (u0 & 3) if GU else u0
                        kl = (lane >> 3) if GU else (lane >> 4)
                        k = rows_per * uu + kl
                        cpos = (lane & 7) if GU else (lane & 15)
                        lc = cpos ^ (k & (7 if GU else 15))
                        col = n0 + lc * 16
                        col = np.where(col >= N, 0, col)
                        region = (u0 >> 2) if GU else 0
                        dst = W_ABYTES + (region * (BB // 2) + uu * 1024 if GU else u0 * 1024) + lane * 16
                        krow = ks * W_BK + k
                    else:
                        kl = (lane >> 4) if GU else (lane >> 5)
                        k = kl if GU else 2 * (p & 1) + kl
                        cpos = (lane & 15) if GU else (lane & 31)
                        col = n0 + swz_b(k, cpos) * 8
                        col = np.where(col >= N, 0, col)
                        region = (u >> 3) if GU else 0
                        if GU:
                            krow = ks * W_BK + 4 * (u & 7) + kl
                            dst = W_ABYTES + region * (BB // 2) + (u & 7) * 1024 + lane * 16
                        else:
                            krow = ks * W_BK + 2 * u + kl
                            dst = W_ABYTES + u * 1024 + lane * 16
                    assert krow.max() < K and (col + 16 // eb).max() <= N
                    gidx = e * K * N + krow * N + col
                    assert gidx.min() >= 0 and gidx.max() + 16 // eb <= n_e * K * N
                    assert dst.min() >= W_ABYTES and (dst + 16).max() <= stage
                    lds[dst // 16] = (gidx * eb) + (region << 44)
            # fragment reads: A rows of every wave, B columns of every wave
            g, gi = lane >> 4, lane & 15
            tr_r, tr_c4 = gi >> 2, gi & 3
            for wave in range(NW):
                ch = wave & 1
                for i in range(MI):
                    row = wide_subtile_row(wave, i, NW) + (lane & 31)
                    for kk in (0, 1):
                        addr = row * 64 + swz_a(row, kk * 2 + (lane >> 5)) * 16
                        assert (addr + 16).max() <= W_ABYTES
                        rr = np.where(row < valid, row, 0)
                        src_row = gather[m0 + rr] if gather is not None else m0 + rr
                        want = (src_row * K + ks * W_BK + (kk * 2 + (lane >> 5)) * 8) * 2
                        assert np.all(lds[addr // 16] == want), ("A", op, fp8, wave, i, kk)
                for j in range(4):
                    region = (j >> 1) if GU else 0
                    jb = (j & 1) if GU else j
                    col0 = ch * 64 + jb * 32 if GU else ch * 128 + jb * 32
                    for kk in (0, 1):
                        if fp8:
                            k = 8 * (g >> 1) + (gi >> 1)
                            chunk = col0 // 16 + (g & 1)
                            pc = chunk ^ (k & (7 if GU else 15))
                            addr = W_ABYTES + region * (BB // 2) + k * pitch + pc * 16 + (gi & 1) * 8 + kk * 16 * pitch
                            krow = ks * W_BK + kk * 16 + k
                            ncol = n0 + chunk * 16 + (gi & 1) * 8
                            pieces = [(addr, krow, ncol)]
                        else:
                            cj = col0 >> 3
                            chunk = (cj ^ (4 * tr_r)) | (2 * (g & 1) + (tr_c4 >> 1))
                            lane_off = ((g >> 1) * 8 + tr_r) * pitch + chunk * 16 + (tr_c4 & 1) * 8
                            pieces = []
                            for hh in (0, 1):
                                addr = W_ABYTES + region * (BB // 2) + lane_off + kk * 16 * pitch + hh * 4 * pitch
                                krow = ks * W_BK + kk * 16 + (g >> 1) * 8 + hh * 4 + tr_r
                                ncol = n0 + col0 + (g & 1) * 16 + 4 * tr_c4
                                pieces.append((addr, krow, ncol))
                        for addr, krow, ncol in pieces:
                            assert addr.min() >= W_ABYTES and (addr + 8).max() <= stage
                            live = ncol < N
                            want = (e * K * N + krow * N + ncol) * eb + (region << 44)
                            got = lds[addr // 16] + addr % 16
                            assert np.all(got[live] == want[live]), ("B", op, fp8, wave, j, kk)
        # epilogue: a row r < valid of the group and an 8-column chunk c < N
        for wave in range(NW):
            r = np.arange(WR)[:, None]
            for ps in range(1 if GU else 2):
                col0 = n0 + ((wave & 1) * 64 if GU else (wave & 1) * 128 + ps * 64)
                gcol = col0 + (lane & 7) * 8
                # staging row r of the wave holds tile row subtile_row(r // 32) + r % 32
                grow = np.array([[wide_subtile_row(wave, int(x) // 32, NW) + int(x) % 32] for x in r[:, 0]])
                ok = (grow < valid) & (gcol[None, :] < N)
                rows = (m0 + grow) * np.ones_like(gcol)[None, :]
                assert np.all(rows[ok] < a_rows) and np.all((gcol[None, :] * np.ones_like(grow) + 8)[ok] <= N)
    # the epilogue staging of every op fits the ring
    assert NW * WR * 72 * 2 <= W_STAGES * W_STAGE
    assert NW * 2 * 32 * 72 * 2 + NW * 4096 <= W_STAGES * W_STAGE


# ---------------------------------------------------------------------------
# Backward grouped GEMMs (moe_backward.hip: k_gg_nt, k_gg_wgrad), functional models:
# the copies, swizzles, transposed LDS reads and MFMA fragment layouts move real numbers,
# so the product they assemble can be compared with numpy.
# ---------------------------------------------------------------------------
BK = 32


def mfma(acc, a_lanes, b_lanes):
    """acc [32,32] += A(32x16) B(16x32); a_lanes[l] = 8 values of A[l%32][(l//32)*8 + j],
    b_lanes[l] = B[(l//32)*8 + j][l%32]."""
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        A[l % 32, (l // 32) * 8:(l // 32) * 8 + 8] = a_lanes[l]
        B[(l // 32) * 8:(l // 32) * 8 + 8, l % 32] = b_lanes[l]
    acc += A @ B


def acc_rc(q, l):
    return (q >> 2) * 8 + (l >> 5) * 4 + (q & 3), l % 32


# ---------------------------------------------------------------- NT
def emu_nt(A, Bt0, Bt1, ldb, ksplit, K, N, tiles, E):
    """tiles: list of (e, m0, valid).  Returns C rows dict."""
    rowsA = A.shape[0]
    C = np.full((rowsA, N), np.nan)
    nk = K // BK
    n_tiles = -(-N // 512)
    Bsz = Bt0.size
    for (e, m0, valid) in tiles:
        for nt in range(n_tiles):
            n0 = nt * 512
            acc = np.zeros((8, 4, 2, 32, 32))
            for ks in range(nk):
                k0 = ks * BK
                sa = np.full((128, 4, 8), np.nan)
                sb = np.full((512, 4, 8), np.nan)
                for w in range(8):
                    for l in range(64):
                        c = (l & 3) ^ ((l >> 4) & 3)
                        row = w * 16 + (l >> 2)
                        rr = row if row < valid else 0
                        g = (m0 + rr) * K + k0 + c * 8
                        assert 0 <= g and g + 8 <= A.size, ("A oob", g)
                        # lands at w*1024 + 16 l -> row w*16 + l//4, phys chunk l & 3
                        prow, pch = (w * 1024 + 16 * l) // 64, ((w * 1024 + 16 * l) % 64) // 16
                        assert prow == row and pch == (l & 3)
                        sa[prow, pch] = A.reshape(-1)[g:g + 8]
                        for p in range(4):
                            n = n0 + (w * 4 + p) * 16 + (l >> 2)
                            nn = n if n < N else 0
                            second = k0 >= ksplit
                            src = Bt1 if second else Bt0
                            kk = k0 - ksplit if second else k0
                            gb = e * N * ldb + nn * ldb + kk + c * 8
                            assert 0 <= gb and gb + 8 <= Bsz, ("B oob", gb)
                            off = (w * 4 + p) * 1024 + 16 * l
                            sb[off // 64, (off % 64) // 16] = src.reshape(-1)[gb:gb + 8]
                for kk in range(2):
                    for w in range(8):
                        a = [[None] * 64 for _ in range(4)]
                        b = [[None] * 64 for _ in range(2)]
                        for l in range(64):
                            for i in range(4):
                                row = i * 32 + (l & 31)
                                a[i][l] = sa[row, swz_a(row, kk * 2 + (l >> 5))]
                            for j in range(2):
                                n = w * 64 + j * 32 + (l & 31)
                                b[j][l] = sb[n, swz_a(n, kk * 2 + (l >> 5))]
                        for i in range(4):
                            for j in range(2):
                                mfma(acc[w, i, j], a[i], b[j])
            for w in range(8):
                for i in range(4):
                    for j in range(2):
                        for q in range(16):
                            for l in range(64):
                                r, cc = acc_rc(q, l)
                                grow = i * 32 + r
                                gcol = n0 + w * 64 + j * 32 + cc
                                if grow < valid and gcol < N:
                                    C[m0 + grow, gcol] = acc[w, i, j][r, cc]
    return C


# ---------------------------------------------------------------- wgrad
def emu_wgrad(X, D, Km, Nn, nsplit, counts, row_off, E):
    C0 = np.full((E, Km, nsplit), np.nan)
    C1 = np.full((E, Km, Nn - nsplit), np.nan) if nsplit < Nn else None
    m_tiles, n_tiles = -(-Km // 128), -(-Nn // 512)
    for e in range(E):
        cnt, r0e = counts[e], row_off[e]
        ns = -(-cnt // BK)
        for mt in range(m_tiles):
            for nt in range(n_tiles):
                m0, n0 = mt * 128, nt * 512
                acc = np.zeros((8, 4, 2, 32, 32))
                for s in range(ns):
                    sx = np.full((32, 16, 8), np.nan)
                    sd = np.full((32, 64, 8), np.nan)
                    for w in range(8):
                        rbase = 32 * s + 4 * w
                        xb = rbase if rbase < cnt else 0
                        for l in range(64):
                            rr = 4 * w + (l >> 4)
                            mcol = m0 + swz_b(rr, l & 15) * 8
                            if mcol >= Km:
                                mcol = 0
                            lr = (l >> 4) if rbase + (l >> 4) < cnt else 0
                            g = (r0e + xb) * Km + lr * Km + mcol
                            assert 0 <= g and g + 8 <= X.size and r0e + xb + lr < X.shape[0], "X oob"
                            off = w * 1024 + 16 * l
                            sx[off // 256, (off % 256) // 16] = X.reshape(-1)[g:g + 8]
                            for p in range(4):
                                r = rbase + p
                                rrow = r if r < cnt else 0
                                ncol = n0 + swz_b(4 * w + p, l) * 8
                                if ncol >= Nn:
                                    ncol = 0
                                gd = (r0e + rrow) * Nn + ncol
                                assert 0 <= gd and gd + 8 <= D.size, "D oob"
                                off = (4 * w + p) * 1024 + 16 * l
                                sd[off // 1024, (off % 1024) // 16] = D.reshape(-1)[gd:gd + 8]
                    # zero tail
                    for w in range(8):
                        rbase = 32 * s + 4 * w
                        if rbase + 4 <= cnt:
                            continue
                        for l in range(64):
                            if rbase + (l >> 4) >= cnt:
                                off = w * 1024 + l * 16
                                sx[off // 256, (off % 256) // 16] = 0
                        for p in range(4):
                            if rbase + p >= cnt:
                                sd[4 * w + p] = 0
                    assert not np.isnan(sx).any() and not np.isnan(sd).any()
                    for kk in range(2):
                        for w in range(8):
                            af = [[None] * 64 for _ in range(4)]
                            bf = [[None] * 64 for _ in range(2)]
                            for (frag, ncnt, region, pitch_ch, colf) in (
                                    (af, 4, sx, 16, lambda i, g, c4: i * 32 + (g & 1) * 16 + 4 * c4),
                                    (bf, 2, sd, 64, lambda j, g, c4: w * 64 + j * 32 + (g & 1) * 16 + 4 * c4)):
                                for idx in range(ncnt):
                                    for g in range(4):
                                        hv = []
                                        for hh in range(2):
                                            data = np.zeros((4, 16))
                                            for gi in range(16):
                                                tr_r, tr_c4 = gi >> 2, gi & 3
                                                k = kk * 16 + (g >> 1) * 8 + hh * 4 + tr_r
                                                col = colf(idx, g, tr_c4)
                                                ch = swz_b(k, col >> 3)
                                                assert 0 <= ch < pitch_ch
                                                vals = region[k, ch, (col & 7):(col & 7) + 4]
                                                data[tr_r, 4 * tr_c4:4 * tr_c4 + 4] = vals
                                            hv.append(data)
                                        for i16 in range(16):
                                            l = g * 16 + i16
                                            frag[idx][l] = np.concatenate([hv[0][:, i16], hv[1][:, i16]])
                            for i in range(4):
                                for j in range(2):
                                    mfma(acc[w, i, j], af[i], bf[j])
                for w in range(8):
                    for i in range(4):
                        for j in range(2):
                            for q in range(16):
                                for l in range(64):
                                    r, cc = acc_rc(q, l)
                                    m = m0 + i * 32 + r
                                    n = n0 + w * 64 + j * 32 + cc
                                    if m >= Km or n >= Nn:
                                        continue
                                    if n < nsplit:
                                        C0[e, m, n] = acc[w, i, j][r, cc]
                                    else:
                                        C1[e, m, n - nsplit] = acc[w, i, j][r, cc]
    return C0, C1


# ---------------------------------------------------------------------------
# 64-row fp8 decode kernel (moe_fp8.hip: k_gg_fp8d<OP>): one 36 KB stage (4 KB of A,
# 32 KB of e4m3 weights), and the slice stream that consecutive items share.
# ---------------------------------------------------------------------------
D_BK, D_ROWS = 32, 64
D_ABYTES = D_ROWS * D_BK * 2
D_BBYTES = 32 * 1024
D_STAGE, D_STAGES = D_ABYTES + D_BBYTES, 4


def check_fp8d_stage(op, K, N):
    """Every B copy of every column tile lands where the transposed fp8 reads look for
    it; sources in bounds; the ring fits the LDS."""
    GU = op == 0
    out_cols = 512 if GU else 1024
    pitch = 512 if GU else 1024
    assert K % D_BK == 0 and N % 16 == 0
    # the ring and the double-buffered block-scale table (kFMaxKB = 256 k-blocks x 8)
    assert D_STAGES * D_STAGE + 2 * 256 * 8 * 4 <= LDS_BYTES
    n_tiles = -(-N // out_cols)
    nk = K // D_BK
    lane = LANES
    for nt in sorted({0, n_tiles - 1}):
        n0 = nt * out_cols
        for ks in sorted({0, nk - 1}):
            lds = _lds_map(D_STAGE)
            for wave in range(8):
                for p in range(4):
                    u = wave * 4 + p
                    if GU:
                        k, pos, row0 = 2 * (u & 15) + (lane >> 5), lane & 31, 2 * (u & 15)
                    else:
                        k, pos, row0 = np.full(64, u), lane, u
                    col = n0 + (pos ^ (k & 15)) * 16
                    col = np.where(col >= N, 0, col)
                    assert (col + 16).max() <= N
                    voff = (k - row0) * N + col
                    g = (ks * D_BK + row0) * N + voff
                    assert g.min() >= 0 and (g + 16).max() <= K * N
                    dst = D_ABYTES + u * 1024 + lane * 16
                    assert (dst + 16).max() <= D_STAGE
                    region = (u >> 4) if GU else 0
                    lds[dst // 16] = g + (region << 44)
            g_, gi = lane >> 4, lane & 15
            for wave in range(8):
                for j in range(4):
                    region = (j >> 1) if GU else 0
                    col0 = wave * 64 + (j & 1) * 32 if GU else wave * 128 + j * 32
                    k = 8 * (g_ >> 1) + (gi >> 1)
                    chunk = col0 // 16 + (g_ & 1)
                    assert chunk.max() < pitch // 16
                    b = region * (D_BBYTES // 2) + k * pitch + (chunk ^ (k & 15)) * 16 + (gi & 1) * 8
                    for kk in (0, 1):
                        addr = D_ABYTES + b + kk * 16 * pitch
                        assert addr.min() >= D_ABYTES and (addr + 8).max() <= D_STAGE
                        ncol = n0 + chunk * 16 + (gi & 1) * 8
                        live = ncol < N
                        want = (ks * D_BK + kk * 16 + k) * N + ncol + (region << 44)
                        got = lds[addr // 16] + addr % 16
                        assert np.all(got[live] == want[live]), (op, wave, j, kk)


def check_fp8d_stream(nk, nitems):
    """The ring schedule of consecutive items: the refill of stream slice gs-1's slot at
    slice gs carries stream slice gs-1+S (this item's, the next item's, or a re-copy of
    this item's last slice when no item follows); every slice is read from the slot that
    holds it."""
    S = D_STAGES
    assert nk >= S
    owner = {p: (0, min(p, nk - 1)) for p in range(S)}
    gbase = 0
    for item in range(nitems):
        has_next = item + 1 < nitems
        for ks in range(nk):
            gs = gbase + ks
            if gs > 0:
                t = gs - 1 + S - gbase
                slot = (gs - 1) % S
                if t < nk:
                    owner[slot] = (item, t)
                elif has_next:
                    assert t - nk <= S - 2
                    owner[slot] = (item + 1, t - nk)
                else:
                    owner[slot] = (item, nk - 1)
            assert owner[gs % S] == (item, ks), (nk, nitems, item, ks)
        gbase += nk


# ---------------------------------------------------------------------------
# 128-row bf16 kernel (moe_gemm.hip: k_gg_bf16_v2): copy sources of every block.
# ---------------------------------------------------------------------------
def check_v2_copies(op, K, N, tiles, n_e, a_rows, block_m=128):
    assert K % 32 == 0
    out_cols = 256 if op == 0 else 512
    n_tiles = -(-N // out_cols)
    nk = K // 32
    lane = LANES
    for (e, m_start, vm) in tiles:
        for sub in range(block_m // 128):
            m0, valid = m_start + sub * 128, min(128, vm - sub * 128)
            if valid <= 0:
                continue
            assert m0 + valid <= a_rows
            for nt in sorted({0, n_tiles - 1}):
                n0 = nt * out_cols
                for wave in range(8):
                    row = wave * 16 + (lane >> 2)
                    c = swz_a(row, lane & 3)
                    rr = np.where(row < valid, row, 0)
                    for ks in sorted({0, nk - 1}):
                        lo = (m0 + rr) * K + ks * 32 + c * 8
                        assert lo.min() >= 0 and (lo + 8).max() <= a_rows * K
                    for i in range(4):
                        q = wave * 4 + i
                        h, pr = q >> 4, q & 15
                        kk = 2 * (pr & 1) + (lane >> 5)
                        col0 = n0 if (op == 0 or h == 0) else n0 + 256
                        col = col0 + swz_b(kk, lane & 31) * 8
                        col = np.where(col >= N, 0, col)
                        for ks in sorted({0, nk - 1}):
                            krow = ks * 32 + 2 * pr + (lane >> 5)
                            idx = e * K * N + krow * N + col
                            assert krow.max() < K and idx.min() >= 0 and (idx + 8).max() <= n_e * K * N


# ---------------------------------------------------------------------------
# The 64-row fp8 kernel's split last round (moe_fp8.hip: k_gg_fp8d, k_fp8d_tail): the
# pieces the work groups compute and the slots the tail kernel adds, integer arithmetic
# written as in the kernels.
# ---------------------------------------------------------------------------
def fp8d_tail_plan(V, G, fits=True, max_grid=256):
    F, R = V // G, V % G
    return F, R, fits and G <= max_grid and R > 0 and 10 * R <= 9 * G and 16 * R >= G


def fp8d_tail_pieces(R, nk, G):
    """{item r: [(q, slot, k0, n), ...]} in the order the work groups compute them."""
    S = R * nk
    out = {}
    for q in range(G):
        lo, hi = q * S // G, (q + 1) * S // G
        sl = lo
        while sl < hi:
            r = sl // nk
            k0 = sl - r * nk
            end = (r + 1) * nk
            n = min(hi, end) - sl
            out.setdefault(r, []).append((q, 2 * q + (0 if sl == lo else 1), k0, n))
            sl = end
    return out


def fp8d_tail_slots(R, nk, G, r):
    """The slots k_fp8d_tail adds for item r, in its order."""
    S = R * nk
    a, b = r * nk, r * nk + nk
    q0 = a // (S // G + 1)
    while q0 > 0 and q0 * S // G > a:
        q0 -= 1
    while (q0 + 1) * S // G <= a:
        q0 += 1
    slots = []
    for q in range(q0, G):
        lo, hi = q * S // G, (q + 1) * S // G
        if lo >= b:
            break
        if hi <= lo:
            continue
        slots.append(2 * q + (0 if lo >= a else 1))
    return slots


def check_fp8d_tail(R, nk, G):
    pieces = fp8d_tail_pieces(R, nk, G)
    assert sorted(pieces) == list(range(R))
    used = set()
    for r in range(R):
        ps = pieces[r]
        # the item's slices, each once, in slice order
        assert [p[2] for p in ps] == sorted(p[2] for p in ps)
        cov = 0
        for (q, slot, k0, n) in ps:
            assert k0 == cov and n >= 1
            cov += n
            assert slot in (2 * q, 2 * q + 1) and slot not in used and 0 <= slot < 2 * G
            used.add(slot)
        assert cov == nk
        assert fp8d_tail_slots(R, nk, G, r) == [p[1] for p in ps]
        assert len(ps) <= 34               # the tail kernel lists at most 64
    # every work group computes at most two pieces
    per_q = {}
    for ps in pieces.values():
        for p in ps:
            per_q[p[0]] = per_q.get(p[0], 0) + 1
    assert max(per_q.values()) <= 2
