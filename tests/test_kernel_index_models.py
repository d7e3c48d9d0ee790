"""CPU checks of the HIP kernels' index arithmetic through the models in
tests/kernel_models.py: bounds of every copy, read and store, and that fragment reads
find the logical elements their copies placed (swizzles and their inverses agree).
The block tables come from the oracle's offsets so that they have real shapes."""
import numpy as np
import pytest

import kernel_models as KM
from oracle import moe_oracle as O


def _table(T, E, k, bm, rng, skew=False, corrupt=False):
    idx = rng.integers(0, max(1, E // 3) if skew else E, size=(T, k))
    idx[0, :] = E - 1
    c = O.expert_counts(idx, E)
    meta = O.block_metadata(c, bm)
    M = T * k
    ne = min(M, E)
    max_blocks = (M + ne * (bm - 1)) // bm
    full = np.zeros((max_blocks, 3), np.int64)
    full[:len(meta)] = meta
    nb = len(meta)
    if corrupt and nb > 3:          # entries a kernel must skip
        full[1] = (E + 5, 0, 128)
        full[nb // 2, 2] = 0
    return full, nb, max_blocks * bm


@pytest.mark.parametrize("TB", [16, 32, 64])
@pytest.mark.parametrize("E8", [1, 2, 4, 8])
def test_route_fused_copies_and_reads(TB, E8):
    EP = 8 * E8
    for E in sorted({EP, EP - 8} - {0}):
        if E8 > 1 and E <= 8 * (E8 // 2):
            continue
        SK = KM.route_fused_params(TB, E8)["SK"]
        for T in (4096, 4100, 16390):
            KM.check_route_fused(TB, E8, E, T, 3 * SK)


def test_route_fused_model_catches_a_wrong_swizzle(monkeypatch):
    """The model's read side recomputes the W_g permutation; a wrong copy-side
    permutation must fail it."""
    monkeypatch.setattr(KM, "wg_swz", lambda row: 2 * ((row >> 3) & 3) + (row & 1))
    with pytest.raises(AssertionError):
        KM.check_route_fused(64, 8, 64, 16384, 2048)


@pytest.mark.parametrize("ngt", [1, 3, 7, 33, 100, 257])
def test_wide_item_order_is_a_bijection(ngt):
    for n_tiles in (1, 3, 8, 11, 16, 28):
        KM.check_wide_item_order(ngt, n_tiles)


@pytest.mark.parametrize("shape", [(600, 1024, 8, 4), (2048, 512, 64, 6), (5000, 512, 3, 2),
                                   (700, 1000, 64, 6), (64, 512, 256, 8)])
@pytest.mark.parametrize("mode", ["random", "skew", "corrupt"])
def test_wide_group_list_matches_its_definition(shape, mode):
    T, d, E, k = shape
    rng = np.random.default_rng(T + E)
    meta, nb, max_rows = _table(T, E, k, 128, rng, skew=mode == "skew", corrupt=mode == "corrupt")
    for GB in (3, 2):
        assert KM.wide_groups_kernel(meta, nb, E, max_rows, GB) == \
            KM.wide_groups_serial(meta, nb, E, max_rows, GB)


def test_wide_group_list_joins_an_unpadded_first_entry():
    """Unpadded tables: an expert's first entry may be partial; the next entry starts
    where it ends and joins its run."""
    meta = np.array([[0, 0, 100], [0, 100, 128], [0, 228, 128], [0, 356, 128], [1, 484, 5]])
    assert KM.wide_groups_kernel(meta, 5, 2, 489) == [(0, 3), (3, 1), (4, 1)]
    assert KM.wide_groups_serial(meta, 5, 2, 489) == [(0, 3), (3, 1), (4, 1)]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("op,K,N", [(0, 1024, 384), (1, 384, 1024), (0, 512, 352), (1, 352, 512),
                                    (0, 256, 136), (1, 1056, 256)])
def test_wide_copies_reads_and_stores(op, K, N, fp8):
    if fp8 and N % 16:
        pytest.skip("fp8 weights need N % 16 == 0")
    rng = np.random.default_rng(K + N)
    T, E, k = 700, 8, 4
    meta, nb, max_rows = _table(T, E, k, 128, rng)
    groups = KM.wide_groups_kernel(meta, nb, E, max_rows)
    out_cols = 128 if op == 0 else 256
    tiles = sorted({0, -(-N // out_cols) - 1})
    for (b, n) in (groups[0], groups[len(groups) // 2], groups[-1]):
        m0 = int(meta[b, 1])
        valid = int(meta[b + n - 1, 1] + meta[b + n - 1, 2]) - m0
        KM.check_wide_item(op, fp8, K, N, int(meta[b, 0]), m0, valid, max_rows, E,
                           n_tiles_check=tiles)
    # the dense segment (shared expert): 384-row spans of T rows, expert 0
    for g in range(-(-T // 384)):
        KM.check_wide_item(op, fp8, K, N, 0, 384 * g, min(384, T - 384 * g), T, 1, n_tiles_check=tiles)


def test_wide_gathered_a_rows():
    """Gate/up with the permutation fused: A rows come from x through row_src / k;
    pad rows (-1) clamp to row 0."""
    rng = np.random.default_rng(3)
    T, E, k, d, de = 500, 8, 4, 512, 256
    idx = rng.integers(0, E, size=(T, k))
    c = O.expert_counts(idx, E)
    meta = O.block_metadata(c, 128)
    pos, row_src = O.permutation(idx, E, 128)
    gather = np.clip(np.where(row_src >= 0, row_src // k, 0), 0, T - 1)
    groups = KM.wide_groups_serial(meta, len(meta), E, len(row_src))
    for (b, n) in groups:
        m0 = int(meta[b, 1])
        valid = int(meta[b + n - 1, 1] + meta[b + n - 1, 2]) - m0
        KM.check_wide_item(0, False, d, de, int(meta[b, 0]), m0, valid, len(row_src), E,
                           gather=gather, n_tiles_check=[0])


def test_wide_row_split():
    KM.check_wide_row_split()


@pytest.mark.parametrize("op,K,N", [(0, 7168, 2048), (1, 2048, 7168), (0, 512, 256),
                                    (1, 1280, 160), (0, 256, 384), (1, 160, 1280)])
def test_fp8d_stage(op, K, N):
    KM.check_fp8d_stage(op, K, N)


@pytest.mark.parametrize("nk", [4, 5, 7, 64, 224])
def test_fp8d_stream(nk):
    for nitems in (1, 2, 3, 7):
        KM.check_fp8d_stream(nk, nitems)


@pytest.mark.parametrize("shape", [(600, 1024, 8, 4, 384), (64, 512, 256, 8, 256),
                                   (2048, 512, 64, 6, 352), (96, 264, 6, 3, 136)])
def test_v2_copies(shape):
    T, d, E, k, de = shape
    rng = np.random.default_rng(T)
    meta, nb, max_rows = _table(T, E, k, 128, rng)
    tiles = [tuple(int(v) for v in meta[b]) for b in range(nb)]
    for op, K, N in ((0, d, de), (1, de, d)):
        if K % 32:
            continue
        KM.check_v2_copies(op, K, N, tiles, E, max_rows)
        dense = [(0, 128 * b, min(128, T - 128 * b)) for b in range(-(-T // 128))]
        KM.check_v2_copies(op, K, N, dense, 1, T)


def test_wgrad_model_computes_the_weight_gradient():
    rng = np.random.default_rng(0)
    E, Km, de, rows = 3, 136, 72, 256
    Nn = 2 * de
    counts, row_off = [37, 0, 70], [0, 128, 128]
    X = rng.standard_normal((rows, Km))
    D = rng.standard_normal((rows, Nn))
    C0, C1 = KM.emu_wgrad(X, D, Km, Nn, de, counts, row_off, E)
    for e in range(E):
        lo, hi = row_off[e], row_off[e] + counts[e]
        ref = X[lo:hi].T @ D[lo:hi]
        np.testing.assert_allclose(C0[e], ref[:, :de], atol=1e-9)
        np.testing.assert_allclose(C1[e], ref[:, de:], atol=1e-9)


def test_nt_model_computes_the_data_gradient():
    rng = np.random.default_rng(1)
    E, rows, de, N = 3, 256, 64, 40
    K = 2 * de
    Bt0 = rng.standard_normal((E, N, de))
    Bt1 = rng.standard_normal((E, N, de))
    A = rng.standard_normal((rows, K))
    tiles = [(0, 0, 37), (2, 128, 70)]
    C = KM.emu_nt(A, Bt0, Bt1, de, de, K, N, tiles, E)
    for (e, m0, valid) in tiles:
        ref = A[m0:m0 + valid] @ np.concatenate([Bt0[e], Bt1[e]], axis=1).T
        np.testing.assert_allclose(C[m0:m0 + valid], ref, atol=1e-9)


@pytest.mark.parametrize("G", [256, 255, 200, 37, 8])
def test_fp8d_split_last_round(G):
    """Every split item's slices are computed once, in order, into distinct slots, and the
    tail kernel adds exactly those slots in slice order; the plan splits only a last
    round that is at most 90 % full."""
    for V in (1, 7, G - 1, G, G + 1, 920, 1610, 3 * G + G // 3, 5 * G + 9 * G // 10,
              2 * G + (G + 15) // 16, 2 * G + max(1, G // 16 - 1)):
        F, R, on = KM.fp8d_tail_plan(V, G)
        assert F * G + R == V and 0 <= R < G
        assert on == (R > 0 and 10 * R <= 9 * G and 16 * R >= G)
        if not on:
            continue
        for nk in (1, 2, 4, 7, 15, 16, 17, 31, 33, 64, 224, 1000, 1024):
            KM.check_fp8d_tail(R, nk, G)
    assert not KM.fp8d_tail_plan(1610, 257)[2]          # grids past the scratch's slots
    assert not KM.fp8d_tail_plan(1610, 256, fits=False)[2]


def test_wide_split_last_round():
    """The 384-row kernel's last-round split on random group lists, grids and column
    tile counts, and on the down launch of the fusedmoe workload's routing (3,136 items,
    12.25 rounds of 256: three trailing groups become nine single blocks)."""
    rng = np.random.default_rng(11)
    for _ in range(3000):
        ng = int(rng.integers(1, 200))
        groups, b = [], 0
        for _ in range(ng):
            n = int(rng.choice([1, 2, 3], p=[0.1, 0.1, 0.8]))
            groups.append((b, n))
            b += n + int(rng.integers(0, 2))
        KM.check_wide_split_tail(groups, int(rng.integers(0, 4)), int(rng.integers(1, 40)),
                                 int(rng.choice([1, 3, 8, 24, 64, 256])))
    # fusedmoe down: 22 dense groups + 90 routed, 28 column tiles, 256 work groups
    routed = [(3 * i, 3) for i in range(90)]
    new, sp = KM.check_wide_split_tail(routed, 22, 28, 256)
    assert sp == 3 and len(new) == 96
    # no split where the items fill whole rounds, or where a single round would not hold
    # only singles
    assert KM.wide_split_tail([(3 * i, 3) for i in range(64)], 0, 16, 256)[1] == 0
    assert KM.wide_split_tail([(3 * i, 3) for i in range(173)], 0, 16, 256)[1] == 0
