"""Host-side model of the bf16 read kernel's data movement (read_bf16_kernel):
which lane holds which element in every 16x16x32 MFMA operand and result, the
permuted order in which W_d is staged, the v_permlane16_swap pairing of the
outputs and the offset of each 16-byte store. CPU only, exact arithmetic.

The model follows one wave's 32-token tile lane by lane with the documented
gfx950 operand layouts and checks that the values stored at each output
address are T(q) of the right token and output channel: the index algebra of
the kernel (not its rounding) is pinned without a GPU.
"""
import numpy as np

D, M = 64, 128
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def mfma16(a_lanes, b_lanes, c_lanes):
    """v_mfma_f32_16x16x32: lane l holds A[l % 16][8 (l // 16) + j],
    B[8 (l // 16) + j][l % 16] (j = 0..7) and C[4 (l // 16) + r][l % 16]
    (r = 0..3). Builds the matrices from the lanes, multiplies, and returns
    the result in the C layout."""
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    C = np.zeros((16, 16))
    for l in range(64):
        A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a_lanes[l]
        B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b_lanes[l]
        C[4 * (l // 16):4 * (l // 16) + 4, l % 16] = c_lanes[l]
    R = A @ B + C
    return np.array([R[4 * (l // 16):4 * (l // 16) + 4, l % 16] for l in range(64)])


def permlane16_swap(x, y):
    """v_permlane16_swap: rows are 16-lane groups; the odd rows of x trade
    places with the even rows of y (new x row 2r+1 = old y row 2r, new y row
    2r = old x row 2r+1)."""
    nx, ny = x.copy(), y.copy()
    for r in (0, 2):
        lo, hi = slice(16 * r, 16 * r + 16), slice(16 * r + 16, 16 * r + 32)
        nx[hi], ny[lo] = y[lo], x[hi]
    return nx, ny


def stage_weights(Wg, Wu, Wd):
    """The LDS images the kernel builds (without the bf16 rounding)."""
    WgP = np.zeros((M, D))
    WuP = np.zeros((M, D))
    for e in range(D):
        for hid in range(M):
            WgP[hid, e] = Wg[e, hid] * -LOG2E
            WuP[hid, e] = Wu[e, hid] * -LN2
    WdP = np.zeros((D, M))
    for o in range(D):
        for kk in range(M):
            s, gg, j = kk >> 5, (kk >> 3) & 3, kk & 7
            hid = 32 * s + (4 * gg + j if j < 4 else 16 + 4 * gg + j - 4)
            WdP[o, kk] = Wd[hid, o]
    return WgP, WuP, WdP


def read_tile_model(Qtile, Wg, Wu, Wd, C_stride):
    """One wave's tile of 32 tokens of one head: returns {element offset from
    the tile's base: value} as the kernel's stores would write them."""
    WgP, WuP, WdP = stage_weights(Wg, Wu, Wd)
    lanes = range(64)
    l16 = [l & 15 for l in lanes]
    g = [l >> 4 for l in lanes]
    # query operand of half b, k-step ks: lane (l16, g) loads channels
    # 32 ks + 8 g .. +7 of token 16 b + l16
    q = [[np.array([Qtile[16 * b + l16[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in lanes])
          for ks in range(2)] for b in range(2)]
    accY = [[np.zeros((64, 4)) for _ in range(4)] for _ in range(2)]
    for s in range(4):
        G0 = [np.zeros((64, 4)) for _ in range(2)]
        G1 = [np.zeros((64, 4)) for _ in range(2)]
        U0 = [np.zeros((64, 4)) for _ in range(2)]
        U1 = [np.zeros((64, 4)) for _ in range(2)]
        for ks in range(2):
            ag0 = np.array([WgP[32 * s + l16[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in lanes])
            au0 = np.array([WuP[32 * s + l16[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in lanes])
            ag1 = np.array([WgP[32 * s + 16 + l16[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in lanes])
            au1 = np.array([WuP[32 * s + 16 + l16[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in lanes])
            for b in range(2):
                G0[b] = mfma16(ag0, q[b][ks], G0[b])
                U0[b] = mfma16(au0, q[b][ks], U0[b])
                G1[b] = mfma16(ag1, q[b][ks], G1[b])
                U1[b] = mfma16(au1, q[b][ks], U1[b])
        for b in range(2):
            h = np.concatenate([G0[b] * U0[b] / (1.0 + np.exp2(G0[b])), G1[b] * U1[b] / (1.0 + np.exp2(G1[b]))],
                               axis=1)  # lane l: the 8 values of its B operand, k = 8 g + j
            for ot in range(4):
                wd = np.array([WdP[16 * ot + l16[l], 32 * s + 8 * g[l]:32 * s + 8 * g[l] + 8] for l in lanes])
                accY[b][ot] = mfma16(wd, h, accY[b][ot])
    stores = {}
    for b in range(2):
        for p in range(2):
            x, y = accY[b][2 * p], accY[b][2 * p + 1]
            xa, xb, ya, yb = x[:, 0:2], x[:, 2:4], y[:, 0:2], y[:, 2:4]  # the packed pairs
            sa0, sa1 = permlane16_swap(xa, ya)
            sb0, sb1 = permlane16_swap(xb, yb)
            for l in lanes:
                vals = np.concatenate([sa0[l], sb0[l], sa1[l], sb1[l]])
                off = (16 * b + l16[l]) * C_stride + 32 * p + 16 * (g[l] & 1) + 8 * (g[l] >> 1)
                for i in range(8):
                    assert off + i not in stores, "two stores write the same element"
                    stores[off + i] = vals[i]
    return stores


def test_read_kernel_layout_puts_every_output_in_place():
    rng = np.random.default_rng(3)
    C = 3 * D  # a row of three heads; the tile base sits at this head's channels
    Qtile = rng.normal(size=(32, D)) / 8
    Wg, Wu, Wd = (rng.normal(size=s) * 0.3 for s in ((D, M), (D, M), (M, D)))
    stores = read_tile_model(Qtile, Wg, Wu, Wd, C)
    # T(q) = (silu(q W_g) * (q W_u)) W_d, by the definition
    Gq, Uq = Qtile @ Wg, Qtile @ Wu
    ref = (Gq / (1.0 + np.exp(-Gq)) * Uq) @ Wd
    assert len(stores) == 32 * D  # every output of the tile, once
    for t in range(32):
        for o in range(D):
            off = t * C + o  # offsets are relative to the tile base at this head's channels
            assert off in stores, (t, o)
            np.testing.assert_allclose(stores[off], ref[t, o], rtol=1e-12, atol=1e-12)


def test_staged_w_d_order_is_a_permutation_of_each_k_step():
    """Every k-step s of the Y product reads the 32 hidden units 32 s .. 32 s
    + 31 of W_d exactly once, in the register order of the G/U result tiles."""
    Wd = np.arange(M * D, dtype=np.float64).reshape(M, D)
    _, _, WdP = stage_weights(np.zeros((D, M)), np.zeros((D, M)), Wd)
    for o in range(D):
        for s in range(4):
            hids = sorted(int(v) // D for v in WdP[o, 32 * s:32 * s + 32])
            assert hids == list(range(32 * s, 32 * s + 32))


def test_permlane16_swap_model_pairs_rows():
    x = np.arange(64)[:, None] * 1.0
    y = 100 + np.arange(64)[:, None] * 1.0
    nx, ny = permlane16_swap(x, y)
    # rows 0 and 2 of x stay; rows 1 and 3 of x come from rows 0 and 2 of y
    assert (nx[0:16] == x[0:16]).all() and (nx[32:48] == x[32:48]).all()
    assert (nx[16:32] == y[0:16]).all() and (nx[48:64] == y[32:48]).all()
    assert (ny[0:16] == x[16:32]).all() and (ny[32:48] == x[48:64]).all()
    assert (ny[16:32] == y[16:32]).all() and (ny[48:64] == y[48:64]).all()
