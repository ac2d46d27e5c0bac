"""Host-side model of the fused conv's LDS ring schedule (the order in which
grad_partial_bf16_kernel<..., FUSE> stages V tiles and forms V' tiles), and of
its multiply-high division. CPU only.

The kernel keeps token rows of V in a ring of 128 rows indexed by token mod
128. Per chunk starting at token t_c: V tiles u = 0..3 (tokens t_c - 48 + 32u
.. + 31) are staged, V'(0) is formed, then tile i stages V tile i + 4 and forms
V'(i + 1). This checks that every in-grid 3x3 tap of every formed token finds
its own token in the ring at that moment, for grids up to the 47 columns the
kernel accepts, and that one more column breaks it (the limit is tight).
"""
import numpy as np
import pytest

RING = 128
T = 32


def _magic(d):
    return 0 if d == 1 else ((1 << 32) + d - 1) // d


def _div(p, magic):
    return p if magic == 0 else (p * magic) >> 32


def _schedule_ok(n_views, gh, gw, ns, P):
    tpv = ns + gh * gw
    n = n_views * tpv
    n_tiles = (n + T - 1) // T
    mt, mg = _magic(tpv), _magic(gw)
    for chunk in range(P):
        tb = n_tiles * chunk // P
        nt = n_tiles * (chunk + 1) // P - tb
        if nt == 0:
            continue
        t_c = tb * T
        ring = [None] * RING

        def stage(u):
            t0 = t_c - 48 + 32 * u
            for r in range(32):
                ring[(t0 + r) % RING] = t0 + r

        def form(j, cpos):
            t0 = (tb + j) * T
            for srow in range(T):
                t = t0 + srow
                p = cpos + srow
                pos = p - _div(p, mt) * tpv
                assert pos == t % tpv
                if t >= n or pos < ns:
                    continue
                pp = pos - ns
                y = _div(pp, mg)
                x = pp - y * gw
                assert (y, x) == divmod(pp, gw)
                for dy in (-1, 0, 1):
                    for dx in (-1, 0, 1):
                        if 0 <= y + dy < gh and 0 <= x + dx < gw:
                            tt = t + dy * gw + dx
                            if ring[tt % RING] != tt:
                                return False
            return True

        cpos = t_c % tpv
        for u in range(4):
            stage(u)
        if not form(0, cpos):
            return False
        for i in range(nt):
            stage(i + 4)
            if i + 1 < nt:
                cpos += T
                while cpos >= tpv:
                    cpos -= tpv
                if not form(i + 1, cpos):
                    return False
    return True


@pytest.mark.parametrize("geom", [(3, 37, 37, 5), (2, 47, 47, 5), (2, 50, 47, 0), (4, 5, 7, 2), (3, 4, 1, 1),
                                  (2, 9, 2, 0), (5, 1, 3, 0), (2, 3, 3, 30), (3, 6, 40, 3)])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_every_tap_finds_its_row(geom, P):
    assert _schedule_ok(*geom, P=P)


def test_one_column_more_breaks_the_ring():
    """At 48 columns some window no longer fits: the kernel's limit of 47 is tight."""
    assert not _schedule_ok(2, 40, 48, 5, P=2)


def test_multiply_high_division_is_exact():
    rng = np.random.default_rng(0)
    for d in list(range(1, 48)) + [1374, 2209 + 5, 4096, 65504]:
        m = _magic(d)
        ps = np.concatenate([np.arange(0, 4096), rng.integers(0, 1 << 16, 20000), [(1 << 16) - 1]])
        for p in ps.tolist():
            assert _div(p, m) == p // d, (p, d)
