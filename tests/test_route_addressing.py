"""Host replay of the routing proxy pass's address arithmetic (CPU only).

proxy_tile_kernel runs one workgroup per (key chunk, KV head, set of up to HPW
query heads of the group): two waves per query head, 64 proxy rows each as two
32-row MFMA tiles, K tiles staged through registers into LDS by every thread of
the workgroup.  An address outside a buffer faults the GPU, so this replays the
formulas as written in route.hip for every workgroup, wave, lane and tile and
checks that

* the key chunks cover every key block exactly once;
* every query head of every KV group is served by exactly one slot;
* each thread's Q operand reads, K staging loads, LDS stores and LDS operand
  reads stay inside their arrays;
* every (head, key tile, proxy row) partial and every (head, chunk, row)
  maximum/normaliser is written exactly once, inside the workspace regions the
  library sizes (crisp_workspace_bytes for the routing call).
"""
import numpy as np
import pytest

BLK = 128
WG_TARGET = 1024


def proxy_hpw(group):
    return 4 if group >= 4 else (2 if group >= 2 else 1)


def chunking(batch, nb, h_kv, group):
    hpw = proxy_hpw(group)
    units = nb * batch * h_kv * ((group + hpw - 1) // hpw)
    ct = (units + WG_TARGET - 1) // WG_TARGET
    ct = max(1, min(ct, 64, nb))
    return ct, (nb + ct - 1) // ct


def align256(x):
    return (x + 255) // 256 * 256


SHAPES = [  # batch, n, h_q, h_kv, d
    (1, 384, 1, 1, 64), (1, 384, 2, 1, 128), (2, 1152, 4, 2, 128), (1, 2048, 7, 1, 128),
    (1, 4096, 2, 2, 64), (1, 32768, 32, 8, 128), (2, 65536, 8, 2, 64), (1, 131072, 32, 8, 128),
]
LARGE = [(1, 524288, 32, 8, 128), (1, 1 << 20, 32, 8, 128), (1, 1 << 20, 28, 4, 128)]


def replay(batch, n, h_q, h_kv, d, full):
    nb, group = n // BLK, h_q // h_kv
    hpw = proxy_hpw(group)
    nt = 128 * hpw
    cpr = d // 8
    kch = BLK * cpr // nt
    assert kch >= 1 and BLK * cpr % nt == 0
    kstr = d + 8
    klds = BLK * kstr
    nstep = d // 16
    ct, nch = chunking(batch, nb, h_kv, group)
    bh_total = batch * h_q

    # chunks: every key block once, every chunk non-empty
    kbs = np.concatenate([np.arange(c * ct, min(nb, c * ct + ct)) for c in range(nch)])
    assert np.array_equal(np.sort(kbs), np.arange(nb))
    assert all(c * ct < nb for c in range(nch))

    # heads: every (b, g, hg) served by exactly one (z, slot)
    served = {}
    for z in range((group + hpw - 1) // hpw):
        for slot in range(hpw):
            hg = z * hpw + slot
            if hg < group:
                assert hg not in served
                served[hg] = (z, slot)
    assert sorted(served) == list(range(group))

    lanes = np.arange(64)
    qb = nb - 1
    # Q operand reads (elements) of every active wave
    q_elems = batch * h_q * n * d
    for b in range(batch):
        for g in range(h_kv):
            for hg in range(group):
                bh = b * h_q + g * group + hg
                for wh in range(2):
                    for t in range(2):
                        row0 = qb * BLK + 64 * wh + 32 * t
                        p = (bh * n + row0) * d + (lanes & 31) * d + 8 * (lanes >> 5)
                        last = p + 16 * (nstep - 1) + 8
                        assert p.min() >= 0 and last.max() <= q_elems
                        assert (64 * wh + 32 * t + (lanes & 31)).max() < BLK

    # K staging: loads inside the KV head's tile, LDS stores inside the buffer, each chunk once
    tid = np.arange(nt)
    c = (np.arange(kch)[:, None] * nt + tid[None, :]).ravel()
    assert np.array_equal(np.sort(c), np.arange(BLK * cpr))
    krow, kcol = c // cpr, (c % cpr) * 8
    assert krow.max() < BLK and (kcol + 8).max() <= d
    k_elems = batch * h_kv * n * d
    last_tile = ((batch * h_kv - 1) * n + (nb - 1) * BLK) * d
    assert last_tile + (krow * d + kcol + 8).max() <= k_elems
    st = krow * kstr + kcol
    assert (st + 8).max() <= klds
    # LDS operand reads: key row key_row_of_lane(l % 32) of each 32-key sub-tile, 16 bytes per step
    l32 = lanes & 31
    krl = (l32 & ~12) | (((l32 >> 2) & 1) << 3) | (((l32 >> 3) & 1) << 2)
    assert np.array_equal(np.sort(krl), np.repeat(np.arange(32), 2))
    for sub in range(4):
        base = (krl + 32 * sub) * kstr + 8 * (lanes >> 5)
        assert (base + 16 * (nstep - 1) + 8).max() <= klds and base.min() >= 0

    # partial outputs: tilep[bh][kb][3][128], part[bh][chunk][128][2]
    tile_floats = bh_total * nb * 3 * BLK
    part_floats = bh_total * nch * BLK * 2
    rows = np.array([64 * wh + 32 * t + l for wh in range(2) for t in range(2) for l in range(32)])
    assert np.array_equal(np.sort(rows), np.arange(BLK))
    top = ((bh_total - 1) * nb + nb - 1) * 3 * BLK + rows.max() + 2 * BLK
    assert top < tile_floats
    assert (((bh_total - 1) * nch + nch - 1) * BLK + rows.max()) * 2 + 1 < part_floats
    if full:
        seen = np.zeros(tile_floats, dtype=np.int8)
        for bh in range(bh_total):
            for kb in range(nb):
                o = (bh * nb + kb) * 3 * BLK + rows
                for j in range(3):
                    seen[o + j * BLK] += 1
        assert seen.min() == 1 and seen.max() == 1
        seenp = np.zeros(part_floats, dtype=np.int8)
        for bh in range(bh_total):
            for ch in range(nch):
                o = ((bh * nch + ch) * BLK + rows) * 2
                seenp[o] += 1
                seenp[o + 1] += 1
        assert seenp.min() == 1 and seenp.max() == 1

    # the workspace regions the library lays out for these partials
    return (align256(part_floats * 4) + align256(bh_total * BLK * 2 * 4) + align256(tile_floats * 4)
            + align256(bh_total * nb * 2 * 4))


@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{b}_n{n}_h{hq}x{hk}_d{d}" for b, n, hq, hk, d in SHAPES])
def test_proxy_pass_addresses(shape):
    batch, n, h_q, h_kv, d = shape
    full = batch * h_q * (n // BLK) <= 32 * 1024
    replay(batch, n, h_q, h_kv, d, full)


@pytest.mark.parametrize("shape", LARGE, ids=[f"b{b}_n{n}_h{hq}x{hk}_d{d}" for b, n, hq, hk, d in LARGE])
def test_proxy_pass_addresses_large(shape):
    replay(*shape, full=False)


@pytest.mark.parametrize("shape", SHAPES + LARGE)
def test_route_workspace_holds_the_partials(shape):
    """The library's routing workspace is exactly the four regions the kernels write."""
    crisp = pytest.importorskip("long_context_sparse_patsearch_amd")
    try:
        crisp.load()
    except Exception as e:  # pragma: no cover - library not built
        pytest.skip(f"library not loadable: {e}")
    batch, n, h_q, h_kv, d = shape
    need = replay(batch, n, h_q, h_kv, d, full=False)
    sh = crisp.Shape(batch, n, h_q, h_kv, d)
    assert crisp.workspace_bytes(sh, crisp.config(), crisp.CALL_ROUTE) == need
