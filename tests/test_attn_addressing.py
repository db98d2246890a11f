"""Host replay of the attention kernels' address arithmetic (CPU only).

The attention kernels fill their LDS stage buffers with direct global->LDS
loads whose per-lane byte offsets are computed once per kernel, read MFMA
operands from those buffers through a chunk swizzle, and take their work
items from per-XCD queues.  An address outside a buffer or array faults the
GPU, so this replays the same formulas, as written in attn.hip, for every
lane, wave, load and stage, and checks that

* each stage load writes exactly the 16-byte chunks of its LDS buffer (every
  chunk once, nothing outside), with the row and swizzled chunk that the
  operand reads expect there;
* each load reads inside the stage's rows of K (row-major) or V^T, for every
  key block of the longest supported input (n = 2^20), without 32-bit offset
  overflow;
* the operand reads stay inside their buffers;
* the work queues hand out every (head, query block) item exactly once.
"""
import numpy as np
import pytest

BLK, KS = 128, 64
NXCD = 8
N_MAX = 1 << 20


def key_row_of_lane(l32):
    return (l32 & ~12) | (((l32 >> 2) & 1) << 3) | (((l32 >> 3) & 1) << 2)


# --- d = 128 (attn_q64_kernel): two waves, eight 16-byte loads per wave and stage ---------------
D128 = dict(D=128, KROW=256, VROW=KS * 2, KBYTES=KS * 256, VBYTES=128 * KS * 2, waves=2)


def q64_direct_loads(n):
    """(wave, lane, i) -> (K byte offset from the stage base, K LDS byte offset in the buffer,
    V^T byte offset from the stage base, V^T LDS byte offset), as attn_q64_kernel computes them."""
    D = 128
    out = []
    for w in range(2):
        for lane in range(64):
            pc = lane & 15
            r0 = 4 * w + (lane >> 4)
            r1 = r0 + 8
            kd0 = (r0 * D + (pc ^ (r0 & 15)) * 8) * 2
            kd1 = (r1 * D + (pc ^ (r1 & 15)) * 8) * 2
            vr0 = 8 * w + (lane >> 3)
            vd0 = (vr0 * n + ((lane & 7) ^ ((vr0 >> 1) & 7)) * 8) * 2
            for i in range(8):
                kd = (kd1 if i & 1 else kd0) + (i >> 1) * 4096
                vd = vd0 + i * 16 * n * 2
                lds = w * 1024 + 2048 * i + 16 * lane      # lds0w + IMM + 16 lane, relative to the buffer
                out.append((w, lane, i, kd, lds, vd, lds))
    return out


@pytest.mark.parametrize("n", [384, 4096, 131072, 524288, N_MAX])
def test_q64_direct_loads_fill_their_buffers(n):
    D, KBYTES, VBYTES = 128, D128["KBYTES"], D128["VBYTES"]
    seen_k = np.zeros(KBYTES // 16, dtype=np.int64)
    seen_v = np.zeros(VBYTES // 16, dtype=np.int64)
    for w, lane, i, kd, klds, vd, vlds in q64_direct_loads(n):
        assert kd < 2 ** 32 and vd < 2 ** 32
        # K: source row and logical chunk; LDS row and physical chunk
        row, chunk = divmod(kd // 2, D)
        assert kd % 16 == 0 and 0 <= row < KS, (w, lane, i)
        p = klds // 16
        assert 0 <= klds and klds + 16 <= KBYTES
        assert p // 16 == row and p % 16 == (chunk // 8) ^ (row & 15), (w, lane, i)
        seen_k[p] += 1
        # V^T: source (head-dim row, key chunk) inside the stage's 64 keys
        vrow, key = divmod(vd // 2, n)
        assert vd % 16 == 0 and 0 <= vrow < D and key % 8 == 0 and key + 8 <= KS, (w, lane, i)
        p = vlds // 16
        assert 0 <= vlds and vlds + 16 <= VBYTES
        assert p // 8 == vrow and p % 8 == (key // 8) ^ ((vrow >> 1) & 7), (w, lane, i)
        seen_v[p] += 1
    assert np.all(seen_k == 1) and np.all(seen_v == 1)


@pytest.mark.parametrize("n", [384, N_MAX])
def test_q64_stage_bases_stay_inside_the_head(n):
    """Stage (kb, hf) of a row reads K bytes [(kb*128 + hf*64)*D*2 + kd, +16) and V^T
    elements at (kb*128 + hf*64) + vd/2; for every block of the longest row both stay
    inside the KV head's array (dummy loads reread a valid block)."""
    D = 128
    loads = q64_direct_loads(n)
    kmax = max(kd for w, l, i, kd, a, vd, b in loads)
    vmax = max(vd for w, l, i, kd, a, vd, b in loads)
    nb = n // BLK
    last_stage = (nb - 1) * BLK + KS                  # kb = nb - 1, hf = 1
    assert last_stage * D * 2 + kmax + 16 <= n * D * 2
    assert last_stage * 2 + vmax + 16 <= D * n * 2
    assert (nb * BLK) * D * 2 < 2 ** 63


def test_q64_operand_reads_match_the_swizzle():
    D, KROW, VROW, KBYTES, VBYTES = 128, 256, KS * 2, D128["KBYTES"], D128["VBYTES"]
    for lane in range(64):
        hi = lane >> 5
        krow = key_row_of_lane(lane & 31)
        kfix = krow & 15
        vrow = lane & 31
        vfix = (vrow >> 1) & 7
        for st in range(8):
            koff = krow * KROW + (((2 * st + hi) ^ kfix) * 16)
            for ks in range(2):
                a = koff + 32 * ks * KROW
                assert 0 <= a and a + 16 <= KBYTES
                row, phys = a // KROW, (a % KROW) // 16
                assert row == krow + 32 * ks and phys == (2 * st + hi) ^ (row & 15)
        for cc in range(4):
            voff = vrow * VROW + (((2 * cc + hi) ^ vfix) * 16)
            for ds in range(4):
                a = voff + 32 * ds * VROW
                assert 0 <= a and a + 16 <= VBYTES
                row, phys = a // VROW, (a % VROW) // 16
                assert row == vrow + 32 * ds and phys == (2 * cc + hi) ^ ((row >> 1) & 7)


def test_q64_lds_layout_fits():
    """Two K and two V^T stage buffers per workgroup (64 KiB), two workgroups per CU."""
    per_wg = 2 * D128["KBYTES"] + 2 * D128["VBYTES"] + 4      # + the work-item slot
    assert 2 * per_wg <= 160 * 1024


# --- d = 64 (attn_kernel): four waves, two 16-byte loads per wave and stage -----------------------
def test_d64_direct_loads_fill_their_buffers():
    D, KROW, KCPR, VCPR = 64, 128, 8, 8
    KBYTES, VBYTES = KS * KROW, D * KS * 2
    for n in (384, 4096, N_MAX):
        seen_k = np.zeros(KBYTES // 16, dtype=np.int64)
        seen_v = np.zeros(VBYTES // 16, dtype=np.int64)
        for w in range(4):
            for lane in range(64):
                p0 = w * 64 + lane
                kr0, vr0 = p0 // KCPR, p0 // VCPR
                k0 = (kr0 * D + ((p0 % KCPR) ^ ((kr0 >> 1) & 7)) * 8) * 2
                v0 = (vr0 * n + ((p0 % VCPR) ^ ((vr0 >> 1) & 7)) * 8) * 2
                for i in range(2):
                    kd = k0 + i * (4 * 64 // KCPR * KROW)
                    vd = v0 + i * (4 * 64 // VCPR) * n * 2
                    lds = w * 1024 + 4096 * i + 16 * lane
                    assert kd < 2 ** 32 and vd < 2 ** 32
                    row, chunk = divmod(kd // 2, D)
                    p = lds // 16
                    assert lds + 16 <= KBYTES and p // KCPR == row and p % KCPR == (chunk // 8) ^ ((row >> 1) & 7)
                    seen_k[p] += 1
                    vrow, key = divmod(vd // 2, n)
                    assert vrow < D and key + 8 <= KS
                    assert lds + 16 <= VBYTES and p // VCPR == vrow and p % VCPR == (key // 8) ^ ((vrow >> 1) & 7)
                    seen_v[p] += 1
        assert np.all(seen_k == 1) and np.all(seen_v == 1)


# --- work queues ------------------------------------------------------------------------------------
def queue_chunk(nb):
    cap = 32 if nb <= 1024 else 64
    qc = nb // 32
    return 1 if qc < 1 else min(qc, cap)


def queue_items(nb, bh_total):
    qc = queue_chunk(nb)
    chunks = (nb + qc - 1) // qc
    per_queue = (chunks + NXCD - 1) // NXCD * bh_total * qc
    span = bh_total * qc
    items = []
    for x in range(NXCD):
        for u in range(per_queue):
            j, rem = divmod(u, span)
            bh = rem // qc
            qtop = (j * NXCD + x) * qc + rem % qc
            if qtop < nb:
                items.append((bh, nb - 1 - qtop))
    return items, per_queue


@pytest.mark.parametrize("nb,bh", [(3, 1), (9, 8), (32, 2), (256, 32), (1024, 32), (2048, 28), (4096, 32), (8192, 4)])
def test_queues_cover_every_item_once(nb, bh):
    items, per_queue = queue_items(nb, bh)
    assert len(items) == len(set(items)) == nb * bh
    assert all(0 <= h < bh and 0 <= q < nb for h, q in items)
    assert per_queue * NXCD < 2 ** 31
