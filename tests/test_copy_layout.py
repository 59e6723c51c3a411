"""Host check of the forward attention's tile-copy addressing.

attn_fwd_bf16_kernel copies each 64-key K and V tile from HBM straight into
LDS (buffer_load ... lds): lane i of a copy writes 16 bytes at LDS offset
1024 j' + 16 i (j' = the copy's index within the tile) and reads them at a
source offset made of a per-lane register and a wave-uniform scalar.  The
kernel states the layout those copies must produce:

* K: LDS row R of a tile holds key 32 (R div 32) + k(R mod 32), with
  k(8q + 4h + r) = 16h + 4q + r (MFMA A-operand row order), and its physical
  16-byte chunk c' holds logical chunk c' XOR (R mod CPR);
* V: LDS row R holds key R, physical chunk c' holds logical chunk
  c' XOR ((R mod 4) << (2 if CPR = 16 else 1)).

The offsets below are the kernel's (lane_src, dk_voff, dk_soff, dv_soff),
restated; the test checks that they produce exactly that image, every LDS
byte written once, for both head sizes.
"""
import pytest

KT = 64


def _offsets(D):
    RB = 2 * D
    TB = KT * RB
    ndma = TB // 4096

    def lane_src(l):
        if D == 128:
            q = l >> 4
            return 256 * q + 16 * ((l & 15) ^ q), 256 * q + 16 * ((l & 15) ^ (4 * q))
        q8, c = l >> 3, l & 7
        return (128 * (16 * ((q8 >> 2) & 1) + (q8 & 3)) + 16 * (c ^ q8),
                128 * q8 + 16 * (c ^ ((q8 & 3) << 1)))

    def dk_voff(l, j):
        k, _ = lane_src(l)
        return k ^ (64 * j) if D == 128 else k

    def dk_soff(rbw, j):
        if D == 128:
            return 256 * (32 * (rbw >> 1) + 8 * (rbw & 1) + 16 * (j & 1) + 4 * (j >> 1))
        return 128 * (32 * (rbw >> 1) + 4 * (2 * (rbw & 1) + j))

    def dv_soff(rbw, j):
        return 256 * (16 * rbw + 4 * j) if D == 128 else 128 * 8 * (2 * rbw + j)

    return RB, TB, ndma, lane_src, dk_voff, dk_soff, dv_soff


def _key_of_krow(r):
    return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3)


@pytest.mark.parametrize("D", [64, 128])
def test_tile_copies_produce_the_stated_lds_image(D):
    RB, TB, ndma, lane_src, dk_voff, dk_soff, dv_soff = _offsets(D)
    CPR = D // 8
    vshift = 2 if CPR == 16 else 1
    seen_k, seen_v = set(), set()
    for rbw in range(4):              # the four waves of a key group
        for j in range(ndma):
            for lane in range(64):
                dst = (rbw * ndma + j) * 1024 + 16 * lane
                R, cp = dst // RB, (dst % RB) // 16
                # K
                src = dk_soff(rbw, j) + dk_voff(lane, j)
                assert src % 16 == 0 and 0 <= src < TB
                assert src // RB == 32 * (R // 32) + _key_of_krow(R % 32), (D, rbw, j, lane)
                assert (src % RB) // 16 == cp ^ (R % CPR), (D, rbw, j, lane)
                seen_k.add(dst)
                # V
                src = dv_soff(rbw, j) + lane_src(lane)[1]
                assert src % 16 == 0 and 0 <= src < TB
                assert src // RB == R, (D, rbw, j, lane)
                assert (src % RB) // 16 == cp ^ ((R & 3) << vshift), (D, rbw, j, lane)
                seen_v.add(dst)
    assert seen_k == seen_v == set(range(0, TB, 16))


def test_key_row_map_is_a_permutation_matching_the_accumulator_layout():
    # accumulator register r of lane l of S^T = K Q^T (32x32x16 MFMA) is A row
    # 8 (r div 4) + 4 (l div 32) + r mod 4; that row must hold key 16 (l div 32) + r
    assert sorted(_key_of_krow(r) for r in range(32)) == list(range(32))
    for lane in range(64):
        for r in range(16):
            a_row = 8 * (r // 4) + 4 * (lane // 32) + r % 4
            assert _key_of_krow(a_row) == 16 * (lane // 32) + r
