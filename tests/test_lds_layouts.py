"""CPU checks of the kernels' LDS layouts, DMA placement and bounds.

Each kernel stages tiles in LDS with direct global->LDS loads
(global_load_lds_dwordx4: lane l of an instruction lands its 16 bytes at the
instruction's LDS base + 16 l) and reads them back with XOR-swizzled
addresses. The address formulas below restate those of the HIP sources
(csrc/device_common.h KLane, csrc/sparse_attn.hip, csrc/block_attn.hip,
csrc/kl_loss.hip); the tests check, for every lane:

  * placement: every 16-byte piece of a tile lands exactly once, inside its
    slot, at the position the read side expects;
  * reads: the bytes a lane reads are the rows and head-dim slices its MFMA
    operand needs;
  * banks: the model is 64 banks of 4 bytes delivering 128 bytes per
    cycle, so a 16-byte read is served 8 consecutive lanes per cycle, an
    8-byte read 16 lanes and a 4-byte read 32 lanes; a read is free of bank
    conflicts when the lanes of each such group touch distinct banks (or the
    same word). Under this model every layout below is conflict-free (with
    256 bytes per cycle the gather, block and index-tile reads would not be,
    and with 32 banks the gather, the pass-2 exchange and the d = 64 key
    tiles would not);
  * bounds: every DMA destination and every read stays inside the kernel's
    dynamic LDS allocation.
"""
import itertools

import pytest

BANKS = 64
BYTES_PER_CYCLE = 128


def conflict_free(addrs, width):
    """addrs[lane] = byte address of a `width`-byte read (16 or 8 or 4)."""
    per_pass = BYTES_PER_CYCLE // width
    for g in range(0, 64, per_pass):
        seen = {}
        for lane in range(g, g + per_pass):
            a = addrs[lane]
            for w in range(width // 4):
                word = a // 4 + w
                bank = word % BANKS
                if bank in seen and seen[bank] != word:
                    return False
                seen[bank] = word
    return True


# ---------------------------------------------------------------- KLane
class KLayout:
    """Key tiles of 32 rows (device_common.h KLayout / KLane)."""

    def __init__(self, d, elem):
        self.cpr = d * elem // 16                 # 16-byte chunks per row
        self.rpi = 64 // self.cpr                 # rows per DMA instruction
        self.nc = self.cpr // 2                   # chunks per lane (its half of a row)
        self.per = {8: 2, 16: 4}.get(self.cpr, 8)
        self.bytes = self.nc * 1024

    def sw(self, r):
        return (r >> 1) & 7 if self.cpr == 8 else r & 15

    def dma(self, c, lane):
        """(row, chunk) that lane `lane` of instruction c brings, and where it lands."""
        row = c * self.rpi + lane // self.cpr
        chunk = (lane % self.cpr) ^ self.sw(lane // self.cpr)
        # the lane offset repeats with period `per` in c: d0 ^ (kXs * (c % per))
        kxs = 16 * (4 if self.cpr == 8 else self.rpi)
        d0 = 16 * ((lane % self.cpr) ^ self.sw(lane // self.cpr))
        col_bytes = d0 ^ (kxs * (c % self.per))
        assert col_bytes // 16 == (lane % self.cpr) ^ self.sw(row), (c, lane)
        return row, col_bytes // 16, 1024 * c + 16 * lane

    def read(self, lane, k):
        r = lane & 31
        rx = (r * self.cpr * 16) | (16 * (((lane >> 5) * self.nc) ^ self.sw(r)))
        return rx ^ (16 * k)


@pytest.mark.parametrize("d,elem", [(128, 2), (64, 2), (128, 4), (64, 4)])
def test_key_tile_dma_and_operand_reads(d, elem):
    L = KLayout(d, elem)
    pos = {}
    for c in range(L.nc):
        for lane in range(64):
            row, chunk, at = L.dma(c, lane)
            assert 0 <= at < L.bytes and at not in pos.values()
            assert row < 32
            pos[(row, chunk)] = at
    assert len(pos) == 32 * L.cpr                 # every piece of the tile exactly once
    for k in range(L.nc):
        addrs = []
        for lane in range(64):
            want = (lane & 31, (lane >> 5) * L.nc + k)   # row lane%32, chunk k of its half
            a = L.read(lane, k)
            assert pos[want] == a, (lane, k)
            addrs.append(a)
        assert conflict_free(addrs, 16), (d, elem, k)


# ------------------------------------------------------------ the gather
@pytest.mark.parametrize("tok", [32, 16])
def test_gather_chunk_layout(tok):
    """sparse_attn_mfma_kernel: chunks of `tok` tokens (32: two sets of 16, for
    token supports; 16: one set, for key blocks) x 256 bytes of keys (values
    alike) in a buffer of tok * 256 bytes, piece x of row R at position
    x ^ 2(R & 7); 16x16x32 key reads, value reads for 16x16x32 (two sets) or
    16x16x16 (one set) products."""
    pos = {}
    for c8 in range(tok // 4):
        for lane in range(64):
            q, m = lane >> 4, lane & 15
            xo = (m ^ (2 * q)) if c8 % 2 == 0 else (m ^ (8 + 2 * q))
            row, at = 4 * c8 + q, 1024 * c8 + 16 * lane
            assert at + 16 <= 256 * tok
            pos[(row, xo)] = at
            assert at == 256 * row + 16 * (xo ^ (2 * (row & 7)))
    assert len(pos) == tok * 16
    # key reads: lane (q, m) of set sigma, step s: row 16 sigma + m, d-chunk 4s + q
    for sigma, s in itertools.product(range(tok // 16), range(4)):
        addrs = []
        for lane in range(64):
            q, m = lane >> 4, lane & 15
            kb0 = 256 * m + 16 * (q ^ (2 * (m & 1))) + 64 * ((m & 7) >> 1)
            a = (kb0 ^ (64 * s)) + 4096 * sigma
            assert a == pos[(16 * sigma + m, 4 * s + q)]
            addrs.append(a)
        assert conflict_free(addrs, 16)
    # value reads (8 bytes each): lane 16q + 4e + b reads row 4q + e of a set,
    # d 16 blk + 4b + [0, 4), i.e. half (b & 1) of d-chunk 2 blk + b/2
    for sigma, blk in itertools.product(range(tok // 16), range(8)):
        addrs = []
        for lane in range(64):
            q, e, b = lane >> 4, (lane >> 2) & 3, lane & 3
            r0 = 4 * q + e
            vb0 = 256 * r0 + 32 * (r0 & 7) + 16 * (b >> 1) + 8 * (b & 1)
            a = (vb0 ^ (32 * blk)) + 4096 * sigma
            chunk_at = pos[(16 * sigma + r0, 2 * blk + (b >> 1))]
            assert a == chunk_at + 8 * (b & 1)
            addrs.append(a)
        assert conflict_free(addrs, 8)


# ------------------------------------------------- block tile attention
def row_swizzle(r):
    return ((r & 3) << 1) | ((r >> 2) & 1)


def test_block_attention_chunk_layout():
    """shared_attn_mfma_kernel: 32 key (value) rows, wave w DMAs rows 4w..4w+3,
    d-chunk x of row R at position x ^ f(R), f(R) = 2(R & 3) + ((R >> 2) & 1);
    32x32x16 key reads and transposing value reads."""
    tile = 8192
    pos = {}
    for w in range(8):
        for lane in range(64):
            dq, dm = lane >> 4, lane & 15
            row = 4 * w + dq
            chunk = dm ^ row_swizzle(row)
            at = 1024 * w + 16 * lane
            assert at + 16 <= tile
            pos[(row, chunk)] = at
    assert len(pos) == 32 * 16
    # keys: lane l reads row R = l % 32, k-step s (d = 16 s + 8 hl): chunk 2s + hl
    for s in range(8):
        addrs = []
        for lane in range(64):
            R, hl = lane & 31, lane >> 5
            ak = 256 * R + 16 * (hl ^ ((R >> 2) & 1)) + 32 * (R & 3)
            a = (ak ^ (32 * (s & 3))) + (128 if s >= 4 else 0)
            assert a == pos[(R, 2 * s + hl)], (lane, s)
            addrs.append(a)
        assert conflict_free(addrs, 16)
    # values: lane 16 G + 4 e + cc reads row 4(G >> 1) + e (+ 16 ks + 8 sec),
    # d 32 dt + 16(G & 1) + 4 cc + [0, 4)
    for dt, ks, sec in itertools.product(range(4), range(2), range(2)):
        addrs = []
        for lane in range(64):
            G16, e, cc = lane >> 4, (lane >> 2) & 3, lane & 3
            u = 2 * (G16 & 1) + (cc >> 1)
            sw = 2 * e + (G16 >> 1)
            av = 256 * (4 * (G16 >> 1) + e) + 8 * (cc & 1) + 16 * (u ^ sw)
            a = (av ^ (64 * dt)) + 4096 * ks + 2048 * sec
            row = 4 * (G16 >> 1) + e + 16 * ks + 8 * sec
            dd = 32 * dt + 16 * (G16 & 1) + 4 * cc
            assert a == pos[(row, dd // 8)] + 2 * (dd % 8), (lane, dt, ks, sec)
            addrs.append(a)
        assert conflict_free(addrs, 8)


# ---------------------------------------------- KL index tiles (d_idx = 64)
def idx_swizzle(r):
    return ((r & 3) << 1) | ((r >> 2) & 1)


def test_kl_index_tile_layout():
    """32 rows x 128 bytes (q_idx / k_idx), d-chunk x of row R at x ^ f(R);
    rows 8w .. 8w+7 by wave w < 4; operand reads and transposing reads."""
    pos = {}
    for w in range(4):
        for lane in range(64):
            drow = 8 * w + (lane >> 3)
            chunk = (lane & 7) ^ idx_swizzle(drow)
            at = 1024 * w + 16 * lane
            pos[(drow, chunk)] = at
            assert at == 128 * drow + 16 * (lane & 7)
    assert len(pos) == 32 * 8
    for s in range(4):            # fragment (row lane%32, d = 16 s + 8 hf): chunk 2s + hf
        addrs = []
        for lane in range(64):
            fr, hf = lane & 31, lane >> 5
            off = 128 * fr + 16 * (hf ^ ((fr >> 2) & 1)) + 32 * (fr & 3)
            a = off ^ (32 * s)
            assert a == pos[(fr, 2 * s + hf)]
            addrs.append(a)
        assert conflict_free(addrs, 16)
    for dt in range(2):           # rows 16 ks + 8 sec + 4(l/32)... as in block attention
        for ks, sec in itertools.product(range(2), range(2)):
            addrs = []
            for lane in range(64):
                G16, e, cc = lane >> 4, (lane >> 2) & 3, lane & 3
                u = 2 * (G16 & 1) + (cc >> 1)
                sw = 2 * e + (G16 >> 1)
                tr_off = 128 * (4 * (G16 >> 1) + e) + 8 * (cc & 1) + 16 * (u ^ sw)
                a = (tr_off ^ (64 * dt)) + 1024 * (2 * ks + sec)
                row = 4 * (G16 >> 1) + e + 16 * ks + 8 * sec
                dd = 32 * dt + 16 * (G16 & 1) + 4 * cc
                assert a == pos[(row, dd // 8)] + 2 * (dd % 8), (lane, dt, ks, sec)
                addrs.append(a)
            assert conflict_free(addrs, 8)


# ------------------------------------------------ KL key-major gradient
def test_kl_key_gradient_lds_map_and_bounds():
    """kl_dk_kernel: two query-tile buffers of 40 KiB (4 query heads' 32-row
    tiles, q_idx rows, dense and student LSE); every DMA piece lands once,
    inside its buffer, where the key-tile reads of KLane expect it."""
    L = KLayout(128, 2)
    buf_bytes, q_off, qidx_off = 40960, 0, 4 * 8192
    lse_off, lset_off = qidx_off + 4096, qidx_off + 4096 + 512
    assert lset_off + 256 <= buf_bytes
    landed = {}
    for buf in range(2):
        for w in range(8):                       # wave w: head w//2, pieces 4(w%2)+p
            hh = w >> 1
            for p in range(4):
                c = 4 * (w & 1) + p
                for lane in range(64):
                    row = 4 * c + (lane >> 4)
                    chunk = (lane & 15) ^ (row & 15)
                    at = buf * buf_bytes + q_off + 8192 * hh + 1024 * c + 16 * lane
                    assert at + 16 <= 2 * buf_bytes and at not in landed
                    landed[at] = (buf, hh, row, chunk)
        for w in range(4):                       # q_idx rows 8w .. 8w+7
            for lane in range(64):
                at = buf * buf_bytes + qidx_off + 1024 * w + 16 * lane
                assert at + 16 <= buf * buf_bytes + lse_off
        for hh in range(4):
            for lane in range(64):
                for k in range(L.nc):
                    a = buf * buf_bytes + q_off + 8192 * hh + L.read(lane, k)
                    assert landed[a] == (buf, hh, lane & 31, 8 * (lane >> 5) + k)
    for w in range(8):                           # the prologue's temporary key slots
        assert 8192 * (w + 1) <= 2 * buf_bytes


# --------------------------------------------------- pass-2 partial masses
def test_pass2_partial_exchange_banks():
    """Partial masses of KV head g, register r, source lane l at word
    g*1088 + 68 r + l: the lane-major writes (one register per instruction)
    and the row owners' reads hit distinct banks, for both ownerships: with
    the KV heads fixed at 8, waves 0..3 own 8 rows each (8 lanes a row, keys
    m = 8 e + j, 4 per lane); otherwise every wave owns 32/Hkv rows (2 Hkv
    lanes a row; here Hkv = 8: 4 rows, 16 lanes, keys m = 16 e + j)."""
    pitch, head = 68, 17 * 64
    for g, r in itertools.product(range(8), range(16)):
        addrs = [4 * (g * head + pitch * r + lane) for lane in range(64)]
        assert conflict_free(addrs, 4)
    # owners: 4 rows per wave, 16 lanes per row, key offsets m = 16 e + j
    for w, e, gg in itertools.product(range(8), range(2), range(8)):
        addrs = []
        for lane in range(64):
            own_n, own_j = 4 * w + lane // 16, lane % 16
            mo = 16 * e + own_j
            r, h2 = ((mo >> 3) << 2) | (mo & 3), (mo >> 2) & 1
            addrs.append(4 * (gg * head + pitch * r + own_n + 32 * h2))
        assert conflict_free(addrs, 4)
    # owners with the KV heads fixed at 8: waves 0..3, 8 rows each, 8 lanes a
    # row, key offsets m = 8 e + j
    for w, e, gg in itertools.product(range(4), range(4), range(8)):
        addrs = []
        for lane in range(64):
            own_n, own_j = 8 * w + lane // 8, lane % 8
            mo = 8 * e + own_j
            r, h2 = ((mo >> 3) << 2) | (mo & 3), (mo >> 2) & 1
            addrs.append(4 * (gg * head + pitch * r + own_n + 32 * h2))
        assert conflict_free(addrs, 4)
    # every (row, key) of the tile has exactly one owner lane and entry
    seen = set()
    for w, lane, e in itertools.product(range(4), range(64), range(4)):
        seen.add((8 * w + lane // 8, 8 * e + lane % 8))
    assert seen == {(n, m) for n in range(32) for m in range(32)}


# ------------------------------------------- pass 2's key operand copy
def test_pass2_key_operand_copy():
    """Pass 2 with 8 KV heads, bf16, d = 128 loads its key tiles from a copy of
    K in MFMA operand order (passes.hip key_operands_kernel): entry
    ((g T + t) 8 + c) 64 + l holds the 16-byte chunk c of lane l's operand of
    tile t of KV head g, and wave g reads tile t as 8 loads of 64 consecutive
    entries (entry t*512 + 64 c + l for lane l). Every lane must get the
    operand chunk the LDS staging gives it (row l % 32, chunk (l/32) nc + c of
    the row's 16 chunks), every chunk of every padded tile must appear
    exactly once, and rows past n repeat row n - 1."""
    L = KLayout(128, 2)
    hkv, nc = 8, 8
    for n in (1, 31, 33, 100):
        ntiles = (n + 31) // 32
        seen = set()
        for idx in range(hkv * ntiles * 512):             # the copy kernel's thread ids
            l, c, gt = idx & 63, (idx >> 6) & 7, idx >> 9
            t, g = gt % ntiles, gt // ntiles
            row = min(t * 32 + (l & 31), n - 1)
            chunk = 8 * (l >> 5) + c                     # d = 64 (l/32) + 8 c, in 16-byte units
            key = (g, t * 32 + (l & 31), chunk)
            assert key not in seen
            seen.add(key)
            if t * 32 + (l & 31) >= n:
                assert row == n - 1
            # the wave's read of tile t, instruction c, lane l hits entry idx
            assert ((g * ntiles + t) * 8 + c) * 64 + l == idx
            assert (row % 32 == (l & 31)) or t * 32 + (l & 31) >= n
            assert (l & 31, chunk) == (l & 31, (l >> 5) * L.nc + c)
        assert len(seen) == hkv * ntiles * 32 * 16
        # the workspace figure (pass2_key_operand_bytes)
        assert hkv * ntiles * 512 * 16 == ntiles * 32 * 8 * 128 * 2
    # each load instruction reads 64 consecutive 16-byte entries: 1 KiB contiguous
    for c in range(nc):
        addrs = [16 * (64 * c + l) for l in range(64)]
        assert addrs == list(range(addrs[0], addrs[0] + 1024, 16))
