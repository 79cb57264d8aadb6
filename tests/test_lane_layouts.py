"""CPU models of the FP8 prefill stage layout and operand reads (no GPU, no library).

The FP8 prefill kernel keeps each 32-key stage's codes in LDS (16-byte chunk c of key row r
at chunk position c ^ swizzle(r)) and widens every MFMA operand after reading it.  These
models restate its address formulas and the measured lane layout of ds_read_b64_tr_b8
(within each 16-lane block, lane 8c + e receives byte e of the 8-byte segments addressed by
lanes c, c + 2, .., c + 14), and check that:

* the K operand of S^T = K Q^T: steps 2p and 2p + 1 take lane group g4's dims
  64p + 16 g4 .. +15 (Q is loaded in the same order), so one 16-byte read gives lane
  (g4, n) those 16 codes of keys n and 16 + n (the 16x16x32 MFMA's A layout, keys on M);
* the K operand of the FP8-MFMA form (v_mfma_scale_f32_16x16x128_f8f6f4, the one-lookup
  path): lane (g4, n) holds dims 128 s + 32 g4 .. +31 of keys n and 16 + n, two 16-byte
  reads per step;
* the V^T operand of O^T += V^T P^T gives lane (g4, n) dim 16t + n of the keys of P's
  k-slots, 4 g4 + 0..3 then 16 + 4 g4 + 0..3 (the order the S^T output leaves P in);
* within a 16-lane block no two lanes read the same 8-byte bank slot of a 256-byte row.
"""

import pytest


def k_swz(row):
    return row & 15


def v_swz_fp8(row):
    return (row & 7) | ((row & 16) >> 1)


def stage(width, swz):
    """Byte address -> (key, dim) of a 32-key FP8 stage of rows `width` bytes wide."""
    m = {}
    for r in range(32):
        for c in range(width // 16):
            for b in range(16):
                m[r * width + 16 * (c ^ swz(r)) + b] = (r, 16 * c + b)
    return m


@pytest.mark.parametrize("dqk", [512, 256])
def test_fp8_k_operand_reads(dqk):
    lds = stage(dqk, k_swz)
    for p in range(dqk // 64):
        for g4 in range(4):
            slots = set()
            for n in range(16):
                kb = n * dqk + 16 * (g4 ^ (n & 3)) + 64 * (n >> 2)
                off = (kb ^ (64 * (p & 3))) + 256 * (p >> 2)
                want = [64 * p + 16 * g4 + e for e in range(16)]
                assert [lds[off + e] for e in range(16)] == [(n, d) for d in want]
                assert [lds[off + 16 * dqk + e] for e in range(16)] == [(16 + n, d) for d in want]
                slots.add((off % 256) // 16)
            assert len(slots) == 16


@pytest.mark.parametrize("dvo", [512, 256])
def test_fp8_v_operand_transpose_reads(dvo):
    lds = stage(dvo, v_swz_fp8)
    for t in range(dvo // 16):
        for g4 in range(4):
            addr = []
            for n in range(16):
                row = 4 * g4 + ((n >> 1) & 3) + 16 * (n >> 3)
                base = row * dvo + 8 * (n & 1) + 16 * v_swz_fp8(row)
                addr.append((base ^ (16 * (t & 15))) + 256 * (t >> 4))
            keys = [4 * g4 + i for i in range(4)] + [16 + 4 * g4 + i for i in range(4)]
            for n in range(16):
                c, e = n // 8, n % 8
                got = [lds[addr[c + 2 * j] + e] for j in range(8)]
                assert got == [(k, 16 * t + n) for k in keys]
            assert len({(a % 256) // 8 for a in addr}) == 16


def test_the_plain_key_order_would_be_wrong():
    """Positive control: reading keys 8 g4 .. 8 g4 + 7 (the natural order of the transpose
    read) does not give P's k-slot order, which is the mistake these models guard."""
    g4 = 1
    natural = [8 * g4 + j for j in range(8)]
    slots = [4 * g4 + i for i in range(4)] + [16 + 4 * g4 + i for i in range(4)]
    assert natural != slots


@pytest.mark.parametrize("dqk", [512, 256])
def test_fp8_mfma_k_operand_reads(dqk):
    lds = stage(dqk, k_swz)
    for s in range(dqk // 128):
        for g4 in range(4):
            for tile in (0, 1):
                slots = set()
                for n in range(16):
                    kb = n * dqk + 128 * (n >> 3) + 16 * ((2 * g4) ^ (n & 7))
                    p0 = (kb ^ (128 * s)) + 16 * dqk * tile
                    p1 = ((kb ^ 16) ^ (128 * s)) + 16 * dqk * tile
                    got = [lds[p0 + e] for e in range(16)] + [lds[p1 + e] for e in range(16)]
                    assert got == [(16 * tile + n, 128 * s + 32 * g4 + b) for b in range(32)]
                    slots.add((p0 % 256) // 16)
                assert len(slots) == 16
