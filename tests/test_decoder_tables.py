"""Pins for the test-side definition of the decoder tables (decoder_tables.py):
entries worked out by hand for a four-symbol code.  CPU only."""
import numpy as np

from decoder_tables import multicode_table, pair_table_section

# symbols 10, 20, 30, 40 with lengths 1, 2, 3, 3: canonical codes 0, 10, 110, 111
LENGTHS = np.zeros(256, np.uint8)
LENGTHS[[10, 20, 30, 40]] = [1, 2, 3, 3]
CODES = np.zeros(256, np.uint32)
CODES[[10, 20, 30, 40]] = [0b0, 0b10, 0b110, 0b111]


def window(bits):
    """Window index whose k-th stream bit is bits[k]."""
    return sum(int(b) << k for k, b in enumerate(bits))


def test_multicode_entries_by_hand():
    # BF16 layout (symbol bytes, rotated right by one bit)
    rot = {s: (s >> 1) | ((s & 1) << 7) for s in (10, 20, 30, 40)}
    tab = multicode_table(0, LENGTHS, CODES, K=4)
    # 0000: four codes "0", starts 0..3, 4 bits
    assert tab[window("0000")] == rot[10] * 0x01010101 | 4 << 32 | 0b111 << 37 | 4 << 56
    # 1011: "10" then "11" is no whole code: one code, 2 bits
    assert tab[window("1011")] == rot[20] | 2 << 32 | 1 << 56
    # 0110: "0" then "110": two codes, the second starting at bit 1, 4 bits
    assert tab[window("0110")] == rot[10] | rot[30] << 8 | 4 << 32 | 0b1 << 37 | 2 << 56
    # 1110: "111" then "0": 4 bits, second code starts at bit 3
    assert tab[window("1110")] == rot[40] | rot[10] << 8 | 4 << 32 | 0b100 << 37 | 2 << 56
    # 1101 (K = 4): "110", then "1" is no whole code
    assert tab[window("1101")] == rot[30] | 3 << 32 | 1 << 56


def test_multicode_uint4_nibbles_by_hand():
    # uint4 symbols 3, 5, 9, 12 with the same lengths and codes: the symbols
    # are nibbles, four bits per code in order
    ln = np.zeros(256, np.uint8)
    ln[[3, 5, 9, 12]] = [1, 2, 3, 3]
    codes = np.zeros(256, np.uint32)
    codes[[3, 5, 9, 12]] = [0b0, 0b10, 0b110, 0b111]
    tab = multicode_table(2, ln, codes, K=4)
    assert tab[window("0000")] == 0x3333 | 4 << 32 | 0b111 << 37 | 4 << 56
    assert tab[window("1011")] == 5 | 2 << 32 | 1 << 56
    assert tab[window("0110")] == 3 | 9 << 4 | 4 << 32 | 0b1 << 37 | 2 << 56
    assert tab[window("1110")] == 12 | 3 << 4 | 4 << 32 | 0b100 << 37 | 2 << 56
    assert tab[window("1101")] == 9 | 3 << 32 | 1 << 56
    five = multicode_table(2, ln, codes, K=6)[window("000000")]
    assert five == 0x33333 | 5 << 32 | 0b1111 << 37 | 5 << 56


def test_multicode_fifth_code_and_bf16_rotation():
    tab = multicode_table(0, LENGTHS, CODES, K=6)
    e = tab[window("000000")]   # five codes "0" fill the entry, the sixth is left
    rot = (10 >> 1) | ((10 & 1) << 7)
    assert e & 0xFFFFFFFF == rot * 0x01010101
    assert (e >> 48) & 0xFF == rot and (e >> 56) == 5 and (e >> 32) & 31 == 5
    assert (e >> 37) & 0x7FF == 0b1111


def test_multicode_empty_window():
    # a code longer than the window leaves the entry zero
    ln = LENGTHS.copy()
    ln[[10, 20, 30, 40]] = [1, 2, 3, 3]
    tab = multicode_table(2, ln, CODES, K=2)
    assert tab[window("11")] == 0 and tab[window("10")] != 0


def test_pair_table_by_hand():
    sec = pair_table_section(LENGTHS, CODES, K=4)
    tab = sec[: 4 << 4].view(np.uint32)
    assert tab[window("0000")] == 2 | 10 << 8 | 10 << 16 | 2 << 24   # two codes at most
    assert tab[window("1011")] == 2 | 20 << 8 | 1 << 24
    assert tab[window("1100")] == 4 | 30 << 8 | 10 << 16 | 2 << 24
    assert np.array_equal(sec[4 << 4:], LENGTHS)
