"""The decoder-side tables the library derives from a codebook's lengths
(its DTAB section), built here the slow way for tests.

These tables are this library's own accelerator for the decode kernels, not
part of the method on the pages (whose tables are the hierarchical 256-entry
ones the oracle builds), so their definition lives with the tests rather than
in the oracle.  Both are built by prefix matching over the canonical code
strings, window by window; the code strings come from the oracle's canonical
codes.

multicode_table (BF16 and uint4, u64 per K-bit window; bit k of the window
index is the k-th stream bit): the whole codes inside the window, at most
five, in order.  Bits 0..31 symbol bytes of codes 0..3 (BF16: the exponent
rotated right by one bit), 32..36 bits consumed, 37..47 a flag for each code
that starts at window bit 1..11, 48..55 symbol byte of code 4, 56..63 number
of codes; 0 when no whole code fits.  uint4 holds the symbols as nibbles:
bits 0..19 the low nibbles of codes 0..4 (4 bits per code, in order).

pair_table_section (uint8): u32 per 13-bit window, at most two codes: bits
0..3 bits consumed, 8..15 and 16..23 the two symbols (0 when one), 24..31
number of codes; 0 when no whole code fits; then the 256 code lengths.
"""
import numpy as np


def code_strings(lengths, codes):
    """symbol -> its code as a string of '0'/'1', first bit first."""
    return {s: format(int(codes[s]), "0%db" % int(lengths[s])) for s in range(256) if lengths[s]}


def _window_codes(inv, bits, most):
    """Symbols and start positions of the whole codes at the front of bits."""
    syms, starts, pos, cur = [], [], 0, ""
    for i, b in enumerate(bits):
        cur += b
        if cur in inv:
            syms.append(inv[cur])
            starts.append(pos)
            pos = i + 1
            cur = ""
            if len(syms) == most:
                break
    return syms, starts, pos


def multicode_table(kind, lengths, codes, K=12):
    inv = {v: k for k, v in code_strings(lengths, codes).items()}
    tab = np.zeros(1 << K, np.uint64)
    for w in range(1 << K):
        bits = "".join(str((w >> k) & 1) for k in range(K))
        syms, starts, pos = _window_codes(inv, bits, 5)
        if not syms:
            continue
        v = 0
        for i, s in enumerate(syms):
            if kind == 2:
                v |= (s & 0xF) << (4 * i)
                continue
            byte = ((s >> 1) | ((s & 1) << 7)) if kind == 0 else s
            v |= byte << (8 * i if i < 4 else 48)
        flags = sum(1 << (st - 1) for st in starts if st > 0)
        tab[w] = v | pos << 32 | flags << 37 | len(syms) << 56
    return tab


def pair_table_section(lengths, codes, K=13):
    inv = {v: k for k, v in code_strings(lengths, codes).items()}
    tab = np.zeros(1 << K, np.uint32)
    for w in range(1 << K):
        bits = "".join(str((w >> k) & 1) for k in range(K))
        syms, _, pos = _window_codes(inv, bits, 2)
        if syms:
            tab[w] = pos | syms[0] << 8 | (syms[1] if len(syms) > 1 else 0) << 16 | len(syms) << 24
    return np.concatenate([tab.view(np.uint8), np.asarray(lengths, np.uint8)])


def dtab_of(kind, lengths, codes):
    """The DTAB section bytes the library should hold for these lengths."""
    if kind == 1:
        return pair_table_section(lengths, codes)
    return multicode_table(kind, lengths, codes).view(np.uint8)
