"""Brute-force references for tiny inputs, written independently of the C
oracle: codes as text, words parsed from bit strings with int(chunk, 2),
float32 arithmetic through numpy scalars.  Used only to pin the oracle.

Follows the MXNet PR "2bit gradient compression" ("Two bit quantization",
"Format of compressed gradient") and CD-SGD 3.4.1 (a sent code is worth the
threshold itself)."""
import numpy as np

F = np.float32


def gc2_bits(g, r, t):
    """Returns (word list, new residual list) for one quantize step."""
    t = F(t)
    text = ""
    r_new = []
    for gi, ri in zip(g, r):
        v = F(gi) + F(ri)
        if v >= t:
            text += "11"
            r_new.append(v - t)
        elif v <= -t:
            text += "10"
            r_new.append(v - (-t))
        else:
            text += "00"
            r_new.append(v - F(0.0))
    while len(text) % 32:
        text += "0"
    words = [int(text[k:k + 32], 2) for k in range(0, len(text), 32)]
    return words, r_new


def codes_from_words(words, n):
    """List of n codes as 2-character strings, read left to right."""
    text = "".join(format(int(w), "032b") for w in words)
    return [text[2 * i:2 * i + 2] for i in range(n)]


def code_value(code, t):
    t = F(t)
    return {"11": t, "10": -t}.get(code, F(0.0))


def dequant_reduce(worker_words, n, t):
    per = [codes_from_words(w, n) for w in worker_words]
    out = []
    for i in range(n):
        a = F(0.0)
        for w in range(len(per)):
            a = a + code_value(per[w][i], t)
        out.append(a)
    return out


def nibbles_from_words(words, n):
    text = "".join(format(int(w), "032b") for w in words)
    return [int(text[4 * i:4 * i + 4], 2) for i in range(n)]


def philox4x32_10(ctr, key):
    """Philox-4x32-10 (Salmon et al., SC'11) in Python integers."""
    m = 0xFFFFFFFF
    c = [x & m for x in ctr]
    k = [x & m for x in key]
    for rnd in range(10):
        if rnd:
            k = [(k[0] + 0x9E3779B9) & m, (k[1] + 0xBB67AE85) & m]
        p0 = 0xD2511F53 * c[0]
        p1 = 0xCD9E8D57 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k[0]) & m, p1 & m, ((p0 >> 32) ^ c[3] ^ k[1]) & m, p0 & m]
    return c


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised twin of philox4x32_10 over numpy uint64 arrays holding
    32-bit values; returns the four output words as uint64 arrays."""
    import numpy as _np

    m = _np.uint64(0xFFFFFFFF)
    c0, c1, c2, c3 = (_np.asarray(x, dtype=_np.uint64) & m for x in (c0, c1, c2, c3))
    k0 = _np.asarray(k0, dtype=_np.uint64) & m
    k1 = _np.asarray(k1, dtype=_np.uint64) & m
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _np.uint64(0x9E3779B9)) & m
            k1 = (k1 + _np.uint64(0xBB67AE85)) & m
        p0 = _np.uint64(0xD2511F53) * c0
        p1 = _np.uint64(0xCD9E8D57) * c2
        c0, c1, c2, c3 = ((p1 >> _np.uint64(32)) ^ c1 ^ k0, p1 & m,
                          (p0 >> _np.uint64(32)) ^ c3 ^ k1, p0 & m)
    return c0, c1, c2, c3
