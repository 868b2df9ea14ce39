"""Writes pack_vectors.json: expected int32 words for hand-chosen code vectors.

Derivation, independent of the oracle's packing loop: a row's packed words are
one little-endian stream of b-bit fields (column i at bits [b*i, b*i+b)), so the
stream of 32 codes read as an integer is the base-2^b numeral whose digits, least
significant first, are the codes.  For b = 3 that numeral is octal.  The words are
its 32-bit limbs, least significant first.
"""
import json
import os


def limbs(v, nbits):
    return [((v >> (32 * k)) & 0xFFFFFFFF) for k in range(nbits // 32)]


def s32(x):
    return x - (1 << 32) if x >= (1 << 31) else x


def main():
    out = {"_about": "Packing vectors for the stated bit layout (a row's codes form a "
                     "little-endian stream, column i at bits [b*i, b*i+b)). Expected words "
                     "derived by reading the stream as a base-2^b numeral (for b=3: base 8), "
                     "independently of the oracle's loop. int32 values as stored.",
           "cases": []}
    n = 32
    for bits in (4, 3, 2, 8):
        maxq = (1 << bits) - 1
        ramp = [i % (1 << bits) for i in range(n)]
        numeral = 0
        for c in reversed(ramp):           # most significant digit first
            numeral = numeral * (1 << bits) + c
        out["cases"].append({"bits": bits, "name": "ramp", "codes": ramp,
                             "words": [s32(w) for w in limbs(numeral, n * bits)]})
        out["cases"].append({"bits": bits, "name": "zeros", "codes": [0] * n,
                             "words": [0] * (n * bits // 32)})
        out["cases"].append({"bits": bits, "name": "all_maxq", "codes": [maxq] * n,
                             "words": [-1] * (n * bits // 32)})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pack_vectors.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
