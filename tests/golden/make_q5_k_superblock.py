"""Writes q5_k_superblock.txt: a hand-built Q5_K superblock (176 bytes).

The pages name the Q5_K type only (blazr README, "Model Formats > GGUF");
the bytes follow GGUF's published Q5_K layout and are packed here field by
field with explicit loops, independently of the input generator's packer and
of the oracle's decoder, so that both are checked against it.  Every decoded
value is an exact dyadic rational: w[i] = d*sc[i//32]*q[i] - dmin*m[i//32].
"""
import os

import numpy as np

D_BITS, DMIN_BITS = 0x2C00, 0x2800          # d = 2^-4, dmin = 2^-5
SC = [1, 17, 33, 63, 5, 21, 47, 60]          # six-bit scales (top bits exercised)
M = [0, 16, 32, 48, 63, 20, 40, 9]           # six-bit mins
Q = [int(v) for v in np.random.default_rng(505).integers(0, 32, 256)]  # 5-bit codes, no period structure


def pack():
    b = bytearray(176)
    b[0], b[1] = D_BITS & 0xFF, D_BITS >> 8
    b[2], b[3] = DMIN_BITS & 0xFF, DMIN_BITS >> 8
    for j in range(4):
        b[4 + j] = (SC[j] & 63) | ((SC[j + 4] >> 4) << 6)
        b[8 + j] = (M[j] & 63) | ((M[j + 4] >> 4) << 6)
        b[12 + j] = (SC[j + 4] & 15) | ((M[j + 4] & 15) << 4)
    for l in range(32):                      # qh[l]: bit j = fifth bit of element 32j + l
        v = 0
        for j in range(8):
            v |= ((Q[32 * j + l] >> 4) & 1) << j
        b[16 + l] = v
    for g in range(4):                       # qs[32g + l]: low nibble element 64g + l, high 64g + 32 + l
        for l in range(32):
            b[48 + 32 * g + l] = (Q[64 * g + l] & 15) | ((Q[64 * g + 32 + l] & 15) << 4)
    return bytes(b)


def main():
    hexs = pack().hex()
    lines = [
        "# Hand-built Q5_K superblock (176 bytes), written by make_q5_k_superblock.py.",
        "#",
        "# The pages give no Q5_K example (blazr README, \"Model Formats > GGUF\", names",
        "# the types only).  GGUF's published Q5_K layout:",
        "#   bytes 0-1 d = 2^-4 (0x2C00), bytes 2-3 dmin = 2^-5 (0x2800)",
        "#   bytes 4-15 six-bit sc[8] and m[8], packed as in Q4_K",
        "#   bytes 16-47 qh: bit j of byte 16+l is the fifth bit of code q[32j+l]",
        "#   bytes 48-175 qs: byte 48+32g+l holds the low four bits of q[64g+l] (low",
        "#              nibble) and of q[64g+32+l] (high nibble)",
        "# Expected element values (closed form): w[i] = d*sc[i//32]*q[i] - dmin*m[i//32].",
        f"d_bits: 0x{D_BITS:04X}",
        f"dmin_bits: 0x{DMIN_BITS:04X}",
        "sc: " + " ".join(map(str, SC)),
        "m: " + " ".join(map(str, M)),
        "q: " + " ".join(map(str, Q)),
        "bytes:",
    ] + [hexs[i:i + 64] for i in range(0, len(hexs), 64)]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "q5_k_superblock.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
