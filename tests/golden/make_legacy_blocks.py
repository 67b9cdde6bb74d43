"""Writes q4_0_block.txt and q5_0_block.txt: hand-built Q4_0 (18 bytes) and
Q5_0 (22 bytes) blocks.

The pages name these types only as GGUF types beyond the three with dedicated
kernels (blazr README, "Model Formats > GGUF"); the bytes follow GGUF's
published layouts and are packed here field by field with explicit loops,
independently of the input generator's packers and of the oracle's decoders,
so that both are checked against them.  Every decoded value is an exact
dyadic rational: w[i] = d*(q[i] - 8) for Q4_0, d*(q[i] - 16) for Q5_0.
"""
import os

import numpy as np

Q4_D_BITS = 0xB000    # d = -2^-3: a negative scale
Q5_D_BITS = 0x2800    # d = 2^-5
Q4 = [0, 15] + [int(v) for v in np.random.default_rng(404).integers(0, 16, 30)]   # both ends of the range
Q5 = [0, 31, 16, 15] + [int(v) for v in np.random.default_rng(505).integers(0, 32, 28)]


def pack_q4_0():
    b = bytearray(18)
    b[0], b[1] = Q4_D_BITS & 0xFF, Q4_D_BITS >> 8
    for j in range(16):                      # byte 2 + j: element j low, element 16 + j high
        b[2 + j] = (Q4[j] & 15) | ((Q4[16 + j] & 15) << 4)
    return bytes(b)


def pack_q5_0():
    b = bytearray(22)
    b[0], b[1] = Q5_D_BITS & 0xFF, Q5_D_BITS >> 8
    for i in range(32):                      # bit i of the little-endian word at bytes 2..5
        if Q5[i] & 16:
            b[2 + i // 8] |= 1 << (i % 8)
    for j in range(16):
        b[6 + j] = (Q5[j] & 15) | ((Q5[16 + j] & 15) << 4)
    return bytes(b)


def write(name, header, d_bits, q, data):
    lines = [f"# Hand-built {name} block ({len(data)} bytes), written by make_legacy_blocks.py.", "#",
             "# The pages give no example of this type (blazr README, \"Model Formats > GGUF\",",
             "# names the GGUF types only).  GGUF's published layout:"] + header + [
        f"d_bits: 0x{d_bits:04X}",
        "q: " + " ".join(map(str, q)),
        "bytes:",
        data.hex(),
    ]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{name.lower()}_block.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    write("Q4_0", ["#   bytes 0-1 d = -2^-3 (0xB000)",
                   "#   bytes 2-17 qs: byte 2+j holds code q[j] (low nibble) and q[16+j] (high nibble)",
                   "# Expected element values (closed form): w[i] = d*(q[i] - 8)."],
          Q4_D_BITS, Q4, pack_q4_0())
    write("Q5_0", ["#   bytes 0-1 d = 2^-5 (0x2800)",
                   "#   bytes 2-5 qh: bit i of this little-endian 32-bit word is bit 4 of q[i]",
                   "#   bytes 6-21 qs: byte 6+j holds the low four bits of q[j] (low nibble) and",
                   "#              of q[16+j] (high nibble)",
                   "# Expected element values (closed form): w[i] = d*(q[i] - 16)."],
          Q5_D_BITS, Q5, pack_q5_0())


if __name__ == "__main__":
    main()
