"""Writes q4_1_blocks.json, q5_0_blocks.json and q5_1_blocks.json: hand-chosen ggml blocks (the
scale, minimum, high-bit word and nibble bytes below) and the value of each of their 32
elements, worked out by plain per-element loops from the block layouts. The loops follow the
layouts only; they import nothing from the oracle or the GPU path, so the oracle's reading of
these types is checked against an independent calculation. Every value is a small integer
times a power of two, so each can also be checked by eye.

Layouts (ggml, every field little-endian; the pages name none of these types, and page
'torad-labs/llama.cpp PR #71' serves the related q4_0):
  q4_1: fp16 d, fp16 m, 16 bytes (byte t: code t low nibble, code t + 16 high); d*code + m
  q5_0: fp16 d, 32-bit h, 16 bytes; code t = nibble + 16 * bit t of h; d*(code - 16)
  q5_1: fp16 d, fp16 m, 32-bit h, 16 bytes; code as q5_0; d*code + m
Run: python tests/golden/block_goldens.py
"""
import json
import os
import struct

HERE = os.path.dirname(os.path.abspath(__file__))
ORIGIN = ("the ggml {t} block; a ggml block type that the pages do not name; page "
          "'torad-labs/llama.cpp PR #71' serves q4_0")
ABOUT = {
    "q4_1": "q4_1 blocks written byte by byte ({o}): little-endian fp16 scale d, little-endian fp16 "
            "minimum m, then 16 bytes, byte t holding code t in its low nibble and code t + 16 in its "
            "high nibble. Expected values are d * code + m, listed element by element.",
    "q5_0": "q5_0 blocks written byte by byte ({o}): little-endian fp16 scale d, a little-endian "
            "32-bit word h, then 16 bytes of nibbles as in q4_0; element t's code is its nibble plus "
            "16 times bit t of h. Expected values are d * (code - 16), listed element by element.",
    "q5_1": "q5_1 blocks written byte by byte ({o}): little-endian fp16 scale d, little-endian fp16 "
            "minimum m, a little-endian 32-bit word h, then 16 bytes of nibbles; element t's code is "
            "its nibble plus 16 times bit t of h. Expected values are d * code + m, listed element "
            "by element.",
}


def f16(hexs):
    """The fp16 whose bits are the hex text (most significant byte first)."""
    return struct.unpack("<e", bytes.fromhex(hexs)[::-1])[0]


def le16(hexs):
    b = bytes.fromhex(hexs)
    return [b[1], b[0]]


def le32(h):
    return [h & 255, (h >> 8) & 255, (h >> 16) & 255, (h >> 24) & 255]


def nibble(qs, t):
    return (qs[t] & 15) if t < 16 else (qs[t - 16] >> 4)


def q4_1(dh, mh, qs):
    d, m = f16(dh), f16(mh)
    vals = [d * nibble(qs, t) + m for t in range(32)]
    return {"d_fp16_hex": dh, "d": d, "m_fp16_hex": mh, "m": m, "bytes": le16(dh) + le16(mh) + qs,
            "values": vals}


def q5(typ, dh, mh, h, qs):
    d = f16(dh)
    m = f16(mh) if mh else 0.0
    vals = []
    for t in range(32):
        code = nibble(qs, t) + 16 * ((h >> t) & 1)
        vals.append(d * (code - 16) if typ == "q5_0" else d * code + m)
    r = {"d_fp16_hex": dh, "d": d, "h": h, "bytes": le16(dh) + (le16(mh) if mh else []) + le32(h) + qs,
         "values": vals}
    if mh:
        r.update({"m_fp16_hex": mh, "m": m})
    return r


BLOCKS = {
    "q4_1": [q4_1("3c00", "0000", [t | ((15 - t) << 4) for t in range(16)]),
             q4_1("3800", "c000", [0x5A] * 16),
             q4_1("b400", "3e00", [((7 * t) % 16) | ((((3 * t) + 1) % 16) << 4) for t in range(16)])],
    "q5_0": [q5("q5_0", "3c00", None, 0, [t | (t << 4) for t in range(16)]),
             q5("q5_0", "3c00", None, 0xFFFFFFFF, [0] * 16),
             q5("q5_0", "3800", None, 0x0000FFFF, [(15 - t) | (t << 4) for t in range(16)]),
             q5("q5_0", "c000", None, 0xA5A5A5A5,
                [((5 * t) % 16) | (((11 * t + 3) % 16) << 4) for t in range(16)])],
    "q5_1": [q5("q5_1", "3c00", "0000", 0, [t | (t << 4) for t in range(16)]),
             q5("q5_1", "3400", "c400", 0xFFFF0000, [t | ((15 - t) << 4) for t in range(16)]),
             q5("q5_1", "b800", "4200", 0x12345678,
                [((9 * t + 2) % 16) | (((13 * t) % 16) << 4) for t in range(16)])],
}


def main():
    for t, blocks in BLOCKS.items():
        with open(os.path.join(HERE, f"{t}_blocks.json"), "w") as f:
            f.write("{\n  \"about\": " + json.dumps(ABOUT[t].format(o=ORIGIN.format(t=t))) + ",\n")
            f.write("  \"blocks\": [\n")
            f.write(",\n".join("    " + json.dumps(b) for b in blocks))
            f.write("\n  ]\n}\n")


if __name__ == "__main__":
    main()
