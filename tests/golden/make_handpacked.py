"""Write handpacked.json: hand-chosen field values of Q4_K / Q5_K / Q6_K / q8_0 blocks
and their packed bytes.

The byte layouts are the public GGUF block formats (the pages only name the
formats: Leone, "What ships": Q4_K and Q6_K weights; LeatEngine, Run: the q8_0
cache as llama.cpp keeps it).  The expected dequantized value of every weight is a
closed form of the fields, stated in each entry's "expect" and checked by
tests/test_oracle_pins.py.  Run from the repo root: python tests/golden/make_handpacked.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from refimpl import pack_q4k_block, pack_q5k_block, pack_q6k_block, pack_q8_0_block  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "handpacked.json")


def main():
    entries = {}
    # Q4_K block A: d=1, dmin=0.5, sc_j=j+1, m_j=2j, q_i=i%16 -> w_i=(j+1)(i%16)-j, j=i//32.
    sc = [j + 1 for j in range(8)]
    mn = [2 * j for j in range(8)]
    q = [i % 16 for i in range(256)]
    entries["q4k_a"] = dict(format="Q4_K", d=1.0, dmin=0.5, sc=sc, m=mn, q="i%16",
                            expect="w_i = (j+1)*(i%16) - j, j = i//32",
                            hex=pack_q4k_block(1.0, 0.5, sc, mn, q).hex())
    # Q4_K block B: every scale and min 63 (both top bits set), d=0.25, dmin=0.125, q_i=15-(i%16).
    q = [15 - (i % 16) for i in range(256)]
    entries["q4k_b"] = dict(format="Q4_K", d=0.25, dmin=0.125, sc=[63] * 8, m=[63] * 8, q="15-(i%16)",
                            expect="w_i = 0.25*63*(15-(i%16)) - 0.125*63",
                            hex=pack_q4k_block(0.25, 0.125, [63] * 8, [63] * 8, q).hex())
    # Q4_K block C: scales 32+j (top bit set only for j>=... all), mins 63-j, q_i=(i*7)%16, d=2, dmin=1.
    sc = [32 + j for j in range(8)]
    mn = [63 - j for j in range(8)]
    q = [(i * 7) % 16 for i in range(256)]
    entries["q4k_c"] = dict(format="Q4_K", d=2.0, dmin=1.0, sc=sc, m=mn, q="(7i)%16",
                            expect="w_i = 2*(32+j)*((7i)%16) - (63-j), j = i//32",
                            hex=pack_q4k_block(2.0, 1.0, sc, mn, q).hex())
    # Q6_K block A: d=1, scales alternate +1/-1 by sub-block of 16, q_i = i%64 -> w_i = +-(i%64 - 32).
    scales = [1 if s % 2 == 0 else -1 for s in range(16)]
    q = [i % 64 for i in range(256)]
    entries["q6k_a"] = dict(format="Q6_K", d=1.0, scales=scales, q="i%64",
                            expect="w_i = (+1 if (i//16) even else -1) * (i%64 - 32)",
                            hex=pack_q6k_block(1.0, scales, q).hex())
    # Q6_K block B: scale -128 everywhere, q=32 on even i (zero weight), 63 on odd i, d=0.5.
    q = [32 if i % 2 == 0 else 63 for i in range(256)]
    entries["q6k_b"] = dict(format="Q6_K", d=0.5, scales=[-128] * 16, q="32 (even i), 63 (odd i)",
                            expect="w_i = 0 (even i), 0.5*-128*31 (odd i)",
                            hex=pack_q6k_block(0.5, [-128] * 16, q).hex())
    # Q6_K block C: scales s-8 (s = sub-block), q_i = (5i+3)%64, d=0.125.
    scales = [s - 8 for s in range(16)]
    q = [(5 * i + 3) % 64 for i in range(256)]
    entries["q6k_c"] = dict(format="Q6_K", d=0.125, scales=scales, q="(5i+3)%64",
                            expect="w_i = 0.125*((i//16)-8)*((5i+3)%64 - 32)",
                            hex=pack_q6k_block(0.125, scales, q).hex())
    # q8_0: d=0.5 and codes -127..127 over 8 blocks (last padded with 0).
    codes = list(range(-127, 128)) + [0]
    hexes = [pack_q8_0_block(0.5, codes[32 * b:32 * b + 32]).hex() for b in range(8)]
    # Q5_K blocks: the Q4_K fields with five-bit quants (the fifth bits in their own bytes).
    sc = [j + 1 for j in range(8)]
    mn = [2 * j for j in range(8)]
    q = [i % 32 for i in range(256)]
    entries["q5k_a"] = dict(format="Q5_K", d=1.0, dmin=0.5, sc=sc, m=mn, q="i%32",
                            expect="w_i = (j+1)*(i%32) - j, j = i//32",
                            hex=pack_q5k_block(1.0, 0.5, sc, mn, q).hex())
    q = [31 - (i % 32) for i in range(256)]
    entries["q5k_b"] = dict(format="Q5_K", d=0.25, dmin=0.125, sc=[63] * 8, m=[63] * 8, q="31-(i%32)",
                            expect="w_i = 0.25*63*(31-(i%32)) - 0.125*63",
                            hex=pack_q5k_block(0.25, 0.125, [63] * 8, [63] * 8, q).hex())
    sc = [32 + j for j in range(8)]
    mn = [63 - j for j in range(8)]
    q = [(i * 7) % 32 for i in range(256)]
    entries["q5k_c"] = dict(format="Q5_K", d=2.0, dmin=1.0, sc=sc, m=mn, q="(7i)%32",
                            expect="w_i = 2*(32+j)*((7i)%32) - (63-j), j = i//32",
                            hex=pack_q5k_block(2.0, 1.0, sc, mn, q).hex())
    entries["q8_0_a"] = dict(format="q8_0", d=0.5, q="-127..127 then 0", expect="x = 0.5*q", hex="".join(hexes))
    with open(OUT, "w") as f:
        json.dump(entries, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
