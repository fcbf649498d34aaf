"""Writes rope_worked_example.txt: the rotary embedding of x = (1, 2, 3, 4) with D = 4 and
theta = 100 at positions 0, 1 and 10, worked with the standard library's cos and sin only
(no code of the oracle or of the library).

Pairs (x0, x1) and (x2, x3) have frequencies theta^(-0/4) = 1 and theta^(-2/4) = 0.1, so at
position p the first pair turns by p radians and the second by p/10 radians:
(a, b) -> (a cos t - b sin t, a sin t + b cos t).

    python tests/golden/make_rope_worked_example.py
"""
import math
import os

HEADER = """# Rotary position embedding, worked out for head width D = 4 and theta = 100.
# Source: LWM deep dive, section "Stage I：长上下文语言模型" and Tables 11 and 13 (RoPE with an
# enlarged base theta); the rotation itself is the textbook rotary embedding: pairs
# (x0, x1) and (x2, x3), frequencies theta^(-0/4) = 1 and theta^(-2/4) = 0.1, so a token at
# position p has its first pair turned by p radians and its second by p/10 radians.
# Values: cos and sin of 0, 1, 10 and 0.1 radians, combined as
#   (a cos t - b sin t, a sin t + b cos t) for each pair (a, b).
# Written by make_rope_worked_example.py (math.cos / math.sin only).
# input x = 1 2 3 4
# columns: position, y0, y1, y2, y3
"""


def turn(a, b, t):
    return a * math.cos(t) - b * math.sin(t), a * math.sin(t) + b * math.cos(t)


def rows():
    x = (1.0, 2.0, 3.0, 4.0)
    for p in (0, 1, 10):
        y0, y1 = turn(x[0], x[1], p * 1.0)
        y2, y3 = turn(x[2], x[3], p * 0.1)
        yield p, (y0, y1, y2, y3)


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_worked_example.txt")
    with open(out, "w") as f:
        f.write(HEADER)
        for p, ys in rows():
            f.write(f"{p} " + " ".join(repr(float(y)) for y in ys) + "\n")


if __name__ == "__main__":
    main()
