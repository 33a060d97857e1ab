"""Writes worked_example.txt from its closed form (no oracle, no HIP path).

The example: scores {1, 0, -1}; dequantised V rows v2, v7, v9 as described in
the file header; out = (e*v2 + v7 + v9/e) / (1 + 2 cosh 1), lse = ln(1 + 2 cosh 1).
"""
import math
import os

HEADER = open(os.path.join(os.path.dirname(__file__), "worked_example.txt")).read().split("\nout =")[0] + "\n"


def main():
    e = math.e
    z = 1 + 2 * math.cosh(1)
    v2, v7, v9 = [0.5, 1, 1.5, 2], [5, 0, -5, 0], [-2, 2, -2, 2]
    out = [(e * a + b + c / e) / z for a, b, c in zip(v2, v7, v9)]
    body = "out = " + " ".join("%.17g" % v for v in out) + "\nlse = %.17g\n" % math.log(z)
    with open(os.path.join(os.path.dirname(__file__), "worked_example.txt"), "w") as f:
        f.write(HEADER + body)


if __name__ == "__main__":
    main()
