"""Writes e4m3fn_values.txt: every OCP E4M3FN code and its exact value, from the format
definition alone (sign bit, 4-bit exponent with bias 7, 3-bit mantissa, subnormals at
exponent 0, S.1111.111 = NaN, no infinities).  Imports nothing from the oracle or the
library, so the table is an independent pin for the oracle's fp8 decoder."""
import os
from fractions import Fraction


def main():
    lines = ["# OCP 8-bit floating point E4M3FN, every code and its exact value (or nan).",
             "# Written from the format definition: sign bit, 4-bit exponent with bias 7, 3-bit mantissa;",
             "# exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity.",
             "# Columns: code (hex), value as an exact fraction."]
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = "nan"
        else:
            mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            v = ("-" if s else "") + str(mag)
        lines.append(f"{c:02x} {v}")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e4m3fn_values.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
