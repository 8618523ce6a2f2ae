"""Writes worked_example_1234.txt: closed forms of the two-block softmax example.

The comfyai.app chapter "6.3 FlashAttention", section 6.3.3, part "A Simple
Example", splits the vector [1, 2, 3, 4] into the blocks [1, 2] and [3, 4]
and computes the softmax block by block; its printed values did not survive
extraction.  This script writes the exact values of every quantity of that
example from closed forms, at 50 significant digits with Python's decimal
module.  It calls nothing in this repository (neither the oracle nor the HIP
path).

Quantities (d = running max, s = running denominator, O = running output with
V = identity so that O is the weight row; names follow the quidproquo.cc
guide's "Expand" boxes):

  after block 1:  d1 = 2,  s1 = 1 + e^-1,  O1 = (e^-1, 1, 0, 0) / s1
  after block 2:  d2 = 4,  s2 = 1 + e^-1 + e^-2 + e^-3,
                  O2_i = e^(i-4) / s2  (= softmax([1,2,3,4])),
                  correction factor (s1 / s2) e^(d1 - d2) = (1 + e^-1) e^-2 / s2
  LSE = 4 + ln(s2);  with scalar values v = (1, 2, 3, 4): sum_i i e^(i-4) / s2
  comfyai block statistics: m~1 = 2, l~1 = 1 + e^-1, m~2 = 4, l~2 = 1 + e^-1,
                  l_new = e^(2-4) l~1 + e^(4-4) l~2 (equals s2)
"""

from decimal import Decimal, getcontext
from pathlib import Path

getcontext().prec = 60


def e(x):
    return Decimal(x).exp()


def main():
    s1 = 1 + e(-1)
    s2 = 1 + e(-1) + e(-2) + e(-3)
    rows = [
        ("d1", [Decimal(2)]),
        ("s1", [s1]),
        ("O1", [e(-1) / s1, 1 / s1, Decimal(0), Decimal(0)]),
        ("d2", [Decimal(4)]),
        ("s2", [s2]),
        ("correction", [s1 / s2 * e(-2)]),
        ("O2", [e(i - 4) / s2 for i in (1, 2, 3, 4)]),
        ("LSE", [4 + s2.ln()]),
        ("O_scalar_v", [sum(Decimal(i) * e(i - 4) for i in (1, 2, 3, 4)) / s2]),
        ("block_m", [Decimal(2), Decimal(4)]),
        ("block_l", [1 + e(-1), 1 + e(-1)]),
        ("l_new", [e(-2) * (1 + e(-1)) + (1 + e(-1))]),
    ]
    lines = [
        "# Two-block softmax of [1, 2, 3, 4] split as [1, 2] | [3, 4].",
        "# Source: comfyai.app '6.3 FlashAttention', section 6.3.3, 'A Simple Example'",
        "# (values stripped on the page); recurrences of the quidproquo.cc guide's",
        "# 'Expand' boxes (slides 18-27). Closed forms written by make_worked_example.py.",
        "# name: values (50 significant digits)",
    ]
    for name, vals in rows:
        lines.append(name + ": " + " ".join(format(v, ".50g") for v in vals))
    Path(__file__).with_name("worked_example_1234.txt").write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
