"""Writes softplus_threshold.txt: the softplus rule of the Megatron-Core API
docs, "core.ssm.ops.gdp.decode_prepare", entry "softplus" (log1p(exp(x)),
the identity once x is above 20), evaluated at a few points in 120-digit
decimal arithmetic, so that the fp64 oracle can be pinned to values that do
not come from any floating-point library.

    python tests/golden/make_softplus_threshold.py          # rewrites the file
    python tests/golden/make_softplus_threshold.py --check  # compares, exit 1 on a difference
"""
from __future__ import annotations

import decimal
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "softplus_threshold.txt")

HEADER = """\
# Source: Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare", entry
# "softplus". The page fixes the rule: log1p(exp(x)) in fp32, returning x itself
# once x is above 20 (torch's (x*beta) > threshold ? x : log1p(exp(x*beta))/beta
# at the default beta = 1), with log1p keeping the far-negative tail.
# Columns: x, softplus(x). Rows with x > 20 are the identity branch; the other
# rows are log(1 + e^x) evaluated to 25 significant digits (decimal arithmetic
# at 120 digits), so they are exact to far below fp64 resolution.
threshold 20
beta 1
"""

# (x as written in the file); the first two lie above the threshold
POINTS = ["20.5", "20.000001", "20.0", "19.0", "5.0", "0.0", "-20.0", "-100.0"]
THRESHOLD = decimal.Decimal(20)


def softplus_row(xs: str) -> str:
    x = decimal.Decimal(xs)
    if x > THRESHOLD:
        return f"{xs} {xs}"
    y = (decimal.Decimal(1) + x.exp()).ln()
    return f"{xs} {format(y, '.25e')}"


def render() -> str:
    with decimal.localcontext() as ctx:
        ctx.prec = 120
        return HEADER + "".join(softplus_row(p) + "\n" for p in POINTS)


def main() -> int:
    text = render()
    if "--check" in sys.argv[1:]:
        with open(OUT) as f:
            same = f.read() == text
        print("softplus_threshold.txt", "matches" if same else "DIFFERS")
        return 0 if same else 1
    with open(OUT, "w") as f:
        f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
