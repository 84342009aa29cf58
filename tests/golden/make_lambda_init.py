"""Writes lambda_init.json: the depth schedule of lambda's starting value as
the pages print it (lambda_init = 0.8 - 0.6 exp(-0.3 (l - 1)), layer l >= 1;
Ultralytics glossary "Differential Transformer", section "How differential
attention works"; esgcw.com.cn write-up, differential attention section),
evaluated at the layers the workloads use with 40-digit decimal arithmetic
(exp from its Taylor series), independently of the oracle and of floating
point.  Run: python tests/golden/make_lambda_init.py"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 40


def dexp(x: Decimal) -> Decimal:
    term, total, n = Decimal(1), Decimal(1), 1
    while True:
        term = term * x / n
        if abs(term) < Decimal(10) ** -45:
            return total
        total += term
        n += 1


def main():
    layers = [1, 2, 12, 24]
    vals = {str(l): str(Decimal("0.8") - Decimal("0.6") * dexp(Decimal("-0.3") * (l - 1))) for l in layers}
    rec = {
        "citation": "Ultralytics glossary 'Differential Transformer' (Korean and Russian editions), section 'How "
                    "differential attention works', and the esgcw.com.cn write-up, differential attention section: "
                    "lambda_init = 0.8 - 0.6 exp(-0.3 (l - 1)) for layer l >= 1",
        "method": "40-digit decimal arithmetic, exp by its Taylor series (tests/golden/make_lambda_init.py)",
        "lambda_init": vals,
        "gap_ratio_exp_minus_0.3": str(dexp(Decimal("-0.3"))),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lambda_init.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
