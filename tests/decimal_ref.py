"""High-precision transcendental helpers for oracle pins.

They use Python's decimal module, whose exp() is computed to the working
precision by decimal's own algorithm, independent of the C math library the
oracle links.  Only tests import this file."""
from decimal import Decimal, getcontext

getcontext().prec = 50


def D(x) -> Decimal:
    return Decimal(float(x))


def dtanh(x: Decimal) -> Decimal:
    e = (2 * x).exp()
    return (e - 1) / (e + 1)


def dsigmoid(x: Decimal) -> Decimal:
    return 1 / (1 + (-x).exp())
