"""Coefficients of exp2_neg's polynomial (sv_device.hpp), for the record.

exp2_neg writes 2^t = 2^n * 2^f with n = rint(t) and |f| <= 1/2, and
evaluates 2^f = 1 + f * q(f), where q is the degree-8 polynomial that
interpolates (2^f - 1) / f at the nine Chebyshev nodes of [-1/2, 1/2] (taken
as the doubles nearest to 0.5 cos((2k + 1) pi / 18)).  The constant term
stays exactly 1, so 2^0 == 1.  The interpolation is solved in 60-digit
decimal arithmetic, with 2^x = exp(x ln 2) to that precision; each
coefficient is then rounded to the nearest double.  Prints the C++ lines.
"""
import math
from decimal import Decimal, getcontext

getcontext().prec = 60
LN2 = Decimal(2).ln()
DEG = 8
nodes = [Decimal(0.5 * math.cos((2 * k + 1) * math.pi / (2 * (DEG + 1)))) for k in range(DEG + 1)]
values = [((x * LN2).exp() - 1) / x if x != 0 else LN2 for x in nodes]
# Vandermonde system, Gaussian elimination with partial pivoting in Decimal
A = [[x ** j for j in range(DEG + 1)] + [y] for x, y in zip(nodes, values)]
n = DEG + 1
for col in range(n):
    piv = max(range(col, n), key=lambda r: abs(A[r][col]))
    A[col], A[piv] = A[piv], A[col]
    for r in range(n):
        if r != col:
            f = A[r][col] / A[col][col]
            A[r] = [a - f * b for a, b in zip(A[r], A[col])]
coef = [A[i][n] / A[i][i] for i in range(n)]
for j in reversed(range(n)):
    print(f"  q{j} = {float(coef[j]).hex()}  # {float(coef[j]):.17g}")
