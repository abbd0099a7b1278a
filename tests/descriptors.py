"""Coefficient tables used as test descriptions (textbook, not from the pages).

Winograd's variant of Strassen's 2x2x2 scheme (rank 7), written out from its
formulas as flat U/V/W tables: blocks are numbered A11, A12, A21, A22 (i*2+k),
B11, B12, B21, B22 (k*2+j), C11, C12, C21, C22 (i*2+j).  With the shared
partial sums S1 = A21 + A22, S2 = S1 - A11, S3 = A11 - A21, S4 = A12 - S2 and
T1 = B12 - B11, T2 = B22 - T1, T3 = B22 - B12, T4 = T2 - B21 the products are
A11 B11, A12 B21, S4 B22, A22 T4, S1 T1, S2 T2, S3 T3, combined as
C11 = M1 + M2, C12 = M1 + M3 + M5 + M6, C21 = M1 - M4 + M6 + M7,
C22 = M1 + M5 + M6 + M7.
"""
import numpy as np

WINOGRAD_U = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [1, 1, -1, -1], [0, 0, 0, 1],
                       [0, 0, 1, 1], [-1, 0, 1, 1], [1, 0, -1, 0]], np.int8)
WINOGRAD_V = np.array([[1, 0, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1], [1, -1, -1, 1],
                       [-1, 1, 0, 0], [1, -1, 0, 1], [0, -1, 0, 1]], np.int8)
WINOGRAD_W = np.array([[1, 1, 1, 1], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, -1, 0],
                       [0, 1, 0, 1], [0, 1, 1, 1], [0, 0, 1, 1]], np.int8)


def equivalent(U, V, W, seed):
    """An equivalent description: products permuted and, per product, U and V
    negated independently (W takes both signs), which keeps Brent's
    identity."""
    U, V, W = (np.asarray(x, np.int64) for x in (U, V, W))
    rng = np.random.default_rng(seed)
    perm = rng.permutation(U.shape[0])
    su = rng.choice([-1, 1], U.shape[0])[:, None]
    sv = rng.choice([-1, 1], U.shape[0])[:, None]
    return ((U * su)[perm].astype(np.int8), (V * sv)[perm].astype(np.int8), (W * su * sv)[perm].astype(np.int8))
