"""Oracle: the two-stage split-K reduction (test infrastructure only).

Follows Event Tensor notes, section "Split-K reduction 示例": an input A of
shape (n*32, 128) is summed along K in four 32-wide slices by first-stage
tasks, then the four partials of each row are summed by second-stage tasks.
Task (i, j) of the first stage covers the 32-row block i and K-slice j and
notifies event E[i]; E has shape (n,) and every element starts at 4.

Reading taken where the page is loose: the page's formula indexes B by row
while its prose says one event per 32 rows; task (i, j) therefore covers rows
32*i .. 32*i+31 (row block i), and B/C are indexed by row.

Pins (tests/test_oracle_splitk.py): the closed form C[r] = sum_k A[r, k]
checked against math.fsum (a correctly rounded sum), integer-valued A (exact),
A == 1 (B == 32, C == 128), and the page's event table re-derived by brute
force enumeration of the producer map.
"""

import numpy as np

SLICES = 4          # K-slices per row (j in [0, 4))
SLICE_W = 32        # width of one K-slice
ROWS_PER_BLOCK = 32  # rows per first-stage task / per event


def stage1(A):
    """B[r, j] = sum_{k=32j}^{32j+31} A[r, k]  (Event Tensor notes, split-K example,
    first-stage formula).  A: (rows, 128) float array. Returns float64 (rows, 4)."""
    A = np.asarray(A, dtype=np.float64)
    rows, cols = A.shape
    if cols != SLICES * SLICE_W:
        raise ValueError("split-K example has 128 columns")
    B = np.zeros((rows, SLICES), dtype=np.float64)
    for j in range(SLICES):
        B[:, j] = A[:, SLICE_W * j:SLICE_W * (j + 1)].sum(axis=1)
    return B


def stage2(B):
    """C[r] = sum_{j=0}^{3} B[r, j]  (same section, second-stage formula)."""
    B = np.asarray(B, dtype=np.float64)
    C = np.zeros(B.shape[0], dtype=np.float64)
    for j in range(SLICES):
        C += B[:, j]
    return C


def splitk_reduce(A):
    """Both stages. Returns (B, C) in float64."""
    B = stage1(A)
    return B, stage2(B)
