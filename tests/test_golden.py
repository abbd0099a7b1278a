"""The oracle against hand-worked values stored under tests/golden/ (each file
cites the passage its values come from).  CPU only."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_keyed(name):
    """`key: v1 v2 ...` lines (comments start with #) -> {key: float array}."""
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            key, vals = line.split(":", 1)
            out[key.strip()] = np.array([float(v) for v in vals.split()])
    return out


def test_each_strassen_product_of_the_worked_integer_example():
    g = load_keyed("strassen_2x2_integer.txt")
    A, B = g["A"].reshape(2, 2), g["B"].reshape(2, 2)
    d = oracle.strassen()
    assert d.rank == 7
    P = []
    for r in range(7):
        a = oracle.combine_block(A, d.U[r], 2, 2)
        b = oracle.combine_block(B, d.V[r], 2, 2)
        P.append(float((a @ b)[0, 0]))
        assert P[r] == g[f"P{r + 1}"][0], (r + 1, P[r])
    C = sum(d.W[r].astype(np.float64) * P[r] for r in range(7))
    assert C.tolist() == g["C"].tolist()
    Cl, n = oracle.lcma(A, B, d, 1)
    assert n == 7 and Cl.reshape(-1).tolist() == g["C"].tolist()
    assert oracle.gemm(A, B).reshape(-1).tolist() == g["C"].tolist()


def test_block_product_counts():
    rows = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "product_counts.txt"))
            if l.strip() and not l.startswith("#")]
    assert [r[0] for r in rows] == [1, 2]
    A = np.arange(1.0, 17.0).reshape(4, 4)
    B = np.arange(2.0, 18.0).reshape(4, 4)
    for levels, classic, strassen in rows:
        _, nc = oracle.lcma(A, B, oracle.naive(), levels)
        _, ns = oracle.lcma(A, B, oracle.strassen(), levels)
        assert (nc, ns) == (classic, strassen)
    assert oracle.strassen2().rank == rows[1][2]
    assert oracle.kron(oracle.naive(), oracle.naive()).rank == rows[1][1]


def test_binary16_operand_rounding_worked_example():
    g = load_keyed("binary16_operand_rounding.txt")
    A, B = g["A"].reshape(2, 2), g["B"].reshape(2, 2)
    C, _ = oracle.lcma(A, B, oracle.strassen(), 1, round_operands="f16")
    assert C.reshape(-1).tolist() == g["C_f16_operands"].tolist()
    Ce, _ = oracle.lcma(A, B, oracle.strassen(), 1)
    assert Ce.reshape(-1).tolist() == g["C_exact"].tolist()
