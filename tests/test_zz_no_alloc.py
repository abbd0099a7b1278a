"""The allocation-free entry point (lcma_gemm_noalloc: the workspace is the
library's static device scratch array) against lcma_gemm with a workspace
from torch: bitwise equal, on two calls in a row, the second smaller (so it
runs on the scratch contents the first call left), for every plan kind that
uses a workspace; plans whose workspace exceeds the array are refused."""
import numpy as np
import pytest
import torch

import complexity_half_precision_amd as L
import seeded_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, first shape, second (smaller) shape, dtype, plan options
    ("classic padded", (1000, 1064, 2050), (257, 13, 64), "bf16", dict(force="classic")),
    ("l1 prepass", (2048, 2048, 2048), (1024, 768, 512), "bf16", dict(force="l1", combine="prepass")),
    ("l1 at load, split", (2560, 2560, 1024), (1024, 1024, 512), "bf16",
     dict(force="l1", combine="at_load", split="all")),
    ("l2", (1024, 1024, 1024), (512, 512, 512), "bf16", dict(force="l2")),
    ("l1 unfused", (1024, 1024, 1024), (512, 512, 256), "f16", dict(force="l1", combine="unfused")),
    ("l1 padded", (1000, 1032, 520), (333, 250, 210), "f16", dict(force="l1")),
    ("classic, K split", (64, 4096, 14336), (40, 4104, 8200), "bf16", dict(force="classic")),
    ("classic, K split, 32-row tiles", (1, 1024, 14336), (16, 2056, 8192), "bf16", dict(force="classic")),
    ("classic, K split, 128 x 128 tiles", (4096, 256, 8192), (1024, 1024, 8192), "bf16", dict(force="classic")),
    ("classic, tail round K split", (4104, 4104, 4104), (2304, 7424, 4096), "bf16", dict(force="classic")),
]


def run(shape, dtype, opts, seed, noalloc):
    M, N, K = shape
    A, B = si.gen(M, N, K, dtype, "uniform" if dtype == "f16" else "normal_sqrtk", seed)
    Ad, Bd = A.to(DEV), B.to(DEV)
    plan = L.lcma_plan_ex(M, N, K, dtype, **opts)
    ws_bytes = L.lcma_plan_info(plan)[1]
    assert 0 < ws_bytes <= L.SCRATCH_BYTES
    C = torch.full((M, N), 3.0, dtype=si.TORCH_DT[dtype], device=DEV)
    if noalloc:
        L.lcma_gemm_noalloc(plan, Ad, Bd, C)
    else:
        L.lcma_gemm(plan, Ad, Bd, C, L.workspace_for(plan))
    torch.cuda.synchronize()
    return si.bits(C)


@pytest.mark.parametrize("name,big,small,dtype,opts", CASES)
def test_noalloc_equals_lcma_gemm_on_two_calls(name, big, small, dtype, opts):
    print("[case] noalloc", name, big, small, flush=True)
    want = [run(s, dtype, opts, 50 + i, noalloc=False) for i, s in enumerate((big, small))]
    got = [run(s, dtype, opts, 50 + i, noalloc=True) for i, s in enumerate((big, small))]
    for w, g in zip(want, got):
        assert np.array_equal(w, g), name


def test_noalloc_refuses_a_workspace_beyond_the_scratch_array():
    print("[case] noalloc refuses", flush=True)
    n = 8192
    plan = L.lcma_plan_ex(n, n, n, "bf16", force="l1", combine="prepass")
    assert L.lcma_plan_info(plan)[1] > L.SCRATCH_BYTES
    A = torch.empty((n, n), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.LcmaError) as e:
        L.lcma_gemm_noalloc(plan, A, A, A)
    assert e.value.status == L.E_WORKSPACE
