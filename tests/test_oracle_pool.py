"""The slab-parallel runner of the oracle's encoder gives exactly the
whole-matrix result: slab boundaries fall on second-level group boundaries, so
every block and group is computed from the same elements (CPU)."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pool
import workloads as WL


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(300, 1088), (64, 11008 // 43 * 4), (33, 22016 // 43 * 2), (40, 512)])
def test_slabs_equal_whole_matrix(rows, cols):
    W = WL.weight_student_t(rows, cols, 0.02, 5, rows * 7 + cols)
    Wf = W.float().numpy()
    codes, absmax = O.nf4_quantize(Wf)
    c2, c1 = O.nf4_double_quant(absmax)
    Wq = O.nf4_dequantize(codes, c2, c1, rows, cols)
    for src in (_bits(W), Wf):
        pc, pa, p2, p1, pq = oracle_pool.quantize(src, workers=3)
        assert np.array_equal(pc, codes) and np.array_equal(p2, c2) and np.array_equal(pq, Wq)
        assert np.array_equal(pa.view(np.uint32), absmax.view(np.uint32))
        assert np.array_equal(p1.view(np.uint32), c1.view(np.uint32))


def test_slab_bounds_are_group_aligned():
    for rows, cols in ((8192, 8192), (22016, 8192), (8192, 22016), (11008, 4096), (4096, 11008), (257, 64)):
        b = oracle_pool.slab_rows(rows, cols, 32)
        assert b[0][0] == 0 and b[-1][1] == rows
        assert all(x[1] == y[0] for x, y in zip(b[:-1], b[1:]))
        assert all((a * cols) % oracle_pool.GROUP_ELEMS == 0 for a, _ in b)
        assert len(b) <= 32
