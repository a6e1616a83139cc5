"""GPU parity of online_softmax_rows (through the C ABI) against the float64 oracle.

Gate: max |y_gpu - y_oracle| <= 1e-5 on every element compared.  Bitwise identities
where the arithmetic is exact: all-equal rows give exactly 1/cols when cols is a power
of two, one-column rows give exactly 1.
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import TOL_F32, max_abs, max_rel, need_gpu, say

pytestmark = pytest.mark.gpu


def _oracle_err(x_cpu, y_cpu, chunk=8192):
    """max abs and max rel (floor 1e-6) error, the oracle evaluated chunk by chunk."""
    xa, ya = x_cpu.numpy(), y_cpu.numpy()
    ea, er = 0.0, 0.0
    for r0 in range(0, xa.shape[0], chunk):
        ref, _, _ = oracle.softmax_rows(xa[r0:r0 + chunk])
        ea = max(ea, max_abs(ya[r0:r0 + chunk], ref))
        er = max(er, max_rel(ya[r0:r0 + chunk], ref, 1e-6))
    return ea, er


def _run(x_cpu, dev):
    y = osm.online_softmax_rows(x_cpu.to(dev))
    torch.cuda.synchronize()
    return y.cpu()


@pytest.mark.parametrize("name", ["softmax_f32_65536x4096", "softmax_f32_65536x4095"])
def test_full_size_workloads(name):
    dev = need_gpu()
    x, sp = workloads.softmax_inputs_for(name)
    say(f"case {name}: rows={x.shape[0]} cols={x.shape[1]}")
    y = _run(x, dev)
    ea, er = _oracle_err(x, y)
    say(f"  max abs err {ea:.3e}  max rel err {er:.3e}")
    assert ea <= TOL_F32
    cols = x.shape[1]
    ae = torch.from_numpy(sp["all_equal"])
    if cols & (cols - 1) == 0:
        assert torch.all(y[ae] == 1.0 / cols)  # exact: exp(0) = 1 and l = cols
    assert torch.all(torch.isfinite(y))


def test_one_column_rows_are_exactly_one():
    dev = need_gpu()
    x, _ = workloads.softmax_inputs_for("softmax_f32_65536x1")
    say("case softmax_f32_65536x1")
    y = _run(x, dev)
    assert torch.all(y == 1.0)


# Every kernel variant: short rows (lane groups), one wavefront per row, four and eight
# wavefronts per row (LDS merge; eight from 769 to 1024 16-byte units, e.g. 3076-4096
# columns), streaming; 16-byte, head-form and 4-byte paths.
COLS = [1, 2, 3, 5, 16, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 1000, 1020, 1023, 1024, 1025,
        1028, 2048, 3072, 3073, 3076, 4095, 4096, 4097, 8192, 12000, 16383, 16384, 16385, 40000, 65536]


@pytest.mark.parametrize("cols", COLS)
def test_shapes(cols):
    dev = need_gpu()
    rows = 37
    x, _ = workloads.softmax_inputs(rows, cols, seed=workloads.SEED_BASE + 4000 + cols,
                                    special_frac=0.1)
    say(f"case rows={rows} cols={cols}")
    y = _run(x, dev)
    ea, _ = _oracle_err(x, y)
    assert ea <= TOL_F32, ea


def test_longest_rows():
    dev = need_gpu()
    cols = 1 << 20
    x, _ = workloads.softmax_inputs(3, cols, seed=workloads.SEED_BASE + 4100)
    say(f"case rows=3 cols={cols}")
    y = _run(x, dev)
    ea, _ = _oracle_err(x, y)
    assert ea <= TOL_F32, ea


def test_in_place():
    dev = need_gpu()
    x, _ = workloads.softmax_inputs(500, 4096, seed=workloads.SEED_BASE + 4200)
    say("case in place 500 x 4096")
    xd = x.to(dev)
    out = osm.online_softmax_rows(xd, out=xd)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr()
    ea, _ = _oracle_err(x, xd.cpu())
    assert ea <= TOL_F32


# Rows off the 16-byte grid.  x and y at the same 16-byte phase (equal offsets) take the
# head form (16-byte units from each row's first boundary, up to three elements on either
# side one by one); different phases take 4-byte units; rows past the register forms
# stream in 4-byte units.
@pytest.mark.parametrize("cols,x_off,y_off", [
    (4096, 1, 1), (1000, 1, 1), (7, 1, 1), (33, 2, 2), (35, 2, 2), (1023, 3, 3), (4095, 0, 0),
    (4095, 1, 1), (4097, 2, 2), (4095, 1, 2), (1000, 0, 3), (40001, 1, 1), (40000, 1, 3)])
def test_unaligned_rows(cols, x_off, y_off):
    dev = need_gpu()
    rows = 64
    x, _ = workloads.softmax_inputs(rows, cols, seed=workloads.SEED_BASE + 4300 + cols)
    say(f"case unaligned rows={rows} cols={cols} x_off={x_off} y_off={y_off}")
    buf = torch.empty(rows * cols + x_off, dtype=torch.float32, device=dev)
    xd = buf[x_off:].view(rows, cols)
    xd.copy_(x.to(dev))
    obuf = torch.empty(rows * cols + y_off, dtype=torch.float32, device=dev)
    yd = obuf[y_off:].view(rows, cols)
    osm.online_softmax_rows(xd, out=yd)
    torch.cuda.synchronize()
    ea, _ = _oracle_err(x, yd.cpu())
    assert ea <= TOL_F32


def test_in_place_unaligned():
    dev = need_gpu()
    rows, cols = 300, 4095
    x, _ = workloads.softmax_inputs(rows, cols, seed=workloads.SEED_BASE + 4250)
    say("case in place, unaligned 300 x 4095 at offset 1")
    buf = torch.empty(rows * cols + 1, dtype=torch.float32, device=dev)
    xd = buf[1:].view(rows, cols)
    xd.copy_(x.to(dev))
    out = osm.online_softmax_rows(xd, out=xd)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr()
    ea, _ = _oracle_err(x, xd.cpu())
    assert ea <= TOL_F32


def test_empty_batch():
    dev = need_gpu()
    x = torch.empty((0, 128), dtype=torch.float32, device=dev)
    y = osm.online_softmax_rows(x)
    assert y.shape == (0, 128)


def test_repeat_runs_bitwise_identical():
    dev = need_gpu()
    x, _ = workloads.softmax_inputs(2048, 4096, seed=workloads.SEED_BASE + 4400)
    say("case determinism 2048 x 4096")
    xd = x.to(dev)
    a = osm.online_softmax_rows(xd)
    b = osm.online_softmax_rows(xd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# Masked entries (-inf) in every kernel variant: lane groups, one, four and eight
# wavefronts per row, the head form (rows off the 16-byte grid) and the streaming form.
@pytest.mark.parametrize("cols", [5, 33, 1000, 3072, 4095, 4096, 20000])
def test_masked_rows(cols):
    dev = need_gpu()
    rows = 40
    x, _ = workloads.softmax_inputs(rows, cols, seed=workloads.SEED_BASE + 4500 + cols, special_frac=0.0)
    xa = x.numpy().copy()
    g = np.random.default_rng(workloads.SEED_BASE + 4600 + cols)
    mask = g.random(size=xa.shape) < 0.5
    mask[:, g.integers(cols)] = False  # every row keeps a finite entry ...
    one = int(g.integers(cols))
    mask[0, :] = True
    mask[0, one] = False               # ... row 0 exactly one
    mask[1, : cols // 2] = True        # row 1: the first half masked
    mask[2, :] = True                  # row 2: nothing finite
    mask[3, :-1] = True
    mask[3, -1] = False                # row 3: only the last entry
    xa[mask] = -np.inf
    say(f"case masked rows={rows} cols={cols}")
    y = _run(torch.from_numpy(xa), dev).numpy()
    assert np.all(np.isnan(y[2])), "a row of -inf only has normaliser 0"
    live = np.ones(rows, dtype=bool)
    live[2] = False
    assert np.all(y[live][mask[live]] == 0.0)
    assert y[0, one] == 1.0 and y[3, -1] == 1.0
    ref, _, _ = oracle.softmax_rows(xa[live])
    assert max_abs(y[live], ref) <= TOL_F32
