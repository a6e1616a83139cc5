"""GPU parity of fused_add_rmsnorm / fused_add_layernorm (through the C ABI) against the
float64 oracle (oracle.norms).

Gate (bf16 output, float32 statistics): every output element within one bf16 rounding of
the float64 value plus a small float32 allowance, |y - y_ref| <= 2^-8 |y_ref| + 2e-3.  The
residual output h is a single rounding of the exact sum x + residual to bf16: it must be
within one bf16 unit in the last place of the exact sum everywhere, and equal to the
correctly rounded sum for all but a vanishing share of elements (float32 can round the sum
once before the bf16 rounding when the two addends differ by more than 2^16).
"""

import numpy as np
import pytest
import torch

import online_softmax_09_amd as osm
import oracle
import workloads
from parity import need_gpu, say

pytestmark = pytest.mark.gpu


def _bf16_round(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).float().numpy()


def _check(tag, y, h, y_ref, h_ref):
    y_err = np.abs(y - y_ref) - (2.0 ** -8 * np.abs(y_ref) + 2e-3)
    h_round = _bf16_round(h_ref)          # float64 -> bf16: one rounding of the exact sum
    ulp = np.abs(np.spacing(h_round.astype(np.float32)).astype(np.float64)) * 65536.0  # bf16 ulp
    h_dev = np.abs(h - h_ref.astype(np.float64))
    exact = float(np.mean(h == h_round))
    say(f"  {tag}: y max excess {y_err.max():.3e}  max |y-y_ref| {np.abs(y - y_ref).max():.3e}  "
        f"h exact share {exact:.6f}")
    return y_err.max() <= 0.0 and np.all(h_dev <= ulp) and exact >= 0.9999


@pytest.mark.parametrize("layer", [False, True])
# 16-byte rows take 128 threads up to 256 units (2048 columns) and 512 above (2056: 257
# units, one per thread, the other 255 threads idle); 2-byte rows (1000, 4095, 24, 1) take 256.
@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 64), (7, 1000), (4, 2048), (4, 2056), (5, 4096), (2, 8192),
                                       (3, 32768), (4, 4095), (9, 1), (2, 24)])
def test_norm_shapes(layer, rows, cols):
    dev = need_gpu()
    say(f"case norm layer={layer} rows={rows} cols={cols}")
    x, r, g, b, _ = workloads.norm_inputs(rows, cols, seed=workloads.SEED_BASE + 9700 + cols, special_frac=0.0)
    if layer:
        y, h = osm.fused_add_layernorm(x.to(dev), r.to(dev), g.to(dev), b.to(dev), eps=1e-5)
        y_ref, h_ref = oracle.layer_norm(x, g, b, 1e-5, residual=r)
    else:
        y, h = osm.fused_add_rmsnorm(x.to(dev), r.to(dev), g.to(dev), eps=1e-5)
        y_ref, h_ref = oracle.rms_norm(x, g, 1e-5, residual=r)
    torch.cuda.synchronize()
    assert _check("shape", y.float().cpu().numpy(), h.float().cpu().numpy(), y_ref, h_ref)


@pytest.mark.parametrize("layer", [False, True])
def test_norm_workload(layer):
    """The 16384 x 8192 workload with its constant rows and +1000 rows."""
    dev = need_gpu()
    c = workloads.CONFIGS["norm_bf16_16384x8192"]
    say(f"case norm workload layer={layer}")
    x, r, g, b, sp = workloads.norm_inputs(c["rows"], c["cols"], c["seed"])
    xd, rd, gd, bd = (t.to(dev) for t in (x, r, g, b))
    if layer:
        y, h = osm.fused_add_layernorm(xd, rd, gd, bd, eps=c["eps"])
    else:
        y, h = osm.fused_add_rmsnorm(xd, rd, gd, eps=c["eps"])
    torch.cuda.synchronize()
    y, h = y.float().cpu().numpy(), h.float().cpu().numpy()
    check_rows = np.unique(np.concatenate([np.arange(0, c["rows"], 97), sp["constant"][:50], sp["plus1000"][:50]]))
    xs, rs = x[check_rows], r[check_rows]
    if layer:
        y_ref, h_ref = oracle.layer_norm(xs, g, b, c["eps"], residual=rs)
    else:
        y_ref, h_ref = oracle.rms_norm(xs, g, c["eps"], residual=rs)
    assert _check("workload", y[check_rows], h[check_rows], y_ref, h_ref)
    if layer:
        # constant rows: (h - mean) = 0 exactly, so y = beta rounded to bf16
        cr = sp["constant"]
        assert np.array_equal(y[cr], np.broadcast_to(b.float().numpy(), (len(cr), c["cols"])))


def test_norm_without_residual_and_in_place():
    dev = need_gpu()
    x, r, g, b, _ = workloads.norm_inputs(6, 2048, seed=workloads.SEED_BASE + 9800, special_frac=0.0)
    xd = x.to(dev)
    y, h = osm.fused_add_layernorm(xd, None, g.to(dev), b.to(dev), eps=1e-5)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.layer_norm(x, g, b, 1e-5)
    assert _check("no residual", y.float().cpu().numpy(), h.float().cpu().numpy(), y_ref, h_ref)
    # in place: y over x, h over residual
    xd, rd = x.to(dev), r.to(dev)
    osm.fused_add_rmsnorm(xd, rd, g.to(dev), eps=1e-5, out=xd, residual_out=rd)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.rms_norm(x, g, 1e-5, residual=r)
    assert _check("in place", xd.float().cpu().numpy(), rd.float().cpu().numpy(), y_ref, h_ref)


def test_norm_deterministic():
    dev = need_gpu()
    x, r, g, b, _ = workloads.norm_inputs(64, 8192, seed=workloads.SEED_BASE + 9900)
    a = osm.fused_add_layernorm(x.to(dev), r.to(dev), g.to(dev), b.to(dev))
    c = osm.fused_add_layernorm(x.to(dev), r.to(dev), g.to(dev), b.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
