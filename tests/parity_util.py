"""Feature checks shared by the GPU parity tests.

The oracle's sums are taken over every requested row, in row chunks on the host's threads (each
chunk is one call of the oracle, so the arithmetic of a row does not depend on the split).
Three figures are reported for every comparison:

* normwise: max |y - ref| / max |ref|, the bar (1e-5 for fp32 storage, 1e-2 for fp16 / bf16);
* elementwise: max |y - ref| / |ref| over the entries with |ref| >= 1e-2 max |ref| (printed);
* componentwise: max |y - ref| / (|b| + sum |W| |f|), bounded by the rounding analysis of the
  kernels' evaluation: fp32 accumulation of K = 27 cin + 1 products and the bias, each product
  and each addition rounded (at most one fp32 ulp, 2^-23 relative, whatever the matrix cores'
  internal rounding mode), then one rounding to the storage type (unit roundoff 2^-8 bf16, 2^-11 fp16,
  2^-24 fp32, to nearest).  With gamma = 2K u / (1 - 2K u), u = 2^-23:
  |y - ref| <= (u_store (1 + gamma) + gamma) (|b| + sum |W| |f|).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
U_STORE = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def as64(t):
    return t.double().cpu().numpy() if hasattr(t, "double") else np.asarray(t, dtype=np.float64)


def oracle_rows(nbr, f, w, b=None, rows=None, chunk=32768):
    """oracle.conv3_rulebook over `rows` (default all), split into row chunks on host threads."""
    rows = np.arange(len(nbr)) if rows is None else np.asarray(rows)
    if len(rows) <= chunk:
        return oracle.conv3_rulebook(nbr, f, w, b, rows=rows)
    parts = np.array_split(rows, -(-len(rows) // chunk))
    with threadpool_limits(limits=1), ThreadPoolExecutor(host_threads()) as ex:
        out = list(ex.map(lambda r: oracle.conv3_rulebook(nbr, f, w, b, rows=r), parts))
    return np.concatenate(out)


def componentwise_bar(dtype: str, cin: int) -> float:
    k2 = 2 * (27 * cin + 1)
    u = 2.0 ** -23
    gamma = k2 * u / (1.0 - k2 * u)
    return U_STORE[dtype] * (1.0 + gamma) + gamma


def check_features(y, nbr, f, w, b, dtype, what, rows=None, mag_rows=None):
    """Compare GPU output rows with the oracle.

    y: GPU output (torch, any device) for `rows` of the rulebook (all rows if None); f, w, b: the
    float64 inputs (numpy).  The normwise bar is asserted on all of `rows`; the componentwise bound
    on `mag_rows` (indices into `rows`' positions; all if None).
    """
    y64 = as64(y)
    ref = oracle_rows(nbr, f, w, b, rows=rows)
    assert y64.shape == ref.shape, (y64.shape, ref.shape)
    err = oracle.normwise_rel_error(y64, ref)
    ew = oracle.elementwise_rel_error(y64, ref)
    pos = np.arange(len(ref)) if mag_rows is None else np.asarray(mag_rows)
    src_rows = (np.arange(len(nbr)) if rows is None else np.asarray(rows))[pos]
    mag = oracle_rows(nbr, np.abs(f), np.abs(w), None if b is None else np.abs(b), rows=src_rows)
    cw = oracle.componentwise_ratio(y64[pos], ref[pos], mag)
    bar = componentwise_bar(dtype, f.shape[1])
    print(f"  {what}: rows {len(ref)} normwise {err:.3e} (tol {TOL[dtype]:g}) elementwise {ew:.3e} "
          f"componentwise {cw:.3e} (bound {bar:.3e}, {len(pos)} rows)", flush=True)
    assert err <= TOL[dtype], f"{what}: normwise error {err:.3e} above {TOL[dtype]}"
    assert cw <= bar, f"{what}: componentwise ratio {cw:.3e} above {bar:.3e}"
    return ref
