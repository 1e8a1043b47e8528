"""The encoder kernels' nearest-centroid lookup for xi and eta, checked on the
host against its definition ([YL] 三元组分解 step 4: the Lloyd-Max index of a
value is the number of midpoints of adjacent centroids below it).

octo_debug_bucket_index evaluates the kernels' own formula (one fma whose
rounding lands the bucket in the mantissa, one table entry, one compare) over
the codebook's table, so these tests pin both the formula and the table the
host builds for it: at every fp32 midpoint and its two fp32 neighbours, at
every bucket edge, at the ends of [-1, 1] and a rounding step past them, and
on a dense grid.
"""
import numpy as np
import pytest

import rotation_preconditioned_quantization_amd as octo

QX, QE = octo.TABLES.index("qx"), octo.TABLES.index("qe")


def _mids32(c):
    """fp32 midpoints of the sorted centroids, rounded from their fp64 values."""
    c = np.asarray(c, dtype=np.float64)
    return (0.5 * (c[:-1] + c[1:])).astype(np.float32)


def _probe_values(m32):
    f32 = np.float32
    pts = [np.linspace(-1.0, 1.0, 20001, dtype=np.float32), m32,
           np.nextafter(m32, f32(np.inf)), np.nextafter(m32, f32(-np.inf))]
    # bucket edges of a centred table of nb buckets over [-1, 1] (the
    # builder takes the smallest of 16 ... 256 that works), and their
    # neighbours
    for n in (16, 32, 64, 128, 256):
        e = (-1.0 + (np.arange(n + 1) + 0.5) * (2.0 / n)).astype(np.float32)
        pts += [e, np.nextafter(e, f32(np.inf)), np.nextafter(e, f32(-np.inf))]
    ends = np.array([-1.0, 1.0, -1.0 - 2.0 ** -22, 1.0 + 2.0 ** -22, 0.0, -0.0], dtype=np.float32)
    pts.append(ends)
    x = np.concatenate(pts).astype(np.float32)
    # the kernels' domain: [-1, 1] up to the rounding of xi and eta
    return x[np.abs(x) <= np.float32(1.0 + 2.0 ** -22)]


@pytest.mark.parametrize("d,b", [(64, 1), (64, 3), (128, 2), (128, 3), (128, 4), (128, 5), (256, 2)])
def test_lookup_equals_midpoint_count(d, b):
    cb = octo.Codebook(d, b, mc_vectors=4096, device=None)
    try:
        cx, ce, _, _, _ = cb.export()
        for table, c in ((QX, cx), (QE, ce)):
            m32 = _mids32(c)
            x = _probe_values(m32)
            got = octo.octo_debug_bucket_index(cb, table, x)
            want = (x[:, None] > m32[None, :]).sum(axis=1).astype(np.uint32)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (table, x[bad[:5]], got[bad[:5]], want[bad[:5]])
    finally:
        cb.close()


def test_lookup_rejects_other_tables_and_out_of_range_values():
    cb = octo.Codebook(128, 3, mc_vectors=4096, device=None)
    try:
        with pytest.raises(octo.OctoError):
            octo.octo_debug_bucket_index(cb, octo.TABLES.index("qr2"), np.zeros(4, np.float32))
        with pytest.raises(octo.OctoError):
            octo.octo_debug_bucket_index(cb, QX, np.array([np.nan], np.float32))
        with pytest.raises(octo.OctoError):
            octo.octo_debug_bucket_index(cb, QE, np.array([4.0], np.float32))
    finally:
        cb.close()
