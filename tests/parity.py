"""Helpers that compare the HIP path with the oracle (imported by the tests).

Agreement rules (the tolerances the method's target statement fixes):
  * indices: equal, except where the oracle's input lies within 1e-6 of a
    decision and the device's index is the valid result of taking that
    decision the other way: one step across a midpoint that the value is
    within 1e-6 of (this covers the fold's equator n_z = 0 as well), or for
    the octahedral fold the mirrored sign within 1e-6 of a lower-hemisphere
    seam p_x = 0 / p_y = 0 (an exact zero takes sgn(0) = +1 only).  Excused
    mismatches may be at most 1e-4 of all indices, unexcused ones none;
  * gamma: relative error <= 1e-6;
  * reconstructed keys and logits: relative error <= 1e-3 (logits against
    max(|l|, |q| gamma / sqrt(d)));
  * softmax . V: |do| / |o| <= 2e-3 per (batch, head, query).
The oracle always decodes the device's own packed stream for the decode-side
checks, so an excused encoder flip cannot leak into decode parity.
"""
from __future__ import annotations

import numpy as np

import oracle as O

BOUNDARY_TOL = 1e-6
MAX_EXCUSED_FRACTION = 1e-4


def unpack_device_codes(packed_words: np.ndarray, cb: O.Codebook, n_seq: int, cap: int, n: int,
                        start: int = 0) -> np.ndarray:
    """Device packed buffer (flat int32/uint32) -> codes (n_seq, n, T, 3)."""
    W = cb.words_per_key
    tiles = packed_words.astype(np.uint32).reshape(n_seq, cap // 64, 64 * W)
    words = O.from_tiles(tiles, W, cap)[:, start:start + n]
    return O.unpack_codes(words.reshape(-1, W), cb.T, cb.alloc).reshape(n_seq, n, cb.T, 3)


def unpack_device_signs(bits: np.ndarray, d: int, n_seq: int, cap: int, n: int, start: int = 0):
    tiles = bits.astype(np.uint32).reshape(n_seq, cap // 64, 64 * (d // 32))
    words = O.from_tiles(tiles, d // 32, cap)[:, start:start + n]
    return O.unpack_signs(words.reshape(-1, d // 32), d).reshape(n_seq, n, d)


def index_ok(g: int, v: float, cent: np.ndarray) -> bool:
    """Is the device index g a valid rounding of the value v?  Either the
    nearest centroid (midpoint rule), or the index one step across the midpoint
    between the two when v lies within BOUNDARY_TOL of that very midpoint."""
    o = int(O.quantize(np.array([v]), cent)[0])
    if g == o:
        return True
    if abs(g - o) != 1:
        return False
    return abs(v - O.midpoints(cent)[min(g, o)]) <= BOUNDARY_TOL


def fold_alternatives(n: np.ndarray):
    """Every (xi, eta) the octahedral fold of the unit triplet n may give when
    a sign decision within BOUNDARY_TOL of its seam is taken either way
    ([YL] 八面体折叠; readings: sgn(0) = +1, n_z = 0 is the upper hemisphere).

    In the lower hemisphere xi = (1 - |p_y|) sgn p_x jumps to its mirror
    image when p_x changes sign (likewise eta with p_y), so near p_x = 0 the
    mirrored value is as valid as the oracle's.  A sign whose oracle value is
    exactly 0 follows the reading alone: an exact zero is not a rounding
    question.  The hemisphere decision needs no alternative: the two branches
    differ by |n_z| / |n|_1, so a device that takes the other branch within
    BOUNDARY_TOL of the equator crosses only a midpoint within BOUNDARY_TOL of
    the oracle's value, which the midpoint rule already covers."""
    x, y, z = (float(c) for c in n)
    l1 = abs(x) + abs(y) + abs(z)
    px, py = x / l1, y / l1
    if not z < 0:
        return [(px, py)]
    sx = [1.0 if px >= 0 else -1.0]
    sy = [1.0 if py >= 0 else -1.0]
    if px != 0.0 and abs(px) <= BOUNDARY_TOL:
        sx.append(-sx[0])
    if py != 0.0 and abs(py) <= BOUNDARY_TOL:
        sy.append(-sy[0])
    return [((1.0 - abs(py)) * a, (1.0 - abs(px)) * c) for a in sx for c in sy]


def compare_codes(gpu_codes: np.ndarray, enc: O.Encoded, cb: O.Codebook):
    """Return (n_mismatch, n_excused, n_unexcused, total, mismatch mask per key).

    A mismatched index is excused only when the device's code is itself a
    valid encoding of the oracle's input:
      * rho: index_ok on the oracle's rho (one step across a midpoint within
        BOUNDARY_TOL of rho);
      * the (xi, eta) pair: for some fold alternative (fold_alternatives: the
        oracle's values, or the mirrored sign at a lower-hemisphere seam
        p_x = 0 or p_y = 0), both device indices pass index_ok on that
        alternative's values.
    Excused mismatches count per index."""
    g = gpu_codes.reshape(-1, cb.T, 3)
    o = enc.codes.reshape(-1, cb.T, 3)
    vals = enc.values.reshape(-1, cb.T, 3)
    mism = g != o
    total = g.size
    if not mism.any():
        return 0, 0, 0, total, np.zeros(g.shape[0], bool)
    excused = np.zeros_like(mism)
    t = O.split_triplets(enc.rotated).reshape(-1, cb.T, 3)
    for k, i in np.argwhere(mism.any(axis=-1)):
        if mism[k, i, 2]:
            excused[k, i, 2] = index_ok(int(g[k, i, 2]), float(vals[k, i, 2]), cb.c_rho)
        if mism[k, i, 0] or mism[k, i, 1]:
            _, n = O.triplet_polar(t[k, i][None, :])
            ok = any(index_ok(int(g[k, i, 0]), xa, cb.c_xi) and index_ok(int(g[k, i, 1]), ea, cb.c_eta)
                     for xa, ea in fold_alternatives(n[0]))
            excused[k, i, 0] = mism[k, i, 0] and ok
            excused[k, i, 1] = mism[k, i, 1] and ok
    n_mis = int(mism.sum())
    n_exc = int((mism & excused).sum())
    return n_mis, n_exc, n_mis - n_exc, total, mism.any(axis=(1, 2))


def assert_codes_match(gpu_codes, enc, cb, label="", cap_fraction=True):
    """cap_fraction=False for hand-made inputs built to sit on decision
    boundaries, where the 1e-4 budget for random data does not apply."""
    n_mis, n_exc, n_unexc, total, _ = compare_codes(gpu_codes, enc, cb)
    assert n_unexc == 0, f"{label}: {n_unexc} unexcused index mismatches of {total}"
    if cap_fraction:
        assert n_exc <= MAX_EXCUSED_FRACTION * total, f"{label}: {n_exc} excused of {total}"
    return n_mis


def rel_err_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = a.reshape(a.shape[0], -1) if a.ndim > 1 else a[:, None]
    b = b.reshape(b.shape[0], -1) if b.ndim > 1 else b[:, None]
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)


def logit_err(gpu: np.ndarray, ref: np.ndarray, qnorm: np.ndarray, gamma: np.ndarray, d: int):
    """max over entries of |dl| / max(|l|, |q| gamma / sqrt(d))."""
    scale = np.maximum(np.abs(ref), qnorm * gamma / np.sqrt(d))
    return float(np.max(np.abs(gpu - ref) / np.maximum(scale, 1e-30)))


def compare_joint_codes(gpu_codes: np.ndarray, enc: O.Encoded, cb: O.Codebook):
    """Joint rounding (the encoder's 3x3 search): a triplet whose device code
    differs from the oracle's is excused when the oracle's error of the
    device's choice, |t - rho^ n^|^2 in fp64, is within 1e-6 |t|^2 of the
    oracle's minimum (the choice was a near-tie for fp32), and the device's
    direction code lies in the 3x3 neighbourhood of the oracle's scalar
    indices moved by at most one more step (a scalar index on a midpoint may
    move the search's centre).  Counts are of indices, as for scalar
    rounding: (n_mismatch, n_excused, n_unexcused, total indices), an excused
    triplet counting each of its indices that differ."""
    g = gpu_codes.reshape(-1, 3)
    o = enc.codes.reshape(-1, 3)
    t = O.split_triplets(enc.rotated).reshape(-1, 3)
    diff = g != o
    mism = np.any(diff, axis=1)
    if not mism.any():
        return 0, 0, 0, g.size
    err = lambda c: np.sum((cb.c_rho[c[:, 2]][:, None]  # noqa: E731
                            * O.octa_decode(cb.c_xi[c[:, 0]], cb.c_eta[c[:, 1]]) - t) ** 2, axis=1)
    eg, eo = err(g), err(o)
    tt = np.sum(t * t, axis=1)
    _, n = O.triplet_polar(t)
    xi, eta = O.octa_encode(n)
    sx, se = O.quantize(xi, cb.c_xi), O.quantize(eta, cb.c_eta)
    near = (np.abs(g[:, 0] - sx) <= 2) & (np.abs(g[:, 1] - se) <= 2)
    excused = mism & (eg - eo <= BOUNDARY_TOL * np.maximum(tt, 1e-30)) & near
    n_mis, n_exc = int(diff.sum()), int(diff[excused].sum())
    return n_mis, n_exc, n_mis - n_exc, g.size
