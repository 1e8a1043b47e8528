"""Helpers that compare the HIP path with the oracle (imported by the tests).

Agreement rules (the tolerances the method's target statement fixes):
  * indices: equal, except where the oracle's value lies within 1e-6 of the
    decision it crossed (a midpoint, or for the octahedral fold the equator
    n_z = 0 or the seams p_x = 0 / p_y = 0 of the lower hemisphere); excused
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


def compare_codes(gpu_codes: np.ndarray, enc: O.Encoded, cb: O.Codebook):
    """Return (n_mismatch, n_excused, n_unexcused, total, mismatch mask per key)."""
    g = gpu_codes.reshape(-1, cb.T, 3)
    o = enc.codes.reshape(-1, cb.T, 3)
    vals = enc.values.reshape(-1, cb.T, 3)
    mism = g != o
    total = g.size
    if not mism.any():
        return 0, 0, 0, total, np.zeros(g.shape[0], bool)
    excused = np.zeros_like(mism)
    # distance of the oracle value to the midpoints between the two indices
    for c, cent in enumerate((cb.c_xi, cb.c_eta, cb.c_rho)):
        mids = O.midpoints(cent)
        idx = np.argwhere(mism[..., c])
        for k, i in idx:
            lo, hi = sorted((g[k, i, c], o[k, i, c]))
            crossed = mids[lo:hi]
            if crossed.size and np.min(np.abs(vals[k, i, c] - crossed)) <= BOUNDARY_TOL:
                excused[k, i, c] = True
    # octahedral fold decisions: equator and lower-hemisphere seams
    t = O.split_triplets(enc.rotated).reshape(-1, cb.T, 3)
    _, n = O.triplet_polar(t.reshape(-1, 3))
    n = n.reshape(-1, cb.T, 3)
    l1 = np.abs(n).sum(-1)
    px, py, nz = n[..., 0] / l1, n[..., 1] / l1, n[..., 2]
    seam = (np.abs(nz) <= BOUNDARY_TOL) | ((nz < 0) & ((np.abs(px) <= BOUNDARY_TOL) |
                                                      (np.abs(py) <= BOUNDARY_TOL)))
    excused[..., 0] |= mism[..., 0] & seam
    excused[..., 1] |= mism[..., 1] & seam
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
    move the search's centre).  Returns (n_mismatch, n_excused, n_unexcused,
    total triplets)."""
    g = gpu_codes.reshape(-1, 3)
    o = enc.codes.reshape(-1, 3)
    t = O.split_triplets(enc.rotated).reshape(-1, 3)
    mism = np.any(g != o, axis=1)
    if not mism.any():
        return 0, 0, 0, g.shape[0]
    err = lambda c: np.sum((cb.c_rho[c[:, 2]][:, None]  # noqa: E731
                            * O.octa_decode(cb.c_xi[c[:, 0]], cb.c_eta[c[:, 1]]) - t) ** 2, axis=1)
    eg, eo = err(g), err(o)
    tt = np.sum(t * t, axis=1)
    _, n = O.triplet_polar(t)
    xi, eta = O.octa_encode(n)
    sx, se = O.quantize(xi, cb.c_xi), O.quantize(eta, cb.c_eta)
    near = (np.abs(g[:, 0] - sx) <= 2) & (np.abs(g[:, 1] - se) <= 2)
    excused = mism & (eg - eo <= BOUNDARY_TOL * np.maximum(tt, 1e-30)) & near
    n_mis, n_exc = int(mism.sum()), int(excused.sum())
    return n_mis, n_exc, n_mis - n_exc, g.shape[0]
