"""The GPU-vs-oracle index rules (tests/parity.py) on synthetic device codes.

CPU only: "device" codes are made by hand from the oracle's own, so every
excuse the rules grant is checked to be the valid encoding of a decision
taken the other way, and every other change to be caught:
  * a mirrored xi at a lower-hemisphere sign seam p_x ~ 0 passes; any other
    code there fails; the mirror of an exact zero fails (sgn(0) = +1);
  * one step across a midpoint the value is within 1e-6 of passes; two steps,
    or one step the other way, fail;
  * near the equator nothing but the midpoint rule applies;
  * the 1e-4 cap on excused indices holds for random data.
"""
import numpy as np
import pytest

import oracle as O
from parity import (BOUNDARY_TOL, assert_codes_match, compare_codes, compare_joint_codes,
                    fold_alternatives, index_ok)

D, BITS = 128, 3


@pytest.fixture(scope="module")
def cb():
    return O.build_codebook(D, BITS)


def encoded_from_rotated(up: np.ndarray, cb) -> O.Encoded:
    """The oracle's encoding of rotated unit keys up (n, d), exactly as
    O.encode computes it after the rotation (so crafted values stay exact)."""
    rho, n = O.triplet_polar(O.split_triplets(up).reshape(-1, 3))
    xi, eta = O.octa_encode(n)
    nk = up.shape[0]
    values = np.stack([xi, eta, rho], axis=-1).reshape(nk, cb.T, 3)
    codes = np.stack([O.quantize(xi, cb.c_xi), O.quantize(eta, cb.c_eta),
                      O.quantize(rho, cb.c_rho)], axis=-1).reshape(nk, cb.T, 3)
    return O.Encoded(codes, np.ones(nk, np.float32), values, up)


def key_with_triplet0(t0, seed=0):
    """A rotated unit key whose first triplet is rho * t0 / |t0| (rho = 0.2)
    and whose other coordinates are random."""
    rng = np.random.default_rng(seed)
    up = rng.standard_normal(D)
    t0 = np.asarray(t0, dtype=np.float64)
    up[3:] *= np.sqrt(1.0 - 0.2 ** 2) / np.linalg.norm(up[3:])
    up[:3] = 0.2 * t0 / np.linalg.norm(t0)
    return up[None, :]


def counts(dev_codes, enc, cb):
    n_mis, n_exc, n_unexc, _, _ = compare_codes(dev_codes, enc, cb)
    return n_mis, n_exc, n_unexc


def test_identical_codes_pass(cb):
    enc = encoded_from_rotated(key_with_triplet0([0.3, -0.2, 0.5]), cb)
    assert counts(enc.codes.copy(), enc, cb) == (0, 0, 0)


@pytest.mark.parametrize("comp", [0, 1])
def test_lower_seam_mirror_passes(cb, comp):
    """p_x (or p_y) a hair above zero in the lower hemisphere: the device may
    take the other sign, and its code is then the oracle's code of -xi."""
    t0 = [1e-9, 0.3, -0.8] if comp == 0 else [0.3, 1e-9, -0.8]
    enc = encoded_from_rotated(key_with_triplet0(t0), cb)
    cent = cb.c_xi if comp == 0 else cb.c_eta
    v = enc.values[0, 0, comp]
    mirror = int(O.quantize(np.array([-v]), cent)[0])
    assert mirror != enc.codes[0, 0, comp]
    dev = enc.codes.copy()
    dev[0, 0, comp] = mirror
    assert counts(dev, enc, cb) == (1, 1, 0)


def test_lower_seam_other_code_fails(cb):
    enc = encoded_from_rotated(key_with_triplet0([1e-9, 0.3, -0.8]), cb)
    v = enc.values[0, 0, 0]
    mirror = int(O.quantize(np.array([-v]), cb.c_xi)[0])
    o = int(enc.codes[0, 0, 0])
    for wrong in range(cb.c_xi.size):
        if wrong in (o, mirror):
            continue
        dev = enc.codes.copy()
        dev[0, 0, 0] = wrong
        assert counts(dev, enc, cb)[2] == 1, wrong


def test_lower_seam_mirror_with_eta_change_fails(cb):
    """The mirror moves xi only; a changed eta beside it is not excused."""
    enc = encoded_from_rotated(key_with_triplet0([1e-9, 0.3, -0.8]), cb)
    dev = enc.codes.copy()
    dev[0, 0, 0] = int(O.quantize(np.array([-enc.values[0, 0, 0]]), cb.c_xi)[0])
    dev[0, 0, 1] = (dev[0, 0, 1] + 1) % cb.c_eta.size
    assert counts(dev, enc, cb)[2] == 2


def test_exact_zero_sign_is_not_excused(cb):
    """x = 0 exactly in the lower hemisphere: sgn(0) = +1 is the reading, so
    the mirrored code (what a -0.0 fold would give) must not pass."""
    enc = encoded_from_rotated(key_with_triplet0([0.0, 0.3, -0.8]), cb)
    assert enc.rotated[0, 0] == 0.0 and enc.values[0, 0, 0] > 0
    dev = enc.codes.copy()
    dev[0, 0, 0] = int(O.quantize(np.array([-enc.values[0, 0, 0]]), cb.c_xi)[0])
    assert counts(dev, enc, cb)[2] == 1


def test_upper_hemisphere_has_no_sign_seam(cb):
    """In the upper hemisphere xi = p_x is continuous through p_x = 0: a
    mirrored code is not a valid encoding there."""
    enc = encoded_from_rotated(key_with_triplet0([1e-9, 0.3, 0.8]), cb)
    alts = fold_alternatives(enc.rotated[0, :3] / np.linalg.norm(enc.rotated[0, :3]))
    assert len(alts) == 1
    dev = enc.codes.copy()
    dev[0, 0, 1] = cb.c_eta.size - 1 - dev[0, 0, 1]
    assert counts(dev, enc, cb)[2] == 1


def _upper_triplet_with_xi(xi, eta=0.25):
    """Upper-hemisphere direction with p = (xi, eta) exactly (|n|_1 scaling)."""
    return [xi, eta, 1.0 - abs(xi) - abs(eta)]


def test_midpoint_one_step_passes_two_steps_fail(cb):
    mids = O.midpoints(cb.c_xi)
    k = 9
    enc = encoded_from_rotated(key_with_triplet0(_upper_triplet_with_xi(mids[k] + 3e-7)), cb)
    o = int(enc.codes[0, 0, 0])
    assert o == k + 1
    cases = {k: (1, 1, 0),       # one step across m_k: valid
             k - 1: (1, 0, 1),   # two steps: crosses m_k and m_k-1
             k + 2: (1, 0, 1)}   # one step, across m_k+1, which is far
    for g, want in cases.items():
        dev = enc.codes.copy()
        dev[0, 0, 0] = g
        assert counts(dev, enc, cb) == want, g


def test_midpoint_just_outside_tolerance_fails(cb):
    mids = O.midpoints(cb.c_xi)
    enc = encoded_from_rotated(key_with_triplet0(_upper_triplet_with_xi(mids[4] + 3e-6)), cb)
    dev = enc.codes.copy()
    dev[0, 0, 0] -= 1
    assert counts(dev, enc, cb) == (1, 0, 1)


def test_rho_midpoint_rule(cb):
    """rho: one step across a midpoint within 1e-6 passes, two steps fail."""
    mids = O.midpoints(cb.c_rho)
    up = key_with_triplet0([0.3, -0.2, 0.5])
    # set triplet 0's norm onto a midpoint (the rest rescaled to keep |u'| = 1)
    target = mids[1] + 2e-7
    up[0, :3] *= target / np.linalg.norm(up[0, :3])
    up[0, 3:] *= np.sqrt(1 - target ** 2) / np.linalg.norm(up[0, 3:])
    enc = encoded_from_rotated(up, cb)
    assert enc.codes[0, 0, 2] == 2
    for g, want in {1: (1, 1, 0), 0: (1, 0, 1), 3: (1, 0, 1)}.items():
        dev = enc.codes.copy()
        dev[0, 0, 2] = g
        assert counts(dev, enc, cb) == want, g


def test_equator_excuses_only_midpoints(cb):
    """n_z a hair below zero: the other hemisphere moves xi by |n_z|/|n|_1
    only, so a code change far from every midpoint is not excused (it was
    under a blanket equator excuse)."""
    enc = encoded_from_rotated(key_with_triplet0([0.45, 0.5, -1e-9]), cb)
    v = enc.values[0, 0, 0]
    assert np.min(np.abs(O.midpoints(cb.c_xi) - v)) > 1e-3
    dev = enc.codes.copy()
    dev[0, 0, 0] += 1
    assert counts(dev, enc, cb)[2] == 1


def test_index_ok_definition(cb):
    mids = O.midpoints(cb.c_xi)
    assert index_ok(8, mids[7] + 1e-7, cb.c_xi) and index_ok(7, mids[7] + 1e-7, cb.c_xi)
    assert not index_ok(6, mids[7] + 1e-7, cb.c_xi)
    assert not index_ok(7, mids[7] + 2e-6, cb.c_xi)


def test_cap_on_excused_fraction(cb):
    """Random keys: excused mismatches above 1e-4 of all indices fail the cap,
    even when every one of them is individually valid."""
    rng = np.random.default_rng(5)
    up = rng.standard_normal((40, D))
    up /= np.linalg.norm(up, axis=1, keepdims=True)
    # put the first triplet of every key just above a xi midpoint
    mids = O.midpoints(cb.c_xi)
    for r in range(up.shape[0]):
        xi = mids[r % mids.size] + 1e-7
        t0 = np.array(_upper_triplet_with_xi(xi, eta=0.1 * np.sign(xi) or 0.1))
        t0 *= 0.15 / np.linalg.norm(t0)
        up[r, 3:] *= np.sqrt(1 - 0.15 ** 2) / np.linalg.norm(up[r, 3:])
        up[r, :3] = t0
    enc = encoded_from_rotated(up, cb)
    dev = enc.codes.copy()
    dev[:, 0, 0] -= 1
    n_mis, n_exc, n_unexc, total, _ = compare_codes(dev, enc, cb)
    assert n_unexc == 0 and n_exc == 40
    with pytest.raises(AssertionError):
        assert_codes_match(dev, enc, cb, "capped")
    assert_codes_match(dev, enc, cb, "uncapped", cap_fraction=False)


def test_joint_counts_are_per_index(cb):
    """compare_joint_codes counts indices like the scalar rule, and rejects a
    code that is not a near-tie of the joint search."""
    rng = np.random.default_rng(3)
    up = rng.standard_normal((30, D))
    up /= np.linalg.norm(up, axis=1, keepdims=True)
    enc = O.encode(up @ cb.R, cb, rounding="joint")
    n_mis, n_exc, n_unexc, total = compare_joint_codes(enc.codes.copy(), enc, cb)
    assert (n_mis, total) == (0, enc.codes.size)
    dev = enc.codes.copy()
    dev[4, 7, 2] = (dev[4, 7, 2] + 2) % cb.c_rho.size
    n_mis, n_exc, n_unexc, total = compare_joint_codes(dev, enc, cb)
    assert (n_mis, n_exc, n_unexc) == (1, 0, 1)


def test_boundary_tolerance_is_the_target_statement():
    assert BOUNDARY_TOL == 1e-6
