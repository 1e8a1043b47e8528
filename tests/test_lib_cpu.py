"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, builds host-only codebooks that match the oracle's
independently built ones, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "octo.h")

octo = pytest.importorskip("rotation_preconditioned_quantization_amd")
if not os.path.exists(octo.LIB_PATH):
    pytest.skip("liboctox.so not built", allow_module_level=True)


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(octo_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    lib = octo.lib()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(octo.exported_symbols())


@pytest.mark.parametrize("d,b,qjl", [(128, 4, False), (128, 3, True), (128, 2, False), (64, 3, False),
                                      (128, 1, False), (64, 5, True), (256, 3, False)])
def test_host_codebook_matches_oracle(d, b, qjl):
    cb = octo.Codebook(d, b, seed=5, cb_seed=7, qjl=qjl, device=None)
    cx, ce, cr, sg, S = cb.export()
    ref = O.build_codebook(d, b, seed=5, cb_seed=7)
    assert np.max(np.abs(cx - ref.c_xi)) <= 1e-9 * np.max(np.abs(ref.c_xi))
    assert np.max(np.abs(ce - ref.c_eta)) <= 1e-9 * np.max(np.abs(ref.c_eta))
    assert np.max(np.abs(cr / ref.c_rho - 1)) <= 1e-9
    assert np.array_equal(sg.astype(np.float64), ref.signs)
    if qjl:
        # the host orthonormalises in its own order (Gram-Schmidt) and the
        # oracle through LAPACK's QR: the same Q up to fp64 rounding, so the
        # fp32 S agree to within one fp32 rounding
        Sref = O.qjl_matrix(d, 5)
        assert np.max(np.abs(S - Sref) / np.maximum(np.abs(Sref), 1.0)) <= 2.0 ** -23
        S64 = S.astype(np.float64)
        assert np.max(np.abs(S64 @ S64.T - d * np.eye(d))) <= 1e-4 * d
    lay = cb.layout
    assert (lay.b_xi, lay.b_eta, lay.b_rho) == (b + 1, b + 1, b - 1)
    assert lay.bits_per_triplet == 3 * b + 1 and lay.n_triplets == O.n_triplets(d)
    assert lay.words_per_key == O.layout(d, ref.alloc)["words_per_key"]
    assert cb.packed_words(3, 128) == 3 * 128 * lay.words_per_key
    cb.close()


def test_host_codebook_uniform_allocation_is_3b_bits():
    cb = octo.Codebook(128, 3, alloc=(3, 3, 3), device=None)
    assert cb.layout.bits_per_triplet == 9
    ref = O.build_codebook(128, 3, alloc=(3, 3, 3))
    cx, _, cr, _, _ = cb.export()
    assert np.max(np.abs(cx - ref.c_xi)) < 1e-9 and np.max(np.abs(cr - ref.c_rho)) < 1e-9


def test_argument_errors_before_any_launch():
    lib = octo.lib()
    p = octo.octo_params()
    p.d, p.b, p.b_xi, p.b_eta, p.b_rho, p.device = 100, 3, -1, -1, -1, -1
    h = ctypes.c_void_p()
    assert lib.octo_codebook_build(ctypes.byref(p), ctypes.byref(h)) == octo.OCTO_ERR_INVALID_ARG
    assert b"power of two" in lib.octo_last_error()
    p.d, p.b, p.device = 128, 9, -1
    assert lib.octo_codebook_build(ctypes.byref(p), ctypes.byref(h)) == octo.OCTO_ERR_INVALID_ARG
    p.d, p.b, p.device = 512, 3, 0       # no kernel for d=512: refused before any upload
    assert lib.octo_codebook_build(ctypes.byref(p), ctypes.byref(h)) == octo.OCTO_ERR_UNSUPPORTED
    assert lib.octo_codebook_build(None, ctypes.byref(h)) == octo.OCTO_ERR_INVALID_ARG
    cb = octo.Codebook(128, 3, device=None)
    # host-only codebooks are refused by every kernel entry point
    st = lib.octo_encode(cb.handle, None, 1, 1, 64, 8192, 128, 0, 64, None, None, None, None, None)
    assert st == octo.OCTO_ERR_INVALID_ARG and b"host-only" in lib.octo_last_error()
    st = lib.octo_decode_logits(cb.handle, None, 1, 1, 4, 2, None, None, None, None, 64, 64, None,
                                None, 0, None)
    assert st == octo.OCTO_ERR_INVALID_ARG
    st = lib.octo_decode_attn(cb.handle, None, 1, 1, 4, 2, 1, None, None, None, None, None, 1, 64, 64,
                              0.0, None, None, 0, None)
    assert st == octo.OCTO_ERR_INVALID_ARG
    assert lib.octo_debug_reconstruct(None, None, None, 1, 1, 64, None, None) == octo.OCTO_ERR_INVALID_ARG
    assert lib.octo_status_str(octo.OCTO_ERR_WORKSPACE) == b"OCTO_ERR_WORKSPACE"
    # workspace sizing is pure host arithmetic
    n0 = lib.octo_decode_workspace_bytes(cb.handle, 0, 1, 32, 8, 1, 32768)
    n1 = lib.octo_decode_workspace_bytes(cb.handle, 1, 1, 32, 8, 1, 32768)
    assert 0 < n0 < n1 and n0 % 256 == 0
    cb.close()
