"""The Python binding refuses mismatched shapes before any library call.

The C ABI receives bare pointers and cannot see tensor sizes, so the binding
compares every tensor with the cache and the codebook first: a mismatch is a
ValueError, never an out-of-bounds kernel access.  CPU only: the codebook is
host-only and the tensors live on the CPU; every call below stops at a shape
check (the device check comes after the shapes), so nothing is launched.
"""
import pytest

torch = pytest.importorskip("torch")

import rotation_preconditioned_quantization_amd as octo  # noqa: E402

D = 128


@pytest.fixture(scope="module")
def cb():
    try:
        octo.lib()
    except RuntimeError as e:  # pragma: no cover
        pytest.skip(str(e))
    return octo.Codebook(D, 3, device=None)


@pytest.fixture()
def cache(cb):
    return octo.Cache(cb, n_seq=4, cap=128, device="cpu")


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_encode_checks(cb, cache):
    keys = torch.zeros((4, 10, D), dtype=torch.bfloat16)
    raises("cache.n_seq", octo.octo_encode, cb, torch.zeros((5, 10, D), dtype=torch.bfloat16), cache)
    raises("capacity", octo.octo_encode, cb, keys, cache, pos0=120)
    raises("capacity", octo.octo_encode, cb, keys, cache, pos0=-1)
    raises("contiguous last dim", octo.octo_encode, cb, torch.zeros((4, 10, 64), dtype=torch.bfloat16), cache)
    raises("contiguous last dim", octo.octo_encode, cb, torch.zeros((4, D, 10), dtype=torch.bfloat16).transpose(1, 2), cache)
    raises("float32, bfloat16 or float16", octo.octo_encode, cb, keys.to(torch.float64), cache)
    raises(r"\[n_seq, n_new, d\]", octo.octo_encode, cb, keys[0], cache)
    raises("CUDA tensor", octo.octo_encode, cb, keys, cache)          # all shapes fine: device last
    raises("cache.n_seq", octo.octo_encode_joint, cb, torch.zeros((3, 10, D)), cache)


def test_other_codebook_layout_is_refused(cb, cache):
    other = octo.Codebook(D, 4, device=None)
    raises("another codebook", octo.octo_encode, other, torch.zeros((4, 10, D)), cache)
    other.close()


def test_logits_checks(cb, cache):
    q = torch.zeros((2, 8, D), dtype=torch.bfloat16)
    raises("B \\* Hkv", octo.octo_decode_logits, cb, q, cache, 100, Hkv=4)        # 2*4 != 4
    raises("multiple of Hkv", octo.octo_decode_logits, cb, torch.zeros((2, 7, D)), cache, 100, Hkv=2)
    raises("head dim", octo.octo_decode_logits, cb, torch.zeros((2, 8, 64)), cache, 100, Hkv=2)
    raises("n_keys", octo.octo_decode_logits, cb, q, cache, 129, Hkv=2)
    raises("contiguous", octo.octo_decode_logits, cb, torch.zeros((2, D, 8)).transpose(1, 2), cache, 100, Hkv=2)
    raises("logits must have shape", octo.octo_decode_logits, cb, q, cache, 100, Hkv=2,
           logits=torch.zeros((2, 8, 99)))
    raises("QJL", octo.octo_decode_logits, cb, q, cache, 100, Hkv=2, use_qjl=True)
    raises("CUDA tensor", octo.octo_decode_logits, cb, q, cache, 100, Hkv=2)


def test_attention_checks(cb, cache):
    q = torch.zeros((2, 8, 1, D), dtype=torch.bfloat16)
    v = torch.zeros((4, 128, D), dtype=torch.bfloat16)
    raises("v must have shape", octo.octo_decode_attn, cb, q, cache, torch.zeros((4, 100, D), dtype=torch.bfloat16),
           100, Hkv=2)
    raises("v must have shape", octo.octo_decode_attn, cb, q, cache, torch.zeros((8, 128, D), dtype=torch.bfloat16),
           100, Hkv=2)
    raises("contiguous bfloat16", octo.octo_decode_attn, cb, q, cache, v.float(), 100, Hkv=2)
    raises("B \\* Hkv", octo.octo_decode_attn, cb, q, cache, v, 100, Hkv=1)
    raises("out must have shape", octo.octo_decode_attn, cb, q, cache, v, 100, Hkv=2,
           out=torch.zeros((2, 8, 2, D)))
    raises("contiguous float32", octo.octo_decode_attn, cb, q, cache, v, 100, Hkv=2,
           out=torch.zeros((2, 8, 1, D), dtype=torch.float16))
    raises("workspace holds", octo.octo_decode_attn, cb, q, cache, v, 100, Hkv=2,
           workspace=torch.zeros(16, dtype=torch.uint8))
    raises("CUDA tensor", octo.octo_decode_attn, cb, q, cache, v, 100, Hkv=2)


def test_append_checks(cb, cache):
    q = torch.zeros((2, 8, 1, D), dtype=torch.bfloat16)
    v = torch.zeros((4, 128, D), dtype=torch.bfloat16)
    nk = torch.zeros((4, D), dtype=torch.bfloat16)
    raises("new_keys must be", octo.octo_decode_attn_append, cb, torch.zeros((3, D)), q, cache, v, 50, Hkv=2)
    raises("one query token", octo.octo_decode_attn_append, cb, nk, torch.zeros((2, 8, 2, D)), cache, v, 50, Hkv=2)
    raises("n_keys >= 1", octo.octo_decode_attn_append, cb, nk, q, cache, v, 0, Hkv=2)
    raises("n_keys", octo.octo_decode_attn_append, cb, nk, q, cache, v, 129, Hkv=2)
    raises("CUDA tensor", octo.octo_decode_attn_append, cb, nk, q, cache, v, 50, Hkv=2)


def test_debug_helpers_check(cb, cache):
    raises("out must have shape", octo.octo_debug_reconstruct, cb, cache, 10, out=torch.zeros((4, 11, D)))
    raises("n_keys", octo.octo_debug_reconstruct, cb, cache, 200)
    raises("differ in size", octo.octo_debug_copy, torch.zeros(4), torch.zeros(8))
