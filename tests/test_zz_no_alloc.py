"""octo_decode_attn_static (the decode entry point that allocates nothing)
against octo_decode_attn through the C ABI: two calls in a row, the second
smaller, on the single-query and the multi-query kernels; the results must
agree to the attention tolerance (they share the kernels and the launch
configuration, so in fact bit for bit).  An oversized call is refused before
any launch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as WL  # noqa: E402

pytestmark = pytest.mark.gpu


def _octo():
    import rotation_preconditioned_quantization_amd as octo
    return octo


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _octo().lib()


def _case(cb, cfg, B, Hkv, G, n_q, n, cap, seed):
    octo = _octo()
    keys = WL.make_keys(cfg, "cuda", seed=seed, n_seq=B * Hkv, n=n)
    cache = octo.Cache(cb, B * Hkv, cap)
    octo.octo_encode(cb, keys, cache)
    v = WL.make_values(cfg, "cuda", seed=seed, n_seq=B * Hkv, cap=cap)
    q = WL.make_queries(cfg.scaled(Hq=Hkv * G, n_q=n_q), "cuda", seed=seed, B=B).contiguous()
    return cache, v, q


@pytest.mark.parametrize("path", ["single", "multi", "multi-d256"])
def test_static_scratch_equals_workspace_call(path):
    octo = _octo()
    if path == "single":
        cfg = WL.WORKLOADS["extreme"]
        cb = octo.Codebook(128, 2, device=0)
        shapes = [(2, 4, 4, 1, 20000, 20032), (1, 2, 4, 1, 3000, 3008)]   # second call smaller
    elif path == "multi-d256":
        # two value-dim workgroups per query block and split
        cfg = WL.WORKLOADS["video_block"].scaled(d=256, b=3)
        cb = octo.Codebook(256, 3, device=0)
        shapes = [(1, 2, 1, 300, 3000, 3008), (1, 1, 1, 70, 500, 512)]
    else:
        cfg = WL.WORKLOADS["video_block"]
        cb = octo.Codebook(64, 3, device=0)
        shapes = [(1, 4, 1, 300, 9000, 9024), (1, 2, 1, 70, 1000, 1024)]
    out_static = None
    for i, (B, Hkv, G, n_q, n, cap) in enumerate(shapes):
        cache, v, q = _case(cb, cfg, B, Hkv, G, n_q, n, cap, seed=40 + i)
        ref = octo.octo_decode_attn(cb, q, cache, v, n, Hkv)
        out_static = torch.full_like(ref, float("nan"))
        octo.octo_decode_attn_static(cb, q, cache, v, n, Hkv, out=out_static)
        torch.cuda.synchronize()
        a, b = out_static.double().cpu().numpy(), ref.double().cpu().numpy()
        rel = np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)
        print(f"[static {path} call {i}] {tuple(q.shape)} over {n} keys: max rel diff {rel.max():.2e}",
              flush=True)
        assert np.all(rel <= 2e-3)
        assert torch.equal(out_static, ref)


def test_static_scratch_refuses_oversized_calls():
    octo = _octo()
    cb = octo.Codebook(64, 3, device=0)
    # 32 heads x 4096 query rows over a 2^20-key cache need 66 MiB of partials
    assert cb.workspace_bytes(1, 1, 32, 1, 4096, 1 << 20) > (64 << 20)
    big_q = torch.zeros((1, 32, 4096, 64), dtype=torch.bfloat16, device="cuda")
    big_cache = octo.Cache(cb, 1, 1 << 20)
    big_v = torch.zeros((1, 1 << 20, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(octo.OctoError) as e:
        octo.octo_decode_attn_static(cb, big_q, big_cache, big_v, 1 << 20, 1)
    assert e.value.status == octo.OCTO_ERR_WORKSPACE
