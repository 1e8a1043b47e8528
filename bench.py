#!/usr/bin/env python3
"""Benchmark: fused compressed-K decode GB/s (% of HBM peak) + encode Mkeys/s, d=128.

Default workload (one GPU): the extreme-compression shape -- batch 4, 32
query heads over 8 KV heads, head dim 128, 131072 cached keys per KV head,
b = 2 (7 bits per triplet), bf16 Student-t(5) keys with log-normal per-token
norms, bf16 values, one bf16 query token: 1248 MB of compressed K and V per
decode, the largest d = 128 decode that fits one GPU.  Synthetic seeded
inputs stand in for the pages' model KV caches.  --config selects the other
workloads (2: the LLM-decode shape, 32768 keys per KV head at b = 4).

One step = the whole hot path over one batch: encode every key of the cache
(octo_encode) and run the fused decode attention over it (octo_decode_attn:
split-K fused kernel, combine).  Inputs sit in HBM before the timed region;
R rotating copies of every buffer (>= 1 GiB in total) keep each step's reads
out of the 256 MB Infinity Cache.  Each step is captured once into a HIP
graph and replayed.

Prints one JSON line.  `value` is the decode throughput (algorithmic bytes of
packed K + gamma + V per decode call / its time); `roofline` prices the
dominant kernel (the fused attention kernel) against 8 TB/s, with `traffic`
from the committed rocprofv3 counter summary of that workload; `cpu_baseline`
times the fp64 oracle on a bounded sample of the same workload on the host
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    1: "toy: 1 head, d=128, 4096 fp32 keys, b=3, 1 fp32 query (logits)",
    2: "llm_decode: B=1, Hq=32, Hkv=8, d=128, 32768 keys/KV head, b=4, bf16 K (4 outlier "
       "channels x10) and V, 1 query token",
    3: "extreme: B=4, Hq=32, Hkv=8, d=128, 131072 keys/KV head, b=2, bf16 Student-t(5) K with "
       "log-normal norms, bf16 V, 1 query token",
    4: "video_block: d=64, 24 heads, b=3, 65536-key cache with a 16384-key chunk encoded per "
       "step, 256 bf16 queries per head (multi-query MFMA attention)",
    5: "qjl: B=8, Hq=32, Hkv=8, d=128, 65536 keys/KV head, b=3 + 1-bit QJL residual signs, "
       "1 query token (logits)",
}
# committed HBM-traffic summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE passes of
# `bench.py --counters --config N`), one per workload
TRAFFIC_PROFILE = {c: os.path.join(ROOT, "profiles", f"{n}_hbm_traffic.txt") for c, n in
                   {1: "toy", 2: "llm_decode", 3: "extreme", 4: "video_block", 5: "qjl"}.items()}
# sources of the decode kernels whose counters a summary holds
KERNEL_SOURCES = {"attn": ("k_decode.hip", "octo_device.hpp", "octo_internal.hpp", "octo_encode_dev.hpp"),
                  "logits": ("k_decode.hip", "octo_device.hpp", "octo_internal.hpp", "octo_encode_dev.hpp"),
                  "attn_mq": ("k_mq.hip", "octo_device.hpp", "octo_internal.hpp")}
MAIN_KERNEL = {"logits": "k_logits", "attn": "k_attn", "attn_mq": "k_mq_attn"}


def kernel_source_hash(mode: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[mode]:
        with open(os.path.join(ROOT, "rotation_preconditioned_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(cfg):
    """HBM bytes per launch of the workload's dominant decode kernel from its
    committed counter summary, or None when there is none or the kernel's
    sources changed since the counters were taken."""
    path = TRAFFIC_PROFILE.get(cfg.cid)
    if not path or not os.path.exists(path):
        return None
    pc = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(("#", "|", "command")):
                k, v = ln.split(":", 1)
                pc[k.strip()] = v.strip()
    if pc.get("kernel_source_hash") != kernel_source_hash(cfg.mode):
        return None
    v = pc.get(f"{MAIN_KERNEL[cfg.mode]}.hbm_bytes_per_launch")
    return int(float(v)) if v else None


def algorithmic_bytes(cfg, lay):
    """Algorithmic bytes per decode call and per encode call: the packed codes
    at their exact bit count, gamma, the QJL signs and norm when present, the
    bf16 V rows (attention), the queries and outputs; the encoder reads the
    keys and writes codes and gamma."""
    n = cfg.n_seq * cfg.N
    packed = lay.n_triplets * lay.bits_per_triplet / 8.0     # bits actually used per key
    per_key = packed + 4.0                                   # packed stream + fp32 gamma
    if cfg.qjl:
        per_key += cfg.d / 8.0 + 2.0                         # sign bits + fp16 residual norm
    k_bytes = n * per_key
    qb = 4 if cfg.qdtype == "f32" else 2
    if cfg.mode == "logits":
        dec = k_bytes + cfg.B * cfg.Hq * cfg.d * qb + cfg.B * cfg.Hq * cfg.N * 4.0
    else:
        v_bytes = n * cfg.d * 2.0                            # bf16 V
        dec = k_bytes + v_bytes + cfg.B * cfg.Hq * cfg.n_q * cfg.d * (qb + 4)
    kb = 4 if cfg.kdtype == "f32" else 2
    enc = n * (cfg.d * kb + per_key)                         # keys in, packed + gamma out
    return dec, enc, n


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands, on a bounded sample of the same workload: one
    KV head (one head for the multi-query shape) of the workload's keys,
    values and queries, encoded and decoded in fp64 NumPy on the host cores
    (BLAS threads = the cores this process may run on) until `seconds` have
    passed.  The value is the decode's algorithmic bytes per second, the same
    per-key bytes as the GPU row."""
    import numpy as np

    import oracle as O
    import workloads as WL
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # threadpoolctl absent: BLAS keeps its own default
        limiter = None
    cb = O.build_codebook(cfg.d, cfg.b)            # setup, not timed
    S = O.qjl_matrix(cfg.d, 0) if cfg.qjl else None
    n_keys = min(8192, cfg.N)
    f64 = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    keys = f64(WL.make_keys(cfg, "cpu", seed=7, n_seq=1, n=n_keys)[0])
    qs = f64(WL.make_queries(cfg, "cpu", seed=7)[0])          # [Hq, n_q, d]
    if cfg.mode == "attn_mq":
        q, heads = qs[0], 1                                    # 256 queries of one head
    else:
        q, heads = qs[: cfg.G, 0], cfg.G                       # the G heads of one KV head
    v = None if cfg.mode == "logits" else f64(WL.make_values(cfg, "cpu", seed=7, n_seq=1, cap=n_keys)[0])
    t_enc = t_dec = 0.0
    reps = 0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        enc = O.encode(keys, cb)
        qe = O.qjl_encode(enc.rotated, O.decode_rotated(enc.codes, cb), S) if cfg.qjl else None
        t1 = time.perf_counter()
        uh = O.decode_rotated(enc.codes, cb)                   # the decode starts from the codes
        if cfg.mode == "logits":
            for h in range(heads):
                (O.qjl_logits(q[h], uh, enc.gamma, qe, S, cb) if cfg.qjl
                 else O.logits_rotated(q[h], uh, enc.gamma, cb))
        elif cfg.mode == "attn_mq":
            O.softmax_attention(O.logits_rotated(q, uh, enc.gamma, cb) / math.sqrt(cfg.d), v)
        else:
            for h in range(heads):
                O.softmax_attention(O.logits_rotated(q[h], uh, enc.gamma, cb) / math.sqrt(cfg.d), v)
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        reps += 1
        if time.perf_counter() - t_start > seconds:
            break
    if limiter is not None:
        limiter.unregister()
    per_key = O.n_triplets(cfg.d) * sum(O.default_alloc(cfg.b)) / 8.0 + 4.0
    if cfg.qjl:
        per_key += cfg.d / 8.0 + 2.0
    per_key += 4.0 * heads if cfg.mode == "logits" else 2.0 * cfg.d
    dec_bytes = reps * n_keys * per_key
    what = {"logits": f"{heads} query heads' logits" + (" with the QJL term" if cfg.qjl else ""),
            "attn": f"{heads} query heads' softmax.V",
            "attn_mq": f"{q.shape[0]} queries' softmax.V"}[cfg.mode]
    return {
        "value": dec_bytes / t_dec / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"1 {'head' if cfg.mode == 'attn_mq' else 'KV head'} x {n_keys} keys of the "
                   f"{cfg.name} workload, {what}, {reps} repetitions ({t_enc + t_dec:.1f} s): fp64 decode "
                   f"{dec_bytes / t_dec / 1e9:.4f} GB/s; fp64 encode {reps * n_keys / t_enc / 1e6:.4f} Mkeys/s"),
        "encode_mkeys_per_s": reps * n_keys / t_enc / 1e6,
    }


def qjl_bias_study(cfg, dev, n_seeds: int = 64, n_keys: int = 4096):
    """Seed-averaged bias of the QJL and the plain logit estimates on the GPU path.

    For seeds 0..n_seeds-1 (WHT signs and QJL matrix; cb_seed fixed) the same
    bf16 keys of one KV head are encoded and their logits against G query heads
    computed with and without the 1-bit residual term.  bias(q, k) =
    mean_s l^_s - <q, k>; reported as the slope beta = sum bias l / sum l^2
    (mean and standard error over the per-seed slopes) and as the mean and RMS
    of the bias, in units of the RMS exact logit.
    """
    import numpy as np
    import torch

    import rotation_preconditioned_quantization_amd as octo
    import workloads as WL
    kc = cfg.scaled(B=1, Hq=cfg.G, Hkv=1, N=n_keys)
    keys = WL.make_keys(kc, dev, seed=11, n_seq=1, n=n_keys)
    q = WL.make_queries(kc, dev, seed=11)[:, :, 0].contiguous()
    exact = q[0].double().cpu().numpy() @ keys[0].double().cpu().numpy().T   # [G, N]
    ee = float(np.sum(exact * exact))
    slopes = {"qjl": [], "octopus": []}
    acc = {"qjl": np.zeros_like(exact), "octopus": np.zeros_like(exact)}
    t0 = time.perf_counter()
    for s in range(n_seeds):
        cb = octo.Codebook(cfg.d, cfg.b, seed=s, cb_seed=0, qjl=True, device=0)
        cache = octo.Cache(cb, 1, kc.cap, qjl=True)
        octo.octo_encode(cb, keys, cache)
        for name, use in (("qjl", True), ("octopus", False)):
            lg = octo.octo_decode_logits(cb, q, cache, n_keys, 1, use_qjl=use)[0].double().cpu().numpy()
            acc[name] += lg
            slopes[name].append(float(np.sum((lg - exact) * exact)) / ee)
        cb.close()
    rms_l = math.sqrt(ee / exact.size)
    out = {"seeds": n_seeds, "keys": n_keys, "query_heads": cfg.G,
           "seconds": round(time.perf_counter() - t0, 1)}
    for name in ("qjl", "octopus"):
        bias = acc[name] / n_seeds - exact
        sl = np.array(slopes[name])
        out[f"beta_{name}"] = float(sl.mean())
        out[f"beta_{name}_se"] = float(sl.std(ddof=1) / math.sqrt(n_seeds))
        out[f"mean_bias_{name}"] = float(bias.mean() / rms_l)
        out[f"rms_bias_{name}"] = float(math.sqrt(np.mean(bias * bias)) / rms_l)
    return out


def quality_harness(dev, repeats: int = 64, bits=(2, 3, 4)):
    """The pages' synthetic quality experiment on the GPU path ([YL] 实验结果:
    d=128 isotropic Gaussian keys, 1024 random keys and 16 queries, 64 repeats;
    the needle among 2048 random distractors; [YL] 可选的残差修正 for the QJL
    inner products).  Keys go through octo_encode, their reconstruction through
    octo_debug_reconstruct, the inner products through octo_decode_logits.
    Per bit width: normalised MSE E|k - k^|^2/|k|^2, mean cosine(k, k^),
    inner-product error RMS(<q,k^> - <q,k>)/RMS(<q,k>) without and with the
    1-bit QJL term, and the softmax mass (scale 1/sqrt(d)) on the needle when
    the query is the needle key, without and with the QJL term (the exact
    keys' mass beside it).  The
    needle's query and the softmax scale are readings: the pages do not print
    them."""
    import numpy as np
    import torch

    import rotation_preconditioned_quantization_amd as octo
    import workloads as WL
    d = 128
    out = {"repeats": repeats, "keys": 1024, "queries": 16, "distractors": 2048, "d": d,
           "printed": {"mse_b4": 0.0071, "mse_b2": 0.0897, "needle_mass_b2": 0.92}}
    rms = lambda x: float(torch.sqrt(torch.mean(x.double() ** 2)))  # noqa: E731
    for b in bits:
        cb = octo.Codebook(d, b, qjl=True, device=0)
        acc = {k: [] for k in ("mse", "cos", "ip", "ip_qjl", "needle", "needle_qjl", "needle_exact")}
        for r in range(repeats):
            keys, q, nk, nq, pos = WL.make_quality_inputs(dev, seed=r)
            cache = octo.Cache(cb, 1, 1024, qjl=True)
            octo.octo_encode(cb, keys, cache)
            kh = octo.octo_debug_reconstruct(cb, cache, 1024)[0].double()
            kk = keys[0].double()
            acc["mse"].append(float(torch.mean(((kh - kk) ** 2).sum(1) / (kk ** 2).sum(1))))
            acc["cos"].append(float(torch.mean((kh * kk).sum(1) / (kh.norm(dim=1) * kk.norm(dim=1)))))
            exact = q[0].double() @ kk.T
            lg = octo.octo_decode_logits(cb, q, cache, 1024, 1, use_qjl=False)[0].double()
            lq = octo.octo_decode_logits(cb, q, cache, 1024, 1, use_qjl=True)[0].double()
            acc["ip"].append(rms(lg - exact) / rms(exact))
            acc["ip_qjl"].append(rms(lq - exact) / rms(exact))
            ncache = octo.Cache(cb, 1, ((nk.shape[1] + 63) // 64) * 64, qjl=True)
            octo.octo_encode(cb, nk, ncache)
            nl = octo.octo_decode_logits(cb, nq, ncache, nk.shape[1], 1, use_qjl=False)[0, 0].double()
            acc["needle"].append(float(torch.softmax(nl / math.sqrt(d), 0)[pos]))
            nlq = octo.octo_decode_logits(cb, nq, ncache, nk.shape[1], 1, use_qjl=True)[0, 0].double()
            acc["needle_qjl"].append(float(torch.softmax(nlq / math.sqrt(d), 0)[pos]))
            ne = (nq[0, 0].double() @ nk[0].double().T) / math.sqrt(d)
            acc["needle_exact"].append(float(torch.softmax(ne, 0)[pos]))
        cb.close()
        out[f"b{b}"] = {k: round(float(np.mean(v)), 5) for k, v in acc.items()}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate-gib", type=float, default=1.0,
                    help="total size of the rotating input copies")
    ap.add_argument("--kernel-reps", type=int, default=50,
                    help="graph replays used to time each kernel on its own (median)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qjl-bias", action="store_true",
                    help="skip the 64-seed bias study of the QJL workload")
    ap.add_argument("--quality", action="store_true",
                    help="run the pages' synthetic quality experiment on the GPU path and print "
                         "its JSON line (no timing)")
    ap.add_argument("--quality-repeats", type=int, default=64)
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection run for rocprofv3 --pmc: per step a plain copy "
                         "kernel of 64 MiB (the counter scale), then encode and decode, eagerly")
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOADS),
                    help="workload (3 = the extreme-compression shape, the largest d = 128 decode "
                         "on one GPU, which the headline is quoted on; the others are the "
                         "remaining shapes of the pages' workloads)")
    ap.add_argument("--head-dim", type=int, default=0, choices=(0, 64, 128, 256),
                    help="override the workload's head dim (0: keep it)")
    ap.add_argument("--bits", type=int, default=0, choices=(0, 1, 2, 3, 4, 5),
                    help="override the workload's bit budget b (0: keep it)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding of "
                          "the codec is a design note, not a measured path",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import rotation_preconditioned_quantization_amd as octo
    import workloads as WL

    if not torch.cuda.is_available():  # noqa: SIM102
        print(json.dumps({"error": "no GPU"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.quality:
        print(json.dumps({"quality": quality_harness(dev, args.quality_repeats)}), flush=True)
        return
    cfg = WL.CONFIGS[args.config]
    workload = WORKLOADS[args.config]
    if args.head_dim or args.bits:
        cfg = cfg.scaled(d=args.head_dim or cfg.d, b=args.bits or cfg.b)
        workload += f" [overridden: d={cfg.d}, b={cfg.b}]"
    with_joint = True
    cb = octo.Codebook(cfg.d, cfg.b, seed=0, cb_seed=0, qjl=cfg.qjl, device=0)
    lay = cb.layout
    dec_bytes, enc_bytes, n_keys_total = algorithmic_bytes(cfg, lay)
    mq = cfg.mode == "attn_mq"
    logits_mode = cfg.mode == "logits"

    kdt_bytes = 4 if cfg.kdtype == "f32" else 2
    set_bytes = (cfg.n_seq * cfg.cap * cfg.d * kdt_bytes + cb.packed_words(cfg.n_seq, cfg.cap) * 4
                 + cfg.n_seq * cfg.cap * 4)
    if not logits_mode:
        set_bytes += cfg.n_seq * cfg.cap * cfg.d * 2
    R = max(2, int(math.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    mode = 0 if logits_mode else 1
    ws_bytes = cb.workspace_bytes(mode, cfg.B, cfg.Hq, cfg.Hkv, cfg.n_q, cfg.N)
    sets = []
    for r in range(R):
        keys = WL.make_keys(cfg, dev, seed=r)
        v = None if logits_mode else WL.make_values(cfg, dev, seed=r)
        q = WL.make_queries(cfg, dev, seed=r).contiguous()
        if logits_mode:
            q = q[:, :, 0].contiguous()
        cache = octo.Cache(cb, cfg.n_seq, cfg.cap, qjl=cfg.qjl)
        if logits_mode:
            out = torch.empty((cfg.B, cfg.Hq, cfg.N), dtype=torch.float32, device=dev)
        else:
            out = torch.empty((cfg.B, cfg.Hq, cfg.n_q, cfg.d), dtype=torch.float32, device=dev)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        sets.append(dict(keys=keys, v=v, q=q, cache=cache, out=out, ws=ws))

    # the video-block workload encodes only the newest chunk at the end of the cache
    enc_pos0 = cfg.N - cfg.chunk if cfg.chunk else 0
    if cfg.chunk:
        n_keys_total = cfg.n_seq * cfg.chunk
        enc_bytes = n_keys_total * (cfg.d * kdt_bytes + lay.n_triplets * lay.bits_per_triplet / 8 + 4)

    def encode(s):
        k = s["keys"][:, enc_pos0:] if enc_pos0 else s["keys"]
        octo.octo_encode(cb, k, s["cache"], pos0=enc_pos0)

    def decode(s, stages=octo.STAGE_ALL):
        if logits_mode:
            octo.octo_decode_logits(cb, s["q"], s["cache"], cfg.N, cfg.Hkv, logits=s["out"],
                                    workspace=s["ws"], stages=stages & 3)
        else:
            octo.octo_decode_attn(cb, s["q"], s["cache"], s["v"], cfg.N, cfg.Hkv, out=s["out"],
                                  workspace=s["ws"], stages=stages)

    if args.counters:
        # a plain 64 MiB copy with the codec kernels' access pattern: its
        # FETCH_SIZE / WRITE_SIZE readings for known bytes give the counter scale
        src = torch.ones(16 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for s in sets:
            if enc_pos0:
                octo.octo_encode(cb, s["keys"][:, :enc_pos0], s["cache"], pos0=0)
        for k in range(args.steps):
            octo.octo_debug_copy(dst, src)
            encode(sets[k % R])
            decode(sets[k % R])
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "steps": args.steps, "config": args.config,
                          "copy_bytes_each_way": 64 << 20,
                          "kernel_source_hash": kernel_source_hash(cfg.mode)}), flush=True)
        return

    # eager warm-up (the prefix of a chunked cache is encoded once here) and
    # reference outputs
    for s in sets:
        if enc_pos0:
            octo.octo_encode(cb, s["keys"][:, :enc_pos0], s["cache"], pos0=0)
    for i in range(max(1, args.warmup)):
        for s in sets:
            encode(s)
            decode(s)
    torch.cuda.synchronize()
    eager_out = [s["out"].clone() for s in sets]

    side = torch.cuda.Stream()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn()
        return g

    step_graphs = [capture(lambda s=s: (encode(s), decode(s))) for s in sets]
    enc_graph = capture(lambda: [encode(s) for s in sets])
    # the joint-rounding encoder mode (reported beside the scalar encoder, not
    # part of the step): into a scratch cache per set
    jcaches = [octo.Cache(cb, cfg.n_seq, cfg.cap, qjl=cfg.qjl) for _ in sets]

    def encode_joint(s, jc):
        k = s["keys"][:, enc_pos0:] if enc_pos0 else s["keys"]
        octo.octo_encode_joint(cb, k, jc, pos0=enc_pos0)

    if with_joint:
        joint_graph = capture(lambda: [encode_joint(s, jc) for s, jc in zip(sets, jcaches)])
    # the autoregressive step (single-query attention workloads): append the
    # newest key of every sequence at position N - 1, then attend over N keys
    step_append = cfg.mode == "attn"
    if step_append:
        for s in sets:
            s["new_key"] = s["keys"][:, cfg.N - 1].contiguous()

        def append_step(s):
            octo.octo_decode_attn_append(cb, s["new_key"], s["q"], s["cache"], s["v"], cfg.N,
                                         cfg.Hkv, out=s["out"], workspace=s["ws"])

        def append_encode(s):
            octo.octo_encode(cb, s["new_key"].view(cfg.n_seq, 1, cfg.d), s["cache"], pos0=cfg.N - 1)

        app_graph = capture(lambda: [append_step(s) for s in sets])
        app_enc_graph = capture(lambda: [append_encode(s) for s in sets])
    dec_graph = capture(lambda: [decode(s) for s in sets])
    main_graph = capture(lambda: [decode(s, octo.STAGE_MAIN) for s in sets])
    torch.cuda.synchronize()
    # each replay must reproduce the eager result (checked on every set once)
    for r, g in enumerate(step_graphs):
        sets[r]["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(sets[r]["out"], eager_out[r]):
            raise RuntimeError(f"graph replay of step {r} differs from the eager result")

    means = []  # the mean replay time of each time_graph call, in call order

    def time_graph(g, reps, warm=5, per=4):
        """One replay's time: the median over `reps` samples (after `warm`
        untimed replays), a sample being `per` back-to-back replays between two
        HIP events on the graph's stream (an event between every replay would
        add its own cost to each)."""
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        with torch.cuda.stream(side):
            for _ in range(warm):
                g.replay()
            evs[0].record(side)
            for i in range(reps):
                for _ in range(per):
                    g.replay()
                evs[i + 1].record(side)
        torch.cuda.synchronize()
        ts = [evs[i].elapsed_time(evs[i + 1]) / per for i in range(reps)]
        means.append(sum(ts) / reps / 1e3)
        return statistics.median(ts) / 1e3

    t_enc = time_graph(enc_graph, args.kernel_reps) / R
    t_joint = time_graph(joint_graph, max(1, args.kernel_reps // 4)) / R if with_joint else None
    if step_append:
        t_app = time_graph(app_graph, args.kernel_reps) / R
        t_app_enc = time_graph(app_enc_graph, args.kernel_reps) / R
    t_dec = time_graph(dec_graph, args.kernel_reps) / R
    t_dec_mean = means[-1] / R
    t_main = time_graph(main_graph, args.kernel_reps) / R
    t_main_mean = means[-1] / R

    # timed region: exactly K steps
    for w in range(args.warmup):
        step_graphs[w % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_graphs[k % R].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    dec_gbs = dec_bytes / t_dec / 1e9
    main_gbs = dec_bytes / t_main / 1e9
    traffic = None if (args.head_dim or args.bits) else profiled_traffic(cfg)
    kernel_name = {"logits": "k_logits (fused compressed-K logits)",
                   "attn": "k_attn (fused decode attention)",
                   "attn_mq": "k_mq_attn (multi-query MFMA attention)"}[cfg.mode]
    roofline = {"bound": "hbm", "kernel": kernel_name, "achieved": round(main_gbs, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(main_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel_us": round(t_main * 1e6, 3),
                "algorithmic_bytes_per_launch": int(dec_bytes)}
    if mq:
        flops = 4.0 * cfg.B * cfg.Hq * cfg.n_q * cfg.N * cfg.d
        tf = flops / t_main / 1e12
        roofline = {"bound": "mfma", "kernel": kernel_name, "achieved": round(tf, 2),
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "kernel_us": round(t_main * 1e6, 3), "algorithmic_flops_per_launch": int(flops),
                    "hbm_gbs": round(main_gbs, 2)}

    line = {
        "metric": f"fused compressed-K decode GB/s (% HBM peak) + encode Mkeys/s, d={cfg.d}",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.kdtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": cfg.B, "seq_len": cfg.N,
                   "parallelism": "none (1 GPU)", "rotating_copies": R},
        "pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "decode_us": round(t_dec * 1e6, 3),
        "decode_us_mean": round(t_dec_mean * 1e6, 3),
        "kernel_us_mean": round(t_main_mean * 1e6, 3),
        "encode_mkeys_per_s": round(n_keys_total / t_enc / 1e6, 1),
        "encode_gbs": round(enc_bytes / t_enc / 1e9, 2),
        "encode_us": round(t_enc * 1e6, 3),
        "encode_pct_hbm_peak": round(100 * enc_bytes / t_enc / 1e9 / HBM_PEAK_GBS, 2),
        **({"encode_joint_us": round(t_joint * 1e6, 3),
            "encode_joint_mkeys_per_s": round(n_keys_total / t_joint / 1e6, 1)} if with_joint else {}),
        **({"append_step_us": round(t_app * 1e6, 3), "append_encode_us": round(t_app_enc * 1e6, 3),
            "append_keys_per_step": cfg.n_seq} if step_append else {}),
        "roofline": roofline,
    }
    if cfg.qjl and not args.no_qjl_bias:
        line["qjl_bias"] = qjl_bias_study(cfg, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
