"""Benchmark of the packed-QKV split + per-head RMSNorm + RoPE path on one MI355X.

One step = one training layer of the Qwen3-8B-like sectioned workload at
T = 16384 tokens: ``qkvnr_forward`` (split, q/k RMSNorm, RoPE, v copy) then
``qkvnr_backward`` (inverse RoPE, RMSNorm backward, packed dqkv, norm-weight
grads), bf16, inputs resident in HBM.  ``value`` is algorithmic bytes per step
(each input byte read once, each output byte written once; the backward's
re-read of the packed input counts) divided by the step's wall time: HBM GB/s.

Cache hygiene: MI355X has a 256 MB Infinity Cache and one step touches
~0.97 GB.  Three buffer sets rotate: step i runs the forward on set i mod 3 and
the backward on set (i - 1) mod 3 (a batch whose forward ran a step earlier,
as in a model where other layers run between a layer's forward and backward),
so no read finds data left in the cache by the previous ~0.97 GB of traffic.

Clock settling: an idle GPU takes tens of milliseconds to reach its working
clocks.  Before the counted ``--warmup`` steps, full steps run until the clocks
have settled (at least 250 ms, then until two successive 25-step batches agree
within 1 %, at most 3 s); the JSON line reports how long (``settle``).  The
timed region is exactly ``--steps`` steps either way.

Also reported (``extras``, legs chosen with ``--legs``): Muse-Spark decode at
T = 1/8/64/256 (HIP-graph replays, us per call), Muse prefill at T = 16384 as a
RoPE and a NoPE layer (us, GB/s), the MLA latent paged store (us), the MLA
drafter layer's schedules, per-head Newton-Schulz and the fused projection.
The CPU oracle runs first, on one host core and on all of them, on bounded
samples of every workload (``cpu_baseline``; its us per layer also sit beside
each GPU figure in ``extras`` as ``*_oracle_us``).

Prints one JSON line.  Only one GPU: ``--gpus`` above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "qkv split+norm+RoPE µs/layer & HBM GB/s (% peak): T=16k fwd+bwd, T=1 decode"
KERNEL_SOURCES = ["qkv_split_head_amd/csrc/kernels.h", "qkv_split_head_amd/csrc/device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_gqa_bf16_d128_train16k_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def gqa_bytes(T, n_q, n_kv, D, es, rope=True):
    """Algorithmic bytes: forward reads the packed row and writes q/k/v; backward reads
    the q/k slots of the packed row, dq/dk/dv, and writes the packed dqkv."""
    row = (n_q + 2 * n_kv) * D * es
    fwd = 2 * row * T
    bwd = ((n_q + n_kv) * D * es + 2 * row) * T
    return fwd, bwd


def traffic_from_profile():
    """HBM bytes per backward launch from the committed rocprofv3 counter summary, or None
    if it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- CPU oracle baseline

# The oracle's sample of each workload: the generator's batch of the same shape
# (the training and prefill configs: its first 2048 tokens, positions 0..2047),
# keyed by the name its GPU figure has in ``extras``.
_CPU_W = {}
_CPU_CHUNK = 256


def _cpu_workloads():
    from qkv_inputs import decode_interleaved, latent_paged, prefill_interleaved, train_sectioned

    w = {"train_fwd_plus_bwd": train_sectioned(2048),
         "prefill_rope": prefill_interleaved(2048, rope=True),
         "prefill_nope": prefill_interleaved(2048, rope=False)}
    for T in (1, 8, 64, 256):
        w[f"decode_T{T}"] = decode_interleaved(T)
    w["mla_latent_paged_B4xT16"] = latent_paged()
    return w


def _oracle_gqa(name, t0, t1):
    """The oracle's path over tokens [t0, t1) of a GQA workload: outputs rounded once to bf16
    (forward), and for the training config also the backward's packed grad."""
    import oracle

    w = _CPU_W[name]
    sl = slice(t0, t1)
    rope = w.rope_dim > 0
    q64, k64, _ = oracle.forward_gqa(w.qkv[sl], w.dtype, w.kind, w.n_kv, w.q_per_kv, w.head_dim, w.positions[sl],
                                     w.q_norm_w, w.k_norm_w, w.eps, w.theta, rope=rope)
    oracle.round_to_storage(q64, w.dtype)
    oracle.round_to_storage(k64, w.dtype)
    if w.dq is not None:
        ref = oracle.backward_gqa(w.qkv[sl], w.dtype, w.kind, w.n_kv, w.q_per_kv, w.head_dim, w.positions[sl],
                                  w.q_norm_w, w.k_norm_w, w.eps, w.theta, w.dq[sl], w.dk[sl], w.dv[sl], rope=rope)
        oracle.round_to_storage(ref["dqkv64"], w.dtype)
    return t1 - t0


def _oracle_latent_rows(t0, t1):
    import oracle

    w = _CPU_W["mla_latent_paged_B4xT16"]
    rows = oracle.latent_forward(w.qkv[t0:t1], "bf16", w.positions[t0:t1], w.k_norm_w, w.eps, w.theta, 512, 64)
    return oracle.round_to_storage(rows, "bf16")


def _oracle_latent_store(pool, rows):
    import oracle

    w = _CPU_W["mla_latent_paged_B4xT16"]
    page, off = oracle.paged_slots(w.positions, w.block_table, w.tokens_per_req, w.page_size)
    return oracle.staged_then_scatter(pool, rows, page, off)


def _timed_chunks(name, first_chunk, target_s):
    """Chunks of _CPU_CHUNK tokens (cycling over the sample from `first_chunk` on) for
    about target_s of wall time; returns (tokens, seconds)."""
    T = _CPU_W[name].T
    n_chunks = T // _CPU_CHUNK
    done, i = 0, first_chunk
    t0 = time.perf_counter()
    while True:
        c = i % n_chunks
        done += _oracle_gqa(name, c * _CPU_CHUNK, (c + 1) * _CPU_CHUNK)
        i += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            return done, el


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(target_s: float = 2.5, reps: int = 5):
    """The oracle (NumPy fp64) on a bounded sample of every workload, on one host core and on
    all of this process's host cores (token shards over one forked worker process per core,
    at most 16), in the same run as the GPU figures.

    Large workloads (training fwd+bwd, prefill): 256-token chunks for about target_s each way,
    scaled to us per 16384-token layer.  Small workloads (decode, the MLA paged store): the
    median of `reps` calls on the whole batch.  Runs before the GPU is touched, so the workers
    are forked from a process that has not initialised HIP.
    """
    import multiprocessing as mp
    import statistics

    from threadpoolctl import threadpool_limits

    import oracle  # noqa: F401  (imported once here, inherited by the forked workers)

    _CPU_W.update(_cpu_workloads())
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    fwd_b, bwd_b = gqa_bytes(1, 32, 8, 128, 2)
    out = {}
    with threadpool_limits(1), mp.get_context("fork").Pool(cores) as pool:
        pool.starmap(_oracle_gqa, [("decode_T1", 0, 1)] * cores)  # every worker up and importing
        for name in ("train_fwd_plus_bwd", "prefill_rope", "prefill_nope"):
            tok1, el1 = _timed_chunks(name, 0, target_s)
            res = pool.starmap(_timed_chunks, [(name, i, target_s) for i in range(cores)])
            tokn, eln = sum(r[0] for r in res), max(r[1] for r in res)
            out[name] = {"1_core": round(el1 / tok1 * 16384 * 1e6, 1),
                         f"{cores}_cores": round(eln / tokn * 16384 * 1e6, 1),
                         "tokens_1_core": tok1, f"tokens_{cores}_cores": tokn}
        for T in (1, 8, 64, 256):
            name = f"decode_T{T}"
            shards = [(name, T * i // min(cores, T), T * (i + 1) // min(cores, T)) for i in range(min(cores, T))]
            one, many = [], []
            for _ in range(reps):
                t0 = time.perf_counter()
                _oracle_gqa(name, 0, T)
                one.append(time.perf_counter() - t0)
                t0 = time.perf_counter()
                pool.starmap(_oracle_gqa, shards)
                many.append(time.perf_counter() - t0)
            out[name] = {"1_core": round(statistics.median(one) * 1e6, 1),
                         f"{cores}_cores": round(statistics.median(many) * 1e6, 1)}
        lw = _CPU_W["mla_latent_paged_B4xT16"]
        lpool = np.zeros((lw.num_pages, lw.page_size, 576), dtype=np.uint16)
        shards = [(lw.T * i // cores, lw.T * (i + 1) // cores) for i in range(cores)]
        one, many = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            _oracle_latent_store(lpool, _oracle_latent_rows(0, lw.T))
            one.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            _oracle_latent_store(lpool, np.concatenate(pool.starmap(_oracle_latent_rows, shards)))
            many.append(time.perf_counter() - t0)
        out["mla_latent_paged_B4xT16"] = {"1_core": round(statistics.median(one) * 1e6, 1),
                                          f"{cores}_cores": round(statistics.median(many) * 1e6, 1)}
    step_b = fwd_b + bwd_b
    tr = out["train_fwd_plus_bwd"]
    return {
        "value": round(step_b * 16384 / (tr[f"{cores}_cores"] * 1e-6) / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"training fwd+bwd (sectioned 32q/8kv/D128 bf16): {tr[f'tokens_{cores}_cores']} tokens in "
                   f"256-token chunks of the generator's 2048-token batch over {cores} forked processes, "
                   f"~{target_s:.1f} s; also prefill RoPE/NoPE the same way, decode T=1/8/64/256 and the MLA "
                   f"paged store (median of {reps} calls); NumPy fp64, BLAS limited to 1 thread per process"),
        "cpu_model": _cpu_model(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "single_core": {"value": round(step_b * 16384 / (tr["1_core"] * 1e-6) / 1e9, 4), "unit": "GB/s",
                        "cores": 1},
        "us_per_layer": out,
    }


def drafter_extras(dev_bf16, stream, layers_n: int = 4, n: int = 30):
    """Per-layer decode-step time of a 4-layer MLA drafter step (distinct weights and
    pools per layer, DeepSeek-V3-style shapes at one rank's share of TP8) under HIP
    graph replay: serial, split (kv path on a second stream, fork/join) or merged
    (one q_a|kv_a projection, one stream) schedules, direct or staged pool write,
    B = 1 and 4 requests of 16 draft tokens.  Latency-bound: microseconds, no
    bandwidth figure."""
    import torch
    from qkv_inputs import mla_drafter_layer
    from qkv_split_head_amd.mla_drafter import MlaDims, MlaDrafterLayer, staged_slots

    names = ("w_input_ln", "w_q_a", "w_q_a_ln", "w_q_b", "w_uk", "w_kv_a", "w_kv_a_ln")
    ins = [mla_drafter_layer(4, 16, seed=70 + i) for i in range(layers_n)]
    layers = [MlaDrafterLayer({k: dev_bf16(getattr(m, k)) for k in names}, MlaDims()) for m in ins]
    pools = [torch.zeros((m.num_pages, m.page_size, 576), dtype=torch.bfloat16, device="cuda") for m in ins]
    out = {"layers_per_step": layers_n, "graph_replays": n}
    for B in (1, 4):
        m0 = ins[0]
        x = dev_bf16(m0.x[:B * 16])
        pos = torch.from_numpy(m0.positions[:B * 16]).cuda()
        bt = torch.from_numpy(m0.block_table[:B]).cuda()
        res = {}
        for split, merge in ((False, False), (True, False), (False, True)):
            for direct in (False, True):
                def step():
                    # the staged write's slots: once per step, shared by the layers
                    slots = None if direct else staged_slots(pos, bt, 16, 64, pools[0].shape[0] * 64)
                    for lay, pool in zip(layers, pools):
                        lay.forward(x, pos, bt, pool, 16, split_streams=split, direct_pool_write=direct,
                                    merge_kv_a=merge, slots=slots)
                side = torch.cuda.Stream()
                side.wait_stream(stream)
                with torch.cuda.stream(side):
                    for _ in range(2):
                        step()
                stream.wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step()
                for _ in range(5):
                    g.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                key = ("split" if split else "merged" if merge else "serial") + ("_direct" if direct else "_staged")
                res[key] = round(e0.elapsed_time(e1) / (n * layers_n) * 1e3, 2)
                del g
        res["split_streams_saving_us"] = round(res["serial_direct"] - res["split_direct"], 2)
        res["merged_projection_saving_us"] = round(res["serial_direct"] - res["merged_direct"], 2)
        res["direct_write_saving_us"] = round(res["serial_staged"] - res["serial_direct"], 2)
        out[f"B{B}_us_per_layer"] = res
    return out


def muon_extras(stream, n: int = 10):
    """One Muon orthogonalisation (5 quintic Newton-Schulz steps) of the Qwen3-8B-like fused
    q|k|v weight [6144, 4096] (seeded N(0,1)): per head (48 blocks of 128 rows) in bf16 (one launch a
    step) and fp32, and on the whole matrix in bf16 (the full-matrix path, library products only)."""
    import torch
    from qkv_split_head_amd.muon import per_head_newton_schulz

    g = torch.Generator(device="cuda").manual_seed(80)
    G = torch.randn((6144, 4096), generator=g, device="cuda").to(torch.bfloat16)
    a, b_, c = 3.4445, -4.7750, 2.0315

    def full_matrix():
        X = G.t().contiguous()                    # wide orientation [4096, 6144]
        X = X / (X.float().norm() + 1e-7).to(X.dtype)
        for _ in range(5):
            A = X @ X.t().contiguous()
            X = a * X + (b_ * A + c * (A @ A)) @ X
        return X.t() * (6144 / 4096) ** 0.5

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / n * 1e3, 1)

    out = {
        "weight": [6144, 4096], "head_blocks": 48, "steps": 5,
        "per_head_bf16_us": timed(lambda: per_head_newton_schulz(G, 32, 8, 128)),
        "per_head_fp32_us": timed(lambda: per_head_newton_schulz(G, 32, 8, 128, compute_dtype=torch.float32)),
        "full_matrix_bf16_us": timed(full_matrix),
    }
    # HBM bytes of the collapsed bf16 path: G read twice (Gram, apply) and Y written once, the fp32 Gram
    # partials (48 blocks x 5 slices) written and read once, M (two bf16 terms) written and read once
    nbytes = 3 * 48 * 128 * 4096 * 2 + 2 * 48 * 5 * 128 * 128 * 4 + 2 * 48 * 2 * 128 * 128 * 2
    out["per_head_bf16_hbm_bytes"] = nbytes
    out["per_head_bf16_GBps"] = round(nbytes / (out["per_head_bf16_us"] * 1e-6) / 1e9, 1)
    return out


def proj_extras(stream, n: int = 20):
    """The QKV projection of the Qwen3-8B-like training layer (x [16384, 4096] @ w_qkv[6144, 4096]^T, bf16)
    with split + q/k RMSNorm + RoPE fused into its epilogue, against the library GEMM followed by the
    region's forward, and the library GEMM alone.  MFMA-bound: 2 T hidden width flops."""
    import torch
    import torch.nn.functional as F
    import qkv_split_head_amd as qk

    T, H, n_kv, Q, D = 16384, 4096, 8, 4, 128
    W = (n_kv * Q + 2 * n_kv) * D
    g = torch.Generator(device="cuda").manual_seed(81)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((W, H), generator=g, device="cuda") * H ** -0.5).to(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    wq = (1.0 + 0.1 * torch.randn(D, generator=g, device="cuda")).to(torch.bfloat16)
    wk = (1.0 + 0.1 * torch.randn(D, generator=g, device="cuda")).to(torch.bfloat16)
    shapes = ((T, n_kv * Q, D), (T, n_kv, D), (T, n_kv, D))
    out = tuple(torch.empty(sh, dtype=torch.bfloat16, device="cuda") for sh in shapes)
    out2 = tuple(torch.empty(sh, dtype=torch.bfloat16, device="cuda") for sh in shapes)
    kw = dict(kind="sectioned", n_kv=n_kv, q_per_kv=Q, head_dim=D, theta=1e6)

    def fused():
        qk.proj_forward(x, w, pos, wq, wk, out=out, stream=stream, **kw)

    def unfused():
        qk.forward(F.linear(x, w), pos, wq, wk, out=out2, stream=stream, **kw)

    def gemm():
        F.linear(x, w)

    def timed(fn):
        for _ in range(10):  # about 8 ms of warm-up: the clocks of an idle GPU take that long to come up
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / n * 1e3, 1)

    timed(gemm)  # warm-up of the whole set first
    res = {"shape": [T, H, W], "gemm_alone_us": timed(gemm), "gemm_then_region_us": timed(unfused),
           "fused_us": timed(fused)}
    flops = 2 * T * H * W
    res["fused_TFLOPs"] = round(flops / (res["fused_us"] * 1e-6) / 1e12, 1)
    res["fused_frac_of_bf16_mfma_peak"] = round(flops / (res["fused_us"] * 1e-6) / 2.5e15, 3)
    res["gemm_alone_TFLOPs"] = round(flops / (res["gemm_alone_us"] * 1e-6) / 1e12, 1)
    return res


LEGS = ("prefill", "decode", "mla", "drafter", "muon", "proj")


def settle_clocks(step, min_ms: float = 250.0, max_ms: float = 3000.0, batch: int = 25, tol: float = 0.01):
    """Runs full steps until the GPU's clocks have settled: at least min_ms of back-to-back
    steps, then until two successive batches of `batch` steps agree within `tol` (at most
    max_ms).  An idle GPU takes tens of milliseconds to reach its working clocks, so a
    handful of warm-up steps would time the ramp.  Returns (ms, steps, last batch's ms/step)."""
    import torch

    t_start = time.perf_counter()
    prev, n = None, 0
    while True:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(batch):
            step(n)
            n += 1
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / batch
        el = (time.perf_counter() - t_start) * 1e3
        if el >= max_ms or (el >= min_ms and prev is not None and abs(per - prev) <= tol * prev):
            return el, n, per * 1e3
        prev = per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--legs", default="all",
                    help="comma list of extra legs after the training step: " + ",".join(LEGS) + " (or all, none)")
    ap.add_argument("--no-extras", action="store_true", help="only the training step (same as --legs none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="minimum clock-settling time before the warm-up steps (0: none, e.g. for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy exactly 256 MiB device-to-device 3 times (a known-size reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    legs = set(LEGS) if args.legs == "all" else set() if args.legs == "none" else set(args.legs.split(","))
    if legs - set(LEGS):
        ap.error(f"unknown legs {sorted(legs - set(LEGS))}")
    if args.no_extras:
        legs = set()

    # the oracle first: its worker processes are forked before this process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline()

    import torch

    import qkv_split_head_amd as qk
    from qkv_inputs import decode_interleaved, latent_paged, prefill_interleaved, train_sectioned

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda"

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- training step (T = 16k)
    T, n_q, n_kv, D = 16384, 32, 8, 128
    w = train_sectioned(T)
    base = dict(qkv=dev_bf16(w.qkv), dq=dev_bf16(w.dq), dk=dev_bf16(w.dk), dv=dev_bf16(w.dv))
    pos = torch.from_numpy(w.positions).to(dev)
    wq, wk = dev_bf16(w.q_norm_w), dev_bf16(w.k_norm_w)
    del w
    sets = []
    for i in range(3):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        s["q"] = torch.empty((T, n_q, D), dtype=torch.bfloat16, device=dev)
        s["k"] = torch.empty((T, n_kv, D), dtype=torch.bfloat16, device=dev)
        s["v"] = torch.empty((T, n_kv, D), dtype=torch.bfloat16, device=dev)
        s["dqkv"] = torch.empty_like(s["qkv"])
        s["dwq"] = torch.empty(D, dtype=torch.float32, device=dev)
        s["dwk"] = torch.empty(D, dtype=torch.float32, device=dev)
        sets.append(s)
    kw = dict(kind="sectioned", n_kv=n_kv, q_per_kv=n_q // n_kv, head_dim=D, eps=1e-6, theta=1e6)
    stream = torch.cuda.current_stream()
    # Each buffer set goes once through the tensor-level wrappers, which check every tensor's
    # device, dtype and shape.  The steps then call the same C entry points through the raw
    # binding with those tensors' addresses (the library still validates every call on the
    # host), so the host's submission time per step is lower than the GPU's.
    for s in sets:
        qk.forward(s["qkv"], pos, wq, wk, out=(s["q"], s["k"], s["v"]), **kw)
        qk.backward(s["qkv"], pos, wq, wk, s["dq"], s["dk"], s["dv"], out=(s["dqkv"], s["dwq"], s["dwk"]), **kw)
    torch.cuda.synchronize()
    layout = qk.gqa_layout(base["qkv"], "sectioned", n_kv, n_q // n_kv, D, True)
    workspace = qk.backward_workspace()
    ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    sp, pp, wqp, wkp = stream.cuda_stream, pos.data_ptr(), wq.data_ptr(), wk.data_ptr()
    addr = [{k: v.data_ptr() for k, v in s.items()} for s in sets]

    def fwd(i):
        a = addr[i % 3]
        qk.qkvnr_forward(layout, a["qkv"], pp, wqp, wkp, 1e-6, 1e6, a["q"], a["k"], a["v"], sp)

    def bwd(i):
        a = addr[i % 3]
        qk.qkvnr_backward(layout, a["qkv"], pp, wqp, wkp, 1e-6, 1e6, a["dq"], a["dk"], a["dv"], a["dqkv"], a["dwq"],
                          a["dwk"], ws_ptr, ws_bytes, sp)

    def step(i):
        fwd(i)
        bwd(i - 1)

    settle_ms, settle_steps, settle_last = (settle_clocks(step, min_ms=args.settle_ms) if args.settle_ms > 0
                                            else (0.0, 0, 0.0))
    for i in range(args.warmup):
        step(i)

    # the timed region: exactly K steps, nothing else enqueued between them
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-kernel launch durations, live in the same run: HIP events on the
    # launch stream around K back-to-back launches of one kernel, same rotation
    def per_launch_ms(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    fwd_ms = per_launch_ms(fwd, K)
    bwd_ms = per_launch_ms(bwd, K)
    # practical ceiling beside the 8 TB/s figure: the runtime's device copy of
    # the packed input (the forward's byte count: read + write), same rotation
    copy_ms = per_launch_ms(lambda i: sets[i % 3]["dqkv"].copy_(sets[(i + 1) % 3]["qkv"]), K)
    fwd_b, bwd_b = gqa_bytes(T, n_q, n_kv, D, 2)
    ms_per_step = wall / K * 1e3
    value = (fwd_b + bwd_b) / (ms_per_step * 1e-3) / 1e9
    bwd_gbs = bwd_b / (bwd_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()
    del sets, base

    extras = {
        "train_fwd_us": round(fwd_ms * 1e3, 2),
        "train_fwd_GBps": round(fwd_b / (fwd_ms * 1e-3) / 1e9, 1),
        "train_bwd_us": round(bwd_ms * 1e3, 2),
        "train_bwd_GBps": round(bwd_gbs, 1),
        "train_fwd_plus_bwd_us": round((fwd_ms + bwd_ms) * 1e3, 2),
        "train_algorithmic_bytes": {"fwd": fwd_b, "bwd": bwd_b},
        "copy_ceiling_us": round(copy_ms * 1e3, 2),
        "copy_ceiling_GBps": round(fwd_b / (copy_ms * 1e-3) / 1e9, 1),
    }

    if "prefill" in legs:
        # ------------------------------------------------------------ Muse prefill, RoPE and NoPE layers
        for rope in (True, False):
            pw = prefill_interleaved(16384, rope=rope)
            pq = dev_bf16(pw.qkv)
            pp = torch.from_numpy(pw.positions).to(dev)
            pwq, pwk = dev_bf16(pw.q_norm_w), dev_bf16(pw.k_norm_w)
            pk = dict(kind="interleaved", n_kv=16, q_per_kv=8, head_dim=64, rope=rope, eps=1e-6, theta=5e5)
            bufs = [(pq if i == 0 else pq.clone()) for i in range(2)]
            outs = [(torch.empty((16384, 128, 64), dtype=torch.bfloat16, device=dev),
                     torch.empty((16384, 16, 64), dtype=torch.bfloat16, device=dev),
                     torch.empty((16384, 16, 64), dtype=torch.bfloat16, device=dev)) for _ in range(2)]
            for i in range(4):
                qk.forward(bufs[i % 2], pp, pwq, pwk, out=outs[i % 2], **pk)
            n = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                qk.forward(bufs[i % 2], pp, pwq, pwk, out=outs[i % 2], **pk)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            pb, _ = gqa_bytes(16384, 128, 16, 64, 2)
            tag = "rope" if rope else "nope"
            extras[f"prefill_{tag}_us"] = round(us, 2)
            extras[f"prefill_{tag}_GBps"] = round(pb / (us * 1e-6) / 1e9, 1)
            del bufs, outs, pq

    # ------------------------------------------------------------ decode, HIP-graph replays
    CALLS = 32  # forward calls per graph in the latency-bound legs
    if "decode" in legs:
        # one graph holds CALLS forward calls (as a decode step holds every layer's), so the
        # per-call figure is GPU time plus the in-graph launch gap, not host submission
        for Td in (1, 8, 64, 256):
            dw = decode_interleaved(Td)
            dq_ = dev_bf16(dw.qkv)
            dp = torch.from_numpy(dw.positions).to(dev)
            dwq_, dwk_ = dev_bf16(dw.q_norm_w), dev_bf16(dw.k_norm_w)
            o = (torch.empty((Td, 128, 64), dtype=torch.bfloat16, device=dev),
                 torch.empty((Td, 16, 64), dtype=torch.bfloat16, device=dev),
                 torch.empty((Td, 16, 64), dtype=torch.bfloat16, device=dev))
            dk_ = dict(kind="interleaved", n_kv=16, q_per_kv=8, head_dim=64, eps=1e-6, theta=5e5)
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for _ in range(3):
                    qk.forward(dq_, dp, dwq_, dwk_, out=o, **dk_)
            stream.wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(CALLS):
                    qk.forward(dq_, dp, dwq_, dwk_, out=o, **dk_)
            for _ in range(5):
                g.replay()
            n = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            extras[f"decode_T{Td}_us"] = round(e0.elapsed_time(e1) / (n * CALLS) * 1e3, 2)
            del g

    # ------------------------------------------------------------ MLA latent rows into the paged pool
    if "mla" in legs:
        lw = latent_paged()
        rows, lp, lwk = dev_bf16(lw.qkv), torch.from_numpy(lw.positions).to(dev), dev_bf16(lw.k_norm_w)
        bt = torch.from_numpy(lw.block_table).to(dev)
        pool = torch.zeros((lw.num_pages, lw.page_size, 576), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            qk.forward_latent_paged(rows, lp, lwk, bt, pool, tokens_per_req=lw.tokens_per_req)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(CALLS):
                qk.forward_latent_paged(rows, lp, lwk, bt, pool, tokens_per_req=lw.tokens_per_req)
        for _ in range(5):
            g.replay()
        n = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        extras["mla_latent_paged_B4xT16_us"] = round(e0.elapsed_time(e1) / (n * CALLS) * 1e3, 2)
        del pool, g

    # ------------------------------------------------------------ MLA drafter layers: kv path beside q path
    if "drafter" in legs:
        extras["mla_drafter"] = drafter_extras(dev_bf16, stream)

    # ------------------------------------------------------------ per-head Newton-Schulz on the fused weight
    if "muon" in legs:
        extras["muon_newton_schulz"] = muon_extras(stream)

    # ------------------------------------------------------------ QKV projection with the region in its epilogue
    if "proj" in legs:
        extras["fused_qkv_projection"] = proj_extras(stream)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        # before the counted warm-up: full steps until the clocks settled (not timed, not counted)
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps,
                   "last_batch_us_per_step": round(settle_last * 1e3, 2)},
        "ms_per_step": round(ms_per_step, 4),
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(1,0.1) norm weights)",
        "config": {
            "workload": "Qwen3-8B-like training layer, sectioned packed qkv [16384, (32+8+8)*128] bf16, "
                        "q/k RMSNorm + RoPE theta 1e6, forward + backward",
            "tokens": T, "n_q": n_q, "n_kv": n_kv, "head_dim": D, "layout": "sectioned",
            "buffer_sets_rotated": 3,
        },
        "roofline": {
            "kernel": "one qkvnr_backward call: bwd_gqa_kernel<bf16, D=128, RoPE> + its one-block weight-grad fold "
                      "(wgrad_fold_kernel), HIP events over the per-launch loop",
            "bound": "hbm",
            "achieved": round(bwd_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(bwd_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "extras": extras,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
        # the oracle's time beside each GPU figure it matches
        for name, t in cpu["us_per_layer"].items():
            extras[f"{name}_oracle_us"] = {k: v for k, v in t.items() if not k.startswith("tokens")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
