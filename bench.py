"""Benchmark: masked attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--cold]
                    [--prewarm-ms MS]

One step is one fa_fwd call (fa_fwd_paged with --block-size) over the whole workload (inputs
already resident in HBM). The metric is effective TFLOP/s: 4 * D flops per visible (query,
key) pair, summed over batches and heads, divided by the step time; masked or skipped work
is never counted. The visible
pair count comes from the library's mask probe (checked bit-exactly against the oracle by
the test suite) and is cross-checked against a closed form where one exists.

Prints one JSON line. Timing uses HIP events recorded on the stream fa_fwd is launched on
(torch's current stream). Before the counted warm-up steps, untimed steps run for --prewarm-ms
of wall time (default 500): the GPU raises its clock over the first tens of milliseconds of load,
so without them a short timed region measures the ramp rather than the sustained rate. The CPU baseline times the fp64 oracle on a bounded sample of
the same workload (a few whole heads) on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
# Sources that decide the dominant kernel's memory traffic (its code and its launch order).
KERNEL_SOURCES = ["masked_attention_forward_amd/csrc/fa_kernels.hip",
                  "masked_attention_forward_amd/csrc/fa_fwd_ps.hip",
                  "masked_attention_forward_amd/csrc/fa_fwd_common.h",
                  "masked_attention_forward_amd/csrc/fa_mask.h",
                  "masked_attention_forward_amd/csrc/fa_plan.cpp",
                  "masked_attention_forward_amd/csrc/fa_plan.h"]
DOMINANT_KERNEL = "fa_fwd_pp"
DECODE_KERNEL = "fa_decode_split"
METRIC = "effective TFLOP/s (unmasked FLOPs) attn fwd bf16 D=128; % of MFMA peak"
DECODE_METRIC = "effective HBM GB/s attn decode (Q, K, V read once, O and LSE written once)"


SCATTER_SOURCES = ["masked_attention_forward_amd/csrc/fa_kv_cache.hip"]


def kernel_sources_sha(sources=None) -> str:
    """Hash of the code lines of `sources` (KERNEL_SOURCES by default; full-line comments and
    blank lines skipped, so a comment edit does not invalidate recorded counters; any code
    change does)."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            for line in f:
                t = line.strip()
                if t and not t.startswith(b"//"):
                    h.update(t + b"\n")
    return h.hexdigest()[:16]


def prewarm(step, ms_target: float) -> int:
    """Untimed steps for about `ms_target` ms of wall time, before the counted warm-up steps.

    After idle the GPU raises its clock over the first tens of milliseconds of load: measured on
    the causal 8192 prefill, launches in the first 40 ms after a 1 s pause ran 7% slower than from
    80 ms on, where the rate then held for seconds. A few counted warm-up steps of a short workload
    end inside that ramp, so the timed steps would measure it rather than the sustained rate.
    Steps go out in chunks of about 20 ms with a synchronize after each. Returns the step count."""
    import torch

    if ms_target <= 0:
        return 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    chunk = max(1, int(20.0 / max((time.perf_counter() - t0) * 1e3, 1e-3)))
    n = 1
    while (time.perf_counter() - t0) * 1e3 < ms_target:
        for _ in range(chunk):
            step()
        torch.cuda.synchronize()
        n += chunk
    return n


def recorded_traffic(workload: str, path=None, sources=None, kernel=DOMINANT_KERNEL):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = path or os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_sources_sha(sources):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def visible_pairs(w, dev):
    """(visible (row, key) pairs summed over batches and heads, scores the forward kernel
    computes): the second is every entry of every tile it visits, from the same device mask
    code (fa_mask_probe's tile map) and the tile shape the forward plans."""
    import torch
    from masked_attention_forward_amd import binding as fb

    from masked_attention_forward_amd import synth

    qk = w.shapes()
    q = torch.empty(qk[0], dtype=synth.DTYPES[w.dtype], device="meta")
    k = torch.empty(qk[1], dtype=synth.DTYPES[w.dtype], device="meta")
    dims = fb.dims_of(q, k, w.layout, w.actual_seq_qlen)
    mask, bcast = w.mask()
    counts, tiles = fb.fa_mask_probe(dims, w.layout, w.sparse_mode, device=dev, pre_tokens=w.pre_tokens,
                                     next_tokens=w.next_tokens, actual_seq_qlen=w.actual_seq_qlen,
                                     actual_seq_kvlen=w.actual_seq_kvlen, prefix=w.prefix, tiles=True,
                                     atten_mask=None if mask is None else mask.to(dev), mask_bcast=bcast)
    total = int(counts.sum().item())
    if w.sparse_mode == 3 and w.layout != "TND" and w.Sq <= w.Skv:
        per_head = w.Sq * (w.Skv - w.Sq) + w.Sq * (w.Sq + 1) // 2
        assert total == per_head * w.B * w.N, (total, per_head)
    bm, bn, _, _ = fb.fa_tile_shape(dims, w.layout, w.actual_seq_qlen, w.actual_seq_kvlen)
    visited = int(((tiles == 1) | (tiles == 2)).sum().item())
    # The mode-1 map has a row per (batch, head, q tile); the others one per (batch, q tile).
    computed = visited * bm * bn * (1 if w.sparse_mode == 1 else w.N)
    return total, computed


def exp2_rate(dev, iters: int = 64, launches: int = 10) -> float:
    """Measured exp2 throughput of the chip (exponentials per second) from the library's
    calibration kernel: 2048 workgroups x 256 threads, nothing but v_exp_f32 in the loop."""
    import torch
    from masked_attention_forward_amd import binding as fb

    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        n = fb.fa_exp2_rate_probe(out, iters)
    torch.cuda.synchronize()
    # Every thread's chains converge to 8 times the root of x = 2^(-x).
    assert abs(float(out.min()) - 5.1294860) < 1e-4 and abs(float(out.max()) - 5.1294860) < 1e-4
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        fb.fa_exp2_rate_probe(out, iters)
    e1.record(stream)
    torch.cuda.synchronize()
    return n * launches / (e0.elapsed_time(e1) * 1e-3)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, heads: int, decode: bool = False):
    """Time the fp64 oracle on `heads` whole (batch, head) slices of the workload (TFLOP/s, or
    algorithmic GB/s for a decode workload)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v = w.tensors()
    mask, _ = w.mask()
    mask = None if mask is None else mask.numpy()   # [1, 1, Sq, Skv]: shared by every slice
    assert w.layout == "BNSD"
    sel = [(b, h) for b in range(w.B) for h in range(w.N)][:heads]
    flops = 0
    t_total = 0.0
    for b, h in sel:
        qs = q[b:b + 1, h:h + 1].double().numpy()
        ks = k[b:b + 1, h:h + 1].double().numpy()
        vs = v[b:b + 1, h:h + 1].double().numpy()
        slopes = [w.slopes()[h]] if w.alibi else None
        prefix = [w.prefix[b]] if w.prefix is not None else None
        t0 = time.perf_counter()
        _, lse = oracle.attention(qs, ks, vs, layout="BNSD", sparse_mode=w.sparse_mode,
                                  scale=w.softmax_scale, pre_tokens=w.pre_tokens,
                                  next_tokens=w.next_tokens, prefix=prefix, alibi_slopes=slopes,
                                  atten_mask=mask)
        t_total += time.perf_counter() - t0
        if mask is not None:
            vis = mask[0, 0] == 0
        else:
            vis = oracle.visible_matrix(w.sparse_mode, w.Sq, w.Skv, pre_tokens=w.pre_tokens,
                                        next_tokens=w.next_tokens,
                                        prefix_len=prefix[0] if prefix else 0)
        flops += 4 * w.D * int(vis.sum())
    if decode:
        elem = q.element_size()
        moved = len(sel) * ((2 * w.Sq * w.D + 2 * w.Skv * w.D) * elem + 4 * w.Sq)
        value, unit = moved / t_total / 1e9, "GB/s"
    else:
        value, unit = flops / t_total / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{len(sel)} of {w.B * w.N} (batch, head) slices at full Sq={w.Sq}, Skv={w.Skv}; "
                      f"{t_total:.1f} s of fp64 numpy (BLAS threads={threads}, elementwise on 1 core)"}


def paged_caches(w, k, v, bs, cache_layout, dev):
    """K / V of workload w moved into paged caches ("aclnnScatterPaKvCache" layouts) with
    randomly permuted distinct pages; returns (key_cache, value_cache, block_table int32)."""
    import numpy as np
    import torch

    if w.layout == "BNSD":
        seqs_k = [k[b].transpose(0, 1) for b in range(w.B)]
        seqs_v = [v[b].transpose(0, 1) for b in range(w.B)]
    elif w.layout == "BSND":
        seqs_k, seqs_v = [k[b] for b in range(w.B)], [v[b] for b in range(w.B)]
    else:
        ends = w.actual_seq_kvlen
        starts = [0] + list(ends[:-1])
        seqs_k = [k[s:e] for s, e in zip(starts, ends)]
        seqs_v = [v[s:e] for s, e in zip(starts, ends)]
    lens = [int(x.shape[0]) for x in seqs_k]
    need = [-(-L // bs) for L in lens]
    nb = sum(need)
    perm = np.random.default_rng(17).permutation(nb)
    bt = np.zeros((len(lens), max(need + [1])), dtype=np.int32)
    p = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[p:p + n]
        p += n
    N, D = w.N, w.D
    shape = (nb, bs, N, D) if cache_layout == "Norm" else (nb, N, bs, D)
    caches = []
    for seqs in (seqs_k, seqs_v):
        c = torch.zeros(shape, dtype=k.dtype, device=dev)
        view = c if cache_layout == "Norm" else c.permute(0, 2, 1, 3)
        for b, s in enumerate(seqs):
            j = torch.arange(lens[b], device=dev)
            pages = torch.from_numpy(bt[b].astype(np.int64)).to(dev)[j // bs]
            view[pages, j % bs] = s
        caches.append(c)
    return caches[0], caches[1], torch.from_numpy(bt).to(dev)


def bench_bwd(args, dev):
    """Backward pass of the workload: fa_fwd once for out and softmax_lse, then fa_bwd timed
    alone with a seeded dO. Effective TFLOP/s count 10 D flops per visible pair, the five
    products of the backward (S recomputed, dP, dV, dK, dQ)."""
    import torch
    from masked_attention_forward_amd import binding as fb
    from masked_attention_forward_amd import synth

    w = synth.workloads()[args.workload]
    q, k, v = (x.to(dev) for x in w.tensors())
    do = synth.randn(tuple(q.shape), q.dtype, w.seed * 3 + 7).to(dev)
    slopes = torch.tensor(w.slopes(), dtype=torch.float32, device=dev) if w.alibi else None
    kw = dict(layout=w.layout, sparse_mode=w.sparse_mode, pre_tokens=w.pre_tokens, next_tokens=w.next_tokens,
              actual_seq_qlen=w.actual_seq_qlen, actual_seq_kvlen=w.actual_seq_kvlen, prefix=w.prefix,
              alibi_slopes=slopes, alibi_mode=args.alibi_mode, scale=w.softmax_scale)
    out, lse = fb.flash_attention(q, k, v, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dims = fb.dims_of(q, k, w.layout, w.actual_seq_qlen)
    ws_bytes = fb.fa_bwd_workspace_size(dims, w.layout, w.sparse_mode, w.actual_seq_qlen, w.actual_seq_kvlen)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        fb.fa_bwd(q, k, v, out, lse, do, dq, dk, dv, workspace=ws if ws_bytes else None, **kw)

    pairs, _ = visible_pairs(w, dev)
    flops = 10 * w.D * pairs
    n_pre = prewarm(step, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "effective TFLOP/s attn bwd (10 D flops per visible pair)", "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "f32": "f32"}[w.dtype], "data": "synthetic (seeded N(0,1) q/k/v/dO)",
        "timing": {"cache": "warm", "prewarm_ms": args.prewarm_ms, "prewarm_steps": n_pre},
        "config": {"workload": args.workload, "layout": w.layout, "sparse_mode": w.sparse_mode, "B": w.B, "N": w.N,
                   "Sq": w.Sq, "Skv": w.Skv, "D": w.D, "visible_pairs": pairs, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}}), flush=True)


def bench_scatter(args, dev):
    """Paged KV cache scatter ("aclnnScatterPaKvCache", Norm cache): a prefill chunk of
    32768 tokens x 32 heads x D 128 bf16 keys and values written to random distinct slots of a
    65536-slot cache (512 blocks of 128). HBM-bound: every byte is read once and written once."""
    import torch
    from masked_attention_forward_amd import binding as fb

    T, N, D, nb, bs = 32768, 32, 128, 512, 128
    g = torch.Generator().manual_seed(11)
    key = torch.randn(T, N, D, generator=g).to(torch.bfloat16).to(dev)
    val = torch.randn(T, N, D, generator=g).to(torch.bfloat16).to(dev)
    kc = torch.zeros(nb, bs, N, D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64).to(dev)
    n_pre = prewarm(lambda: fb.fa_scatter_kv_cache(key, kc, slots, val, vc), args.prewarm_ms)
    for _ in range(args.warmup):
        fb.fa_scatter_kv_cache(key, kc, slots, val, vc)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fb.fa_scatter_kv_cache(key, kc, slots, val, vc)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    moved = 2 * 2 * T * N * D * 2 + T * 8   # K and V read + written, plus the slots
    gbs = moved / (ms * 1e-3) / 1e9
    # Context: a plain device-to-device copy of the same K and V bytes (torch's copy kernel)
    # on the same GPU, right after.
    src = torch.cat([key.view(-1), val.view(-1)])
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * src.element_size() / (e0.elapsed_time(e1) / args.steps * 1e-3) / 1e9
    del src, dst
    print(json.dumps({
        "metric": "paged KV cache scatter bandwidth (bytes read + written)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values, random distinct slots)",
        "timing": {"cache": "warm", "prewarm_ms": args.prewarm_ms, "prewarm_steps": n_pre},
        "device_copy_gbs": round(copy_gbs, 1),
        "config": {"workload": "kv_scatter_prefill", "num_tokens": T, "N": N, "D": D, "num_blocks": nb,
                   "block_size": bs, "layout": "Norm"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic("kv_scatter_prefill",
                                                 os.path.join(ROOT, "profiles", "fa_kv_scatter_prefill_trace.md"),
                                                 SCATTER_SOURCES),
                     "algorithmic_bytes": moved, "kernel_sources_sha256": kernel_sources_sha(SCATTER_SOURCES)}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--alibi-mode", default="right", choices=["right", "sqrt", "left"],
                    help="alibi variant for workloads with alibi")
    ap.add_argument("--cpu-heads", type=int, default=48,
                    help="(batch, head) slices of the workload the CPU oracle is timed on")
    ap.add_argument("--op", default="attention", choices=["attention", "scatter_kv", "bwd"],
                    help="attention (the default metric), the paged KV cache scatter, or the backward pass")
    ap.add_argument("--block-size", type=int, default=0,
                    help="> 0: read K / V through fa_fwd_paged from caches of pages of this many keys")
    ap.add_argument("--cache-layout", default="Norm", choices=["Norm", "NHSD"],
                    help="paged cache layout (with --block-size)")
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed steps for this many ms of wall time before the warm-up steps "
                         "(the GPU clock ramps up over the first tens of ms of load; 0: none)")
    ap.add_argument("--cold", action="store_true",
                    help="cold caches: read a 512 MiB buffer before every timed launch (more than "
                         "L2 and the 256 MB Infinity Cache) and time each launch alone with HIP events")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from masked_attention_forward_amd import binding as fb
    from masked_attention_forward_amd import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.warmup + args.steps}))
        return
    if args.op == "scatter_kv":
        bench_scatter(args, dev)
        return
    if args.op == "bwd":
        bench_bwd(args, dev)
        return
    w = synth.workloads()[args.workload]
    q, k, v = (x.to(dev) for x in w.tensors())
    slopes = torch.tensor(w.slopes(), dtype=torch.float32, device=dev) if w.alibi else None
    mask, mask_bcast = w.mask()
    mask = None if mask is None else mask.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(fb.lse_shape(q, w.layout), dtype=torch.float32, device=dev)
    dims = fb.dims_of(q, k, w.layout, w.actual_seq_qlen)
    paged = None
    if args.block_size > 0:
        paged = paged_caches(w, k, v, args.block_size, args.cache_layout, dev)
        pk = fb.paged_kv(paged[2], paged[0], cache_layout=args.cache_layout)
        ws_bytes = fb.fa_fwd_paged_workspace_size(dims, w.layout, w.sparse_mode, pk, w.actual_seq_qlen,
                                                  w.actual_seq_kvlen)
    elif w.sparse_mode == 1:
        ws_bytes = fb.fa_fwd_mask_workspace_size(dims, w.layout, mask_bcast)
    else:
        ws_bytes = fb.fa_fwd_workspace_size(dims, w.layout, w.sparse_mode, w.actual_seq_qlen, w.actual_seq_kvlen)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    kw = dict(layout=w.layout, sparse_mode=w.sparse_mode, pre_tokens=w.pre_tokens, next_tokens=w.next_tokens,
              actual_seq_qlen=w.actual_seq_qlen, actual_seq_kvlen=w.actual_seq_kvlen, prefix=w.prefix,
              alibi_slopes=slopes, alibi_mode=args.alibi_mode, scale=w.softmax_scale,
              atten_mask=mask, mask_bcast=mask_bcast, workspace=ws if ws_bytes else None)
    if paged is not None:
        kc, vc, bt = paged
        pkw = dict(kw, cache_layout=args.cache_layout, kv_seqlen=w.Skv)

        def step():
            fb.fa_fwd_paged(q, kc, vc, bt, out, lse, **pkw)
    else:
        def step():
            fb.fa_fwd(q, k, v, out, lse, **kw)
    pairs, computed_pairs = visible_pairs(w, dev)
    flops = 4 * w.D * pairs
    elem = q.element_size()
    rows_q = q.numel() // w.D
    rows_kv = k.numel() // w.D
    alg_bytes = (2 * rows_q * w.D + 2 * rows_kv * w.D) * elem + 4 * rows_q

    n_pre = prewarm(step, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    timing = {"cache": "warm"}
    if args.cold:
        # A read, not a write, evicts the inputs: written lines would leave up to 256 MB dirty in the
        # caches, and their write-back would fall inside the next timed launch. The read runs on the
        # same stream before each launch's first event, outside its timed span.
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        sums = []
        torch.cuda.synchronize()
        for a0, a1 in evs:
            sums.append(flush.sum())
            a0.record(stream)
            step()
            a1.record(stream)
        torch.cuda.synchronize()
        assert all(int(x) == flush.numel() for x in sums)
        per = sorted(a0.elapsed_time(a1) for a0, a1 in evs)
        ms = sum(per) / len(per)
        timing = {"cache": "cold (512 MiB read before each launch; launches timed one by one)",
                  "ms_median": round(per[len(per) // 2], 4), "ms_min": round(per[0], 4)}
    else:
        # One event between consecutive launches on the launching stream: the first-to-last span
        # is the K-step timed region, and each gap is one launch (back to back, warm caches).
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[-1]) / args.steps
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        timing.update(ms_median=round(per[len(per) // 2], 4), ms_min=round(per[0], 4),
                      ms_max=round(per[-1], 4))
    timing.update(prewarm_ms=args.prewarm_ms, prewarm_steps=n_pre)
    tflops = flops / (ms * 1e-3) / 1e12
    # At most 16 query rows per sequence: the split-KV decode path, bound by HBM.
    decode = max(w.qlens) <= 16 if w.layout == "TND" else w.Sq <= 16
    traffic = (recorded_traffic(args.workload, kernel=DECODE_KERNEL if decode else DOMINANT_KERNEL)
               if paged is None else None)
    gbs = alg_bytes / (ms * 1e-3) / 1e9

    res = {
        "metric": DECODE_METRIC if decode else METRIC,
        "value": round(gbs if decode else tflops, 2),
        "unit": "GB/s" if decode else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "f32": "f32"}[w.dtype],
        "data": "synthetic (seeded N(0,1) q/k/v)",
        "timing": timing,
        "config": {"workload": args.workload, "layout": w.layout, "sparse_mode": w.sparse_mode,
                   "B": w.B, "N": w.N, "Sq": w.Sq, "Skv": w.Skv, "D": w.D,
                   "pre_tokens": w.pre_tokens, "next_tokens": w.next_tokens,
                   "alibi": (args.alibi_mode if w.alibi else False), "visible_pairs": pairs,
                   "flop_per_step": flops,
                   "paged_kv": ({"block_size": args.block_size, "cache_layout": args.cache_layout}
                                if paged is not None else None)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": alg_bytes,
                     "kernel_sources_sha256": kernel_sources_sha()},
    }
    if decode:
        res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                           "algorithmic_bytes": alg_bytes, "kernel_sources_sha256": kernel_sources_sha()}
        res["config"]["effective_tflops"] = round(tflops, 3)
    if not decode:
        # Second roofline: one exp2 per computed score against the measured exp2 rate.
        peak_exp = exp2_rate(dev)
        achieved = computed_pairs / (ms * 1e-3)
        res["exp_roofline"] = {"bound": "exp2 (v_exp_f32)", "achieved": round(achieved / 1e12, 3),
                               "peak": round(peak_exp / 1e12, 3), "unit": "Texp/s",
                               "frac": round(achieved / peak_exp, 4), "computed_pairs": computed_pairs,
                               "visible_pairs": pairs,
                               "visible_frac": round(pairs / (ms * 1e-3) / peak_exp, 4),
                               "peak_source": "fa_exp2_rate_probe, 2048 x 256 threads, 64 x 128 exp2 each"}
    if not args.no_cpu_baseline and w.layout == "BNSD":
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_heads, decode)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
