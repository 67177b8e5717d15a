"""Benchmark: paged MLA decode on one MI355X, DeepSeek-V3 shape, bf16 cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3]

A step is one decode step of the whole hot path for a batch: one
mla_decode_write call, which writes the batch's newest tokens into the cache
(write-then-attend; extra workgroups of the absorb launch do it) and then
decodes (absorb, device-side split plan, split-KV attention, combine,
up-projection).  The index-list workload keeps mla_write_kv followed by
mla_sparse_attention; the write workload (--workload write) times
mla_write_kv_fused (RMSNorm + RoPE + cache write) on 262 144 tokens, with
mla_write_kv beside it.  Inputs
are seeded synthetic data with the V3 shape (128 heads, kv_lora_rank 512 +
qk_rope 64, page size 64, batch 64, contexts uniform in [1024, 32768],
shuffled block tables), resident in HBM before the timed region.

Two measurements run, in this order:
  1. the per-step protocol: --protocol-steps steps (default 300), each
     bracketed by its own HIP events and, when the KV working set is smaller
     than 512 MB (V2-Lite: 151 MB), preceded by a 512 MB device write that
     evicts the 256 MB Infinity Cache and the L2s; median / min / mean of the
     step and of the attention kernel (also per half, so the ramp shows), and
     the shader, memory and fabric clock levels read from sysfs while the
     steps run;
  2. the contract: W untimed warm-up steps, then K steps timed back to back
     between two device synchronisations; `value` and `ms_per_step` come from
     this loop.
After the GPU has idled (input generation takes seconds), the attention
kernel runs 10-30 % slower over its first ~200 launches while the power
management raises the memory-side clocks (the shader clock meanwhile falls
from 2.4 GHz towards its sustained ~1.6 GHz); the protocol steps run first,
so the contract's loop is timed at the clocks a sustained serving loop runs
at, and the protocol's first-half figures show the ramp.  (A 512 MB write
between steps lowers the sustained shader clock by a quarter, which is why
the larger working sets, which stream through the cache anyway, are not
flushed.)  For the V3 shape the KV working set (1.25 GB) is five times the
Infinity Cache, so the back-to-back loop needs no flush; V2-Lite's (151 MB)
fits in it, and only the protocol figures evict it.

One JSON line is printed.  `value` is attended KV tokens per second for the
whole job.  `roofline` is for the dominant kernel (the split-KV attention
kernel), timed live with HIP events recorded around it on the call's stream:
achieved = algorithmic bytes per launch (attended tokens x (R + Dr) x 2 B) /
mean launch time, against the 8 TB/s HBM peak.  `traffic` is the HBM traffic
rocprofv3 counted for that kernel (FETCH_SIZE + WRITE_SIZE, scaled by what
the same counters read for a 1 GiB copy), per launch over the same mean
launch time; it is read from the committed counter summary under profiles/
and reported only while the kernel source still hashes to the one that
summary was taken on (null otherwise).  `cpu_baseline` times the fp64
oracle (numpy, absorbed form) on a bounded sample of the same requests; its
outputs are also compared with the GPU's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
METRIC = "paged MLA decode attended-KV-tokens/s + HBM GB/s % peak, V3 shape bf16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="v3", choices=["v3", "v3fp8", "v2lite", "mixed", "v3sparse", "write"])
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="CPU time budget for the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--event-every", type=int, default=4,
                   help="time the attention kernel with HIP events on every n-th timed step")
    p.add_argument("--generic", action="store_true", help="force the plain (non-MFMA) kernels")
    p.add_argument("--fp8-mfma", action="store_true",
                   help="fp8 caches: queries and probabilities in E4M3 on the fp8 matrix cores "
                        "(approximate; MLA_FLAG_FP8_MFMA)")
    p.add_argument("--protocol-steps", type=int, default=300,
                   help="steps of the per-step protocol (512 MB cache-evicting write between steps, "
                        "median/min from HIP events), run before the timed loop; 0 skips it")
    p.add_argument("--prefill-form", default="auto", choices=["auto", "absorbed", "expanded"],
                   help="mixed workload: the prefill form (auto lets the library choose)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a 1 GiB device copy 3 times (the known-size kernel that "
                        "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_decode_v3_bf16_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_mla_latent_write_amd", "csrc", f)
                  for f in ("attn_mfma.hip", "attn_mfma_asm.inc", "device_utils.h")]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        if os.path.exists(f):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary.

    Returns None unless the summary was taken on this workload with the kernel
    source as it is now (its hash is recorded in the summary)."""
    if workload != "v3" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith(" "):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info():
    """CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])


def gpu_sclk_mhz(table="pp_dpm_sclk"):
    """Current clock level (MHz) of an amdgpu sysfs DPM table (shader clock by
    default; pp_dpm_mclk memory, pp_dpm_fclk fabric), or None where it cannot
    be read."""
    import glob
    import re

    for f in sorted(glob.glob(f"/sys/class/drm/card*/device/{table}")):
        try:
            with open(f) as fh:
                for ln in fh:
                    if "*" in ln:
                        m = re.search(r"(\d+)\s*mhz", ln, re.I)
                        if m:
                            return float(m.group(1))
        except OSError:
            continue
    return None


def stats_ms(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(xs)), "min": float(xs.min()), "mean": float(xs.mean()),
            "n": int(xs.size)}


# A step whose KV working set is below this is timed with a 512 MB device write
# before it (evicting the 256 MB Infinity Cache and the L2s); a larger working
# set streams through the cache and evicts it by itself.
FLUSH_BELOW_BYTES = 512 << 20


def protocol_phase(torch, step, n, dev, flush_each, kernel_events=True):
    """n steps, each between its own pair of HIP events (and, with
    flush_each, after a 512 MB device write that evicts the Infinity Cache and
    the L2s); the attention kernel is bracketed by a second pair.  Returns
    step and kernel statistics (ms) and the clock levels sampled while the
    steps run."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush_each else None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    for e in ev:  # torch creates its events lazily, at the first record
        for x in e:
            x.record()
    torch.cuda.synchronize()
    clocks = {t: [] for t in CLOCK_TABLES}
    for k in range(n):
        if flush is not None:
            flush.fill_(k & 0xFF)
        ev[k][0].record()
        step((ev[k][1], ev[k][2]) if kernel_events else None)
        ev[k][3].record()
        if k % 16 == 15:
            for t in CLOCK_TABLES:
                clocks[t].append(gpu_sclk_mhz(t))
    torch.cuda.synchronize()
    del flush
    step_ms = [e[0].elapsed_time(e[3]) for e in ev]
    h = n // 2
    out = {"flush": ("512 MB device write before each step, outside its events" if flush_each else
                     "none: the KV working set is larger than twice the Infinity Cache"),
           "step_ms": stats_ms(step_ms), "step_ms_first_half": stats_ms(step_ms[:h]),
           "step_ms_second_half": stats_ms(step_ms[h:])}
    if kernel_events:
        kern = [e[1].elapsed_time(e[2]) for e in ev]
        out["kernel_ms"] = stats_ms(kern)
        out["kernel_ms_first_half"] = stats_ms(kern[:h])
        out["kernel_ms_second_half"] = stats_ms(kern[h:])
    out["clock_mhz_median"] = clock_medians(clocks)
    return out


# sysfs DPM tables sampled while the protocol runs: shader, memory, fabric
CLOCK_TABLES = ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk")


def clock_medians(clocks):
    res = {}
    for t, v in clocks.items():
        v = [c for c in v if c is not None]
        res[t.replace("pp_dpm_", "")] = float(np.median(v)) if v else None
    return res


SPARSE_TOPK = 2048


def cpu_baseline(case, budget_s, gpu_out_f64, lists=None):
    """Time the oracle on requests taken in order until the budget is spent."""
    from oracle import mla_oracle as O

    ps, D = case.dims.page_size, case.dims.D
    hc = np.full((1, case.num_pages, ps, D), 0, dtype=np.uint16 if case.kv_dtype == "bf16" else np.uint8)
    hs = np.ones((1, case.num_pages, ps), dtype=np.float32)
    t0 = time.perf_counter()
    O.write_kv(hc, hs, 0, case.ctx_c_kv, case.ctx_k_pe, case.ctx_slots, case.kv_dtype)
    write_s = time.perf_counter() - t0
    done, tokens, elapsed = [], 0, 0.0
    outs = []
    while len(done) < case.batch and (elapsed < budget_s or len(done) < 1):
        b = len(done)
        t0 = time.perf_counter()
        if lists is None:
            out, _ = O.decode(hc, hs, case.kv_dtype, 0, case.q_nope, case.q_pe, case.block_tables,
                              case.context_lens, case.w_uk, case.w_uv, case.scale, case.window,
                              requests=[b])
            tokens += int(case.context_lens[b])
        else:
            out, _ = O.sparse_attention(hc, hs, case.kv_dtype, 0, case.q_nope, case.q_pe, lists,
                                        case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                        case.scale, case.window, rows=[b])
            tokens += int(np.sum((lists[b] >= 0) & (lists[b] < case.context_lens[b])))
        elapsed += time.perf_counter() - t0
        outs.append(out[b])
        done.append(b)
    threads = blas_threads()
    model, affinity = host_info()
    ref = np.stack(outs)
    got = gpu_out_f64[done]
    err = {"max_abs": float(np.max(np.abs(got - ref))),
           "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref))}
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "cores_available": affinity,
            "sample": f"fp64 numpy oracle (absorbed form{'' if lists is None else ', key lists'}) on "
                      f"the first {len(done)} of {case.batch} "
                      f"requests ({tokens} attended tokens, {elapsed:.1f} s); cache write "
                      f"{write_s:.1f} s untimed"}, err


MIXED_METRIC = "mixed MLA layer step (write + chunked prefill + decode, sliding-window layers) attended-KV-pairs/s"


def mixed_pairs(ml):
    """(prefill, decode) attended (query row, key) pairs of one mixed layer."""
    P, w = ml.n_prefill, ml.window
    pre = 0
    for b in range(P):
        n = int(ml.context_lens[b])
        m = int(ml.query_start_loc[b + 1] - ml.query_start_loc[b])
        p = np.arange(n - m, n, dtype=np.int64)
        pre += int(np.sum(p + 1 if w <= 0 else np.minimum(w, p + 1)))
    n = ml.context_lens[P:].astype(np.int64)
    dec = int(np.sum(n if w <= 0 else np.minimum(w, n)))
    return pre, dec


def main_mixed(args):
    """The mixed step at full size: per layer, write the step's new tokens
    (8 chunks of 512 + 120 decode tokens), prefill the chunks, decode the 120
    requests; layers 0 and 2 use a 128-token window."""
    import torch

    from paged_mla_latent_write_amd import mla
    from paged_mla_latent_write_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)

    def i(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    layers = []
    cache = None
    for l in range(len(W.MIXED_WINDOWS)):
        ml = W.mixed(l)
        if cache is None:
            cache = mla.KVCache.empty(ml.num_layers, ml.num_pages, ml.dims.page_size, ml.dims.R, ml.dims.Dr)
            cache.data.view(torch.int16).fill_(0x7FC0)
        mla.write_kv(cache, l, bf16(ml.pre_c_kv), bf16(ml.pre_k_pe), i(ml.pre_slots))
        P = ml.n_prefill
        layers.append(dict(
            ml=ml, new=(bf16(ml.new_c_kv), bf16(ml.new_k_pe), i(ml.new_slots)),
            qp=(bf16(ml.q_nope_p), bf16(ml.q_pe_p)), qd=(bf16(ml.q_nope_d), bf16(ml.q_pe_d)),
            w=(bf16(ml.w_uk), bf16(ml.w_uv)), qsl=i(ml.query_start_loc),
            bt_p=i(ml.block_tables[:P]), ctx_p=i(ml.context_lens[:P]),
            bt_d=i(ml.block_tables[P:]), ctx_d=i(ml.context_lens[P:]),
            pairs=mixed_pairs(ml)))
        print(f"[bench] mixed: layer {l} built", file=sys.stderr, flush=True)
    d = layers[0]["ml"].dims
    chunk = int(np.max(np.diff(layers[0]["ml"].query_start_loc)))
    K = args.steps
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in layers] for _ in range(K)]

    pflags = {"auto": 0, "absorbed": mla.MLA_FLAG_PREFILL_ABSORBED,
              "expanded": mla.MLA_FLAG_PREFILL_EXPANDED}[args.prefill_form]
    for L in layers:
        ml = L["ml"]
        L["pout"] = torch.empty((ml.q_nope_p.shape[0], d.H, d.Dv), dtype=torch.bfloat16, device=dev)
        L["dout"] = torch.empty((ml.q_nope_d.shape[0], d.H, d.Dv), dtype=torch.bfloat16, device=dev)
        L["ws"] = (mla.Workspace(), mla.Workspace())

    def step(k=None):
        for li, L in enumerate(layers):
            ml = L["ml"]
            e = ev[k][li] if k is not None else None
            if e: e[0].record()
            mla.write_kv(cache, ml.layer, *L["new"])
            if e: e[1].record()
            mla.prefill_chunk(cache, ml.layer, *L["qp"], L["qsl"], chunk, L["bt_p"], L["ctx_p"],
                              scale=ml.scale, w_uk=L["w"][0], w_uv=L["w"][1], window=ml.window,
                              out=L["pout"], want_lse=False, workspace=L["ws"][0], flags=pflags)
            if e: e[2].record()
            mla.decode(cache, ml.layer, *L["qd"], L["bt_d"], L["ctx_d"], scale=ml.scale,
                       w_uk=L["w"][0], w_uv=L["w"][1], window=ml.window, out=L["dout"],
                       want_lse=False, workspace=L["ws"][1])
            if e: e[3].record()

    # per-step protocol first (each step streams several GB of cache, so no
    # flush is needed between steps)
    protocol = None
    if args.protocol_steps > 0:
        n_proto = max(3, min(args.protocol_steps, 10))
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_proto)]
        clocks = {t: [] for t in CLOCK_TABLES}
        for k in range(n_proto):
            pev[k][0].record()
            step()
            pev[k][1].record()
            for t in CLOCK_TABLES:
                clocks[t].append(gpu_sclk_mhz(t))
        torch.cuda.synchronize()
        protocol = {"flush": "none: each step streams several GB of cache",
                    "step_ms": stats_ms([a.elapsed_time(b) for a, b in pev]),
                    "clock_mhz_median": clock_medians(clocks)}
        print(f"[bench] mixed protocol: {protocol}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] mixed: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(K):
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_layer = {}
    for li, L in enumerate(layers):
        ts = np.array([[ev[k][li][c].elapsed_time(ev[k][li][c + 1]) for c in range(3)] for k in range(K)])
        med = np.median(ts, axis=0)
        pre, dec = L["pairs"]
        per_layer[f"L{li}"] = {"window": L["ml"].window, "write_ms": float(med[0]),
                               "prefill_ms": float(med[1]), "decode_ms": float(med[2]),
                               "prefill_pairs": pre, "decode_tokens": dec,
                               "prefill_tflops": float(pre * 2 * d.H * (2 * d.R + d.Dr) / (med[1] * 1e-3) / 1e12),
                               "decode_gbs": float(dec * d.D * 2 / (med[2] * 1e-3) / 1e9)}
        print(f"[bench] mixed L{li}: {per_layer[f'L{li}']}", file=sys.stderr, flush=True)
    pairs = sum(sum(L["pairs"]) for L in layers)
    flops = pairs * 2 * d.H * (2 * d.R + d.Dr)
    step_s = wall / K
    tflops = flops / step_s / 1e12
    line = {
        "metric": MIXED_METRIC, "value": pairs * K / wall, "unit": "pairs/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1)/sqrt(dim) latents and queries, random-init W_UK/W_UV)",
        "config": {"workload": "mixed step: 8 x 512-token chunks + 120 decode requests per layer, "
                               "4 layers, windows (128, 0, 128, 0)",
                   "heads": d.H, "kv_lora_rank": d.R, "qk_rope": d.Dr, "page_size": d.page_size,
                   "attended_pairs": pairs, "prefill_form": args.prefill_form},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "whole step (prefill dominates the flops)"},
        "per_layer": per_layer,
        "protocol": protocol,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        base, err = cpu_baseline_mixed(layers[1], args.cpu_seconds)
        line["cpu_baseline"] = base
        line["parity_sample"] = err
    print(json.dumps(line), flush=True)


def cpu_baseline_mixed(L, budget_s):
    """The oracle on a full-attention layer's prefill: every 8th query row of
    each chunk plus its last row, chunk after chunk until the budget is spent
    (pairs per second on that sample), compared with the GPU's rows."""
    from oracle import mla_oracle as O

    ml = L["ml"]
    d = ml.dims
    P = ml.n_prefill
    hc = np.zeros((1, ml.num_pages, d.page_size, d.D), dtype=np.uint16)
    hs = np.ones((1, ml.num_pages, d.page_size), dtype=np.float32)
    O.write_kv(hc, hs, 0, ml.pre_c_kv, ml.pre_k_pe, ml.pre_slots)
    O.write_kv(hc, hs, 0, ml.new_c_kv, ml.new_k_pe, ml.new_slots)
    bits = L["pout"].view(__import__("torch").int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    gpu = bits.view(np.float32).astype(np.float64)
    elapsed, pairs, rows_done, errs = 0.0, 0, [], []
    for b in range(P):
        if elapsed >= budget_s and rows_done:
            break
        s0, s1 = int(ml.query_start_loc[b]), int(ml.query_start_loc[b + 1])
        rows = sorted(set(list(range(s0, s1, 8)) + [s1 - 1]))
        n, m = int(ml.context_lens[b]), s1 - s0
        t0 = time.perf_counter()
        ref, _ = O.prefill_chunk(hc, hs, O.KV_BF16, 0, ml.q_nope_p, ml.q_pe_p, ml.query_start_loc,
                                 ml.block_tables[:P], ml.context_lens[:P], ml.w_uk, ml.w_uv,
                                 ml.scale, ml.window, rows=rows)
        elapsed += time.perf_counter() - t0
        for r in rows:
            p = n - m + (r - s0)
            pairs += p + 1 if ml.window <= 0 else min(ml.window, p + 1)
        rows_done += rows
        errs.append((gpu[rows], ref[rows]))
    got = np.concatenate([g for g, _ in errs])
    ref = np.concatenate([r for _, r in errs])
    model, affinity = host_info()
    err = {"max_abs": float(np.max(np.abs(got - ref))),
           "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref))}
    return {"value": pairs / elapsed, "unit": "pairs/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": model, "cores_available": affinity,
            "sample": f"fp64 numpy oracle (absorbed form), layer {ml.layer} (full attention) prefill: "
                      f"every 8th row of each chunk plus its last, {len(rows_done)} rows of "
                      f"{int(ml.query_start_loc[-1])} ({pairs} pairs, "
                      f"{elapsed:.1f} s)"}, err


WRITE_METRIC = "fused RMSNorm + RoPE latent cache write (mla_write_kv_fused) tokens/s, prefill-sized batch"
WRITE_TOKENS = 262144


def write_bytes_per_token(d, fp8):
    """Algorithmic HBM bytes of one written token: the latent and rope rows
    read (bf16), its slot and position (int64), and the cache row written
    (bf16 values, or E4M3 codes and an fp32 scale).  The norm weight and the
    cos/sin table rows are shared by every token and stay in the caches."""
    return 2 * (d.R + d.Dr) + 8 + 8 + (d.D + 4 if fp8 else 2 * d.D)


def main_write(args):
    """f3 at a prefill-sized batch: one mla_write_kv_fused call of 262 144
    tokens (RMSNorm over the 512-wide latent, interleaved RoPE over the 64-wide
    rope part, then the cache write) per step, into a bf16 cache (the line's
    value) and an fp8 E4M3 cache; mla_write_kv of the same rows timed beside
    it.  About 600 MB move per bf16 call, more than the 256 MB Infinity Cache,
    so back-to-back calls stream from HBM."""
    import torch

    from paged_mla_latent_write_amd import mla
    from paged_mla_latent_write_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = W.MLA_DIMS_128
    T = WRITE_TOKENS
    fc = W.fused_write_case(d, T, seed=7)
    print(f"[bench] write: {T} tokens generated", file=sys.stderr, flush=True)

    def bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)

    def i(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    c_kv, k_pe, slots, pos = bf16(fc.c_kv), bf16(fc.k_pe), i(fc.slots), i(fc.positions)
    w, cs = bf16(fc.norm_weight), i(fc.cos_sin)
    caches = {kv: mla.KVCache.empty(1, fc.num_pages, d.page_size, d.R, d.Dr, fp8=(kv == "fp8_e4m3"))
              for kv in ("bf16", "fp8_e4m3")}

    def fused(kv):
        mla.write_kv_fused(caches[kv], 0, c_kv, k_pe, slots, positions=pos, norm_weight=w, eps=fc.eps,
                           cos_sin=cs, interleaved=True)

    def plain(kv):
        mla.write_kv(caches[kv], 0, c_kv, k_pe, slots)

    K = args.steps

    def timed(fn):
        """Warm-up, then K calls back to back (wall clock between two
        synchronisations) with every call also between its own HIP events on
        the stream it is launched on; returns (ms per step, event stats)."""
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / K, stats_ms([a.elapsed_time(b) for a, b in ev])

    res = {}
    for kv in ("bf16", "fp8_e4m3"):
        for name, fn in (("fused", fused), ("plain", plain)):
            res[(kv, name)] = timed(lambda: fn(kv))
            ms, ev = res[(kv, name)]
            print(f"[bench] write {name} {kv}: {ms:.4f} ms/step, kernel median {ev['median']:.4f} ms",
                  file=sys.stderr, flush=True)

    def roof(kv, name):
        ms, ev = res[(kv, name)]
        nbytes = T * write_bytes_per_token(d, kv == "fp8_e4m3")
        gbs = nbytes / (ev["mean"] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": f"{name} write, {kv} cache",
                "kernel_ms": ev["mean"], "kernel_ms_stats": ev, "alg_bytes_per_launch": nbytes,
                "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3)}

    ms = res[("bf16", "fused")][0]
    line = {
        "metric": WRITE_METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 arithmetic, bf16 cache",
        "data": "synthetic (seeded; N(0,1) latent and rope rows, norm weight 1 + 0.1 N(0,1), "
                "positions uniform in [0, 40000), slots a random permutation of the pages)",
        "config": {"workload": f"fused latent write: {T} tokens, R {d.R} + Dr {d.Dr}, page size "
                               f"{d.page_size}, RMSNorm (eps {fc.eps}) + interleaved RoPE",
                   "tokens": T, "kv_lora_rank": d.R, "qk_rope": d.Dr, "page_size": d.page_size},
        "roofline": roof("bf16", "fused"),
        "plain_write_bf16": roof("bf16", "plain"),
        "fused_write_fp8": roof("fp8_e4m3", "fused"),
        "plain_write_fp8": roof("fp8_e4m3", "plain"),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O

        fused("bf16")
        torch.cuda.synchronize()
        got = caches["bf16"].data[0].view(torch.int16).cpu().numpy().view(np.uint16)
        hc = np.zeros((1, fc.num_pages, d.page_size, d.D), dtype=np.uint16)
        hs = np.ones((1, fc.num_pages, d.page_size), dtype=np.float32)
        done, elapsed, chunk = 0, 0.0, 4096
        while done < T and (elapsed < args.cpu_seconds or done == 0):
            sl = slice(done, min(T, done + chunk))
            t0 = time.perf_counter()
            O.write_kv_fused(hc, hs, 0, fc.c_kv[sl], fc.k_pe[sl], fc.slots[sl], fc.positions[sl],
                             fc.norm_weight, fc.eps, fc.cos_sin, True, O.KV_BF16)
            elapsed += time.perf_counter() - t0
            done = sl.stop
        s = fc.slots[:done]
        pg, off = s // d.page_size, s % d.page_size
        ref = O.bf16_bits_to_f64(hc[0][pg, off])
        gpu = O.bf16_bits_to_f64(got[pg, off])
        model, affinity = host_info()
        line["cpu_baseline"] = {
            "value": done / elapsed, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": model, "cores_available": affinity,
            "sample": f"fp64 numpy oracle write_kv_fused (bf16 cache) on the first {done} of {T} tokens "
                      f"({elapsed:.1f} s)"}
        line["parity_sample"] = {
            "max_abs": float(np.max(np.abs(gpu - ref))),
            "rel_l2": float(np.linalg.norm(gpu - ref) / np.linalg.norm(ref)),
            "bf16_values_differing": float(np.mean(hc[0][pg, off] != got[pg, off]))}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    if args.workload == "mixed":
        return main_mixed(args)
    if args.workload == "write":
        return main_write(args)
    import torch

    from paged_mla_latent_write_amd import mla
    from paged_mla_latent_write_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    case = {"v3": W.v3, "v3fp8": W.v3fp8, "v2lite": W.v2lite, "v3sparse": W.v3}[args.workload]()
    d = case.dims
    B = case.batch
    sparse = args.workload == "v3sparse"
    lists_np = lists = None
    if sparse:
        # one 2048-entry key list per request: distinct positions of its context
        lists_np = W.key_lists(1400, case.context_lens - 1, case.context_lens, SPARSE_TOPK,
                               pad_frac=0.0, invalid_frac=0.0)
        lists = torch.from_numpy(lists_np).to(dev)

    def bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)

    fp8 = case.kv_dtype != "bf16"
    cache = mla.KVCache.empty(case.num_layers, case.num_pages, d.page_size, d.R, d.Dr, fp8=fp8)
    if fp8:
        cache.data.fill_(0x7F)
        cache.scale.fill_(float("nan"))
    else:
        cache.data.view(torch.int16).fill_(0x7FC0)
    mla.write_kv(cache, case.layer, bf16(case.ctx_c_kv), bf16(case.ctx_k_pe),
                 torch.from_numpy(case.ctx_slots).to(dev))
    newest = case.new_token_rows()
    new_c, new_r = bf16(case.ctx_c_kv[newest]), bf16(case.ctx_k_pe[newest])
    new_slots = torch.from_numpy(case.ctx_slots[newest]).to(dev)
    q_nope, q_pe = bf16(case.q_nope), bf16(case.q_pe)
    w_uk, w_uv = bf16(case.w_uk), bf16(case.w_uv)
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty((B, d.H, d.Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, d.H), dtype=torch.float32, device=dev)
    ws = mla.Workspace()
    flags = mla.MLA_FLAG_GENERIC_KERNELS if args.generic else 0
    if args.fp8_mfma and fp8:
        flags |= mla.MLA_FLAG_FP8_MFMA
    K = args.steps
    # The attention kernel is timed by a pair of HIP events on every
    # args.event_every-th timed step: each recorded pair leaves ~12 us of idle
    # GPU time between the kernels around it (measured with a kernel trace),
    # which would otherwise be charged to every step.
    timed = [k for k in range(K) if k % args.event_every == 0]
    events = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for k in timed}
    for a, b in events.values():  # torch creates its events lazily, at the first record
        a.record()
        b.record()

    def step(ev=None):
        if sparse:
            mla.write_kv(cache, case.layer, new_c, new_r, new_slots)
            mla.sparse_attention(cache, case.layer, q_nope, q_pe, lists, bt, ctx, scale=case.scale,
                                 w_uk=w_uk, w_uv=w_uv, window=case.window, out=out, lse=lse,
                                 workspace=ws, flags=flags, kernel_events=ev)
        else:
            mla.decode(cache, case.layer, q_nope, q_pe, bt, ctx, scale=case.scale, w_uk=w_uk,
                       w_uv=w_uv, window=case.window, out=out, lse=lse, workspace=ws, flags=flags,
                       kernel_events=ev, new_tokens=(new_c, new_r, new_slots))

    protocol = None
    if args.protocol_steps > 0:
        kept = (int(np.sum((lists_np >= 0) & (lists_np < case.context_lens[:, None]))) if sparse
                else int(case.context_lens.astype(np.int64).sum()))
        kv_set = kept * (d.D * (1 if fp8 else 2) + (4 if fp8 else 0))
        protocol = protocol_phase(torch, step, args.protocol_steps, dev, kv_set < FLUSH_BELOW_BYTES)
        print(f"[bench] protocol: {protocol}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy calibration: 3 x 1 GiB device copies done", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(K):
        step(events.get(k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_all = [a.elapsed_time(b) for a, b in events.values()]
    kern_ms = float(np.mean(kern_all))
    print(f"[bench] timed {K} steps: {wall * 1e3 / K:.3f} ms/step, attention kernel {kern_ms:.3f} ms",
          file=sys.stderr, flush=True)

    if sparse:
        tokens = int(np.sum((lists_np >= 0) & (lists_np < case.context_lens[:, None])))
    else:
        tokens = int(case.context_lens.astype(np.int64).sum())
    per_tok_bytes = d.D * (1 if fp8 else 2) + (4 if fp8 else 0)
    kv_bytes = tokens * per_tok_bytes
    flops = tokens * 2 * d.H * (2 * d.R + d.Dr)
    fixed_bytes = 2 * d.H * d.Dn * d.R * 2 + B * d.H * (d.Dn + d.Dr + d.Dv) * 2
    step_s = wall / K
    achieved = kv_bytes / (kern_ms * 1e-3) / 1e9
    traffic_bytes = None if (args.generic or fp8) else measured_traffic(args.workload)
    traffic = None if traffic_bytes is None else traffic_bytes / (kern_ms * 1e-3) / 1e9
    tflops = flops / (kern_ms * 1e-3) / 1e12
    # the matrix-core peak of the arithmetic the kernel runs (fp8 for the
    # fp8-MFMA path, else bf16)
    mfma_peak = FP8_MFMA_PEAK_TFLOPS if (args.fp8_mfma and fp8) else BF16_MFMA_PEAK_TFLOPS
    if flops / kv_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        # past the ridge (the fp8 cache on bf16 matrix cores: 580 B per token
        # for the same flops): the matrix cores bind
        roofline = {"bound": "mfma", "achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": tflops / mfma_peak, "traffic": None,
                    "kernel": "split-KV attention", "kernel_ms": kern_ms,
                    "alg_flops_per_launch": flops, "hbm_gbs": achieved,
                    "hbm_frac": achieved / HBM_PEAK_GBS}
    else:
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                    "kernel": "split-KV attention", "kernel_ms": kern_ms,
                    "alg_bytes_per_launch": kv_bytes, "traffic_bytes_per_launch": traffic_bytes,
                    "mfma_tflops": tflops}
    line = {
        "metric": METRIC,
        "value": tokens * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not fp8 else "fp8_e4m3 cache, bf16 compute",
        "data": "synthetic (seeded; N(0,1)/sqrt(dim) latents and queries, random-init W_UK/W_UV)",
        "config": {
            "workload": {"v3": "DeepSeek-V3-shape MLA decode, one GPU's full head set",
                         "v3fp8": "V3-shape MLA decode with fp8 e4m3 latent cache",
                         "v2lite": "DeepSeek-V2-Lite-shape MLA decode",
                         "v3sparse": f"V3-shape MLA decode over {SPARSE_TOPK}-entry key lists "
                                     f"(index-list attention)"}[args.workload],
            "batch": B, "heads": d.H, "kv_lora_rank": d.R, "qk_rope": d.Dr, "qk_nope": d.Dn,
            "v_head": d.Dv, "page_size": d.page_size,
            "context_lens": f"{int(case.context_lens.min())}..{int(case.context_lens.max())}",
            "attended_tokens": tokens, "kv_cache": case.kv_dtype,
            "step": ("mla_write_kv(batch newest tokens) + mla_sparse_attention" if sparse
                     else "mla_decode_write(batch newest tokens written, then the decode)"),
            "kernels": ("generic" if args.generic else
                        "fp8 matrix cores (E4M3 queries and probabilities)" if (args.fp8_mfma and fp8)
                        else "default"),
        },
        "step_hbm_gbs": (kv_bytes + fixed_bytes) / step_s / 1e9,
        "step_tflops": flops / step_s / 1e12,
        "step_frac_of_hbm_roofline": (kv_bytes + fixed_bytes) / step_s / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline,
        "cpu_baseline": None,
        "kernel_ms_timed_loop": stats_ms(kern_all),
        "protocol": protocol,
    }
    if not args.no_cpu_baseline:
        bits = out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        gpu_out = bits.view(np.float32).astype(np.float64)
        base, err = cpu_baseline(case, args.cpu_seconds, gpu_out, lists_np)
        line["cpu_baseline"] = base
        line["parity_sample"] = err
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
