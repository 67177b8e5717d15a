"""Helpers for the GPU parity tests: upload seeded cases, populate the device
cache through mla_write_kv, build the oracle's own host cache, and measure
errors the way the tolerances are stated (max-abs and relative L2 over a
call's output tensor)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

BF16_TOL = (2e-2, 5e-3)   # (max-abs, rel-L2) for a bf16 cache
FP8_TOL = (1e-1, 3e-2)    # for an fp8 e4m3 cache


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_available():
    return torch.cuda.is_available()


def dev_bf16(u16):
    a = np.ascontiguousarray(u16, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_host_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_host_f64(t):
    return O.bf16_bits_to_f64(bf16_host_bits(t))


def new_device_cache(mla, num_layers, num_pages, dims, kv_dtype):
    cache = mla.KVCache.empty(num_layers, num_pages, dims.page_size, dims.R, dims.Dr,
                              fp8=(kv_dtype == O.KV_FP8))
    if cache.fp8:
        cache.data.fill_(int(W.E4M3_NAN))
        cache.scale.fill_(float("nan"))
    else:
        cache.data.view(torch.int16).fill_(int(W.BF16_NAN))
    return cache


def populate_device(mla, case, num_layers=None, layer=None, cache=None):
    """Device cache: NaN everywhere, then the case's population written with
    mla_write_kv (the same route a serving step takes)."""
    L = num_layers or case.num_layers
    layer = case.layer if layer is None else layer
    if cache is None:
        cache = new_device_cache(mla, L, case.num_pages, case.dims, case.kv_dtype)
    if case.ctx_slots.size:
        mla.write_kv(cache, layer, dev_bf16(case.ctx_c_kv), dev_bf16(case.ctx_k_pe),
                     dev(case.ctx_slots.astype(np.int64)))
    torch.cuda.synchronize()
    return cache


WRITE_CHUNK = 1 << 15  # tokens per oracle write call (bounds the fp8 encoder's temporaries)


def oracle_write_chunked(cache, scale, layer, c_kv, k_pe, slots, kv_dtype):
    """The oracle's write over a long token list, a chunk of tokens at a time
    (the slots of one call are distinct, so the chunks are independent and
    write disjoint cache rows; they run on a few host threads, since numpy
    releases the interpreter lock inside the encoder)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(t0):
        t1 = min(len(slots), t0 + WRITE_CHUNK)
        O.write_kv(cache, scale, layer, c_kv[t0:t1], k_pe[t0:t1], slots[t0:t1], kv_dtype)

    starts = range(0, len(slots), WRITE_CHUNK)
    if kv_dtype == O.KV_BF16 or len(starts) < 2:
        for t0 in starts:
            one(t0)
        return
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, starts))


def host_cache(case):
    """The oracle's own one-layer host cache, written by the oracle's write."""
    fill = W.BF16_NAN if case.kv_dtype == O.KV_BF16 else W.E4M3_NAN
    dt = np.uint16 if case.kv_dtype == O.KV_BF16 else np.uint8
    cache = np.full((1, case.num_pages, case.dims.page_size, case.dims.D), fill, dtype=dt)
    scale = np.full((1, case.num_pages, case.dims.page_size), np.nan, dtype=np.float32)
    oracle_write_chunked(cache, scale, 0, case.ctx_c_kv, case.ctx_k_pe, case.ctx_slots, case.kv_dtype)
    return cache, scale


def weights(case):
    return dev_bf16(case.w_uk), dev_bf16(case.w_uv)


def gpu_decode(mla, case, cache, layer=None, **kw):
    w_uk, w_uv = weights(case)
    out, lse = mla.decode(cache, case.layer if layer is None else layer, dev_bf16(case.q_nope),
                          dev_bf16(case.q_pe), dev(case.block_tables), dev(case.context_lens),
                          scale=case.scale, w_uk=kw.pop("w_uk", w_uk), w_uv=kw.pop("w_uv", w_uv),
                          window=kw.pop("window", case.window), **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(case, hcache, requests=None, window=None, **kw):
    hc, hs = hcache
    return O.decode(hc, hs, case.kv_dtype, 0, case.q_nope, case.q_pe, case.block_tables,
                    case.context_lens, kw.pop("w_uk", case.w_uk), kw.pop("w_uv", case.w_uv),
                    case.scale, case.window if window is None else window, requests=requests)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output"
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    return max_abs, rel_l2


def assert_close(got, ref, tol, what=""):
    max_abs, rel_l2 = errors(got, ref)
    say(f"  {what}: max-abs {max_abs:.3e}  rel-L2 {rel_l2:.3e}")
    assert max_abs <= tol[0] and rel_l2 <= tol[1], (what, max_abs, rel_l2)
    return max_abs, rel_l2


def assert_lse_close(got, ref, atol=2e-3, what="lse"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert (np.isneginf(got) == np.isneginf(ref)).all(), what
    d = np.abs(np.where(both_inf, 0.0, got) - np.where(both_inf, 0.0, ref))
    say(f"  {what}: max-abs {float(d.max()) if d.size else 0.0:.3e}")
    assert (d <= atol).all(), (what, float(d.max()))
