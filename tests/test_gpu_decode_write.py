"""mla_decode_write, through the C ABI: the step's new-token write and the
decode in one call.  Its results are those of mla_write_kv followed by
mla_decode on the same stream, bit for bit (cache codes and scales, out,
lse), whether the tokens ride in the matrix-core absorb launch or, on the
other routes, in a write launch of their own; and the decode equals the
oracle's over the oracle-written cache ("[SHIM] Root causes", item 2: a
decode step writes its token before it attends over it).
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, bf16_host_bits, dev, dev_bf16,
                         new_device_cache, say)

pytestmark = pytest.mark.gpu

DIMS = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def split_rows(case, last):
    """Population rows split into (already cached, written by this step): the
    last `last[b]` tokens of request b are the step's."""
    ends = np.cumsum(case.context_lens.astype(np.int64))
    starts = ends - case.context_lens
    new = np.concatenate([np.arange(e - k, e) for e, k in zip(ends, last)])
    old = np.setdiff1d(np.arange(int(ends[-1])), new)
    assert all(k <= e - s for s, e, k in zip(starts, ends, last))
    return old, new


def with_pads(rng, c, r, slots, n_pads):
    """The step's rows with n_pads pad rows (slot -1, random values) spread
    among them."""
    T = len(slots) + n_pads
    at = np.sort(rng.choice(T, n_pads, replace=False))
    keep = np.setdiff1d(np.arange(T), at)
    cc = np.zeros((T, c.shape[1]), dtype=np.uint16)
    rr = np.zeros((T, r.shape[1]), dtype=np.uint16)
    ss = np.full(T, -1, dtype=np.int64)
    cc[keep], rr[keep], ss[keep] = c, r, slots
    cc[at] = W.bf16_normal(rng, (n_pads, c.shape[1]), 0.5)
    rr[at] = W.bf16_normal(rng, (n_pads, r.shape[1]), 0.5)
    return cc, rr, ss


def cache_bits(cache):
    data = bf16_host_bits(cache.data) if not cache.fp8 else cache.data.cpu().numpy()
    scale = None if cache.scale is None else cache.scale.cpu().numpy().view(np.uint32)
    return data, scale


def run_both(mla, case, step, **kw):
    """(write_kv then decode) and decode_write, each on its own cache holding
    the rows written before the step; returns both results."""
    old, _ = step["split"]
    res = []
    for fused in (False, True):
        cache = new_device_cache(mla, case.num_layers, case.num_pages, case.dims, case.kv_dtype)
        mla.write_kv(cache, case.layer, dev_bf16(case.ctx_c_kv[old]), dev_bf16(case.ctx_k_pe[old]),
                     dev(case.ctx_slots[old]))
        c, r, s = dev_bf16(step["c"]), dev_bf16(step["r"]), dev(step["s"])
        args = (dev_bf16(case.q_nope), dev_bf16(case.q_pe), dev(case.block_tables), dev(case.context_lens))
        if fused:
            out, lse = mla.decode(cache, case.layer, *args, scale=case.scale, new_tokens=(c, r, s), **kw)
        else:
            mla.write_kv(cache, case.layer, c, r, s)
            out, lse = mla.decode(cache, case.layer, *args, scale=case.scale, **kw)
        torch.cuda.synchronize()
        res.append((cache_bits(cache), bf16_host_bits(out), lse.cpu().numpy().view(np.uint32)))
    return res


def step_tokens(case, last, n_pads, seed):
    old, new = split_rows(case, last)
    rng = np.random.default_rng(seed)
    c, r, s = with_pads(rng, case.ctx_c_kv[new], case.ctx_k_pe[new], case.ctx_slots[new], n_pads)
    return dict(split=(old, new), c=c, r=r, s=s)


# newest token only (a decode step), and the last up to 40 tokens of each
# request (several extra workgroup columns of the absorb launch)
@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
@pytest.mark.parametrize("many", [False, True])
@pytest.mark.parametrize("route", ["mfma", "generic", "latent"])
def test_decode_write_equals_write_then_decode(mla, kv, many, route):
    ctx = [1, 31, 33, 700, 2049, 64, 3000, 5]
    last = [min(c, 40) for c in ctx] if many else [1] * len(ctx)
    say(f"decode_write kv={kv} many={many} route={route}")
    case = W.custom(DIMS, ctx, seed=1200 + many, kv_dtype=kv, num_layers=2, layer=1, sharp=True)
    step = step_tokens(case, last, n_pads=3, seed=1210)
    kw = dict(w_uk=dev_bf16(case.w_uk), w_uv=dev_bf16(case.w_uv))
    if route == "generic":
        kw["flags"] = 1  # MLA_FLAG_GENERIC_KERNELS
    elif route == "latent":
        # latent queries (no W_UK, so no absorb launch): the query is q_nope . W_UK
        # precomputed on the host in bf16, out is the latent
        q = np.einsum("bhn,hnr->bhr", O.bf16_bits_to_f64(case.q_nope), O.bf16_bits_to_f64(case.w_uk))
        case.q_nope = W.f32_to_bf16_bits(q.astype(np.float32))
        kw = {}
    (ca, oa, la), (cb, ob, lb) = run_both(mla, case, step, **kw)
    assert np.array_equal(ca[0], cb[0]), f"{int((ca[0] != cb[0]).sum())} cache elements differ"
    if kv == O.KV_FP8:
        assert np.array_equal(ca[1], cb[1]), "fp8 scales differ"
    assert np.array_equal(oa, ob), f"{int((oa != ob).sum())} outputs differ"
    assert np.array_equal(la, lb)
    if route == "mfma":
        # the decode over the step's cache equals the oracle's
        hc = np.full((2, case.num_pages, DIMS.page_size, DIMS.D),
                     W.BF16_NAN if kv == O.KV_BF16 else W.E4M3_NAN,
                     dtype=np.uint16 if kv == O.KV_BF16 else np.uint8)
        hs = np.full((2, case.num_pages, DIMS.page_size), np.nan, dtype=np.float32)
        old, _ = step["split"]
        O.write_kv(hc, hs, 1, case.ctx_c_kv[old], case.ctx_k_pe[old], case.ctx_slots[old], kv)
        O.write_kv(hc, hs, 1, step["c"], step["r"], step["s"], kv)
        assert np.array_equal(cb[0], hc), "decode_write's cache differs from the oracle's write"
        ref, _ = O.decode(hc, hs, kv, 1, case.q_nope, case.q_pe, case.block_tables, case.context_lens,
                          case.w_uk, case.w_uv, case.scale, 0)
        assert_close(O.bf16_bits_to_f64(ob), ref, FP8_TOL if kv == O.KV_FP8 else BF16_TOL,
                     f"decode_write kv={kv} many={many}")


def test_decode_write_with_no_requests_writes_only(mla):
    say("decode_write batch 0")
    case = W.custom(DIMS, [300, 17], seed=1220, num_layers=2, layer=1)
    step = step_tokens(case, [300, 17], n_pads=5, seed=1221)
    caches = []
    for fused in (False, True):
        cache = new_device_cache(mla, 2, case.num_pages, DIMS, O.KV_BF16)
        c, r, s = dev_bf16(step["c"]), dev_bf16(step["r"]), dev(step["s"])
        if fused:
            q0 = torch.empty((0, DIMS.H, DIMS.Dn), dtype=torch.bfloat16, device="cuda")
            p0 = torch.empty((0, DIMS.H, DIMS.Dr), dtype=torch.bfloat16, device="cuda")
            out, lse = mla.decode(cache, 1, q0, p0, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                                  torch.zeros(0, dtype=torch.int32, device="cuda"), scale=case.scale,
                                  w_uk=dev_bf16(case.w_uk), w_uv=dev_bf16(case.w_uv), new_tokens=(c, r, s))
            assert out.shape[0] == 0
        else:
            mla.write_kv(cache, 1, c, r, s)
        torch.cuda.synchronize()
        caches.append(cache_bits(cache)[0])
    assert np.array_equal(caches[0], caches[1])


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
def test_decode_write_two_item_blocks(mla, kv):
    """48 requests: the absorb launch's workgroups each take two 32-item
    blocks of one W_UK column block, beside the plan's and the new tokens'
    workgroups; the result is still write-then-decode's, and the oracle's."""
    ctx = [1, 31, 33, 700, 2049, 64, 3000, 5] * 6
    say(f"decode_write kv={kv} B={len(ctx)}")
    case = W.custom(DIMS, ctx, seed=1230, kv_dtype=kv, num_layers=2, layer=1, sharp=True)
    step = step_tokens(case, [1] * len(ctx), n_pads=2, seed=1231)
    kw = dict(w_uk=dev_bf16(case.w_uk), w_uv=dev_bf16(case.w_uv))
    (ca, oa, la), (cb, ob, lb) = run_both(mla, case, step, **kw)
    assert np.array_equal(ca[0], cb[0]), f"{int((ca[0] != cb[0]).sum())} cache elements differ"
    assert np.array_equal(oa, ob), f"{int((oa != ob).sum())} outputs differ"
    assert np.array_equal(la, lb)
    hc = np.full((2, case.num_pages, DIMS.page_size, DIMS.D),
                 W.BF16_NAN if kv == O.KV_BF16 else W.E4M3_NAN,
                 dtype=np.uint16 if kv == O.KV_BF16 else np.uint8)
    hs = np.full((2, case.num_pages, DIMS.page_size), np.nan, dtype=np.float32)
    old, _ = step["split"]
    O.write_kv(hc, hs, 1, case.ctx_c_kv[old], case.ctx_k_pe[old], case.ctx_slots[old], kv)
    O.write_kv(hc, hs, 1, step["c"], step["r"], step["s"], kv)
    ref, _ = O.decode(hc, hs, kv, 1, case.q_nope, case.q_pe, case.block_tables, case.context_lens,
                      case.w_uk, case.w_uv, case.scale, 0)
    assert_close(O.bf16_bits_to_f64(ob), ref, FP8_TOL if kv == O.KV_FP8 else BF16_TOL,
                 f"decode_write kv={kv} B={len(ctx)}")
