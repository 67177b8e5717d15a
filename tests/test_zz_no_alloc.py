"""mla_decode_noalloc (the library-owned scratch array as workspace) against
mla_decode with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller input, each bit-identical to the workspace call
(same kernels, same work partition) and within the bf16 tolerance of the
oracle; a call needing more than the scratch array holds is refused before
anything is enqueued."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, bf16_host_bits, dev, dev_bf16,
                         host_cache, oracle_decode, populate_device, say, weights)

pytestmark = pytest.mark.gpu

MLA_DIMS = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def run_both(mla, case, cache):
    w_uk, w_uv = weights(case)
    args = (cache, case.layer, dev_bf16(case.q_nope), dev_bf16(case.q_pe), dev(case.block_tables),
            dev(case.context_lens))
    kw = dict(scale=case.scale, w_uk=w_uk, w_uv=w_uv, window=case.window)
    out_ws, lse_ws = mla.decode(*args, **kw)
    out = torch.empty_like(out_ws)
    lse = torch.empty_like(lse_ws)
    mla.decode_noalloc(*args, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return (bf16_host_bits(out_ws), lse_ws.cpu().numpy()), (bf16_host_bits(out), lse.cpu().numpy())


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
def test_noalloc_matches_workspace_call_twice(mla, kv):
    tol = FP8_TOL if kv == O.KV_FP8 else BF16_TOL
    big = W.custom(MLA_DIMS, [3000, 5000, 33, 2049, 700, 1, 4096, 129], seed=990, kv_dtype=kv,
                   sharp=True)
    small = W.custom(MLA_DIMS, [65, 300, 7], seed=991, kv_dtype=kv, sharp=True, window=100)
    for label, case in (("first (8 requests)", big), ("second (3 requests, window)", small)):
        say(f"noalloc {kv} {label}")
        cache = populate_device(mla, case)
        (o_ws, l_ws), (o_na, l_na) = run_both(mla, case, cache)
        assert np.array_equal(o_na, o_ws), f"{label}: outputs differ from the workspace call"
        assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32)), f"{label}: lse differs"
        ref, _ = oracle_decode(case, host_cache(case))
        assert_close(O.bf16_bits_to_f64(o_na), ref, tol, f"noalloc {kv} {label}")


def test_noalloc_refuses_oversized_and_allocates_nothing(mla):
    say("noalloc refusal")
    case = W.custom(MLA_DIMS, [100, 200], seed=992, sharp=True)
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    out = torch.empty((2, 128, 128), dtype=torch.bfloat16, device="cuda")
    # 4096 forced workgroups: the partial slots alone need 2 x 4096 x 128 x 512 x 4 B = 2 GiB
    with pytest.raises(mla.MlaError) as e:
        mla.decode_noalloc(cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe),
                           dev(case.block_tables), dev(case.context_lens), scale=case.scale,
                           w_uk=w_uk, w_uv=w_uv, out=out, num_workgroups=4096)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
    # a normal call after the refusal, with the caching allocator's counters
    # unchanged by the call itself
    q_nope, q_pe = dev_bf16(case.q_nope), dev_bf16(case.q_pe)
    bt, ctx = dev(case.block_tables), dev(case.context_lens)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    mla.decode_noalloc(cache, 0, q_nope, q_pe, bt, ctx, scale=case.scale, w_uk=w_uk, w_uv=w_uv,
                       out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    ref, _ = oracle_decode(case, host_cache(case))
    assert_close(O.bf16_bits_to_f64(bf16_host_bits(out)), ref, BF16_TOL, "noalloc after refusal")
