"""Index-list (top-k) attention on the GPU (mla_sparse_attention through the C
ABI) against the oracle's sparse_attention: decode and prefill rows, bf16 and
fp8 caches, windows, lists with unused slots and positions the row must
ignore, empty lists, and query rows spread over several compaction chunks.
Tolerances as for the dense calls."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, assert_lse_close, bf16_host_f64, dev,
                         dev_bf16, host_cache, populate_device, say, weights)

pytestmark = pytest.mark.gpu

LSE_ATOL = {O.KV_BF16: 2e-2, O.KV_FP8: 5e-2}


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def query_positions(case):
    """Each query row's position and its request's context length."""
    if case.query_start_loc is None:
        return case.context_lens - 1, case.context_lens
    pos, ctx = [], []
    for b in range(case.batch):
        s0, s1 = int(case.query_start_loc[b]), int(case.query_start_loc[b + 1])
        n = int(case.context_lens[b])
        for i in range(s1 - s0):
            pos.append(n - (s1 - s0) + i)
            ctx.append(n)
    return np.array(pos), np.array(ctx)


def run_sparse(mla, case, lists, window=0):
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    prefill = case.query_start_loc is not None
    out, lse = mla.sparse_attention(
        cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe), dev(lists), dev(case.block_tables),
        dev(case.context_lens), scale=case.scale, w_uk=w_uk, w_uv=w_uv, window=window,
        query_start_loc=dev(case.query_start_loc) if prefill else None,
        max_q_len=int(np.max(np.diff(case.query_start_loc))) if prefill else 0)
    torch.cuda.synchronize()
    hc, hs = host_cache(case)
    ref, ref_lse = O.sparse_attention(hc, hs, case.kv_dtype, 0, case.q_nope, case.q_pe, lists,
                                      case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                      case.scale, window, query_start_loc=case.query_start_loc)
    return bf16_host_f64(out), lse.cpu().numpy(), ref, ref_lse


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
@pytest.mark.parametrize("window", [0, 500])
def test_sparse_decode(mla, kv, window):
    say(f"sparse decode kv={kv} window={window}")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [3000, 5000, 700, 33, 1, 4096, 2049, 129], seed=1300 + window, kv_dtype=kv,
                    sharp=True)
    pos, ctx = query_positions(case)
    lists = W.key_lists(1301, pos, ctx, 2048)
    got, lse, ref, ref_lse = run_sparse(mla, case, lists, window)
    tol = FP8_TOL if kv == O.KV_FP8 else BF16_TOL
    assert_close(got, ref, tol, f"sparse decode kv={kv} w={window}")
    assert_lse_close(lse, ref_lse, LSE_ATOL[kv], "sparse decode lse")


def test_sparse_prefill_several_chunks(mla):
    """300 prefill rows with 2048-entry lists: more rows than one 512 MiB
    compaction chunk holds, so the rows run in two chunks."""
    say("sparse prefill, 300 rows, topk 2048")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [4000, 37, 2500], [100, 120, 80], seed=1310, sharp=True)
    pos, ctx = query_positions(case)
    lists = W.key_lists(1311, pos, ctx, 2048)
    got, lse, ref, ref_lse = run_sparse(mla, case, lists)
    assert_close(got, ref, BF16_TOL, "sparse prefill")
    assert_lse_close(lse, ref_lse, LSE_ATOL[O.KV_BF16], "sparse prefill lse")


def test_sparse_lists_equal_to_ranges(mla):
    """A list holding a row's whole visible range gives the dense call's
    answer; the window as a list gives the windowed call's; empty lists give
    zeros and -inf."""
    say("sparse lists as ranges")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [1500, 64, 333, 1], seed=1320, sharp=True)
    n = case.context_lens
    full = np.full((case.batch, 1600), -1, np.int32)
    win = np.full((case.batch, 1600), -1, np.int32)
    empty = np.full((case.batch, 64), -1, np.int32)
    rng = np.random.default_rng(1321)
    for b in range(case.batch):
        full[b, :n[b]] = rng.permutation(int(n[b]))
        w0 = max(0, int(n[b]) - 100)
        win[b, :n[b] - w0] = np.arange(w0, n[b])[::-1]
    got, _, ref, _ = run_sparse(mla, case, full)
    dense, _ = O.decode(*host_cache(case), case.kv_dtype, 0, case.q_nope, case.q_pe,
                        case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale, 0)
    assert np.max(np.abs(ref - dense)) < 1e-12
    assert_close(got, dense, BF16_TOL, "sparse full list vs dense")
    got, _, _, _ = run_sparse(mla, case, win)
    dense_w, _ = O.decode(*host_cache(case), case.kv_dtype, 0, case.q_nope, case.q_pe,
                          case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale, 100)
    assert_close(got, dense_w, BF16_TOL, "sparse window list vs windowed decode")
    got, lse, _, _ = run_sparse(mla, case, empty)
    assert (got == 0).all() and np.isneginf(lse).all()
