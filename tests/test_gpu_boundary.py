"""GPU tests of the boundary's promises, through the C ABI:

* the calls read only the buffers passed: a workspace filled with NaN before
  every call gives the same bits as a zeroed one (no stale partial slot, plan
  entry or flag is ever read);
* write + decode captured in a HIP graph replay to the eager result, also after
  the block tables, context lengths and queries are rewritten in place
  ("[unified-memory] Let Kimi-Linear use the paged MLA attention backends",
  Cuda-graph safety and Correction: a backend that copied its block table at
  plan time gave silently wrong output under capture only);
* the MLA_DEBUG_CHECK host path rejects the device-array contract violations
  ("[unified-memory] ...", Two pre-existing issues, item 1);
* calls from two host threads on two streams give the single-thread bits.
"""
import threading

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, bf16_host_bits, bf16_host_f64, dev,
                         dev_bf16, host_cache, oracle_decode, populate_device, say, weights)

pytestmark = pytest.mark.gpu

MLA_DIMS = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def filled_workspace(mla, nbytes, fill):
    ws = mla.Workspace()
    ws.buf = torch.empty(max(nbytes, 256) // 4 + 1, dtype=torch.float32, device="cuda").fill_(fill)
    ws.buf = ws.buf.view(torch.uint8)
    return ws


def ws_bytes(mla, case, cache, G=0, prefill=False):
    w_uk, w_uv = weights(case)
    attn = mla._attn_struct(case.dims.H, case.dims.Dn, case.dims.Dv, w_uk, w_uv, case.scale,
                            case.window, G, 0)
    if prefill:
        return mla.prefill_workspace_size(cache, attn, case.batch, int(case.q_nope.shape[0]),
                                          case.max_blocks)
    return mla.decode_workspace_size(cache, attn, case.batch, case.max_blocks)


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
@pytest.mark.parametrize("G", [0, 5])
def test_decode_reads_no_stale_workspace(mla, kv, G):
    say(f"NaN workspace decode kv={kv} G={G}")
    ctx = [1, 31, 33, 700, 2049, 64, 3000, 5]
    case = W.custom(MLA_DIMS, ctx, seed=900 + G, kv_dtype=kv, sharp=True)
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    nbytes = ws_bytes(mla, case, cache, G)
    outs = []
    for fill in (0.0, float("nan"), float("nan")):
        ws = filled_workspace(mla, nbytes, fill)
        out, lse = mla.decode(cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe),
                              dev(case.block_tables), dev(case.context_lens), scale=case.scale,
                              w_uk=w_uk, w_uv=w_uv, workspace=ws, num_workgroups=G)
        torch.cuda.synchronize()
        outs.append((bf16_host_bits(out), lse.cpu().numpy()))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0])
        assert np.array_equal(l.view(np.uint32), outs[0][1].view(np.uint32))
    ref, _ = oracle_decode(case, host_cache(case))
    assert_close(O.bf16_bits_to_f64(outs[1][0]), ref, FP8_TOL if kv == O.KV_FP8 else BF16_TOL,
                 f"NaN workspace kv={kv} G={G}")


def test_prefill_reads_no_stale_workspace(mla):
    say("NaN workspace prefill")
    case = W.prefill_case(W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64),
                          [0, 37, 900], [100, 120, 80], seed=950, window=50, sharp=True)
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    nbytes = ws_bytes(mla, case, cache, prefill=True)
    outs = []
    for fill in (0.0, float("nan")):
        ws = filled_workspace(mla, nbytes, fill)
        out, lse = mla.prefill_chunk(cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe),
                                     dev(case.query_start_loc), 120, dev(case.block_tables),
                                     dev(case.context_lens), scale=case.scale, w_uk=w_uk,
                                     w_uv=w_uv, window=case.window, workspace=ws)
        torch.cuda.synchronize()
        outs.append((bf16_host_bits(out), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
def test_graph_capture_replays_after_in_place_rewrite(mla, kv):
    """Capture mla_write_kv + mla_decode once; then rewrite block tables,
    context lengths and queries in place and replay.  Every replay equals an
    eager call on the same inputs bit for bit."""
    say(f"graph capture kv={kv}")
    d = MLA_DIMS
    a = W.custom(d, [100, 3000, 777, 2049], seed=960, kv_dtype=kv, sharp=True)
    b = W.custom(d, [2500, 1, 64, 1500], seed=961, kv_dtype=kv, sharp=True)
    # both populations in one cache: request pages of b placed after a's
    num_pages = a.num_pages + b.num_pages
    bt_b = b.block_tables + a.num_pages
    max_blocks = max(a.max_blocks, b.max_blocks)
    cache = mla.KVCache.empty(1, num_pages, d.page_size, d.R, d.Dr, fp8=(kv == O.KV_FP8))
    if cache.fp8:
        cache.data.fill_(int(W.E4M3_NAN))
        cache.scale.fill_(float("nan"))
    else:
        cache.data.view(torch.int16).fill_(int(W.BF16_NAN))
    slots_b = W.slots_for(bt_b, b.context_lens, d.page_size)
    mla.write_kv(cache, 0, dev_bf16(a.ctx_c_kv), dev_bf16(a.ctx_k_pe), dev(a.ctx_slots))
    mla.write_kv(cache, 0, dev_bf16(b.ctx_c_kv), dev_bf16(b.ctx_k_pe), dev(slots_b))

    def table(bt):
        t = np.full((bt.shape[0], max_blocks), num_pages - 1, dtype=np.int32)
        t[:, :bt.shape[1]] = bt
        return t

    # the step's write: each request's newest token again (same bytes)
    def newest(case, slots):
        rows = case.new_token_rows()
        return dev_bf16(case.ctx_c_kv[rows]), dev_bf16(case.ctx_k_pe[rows]), dev(slots[rows])

    w_uk, w_uv = dev_bf16(a.w_uk), dev_bf16(a.w_uv)
    B, H = a.batch, d.H
    q_nope = dev_bf16(a.q_nope)
    q_pe = dev_bf16(a.q_pe)
    bt = dev(table(a.block_tables))
    ctx = dev(a.context_lens)
    new_c, new_r, new_s = newest(a, a.ctx_slots)
    out = torch.empty((B, H, d.Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = mla.Workspace()
    s = torch.cuda.Stream()

    def step():
        mla.write_kv(cache, 0, new_c, new_r, new_s)
        mla.decode(cache, 0, q_nope, q_pe, bt, ctx, scale=a.scale, w_uk=w_uk, w_uv=w_uv, out=out,
                   lse=lse, workspace=ws)

    with torch.cuda.stream(s):
        step()  # eager: loads the kernels and sizes the workspace
    torch.cuda.synchronize()
    eager_a = (bf16_host_bits(out), lse.cpu().numpy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()

    def replay_check(expect, what):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host_bits(out), expect[0]), what
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), expect[1].view(np.uint32)), what

    for k in range(3):
        replay_check(eager_a, f"replay {k} of the captured inputs")
        _ = torch.randn(1 << 20, device="cuda").sum().item()  # unrelated eager work in between

    # rewrite the captured inputs in place with request set b
    bt.copy_(dev(table(bt_b)))
    ctx.copy_(dev(b.context_lens))
    q_nope.copy_(dev_bf16(b.q_nope))
    q_pe.copy_(dev_bf16(b.q_pe))
    nc, nr, ns = newest(b, slots_b)
    new_c.copy_(nc)
    new_r.copy_(nr)
    new_s.copy_(ns)
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager_b = (bf16_host_bits(out), lse.cpu().numpy())
    for k in range(3):
        replay_check(eager_b, f"replay {k} after the in-place rewrite")
    # and the replayed b is the oracle's b
    hc = np.full((1, num_pages, d.page_size, d.D), W.BF16_NAN if kv == O.KV_BF16 else W.E4M3_NAN,
                 dtype=np.uint16 if kv == O.KV_BF16 else np.uint8)
    hs = np.full((1, num_pages, d.page_size), np.nan, dtype=np.float32)
    O.write_kv(hc, hs, 0, b.ctx_c_kv, b.ctx_k_pe, slots_b, kv)
    ref, _ = O.decode(hc, hs, kv, 0, b.q_nope, b.q_pe, table(bt_b), b.context_lens, a.w_uk, a.w_uv,
                      b.scale, 0)
    assert_close(O.bf16_bits_to_f64(eager_b[0]), ref, FP8_TOL if kv == O.KV_FP8 else BF16_TOL,
                 f"graph replay b kv={kv}")


def test_debug_check_rejects_contract_violations(mla, monkeypatch):
    say("MLA_DEBUG_CHECK")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [10, 70], [5, 9], seed=970)
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    monkeypatch.setenv("MLA_DEBUG_CHECK", "1")
    bt, ctx, qsl = case.block_tables, case.context_lens, case.query_start_loc

    def dec(bt=bt, ctx=ctx):
        return mla.decode(cache, 0, dev_bf16(case.q_nope[:2]), dev_bf16(case.q_pe[:2]), dev(bt),
                          dev(ctx), scale=case.scale, w_uk=w_uk, w_uv=w_uv)

    def pre(qsl=qsl, ctx=ctx, max_q=9):
        return mla.prefill_chunk(cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe), dev(qsl),
                                 max_q, dev(bt), dev(ctx), scale=case.scale, w_uk=w_uk, w_uv=w_uv)

    def rejected(fn, **kw):
        with pytest.raises(mla.MlaError) as e:
            fn(**kw)
        assert e.value.status == mla.MLA_ERR_INVALID_ARGUMENT

    good, _ = dec()
    monkeypatch.delenv("MLA_DEBUG_CHECK")
    plain, _ = dec()
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_bits(good), bf16_host_bits(plain))
    monkeypatch.setenv("MLA_DEBUG_CHECK", "1")
    pre()
    too_long = ctx.copy()
    too_long[1] = bt.shape[1] * d.page_size + 1
    rejected(dec, ctx=too_long)
    negative = ctx.copy()
    negative[0] = -3
    rejected(dec, ctx=negative)
    bad_page = bt.copy()
    bad_page[1, 0] = case.num_pages
    rejected(dec, bt=bad_page)
    bad_qsl = qsl.copy()
    bad_qsl[-1] += 1  # disagrees with total_q_tokens
    rejected(pre, qsl=bad_qsl)
    rejected(pre, max_q=8)  # a chunk longer than max_q_len
    short_ctx = ctx.copy()
    short_ctx[0] = 2      # chunk of 5 rows in a 2-token context
    rejected(pre, ctx=short_ctx)
    c_kv, k_pe = dev_bf16(case.ctx_c_kv[:3]), dev_bf16(case.ctx_k_pe[:3])
    with pytest.raises(mla.MlaError):
        mla.write_kv(cache, 0, c_kv, k_pe, dev(np.array([4, -1, 4], np.int64)))  # duplicate slot
    with pytest.raises(mla.MlaError):
        mla.write_kv(cache, 0, c_kv, k_pe, dev(np.array([0, 1, case.num_pages * 64], np.int64)))
    mla.write_kv(cache, 0, c_kv, k_pe, dev(case.ctx_slots[:3]))  # valid: passes


def test_two_threads_two_streams(mla):
    """Concurrent calls from two host threads, each with its own stream,
    workspace and outputs, give the single-thread bits."""
    say("two threads")
    cases = [W.custom(MLA_DIMS, ctx, seed=980 + i, sharp=True)
             for i, ctx in enumerate(([500, 3000, 40], [2049, 7, 1200, 64]))]
    caches = [populate_device(mla, c) for c in cases]
    args = []
    for c in cases:
        w_uk, w_uv = weights(c)
        args.append((dev_bf16(c.q_nope), dev_bf16(c.q_pe), dev(c.block_tables), dev(c.context_lens),
                     w_uk, w_uv, c.scale))
    ref = []
    for cache, (qn, qp, bt, ctx, w_uk, w_uv, sc) in zip(caches, args):
        out, _ = mla.decode(cache, 0, qn, qp, bt, ctx, scale=sc, w_uk=w_uk, w_uv=w_uv)
        torch.cuda.synchronize()
        ref.append(bf16_host_bits(out))
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            cache, (qn, qp, bt, ctx, w_uk, w_uv, sc) = caches[i], args[i]
            ws = mla.Workspace()
            with torch.cuda.stream(s):
                for _ in range(10):
                    out, _ = mla.decode(cache, 0, qn, qp, bt, ctx, scale=sc, w_uk=w_uk, w_uv=w_uv,
                                        workspace=ws, stream=s)
                s.synchronize()
                if not np.array_equal(bf16_host_bits(out), ref[i]):
                    errors.append(f"thread {i}: output differs")
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(f"thread {i}: {e!r}")

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in th), "a thread did not finish"
    assert not errors, errors
