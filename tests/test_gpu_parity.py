"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Writes are compared bit for bit; attention outputs within
max-abs 2e-2 / rel-L2 5e-3 (bf16 cache) or 0.1 / 3e-2 (fp8 cache), over the
call's output tensor.  At full sizes every request is compared; the mixed
step's prefill compares every 8th row of each chunk plus its last row."""
import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, assert_lse_close, bf16_host_bits,
                         bf16_host_f64, dev, dev_bf16, gpu_decode, host_cache, new_device_cache,
                         oracle_decode, populate_device, say, weights)

pytestmark = pytest.mark.gpu

# lse has no stated tolerance; these are about 8 standard deviations of the
# error that rounding q_lat to bf16 puts into the scores in the sharp regime.
LSE_ATOL = {O.KV_BF16: 2e-2, O.KV_FP8: 5e-2}


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def tol_for(case):
    return FP8_TOL if case.kv_dtype == O.KV_FP8 else BF16_TOL


# ---------------------------------------------------------------------------
# mla_write_kv: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", [O.KV_BF16, O.KV_FP8])
def test_write_kv_bit_exact_with_pads_layers_and_overwrite(mla, kv_dtype):
    say(f"write_kv bit-exact {kv_dtype}")
    d = W.Dims(H=4, R=512, Dr=64, Dn=128, Dv=128, page_size=16)
    case = W.custom(d, [5, 40, 77], seed=101, kv_dtype=kv_dtype, num_layers=3, layer=1)
    # pad rows interleaved with real ones
    T = case.ctx_slots.size
    slots = case.ctx_slots.copy()
    slots[::7] = -1
    cache = new_device_cache(mla, 3, case.num_pages, d, kv_dtype)
    mla.write_kv(cache, 1, dev_bf16(case.ctx_c_kv), dev_bf16(case.ctx_k_pe), dev(slots))
    # overwrite the first few live tokens with new values
    rng = np.random.default_rng(5)
    new_c = W.bf16_normal(rng, (4, d.R), 0.3)
    new_r = W.bf16_normal(rng, (4, d.Dr), 0.3)
    live = np.nonzero(slots >= 0)[0][:4]
    mla.write_kv(cache, 1, dev_bf16(new_c), dev_bf16(new_r), dev(slots[live]))
    torch.cuda.synchronize()

    fill = W.BF16_NAN if kv_dtype == O.KV_BF16 else W.E4M3_NAN
    dt = np.uint16 if kv_dtype == O.KV_BF16 else np.uint8
    hc = np.full((3, case.num_pages, d.page_size, d.D), fill, dtype=dt)
    hs = np.full((3, case.num_pages, d.page_size), np.nan, dtype=np.float32)
    O.write_kv(hc, hs, 1, case.ctx_c_kv, case.ctx_k_pe, slots, kv_dtype)
    O.write_kv(hc, hs, 1, new_c, new_r, slots[live], kv_dtype)
    if kv_dtype == O.KV_BF16:
        got = bf16_host_bits(cache.data)
    else:
        got = cache.data.cpu().numpy()
        gs = cache.scale.cpu().numpy()
        assert np.array_equal(gs.view(np.uint32), hs.view(np.uint32)), "fp8 scales differ"
    assert got.shape == hc.shape
    assert np.array_equal(got, hc), f"{int((got != hc).sum())} cache elements differ"
    assert T > 0


@pytest.fixture(scope="module")
def v3fp8_population(mla):
    """The V3 fp8 workload's cache, written once: on the device by
    mla_write_kv, on the host by the oracle's write.  Plain and sharp variants
    share it (their queries differ, their population does not)."""
    case = W.v3fp8()
    say("v3fp8 population: device write + oracle write")
    cache = populate_device(mla, case)
    hc = host_cache(case)
    yield case, cache, hc
    del cache
    torch.cuda.empty_cache()


def test_write_fp8_full_size_every_token(mla, v3fp8_population):
    """fp8 quantisation at the V3 fp8 workload's size (128 requests x 8192
    tokens): the whole device cache, codes and scales, equals the oracle's
    byte for byte, unused rows included."""
    say("write_kv fp8 v3fp8 population, every byte")
    case, cache, (hc, hs) = v3fp8_population
    got = cache.data.cpu().numpy()
    assert got.shape == hc.shape
    diff = int(np.count_nonzero(got != hc))
    assert diff == 0, f"{diff} code bytes differ"
    gs = cache.scale.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), hs.view(np.uint32)), "fp8 scales differ"


def test_write_fp8_codec_edges(mla):
    """Values at every E4M3 midpoint, the saturation bound and zeros, written
    through the fp8 cache (one token per row, scale forced to 1 by amax 448)."""
    say("write_kv fp8 codec edges")
    mags = O.E4M3_TABLE[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, -mids, O.E4M3_TABLE[:0x7F].astype(np.float32), [0.0, -0.0]])
    # only bf16-representable values survive the bf16 input; keep those
    bits = W.f32_to_bf16_bits(vals)
    keep = O.bf16_bits_to_f32(bits) == vals
    vals = vals[keep]
    D = 64
    n_val = (len(vals) + D - 2) // (D - 1)
    n_tok = n_val + 2
    rows = np.zeros((n_tok, D), dtype=np.float32)
    flat = np.concatenate([vals, np.zeros(n_val * (D - 1) - len(vals), np.float32)])
    rows[2:, 1:] = flat.reshape(n_val, D - 1)
    rows[2:, 0] = 448.0  # amax 448 -> scale exactly 1
    rows[1, 0] = 448.0
    rows[1, 1:] = -0.0   # signed zeros keep their sign
    # row 0 stays all zero: scale 1.0, codes 0
    row_bits = W.f32_to_bf16_bits(rows)
    d = W.Dims(H=1, R=48, Dr=16, Dn=8, Dv=8, page_size=16)
    cache = new_device_cache(mla, 1, (n_tok + 15) // 16 + 1, d, O.KV_FP8)
    slots = np.arange(n_tok, dtype=np.int64)
    mla.write_kv(cache, 0, dev_bf16(row_bits[:, :48]), dev_bf16(row_bits[:, 48:]), dev(slots))
    torch.cuda.synchronize()
    codes, scl = O.fp8_quantize_tokens(row_bits)
    got = cache.data[0].view(-1, D)[:n_tok].cpu().numpy()
    gs = cache.scale[0].reshape(-1)[:n_tok].cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), scl.view(np.uint32))
    assert np.array_equal(got, codes)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def check_decode(mla, case, requests=None, flags=0, num_workgroups=0, tol=None, label=""):
    cache = populate_device(mla, case)
    out, lse = gpu_decode(mla, case, cache, flags=flags, num_workgroups=num_workgroups)
    hc = host_cache(case)
    ref, ref_lse = oracle_decode(case, hc, requests=requests)
    sel = slice(None) if requests is None else list(requests)
    got = bf16_host_f64(out)[sel]
    assert_close(got, ref[sel], tol or tol_for(case), f"{case.name}{label} out")
    assert_lse_close(lse.cpu().numpy()[sel], ref_lse[sel], LSE_ATOL[case.kv_dtype], f"{case.name}{label} lse")
    return cache, out, lse


@pytest.mark.parametrize("sharp", [False, True])
def test_decode_tiny(mla, sharp):
    say(f"decode tiny sharp={sharp}")
    check_decode(mla, W.tiny(sharp=sharp))


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("sharp", [False, True])
def test_decode_v2lite(mla, sharp, flags):
    say(f"decode v2lite sharp={sharp} flags={flags}")
    check_decode(mla, W.v2lite(sharp=sharp), flags=flags)


@pytest.mark.parametrize("sharp", [False, True])
def test_decode_v3_full_size(mla, sharp):
    """DeepSeek-V3 shape, every one of the 64 requests compared."""
    say(f"decode v3 sharp={sharp}")
    check_decode(mla, W.v3(sharp=sharp))


@pytest.mark.parametrize("f8mfma", [False, True])
@pytest.mark.parametrize("sharp", [False, True])
def test_decode_v3fp8_full_size(mla, v3fp8_population, sharp, f8mfma):
    """V3 shape over the fp8 cache, every one of the 128 requests compared;
    also with the fp8 matrix cores (queries and probabilities in E4M3)."""
    say(f"decode v3fp8 sharp={sharp} f8mfma={f8mfma}")
    base, cache, hcache = v3fp8_population
    case = W.v3fp8(sharp=sharp)
    assert np.array_equal(case.ctx_slots, base.ctx_slots)
    assert np.array_equal(case.ctx_c_kv[::4096], base.ctx_c_kv[::4096])
    out, lse = gpu_decode(mla, case, cache, flags=mla.MLA_FLAG_FP8_MFMA if f8mfma else 0)
    ref, ref_lse = oracle_decode(case, hcache)
    tag = f"v3fp8 sharp={sharp} f8mfma={f8mfma}"
    assert_close(bf16_host_f64(out), ref, FP8_TOL, f"{tag} out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, LSE_ATOL[O.KV_FP8], f"{tag} lse")


@pytest.mark.parametrize("G", [1, 3, 7, 1000])
def test_decode_forced_partitions(mla, G):
    """The split plan: any workgroup count gives the oracle's answer."""
    say(f"decode forced G={G}")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [1, 31, 32, 33, 64, 65, 700, 2049], seed=201, sharp=True)
    check_decode(mla, case, num_workgroups=G, label=f" G={G}")


@pytest.mark.parametrize("B", [40, 72])
@pytest.mark.parametrize("G", [1, 3, 7, 1000])
def test_decode_forced_partitions_wide_batch(mla, G, B):
    """128 heads and 40 or 72 requests: enough 32-item blocks x heads to fill
    the chip, so the combine runs its 32-items-per-workgroup forms -- up to
    eight segments per round trip with 256 workgroups (40 requests: as many
    as a 256-CU chip has compute units), four with 384 (72 requests) -- whose
    merge of cut items (several rounds of segments, empty ranges, both
    partial slots of a workgroup) is then checked in full."""
    say(f"decode forced G={G}, 128 heads x {B} requests")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    ctx = [1, 31, 32, 33, 64, 65, 700, 2049] * (B // 8)
    case = W.custom(d, ctx, seed=210 + G + (0 if B == 40 else 100), sharp=True)
    check_decode(mla, case, num_workgroups=G, label=f" G={G} B={B}")


@pytest.mark.parametrize("G", [1, 7, 1000])
def test_prefill_forced_partitions_many_rows(mla, G):
    """More query rows than compute units: the prefill-sized combine form,
    with rows cut across workgroups under every forced partition."""
    say(f"prefill forced G={G}, 300 rows")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [0, 37, 900], [100, 120, 80], seed=230 + G, sharp=True)
    check_prefill(mla, case, num_workgroups=G, label=f" G={G} rows=300")


@pytest.mark.parametrize("window", [1, 2, 31, 32, 33, 128, 5000])
def test_decode_windows(mla, window):
    say(f"decode window={window}")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [1, 2, 100, 129, 1000, 4097], seed=300 + window, sharp=True, window=window)
    check_decode(mla, case)


@pytest.mark.parametrize("ps", [16, 32, 128])
def test_decode_page_sizes(mla, ps):
    say(f"decode page size {ps}")
    d = W.Dims(H=32, R=512, Dr=64, Dn=128, Dv=128, page_size=ps)
    case = W.custom(d, [3, 200, 1111], seed=400 + ps, sharp=True)
    check_decode(mla, case)


def test_decode_edge_contexts(mla):
    """n = 0 (out 0, lse -inf), n = 1 (the token's value), mixed in one batch."""
    say("decode edge contexts")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [0, 1, 2, 0, 64], seed=500, sharp=True)
    cache, out, lse = check_decode(mla, case)
    o = bf16_host_f64(out)
    assert (o[0] == 0).all() and (o[3] == 0).all()
    assert np.isneginf(lse.cpu().numpy()[[0, 3]]).all()


def test_decode_page_permutation_bitwise(mla):
    """Physical page placement does not change a single output bit."""
    say("decode page permutation")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    base = W.custom(d, [100, 3000, 777], seed=600, sharp=True)
    outs = []
    for perm_seed in (1, 2):
        rng = np.random.default_rng(perm_seed)
        bt, npg, _ = W.assign_pages(rng, base.context_lens, 64, num_pages=base.num_pages + 5)
        c = W.Case(**{**base.__dict__, "block_tables": bt, "num_pages": npg,
                      "ctx_slots": W.slots_for(bt, base.context_lens, 64)})
        cache = populate_device(mla, c)
        out, lse = gpu_decode(mla, c, cache)
        outs.append((bf16_host_bits(out), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_decode_latent_io_and_needle(mla):
    """No W_UK / W_UV (latent query in, latent output out) and a needle query:
    the output is the needle token's latent."""
    say("decode latent io + needle")
    d = W.Dims(H=32, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [300, 41], seed=700)
    cache = populate_device(mla, case)
    j = 123
    c_j = O.bf16_bits_to_f64(case.ctx_c_kv[j])
    q_lat = np.zeros((2, d.H, d.R))
    q_lat[0] = 40.0 / (case.scale * (c_j @ c_j)) * c_j  # score gap >> 30 against the others
    q_bits = W.f32_to_bf16_bits(q_lat.astype(np.float32))
    out, lse = mla.decode(cache, 0, dev_bf16(q_bits), dev_bf16(case.q_pe), dev(case.block_tables),
                          dev(case.context_lens), scale=case.scale)
    torch.cuda.synchronize()
    hc = host_cache(case)
    ref, _ = O.decode(hc[0], hc[1], case.kv_dtype, 0, q_bits, case.q_pe, case.block_tables,
                      case.context_lens, None, None, case.scale, 0)
    assert_close(bf16_host_f64(out), ref, BF16_TOL, "latent io")
    assert np.max(np.abs(bf16_host_f64(out)[0] - c_j[None, :])) < 2e-2


@pytest.mark.parametrize("ps", [16, 32, 64, 128])
def test_decode_fp8_mfma_page_sizes(mla, ps):
    """fp8 cache on the matrix-core path: ragged contexts (tile edges, one-token
    and multi-page requests) over every supported page size, sharp queries."""
    say(f"decode fp8 mfma ps={ps}")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=ps)
    case = W.custom(d, [1, 31, 32, 33, 64, 65, 700, 2049], seed=710 + ps, kv_dtype=O.KV_FP8, sharp=True)
    check_decode(mla, case, label=f" ps={ps}")
    check_decode(mla, case, num_workgroups=7, label=f" ps={ps} G=7")


@pytest.mark.parametrize("window", [1, 33, 500])
def test_decode_fp8_mfma_window(mla, window):
    say(f"decode fp8 mfma window={window}")
    d = W.Dims(H=64, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [40, 700, 2049], seed=730 + window, kv_dtype=O.KV_FP8, window=window, sharp=True)
    check_decode(mla, case, label=f" w={window}")


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
@pytest.mark.parametrize("H", [40, 100])
def test_decode_mfma_partly_filled_waves(mla, kv, H):
    """Head counts that leave a wave partly filled (its lanes past H hold zero
    queries and store nothing) and, for 40 heads, whole waves without heads,
    which still copy -- and on the fp8 path convert -- their share of every
    tile; ragged contexts, sharp queries, one and several workgroups."""
    say(f"decode mfma H={H} {kv}")
    d = W.Dims(H=H, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [1, 33, 700, 2049], seed=750 + H, kv_dtype=kv, sharp=True)
    check_decode(mla, case, label=f" H={H}")
    check_decode(mla, case, num_workgroups=5, label=f" H={H} G=5")


@pytest.mark.parametrize("G", [1, 2])
def test_decode_fp8_score_jump_moves_the_reference(mla, G):
    """fp8 cache: a key whose score passes its segment's first-tile maximum by
    about 2^97 (log2 units) moves the matrix-core kernel's reference maximum
    up, with a rescale of the accumulators; the output is still the oracle's
    (the needle's latent)."""
    say(f"decode fp8 score jump G={G}")
    d = W.Dims(H=32, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [300, 41], seed=740, kv_dtype=O.KV_FP8)
    cache = populate_device(mla, case)
    hc, hs = host_cache(case)
    X = O.gather_latent(hc, hs, case.kv_dtype, 0, case.block_tables[0], int(case.context_lens[0]))
    j = 260  # tile 8 of request 0: not the first tile of its segment with one or two workgroups
    c_j = X[j, :d.R]
    q_lat = np.zeros((2, d.H, d.R))
    q_lat[0] = 70.0 / (case.scale * (c_j @ c_j)) * c_j
    q_bits = W.f32_to_bf16_bits(q_lat.astype(np.float32))
    out, lse = mla.decode(cache, 0, dev_bf16(q_bits), dev_bf16(case.q_pe), dev(case.block_tables),
                          dev(case.context_lens), scale=case.scale, num_workgroups=G)
    torch.cuda.synchronize()
    ref, ref_lse = O.decode(hc, hs, case.kv_dtype, 0, q_bits, case.q_pe, case.block_tables,
                            case.context_lens, None, None, case.scale, 0)
    assert_close(bf16_host_f64(out), ref, FP8_TOL, f"fp8 jump G={G}")
    assert_lse_close(lse.cpu().numpy(), ref_lse, LSE_ATOL[case.kv_dtype], f"fp8 jump G={G} lse")
    assert np.max(np.abs(bf16_host_f64(out)[0] - c_j[None, :])) < 2e-2


# ---------------------------------------------------------------------------
# fp8 matrix cores (MLA_FLAG_FP8_MFMA): queries as a two-term E4M3 expansion,
# probabilities in E4M3; an approximation held to the fp8 cache's tolerance
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ps", [16, 32, 64, 128])
def test_decode_f8mfma_page_sizes(mla, ps):
    """Ragged contexts (64-token step edges, one-token and multi-page
    requests) over every page size, sharp queries, one and seven workgroups
    (contexts cut at odd tiles: half-masked steps)."""
    say(f"decode f8mfma ps={ps}")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=ps)
    case = W.custom(d, [1, 31, 32, 33, 63, 64, 65, 700, 2049], seed=1710 + ps, kv_dtype=O.KV_FP8, sharp=True)
    f = mla.MLA_FLAG_FP8_MFMA
    check_decode(mla, case, flags=f, label=f" f8mfma ps={ps}")
    check_decode(mla, case, flags=f, num_workgroups=7, label=f" f8mfma ps={ps} G=7")


@pytest.mark.parametrize("sharp", [False, True])
@pytest.mark.parametrize("window", [1, 33, 500])
def test_decode_f8mfma_window(mla, window, sharp):
    say(f"decode f8mfma window={window} sharp={sharp}")
    d = W.Dims(H=64, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [40, 700, 2049], seed=1730 + window, kv_dtype=O.KV_FP8, window=window, sharp=sharp)
    check_decode(mla, case, flags=mla.MLA_FLAG_FP8_MFMA, label=f" f8mfma w={window}")


@pytest.mark.parametrize("H", [16, 40, 100])
def test_decode_f8mfma_partly_filled_waves(mla, H):
    """Head counts that leave waves partly filled or empty (those still copy
    their share of every step); forced partitions put items in split slots."""
    say(f"decode f8mfma H={H}")
    d = W.Dims(H=H, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [1, 33, 700, 2049], seed=1750 + H, kv_dtype=O.KV_FP8, sharp=True)
    f = mla.MLA_FLAG_FP8_MFMA
    check_decode(mla, case, flags=f, label=f" f8mfma H={H}")
    check_decode(mla, case, flags=f, num_workgroups=5, label=f" f8mfma H={H} G=5")


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("gap", [25.0, 70.0])
def test_decode_f8mfma_score_jump(mla, G, gap):
    """A key whose score passes its segment's first-step maximum by ~36
    octaves (the reference moves and later weights are scaled up through the
    matrix instruction's operand scale) or by ~97 (past 64 octaves the old
    contributions are dropped and the units restart): the output is still
    the oracle's, the needle's latent."""
    say(f"decode f8mfma score jump gap={gap} G={G}")
    d = W.Dims(H=32, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [300, 41], seed=740, kv_dtype=O.KV_FP8)
    cache = populate_device(mla, case)
    hc, hs = host_cache(case)
    X = O.gather_latent(hc, hs, case.kv_dtype, 0, case.block_tables[0], int(case.context_lens[0]))
    j = 260  # step 4 of request 0: not the first step of its segment with one or two workgroups
    c_j = X[j, :d.R]
    q_lat = np.zeros((2, d.H, d.R))
    q_lat[0] = gap / (case.scale * (c_j @ c_j)) * c_j
    q_bits = W.f32_to_bf16_bits(q_lat.astype(np.float32))
    out, lse = mla.decode(cache, 0, dev_bf16(q_bits), dev_bf16(case.q_pe), dev(case.block_tables),
                          dev(case.context_lens), scale=case.scale, num_workgroups=G,
                          flags=mla.MLA_FLAG_FP8_MFMA)
    torch.cuda.synchronize()
    ref, ref_lse = O.decode(hc, hs, case.kv_dtype, 0, q_bits, case.q_pe, case.block_tables,
                            case.context_lens, None, None, case.scale, 0)
    assert_close(bf16_host_f64(out), ref, FP8_TOL, f"f8mfma jump gap={gap} G={G}")
    assert_lse_close(lse.cpu().numpy(), ref_lse, LSE_ATOL[case.kv_dtype], f"f8mfma jump gap={gap} G={G} lse")
    assert np.max(np.abs(bf16_host_f64(out)[0] - c_j[None, :])) < 5e-2


@pytest.mark.parametrize("window", [0, 64])
def test_prefill_f8mfma(mla, window):
    """Absorbed-form prefill rows over an fp8 cache on the fp8 matrix cores."""
    say(f"prefill f8mfma window={window}")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [0, 5, 100, 640], [7, 1, 70, 33], seed=1800 + window, window=window,
                          sharp=True, kv_dtype=O.KV_FP8)
    check_prefill(mla, case, flags=mla.MLA_FLAG_FP8_MFMA | mla.MLA_FLAG_PREFILL_ABSORBED,
                  label=f" f8mfma w={window}")


# ---------------------------------------------------------------------------
# Combine
# ---------------------------------------------------------------------------

def test_decode_combine_abi(mla):
    say("decode_combine")
    rng = np.random.default_rng(9)
    S, B, H, D = 5, 3, 4, 64
    o = rng.normal(size=(S, B, H, D)).astype(np.float32)
    lse = rng.normal(scale=3, size=(S, B, H)).astype(np.float32)
    lse[1, 0, :] = -np.inf
    o[1, 0, :] = np.nan          # empty partials are not read
    lse[:, 2, 1] = -np.inf       # a row with nothing at all
    go, gl = mla.decode_combine(dev(o), dev(lse))
    torch.cuda.synchronize()
    ro, rl = O.combine(o, lse)
    assert np.max(np.abs(go.cpu().numpy() - ro)) < 1e-5
    gl = gl.cpu().numpy()
    assert np.isneginf(gl[2, 1]) and np.isneginf(rl[2, 1])
    m = ~np.isneginf(rl)
    assert np.max(np.abs(gl[m] - rl[m])) < 1e-5
    assert (go.cpu().numpy()[2, 1] == 0).all()


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------

def check_prefill(mla, case, rows=None, flags=0, num_workgroups=0, label=""):
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    out, lse = mla.prefill_chunk(cache, case.layer, dev_bf16(case.q_nope), dev_bf16(case.q_pe),
                                 dev(case.query_start_loc),
                                 int(np.max(np.diff(case.query_start_loc))), dev(case.block_tables),
                                 dev(case.context_lens), scale=case.scale, w_uk=w_uk, w_uv=w_uv,
                                 window=case.window, flags=flags, num_workgroups=num_workgroups)
    torch.cuda.synchronize()
    hc, hs = host_cache(case)
    ref, ref_lse = O.prefill_chunk(hc, hs, case.kv_dtype, 0, case.q_nope, case.q_pe,
                                   case.query_start_loc, case.block_tables, case.context_lens,
                                   case.w_uk, case.w_uv, case.scale, case.window, rows=rows)
    sel = slice(None) if rows is None else list(rows)
    assert_close(bf16_host_f64(out)[sel], ref[sel], tol_for(case), f"prefill{label}")
    assert_lse_close(lse.cpu().numpy()[sel], ref_lse[sel], LSE_ATOL[case.kv_dtype], f"prefill{label} lse")
    return out, lse


@pytest.mark.parametrize("window", [0, 3, 64])
@pytest.mark.parametrize("flags", [0, 1])
def test_prefill_small(mla, window, flags):
    say(f"prefill small window={window} flags={flags}")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [0, 5, 100, 64], [7, 1, 70, 33], seed=800 + window, window=window,
                          sharp=True)
    check_prefill(mla, case, flags=flags, label=f" w={window}")


@pytest.mark.parametrize("window", [0, 3, 64])
def test_prefill_expanded_small(mla, window):
    """The expanded form (keys and values up-projected per head) on the same
    ragged chunks as the absorbed form's test, including a one-row chunk."""
    say(f"prefill expanded small window={window}")
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [0, 5, 100, 64], [7, 1, 70, 33], seed=800 + window, window=window,
                          sharp=True)
    check_prefill(mla, case, flags=mla.MLA_FLAG_PREFILL_EXPANDED, label=f" expanded w={window}")


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
@pytest.mark.parametrize("window", [0, 128])
def test_prefill_expanded_multi_pass(mla, kv, window):
    """Contexts longer than one 2048-key pass (the running state is merged
    across passes), chunks longer than a 128-row block, 128 heads."""
    say(f"prefill expanded multi-pass kv={kv} window={window}")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [4500, 0, 2047], [300, 130, 2], seed=850 + window, window=window,
                          sharp=True, kv_dtype=kv)
    check_prefill(mla, case, flags=mla.MLA_FLAG_PREFILL_EXPANDED, label=f" expanded {kv} w={window}")


def test_prefill_expanded_passes_merged(mla):
    """A context whose up-projected keys exceed the expanded form's 1.25 GiB
    workspace share (24000 keys x 128 heads) runs in two merged passes."""
    say("prefill expanded, two passes")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [23850, 100], [150, 40], seed=880, sharp=True)
    check_prefill(mla, case, flags=mla.MLA_FLAG_PREFILL_EXPANDED, label=" expanded 2 passes")


def test_prefill_expanded_equals_absorbed_on_gpu(mla):
    """Both forms of the same call agree to the tolerance."""
    say("prefill expanded vs absorbed")
    d = W.Dims(H=32, R=512, Dr=64, Dn=128, Dv=128, page_size=32)
    case = W.prefill_case(d, [1000, 77], [200, 64], seed=870, sharp=True)
    a, _ = check_prefill(mla, case, flags=mla.MLA_FLAG_PREFILL_ABSORBED, label=" absorbed")
    e, _ = check_prefill(mla, case, flags=mla.MLA_FLAG_PREFILL_EXPANDED, label=" expanded")
    assert np.max(np.abs(bf16_host_f64(a) - bf16_host_f64(e))) < 2e-2


def test_prefill_tiny_dims(mla):
    say("prefill tiny dims")
    case = W.prefill_case(W.TINY_DIMS, [10, 0], [27, 5], seed=810, sharp=True,
                          stds=W.Stds(0.5, 0.5, 0.5, 0.5, 0.5), scale=1 / math.sqrt(48))
    check_prefill(mla, case)


def test_prefill_rows_match_decode_on_gpu(mla):
    """A prefill row and the decode of the same position agree to the tolerance."""
    say("prefill row vs decode")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.prefill_case(d, [300], [40], seed=820, sharp=True)
    out, _ = check_prefill(mla, case)
    cache = populate_device(mla, case)
    w_uk, w_uv = weights(case)
    r = 17
    dout, _ = mla.decode(cache, 0, dev_bf16(case.q_nope[[r]]), dev_bf16(case.q_pe[[r]]),
                         dev(case.block_tables), dev(np.array([300 + r + 1], np.int32)),
                         scale=case.scale, w_uk=w_uk, w_uv=w_uv)
    torch.cuda.synchronize()
    a, b = bf16_host_f64(out)[r], bf16_host_f64(dout)[0]
    assert np.max(np.abs(a - b)) < 2e-2


# ---------------------------------------------------------------------------
# Mixed batch with sliding window (4-layer cache)
# ---------------------------------------------------------------------------

def mixed_rows(ml):
    """Prefill rows compared: every 8th row of each chunk plus its last row."""
    rows = []
    for b in range(ml.n_prefill):
        s0, s1 = int(ml.query_start_loc[b]), int(ml.query_start_loc[b + 1])
        rows += list(range(s0, s1, 8)) + [s1 - 1]
    return sorted(set(rows))


@pytest.fixture(scope="module")
def mixed_step(mla):
    """The whole mixed step at full size, as the serving step runs it: one
    4-layer cache holding every layer's population, then per layer the write
    of the step's 4216 new tokens, the prefill of the 8 chunks (in the
    absorbed form, and again in the expanded form) and the decode of the 120
    single-token requests.  Returns the layers and their outputs (host
    copies)."""
    from concurrent.futures import ThreadPoolExecutor

    say("mixed step: generating 4 layers")
    with ThreadPoolExecutor(4) as ex:
        layers = list(ex.map(lambda l: W.mixed(l, sharp=True), range(len(W.MIXED_WINDOWS))))
    d = layers[0].dims
    cache = new_device_cache(mla, layers[0].num_layers, layers[0].num_pages, d, O.KV_BF16)
    for ml in layers:
        mla.write_kv(cache, ml.layer, dev_bf16(ml.pre_c_kv), dev_bf16(ml.pre_k_pe), dev(ml.pre_slots))
    torch.cuda.synchronize()
    results = []
    for ml in layers:
        say(f"mixed step: layer {ml.layer} (window {ml.window})")
        P = ml.n_prefill
        bt, ctx = dev(ml.block_tables), dev(ml.context_lens)
        w_uk, w_uv = dev_bf16(ml.w_uk), dev_bf16(ml.w_uv)
        mla.write_kv(cache, ml.layer, dev_bf16(ml.new_c_kv), dev_bf16(ml.new_k_pe), dev(ml.new_slots))
        pout, plse = mla.prefill_chunk(cache, ml.layer, dev_bf16(ml.q_nope_p), dev_bf16(ml.q_pe_p),
                                       dev(ml.query_start_loc), 512, bt[:P].contiguous(),
                                       ctx[:P].contiguous(), scale=ml.scale, w_uk=w_uk, w_uv=w_uv,
                                       window=ml.window, flags=mla.MLA_FLAG_PREFILL_ABSORBED)
        dout, dlse = mla.decode(cache, ml.layer, dev_bf16(ml.q_nope_d), dev_bf16(ml.q_pe_d),
                                bt[P:].contiguous(), ctx[P:].contiguous(), scale=ml.scale,
                                w_uk=w_uk, w_uv=w_uv, window=ml.window)
        xout, xlse = mla.prefill_chunk(cache, ml.layer, dev_bf16(ml.q_nope_p), dev_bf16(ml.q_pe_p),
                                       dev(ml.query_start_loc), 512, bt[:P].contiguous(),
                                       ctx[:P].contiguous(), scale=ml.scale, w_uk=w_uk, w_uv=w_uv,
                                       window=ml.window, flags=mla.MLA_FLAG_PREFILL_EXPANDED)
        torch.cuda.synchronize()
        results.append((bf16_host_f64(pout), plse.cpu().numpy(), bf16_host_f64(dout),
                        dlse.cpu().numpy(), bf16_host_f64(xout), xlse.cpu().numpy()))
    del cache
    torch.cuda.empty_cache()
    return layers, results


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_mixed_step_full_size(mla, mixed_step, layer):
    """One layer of the mixed step against the oracle: all 120 decodes, and
    every 8th prefill row of each chunk plus its last row (520 of 4096)."""
    layers, results = mixed_step
    ml = layers[layer]
    pout, plse, dout, dlse, xout, xlse = results[layer]
    say(f"mixed step layer {layer}: oracle")
    d = ml.dims
    P = ml.n_prefill
    hc = np.full((1, ml.num_pages, 64, d.D), W.BF16_NAN, dtype=np.uint16)
    hs = np.full((1, ml.num_pages, 64), np.nan, dtype=np.float32)
    O.write_kv(hc, hs, 0, ml.pre_c_kv, ml.pre_k_pe, ml.pre_slots)
    O.write_kv(hc, hs, 0, ml.new_c_kv, ml.new_k_pe, ml.new_slots)
    rows = mixed_rows(ml)
    ref, ref_lse = O.prefill_chunk(hc, hs, O.KV_BF16, 0, ml.q_nope_p, ml.q_pe_p, ml.query_start_loc,
                                   ml.block_tables[:P], ml.context_lens[:P], ml.w_uk, ml.w_uv,
                                   ml.scale, ml.window, rows=rows)
    assert_close(pout[rows], ref[rows], BF16_TOL, f"mixed L{layer} prefill ({len(rows)} rows)")
    assert_lse_close(plse[rows], ref_lse[rows], LSE_ATOL[O.KV_BF16], f"mixed L{layer} prefill lse")
    assert_close(xout[rows], ref[rows], BF16_TOL, f"mixed L{layer} expanded prefill")
    assert_lse_close(xlse[rows], ref_lse[rows], LSE_ATOL[O.KV_BF16], f"mixed L{layer} expanded lse")
    dref, dref_lse = O.decode(hc, hs, O.KV_BF16, 0, ml.q_nope_d, ml.q_pe_d, ml.block_tables[P:],
                              ml.context_lens[P:], ml.w_uk, ml.w_uv, ml.scale, ml.window)
    assert_close(dout, dref, BF16_TOL, f"mixed L{layer} decode (all 120)")
    assert_lse_close(dlse, dref_lse, LSE_ATOL[O.KV_BF16], f"mixed L{layer} decode lse")
