"""mla_write_kv_fused on the GPU against the oracle's write_kv_fused.

The device computes the RMSNorm and the rotation in fp32, the oracle in fp64;
both round to bf16 to nearest even.  The two can differ only where the fp32
result lands on the other side of a bf16 rounding boundary than the exact
one, so the bar is: every written bf16 value is within one bf16 ulp of the
exact value, plus, for a rotated value a cos - b sin (or b cos + a sin), the
fp32 evaluation's own error 2^-22 (|a cos| + |b sin|), which dominates where
the two products cancel; and at most 1e-3 of the values differ from the
oracle's rounded ones.  For the fp8 cache the dequantised values are within half an E4M3 step
(plus the bf16 rounding) of the exact ones, and at most 1e-3 of the code bytes
differ from the oracle's.  With neither norm nor rotation the fused write is
bit-identical to mla_write_kv."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

from gpu_support import (BF16_TOL, FP8_TOL, assert_close, bf16_host_bits, dev, dev_bf16,
                         new_device_cache, say)

pytestmark = pytest.mark.gpu

D512 = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_mla_latent_write_amd import mla as m
    return m


def offset_bf16(bits):
    """bf16 rows [T, n] as a view 8 bytes into the rows of a wider device
    tensor: not 16-byte aligned, so the write kernels take their
    lane-strided form (element j of a row in lane j % 64) instead of the
    16-byte chunk form."""
    T, n = bits.shape
    wide = np.zeros((T, n + 8), dtype=np.uint16)
    wide[:, 4:4 + n] = bits
    return dev_bf16(wide)[:, 4:4 + n]


def gpu_fused(mla, fc, kv, *, norm=True, rope=True, interleaved=True, layer=1, num_layers=2,
              unaligned=False):
    cache = new_device_cache(mla, num_layers, fc.num_pages, fc.dims, kv)
    c_kv = offset_bf16(fc.c_kv) if unaligned else dev_bf16(fc.c_kv)
    mla.write_kv_fused(cache, layer, c_kv, dev_bf16(fc.k_pe), dev(fc.slots),
                       positions=dev(fc.positions), norm_weight=dev_bf16(fc.norm_weight) if norm else None,
                       eps=fc.eps, cos_sin=dev(fc.cos_sin) if rope else None, interleaved=interleaved)
    torch.cuda.synchronize()
    return cache


def oracle_fused(fc, kv, *, norm=True, rope=True, interleaved=True, layer=1, num_layers=2):
    d = fc.dims
    fill = W.BF16_NAN if kv == O.KV_BF16 else W.E4M3_NAN
    hc = np.full((num_layers, fc.num_pages, d.page_size, d.D), fill,
                 dtype=np.uint16 if kv == O.KV_BF16 else np.uint8)
    hs = np.full((num_layers, fc.num_pages, d.page_size), np.nan, dtype=np.float32)
    O.write_kv_fused(hc, hs, layer, fc.c_kv, fc.k_pe, fc.slots, fc.positions,
                     fc.norm_weight if norm else None, fc.eps, fc.cos_sin if rope else None,
                     interleaved, kv)
    return hc, hs


def exact_rows(fc, interleaved):
    """The transformed rows in fp64, before any rounding."""
    return np.concatenate([O.rms_norm(fc.c_kv, fc.norm_weight, fc.eps),
                           O.rope_rotate(fc.k_pe, fc.positions, fc.cos_sin, interleaved)], axis=1)


def bf16_ulp(y):
    _, e = np.frexp(np.abs(y))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def fp32_slack(fc, interleaved):
    """Bound on the fp32 evaluation error of each transformed value: zero
    for the latent (a product, relative error ~2^-22), 2^-22 times the sum of
    the two products' magnitudes for a rotated value."""
    d = fc.dims
    x = O.bf16_bits_to_f64(fc.k_pe)
    tab = np.asarray(fc.cos_sin, np.float32).astype(np.float64)[fc.positions]
    h = d.Dr // 2
    c, s = np.abs(tab[:, :h]), np.abs(tab[:, h:])
    first, second = O.rope_pairs(d.Dr, interleaved)
    a, b = np.abs(x[:, first]), np.abs(x[:, second])
    mag = np.zeros_like(x)
    mag[:, first] = a * c + b * s
    mag[:, second] = b * c + a * s
    return np.concatenate([np.zeros((x.shape[0], d.R)), 2.0 ** -22 * mag], axis=1)


# unaligned: the latent rows handed over 8 bytes off 16-byte alignment (the
# kernels' lane-strided form); else aligned (their 16-byte chunk form)
@pytest.mark.parametrize("unaligned", [False, True])
@pytest.mark.parametrize("interleaved", [True, False])
def test_fused_write_bf16(mla, interleaved, unaligned):
    say(f"fused write bf16 interleaved={interleaved} unaligned={unaligned}")
    fc = W.fused_write_case(D512, 4096, seed=1200 + interleaved, pad_every=9, c_std=2.0)
    got = bf16_host_bits(gpu_fused(mla, fc, O.KV_BF16, interleaved=interleaved, unaligned=unaligned).data)
    hc, _ = oracle_fused(fc, O.KV_BF16, interleaved=interleaved)
    live = fc.slots >= 0
    # rows the call must not touch: other layer, pad rows, unused slots
    untouched = np.ones(got.shape[:3], dtype=bool)
    ps = D512.page_size
    untouched[1, fc.slots[live] // ps, fc.slots[live] % ps] = False
    assert np.array_equal(got[untouched], hc[untouched])
    g = got[1].reshape(-1, D512.D)[fc.slots[live]]
    r = hc[1].reshape(-1, D512.D)[fc.slots[live]]
    y = exact_rows(fc, interleaved)[live]
    gv = O.bf16_bits_to_f64(g)
    bad = ~(np.abs(gv - y) <= bf16_ulp(y) + fp32_slack(fc, interleaved)[live])
    if bad.any():
        t, j = np.nonzero(bad)
        say(f"  {int(bad.sum())} values off by more than an ulp; columns {np.unique(j)[:20]}; "
            f"tokens {np.unique(t)[:10]}; got {gv[t[:5], j[:5]]} want {y[t[:5], j[:5]]}")
    assert not bad.any(), "a value is more than one bf16 ulp off"
    frac = float(np.mean(g != r))
    say(f"  bf16 values differing from the oracle's rounding: {frac:.2e}")
    assert frac <= 1e-3


@pytest.mark.parametrize("unaligned", [False, True])
def test_fused_write_fp8(mla, unaligned):
    say(f"fused write fp8 unaligned={unaligned}")
    fc = W.fused_write_case(D512, 4096, seed=1210, pad_every=11, c_std=2.0)
    cache = gpu_fused(mla, fc, O.KV_FP8, unaligned=unaligned)
    codes = cache.data.cpu().numpy()
    scl = cache.scale.cpu().numpy()
    hc, hs = oracle_fused(fc, O.KV_FP8)
    live = fc.slots >= 0
    ps = D512.page_size
    pg, off = fc.slots[live] // ps, fc.slots[live] % ps
    g = codes[1, pg, off]
    r = hc[1, pg, off]
    frac = float(np.mean(g != r))
    say(f"  code bytes differing from the oracle's: {frac:.2e}")
    assert frac <= 1e-3
    gs = scl[1, pg, off].astype(np.float64)
    deq = O.E4M3_TABLE[g] * gs[:, None]
    y = exact_rows(fc, True)[live]
    bound = ((2.0 ** -4 + 2.0 ** -8) * np.abs(y) + 2.0 ** -9 * gs[:, None]
             + 2 * fp32_slack(fc, True)[live])
    assert np.all(np.abs(deq - y) <= bound)
    mask = np.ones(codes.shape[:3], dtype=bool)
    mask[1, pg, off] = False
    assert np.array_equal(codes[mask], hc[mask])


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
def test_fused_write_without_transform_is_plain_write(mla, kv):
    say(f"fused write identity {kv}")
    fc = W.fused_write_case(D512, 700, seed=1220, pad_every=7)
    a = gpu_fused(mla, fc, kv, norm=False, rope=False)
    b = new_device_cache(mla, 2, fc.num_pages, fc.dims, kv)
    mla.write_kv(b, 1, dev_bf16(fc.c_kv), dev_bf16(fc.k_pe), dev(fc.slots))
    torch.cuda.synchronize()
    assert torch.equal(a.data.view(torch.uint8), b.data.view(torch.uint8))
    if kv == O.KV_FP8:
        assert torch.equal(a.scale.view(torch.int32), b.scale.view(torch.int32))


@pytest.mark.parametrize("kv", [O.KV_BF16, O.KV_FP8])
def test_write_forms_bit_identical(mla, kv):
    """The plain write in its lane-strided form (latent rows off 16-byte
    alignment) and in its 16-byte chunk form, and the fused write without
    transforms in the lane-strided form: the same bytes and scales (the E4M3
    row rule depends on no order of operations)."""
    say(f"write forms {kv}")
    fc = W.fused_write_case(D512, 900, seed=1240, pad_every=7, c_std=3.0)
    caches = []
    for unaligned in (False, True):
        cache = new_device_cache(mla, 2, fc.num_pages, fc.dims, kv)
        c_kv = offset_bf16(fc.c_kv) if unaligned else dev_bf16(fc.c_kv)
        mla.write_kv(cache, 1, c_kv, dev_bf16(fc.k_pe), dev(fc.slots))
        caches.append(cache)
    caches.append(gpu_fused(mla, fc, kv, norm=False, rope=False, unaligned=True))
    torch.cuda.synchronize()
    for c in caches[1:]:
        assert torch.equal(caches[0].data.view(torch.uint8), c.data.view(torch.uint8))
        if kv == O.KV_FP8:
            assert torch.equal(caches[0].scale.view(torch.int32), c.scale.view(torch.int32))


def test_fused_write_nan_rows(mla):
    """NaN inputs (with payloads and either sign): a NaN in a row's latent
    makes its whole normalised latent NaN (the sum of squares is NaN), a NaN
    rope element makes its rotation pair NaN; every such bf16 value is the
    canonical 0x7FC0 in both forms of the kernel (16-byte chunks, and
    element per lane), and no other value is NaN."""
    say("fused write NaN rows")
    fc = W.fused_write_case(D512, 256, seed=1250)
    c_kv, k_pe = fc.c_kv.copy(), fc.k_pe.copy()
    c_kv[3, 17], c_kv[50, 400] = 0x7FC1, 0xFFA5
    k_pe[7, 5], k_pe[90, 62] = 0xFFC3, 0x7F81
    fc.c_kv, fc.k_pe = c_kv, k_pe
    want = np.zeros((256, D512.D), dtype=bool)
    want[[3, 50], :D512.R] = True
    want[7, D512.R + 4:D512.R + 6] = True    # interleaved pair (4, 5)
    want[90, D512.R + 62:D512.R + 64] = True  # pair (62, 63)
    ps = D512.page_size
    for unaligned in (False, True):
        got = bf16_host_bits(gpu_fused(mla, fc, O.KV_BF16, unaligned=unaligned).data)
        rows = got[1].reshape(-1, D512.D)[fc.slots]
        nan = (rows & 0x7FFF) > 0x7F80
        assert np.array_equal(nan, want), f"unaligned={unaligned}: NaN positions differ"
        assert np.all(rows[nan] == 0x7FC0), f"unaligned={unaligned}: a NaN is not 0x7FC0"


def test_decode_over_a_fused_written_cache(mla):
    """End to end: the context is written with the norm and rotation folded
    in, then decoded; the oracle does the same with its own fused write."""
    say("decode over fused-written cache")
    d = W.Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    case = W.custom(d, [300, 2049, 77], seed=1230)
    fc = W.fused_write_case(d, int(case.context_lens.sum()), seed=1231, c_std=2.0)
    # the case's own population slots, the fused case's raw rows and positions
    slots = case.ctx_slots
    cache = new_device_cache(mla, 1, case.num_pages, d, O.KV_BF16)
    mla.write_kv_fused(cache, 0, dev_bf16(fc.c_kv), dev_bf16(fc.k_pe), dev(slots),
                       positions=dev(fc.positions), norm_weight=dev_bf16(fc.norm_weight), eps=fc.eps,
                       cos_sin=dev(fc.cos_sin))
    out, _ = mla.decode(cache, 0, dev_bf16(case.q_nope), dev_bf16(case.q_pe), dev(case.block_tables),
                        dev(case.context_lens), scale=case.scale, w_uk=dev_bf16(case.w_uk),
                        w_uv=dev_bf16(case.w_uv))
    torch.cuda.synchronize()
    hc = np.full((1, case.num_pages, 64, d.D), W.BF16_NAN, dtype=np.uint16)
    hs = np.full((1, case.num_pages, 64), np.nan, dtype=np.float32)
    O.write_kv_fused(hc, hs, 0, fc.c_kv, fc.k_pe, slots, fc.positions, fc.norm_weight, fc.eps,
                     fc.cos_sin, True)
    ref, _ = O.decode(hc, hs, O.KV_BF16, 0, case.q_nope, case.q_pe, case.block_tables,
                      case.context_lens, case.w_uk, case.w_uv, case.scale, 0)
    assert_close(O.bf16_bits_to_f64(bf16_host_bits(out)), ref, BF16_TOL, "decode over fused write")
