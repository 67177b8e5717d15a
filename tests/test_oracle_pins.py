"""Pins for the fp64 oracle: each check ties it to something other than itself
(the E4M3 specification, a library routine, a closed form, a scalar brute
force on contiguous data, or an invariant the pages fix), so that a plausible
slip in the oracle (a dropped term, a wrong index or sign, a transposed
operand, an off-by-one window) fails at least one of them.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import mla_oracle as O
from paged_mla_latent_write_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers (test-side, no oracle arithmetic)
# ---------------------------------------------------------------------------

def build_cache(case, kv_dtype=None, num_layers=None, layer=None, page_size=None, perm_seed=None):
    """Populate a host cache through the oracle's write (the same route the
    GPU tests take through mla_write_kv)."""
    kv_dtype = kv_dtype or case.kv_dtype
    L = num_layers or 1
    layer = 0 if layer is None else layer
    ps = case.dims.page_size
    fill = W.BF16_NAN if kv_dtype == O.KV_BF16 else W.E4M3_NAN
    dt = np.uint16 if kv_dtype == O.KV_BF16 else np.uint8
    cache = np.full((L, case.num_pages, ps, case.dims.D), fill, dtype=dt)
    scale = np.full((L, case.num_pages, ps), np.nan, dtype=np.float32)
    O.write_kv(cache, scale, layer, case.ctx_c_kv, case.ctx_k_pe, case.ctx_slots, kv_dtype)
    return cache, scale


def small_dims(H=2, R=8, Dr=4, Dn=4, Dv=4, ps=4):
    return W.Dims(H=H, R=R, Dr=Dr, Dn=Dn, Dv=Dv, page_size=ps)


def run_decode(case, cache, scale, layer=0, window=None, form="absorbed", wuk=True, wuv=True,
               block_tables=None, q_nope=None):
    return O.decode(cache, scale, case.kv_dtype, layer,
                    case.q_nope if q_nope is None else q_nope, case.q_pe,
                    case.block_tables if block_tables is None else block_tables,
                    case.context_lens, case.w_uk if wuk else None, case.w_uv if wuv else None,
                    case.scale, case.window if window is None else window, form=form)


def request_rows(case, b):
    """Population rows of request b in logical order (contiguous data)."""
    start = int(np.sum(case.context_lens[:b]))
    return slice(start, start + int(case.context_lens[b]))


def brute_force_request(case, b, window, use_wuk=True, use_wuv=True, p=None):
    """Scalar loops over contiguous float lists with math.exp and math.fsum.
    Keys are built as [W_UK[h] c_t ; r_t] with W_UK[h] indexed [d][r] as the
    documented layout [H, Dn, R] says, values as W_UV[h] c_t."""
    d = case.dims
    rows = request_rows(case, b)
    c = O.bf16_bits_to_f64(case.ctx_c_kv[rows]).tolist()
    r = O.bf16_bits_to_f64(case.ctx_k_pe[rows]).tolist()
    n = len(c)
    p = n - 1 if p is None else p
    lo = 0 if window <= 0 else max(0, p - window + 1)
    keys_t = range(lo, p + 1)
    qn = O.bf16_bits_to_f64(case.q_nope[b]).tolist()
    qp = O.bf16_bits_to_f64(case.q_pe[b]).tolist()
    wuk = O.bf16_bits_to_f64(case.w_uk).tolist()
    wuv = O.bf16_bits_to_f64(case.w_uv).tolist()
    outs, lses = [], []
    for h in range(d.H):
        scores, values = [], []
        for t in keys_t:
            if use_wuk:
                k_nope = [math.fsum(wuk[h][i][j] * c[t][j] for j in range(d.R)) for i in range(d.Dn)]
            else:
                k_nope = c[t]
            dot = math.fsum([qn[h][i] * k_nope[i] for i in range(len(k_nope))]
                            + [qp[h][i] * r[t][i] for i in range(d.Dr)])
            scores.append(case.scale * dot)
            if use_wuv:
                values.append([math.fsum(wuv[h][i][j] * c[t][j] for j in range(d.R)) for i in range(d.Dv)])
            else:
                values.append(c[t])
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        tot = math.fsum(e)
        outs.append([math.fsum(e[k] * values[k][j] for k in range(len(e))) / tot
                     for j in range(len(values[0]))])
        lses.append(m + math.log(tot))
    return np.array(outs), np.array(lses)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# E4M3 codec (OFP8)
# ---------------------------------------------------------------------------

def test_e4m3_table_matches_spec_fixture():
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        got = O.E4M3_TABLE[code]
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), (code_s, got)


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_TABLE
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.E4M3_TABLE[codes].astype(np.float32)
    assert np.array_equal(O.e4m3_encode_satfinite(vals), codes)


def test_e4m3_encode_ties_to_even_at_every_midpoint():
    mags = O.E4M3_TABLE[:0x7F]
    for c in range(0x7E):
        mid = np.float32((mags[c] + mags[c + 1]) / 2)  # exact in fp32
        assert float(mid) == (mags[c] + mags[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert O.e4m3_encode_satfinite(np.array([mid]))[0] == want
        assert O.e4m3_encode_satfinite(np.array([-mid]))[0] == want | 0x80
        # just off the midpoint goes to the nearer neighbour
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        assert O.e4m3_encode_satfinite(np.array([below]))[0] == c
        assert O.e4m3_encode_satfinite(np.array([above]))[0] == c + 1


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1e-2, 200000),
                        rng.normal(0, 1e-3, 100000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode_satfinite(x), ref)


def test_e4m3_encode_saturates():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e30, -500.0, -448.5], dtype=np.float32)
    assert O.e4m3_encode_satfinite(x).tolist() == [0x7E] * 5 + [0xFE] * 2
    assert O.e4m3_encode_satfinite(np.array([np.nan], np.float32))[0] == 0x7F


def test_fp8_token_quantisation_rules():
    rng = np.random.default_rng(3)
    rows = W.f32_to_bf16_bits(rng.normal(0, 0.05, (64, 576)).astype(np.float32))
    rows[5] = 0  # all-zero token -> scale 1.0, codes 0
    codes, scale = O.fp8_quantize_tokens(rows)
    assert scale.dtype == np.float32 and scale[5] == 1.0 and not codes[5].any()
    x = O.bf16_bits_to_f64(rows)
    amax = np.abs(x).max(axis=1)
    live = amax > 0
    # scale is amax / 448 rounded to fp32 (within half an fp32 ulp of the exact quotient)
    assert np.all(np.abs(scale[live] - amax[live] / 448) <= np.spacing(scale[live].astype(np.float32)) / 2)
    # the largest magnitude lands on +-448
    arg = np.abs(x).argmax(axis=1)
    top = codes[np.arange(64), arg]
    assert np.all((top[live] & 0x7F) == 0x7E)
    # dequantised values stay within the E4M3 rounding bound:
    # normals 2^-4 relative, subnormals 2^-10 * scale absolute
    deq = O.E4M3_TABLE[codes] * scale[:, None]
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None].astype(np.float64)) * 1.0001
    assert np.all(err <= bound)


# ---------------------------------------------------------------------------
# Write: layer isolation, pad rows, overwrite
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype", [O.KV_BF16, O.KV_FP8])
def test_write_layer_isolation_pads_and_overwrite(kv_dtype):
    case = W.custom(small_dims(), [5, 9], seed=11)
    cache, sc = build_cache(case, kv_dtype=kv_dtype, num_layers=3, layer=1)
    fill = W.BF16_NAN if kv_dtype == O.KV_BF16 else W.E4M3_NAN
    # other layers untouched (bitwise)
    assert (cache[0] == fill).all() and (cache[2] == fill).all()
    assert np.isnan(sc[0]).all() and np.isnan(sc[2]).all()
    # what was written is the token's row (bf16: bit copy)
    if kv_dtype == O.KV_BF16:
        s = case.ctx_slots
        got = cache[1, s // 4, s % 4]
        assert np.array_equal(got, np.concatenate([case.ctx_c_kv, case.ctx_k_pe], axis=1))
    # pad rows write nothing
    before = cache.copy(), sc.copy()
    O.write_kv(cache, sc, 1, case.ctx_c_kv[:3] ^ 1, case.ctx_k_pe[:3], np.array([-1, -1, -7]), kv_dtype)
    assert np.array_equal(cache, before[0])
    assert np.array_equal(sc, before[1], equal_nan=True)
    # a later write to a slot wins
    new_c = case.ctx_c_kv[:1] ^ 3
    O.write_kv(cache, sc, 1, new_c, case.ctx_k_pe[:1], case.ctx_slots[:1], kv_dtype)
    s0 = case.ctx_slots[0]
    if kv_dtype == O.KV_BF16:
        assert np.array_equal(cache[1, s0 // 4, s0 % 4, :8], new_c[0])
    with pytest.raises(AssertionError):
        O.write_kv(cache, sc, 1, case.ctx_c_kv[:2], case.ctx_k_pe[:2], np.array([3, 3]), kv_dtype)


# ---------------------------------------------------------------------------
# Attention pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 3, 7])
@pytest.mark.parametrize("sharp", [False, True])
def test_brute_force_contiguous_matches_paged_oracle(window, sharp):
    """P2: scalar loops over contiguous data == paged oracle (both forms)."""
    case = W.custom(small_dims(), [1, 6, 13], seed=21 + window, sharp=sharp)
    cache, sc = build_cache(case)
    for form in ("absorbed", "expanded"):
        out, lse = run_decode(case, cache, sc, window=window, form=form)
        for b in range(case.batch):
            bo, bl = brute_force_request(case, b, window)
            assert rel(out[b], bo) < 1e-12, (form, b)
            assert np.max(np.abs(lse[b] - bl)) < 1e-12


def test_brute_force_latent_io():
    """w_uk / w_uv absent: latent query in, latent output out."""
    d = small_dims(Dn=8)
    case = W.custom(d, [4, 11], seed=5, sharp=True)
    cache, sc = build_cache(case)
    qn_lat = W.bf16_normal(np.random.default_rng(2), (2, d.H, d.R), 1.0)
    for form in ("absorbed", "expanded"):
        out, lse = run_decode(case, cache, sc, form=form, wuk=False, wuv=False, q_nope=qn_lat)
        c2 = W.Case(**{**case.__dict__, "q_nope": qn_lat})
        for b in range(2):
            bo, bl = brute_force_request(c2, b, 0, use_wuk=False, use_wuv=False)
            assert rel(out[b], bo) < 1e-12


def test_absorbed_equals_expanded_at_mla_dims():
    """P1 at the real MLA dims (H 16, R 512, Dr 64, Dn = Dv = 128), bf16 and fp8."""
    d = W.Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
    for kv in (O.KV_BF16, O.KV_FP8):
        case = W.custom(d, [1, 70, 300], seed=9, kv_dtype=kv, sharp=True)
        cache, sc = build_cache(case)
        a, la = run_decode(case, cache, sc, form="absorbed")
        e, le = run_decode(case, cache, sc, form="expanded")
        assert rel(a, e) < 1e-12 and np.max(np.abs(la - le)) < 1e-12


def test_one_token_context_returns_its_value():
    """P3: n = 1 gives weight exactly 1 on token 0: out = W_UV[h] c_0."""
    case = W.custom(small_dims(), [1, 1], seed=4, sharp=True)
    cache, sc = build_cache(case)
    out, lse = run_decode(case, cache, sc)
    for b in range(2):
        c0 = O.bf16_bits_to_f64(case.ctx_c_kv[request_rows(case, b)][0]).tolist()
        wuv = O.bf16_bits_to_f64(case.w_uv).tolist()
        for h in range(case.dims.H):
            want = [math.fsum(wuv[h][i][j] * c0[j] for j in range(case.dims.R)) for i in range(case.dims.Dv)]
            assert np.max(np.abs(out[b, h] - want)) <= 1e-15 * max(1.0, np.max(np.abs(want)))


def test_window_at_least_context_equals_full():
    """P4."""
    case = W.custom(small_dims(), [1, 9, 16], seed=8, sharp=True)
    cache, sc = build_cache(case)
    full, lf = run_decode(case, cache, sc, window=0)
    for w in (16, 17, 1000):
        win, lw = run_decode(case, cache, sc, window=w)
        assert np.array_equal(full, win) and np.array_equal(lf, lw)


def test_window_equals_repaged_last_w_tokens():
    """P5: window w == full attention over a cache holding only the last w
    tokens of each request; w = 1 returns the newest token's value."""
    case = W.custom(small_dims(), [3, 10, 17], seed=12, sharp=True)
    cache, sc = build_cache(case)
    for w in (1, 2, 5, 8):
        win, lw = run_decode(case, cache, sc, window=w)
        # re-page: keep only the last min(w, n) tokens, in order, as a new request
        keep = [np.arange(int(n))[-w:] + int(np.sum(case.context_lens[:b]))
                for b, n in enumerate(case.context_lens)]
        lens = np.array([len(k) for k in keep], dtype=np.int32)
        rng = np.random.default_rng(w)
        bt, npg, _ = W.assign_pages(rng, lens, 4)
        idx = np.concatenate(keep)
        c2 = W.Case(**{**case.__dict__, "ctx_c_kv": case.ctx_c_kv[idx], "ctx_k_pe": case.ctx_k_pe[idx],
                       "ctx_slots": W.slots_for(bt, lens, 4), "block_tables": bt, "context_lens": lens,
                       "num_pages": npg})
        cache2, sc2 = build_cache(c2)
        full, lf = run_decode(c2, cache2, sc2, window=0)
        assert np.array_equal(win, full) and np.array_equal(lw, lf), w
        if w == 1:
            for b in range(case.batch):
                cl = O.bf16_bits_to_f64(case.ctx_c_kv[request_rows(case, b)][-1])
                want = np.einsum("hvr,r->hv", O.bf16_bits_to_f64(case.w_uv), cl)
                assert rel(win[b], want) < 1e-14


@pytest.mark.parametrize("kv_dtype", [O.KV_BF16, O.KV_FP8])
def test_page_permutation_and_page_size_invariance(kv_dtype):
    """P6: any physical page placement and page sizes 1, 16, 64, 128 give the
    same result (bitwise)."""
    base = W.custom(W.Dims(H=4, R=32, Dr=16, Dn=16, Dv=16, page_size=16), [1, 40, 130, 257],
                    seed=31, kv_dtype=kv_dtype, sharp=True)
    ref = None
    for ps in (1, 16, 64, 128):
        for perm_seed in (0, 1):
            rng = np.random.default_rng(100 * ps + perm_seed)
            bt, npg, _ = W.assign_pages(rng, base.context_lens, ps)
            dims = W.Dims(**{**base.dims.__dict__, "page_size": ps})
            c = W.Case(**{**base.__dict__, "dims": dims, "block_tables": bt, "num_pages": npg,
                          "ctx_slots": W.slots_for(bt, base.context_lens, ps)})
            cache, sc = build_cache(c)
            out = run_decode(c, cache, sc, window=0)
            if ref is None:
                ref = out
            assert np.array_equal(out[0], ref[0]) and np.array_equal(out[1], ref[1]), (ps, perm_seed)


def test_combine_of_contiguous_splits_equals_unsplit():
    """P7: partials over a contiguous partition of the visible keys (one of
    them empty) merge to the unsplit result; lse agrees with scipy."""
    case = W.custom(small_dims(), [23], seed=17, sharp=True)
    cache, sc = build_cache(case)
    full, lf = run_decode(case, cache, sc, wuv=False)
    X = O.gather_latent(cache, sc, case.kv_dtype, 0, case.block_tables[0], 23)
    qn = O.bf16_bits_to_f64(case.q_nope[0])
    qp = O.bf16_bits_to_f64(case.q_pe[0])
    wuk = O.bf16_bits_to_f64(case.w_uk)
    for cuts in ([0, 5, 5, 23], [0, 1, 2, 22, 23], [0, 23]):
        parts = [O.attend_absorbed(qn, qp, X[a:b], wuk, None, case.scale, 8)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, l = O.combine([p[0] for p in parts], [p[1] for p in parts])
        assert rel(o, full[0]) < 1e-13 and np.max(np.abs(l - lf[0])) < 1e-13
        assert np.allclose(l, logsumexp(np.stack([p[1] for p in parts]), axis=0), rtol=0, atol=1e-14)
    # all-empty -> 0, -inf
    o, l = O.combine(np.full((2, 3, 4), np.nan), np.full((2, 3), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_lse_matches_scipy_on_bruteforce_scores():
    case = W.custom(small_dims(), [12], seed=3, sharp=True)
    cache, sc = build_cache(case)
    _, lse = run_decode(case, cache, sc)
    X = O.bf16_bits_to_f64(case.ctx_c_kv)
    Rp = O.bf16_bits_to_f64(case.ctx_k_pe)
    wuk = O.bf16_bits_to_f64(case.w_uk)
    qn = O.bf16_bits_to_f64(case.q_nope[0])
    qp = O.bf16_bits_to_f64(case.q_pe[0])
    for h in range(case.dims.H):
        s = case.scale * ((X @ wuk[h].T) @ qn[h] + Rp @ qp[h])
        assert abs(lse[0, h] - logsumexp(s)) < 1e-13


def test_prefill_rows_equal_decodes_and_chunk_splitting():
    """P8: prefill row i equals a decode with n = prefix + i + 1; a chunk of
    one row equals decode; splitting a chunk into two changes nothing."""
    d = small_dims()
    for window in (0, 3):
        case = W.prefill_case(d, [0, 5, 9], [4, 1, 6], seed=40 + window, window=window, sharp=True)
        cache, sc = build_cache(case)
        out, lse = O.prefill_chunk(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe,
                                   case.query_start_loc, case.block_tables, case.context_lens,
                                   case.w_uk, case.w_uv, case.scale, window)
        qsl = case.query_start_loc
        for b in range(3):
            m = qsl[b + 1] - qsl[b]
            for i in range(m):
                r = qsl[b] + i
                lens = case.context_lens.copy()
                lens[b] = case.context_lens[b] - m + i + 1
                do, dl = O.decode(cache, sc, case.kv_dtype, 0, case.q_nope[[r]], case.q_pe[[r]],
                                  case.block_tables[[b]], lens[[b]], case.w_uk, case.w_uv,
                                  case.scale, window)
                assert rel(out[r], do[0]) < 1e-13 and np.max(np.abs(lse[r] - dl[0])) < 1e-13
        # split request 2's chunk (6 rows) into 2 + 4 rows as two sequential calls
        b = 2
        n, m = int(case.context_lens[b]), 6
        r0 = int(qsl[b])
        first = O.prefill_chunk(cache, sc, case.kv_dtype, 0, case.q_nope[r0:r0 + 2], case.q_pe[r0:r0 + 2],
                                np.array([0, 2]), case.block_tables[[b]], np.array([n - 4]),
                                case.w_uk, case.w_uv, case.scale, window)
        second = O.prefill_chunk(cache, sc, case.kv_dtype, 0, case.q_nope[r0 + 2:r0 + 6],
                                 case.q_pe[r0 + 2:r0 + 6], np.array([0, 4]), case.block_tables[[b]],
                                 np.array([n]), case.w_uk, case.w_uv, case.scale, window)
        joined = np.concatenate([first[0], second[0]])
        assert rel(joined, out[r0:r0 + 6]) < 1e-13


def test_prefill_brute_force_rows():
    d = small_dims()
    case = W.prefill_case(d, [3, 0], [5, 4], seed=77, window=4, sharp=True)
    cache, sc = build_cache(case)
    out, _ = O.prefill_chunk(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, case.query_start_loc,
                             case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale, 4)
    qsl = case.query_start_loc
    for b in range(2):
        m = qsl[b + 1] - qsl[b]
        for i in range(m):
            r = qsl[b] + i
            c2 = W.Case(**{**case.__dict__, "q_nope": case.q_nope[[r] * 2], "q_pe": case.q_pe[[r] * 2]})
            bo, _ = brute_force_request(c2, b, 4, p=int(case.context_lens[b]) - m + i)
            assert rel(out[r], bo) < 1e-12


def test_causality_future_keys_do_not_matter():
    """P9: changing cached tokens after position p leaves row p unchanged."""
    d = small_dims()
    case = W.prefill_case(d, [6], [6], seed=50, sharp=True)
    cache, sc = build_cache(case)
    args = (case.q_nope, case.q_pe, case.query_start_loc, case.block_tables, case.context_lens,
            case.w_uk, case.w_uv, case.scale, 0)
    out, _ = O.prefill_chunk(cache, sc, case.kv_dtype, 0, *args)
    cache2 = cache.copy()
    for t in range(9, 12):  # positions after row 2 (p = 6 + 2 = 8)
        pg, off = divmod(t, 4)
        cache2[0, case.block_tables[0, pg], off] ^= np.uint16(0x0101)
    out2, _ = O.prefill_chunk(cache2, sc, case.kv_dtype, 0, *args)
    assert np.array_equal(out[:3], out2[:3])
    assert not np.array_equal(out[3:], out2[3:])


def test_needle_selects_one_key():
    """P13: a query aligned with one key's rope part by a margin >= 40 in the
    scaled score returns that key's value."""
    d = small_dims(Dr=16)
    case = W.custom(d, [20], seed=60)
    cache, sc = build_cache(case)
    j = 13
    kpe = O.bf16_bits_to_f64(case.ctx_k_pe)
    qpe = np.zeros((1, d.H, d.Dr))
    # score_t = scale * alpha * (k_j . k_t); choose alpha for a gap of >= 40
    gaps = kpe[j] @ kpe[j] - np.delete(kpe @ kpe[j], j)
    alpha = 40.0 / (case.scale * gaps.min())
    qpe[0, :, :] = alpha * kpe[j]
    qpe_bits = W.f32_to_bf16_bits(qpe.astype(np.float32))
    c2 = W.Case(**{**case.__dict__, "q_pe": qpe_bits, "q_nope": np.zeros_like(case.q_nope)})
    out, _ = run_decode(c2, cache, sc)
    want = np.einsum("hvr,r->hv", O.bf16_bits_to_f64(case.w_uv), O.bf16_bits_to_f64(case.ctx_c_kv[j]))
    assert rel(out[0], want) < 1e-12


def test_closed_form_two_keys():
    """Closed form: one head, scale 1, scores 0 and 1 give weights 1/(1+e)
    and e/(1+e); lse = log(1 + e).  R = 2, Dr = 1, identity W_UK and W_UV."""
    d = W.Dims(H=1, R=2, Dr=1, Dn=2, Dv=2, page_size=2)
    bits = lambda a: W.f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    case = W.Case(name="closed", dims=d, kv_dtype=O.KV_BF16, num_layers=1, layer=0, num_pages=2,
                  scale=1.0, window=0,
                  ctx_c_kv=bits([[1.0, 0.0], [0.0, 1.0]]), ctx_k_pe=bits([[0.0], [1.0]]),
                  ctx_slots=np.array([2, 3]), block_tables=np.array([[1, 0]], np.int32),
                  context_lens=np.array([2], np.int32),
                  q_nope=bits([[[0.0, 0.5]]]), q_pe=bits([[[0.5]]]),
                  w_uk=bits([[[1.0, 0.0], [0.0, 1.0]]]), w_uv=bits([[[1.0, 0.0], [0.0, 1.0]]]))
    cache, sc = build_cache(case)
    e = math.e
    for form in ("absorbed", "expanded"):
        out, lse = run_decode(case, cache, sc, form=form)
        assert np.allclose(out[0, 0], [1 / (1 + e), e / (1 + e)], rtol=0, atol=1e-15)
        assert abs(lse[0, 0] - math.log(1 + e)) < 1e-15


def test_empty_context_gives_zero_and_neg_inf():
    case = W.custom(small_dims(), [0, 3], seed=2)
    cache, sc = build_cache(case)
    out, lse = run_decode(case, cache, sc)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(out[1]).all()


def test_fp8_decode_uses_dequantised_values():
    """fp8 decode == bf16-form decode over the dequantised values."""
    case = W.custom(small_dims(R=16, Dr=8), [7, 19], seed=70, kv_dtype=O.KV_FP8, sharp=True)
    cache, sc = build_cache(case)
    out, lse = run_decode(case, cache, sc)
    codes, scl = O.fp8_quantize_tokens(np.concatenate([case.ctx_c_kv, case.ctx_k_pe], axis=1))
    deq = O.E4M3_TABLE[codes] * scl[:, None].astype(np.float64)
    qn = O.bf16_bits_to_f64(case.q_nope)
    qp = O.bf16_bits_to_f64(case.q_pe)
    wuk = O.bf16_bits_to_f64(case.w_uk)
    wuv = O.bf16_bits_to_f64(case.w_uv)
    for b in range(2):
        X = deq[request_rows(case, b)]
        o, l = O.attend_expanded(qn[b], qp[b], X, wuk, wuv, case.scale, 16)
        assert rel(out[b], o) < 1e-12


# ---------------------------------------------------------------------------
# Fused RMSNorm + RoPE write
# ---------------------------------------------------------------------------

def test_f64_to_bf16_matches_torch_on_float32_and_ties_to_even():
    rng = np.random.default_rng(7)
    x32 = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 50000),
                          np.array([0.0, -0.0, 1e-40, -1e-40, 3e38], np.float32)]).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(x32.astype(np.float64)), want)
    # exact midpoints between neighbouring bf16 values go to the even one,
    # and the smallest step past a midpoint goes away from it
    grid = O.bf16_bits_to_f64(np.arange(0x3F80, 0x3F90, dtype=np.uint16))  # 1.0 .. 1.1171875
    mids = (grid[:-1] + grid[1:]) / 2
    got = O.f64_to_bf16_bits(mids)
    lo_bits = np.arange(0x3F80, 0x3F8F, dtype=np.uint16)
    assert np.array_equal(got, np.where(lo_bits % 2 == 0, lo_bits, lo_bits + 1))
    assert np.array_equal(O.f64_to_bf16_bits(np.nextafter(mids, np.inf)), lo_bits + 1)
    assert np.array_equal(O.f64_to_bf16_bits(np.nextafter(mids, -np.inf)), lo_bits)
    # a float64 just past a midpoint that float32 would round onto the midpoint
    # (double rounding) still goes up
    tricky = grid[0] + 2.0 ** -8 + 2.0 ** -40
    assert O.f64_to_bf16_bits(np.array([tricky]))[0] == 0x3F81


def test_rms_norm_closed_forms_and_torch():
    rng = np.random.default_rng(8)
    R = 512
    c = W.f32_to_bf16_bits(np.full((1, R), 0.75, np.float32))
    w = W.f32_to_bf16_bits(np.full(R, 1.5, np.float32))
    y = O.rms_norm(c, w, 0.0)
    assert np.allclose(y, 1.5, rtol=0, atol=1e-15)          # constant row -> weight
    y = O.rms_norm(c, w, 1.0)
    assert np.allclose(y, 0.75 / math.sqrt(0.5625 + 1.0) * 1.5, rtol=1e-15)
    x = W.bf16_normal(rng, (16, R), 2.0)
    wr = W.f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(R)).astype(np.float32))
    want = torch.nn.functional.rms_norm(torch.from_numpy(O.bf16_bits_to_f64(x)), (R,),
                                        torch.from_numpy(O.bf16_bits_to_f64(wr)), eps=1e-6).numpy()
    assert np.max(np.abs(O.rms_norm(x, wr, 1e-6) - want)) < 1e-13
    # scale invariance with eps = 0
    x2 = W.f32_to_bf16_bits(O.bf16_bits_to_f32(x) * np.float32(4.0))
    assert np.max(np.abs(O.rms_norm(x2, wr, 0.0) - O.rms_norm(x, wr, 0.0))) < 1e-13


@pytest.mark.parametrize("interleaved", [True, False])
def test_rope_relative_position_property(interleaved):
    """RoPE's defining property: <rope(q, p), rope(k, p')> depends on p - p'
    only; and position 0 is the identity, pair norms are kept."""
    rng = np.random.default_rng(9)
    Dr = 64
    tab = W.rope_table(4096, Dr)
    q = W.bf16_normal(rng, (1, Dr), 1.0)
    k = W.bf16_normal(rng, (1, Dr), 1.0)
    dots = []
    for base in (0, 77, 1000, 3000):
        qa = O.rope_rotate(q, [base + 19], tab, interleaved)
        kb = O.rope_rotate(k, [base], tab, interleaved)
        dots.append(float((qa @ kb.T)[0, 0]))
    assert max(dots) - min(dots) < 2e-5 * max(abs(d) for d in dots)
    assert np.array_equal(O.rope_rotate(q, [0], tab, interleaved), O.bf16_bits_to_f64(q))
    y = O.rope_rotate(q, [1234], tab, interleaved)
    a, b = O.rope_pairs(Dr, interleaved)
    x = O.bf16_bits_to_f64(q)
    n_in = x[:, a] ** 2 + x[:, b] ** 2
    n_out = y[:, a] ** 2 + y[:, b] ** 2
    assert np.allclose(n_in, n_out, rtol=2e-7)


def test_rope_layouts_agree_through_the_pair_permutation():
    rng = np.random.default_rng(10)
    Dr = 64
    tab = W.rope_table(100, Dr)
    x = W.bf16_normal(rng, (5, Dr), 1.0)
    pos = rng.integers(0, 100, 5)
    ia, ib = O.rope_pairs(Dr, True)
    ha, hb = O.rope_pairs(Dr, False)
    perm = np.empty(Dr, dtype=np.int64)
    perm[ha], perm[hb] = ia, ib          # half-split slot j holds interleaved element perm[j]
    y_int = O.rope_rotate(x, pos, tab, True)
    y_half = O.rope_rotate(x[:, perm], pos, tab, False)
    assert np.array_equal(y_half, y_int[:, perm])


def test_fused_write_without_norm_or_rope_is_write_kv():
    d = W.Dims(H=1, R=64, Dr=16, Dn=8, Dv=8, page_size=16)
    fc = W.fused_write_case(d, 40, seed=11, pad_every=5)
    for kv in (O.KV_BF16, O.KV_FP8):
        dt = np.uint16 if kv == O.KV_BF16 else np.uint8
        a = np.zeros((1, fc.num_pages, 16, d.D), dt)
        b = np.zeros_like(a)
        sa = np.zeros((1, fc.num_pages, 16), np.float32)
        sb = np.zeros_like(sa)
        O.write_kv(a, sa, 0, fc.c_kv, fc.k_pe, fc.slots, kv)
        O.write_kv_fused(b, sb, 0, fc.c_kv, fc.k_pe, fc.slots, fc.positions, None, 0.0, None, True, kv)
        assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_fused_write_rows_are_normed_and_rotated():
    """Read back through the cache: the latent part has unit RMS up to the
    weight and bf16 rounding, and the rope part keeps each pair's norm."""
    d = W.Dims(H=1, R=512, Dr=64, Dn=8, Dv=8, page_size=64)
    fc = W.fused_write_case(d, 30, seed=12, c_std=3.0)
    cache = np.zeros((1, fc.num_pages, 64, d.D), np.uint16)
    O.write_kv_fused(cache, None, 0, fc.c_kv, fc.k_pe, fc.slots, fc.positions, fc.norm_weight,
                     fc.eps, fc.cos_sin, True)
    rows = O.bf16_bits_to_f64(cache[0].reshape(-1, d.D)[fc.slots])
    w = O.bf16_bits_to_f64(fc.norm_weight)
    rms = np.sqrt(np.mean((rows[:, :512] / w) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=5e-3)
    x = O.bf16_bits_to_f64(fc.k_pe)
    a, b = O.rope_pairs(64, True)
    assert np.allclose(rows[:, 512:][:, a] ** 2 + rows[:, 512:][:, b] ** 2, x[:, a] ** 2 + x[:, b] ** 2,
                       rtol=2e-2, atol=1e-6)


def test_planted_rope_sign_is_caught(monkeypatch):
    real = O.rope_rotate

    def bad(x_bits, positions, cos_sin, interleaved):
        tab = np.asarray(cos_sin, np.float32).copy()
        tab[:, tab.shape[1] // 2:] *= -1  # rotate the wrong way for one operand only
        return real(x_bits, positions, tab if np.asarray(positions).ravel()[0] % 2 else cos_sin,
                    interleaved)
    monkeypatch.setattr(O, "rope_rotate", bad)
    with pytest.raises(AssertionError):
        test_rope_relative_position_property(True)


# ---------------------------------------------------------------------------
# Index-list (top-k) attention
# ---------------------------------------------------------------------------

def _sparse_case(window=0, sharp=True, ctx=(40, 77, 5)):
    case = W.custom(small_dims(H=3, R=16, Dr=8, Dn=8, Dv=8, ps=8), list(ctx), seed=61, sharp=True,
                    window=window)
    return case


def test_sparse_list_covering_the_range_equals_dense():
    """A list holding every visible position (shuffled, with pads, future and
    out-of-range positions) gives the dense result."""
    for window in (0, 6):
        case = _sparse_case(window)
        cache, sc = build_cache(case)
        rng = np.random.default_rng(5)
        K = 100
        lists = np.full((case.batch, K), -1, np.int32)
        for b, n in enumerate(case.context_lens):
            vals = np.concatenate([rng.permutation(int(n)), [int(n) + 3, int(n) + 50]])
            lists[b, rng.permutation(K)[:len(vals)]] = vals
        got, glse = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, lists,
                                       case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                       case.scale, window)
        ref, rlse = run_decode(case, cache, sc, window=window)
        assert rel(got, ref) < 1e-12 and np.max(np.abs(glse - rlse)) < 1e-12


def test_sparse_list_brute_force_and_window_as_list():
    """Scalar brute force over the listed keys (contiguous rows, math.fsum),
    and the window expressed as a key list equals the windowed decode."""
    case = _sparse_case()
    cache, sc = build_cache(case)
    d = case.dims
    qpos = case.context_lens - 1
    lists = W.key_lists(62, qpos, case.context_lens, 24)
    got, _ = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, lists,
                                case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale)
    wuk = O.bf16_bits_to_f64(case.w_uk)
    wuv = O.bf16_bits_to_f64(case.w_uv)
    for b in range(case.batch):
        rows = request_rows(case, b)
        c = O.bf16_bits_to_f64(case.ctx_c_kv[rows])
        r = O.bf16_bits_to_f64(case.ctx_k_pe[rows])
        keys = [int(t) for t in lists[b] if 0 <= t <= qpos[b]]
        qn = O.bf16_bits_to_f64(case.q_nope[b])
        qp = O.bf16_bits_to_f64(case.q_pe[b])
        for h in range(d.H):
            sc_ = [case.scale * math.fsum([math.fsum(qn[h][i] * wuk[h][i][j] * c[t][j]
                                                     for i in range(d.Dn) for j in range(d.R)),
                                           math.fsum(qp[h][i] * r[t][i] for i in range(d.Dr))])
                   for t in keys]
            m = max(sc_)
            e = [math.exp(x - m) for x in sc_]
            tot = math.fsum(e)
            want = [math.fsum(e[k] * math.fsum(wuv[h][v][j] * c[keys[k]][j] for j in range(d.R))
                              for k in range(len(keys))) / tot for v in range(d.Dv)]
            assert rel(got[b, h], np.array(want)) < 1e-11
    # window 6 as a key list
    w = 6
    wl = np.full((case.batch, 10), -1, np.int32)
    for b, n in enumerate(case.context_lens):
        pos = np.arange(max(0, int(n) - w), int(n))
        wl[b, :len(pos)] = pos[::-1]
    got, _ = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, wl,
                                case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale)
    ref, _ = run_decode(case, cache, sc, window=w)
    assert rel(got, ref) < 1e-12


def test_sparse_prefill_rows_and_edge_lists():
    """Prefill rows see only listed keys up to their own position; a
    one-entry list returns that token's value; an empty list gives 0, -inf;
    a repeated position is refused."""
    d = small_dims(H=2, R=16, Dr=8, Dn=8, Dv=8, ps=8)
    case = W.prefill_case(d, [20, 3], [6, 4], seed=63, sharp=True)
    cache, sc = build_cache(case)
    Tq = case.q_nope.shape[0]
    lists = np.full((Tq, 30), -1, np.int32)
    for b in range(2):
        s0, s1 = int(case.query_start_loc[b]), int(case.query_start_loc[b + 1])
        n = int(case.context_lens[b])
        for r in range(s0, s1):
            lists[r, :n] = np.random.default_rng(r).permutation(n)  # includes future keys
    got, _ = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, lists,
                                case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                case.scale, query_start_loc=case.query_start_loc)
    ref, _ = O.prefill_chunk(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, case.query_start_loc,
                             case.block_tables, case.context_lens, case.w_uk, case.w_uv, case.scale)
    assert rel(got, ref) < 1e-12
    one = np.full((Tq, 4), -1, np.int32)
    one[:, 1] = 2
    got, lse = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, one,
                                  case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                  case.scale, query_start_loc=case.query_start_loc)
    X0 = O.gather_latent(cache, sc, case.kv_dtype, 0, case.block_tables[0], 26)
    want = np.einsum("hvr,r->hv", O.bf16_bits_to_f64(case.w_uv), X0[2, :16])
    assert np.max(np.abs(got[0] - want)) < 1e-13
    none = np.full((Tq, 4), -1, np.int32)
    got, lse = O.sparse_attention(cache, sc, case.kv_dtype, 0, case.q_nope, case.q_pe, none,
                                  case.block_tables, case.context_lens, case.w_uk, case.w_uv,
                                  case.scale, query_start_loc=case.query_start_loc)
    assert (got == 0).all() and np.isneginf(lse).all()
    with pytest.raises(AssertionError):
        O.sparse_visible([3, 5, 3], 10, 0)


def test_planted_sparse_future_key_is_caught(monkeypatch):
    """A key list filter that forgets the causal bound lets prefill rows see
    listed future tokens; the prefill pin catches it."""
    def no_causal_bound(key_list, p, window):
        lst = np.asarray(key_list, dtype=np.int64)
        return lst[lst >= O.visible_range(p, window)[0]]
    monkeypatch.setattr(O, "sparse_visible", no_causal_bound)
    with pytest.raises(AssertionError):
        test_sparse_prefill_rows_and_edge_lists()


# ---------------------------------------------------------------------------
# Planted mistakes: the pins above must catch them
# ---------------------------------------------------------------------------

def _planted(monkeypatch, attend):
    monkeypatch.setattr(O, "attend_absorbed", attend)


def _bruteforce_agrees(window=0):
    case = W.custom(small_dims(), [9, 14], seed=91, sharp=True)
    cache, sc = build_cache(case)
    out, _ = run_decode(case, cache, sc, window=window)
    return all(rel(out[b], brute_force_request(case, b, window)[0]) < 1e-12 for b in range(2))


def test_planted_dropped_rope_term_is_caught(monkeypatch):
    real = O.attend_absorbed
    _planted(monkeypatch, lambda qn, qp, X, *a: real(qn, np.zeros_like(qp), X, *a))
    assert not _bruteforce_agrees()


def test_planted_transposed_wuk_is_caught(monkeypatch):
    real = O.attend_absorbed

    def bad(qn, qp, X, wuk, wuv, scale, R):
        return real(qn, qp, X, np.ascontiguousarray(np.swapaxes(wuk, 1, 2)[:, :, :R]
                                                    if wuk.shape[1] == wuk.shape[2] else wuk[:, ::-1]),
                    wuv, scale, R)
    _planted(monkeypatch, bad)
    assert not _bruteforce_agrees()


def test_planted_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(O, "visible_range", lambda p, w: (0 if w <= 0 else max(0, p - w), p + 1))
    assert not _bruteforce_agrees(window=3)


def test_planted_wrong_scale_is_caught(monkeypatch):
    real = O.attend_absorbed
    _planted(monkeypatch, lambda qn, qp, X, wuk, wuv, scale, R: real(qn, qp, X, wuk, wuv, scale * 1.01, R))
    assert not _bruteforce_agrees()


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

def test_workloads_are_deterministic_and_shaped():
    a, b = W.tiny(), W.tiny()
    for k in ("ctx_c_kv", "ctx_k_pe", "q_nope", "q_pe", "w_uk", "w_uv", "block_tables"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert a.block_tables.shape == (2, 8) and sorted(a.block_tables.ravel().tolist()) == list(range(16))
    assert a.context_lens.tolist() == [37, 70]
    lens = W.v3_context_lens()
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 32768
    ctx, bt, npg, poison, qsl = W.mixed_layout()
    assert ctx.shape == (128,) and qsl.tolist() == [i * 512 for i in range(9)]
    assert (bt[:, :][bt != poison] < npg).all()
