"""Plain, slow, fp64 CPU oracle for paged multi-head latent attention (MLA)
over a block-table-indexed latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, links or runs
this module.  Only the test-suite, the smoke entry point and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP path: the only thing
both sides share is the seeded input generator, which holds none of the
method's arithmetic.

Sources (web pages, cited by title and section):
  [SHIM]    "feat(serving): DeepSeek-V2/V3 paged-attention shim (MLA)"
            (MoE-Infinity pull request 195)
  [SWA]     "[Models] Support MLA_SWA functionality" (FastDeploy pull request 8049)
  [CHUNK]   "[Attention] MLA with chunked prefill" (vLLM pull request 12639)
  [UNIFIED] "[unified-memory] Let Kimi-Linear use the paged MLA attention
            backends" (SGLang pull request 32972)
  [OFP8]    OCP 8-bit Floating Point Specification (OFP8), E4M3 format
            (the pages name "fp8_e4m3" but do not define it).

What is computed (all in float64 unless stated):

* Cache layout: one latent vector per token, [c_kv (R values) | k_pe (Dr
  values)], stored per layer and per page: cache[L, P, ps, R + Dr].  The
  leading layer dimension comes from [SHIM] "Root causes" item 5 and
  "Changes" (per-layer KV cache with a leading layer dim); the 512 + 64 split
  from [UNIFIED] "Validation" (kv_lora_rank 512 + qk_rope_head_dim 64).
* Head dimensions: keys are qk_nope + qk_rope, values v_head_dim, and the
  softmax scale is an explicit argument ([SHIM] "Root causes" item 3 and
  "Changes": the MLA scale is passed, not derived from a padded head dim).
* The latent up-projection kv_b_proj (named in [CHUNK] "Future work") is
  taken as W_UK[h] : [Dn, R] and W_UV[h] : [Dv, R], so that
  k_nope = W_UK[h] c and v = W_UV[h] c.  Reading: the pages name kv_b_proj
  but not its layout.
* Decode attends to every cached token of the request including the token
  just written; the query sits at position n - 1 ([SHIM] "Root causes"
  items 2 and 4: decode tokens are written before attention and the context
  length must not count one token too many).
* Sliding window ([SWA] "Motivation"): with w > 0 a query at position p sees
  keys t with p - w < t <= p.  Reading: the pages give no boundary
  convention; this one keeps exactly min(w, p + 1) keys, the query's own
  token included.
* Chunked prefill ([CHUNK] title and lm_eval runs): the m new tokens of a
  request sit at positions n - m .. n - 1 and row i sees keys t <= n - m + i.
* fp8 cache ([SWA] "Modifications": uint8 MLA cache; [UNIFIED] "Validation":
  fp8_e4m3 KV at page size 64).  Reading: one fp32 scale per token covering
  all R + Dr values; scale = amax / 448 (fp32 division), 1.0 when amax is 0;
  code = E4M3 round-to-nearest-even, saturating at +-448, of x / scale (fp32
  division).  Dequantised value = e4m3(code) * scale, exact in float64.
* Pad rows: a negative slot writes nothing ([UNIFIED] "Cuda-graph safety":
  stale pad-row locations scatter garbage into live pages).
* Split-KV combine: the log-sum-exp merge of partial results over disjoint
  key subsets (the pages are silent; this is the textbook identity).
* Fused write ("Support dsv4 model", Model Architecture and Inference: fused
  normalization/RoPE and packed KV writers; [CHUNK] "Future work": the cache
  holds kv_c_normed): RMSNorm of the latent and RoPE of the rope part, each
  rounded to bf16, then the ordinary write.  The readings are stated at
  write_kv_fused.
"""
from __future__ import annotations

import math

import numpy as np

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3"

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly: bf16 is the
    top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def e4m3_value(code: int) -> float:
    """[OFP8] E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
    no infinities, S.1111.111 is NaN, subnormals at exponent field 0."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
# Non-negative finite magnitudes, indexed by code 0x00..0x7E; strictly increasing.
_E4M3_MAGS = E4M3_TABLE[:0x7F].copy()


def e4m3_encode_satfinite(x32) -> np.ndarray:
    """Encode float32 values as E4M3 codes: round to the nearest representable
    value, ties to the even code, magnitudes beyond 448 saturate to 448, the
    sign is kept (also for results that round to zero).  NaN maps to 0x7F."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    a = np.abs(flat)
    hi = np.searchsorted(_E4M3_MAGS, a, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E4M3_MAGS[hi], hi, code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    out[:] = code.astype(np.uint8)
    out |= np.where(np.signbit(flat), 0x80, 0).astype(np.uint8)
    out[np.isnan(flat)] = 0x7F
    return out.reshape(x.shape)


def fp8_quantize_tokens(rows_bits):
    """Per-token fp8 quantisation of bf16 rows [T, D] (reading of the uint8 MLA
    cache, see module docstring).  All arithmetic is IEEE float32, as numpy
    float32 operations are correctly rounded.  Returns (codes uint8 [T, D],
    scale float32 [T])."""
    x = bf16_bits_to_f32(rows_bits)
    amax = np.max(np.abs(x), axis=-1).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode_satfinite(q), scale


# --------------------------------------------------------------------------
# Cache write: [SHIM] "Root causes" item 2 and "Changes" (write KV whenever a
# slot mapping is present, for prefill and decode tokens alike).
# --------------------------------------------------------------------------


def write_kv(cache, cache_scale, layer, c_kv_bits, k_pe_bits, slot_mapping, kv_dtype=KV_BF16):
    """cache[layer, s // ps, s % ps, :] = [c_kv_i | k_pe_i] for each token i with
    slot s = slot_mapping[i] >= 0.  bf16: bit copy.  fp8: per-token
    quantisation with the scale stored in cache_scale[layer, s // ps, s % ps].
    Negative slots are pad rows and write nothing.  Non-negative slots in one
    call must be distinct (a caller error otherwise)."""
    L, P, ps, D = cache.shape
    c_kv = np.asarray(c_kv_bits, dtype=np.uint16)
    k_pe = np.asarray(k_pe_bits, dtype=np.uint16)
    assert c_kv.shape[1] + k_pe.shape[1] == D
    slots = np.asarray(slot_mapping, dtype=np.int64)
    assert 0 <= layer < L
    live = np.nonzero(slots >= 0)[0]
    s = slots[live]
    assert np.unique(s).size == s.size, "duplicate slots in one write"
    assert (s < P * ps).all(), "slot beyond the cache"
    rows = np.concatenate([c_kv[live], k_pe[live]], axis=1)
    pages, offs = s // ps, s % ps
    if kv_dtype == KV_BF16:
        cache[layer, pages, offs, :] = rows
    else:
        codes, sc = fp8_quantize_tokens(rows)
        cache[layer, pages, offs, :] = codes
        cache_scale[layer, pages, offs] = sc


# --------------------------------------------------------------------------
# Fused normalisation and RoPE before the cache write ("Support dsv4 model",
# Model Architecture and Inference: fused normalization/RoPE and packed KV
# writers; "[Attention] MLA with chunked prefill", Future work: the cache holds
# kv_c_normed, the latent after its RMSNorm; "feat(serving): DeepSeek-V2/V3
# paged-attention shim (MLA)", Changes: the HF MLA projection + RoPE are
# reproduced before the cache).  Readings, since the pages give no formulas:
#   * RMSNorm over the R latent values: y = x / sqrt(mean(x^2) + eps) * w, with
#     a bf16 weight w [R] and the caller's eps;
#   * RoPE on the Dr rope values with a caller-supplied table cos_sin
#     [max_pos, Dr] (cos of the Dr/2 angles of a position, then their sines),
#     on pairs (2i, 2i+1) ("interleaved") or (i, i + Dr/2) ("half split"):
#     (a, b) -> (a cos - b sin, b cos + a sin), angle i of the position;
#   * both results are rounded to bf16 (nearest even) before the write, as the
#     unfused producer would hand bf16 rows to the write; the write itself is
#     write_kv's (bit copy, or the fp8 quantisation).
# --------------------------------------------------------------------------


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even) in one step
    (no intermediate float32 rounding).  Finite inputs below 2^128."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    _, e = np.frexp(np.abs(x[nz]))              # |x| = f * 2^e, f in [0.5, 1)
    # bf16 keeps 8 significant bits for normal values (exponent >= -126) and
    # a fixed quantum of 2^-133 below that
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    out[nz] = np.rint(x[nz] / quantum) * quantum  # exact scaling; rint ties to even
    assert np.all(np.abs(out) < 2.0 ** 128), "bf16 overflow"
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    # keep the sign of values that round to zero
    bits |= np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    return bits


def rms_norm(x_bits, weight_bits, eps):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis, in float64."""
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(weight_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * w


def rope_pairs(dr, interleaved):
    """Index pairs (first, second) the rotation acts on, one per angle."""
    h = dr // 2
    i = np.arange(h)
    return (2 * i, 2 * i + 1) if interleaved else (i, i + h)


def rope_rotate(x_bits, positions, cos_sin, interleaved):
    """Rotate each pair (a, b) of x [T, Dr] by angle i of its token's position:
    (a cos - b sin, b cos + a sin), cos / sin read from the fp32 table
    cos_sin[position] (first half cosines, second half sines).  float64."""
    x = bf16_bits_to_f64(x_bits)
    pos = np.asarray(positions, dtype=np.int64)
    tab = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    dr = x.shape[-1]
    h = dr // 2
    cos, sin = tab[pos, :h], tab[pos, h:]
    first, second = rope_pairs(dr, interleaved)
    a, b = x[:, first], x[:, second]
    y = np.empty_like(x)
    y[:, first] = a * cos - b * sin
    y[:, second] = b * cos + a * sin
    return y


def write_kv_fused(cache, cache_scale, layer, c_kv_bits, k_pe_bits, slot_mapping, positions,
                   norm_weight_bits, eps, cos_sin, interleaved, kv_dtype=KV_BF16):
    """The cache write with the latent's RMSNorm and the rope part's rotation
    folded in: write_kv of bf16(rms_norm(c_kv)) and bf16(rope(k_pe)).  A None
    weight skips the norm, a None table the rotation (the row is then copied
    as given).  Pad rows (slot < 0) are skipped like write_kv's."""
    c = (c_kv_bits if norm_weight_bits is None
         else f64_to_bf16_bits(rms_norm(c_kv_bits, norm_weight_bits, eps)))
    r = (k_pe_bits if cos_sin is None
         else f64_to_bf16_bits(rope_rotate(k_pe_bits, positions, cos_sin, interleaved)))
    write_kv(cache, cache_scale, layer, c, r, slot_mapping, kv_dtype)
    return c, r


# --------------------------------------------------------------------------
# Gather through the block table ([UNIFIED] "What this does": kernels read the
# block table directly; pages may sit anywhere in the pool).
# --------------------------------------------------------------------------


def gather_latent(cache, cache_scale, kv_dtype, layer, block_table_row, n):
    """Logical token t < n of a request lives at page block_table_row[t // ps],
    offset t % ps.  Only the first ceil(n / ps) table entries are read.
    Returns X [n, R + Dr] in float64 (dequantised for fp8)."""
    ps = cache.shape[2]
    t = np.arange(n, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // ps]
    offs = t % ps
    raw = cache[layer, pages, offs]
    if kv_dtype == KV_BF16:
        return bf16_bits_to_f64(raw)
    sc = cache_scale[layer, pages, offs].astype(np.float64)
    return E4M3_TABLE[raw] * sc[:, None]


def visible_range(p, window):
    """Keys visible to a query at position p: [lo, p + 1)."""
    lo = 0 if window <= 0 else max(0, p - window + 1)
    return lo, p + 1


# --------------------------------------------------------------------------
# Attention for one query token, all heads
# --------------------------------------------------------------------------


def attend_expanded(q_nope, q_pe, X, w_uk, w_uv, scale, R):
    """Definition (non-absorbed MLA, [SHIM] "Root causes" item 3): per head h,
    key_t = [W_UK[h] c_t ; r_t], value_t = W_UV[h] c_t, query = [q_nope ; q_pe],
    s_t = scale * (query . key_t), softmax over the visible keys,
    out = sum_t p_t value_t, lse = log sum_t exp(s_t).
    w_uk None: q_nope is already latent (W_UK = identity).  w_uv None: the
    output is latent (W_UV = identity).  Inputs are float64 arrays."""
    H = q_nope.shape[0]
    n = X.shape[0]
    C, Rp = X[:, :R], X[:, R:]
    dv = R if w_uv is None else w_uv.shape[1]
    out = np.zeros((H, dv))
    lse = np.full(H, -np.inf)
    if n == 0:
        return out, lse
    for h in range(H):
        k_nope = C if w_uk is None else C @ w_uk[h].T
        keys = np.concatenate([k_nope, Rp], axis=1)
        vals = C if w_uv is None else C @ w_uv[h].T
        q = np.concatenate([q_nope[h], q_pe[h]])
        s = scale * (keys @ q)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[h] = (e @ vals) / l
        lse[h] = m + math.log(l)
    return out, lse


def attend_absorbed(q_nope, q_pe, X, w_uk, w_uv, scale, R):
    """The method (absorbed MLA): q_lat = W_UK[h]^T q_nope, scores against the
    latent [c_t ; r_t] directly, the output accumulated in latent space and
    mapped by W_UV[h] at the end.  Equal to attend_expanded by associativity."""
    H = q_nope.shape[0]
    n = X.shape[0]
    C, Rp = X[:, :R], X[:, R:]
    dv = R if w_uv is None else w_uv.shape[1]
    if n == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    q_lat = q_nope if w_uk is None else np.einsum("hd,hdr->hr", q_nope, w_uk)
    S = scale * (q_lat @ C.T + q_pe @ Rp.T)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    o_lat = (E @ C) / l[:, None]
    out = o_lat if w_uv is None else np.einsum("hvr,hr->hv", w_uv, o_lat)
    return out, m + np.log(l)


def _attend(form):
    return attend_absorbed if form == "absorbed" else attend_expanded


def _weights(w_bits):
    return None if w_bits is None else bf16_bits_to_f64(w_bits)


# --------------------------------------------------------------------------
# Decode, prefill, combine
# --------------------------------------------------------------------------


def decode(cache, cache_scale, kv_dtype, layer, q_nope_bits, q_pe_bits, block_tables,
           context_lens, w_uk_bits, w_uv_bits, scale, window=0, form="absorbed", requests=None):
    """One query token per request at position n_b - 1 over the n_b cached
    tokens (window applied).  Returns (out [B, H, Dv or R], lse [B, H]); rows
    not in `requests` are left NaN.  An empty context gives out 0, lse -inf."""
    R = cache.shape[3] - np.asarray(q_pe_bits).shape[-1]
    qn = bf16_bits_to_f64(q_nope_bits)
    qp = bf16_bits_to_f64(q_pe_bits)
    w_uk, w_uv = _weights(w_uk_bits), _weights(w_uv_bits)
    B, H = qn.shape[0], qn.shape[1]
    dv = R if w_uv is None else w_uv.shape[1]
    out = np.full((B, H, dv), np.nan)
    lse = np.full((B, H), np.nan)
    attend = _attend(form)
    for b in (range(B) if requests is None else requests):
        n = int(context_lens[b])
        if n == 0:
            out[b], lse[b] = 0.0, -np.inf
            continue
        lo, hi = visible_range(n - 1, window)
        X = gather_latent(cache, cache_scale, kv_dtype, layer, block_tables[b], n)[lo:hi]
        out[b], lse[b] = attend(qn[b], qp[b], X, w_uk, w_uv, scale, R)
    return out, lse


def prefill_chunk(cache, cache_scale, kv_dtype, layer, q_nope_bits, q_pe_bits, query_start_loc,
                  block_tables, context_lens, w_uk_bits, w_uv_bits, scale, window=0,
                  form="absorbed", rows=None):
    """Causal chunked prefill ([CHUNK]): request b owns query rows
    query_start_loc[b] .. query_start_loc[b+1]-1, m_b rows in all, whose tokens
    are already in the cache at positions n_b - m_b .. n_b - 1.  Row i of the
    request sees keys t <= n_b - m_b + i (and the window).  Returns
    (out [Tq, H, Dv or R], lse [Tq, H]); rows not in `rows` stay NaN."""
    R = cache.shape[3] - np.asarray(q_pe_bits).shape[-1]
    qn = bf16_bits_to_f64(q_nope_bits)
    qp = bf16_bits_to_f64(q_pe_bits)
    w_uk, w_uv = _weights(w_uk_bits), _weights(w_uv_bits)
    Tq, H = qn.shape[0], qn.shape[1]
    dv = R if w_uv is None else w_uv.shape[1]
    out = np.full((Tq, H, dv), np.nan)
    lse = np.full((Tq, H), np.nan)
    attend = _attend(form)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(qsl) - 1):
        s0, s1 = int(qsl[b]), int(qsl[b + 1])
        m, n = s1 - s0, int(context_lens[b])
        assert 0 <= m <= n, "a chunk cannot be longer than its context"
        mine = [r for r in range(s0, s1) if wanted is None or r in wanted]
        if not mine:
            continue
        X = gather_latent(cache, cache_scale, kv_dtype, layer, block_tables[b], n)
        for r in mine:
            p = n - m + (r - s0)
            lo, hi = visible_range(p, window)
            out[r], lse[r] = attend(qn[r], qp[r], X[lo:hi], w_uk, w_uv, scale, R)
    return out, lse


def sparse_visible(key_list, p, window):
    """Index-list attention ("[Models] Support MLA_SWA functionality",
    Modifications: a top-k indexer builds each query's key list, and the
    sliding window is expressed as such a list; "Support dsv4 model", Model
    Architecture and Inference: sparse index construction).  Reading: a query
    at position p attends to the listed positions that its ordinary visible
    range holds (causal, and the window when w > 0); negative entries are
    unused slots and other entries are ignored.  Listed positions must be
    distinct.  Returns the kept positions in list order."""
    lst = np.asarray(key_list, dtype=np.int64)
    lo, hi = visible_range(p, window)
    keep = lst[(lst >= lo) & (lst < hi)]
    assert np.unique(keep).size == keep.size, "a position listed twice"
    return keep


def sparse_attention(cache, cache_scale, kv_dtype, layer, q_nope_bits, q_pe_bits, key_indices,
                     block_tables, context_lens, w_uk_bits, w_uv_bits, scale, window=0,
                     query_start_loc=None, form="absorbed", rows=None):
    """Attention of each query row over its key list (see sparse_visible).
    Decode (query_start_loc None): row b is request b's query at n_b - 1.
    Prefill: rows query_start_loc[b] .. query_start_loc[b+1]-1 are request b's
    chunk at positions n_b - m_b + i.  key_indices [rows, K] int.  Returns
    (out [rows, H, Dv or R], lse [rows, H]); rows not in `rows` stay NaN."""
    R = cache.shape[3] - np.asarray(q_pe_bits).shape[-1]
    qn = bf16_bits_to_f64(q_nope_bits)
    qp = bf16_bits_to_f64(q_pe_bits)
    w_uk, w_uv = _weights(w_uk_bits), _weights(w_uv_bits)
    Tq, H = qn.shape[0], qn.shape[1]
    dv = R if w_uv is None else w_uv.shape[1]
    out = np.full((Tq, H, dv), np.nan)
    lse = np.full((Tq, H), np.nan)
    attend = _attend(form)
    ctx = np.asarray(context_lens, dtype=np.int64)
    if query_start_loc is None:
        qsl = np.arange(len(ctx) + 1, dtype=np.int64)
    else:
        qsl = np.asarray(query_start_loc, dtype=np.int64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(qsl) - 1):
        s0, s1 = int(qsl[b]), int(qsl[b + 1])
        m, n = s1 - s0, int(ctx[b])
        mine = [r for r in range(s0, s1) if wanted is None or r in wanted]
        if not mine:
            continue
        X = gather_latent(cache, cache_scale, kv_dtype, layer, block_tables[b], n)
        for r in mine:
            p = n - m + (r - s0)
            keep = sparse_visible(key_indices[r], p, window)
            out[r], lse[r] = attend(qn[r], qp[r], X[keep], w_uk, w_uv, scale, R)
    return out, lse


def combine(o_parts, lse_parts):
    """Log-sum-exp merge of partials over disjoint key subsets:
    lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.  A partial with
    lse_s = -inf has weight 0; if every partial is empty, o = 0, lse = -inf.
    o_parts [S, ..., D], lse_parts [S, ...]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    top = np.max(lse_parts, axis=0)
    empty = np.isneginf(top)
    safe_top = np.where(empty, 0.0, top)
    w = np.exp(lse_parts - safe_top[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, safe_top + np.log(np.where(empty, 1.0, tot)))
    frac = w / np.where(empty, 1.0, tot)[None]
    o = np.einsum("s...,s...d->...d", frac, np.nan_to_num(o_parts, nan=0.0, posinf=0.0, neginf=0.0)
                  * (w[..., None] > 0))
    o = np.where(empty[..., None], 0.0, o)
    return o, lse
