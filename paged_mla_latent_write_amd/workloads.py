"""Seeded synthetic inputs for paged MLA (shared by the tests, the benchmark and
the oracle checks).

This module only draws random numbers and lays them out; it holds none of the
attention, write or quantisation arithmetic.  Values are drawn in float32 with
numpy's PCG64 generator and rounded to bfloat16 (round to nearest even), and
handed out as uint16 bit patterns.

Workloads (shapes follow the MLA dimensions the pages use: kv_lora_rank 512 +
qk_rope 64, page size 64, qk_nope 128, v_head 128):

  tiny     batch 2, 4 heads, R 32, Dr 16, Dn 32, Dv 32, page size 16,
           contexts 37 and 70, block table a random permutation of 16 pages
           (8 per request), all values N(0, 0.5^2), scale 1/sqrt(48), 1 layer.
  v2lite   DeepSeek-V2-Lite shape: 16 heads, batch 32, every context 4096,
           27-layer cache, layer 13, 2048 pages, scale 1/sqrt(192).
  v3       DeepSeek-V3 shape, one GPU's full head set: 128 heads, batch 64,
           contexts uniform in [1024, 32768], shuffled block tables.
  v3fp8    as v3 but batch 128, every context 8192, fp8 e4m3 latent cache.
  mixed    4-layer cache; 8 prefill chunks of 512 new tokens over prefixes
           uniform in [2048, 16384] plus 120 decode requests with contexts
           uniform in [2048, 16384]; window 128 on layers 0 and 2.

Except for `tiny`, vectors are N(0, 1) / sqrt(len) with len the vector's own
length (c_kv 512, k_pe 64, q_nope 128, q_pe 64) and W_UK / W_UV are
N(0, 1) / sqrt(R).  "Sharp" variants multiply q_nope and q_pe by constants so
that each of the two score terms has a standard deviation of about 1.5 after
the softmax scale; the plain draws give near-uniform softmax weights, which
would hide a wrong score path.

Unused cache pages, unused layers and block-table entries past a request's
last page point at NaN-filled memory, so that any read the method does not
make shows up as NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
_CHUNK_ROWS = 1 << 16


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_normal(rng, shape, std):
    """N(0, std^2) draws rounded to bf16, generated in row chunks so that very
    large arrays never hold a full float32 copy."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    rows = out.reshape(shape[0], -1)
    for r0 in range(0, rows.shape[0], _CHUNK_ROWS):
        r1 = min(rows.shape[0], r0 + _CHUNK_ROWS)
        x = rng.standard_normal((r1 - r0, rows.shape[1]), dtype=np.float32)
        x *= np.float32(std)
        rows[r0:r1] = f32_to_bf16_bits(x)
    return out


@dataclass
class Dims:
    H: int
    R: int
    Dr: int
    Dn: int
    Dv: int
    page_size: int

    @property
    def D(self):
        return self.R + self.Dr


@dataclass
class Stds:
    c_kv: float
    k_pe: float
    q_nope: float
    q_pe: float
    w: float


def mla_stds(d: Dims) -> Stds:
    return Stds(1 / math.sqrt(d.R), 1 / math.sqrt(d.Dr), 1 / math.sqrt(d.Dn),
                1 / math.sqrt(d.Dr), 1 / math.sqrt(d.R))


def sharp_gains(d: Dims, s: Stds, scale: float, target=1.5):
    """Multipliers for q_nope and q_pe that give each score term a standard
    deviation of `target` (after the softmax scale), from the draw variances:
    var(q_lat . c) = R * Dn * sd(q_nope)^2 * sd(W)^2 * sd(c)^2 and
    var(q_pe . k_pe) = Dr * sd(q_pe)^2 * sd(k_pe)^2."""
    sd_lat = math.sqrt(d.R * d.Dn) * s.q_nope * s.w * s.c_kv
    sd_rope = math.sqrt(d.Dr) * s.q_pe * s.k_pe
    return target / (scale * sd_lat), target / (scale * sd_rope)


@dataclass
class Case:
    """One attention call's synthetic inputs plus the cache population.

    population: ctx_c_kv [T, R], ctx_k_pe [T, Dr] (bf16 bits), ctx_slots [T]
    int64 - every cached token, written through the cache-write op before the
    attention call.  block_tables [B, max_blocks] int32, context_lens [B]
    int32 (tokens attended, the newest included).  q_nope [Nq, H, Dn],
    q_pe [Nq, H, Dr] with Nq = B for decode or the chunk rows for prefill
    (query_start_loc [B + 1] int32 then set).  w_uk [H, Dn, R],
    w_uv [H, Dv, R]."""
    name: str
    dims: Dims
    kv_dtype: str
    num_layers: int
    layer: int
    num_pages: int
    scale: float
    window: int
    ctx_c_kv: np.ndarray
    ctx_k_pe: np.ndarray
    ctx_slots: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    q_nope: np.ndarray
    q_pe: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    query_start_loc: np.ndarray | None = None
    poison_page: int | None = None
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    def new_token_rows(self):
        """Indices into the population of each request's newest token (the
        one a decode step writes before it attends)."""
        ends = np.cumsum(self.context_lens.astype(np.int64))
        return ends - 1


def slots_for(block_tables, context_lens, page_size):
    """Cache slot of every token, request by request in logical order:
    slot = block_tables[b, t // ps] * ps + t % ps."""
    out = []
    for b, n in enumerate(np.asarray(context_lens, dtype=np.int64)):
        t = np.arange(n, dtype=np.int64)
        out.append(block_tables[b, t // page_size].astype(np.int64) * page_size + t % page_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def assign_pages(rng, context_lens, page_size, num_pages=None, max_blocks=None, shuffle=True):
    """Give each request ceil(n / ps) pages taken from a random permutation of
    the pool.  Entries past a request's last page point at a poison page (the
    last page of the pool) that stays NaN-filled."""
    nblk = [(int(n) + page_size - 1) // page_size for n in context_lens]
    used = sum(nblk)
    if num_pages is None:
        num_pages = used + 1
    assert num_pages >= used
    if max_blocks is None:
        max_blocks = max(nblk + [1])
    poison = num_pages - 1 if num_pages > used else None
    perm = _rng_perm(rng, used if poison is not None else num_pages, shuffle)
    bt = np.full((len(nblk), max_blocks), poison if poison is not None else 0, dtype=np.int32)
    off = 0
    for b, k in enumerate(nblk):
        bt[b, :k] = perm[off:off + k]
        off += k
    return bt, num_pages, poison


def _rng_perm(rng, n, shuffle):
    return rng.permutation(n).astype(np.int32) if shuffle else np.arange(n, dtype=np.int32)


def _decode_case(name, seed, dims, ctx, *, kv_dtype="bf16", num_layers=1, layer=0, num_pages=None,
                 stds=None, scale=None, window=0, sharp=False, block_tables=None):
    rng = _rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    if block_tables is None:
        bt, num_pages, poison = assign_pages(rng, ctx, dims.page_size, num_pages)
    else:
        bt, poison = block_tables, None
    s = stds or mla_stds(dims)
    scale = scale if scale is not None else 1 / math.sqrt(dims.Dn + dims.Dr)
    T = int(ctx.sum())
    c_kv = bf16_normal(rng, (T, dims.R), s.c_kv)
    k_pe = bf16_normal(rng, (T, dims.Dr), s.k_pe)
    gn, gp = sharp_gains(dims, s, scale) if sharp else (1.0, 1.0)
    B = len(ctx)
    q_nope = bf16_normal(rng, (B, dims.H, dims.Dn), s.q_nope * gn)
    q_pe = bf16_normal(rng, (B, dims.H, dims.Dr), s.q_pe * gp)
    w_uk = bf16_normal(rng, (dims.H, dims.Dn, dims.R), s.w)
    w_uv = bf16_normal(rng, (dims.H, dims.Dv, dims.R), s.w)
    return Case(name=name, dims=dims, kv_dtype=kv_dtype, num_layers=num_layers, layer=layer,
                num_pages=num_pages, scale=scale, window=window, ctx_c_kv=c_kv, ctx_k_pe=k_pe,
                ctx_slots=slots_for(bt, ctx, dims.page_size), block_tables=bt, context_lens=ctx,
                q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, poison_page=poison,
                meta=dict(seed=seed, sharp=sharp, gain_nope=gn, gain_pe=gp))


TINY_DIMS = Dims(H=4, R=32, Dr=16, Dn=32, Dv=32, page_size=16)
MLA_DIMS_16 = Dims(H=16, R=512, Dr=64, Dn=128, Dv=128, page_size=64)
MLA_DIMS_128 = Dims(H=128, R=512, Dr=64, Dn=128, Dv=128, page_size=64)


def tiny(sharp=False, seed=1):
    """Tiny decode: block table = randperm(16) reshaped to 2 x 8."""
    rng = _rng(seed + 1000)
    bt = rng.permutation(16).astype(np.int32).reshape(2, 8)
    std = Stds(0.5, 0.5, 0.5, 0.5, 0.5)
    return _decode_case("tiny", seed, TINY_DIMS, [37, 70], num_pages=16, stds=std,
                        scale=1 / math.sqrt(48), sharp=sharp, block_tables=bt)


def v2lite(sharp=False, seed=2):
    return _decode_case("v2lite", seed, MLA_DIMS_16, [4096] * 32, num_layers=27, layer=13,
                        num_pages=2048, sharp=sharp)


def v3_context_lens(seed=3, batch=64, lo=1024, hi=32768):
    return _rng(seed + 1000).integers(lo, hi + 1, size=batch).astype(np.int32)


def v3(sharp=False, seed=3, batch=64):
    return _decode_case("v3", seed, MLA_DIMS_128, v3_context_lens(seed, batch), sharp=sharp)


def v3fp8(sharp=False, seed=4, batch=128, ctx=8192):
    return _decode_case("v3fp8", seed, MLA_DIMS_128, [ctx] * batch, kv_dtype="fp8_e4m3",
                        num_pages=batch * ctx // 64, sharp=sharp)


def custom(dims: Dims, ctx, *, seed=0, kv_dtype="bf16", num_layers=1, layer=0, window=0,
           sharp=False, scale=None, stds=None, name="custom"):
    return _decode_case(name, seed, dims, ctx, kv_dtype=kv_dtype, num_layers=num_layers,
                        layer=layer, window=window, sharp=sharp, scale=scale, stds=stds)


# ---------------------------------------------------------------------------
# Mixed prefill + decode step with a sliding window on alternate layers
# ---------------------------------------------------------------------------

MIXED_WINDOWS = (128, 0, 128, 0)


@dataclass
class MixedLayer:
    """One layer of the mixed step.  Requests 0..n_prefill-1 are prefill
    chunks (rows query_start_loc[b]..query_start_loc[b+1]-1 of q_nope_p), the
    rest are single-token decodes.  `pre_*` is the population written before
    the step (every cached token except the step's new ones); `new_*` are the
    step's new tokens (the chunks, then one per decode request)."""
    layer: int
    window: int
    dims: Dims
    num_layers: int
    num_pages: int
    scale: float
    block_tables: np.ndarray
    context_lens: np.ndarray
    n_prefill: int
    query_start_loc: np.ndarray
    pre_c_kv: np.ndarray
    pre_k_pe: np.ndarray
    pre_slots: np.ndarray
    new_c_kv: np.ndarray
    new_k_pe: np.ndarray
    new_slots: np.ndarray
    q_nope_p: np.ndarray
    q_pe_p: np.ndarray
    q_nope_d: np.ndarray
    q_pe_d: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    poison_page: int | None = None


def mixed_layout(seed=5, n_prefill=8, chunk=512, n_decode=120, lo=2048, hi=16384):
    """Context lengths and block tables shared by every layer of the step."""
    rng = _rng(seed + 1000)
    prefix = rng.integers(lo, hi + 1, size=n_prefill)
    dec = rng.integers(lo, hi + 1, size=n_decode)
    ctx = np.concatenate([prefix + chunk, dec]).astype(np.int32)
    bt, num_pages, poison = assign_pages(rng, ctx, 64, None)
    qsl = np.arange(n_prefill + 1, dtype=np.int32) * chunk
    return ctx, bt, num_pages, poison, qsl


def mixed(layer, sharp=False, seed=5, n_prefill=8, chunk=512, n_decode=120):
    ctx, bt, num_pages, poison, qsl = mixed_layout(seed, n_prefill, chunk, n_decode)
    d = MLA_DIMS_128
    s = mla_stds(d)
    scale = 1 / math.sqrt(d.Dn + d.Dr)
    rng = _rng(seed * 100 + layer)
    slots = slots_for(bt, ctx, d.page_size)
    starts = np.concatenate([[0], np.cumsum(ctx.astype(np.int64))[:-1]])
    is_new = np.zeros(slots.shape[0], dtype=bool)
    for b, n in enumerate(ctx):
        m = chunk if b < n_prefill else 1
        is_new[starts[b] + n - m: starts[b] + n] = True
    T = slots.shape[0]
    c_kv = bf16_normal(rng, (T, d.R), s.c_kv)
    k_pe = bf16_normal(rng, (T, d.Dr), s.k_pe)
    gn, gp = sharp_gains(d, s, scale) if sharp else (1.0, 1.0)
    q_nope_p = bf16_normal(rng, (n_prefill * chunk, d.H, d.Dn), s.q_nope * gn)
    q_pe_p = bf16_normal(rng, (n_prefill * chunk, d.H, d.Dr), s.q_pe * gp)
    q_nope_d = bf16_normal(rng, (n_decode, d.H, d.Dn), s.q_nope * gn)
    q_pe_d = bf16_normal(rng, (n_decode, d.H, d.Dr), s.q_pe * gp)
    w_uk = bf16_normal(rng, (d.H, d.Dn, d.R), s.w)
    w_uv = bf16_normal(rng, (d.H, d.Dv, d.R), s.w)
    return MixedLayer(layer=layer, window=MIXED_WINDOWS[layer], dims=d, num_layers=4,
                      num_pages=num_pages, scale=scale, block_tables=bt, context_lens=ctx,
                      n_prefill=n_prefill, query_start_loc=qsl,
                      pre_c_kv=c_kv[~is_new], pre_k_pe=k_pe[~is_new], pre_slots=slots[~is_new],
                      new_c_kv=c_kv[is_new], new_k_pe=k_pe[is_new], new_slots=slots[is_new],
                      q_nope_p=q_nope_p, q_pe_p=q_pe_p, q_nope_d=q_nope_d, q_pe_d=q_pe_d,
                      w_uk=w_uk, w_uv=w_uv, poison_page=poison)


def prefill_case(dims: Dims, prefix_lens, chunk_lens, *, seed=0, window=0, sharp=False,
                 kv_dtype="bf16", scale=None, stds=None, num_layers=1, layer=0):
    """A prefill call: request b has prefix_lens[b] cached tokens and
    chunk_lens[b] new ones (already part of the population, since the chunk is
    written before it attends); q rows are the chunk tokens in order."""
    rng = _rng(seed)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int64)
    ctx = (prefix_lens + chunk_lens).astype(np.int32)
    bt, num_pages, poison = assign_pages(rng, ctx, dims.page_size, None)
    s = stds or mla_stds(dims)
    scale = scale if scale is not None else 1 / math.sqrt(dims.Dn + dims.Dr)
    T = int(ctx.sum())
    c_kv = bf16_normal(rng, (T, dims.R), s.c_kv)
    k_pe = bf16_normal(rng, (T, dims.Dr), s.k_pe)
    gn, gp = sharp_gains(dims, s, scale) if sharp else (1.0, 1.0)
    Tq = int(chunk_lens.sum())
    q_nope = bf16_normal(rng, (Tq, dims.H, dims.Dn), s.q_nope * gn)
    q_pe = bf16_normal(rng, (Tq, dims.H, dims.Dr), s.q_pe * gp)
    w_uk = bf16_normal(rng, (dims.H, dims.Dn, dims.R), s.w)
    w_uv = bf16_normal(rng, (dims.H, dims.Dv, dims.R), s.w)
    qsl = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    return Case(name="prefill", dims=dims, kv_dtype=kv_dtype, num_layers=num_layers, layer=layer,
                num_pages=num_pages, scale=scale, window=window, ctx_c_kv=c_kv, ctx_k_pe=k_pe,
                ctx_slots=slots_for(bt, ctx, dims.page_size), block_tables=bt, context_lens=ctx,
                q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, query_start_loc=qsl,
                poison_page=poison, meta=dict(seed=seed, sharp=sharp))


# ---------------------------------------------------------------------------
# Inputs of the cache write with the latent's RMSNorm and the rope rotation
# folded in
# ---------------------------------------------------------------------------

def rope_table(max_pos, dr, theta=10000.0):
    """A caller's RoPE table, fp32 [max_pos, dr]: for position p the cosines
    of p * theta^(-2i/dr), i < dr/2, then their sines (angles in float64,
    rounded once to float32).  An input of the write, like its rows."""
    inv = theta ** (-np.arange(0, dr, 2, dtype=np.float64) / dr)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclass
class FusedWriteCase:
    """Pre-norm latents c_kv [T, R] and un-rotated k_pe [T, Dr] (bf16 bits),
    their positions [T] int64, slots [T] int64 (some -1 pad rows), a bf16 norm
    weight [R], eps, and a rope table [max_pos, Dr] fp32."""
    dims: Dims
    num_pages: int
    c_kv: np.ndarray
    k_pe: np.ndarray
    positions: np.ndarray
    slots: np.ndarray
    norm_weight: np.ndarray
    eps: float
    cos_sin: np.ndarray


def fused_write_case(dims: Dims, T, *, seed=0, num_pages=None, max_pos=40000, pad_every=0,
                     c_std=1.0, k_std=1.0):
    rng = _rng(seed)
    ps = dims.page_size
    num_pages = num_pages or (T + ps - 1) // ps + 1
    slots = rng.permutation(num_pages * ps)[:T].astype(np.int64)
    if pad_every:
        slots[::pad_every] = -1
    c_kv = bf16_normal(rng, (T, dims.R), c_std)
    k_pe = bf16_normal(rng, (T, dims.Dr), k_std)
    positions = rng.integers(0, max_pos, size=T).astype(np.int64)
    w = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(dims.R)).astype(np.float32))
    return FusedWriteCase(dims=dims, num_pages=num_pages, c_kv=c_kv, k_pe=k_pe, positions=positions,
                          slots=slots, norm_weight=w, eps=1e-6, cos_sin=rope_table(max_pos, dims.Dr))


# ---------------------------------------------------------------------------
# Key lists for index-list (top-k) attention
# ---------------------------------------------------------------------------

def key_lists(seed, query_pos, context_lens_per_row, topk, *, pad_frac=0.1, invalid_frac=0.05):
    """One key list of `topk` int32 entries per query row: distinct positions
    drawn from [0, p] (p the row's query position), in random order; about
    pad_frac of the slots are -1 (unused) and invalid_frac hold positions the
    row must ignore (future positions p < t < n, or t >= n)."""
    rng = _rng(seed)
    rows = len(query_pos)
    out = np.full((rows, topk), -1, dtype=np.int32)
    for r in range(rows):
        p, n = int(query_pos[r]), int(context_lens_per_row[r])
        n_pad = int(round(pad_frac * topk))
        n_bad = int(round(invalid_frac * topk))
        n_ok = min(topk - n_pad - n_bad, p + 1)
        ok = rng.choice(p + 1, size=n_ok, replace=False) if n_ok > 0 else np.zeros(0, np.int64)
        bad = rng.integers(p + 1, n + 1000, size=n_bad)
        bad = np.setdiff1d(bad, ok)  # never a duplicate of a kept key
        vals = np.concatenate([ok, bad])
        rng.shuffle(vals)
        slots = rng.permutation(topk)[:len(vals)]
        out[r, slots] = vals
    return out

