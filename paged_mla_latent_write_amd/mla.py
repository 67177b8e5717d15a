"""Thin ctypes binding over libmla.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into pointers, sizes and strides, allocates outputs
and workspaces with torch on the tensors' device, and raises on a non-OK
status.  Importing it without a built libmla.so raises ImportError: there is
no CPU fallback.

The names follow the C ABI in include/mla.h: write_kv, decode, decode_combine,
prefill_chunk, decode_workspace_size, prefill_workspace_size.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run paged_mla_latent_write_amd.build.build() "
                      "(hipcc, gfx950).  There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
MLA_FLAG_GENERIC_KERNELS = 1
MLA_FLAG_PREFILL_ABSORBED = 2
MLA_FLAG_PREFILL_EXPANDED = 4
MLA_FLAG_FP8_MFMA = 8

EXPORTED = ("mla_write_kv", "mla_write_kv_fused", "mla_decode_workspace_size", "mla_decode", "mla_decode_write",
            "mla_decode_noalloc",
            "mla_decode_combine", "mla_prefill_workspace_size", "mla_prefill_chunk",
            "mla_sparse_workspace_size", "mla_sparse_attention",
            "mla_status_string", "mla_version")
NOALLOC_SCRATCH_BYTES = 192 << 20  # MLA_NOALLOC_SCRATCH_BYTES in include/mla.h


class MlaCacheStruct(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_rope_dim", ctypes.c_int32)]


class MlaAttnStruct(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("qk_nope_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("w_uk", ctypes.c_void_p), ("w_uv", ctypes.c_void_p),
                ("scale", ctypes.c_float), ("window", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("kernel_events", ctypes.c_void_p * 2)]


class MlaKvTransformStruct(ctypes.Structure):
    _fields_ = [("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("cos_sin", ctypes.c_void_p), ("positions", ctypes.c_void_p),
                ("max_position", ctypes.c_int32), ("rope_interleaved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_CP = ctypes.POINTER(MlaCacheStruct)
_AP = ctypes.POINTER(MlaAttnStruct)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_write_kv = _sig("mla_write_kv", _I32, _CP, _I32, _P, _I64, _P, _I64, _P, _I32, _P)
_write_kv_fused = _sig("mla_write_kv_fused", _I32, _CP, _I32, _P, _I64, _P, _I64,
                       ctypes.POINTER(MlaKvTransformStruct), _P, _I32, _P)
_decode_ws = _sig("mla_decode_workspace_size", _SZ, _CP, _AP, _I32, _I32)
_decode = _sig("mla_decode", _I32, _CP, _I32, _AP, _P, _I64, _I64, _P, _I64, _I64, _P, _I32, _P,
               _I32, _P, _P, _P, _SZ, _P)
_decode_write = _sig("mla_decode_write", _I32, _CP, _I32, _AP, _P, _I64, _P, _I64, _P, _I32, _P, _I64, _I64,
                     _P, _I64, _I64, _P, _I32, _P, _I32, _P, _P, _P, _SZ, _P)
_decode_noalloc = _sig("mla_decode_noalloc", _I32, _CP, _I32, _AP, _P, _I64, _I64, _P, _I64, _I64, _P,
                      _I32, _P, _I32, _P, _P, _P)
_combine = _sig("mla_decode_combine", _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P)
_prefill_ws = _sig("mla_prefill_workspace_size", _SZ, _CP, _AP, _I32, _I32, _I32)
_prefill = _sig("mla_prefill_chunk", _I32, _CP, _I32, _AP, _P, _I64, _I64, _P, _I64, _I64, _P, _I32,
                _I32, _P, _I32, _P, _I32, _P, _P, _P, _SZ, _P)
_sparse_ws = _sig("mla_sparse_workspace_size", _SZ, _CP, _AP, _I32, _I32, _I32, _I32)
_sparse = _sig("mla_sparse_attention", _I32, _CP, _I32, _AP, _P, _I64, _I64, _P, _I64, _I64, _P, _I32,
               _P, _I32, _I32, _P, _I32, _P, _I32, _P, _P, _P, _SZ, _P)
_status_string = _sig("mla_status_string", ctypes.c_char_p, _I32)
_version = _sig("mla_version", ctypes.c_char_p)


class MlaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_status_string(status).decode()}")


def _check(status, where):
    if status != MLA_OK:
        raise MlaError(status, where)


def version() -> str:
    return _version().decode()


def status_string(status: int) -> str:
    return _status_string(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _keep_alive_on(stream, *tensors):
    """Tensors this module allocated are used by kernels queued on `stream`.
    When that is not the current stream, tell torch's caching allocator, so
    their memory is not handed to other work before those kernels finish.  A
    raw stream handle cannot be recorded: then every buffer must come from the
    caller."""
    if stream is None:
        return
    if not isinstance(stream, torch.cuda.Stream):
        if tensors:
            raise ValueError("with a raw stream handle, pass out, lse and workspace explicitly")
        return
    if stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    _need(len(devs) <= 1, f"tensors on different devices: {sorted(str(d) for d in devs)}")


@dataclass
class KVCache:
    """Caller-owned latent cache: data [L, P, ps, R + Dr] (bfloat16, or uint8
    E4M3 codes) and, for fp8, scale [L, P, ps] float32."""
    data: torch.Tensor
    scale: torch.Tensor | None
    kv_lora_rank: int
    qk_rope_dim: int

    @classmethod
    def empty(cls, num_layers, num_pages, page_size, kv_lora_rank, qk_rope_dim, fp8=False,
              device="cuda"):
        D = kv_lora_rank + qk_rope_dim
        if fp8:
            data = torch.empty((num_layers, num_pages, page_size, D), dtype=torch.uint8, device=device)
            scale = torch.empty((num_layers, num_pages, page_size), dtype=torch.float32, device=device)
        else:
            data = torch.empty((num_layers, num_pages, page_size, D), dtype=torch.bfloat16, device=device)
            scale = None
        return cls(data, scale, kv_lora_rank, qk_rope_dim)

    @property
    def fp8(self):
        return self.data.dtype == torch.uint8

    @property
    def page_size(self):
        return int(self.data.shape[2])

    def struct(self) -> MlaCacheStruct:
        assert self.data.is_contiguous()
        L, P, ps, D = self.data.shape
        assert D == self.kv_lora_rank + self.qk_rope_dim
        return MlaCacheStruct(self.data.data_ptr(), self.scale.data_ptr() if self.fp8 else None,
                              MLA_KV_FP8_E4M3 if self.fp8 else MLA_KV_BF16, L, P, ps,
                              self.kv_lora_rank, self.qk_rope_dim)


def _event_ptr(ev):
    return None if ev is None else ev.cuda_event


def _attn_struct(num_heads, qk_nope_dim, v_head_dim, w_uk, w_uv, scale, window, num_workgroups,
                 flags, kernel_events=None):
    for w in (w_uk, w_uv):
        assert w is None or (w.is_contiguous() and w.dtype == torch.bfloat16)
    ev = (ctypes.c_void_p * 2)(*(_event_ptr(e) for e in (kernel_events or (None, None))))
    return MlaAttnStruct(num_heads, qk_nope_dim, v_head_dim, _ptr(w_uk), _ptr(w_uv), float(scale),
                         int(window), int(num_workgroups), int(flags), ev)


def _row_strides(q):
    _need(q.dim() == 3 and q.stride(2) == 1 and q.dtype == torch.bfloat16,
          "queries must be bf16 [rows, H, D] with unit inner stride")
    return q.stride(0), q.stride(1)


def _check_heads(cache, q_nope, q_pe, w_uk, w_uv):
    """Host-known shapes of the queries and the per-head weights; returns
    (qk_nope_dim or 0, output width)."""
    R, Dr = cache.kv_lora_rank, cache.qk_rope_dim
    _need(q_nope.dim() == 3 and q_pe.dim() == 3, "q_nope and q_pe must be [rows, H, D]")
    rows, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    _need(tuple(q_pe.shape) == (rows, H, Dr), f"q_pe must be [{rows}, {H}, {Dr}], got {tuple(q_pe.shape)}")
    if w_uk is None:
        dn = 0
        _need(q_nope.shape[2] == R, f"without w_uk, q_nope must be latent: [{rows}, {H}, {R}]")
    else:
        dn = int(w_uk.shape[1])
        _need(w_uk.dim() == 3 and tuple(w_uk.shape) == (H, dn, R),
              f"w_uk must be [{H}, qk_nope_dim, {R}], got {tuple(w_uk.shape)}")
        _need(q_nope.shape[2] == dn, f"q_nope's last dim {q_nope.shape[2]} != w_uk's {dn}")
    if w_uv is None:
        dv = R
    else:
        dv = int(w_uv.shape[1])
        _need(w_uv.dim() == 3 and w_uv.shape[0] == H and w_uv.shape[2] == R,
              f"w_uv must be [{H}, v_head_dim, {R}], got {tuple(w_uv.shape)}")
    return dn, dv


def _check_tables(block_tables, context_lens, B):
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.is_contiguous(), "block_tables: contiguous int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1 and
          context_lens.is_contiguous(), "context_lens: contiguous int32 [B]")
    _need(block_tables.shape[0] == B and context_lens.numel() == B,
          f"block_tables has {block_tables.shape[0]} rows and context_lens {context_lens.numel()} "
          f"entries; the batch has {B}")
    _need(block_tables.shape[1] > 0, "block_tables needs at least one column")


def _check_outputs(out, lse, shape):
    if out is not None:
        _need(tuple(out.shape) == shape and out.dtype == torch.bfloat16 and out.is_contiguous(),
              f"out must be contiguous bf16 {shape}")
    if lse is not None:
        _need(tuple(lse.shape) == shape[:2] and lse.dtype == torch.float32 and lse.is_contiguous(),
              f"lse must be contiguous fp32 {shape[:2]}")


def _check_write(cache, c_kv, k_pe, slot_mapping):
    """mla_write_kv's host-known argument checks; returns the token count."""
    _need(c_kv.dtype == torch.bfloat16 and k_pe.dtype == torch.bfloat16, "c_kv and k_pe must be bf16")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1, "slot_mapping: int64 [T]")
    _need(c_kv.dim() == 2 and c_kv.shape[1] == cache.kv_lora_rank and c_kv.stride(-1) == 1,
          f"c_kv must be [T, {cache.kv_lora_rank}] with unit inner stride")
    _need(k_pe.dim() == 2 and k_pe.shape[1] == cache.qk_rope_dim and k_pe.stride(-1) == 1,
          f"k_pe must be [T, {cache.qk_rope_dim}] with unit inner stride")
    T = int(c_kv.shape[0])
    _need(k_pe.shape[0] == T and slot_mapping.numel() == T and slot_mapping.is_contiguous(),
          "c_kv, k_pe and slot_mapping must have the same number of tokens")
    _same_device(cache.data, c_kv, k_pe, slot_mapping)
    return T


def write_kv(cache: KVCache, layer_idx: int, c_kv: torch.Tensor, k_pe: torch.Tensor,
             slot_mapping: torch.Tensor, stream=None):
    """Scatter rows [c_kv | k_pe] (bf16 [T, R], [T, Dr], unit inner stride)
    into layer `layer_idx` at slot_mapping (int64 [T]; negative = pad row)."""
    T = _check_write(cache, c_kv, k_pe, slot_mapping)
    st = cache.struct()
    _check(_write_kv(ctypes.byref(st), layer_idx, _ptr(c_kv), c_kv.stride(0), _ptr(k_pe),
                     k_pe.stride(0), _ptr(slot_mapping), T, _stream(stream)), "mla_write_kv")


def write_kv_fused(cache: KVCache, layer_idx: int, c_kv: torch.Tensor, k_pe: torch.Tensor,
                   slot_mapping: torch.Tensor, *, positions=None, norm_weight=None, eps=1e-6,
                   cos_sin=None, interleaved=True, stream=None):
    """mla_write_kv of bf16(RMSNorm(c_kv) * norm_weight) and bf16(RoPE(k_pe)):
    c_kv the un-normalised latent bf16 [T, R], k_pe the un-rotated rope part
    bf16 [T, Dr], positions int64 [T], norm_weight bf16 [R] (None: no norm),
    cos_sin fp32 [max_position, Dr] (None: no rotation)."""
    _need(c_kv.dtype == torch.bfloat16 and k_pe.dtype == torch.bfloat16, "c_kv and k_pe must be bf16")
    _need(c_kv.dim() == 2 and c_kv.shape[1] == cache.kv_lora_rank and c_kv.stride(-1) == 1,
          f"c_kv must be [T, {cache.kv_lora_rank}] with unit inner stride")
    _need(k_pe.dim() == 2 and k_pe.shape[1] == cache.qk_rope_dim and k_pe.stride(-1) == 1,
          f"k_pe must be [T, {cache.qk_rope_dim}] with unit inner stride")
    T = int(c_kv.shape[0])
    _need(k_pe.shape[0] == T and slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T
          and slot_mapping.is_contiguous(), "c_kv, k_pe and slot_mapping (int64) must have T tokens")
    if norm_weight is not None:
        _need(norm_weight.dtype == torch.bfloat16 and norm_weight.is_contiguous() and
              norm_weight.numel() == cache.kv_lora_rank, "norm_weight: contiguous bf16 [R]")
    max_pos = 0
    if cos_sin is not None:
        _need(cos_sin.dtype == torch.float32 and cos_sin.dim() == 2 and cos_sin.is_contiguous() and
              cos_sin.shape[1] == cache.qk_rope_dim, "cos_sin: contiguous fp32 [max_position, Dr]")
        _need(positions is not None and positions.dtype == torch.int64 and positions.numel() == T and
              positions.is_contiguous(), "positions: contiguous int64 [T]")
        max_pos = int(cos_sin.shape[0])
    _same_device(cache.data, c_kv, k_pe, slot_mapping, positions, norm_weight, cos_sin)
    tf = MlaKvTransformStruct(_ptr(norm_weight), float(eps), _ptr(cos_sin), _ptr(positions), max_pos,
                              1 if interleaved else 0)
    st = cache.struct()
    _check(_write_kv_fused(ctypes.byref(st), layer_idx, _ptr(c_kv), c_kv.stride(0), _ptr(k_pe),
                           k_pe.stride(0), ctypes.byref(tf), _ptr(slot_mapping), T, _stream(stream)),
           "mla_write_kv_fused")


def decode_workspace_size(cache: KVCache, attn: MlaAttnStruct, batch: int, max_blocks: int) -> int:
    return int(_decode_ws(ctypes.byref(cache.struct()), ctypes.byref(attn), batch, max_blocks))


def prefill_workspace_size(cache: KVCache, attn: MlaAttnStruct, batch: int, total_q: int,
                           max_blocks: int) -> int:
    return int(_prefill_ws(ctypes.byref(cache.struct()), ctypes.byref(attn), batch, total_q,
                           max_blocks))


class Workspace:
    """A reusable device workspace that grows on demand (torch-allocated).
    When it is used on a stream other than the current one, pass that stream
    as a torch.cuda.Stream so the binding can record it on the buffer."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


def decode(cache: KVCache, layer_idx: int, q_nope, q_pe, block_tables, context_lens, *, scale,
           w_uk=None, w_uv=None, window=0, out=None, lse=None, want_lse=True, workspace=None,
           num_workgroups=0, flags=0, kernel_events=None, stream=None, new_tokens=None):
    """Absorbed split-KV decode.  q_nope bf16 [B, H, Dn] (or [B, H, R] latent when
    w_uk is None), q_pe bf16 [B, H, Dr]; block_tables int32 [B, max_blocks];
    context_lens int32 [B].  Returns (out bf16 [B, H, Dv or R], lse fp32 [B, H]).
    new_tokens = (c_kv, k_pe, slot_mapping), as write_kv's arguments: the
    step's tokens are written first, in the same call (mla_decode_write)."""
    B, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    dn, dv = _check_heads(cache, q_nope, q_pe, w_uk, w_uv)
    _check_tables(block_tables, context_lens, B)
    _check_outputs(out, lse, (B, H, dv))
    _same_device(cache.data, q_nope, q_pe, w_uk, w_uv, block_tables, context_lens, out, lse)
    if new_tokens is not None:
        c_kv, k_pe, slots = new_tokens
        T = _check_write(cache, c_kv, k_pe, slots)
    attn = _attn_struct(H, dn, dv, w_uk, w_uv, scale, window, num_workgroups, flags, kernel_events)
    st = cache.struct()
    max_blocks = int(block_tables.shape[1])
    dev = q_nope.device
    fresh = []
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
        fresh.append(out)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        fresh.append(lse)
    nbytes = int(_decode_ws(ctypes.byref(st), ctypes.byref(attn), B, max_blocks))
    if nbytes == 0 and B > 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_decode_workspace_size")
    ws = (workspace or Workspace()).get(nbytes, dev)
    if workspace is None:
        fresh.append(ws)
    elif isinstance(stream, torch.cuda.Stream):
        ws.record_stream(stream)
    _keep_alive_on(stream, *fresh)
    qs_b, qs_h = _row_strides(q_nope)
    ps_b, ps_h = _row_strides(q_pe)
    if new_tokens is not None:
        _check(_decode_write(ctypes.byref(st), layer_idx, ctypes.byref(attn), _ptr(c_kv), c_kv.stride(0),
                             _ptr(k_pe), k_pe.stride(0), _ptr(slots), T, _ptr(q_nope), qs_b, qs_h,
                             _ptr(q_pe), ps_b, ps_h, _ptr(block_tables), max_blocks, _ptr(context_lens), B,
                             _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "mla_decode_write")
        return out, lse
    _check(_decode(ctypes.byref(st), layer_idx, ctypes.byref(attn), _ptr(q_nope), qs_b, qs_h,
                   _ptr(q_pe), ps_b, ps_h, _ptr(block_tables), max_blocks, _ptr(context_lens), B,
                   _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "mla_decode")
    return out, lse


def decode_noalloc(cache: KVCache, layer_idx: int, q_nope, q_pe, block_tables, context_lens, *,
                   scale, out, lse=None, w_uk=None, w_uv=None, window=0, num_workgroups=0, flags=0,
                   stream=None):
    """mla_decode with the library's own device scratch array as workspace:
    no allocation anywhere, so `out` (and `lse`, if wanted) must be given.
    Calls that overlap on one GPU share the scratch array and must not be
    issued."""
    B, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    dn, dv = _check_heads(cache, q_nope, q_pe, w_uk, w_uv)
    _check_tables(block_tables, context_lens, B)
    _need(out is not None, "decode_noalloc allocates nothing: pass out")
    _check_outputs(out, lse, (B, H, dv))
    _same_device(cache.data, q_nope, q_pe, w_uk, w_uv, block_tables, context_lens, out, lse)
    attn = _attn_struct(H, dn, dv, w_uk, w_uv, scale, window, num_workgroups, flags)
    st = cache.struct()
    qs_b, qs_h = _row_strides(q_nope)
    ps_b, ps_h = _row_strides(q_pe)
    _check(_decode_noalloc(ctypes.byref(st), layer_idx, ctypes.byref(attn), _ptr(q_nope), qs_b, qs_h,
                           _ptr(q_pe), ps_b, ps_h, _ptr(block_tables), int(block_tables.shape[1]),
                           _ptr(context_lens), B, _ptr(out), _ptr(lse), _stream(stream)),
           "mla_decode_noalloc")
    return out, lse


def prefill_chunk(cache: KVCache, layer_idx: int, q_nope, q_pe, query_start_loc, max_q_len,
                  block_tables, context_lens, *, scale, w_uk=None, w_uv=None, window=0, out=None,
                  lse=None, want_lse=True, workspace=None, num_workgroups=0, flags=0,
                  kernel_events=None, stream=None):
    """Causal chunked prefill.  q_nope bf16 [Tq, H, Dn], q_pe bf16 [Tq, H, Dr];
    query_start_loc int32 [B + 1]; context_lens int32 [B] (chunk included)."""
    Tq, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    _need(context_lens.dim() == 1, "context_lens: int32 [B]")
    B = int(context_lens.shape[0])
    dn, dv = _check_heads(cache, q_nope, q_pe, w_uk, w_uv)
    _check_tables(block_tables, context_lens, B)
    _need(query_start_loc.dtype == torch.int32 and query_start_loc.dim() == 1 and
          query_start_loc.numel() == B + 1 and query_start_loc.is_contiguous(),
          "query_start_loc: contiguous int32 [B + 1]")
    _check_outputs(out, lse, (Tq, H, dv))
    _same_device(cache.data, q_nope, q_pe, w_uk, w_uv, block_tables, context_lens, query_start_loc,
                 out, lse)
    attn = _attn_struct(H, dn, dv, w_uk, w_uv, scale, window, num_workgroups, flags, kernel_events)
    st = cache.struct()
    max_blocks = int(block_tables.shape[1])
    dev = q_nope.device
    fresh = []
    if out is None:
        out = torch.empty((Tq, H, dv), dtype=torch.bfloat16, device=dev)
        fresh.append(out)
    if lse is None and want_lse:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
        fresh.append(lse)
    nbytes = int(_prefill_ws(ctypes.byref(st), ctypes.byref(attn), B, Tq, max_blocks))
    if nbytes == 0 and Tq > 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_prefill_workspace_size")
    ws = (workspace or Workspace()).get(nbytes, dev)
    if workspace is None:
        fresh.append(ws)
    elif isinstance(stream, torch.cuda.Stream):
        ws.record_stream(stream)
    _keep_alive_on(stream, *fresh)
    qs_t, qs_h = _row_strides(q_nope)
    ps_t, ps_h = _row_strides(q_pe)
    _check(_prefill(ctypes.byref(st), layer_idx, ctypes.byref(attn), _ptr(q_nope), qs_t, qs_h,
                    _ptr(q_pe), ps_t, ps_h, _ptr(query_start_loc), Tq, int(max_q_len),
                    _ptr(block_tables), max_blocks, _ptr(context_lens), B, _ptr(out), _ptr(lse),
                    _ptr(ws), ws.numel(), _stream(stream)), "mla_prefill_chunk")
    return out, lse


def sparse_attention(cache: KVCache, layer_idx: int, q_nope, q_pe, key_indices, block_tables,
                     context_lens, *, scale, query_start_loc=None, max_q_len=0, w_uk=None,
                     w_uv=None, window=0, out=None, lse=None, want_lse=True, workspace=None,
                     num_workgroups=0, flags=0, kernel_events=None, stream=None):
    """Index-list attention: query row r attends to the listed positions
    key_indices[r] (int32 [rows, topk]; -1 unused) inside its causal / window
    range.  Decode when query_start_loc is None (one row per request), else
    prefill rows as in prefill_chunk.  Returns (out, lse)."""
    rows, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    _need(context_lens.dim() == 1, "context_lens: int32 [B]")
    B = int(context_lens.shape[0])
    dn, dv = _check_heads(cache, q_nope, q_pe, w_uk, w_uv)
    _check_tables(block_tables, context_lens, B)
    _need(key_indices.dtype == torch.int32 and key_indices.dim() == 2 and key_indices.is_contiguous()
          and key_indices.shape[0] == rows and key_indices.shape[1] > 0,
          f"key_indices: contiguous int32 [{rows}, topk]")
    if query_start_loc is None:
        _need(rows == B, "decode: one query row per request")
    else:
        _need(query_start_loc.dtype == torch.int32 and query_start_loc.numel() == B + 1 and
              query_start_loc.is_contiguous(), "query_start_loc: contiguous int32 [B + 1]")
    _check_outputs(out, lse, (rows, H, dv))
    _same_device(cache.data, q_nope, q_pe, w_uk, w_uv, key_indices, block_tables, context_lens,
                 query_start_loc, out, lse)
    attn = _attn_struct(H, dn, dv, w_uk, w_uv, scale, window, num_workgroups, flags, kernel_events)
    st = cache.struct()
    topk = int(key_indices.shape[1])
    max_blocks = int(block_tables.shape[1])
    dev = q_nope.device
    fresh = []
    if out is None:
        out = torch.empty((rows, H, dv), dtype=torch.bfloat16, device=dev)
        fresh.append(out)
    if lse is None and want_lse:
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
        fresh.append(lse)
    nbytes = int(_sparse_ws(ctypes.byref(st), ctypes.byref(attn), B, rows, topk, max_blocks))
    if nbytes == 0 and rows > 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_workspace_size")
    ws = (workspace or Workspace()).get(nbytes, dev)
    if workspace is None:
        fresh.append(ws)
    elif isinstance(stream, torch.cuda.Stream):
        ws.record_stream(stream)
    _keep_alive_on(stream, *fresh)
    qs_t, qs_h = _row_strides(q_nope)
    ps_t, ps_h = _row_strides(q_pe)
    _check(_sparse(ctypes.byref(st), layer_idx, ctypes.byref(attn), _ptr(q_nope), qs_t, qs_h,
                   _ptr(q_pe), ps_t, ps_h, _ptr(key_indices), topk, _ptr(query_start_loc), rows,
                   int(max_q_len), _ptr(block_tables), max_blocks, _ptr(context_lens), B, _ptr(out),
                   _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "mla_sparse_attention")
    return out, lse


def decode_combine(o_part, lse_part, stream=None):
    """LSE merge: o_part fp32 [S, B, H, D], lse_part fp32 [S, B, H] -> (o [B, H, D], lse [B, H])."""
    S, B, H, D = (int(x) for x in o_part.shape)
    assert o_part.dtype == torch.float32 and lse_part.dtype == torch.float32
    assert o_part.is_contiguous() and lse_part.is_contiguous()
    o = torch.empty((B, H, D), dtype=torch.float32, device=o_part.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=o_part.device)
    _check(_combine(_ptr(o_part), _ptr(lse_part), S, B, H, D, _ptr(o), _ptr(lse), _stream(stream)),
           "mla_decode_combine")
    return o, lse
