"""Host-side checks of the C ABI that need no GPU: the library builds and loads,
it exports every function include/mla.h declares, and argument errors are
reported before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
LIB = os.path.join(ROOT, "paged_mla_latent_write_amd", "libmla.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from paged_mla_latent_write_amd.build import build
        build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_abi():
    names = declared_functions()
    for want in ("mla_write_kv", "mla_decode", "mla_decode_combine", "mla_prefill_chunk",
                 "mla_decode_workspace_size", "mla_prefill_workspace_size", "mla_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert getattr(lib, n) is not None


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_flags_match_the_header():
    from paged_mla_latent_write_amd import mla
    text = open(HEADER).read()
    for name in ("MLA_FLAG_GENERIC_KERNELS", "MLA_FLAG_PREFILL_ABSORBED", "MLA_FLAG_PREFILL_EXPANDED",
                 "MLA_FLAG_FP8_MFMA"):
        m = re.search(rf"#define {name} (\d+)u", text)
        assert m and int(m.group(1)) == getattr(mla, name), name


def test_status_strings_and_version():
    from paged_mla_latent_write_amd import mla
    assert mla.status_string(0) == "MLA_OK"
    assert mla.status_string(3) == "MLA_ERR_WORKSPACE"
    assert mla.status_string(99) == "MLA_ERR_UNKNOWN"
    assert "gfx950" in mla.version()


def _cache(mla, **kw):
    base = dict(data=0x1000, scale=None, dtype=0, num_layers=2, num_pages=8, page_size=64,
                kv_lora_rank=512, qk_rope_dim=64)
    base.update(kw)
    return mla.MlaCacheStruct(**base)


def _attn(mla, **kw):
    base = dict(num_heads=16, qk_nope_dim=128, v_head_dim=128, w_uk=0x2000, w_uv=0x3000,
                scale=0.07, window=0, num_workgroups=4, flags=0)
    kw.setdefault("kernel_events", (ctypes.c_void_p * 2)(None, None))
    base.update(kw)
    return mla.MlaAttnStruct(**base)


def test_argument_validation_without_device():
    """Every error here is found on the host before any HIP call."""
    from paged_mla_latent_write_amd import mla
    byref = ctypes.byref
    c, a = _cache(mla), _attn(mla)
    P = ctypes.c_void_p
    # write_kv
    assert mla._write_kv(None, 0, P(1), 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla._write_kv(byref(c), 2, P(1), 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla._write_kv(byref(c), 0, P(1), 512, P(1), 64, P(1), 0, None) == mla.MLA_OK
    assert mla._write_kv(byref(c), 0, None, 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla._write_kv(byref(c), 0, P(1), 100, P(1), 64, P(1), 4, None) == mla.MLA_ERR_INVALID_ARGUMENT
    bad_ps = _cache(mla, page_size=48)
    assert mla._write_kv(byref(bad_ps), 0, P(1), 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_UNSUPPORTED
    fp8_no_scale = _cache(mla, dtype=1)
    assert mla._write_kv(byref(fp8_no_scale), 0, P(1), 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_INVALID_ARGUMENT
    odd = _cache(mla, kv_lora_rank=500)
    assert mla._write_kv(byref(odd), 0, P(1), 512, P(1), 64, P(1), 4, None) == mla.MLA_ERR_UNSUPPORTED

    def dec(cache=c, attn=a, layer=0, batch=4, ws=None, ws_bytes=0, q=P(1), bt=P(1), ctx=P(1), out=P(1)):
        return mla._decode(byref(cache), layer, byref(attn), q, 128 * 16, 128, P(1), 64 * 16, 64, bt,
                           4, ctx, batch, out, None, ws, ws_bytes, None)

    assert dec(layer=-1) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(batch=0) == mla.MLA_OK
    assert dec(q=None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(bt=None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(out=None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(attn=_attn(mla, num_heads=0)) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(attn=_attn(mla, scale=float("nan"))) == mla.MLA_ERR_INVALID_ARGUMENT
    # forced workgroup count: the workspace size needs no device
    need = mla._decode_ws(byref(c), byref(a), 4, 4)
    assert need > 0
    assert dec(ws=None) == mla.MLA_ERR_WORKSPACE
    assert dec(ws=P(0x10000), ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    assert dec(ws=P(0x10001), ws_bytes=need + 1024) == mla.MLA_ERR_WORKSPACE  # misaligned
    # workspace grows with batch and with the forced workgroup count
    assert mla._decode_ws(byref(c), byref(a), 8, 4) > need
    assert mla._decode_ws(byref(c), byref(_attn(mla, num_workgroups=64)), 4, 4) > need
    # no W_UK: no q_lat region
    assert mla._decode_ws(byref(c), byref(_attn(mla, w_uk=None)), 4, 4) < need
    assert mla._decode_ws(byref(c), byref(a), -1, 4) == 0
    # prefill
    assert mla._prefill_ws(byref(c), byref(a), 2, 100, 4) > 0
    assert mla._prefill(byref(c), 0, byref(a), P(1), 1, 1, P(1), 1, 1, None, 10, 5, P(1), 4, P(1), 2,
                        P(1), None, P(0x10000), 1 << 30, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla._prefill(byref(c), 0, byref(a), P(1), 1, 1, P(1), 1, 1, P(1), -1, 5, P(1), 4, P(1), 2,
                        P(1), None, P(0x10000), 1 << 30, None) == mla.MLA_ERR_INVALID_ARGUMENT
    # decode_write: the write's errors, then the decode's, all before any launch
    def dw(batch=4, T=4, ws=None, ws_bytes=0, c_kv=P(1), c_stride=512, attn=a, layer=0):
        return mla._decode_write(byref(c), layer, byref(attn), c_kv, c_stride, P(1), 64, P(1), T, P(1),
                                 128 * 16, 128, P(1), 64 * 16, 64, P(1), 4, P(1), batch, P(1), None, ws,
                                 ws_bytes, None)

    assert dw(c_kv=None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dw(c_stride=100) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dw(layer=2) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dw(T=-1) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dw(batch=-1) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dw(batch=0, T=0) == mla.MLA_OK
    assert dw(batch=0, attn=_attn(mla, num_heads=0)) == mla.MLA_ERR_INVALID_ARGUMENT
    # valid tokens, no workspace for the decode: neither runs
    assert dw(ws=None) == mla.MLA_ERR_WORKSPACE
    assert dw(ws=P(0x10000), ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    assert dw(T=0, ws=None) == mla.MLA_ERR_WORKSPACE
    # combine
    assert mla._combine(P(1), P(1), 2, 0, 4, 8, P(1), P(1), None) == mla.MLA_OK
    assert mla._combine(None, P(1), 2, 1, 4, 8, P(1), P(1), None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla._combine(P(1), P(1), -1, 1, 4, 8, P(1), P(1), None) == mla.MLA_ERR_INVALID_ARGUMENT


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU only; asking for more exits with a message
    (before anything touches a GPU)."""
    import json
    import subprocess
    import sys
    from pathlib import Path

    bench = Path(__file__).resolve().parents[1] / "bench.py"
    r = subprocess.run([sys.executable, str(bench), "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_bench_write_bytes_per_token():
    """The write workload's roofline counts, per token at the MLA shape, the
    bf16 latent and rope rows read (2 x 576 B), its int64 slot and position
    (16 B) and the cache row written: 1152 B of bf16, or 576 codes and a 4-byte
    scale."""
    import importlib.util
    from pathlib import Path

    from paged_mla_latent_write_amd import workloads as W

    spec = importlib.util.spec_from_file_location("bench_mod", Path(__file__).resolve().parents[1] / "bench.py")
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    d = W.MLA_DIMS_128
    assert (d.R, d.Dr) == (512, 64)
    assert bench.write_bytes_per_token(d, False) == 1152 + 16 + 1152
    assert bench.write_bytes_per_token(d, True) == 1152 + 16 + 580


def test_binding_rejects_mismatched_shapes():
    """The binding checks every host-known shape before it calls the ABI: a
    short block table or context_lens, queries whose head count or width
    disagrees with the weights or the cache, and wrong output buffers raise
    ValueError (CPU tensors: nothing reaches a device)."""
    import torch

    from paged_mla_latent_write_amd import mla

    B, H, R, Dr, Dn, Dv = 4, 8, 64, 16, 32, 32
    cache = mla.KVCache.empty(1, 16, 16, R, Dr, device="cpu")
    bf = dict(dtype=torch.bfloat16)
    q_nope, q_pe = torch.zeros(B, H, Dn, **bf), torch.zeros(B, H, Dr, **bf)
    w_uk, w_uv = torch.zeros(H, Dn, R, **bf), torch.zeros(H, Dv, R, **bf)
    bt = torch.zeros(B, 4, dtype=torch.int32)
    ctx = torch.ones(B, dtype=torch.int32)

    def dec(**kw):
        args = dict(q_nope=q_nope, q_pe=q_pe, block_tables=bt, context_lens=ctx, w_uk=w_uk, w_uv=w_uv)
        args.update(kw)
        return mla.decode(cache, 0, args.pop("q_nope"), args.pop("q_pe"), args.pop("block_tables"),
                          args.pop("context_lens"), scale=0.1, **args)

    bad = [
        dict(block_tables=bt[:3]),                                   # short block table
        dict(context_lens=ctx[:3]),                                  # short context_lens
        dict(block_tables=bt.to(torch.int64)),                       # wrong index type
        dict(q_pe=torch.zeros(B, H - 1, Dr, **bf)),                  # head count mismatch
        dict(q_pe=torch.zeros(B, H, Dr + 8, **bf)),                  # rope width != cache
        dict(w_uk=torch.zeros(H, Dn, R + 8, **bf)),                  # W_UK rank != cache
        dict(w_uk=torch.zeros(H - 2, Dn, R, **bf)),                  # W_UK heads != queries
        dict(q_nope=torch.zeros(B, H, Dn + 16, **bf)),               # q_nope width != W_UK
        dict(w_uv=torch.zeros(H, Dv, R - 8, **bf)),                  # W_UV rank != cache
        dict(w_uk=None),                                             # latent q must be [.., R]
        dict(out=torch.zeros(B, H, Dv + 1, **bf)),                   # wrong output shape
        dict(lse=torch.zeros(B, H, dtype=torch.float64)),            # wrong lse dtype
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            dec(**kw)

    qsl = torch.tensor([0, 1, 2, 3, 4], dtype=torch.int32)

    def pre(**kw):
        args = dict(q_nope=q_nope, q_pe=q_pe, qsl=qsl, block_tables=bt, context_lens=ctx)
        args.update(kw)
        return mla.prefill_chunk(cache, 0, args.pop("q_nope"), args.pop("q_pe"), args.pop("qsl"), 1,
                                 args.pop("block_tables"), args.pop("context_lens"), scale=0.1,
                                 w_uk=w_uk, w_uv=w_uv, **args)

    for kw in (dict(qsl=qsl[:4]), dict(block_tables=bt[:2]), dict(qsl=qsl.to(torch.int64))):
        with pytest.raises(ValueError):
            pre(**kw)

    slots = torch.zeros(3, dtype=torch.int64)
    for c, r, s in ((torch.zeros(3, R + 1, **bf), torch.zeros(3, Dr, **bf), slots),
                    (torch.zeros(3, R, **bf), torch.zeros(2, Dr, **bf), slots),
                    (torch.zeros(3, R, **bf), torch.zeros(3, Dr, **bf), slots[:2]),
                    (torch.zeros(3, R, **bf), torch.zeros(3, Dr, **bf), slots.to(torch.int32))):
        with pytest.raises(ValueError):
            mla.write_kv(cache, 0, c, r, s)
        with pytest.raises(ValueError):
            dec(new_tokens=(c, r, s))
