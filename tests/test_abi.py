"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/fa.h, and rejects bad arguments before any HIP call.

Every call below is meant to fail validation; none may reach a launch (the
pointers are placeholders, never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from tiled_online_softmax_04_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
P = ctypes.c_void_p(0x100000)   # aligned placeholder, never dereferenced
MISALIGNED = ctypes.c_void_p(0x100008)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (python -m tiled_online_softmax_04_amd.build)")
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_fwd", "fa_fwd_fp8", "fa_fwd_partial", "fa_last_error",
                                    "fa_merge",
                                    "fa_paged_decode", "fa_paged_decode_noalloc",
                                    "fa_paged_decode_workspace_size",
                                    "fa_paged_prefill", "fa_status_string"]


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_imports_no_allocation_or_sync(lib):
    """The library allocates and frees no device or host memory and never
    synchronises (include/fa.h): its dynamic symbol table imports no HIP
    allocation, free or synchronisation routine.  This is what makes the
    tiled call's zero extra device memory hold by construction."""
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    imported = [line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()]
    hip = [s for s in imported if s.startswith("hip")]
    assert "hipLaunchKernel" in hip
    banned = re.compile(r"^hip(Ext)?(Malloc|Free|HostMalloc|HostAlloc|HostFree|MemAlloc|"
                        r"MallocManaged|MallocAsync|FreeAsync|MemPool|"
                        r"DeviceSynchronize|StreamSynchronize|EventSynchronize|Memcpy)")
    assert [s for s in hip if banned.match(s)] == []


def test_status_strings(lib):
    for code, word in [(0, "ok"), (1, "invalid"), (2, "unsupported"), (3, "workspace"), (4, "HIP")]:
        assert word in lib.fa_status_string(code).decode()


def fwd(lib, dt=2, q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, n=128, m=128, d=128, dv=128,
        scale=0.088, causal=0, seq_lens=None):
    return lib.fa_fwd(dt, q, k, v, o, B, Hq, Hkv, n, m, d, dv, scale, causal, seq_lens, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), fa.FA_ERR_INVALID),
    (dict(B=-1), fa.FA_ERR_INVALID),
    (dict(d=0), fa.FA_ERR_INVALID),
    (dict(Hkv=0), fa.FA_ERR_INVALID),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(causal=1, m=64), fa.FA_ERR_INVALID),
    (dict(seq_lens=P, m=64), fa.FA_ERR_INVALID),
    (dict(scale=0.0), fa.FA_ERR_INVALID),
    (dict(scale=-1.0), fa.FA_ERR_INVALID),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(n=1 << 24, m=1 << 24), fa.FA_ERR_INVALID),
    # one 16-bit head of 2^30 elements spans 2^31 bytes: past the 32-bit offsets
    (dict(n=1 << 23, m=1 << 23), fa.FA_ERR_INVALID),
    (dict(n=64, m=1 << 23), fa.FA_ERR_INVALID),
    (dict(dt=0, n=1 << 22, m=1 << 22), fa.FA_ERR_INVALID),
    (dict(d=96, dv=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=128, dv=64), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256, dv=256), fa.FA_ERR_UNSUPPORTED),
    (dict(q=None), fa.FA_ERR_INVALID),
    (dict(o=None), fa.FA_ERR_INVALID),
    (dict(k=None), fa.FA_ERR_INVALID),
    (dict(v=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(q=MISALIGNED), fa.FA_ERR_INVALID),
])
def test_fwd_rejects_before_launch(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_fwd_empty_work_is_ok_without_pointers(lib):
    assert fwd(lib, q=None, k=None, v=None, o=None, B=0) == fa.FA_OK
    assert fwd(lib, q=None, k=None, v=None, o=None, n=0, m=0) == fa.FA_OK
    assert lib.fa_last_error().decode() == ""


def fwd8(lib, q=P, k=P, v=P, o=P, out=2, B=1, Hq=2, Hkv=2, n=128, m=128, d=128, dv=128,
         scale=0.088, qd=0.01, kd=0.01, vd=0.01, causal=0, seq_lens=None):
    return lib.fa_fwd_fp8(q, k, v, o, out, B, Hq, Hkv, n, m, d, dv, scale, qd, kd, vd, causal,
                          seq_lens, None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=3), fa.FA_ERR_INVALID),
    (dict(B=-1), fa.FA_ERR_INVALID),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(causal=1, m=64), fa.FA_ERR_INVALID),
    (dict(seq_lens=P, m=64), fa.FA_ERR_INVALID),
    (dict(scale=0.0), fa.FA_ERR_INVALID),
    (dict(qd=0.0), fa.FA_ERR_INVALID),
    (dict(kd=-1.0), fa.FA_ERR_INVALID),
    (dict(vd=float("nan")), fa.FA_ERR_INVALID),
    (dict(vd=float("inf")), fa.FA_ERR_INVALID),
    (dict(qd=1e-30, kd=1e-30), fa.FA_ERR_INVALID),   # scale * qd * kd underflows
    (dict(d=96, dv=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=128, dv=64), fa.FA_ERR_UNSUPPORTED),
    (dict(q=None), fa.FA_ERR_INVALID),
    (dict(v=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(n=1 << 24, m=1 << 24), fa.FA_ERR_INVALID),
])
def test_fwd_fp8_rejects_before_launch(lib, kw, code):
    assert fwd8(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_fwd_fp8_empty_work_is_ok(lib):
    assert fwd8(lib, q=None, k=None, v=None, o=None, B=0) == fa.FA_OK
    # descales are checked even when there is nothing to compute
    assert fwd8(lib, q=None, k=None, v=None, o=None, B=0, vd=0.0) == fa.FA_ERR_INVALID


def dec(lib, dt=2, q=P, kc=P, vc=P, bt=P, sl=P, bs=16, S=4, Hq=8, Hkv=2, d=128, dv=128, NB=64,
        maxb=16, scale=0.088, o=P, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_paged_decode_workspace_size(S, Hq, Hkv, dv, maxb, bs) if S >= 0 else 0
    return lib.fa_paged_decode(dt, q, kc, vc, bt, sl, bs, S, Hq, Hkv, d, dv, NB, maxb, scale, o,
                               ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), fa.FA_ERR_INVALID),
    (dict(bs=0), fa.FA_ERR_INVALID),
    (dict(maxb=0), fa.FA_ERR_INVALID),
    (dict(NB=0), fa.FA_ERR_INVALID),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(Hkv=0), fa.FA_ERR_INVALID),
    (dict(S=-2), fa.FA_ERR_INVALID),
    (dict(S=70000), fa.FA_ERR_INVALID),
    (dict(NB=1 << 28, bs=16, Hkv=1, Hq=1, d=64, dv=64), fa.FA_ERR_INVALID),  # 2^32 rows
    (dict(scale=0.0), fa.FA_ERR_INVALID),
    (dict(d=80, dv=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(maxb=1 << 26), fa.FA_ERR_UNSUPPORTED),  # 2^30 keys: over 65535 splits
    (dict(bt=None), fa.FA_ERR_INVALID),
    (dict(sl=None), fa.FA_ERR_INVALID),
    (dict(kc=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
])
def test_decode_rejects_before_launch(lib, kw, code):
    assert dec(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def dec_noalloc(lib, dt=2, q=P, kc=P, vc=P, bt=P, sl=P, bs=16, S=4, Hq=8, Hkv=2, d=128, dv=128,
                NB=64, maxb=16, scale=0.088, o=P):
    return lib.fa_paged_decode_noalloc(dt, q, kc, vc, bt, sl, bs, S, Hq, Hkv, d, dv, NB, maxb,
                                       scale, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), fa.FA_ERR_INVALID),
    (dict(bs=0), fa.FA_ERR_INVALID),
    (dict(NB=0), fa.FA_ERR_INVALID),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(d=80, dv=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(o=None), fa.FA_ERR_INVALID),
    (dict(vc=MISALIGNED), fa.FA_ERR_INVALID),
    # split states beyond the static scratch (545 MB for these sizes)
    (dict(S=256, Hq=64, Hkv=8, maxb=2048), fa.FA_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects_before_launch(lib, kw, code):
    assert dec_noalloc(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_decode_noalloc_empty_work_is_ok(lib):
    assert dec_noalloc(lib, q=None, kc=None, vc=None, bt=None, sl=None, o=None, S=0) == fa.FA_OK


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES


def test_decode_workspace_size(lib):
    # 64 sequences x 32 query heads, up to 512 blocks of 16 keys: 768-key splits
    # -> 11 splits, each holding m, l and o[128] in float32
    assert lib.fa_paged_decode_workspace_size(64, 32, 8, 128, 512, 16) == 64 * 32 * 11 * (8 + 512)
    assert lib.fa_paged_decode_workspace_size(64, 32, 8, 128, 0, 16) == 0
    assert lib.fa_paged_decode_workspace_size(64, 32, 0, 128, 512, 16) == 0
    # a lone sequence gets smaller splits so the GPU still fills
    one = lib.fa_paged_decode_workspace_size(1, 32, 8, 128, 512, 16)
    assert one > 32 * 11 * (8 + 512)


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
    q3 = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    cache = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16)
    table = torch.zeros(2, 2, dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.paged_decode(q3, cache, cache, table, lens, 16)
    with pytest.raises(ValueError):
        fa.paged_prefill(q3[:, :, None], cache, cache, table, lens, 16)


def partial(lib, dt=2, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, n=128, m=128, d=128, dv=128,
            scale=0.088, causal=0, seq_lens=None, kb=0, ke=128):
    return lib.fa_fwd_partial(dt, q, k, v, o, lse, B, Hq, Hkv, n, m, d, dv, scale, causal,
                              seq_lens, kb, ke, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kb=-1), fa.FA_ERR_INVALID),
    (dict(kb=10, ke=9), fa.FA_ERR_INVALID),
    (dict(ke=129), fa.FA_ERR_INVALID),
    (dict(lse=None), fa.FA_ERR_INVALID),
    (dict(lse=ctypes.c_void_p(0x100002)), fa.FA_ERR_INVALID),
    (dict(o=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(dt=5), fa.FA_ERR_INVALID),
    (dict(causal=1, m=64, ke=64), fa.FA_ERR_INVALID),
    (dict(d=96, dv=96), fa.FA_ERR_UNSUPPORTED),
])
def test_partial_rejects_before_launch(lib, kw, code):
    assert partial(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_partial_empty_work_is_ok(lib):
    assert partial(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == fa.FA_OK


def merge(lib, dt=2, op=P, lp=P, parts=2, rows=64, dv=128, o=P, lse_out=None):
    return lib.fa_merge(dt, op, lp, parts, rows, dv, o, lse_out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), fa.FA_ERR_INVALID),
    (dict(parts=0), fa.FA_ERR_INVALID),
    (dict(rows=-1), fa.FA_ERR_INVALID),
    (dict(dv=0), fa.FA_ERR_INVALID),
    (dict(dv=63), fa.FA_ERR_UNSUPPORTED),
    (dict(dv=66), fa.FA_ERR_UNSUPPORTED),
    (dict(dv=1028), fa.FA_ERR_UNSUPPORTED),
    (dict(rows=1 << 31), fa.FA_ERR_INVALID),
    (dict(op=None), fa.FA_ERR_INVALID),
    (dict(o=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(lse_out=ctypes.c_void_p(0x100001)), fa.FA_ERR_INVALID),
])
def test_merge_rejects_before_launch(lib, kw, code):
    assert merge(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_merge_empty_rows_is_ok(lib):
    assert merge(lib, rows=0, op=None, lp=None, o=None) == fa.FA_OK


def pprefill(lib, dt=2, q=P, kc=P, vc=P, bt=P, sl=P, bs=16, S=4, Hq=8, Hkv=2, n=33, d=128, dv=128,
             NB=64, maxb=16, scale=0.088, causal=1, o=P):
    return lib.fa_paged_prefill(dt, q, kc, vc, bt, sl, bs, S, Hq, Hkv, n, d, dv, NB, maxb, scale,
                                causal, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), fa.FA_ERR_INVALID),
    (dict(n=-1), fa.FA_ERR_INVALID),
    (dict(bs=0), fa.FA_ERR_INVALID),
    (dict(NB=0), fa.FA_ERR_INVALID),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(bt=None), fa.FA_ERR_INVALID),
    (dict(o=MISALIGNED), fa.FA_ERR_INVALID),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96, dv=96), fa.FA_ERR_UNSUPPORTED),
    (dict(maxb=16385), fa.FA_ERR_UNSUPPORTED),
    (dict(n=1 << 23), fa.FA_ERR_INVALID),   # one head's chunk spans 2^31 bytes
])
def test_paged_prefill_rejects_before_launch(lib, kw, code):
    assert pprefill(lib, **kw) == code
    assert lib.fa_last_error().decode() != ""


def test_paged_prefill_empty_chunk_is_ok(lib):
    assert pprefill(lib, n=0, q=None, o=None) == fa.FA_OK
