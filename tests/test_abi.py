"""CPU checks of the C ABI: the library loads, exports every declared symbol, and rejects bad arguments on the host."""

import ctypes
import os
import re

import pytest
import torch

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "pa_probe.h")
PKG = os.path.join(ROOT, "paged_kv_cache_124_amd")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import paged_kv_cache_124_amd as pa
    names = declared_functions()
    assert "pa_decode" in names and "pa_append_kv" in names and "pa_copy_blocks" in names
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(pa.lib, n)]
    assert not missing, missing


def test_probe_library_exports_its_header_and_nothing_of_the_product():
    """The read-rate probe lives in libpa_probe.so (bench only); libpa.so does not carry it."""
    import paged_kv_cache_124_amd as pa
    names = declared_functions(PROBE_HEADER)
    assert names == ["pa_read_probe"]
    probe = ctypes.CDLL(os.path.join(PKG, "libpa_probe.so"))
    assert all(hasattr(probe, n) for n in names)
    assert not hasattr(pa.lib, "pa_read_probe")
    assert not set(names) & set(declared_functions())


@pytest.mark.parametrize("name", ["libpa_host.so", "libpa_host_asan.so", "libpa_host_collide.so"])
def test_host_only_libraries_export_the_block_manager(name):
    """The host-only builds (g++, no HIP) export every pa_bm_* entry point and the status strings."""
    import subprocess
    path = os.path.join(PKG, name)
    syms = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in syms.splitlines() if ln.strip()}
    want = [n for n in declared_functions() if n.startswith("pa_bm_")] + ["pa_status_string", "pa_version"]
    assert not [n for n in want if n not in exported]
    assert "pa_decode" not in exported and not any(n.startswith("hip") for n in exported)


def test_binding_exposes_entry_points_with_the_c_names():
    import paged_kv_cache_124_amd as pa
    for n in ("pa_decode", "pa_append_kv", "pa_copy_blocks", "pa_decode_workspace_bytes"):
        assert callable(getattr(pa, n))


def test_status_strings_and_version():
    import paged_kv_cache_124_amd as pa
    assert pa.lib.pa_version() == 2
    assert pa.lib.pa_status_string(0) == b"ok"
    assert pa.lib.pa_status_string(3) == b"no free blocks in the pool"
    assert pa.lib.pa_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails or returns before a launch
NUL = ctypes.c_void_p(0)


def _decode(**kw):
    import paged_kv_cache_124_amd as pa
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, n=4, hq=32, hkv=8, d=128, bs=16, scale=0.1,
             maxb=256, maxctx=4096, nb=1000, dtype=pa.PA_BF16, ws=FAKE, wsb=1 << 30, stream=NUL)
    a.update(kw)
    return pa.lib.pa_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["n"], a["hq"], a["hkv"], a["d"],
                            a["bs"], a["scale"], a["maxb"], a["maxctx"], a["nb"], a["dtype"], a["ws"], a["wsb"],
                            a["stream"])


def test_decode_host_validation():
    import paged_kv_cache_124_amd as pa
    assert _decode(n=0) == pa.PA_OK                       # empty batch: nothing enqueued
    assert _decode(hq=30) == 1                            # Hq % Hkv != 0
    assert _decode(d=96) == 2                             # unsupported head size
    assert _decode(bs=64) == 2                            # unsupported block size
    assert _decode(dtype=5) == 1
    assert _decode(maxb=10) == 1                          # table too short for max_context_len
    assert _decode(q=NUL) == 1
    assert _decode(ws=NUL) == 6                           # split needs a workspace
    need = pa.pa_decode_workspace_bytes(4, 32, 8, 128, 16, 4096, pa.PA_BF16)
    assert need > 0 and _decode(wsb=need - 4) == 6


def test_workspace_and_partition_plan():
    import paged_kv_cache_124_amd as pa
    # bf16, G <= 16: balanced persistent kernel, no fixed partition; workspace holds the
    # tile prefix sums and summary records, independent of the context length bound
    for n, ctx, bs in ((64, 4096, 16), (16, 32768, 16), (256, 4096, 8), (256, 4096, 32)):
        assert pa.pa_decode_partition_tokens(n, 32, 8, 128, bs, ctx, pa.PA_BF16) == 0
        ws = pa.pa_decode_workspace_bytes(n, 32, 8, 128, bs, ctx, pa.PA_BF16)
        assert ws >= (n + 1) * 4 and ws % 4 == 0
        assert ws == pa.pa_decode_workspace_bytes(n, 32, 8, 128, bs, 2 * ctx, pa.PA_BF16)
    # fp32: partitioned kernel; one partition covers a short context: no workspace
    part = pa.pa_decode_partition_tokens(1, 8, 2, 64, 16, 100, pa.PA_F32)
    assert part > 0 and pa.pa_decode_workspace_bytes(1, 8, 2, 64, 16, 100, pa.PA_F32) == 0
    # long contexts: N * Hq * P * (D + 2) floats
    for n, ctx in ((4, 1000), (3, 4096)):
        part = pa.pa_decode_partition_tokens(n, 8, 2, 64, 16, ctx, pa.PA_F32)
        p = -(-ctx // part)
        assert pa.pa_decode_workspace_bytes(n, 8, 2, 64, 16, ctx, pa.PA_F32) == n * 8 * p * 66 * 4


def test_append_and_copy_host_validation():
    import paged_kv_cache_124_amd as pa
    L = pa.lib
    assert L.pa_append_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 100, pa.PA_BF16, NUL) == 0
    assert L.pa_append_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 100, 16, 100, pa.PA_BF16, NUL) == 2
    assert L.pa_append_kv(FAKE, FAKE, FAKE, FAKE, NUL, 4, 8, 128, 16, 100, pa.PA_BF16, NUL) == 1
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 0, 8, 128, 16, 100, 1, 0, pa.PA_BF16, NUL) == 0
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 2, 8, 128, 16, 100, 0, 0, pa.PA_BF16, NUL) == 1
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 2, 8, 128, 16, 100, 2, 5, pa.PA_BF16, NUL) == 1  # stride < layer
    assert L.pa_copy_blocks(FAKE, FAKE, NUL, 2, 8, 128, 16, 100, 1, 0, pa.PA_BF16, NUL) == 1


def test_python_binding_rejects_host_tensors():
    import paged_kv_cache_124_amd as pa
    kshape, vshape = pa.pool_shapes(4, 2, 64, 16, 4)
    k = torch.zeros(kshape)
    v = torch.zeros(vshape)
    q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError):
        pa.pa_decode(torch.zeros_like(q), q, k, v, torch.zeros(1, 4, dtype=torch.int32),
                     torch.zeros(1, dtype=torch.int32), 0.125, 64)


def test_pool_shapes_follow_the_header_layout():
    """K and V pools are [num_blocks][Hkv][B][D] for every element type: element d of the token in slot `off` of
    block `pb`, KV head j, is pool[((pb * Hkv + j) * B + off) * D + d], the formula include/pa.h gives."""
    import paged_kv_cache_124_amd as pa
    nb, hkv, bs, d = 3, 2, 8, 16
    for elem in (4, 2, 1):
        ks, vs = pa.pool_shapes(nb, hkv, d, bs, elem)
        assert ks == vs == (nb, hkv, bs, d)
    log = torch.arange(nb * hkv * bs * d, dtype=torch.float32).reshape(nb, hkv, bs, d)
    flat = log.flatten()
    for pb, j, off, dd in ((0, 0, 0, 0), (2, 1, 7, 15), (1, 0, 3, 9), (2, 0, 5, 4)):
        assert flat[((pb * hkv + j) * bs + off) * d + dd] == log[pb, j, off, dd]
    text = open(HEADER).read()
    assert "k_pool[((pb * Hkv + j) * B + off) * D + d]" in text and "v_pool[((pb * Hkv + j) * B + off) * D + d]" in text


def test_fp8_host_validation():
    import paged_kv_cache_124_amd as pa
    L = pa.lib
    # pa_decode_fp8(out, q, k, v, scales, tables, lens, n, Hq, Hkv, d, B, scale, maxb, maxctx, nb, ws, wsb, stream)
    need = pa.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 4096, pa.PA_FP8_E4M3)
    assert need > 0 and need == pa.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 8192, pa.PA_FP8_E4M3)
    assert pa.pa_decode_partition_tokens(64, 32, 8, 128, 16, 4096, pa.PA_FP8_E4M3) == 0

    def dec(n=4, hq=32, hkv=8, d=128, bs=16, sc=FAKE, ws=FAKE, wsb=None, fn=L.pa_decode_fp8):
        wsb = need if wsb is None else wsb
        return fn(FAKE, FAKE, FAKE, FAKE, sc, FAKE, FAKE, n, hq, hkv, d, bs, 0.088, 256, 4096, 1000, ws, wsb, NUL)
    for fn in (L.pa_decode_fp8, L.pa_decode_int8):
        assert dec(n=0, fn=fn) == 0
        assert dec(hq=30, fn=fn) == 1
        assert dec(hq=64, hkv=2, fn=fn) == 2        # 32 query heads per KV head: not served
        assert dec(d=96, fn=fn) == 2 and dec(bs=64, fn=fn) == 2
        assert dec(sc=NUL, fn=fn) == 1
        assert dec(sc=ctypes.c_void_p(0x1004), fn=fn) == 1   # (key, value) pairs are read 8 bytes at a time
        assert dec(ws=NUL, fn=fn) == 6 and dec(wsb=16, fn=fn) == 6
    # pa_append_kv_fp8(k, v, scales, k_new, v_new, slots, T, Hkv, d, B, nb, stream)
    for fn in (L.pa_append_kv_fp8, L.pa_append_kv_int8):
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 100, NUL) == 0
        assert fn(FAKE, FAKE, NUL, FAKE, FAKE, FAKE, 4, 8, 128, 16, 100, NUL) == 1
        assert fn(FAKE, FAKE, ctypes.c_void_p(0x1004), FAKE, FAKE, FAKE, 4, 8, 128, 16, 100, NUL) == 1
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 16, 100, NUL) == 2
    # pa_copy_blocks_fp8(k, v, scales, pairs, P, Hkv, d, B, nb, layers, stride, scale_stride, stream)
    for fn in (L.pa_copy_blocks_fp8, L.pa_copy_blocks_int8):
        assert fn(FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 100, 1, 0, 0, NUL) == 0
        assert fn(FAKE, FAKE, NUL, FAKE, 2, 8, 128, 16, 100, 1, 0, 0, NUL) == 1
        full = 100 * 8 * 128 * 16
        assert fn(FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 100, 2, full, 100 * 8, NUL) == 1   # scale stride < nb*Hkv*2
    # pa_swap_blocks_fp8(dk, dv, dsc, sk, sv, ssc, pairs, P, Hkv, d, B, src_nb, dst_nb, layers, 4 strides, stream)
    for fn in (L.pa_swap_blocks_fp8, L.pa_swap_blocks_int8):
        assert fn(FAKE, FAKE, NUL, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 10, 10, 1, 0, 0, 0, 0, NUL) == 1
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 10, 10, 1, 0, 0, 0, 0, NUL) == 0


def test_fp8_binding_takes_one_interleaved_scale_array():
    """The code-cache bindings take scales as one contiguous float32 [nb][Hkv][2] array (key, value)."""
    import paged_kv_cache_124_amd as pa
    kshape, vshape = pa.pool_shapes(4, 2, 64, 16, 1)
    k = torch.zeros(kshape, dtype=torch.uint8)
    v = torch.zeros(vshape, dtype=torch.uint8)
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    tables = torch.zeros(1, 4, dtype=torch.int32)
    lens = torch.zeros(1, dtype=torch.int32)
    for bad in (torch.zeros(4, 2), torch.zeros(4, 2, 2).transpose(1, 2).contiguous().transpose(1, 2),
                torch.zeros(4, 2, 2, dtype=torch.float64)):
        with pytest.raises(ValueError):
            pa.pa_decode_fp8(torch.zeros_like(q), q, k, v, bad, tables, lens, 0.125, 64)


def test_check_batch_host_validation():
    """pa_check_batch(tables, lens, n, max_blocks, max_ctx, num_blocks, B, status, stream): bad sizes and NULL
    pointers are refused before any launch."""
    import paged_kv_cache_124_amd as pa
    L = pa.lib
    assert L.pa_check_batch(FAKE, FAKE, -1, 4, 64, 10, 16, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, FAKE, 4, 0, 64, 10, 16, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, FAKE, 4, 4, -1, 10, 16, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, FAKE, 4, 4, 64, -1, 16, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, FAKE, 4, 4, 64, 10, 0, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, FAKE, 4, 4, 64, 10, 16, NUL, NUL) == 1
    assert L.pa_check_batch(NUL, FAKE, 4, 4, 64, 10, 16, FAKE, NUL) == 1
    assert L.pa_check_batch(FAKE, NUL, 4, 4, 64, 10, 16, FAKE, NUL) == 1


def test_check_pairs_host_validation():
    """pa_check_pairs(pairs, P, num_blocks, status, stream): bad sizes and NULL pointers refused before any launch;
    pools beyond the two LDS bitmaps (524288 blocks) are unsupported."""
    import paged_kv_cache_124_amd as pa
    L = pa.lib
    assert L.pa_check_pairs(FAKE, -1, 10, FAKE, NUL) == 1
    assert L.pa_check_pairs(FAKE, 1, -1, FAKE, NUL) == 1
    assert L.pa_check_pairs(NUL, 1, 10, FAKE, NUL) == 1
    assert L.pa_check_pairs(FAKE, 1, 10, NUL, NUL) == 1
    assert L.pa_check_pairs(FAKE, 1, (1 << 19) + 1, FAKE, NUL) == 2
