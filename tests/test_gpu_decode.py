"""GPU: pa_decode against the fp64 oracle on the five workloads and the edge cases."""

import numpy as np
import pytest
import torch

import synth
from harness import assert_close, fp8_logical, make_case, oracle_outputs, run_decode
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import int8 as OI

pytestmark = pytest.mark.gpu


def test_tiny_decode_append_decode():
    """fp32, lengths {17, 33, 64, 100}: decode, append one token per sequence (64 -> 65 opens a block), decode.

    The oracle side keeps its own pool: a snapshot taken before the device
    append, updated with the oracle's append rule at the oracle manager's
    slots, decoded through the oracle manager's tables.
    """
    import paged_kv_cache_124_amd as pa
    w = synth.tiny()
    print("[case] tiny", flush=True)
    c = make_case(w)
    out = run_decode(c)
    ref = oracle_outputs(c, range(4))
    assert_close(out, ref, "tiny step 1", max_abs=1e-4, rel_l2=1e-5)

    k_or = c.k.cpu().double().numpy().copy()
    v_or = c.v.cpu().double().numpy().copy()
    st, slots, pairs, _ = c.bm.append_slots(list(range(4)))
    mst, mslots, mpairs, _ = c.model.append_slots(list(range(4)))
    assert st == mst == 0 and list(slots) == mslots and len(pairs) == len(mpairs) == 0
    kn = synth.randn((4, w.hkv, w.d), torch.float32, 1.0, 77, "cuda")
    vn = synth.randn((4, w.hkv, w.d), torch.float32, 1.0, 78, "cuda")
    pa.pa_append_kv(c.k, c.v, kn, vn, torch.tensor(slots, dtype=torch.int32, device="cuda"))
    OA.append_kv(k_or, v_or, kn.cpu().double().numpy(), vn.cpu().double().numpy(), mslots)
    # device pool after the append equals the oracle's pool, NaN slots included
    assert np.array_equal(c.k.cpu().double().numpy(), k_or, equal_nan=True)
    assert np.array_equal(c.v.cpu().double().numpy(), v_or, equal_nan=True)

    lens2 = [s + 1 for s in c.lens]
    st, tables2, l2 = c.bm.build_batch(list(range(4)), c.max_blocks + 1)
    mst, mt2, ml2 = c.model.build_batch(list(range(4)), c.max_blocks + 1)
    assert st == mst == 0 and tables2.tolist() == mt2 and l2.tolist() == ml2 == lens2
    out2 = run_decode(c, lens_dev=torch.tensor(lens2, dtype=torch.int32, device="cuda"),
                      tables_dev=torch.from_numpy(tables2).cuda(), max_ctx=max(lens2))
    ref2 = OA.paged_decode(c.q.cpu().double().numpy(), k_or, v_or, np.array(mt2), ml2, c.scale)
    assert_close(out2, ref2, "tiny step 2", max_abs=1e-4, rel_l2=1e-5)


def test_gqa8b_all_sequences():
    """8B-style GQA layer, 64 sequences of 512..4096 tokens, every output against the oracle."""
    print("[case] gqa8b", flush=True)
    c = make_case(synth.gqa8b())
    out = run_decode(c)
    ref = oracle_outputs(c, range(len(c.lens)))
    assert_close(out, ref, "gqa8b")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_block_size_sweep_every_row(bs):
    """256 sequences of 4096 - r tokens; every output against the oracle; tail waste = sum r."""
    w = synth.sweep(bs)
    print(f"[case] sweep bs={bs}", flush=True)
    c = make_case(w)
    out = run_decode(c)
    ref = oracle_outputs(c, range(len(c.lens)))
    assert_close(out, ref, f"sweep bs={bs}")
    waste = c.bm.stats()["tail_waste_slots"]
    assert waste == sum(4096 - s for s in c.lens) == c.model.stats()["tail_waste_slots"]
    del c
    torch.cuda.empty_cache()


def test_run_to_run_bit_identical():
    c = make_case(synth.gqa8b())
    a = run_decode(c)
    b = run_decode(c)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


EDGE_LENS = [0, 1, 2, 7, 8, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 1500]


@pytest.mark.parametrize("codes", ["bf16", "e4m3", "int8"])
def test_workspace_contents_do_not_matter(codes):
    """Every word of the workspace that a call reads it has written first: a second call over a workspace whose
    every byte is 0xFF (NaN as floats) gives the same bits.  Lengths from 0 to 4000 tokens put segments in one
    wave's range and across up to 8, 9 to 16 and more ranges (each merge path), next to empty rows."""
    import paged_kv_cache_124_amd as pa
    rng = np.random.default_rng(44)
    lens = [0, 1, 31, 32, 33, 2048, 4000, 12000, 24000] + [int(x) for x in rng.integers(256, 2049, size=120)]
    print(f"[case] workspace poison {codes}", flush=True)
    c = make_case(synth.gqa8b(), lens, seed=1144, fp8=codes == "e4m3", int8=codes == "int8")
    out = torch.empty_like(c.q)
    if codes != "bf16":
        make = pa.pa_decode_int8_args if codes == "int8" else pa.pa_decode_fp8_args
        args, ws = make(out, c.q, c.k, c.v, c.scales, c.tables_dev, c.lens_dev, c.scale, c.max_ctx)
        call = pa.lib.pa_decode_int8 if codes == "int8" else pa.lib.pa_decode_fp8
    else:
        args, ws = pa.pa_decode_args(out, c.q, c.k, c.v, c.tables_dev, c.lens_dev, c.scale, c.max_ctx)
        call = pa.lib.pa_decode
    assert call(*args) == 0
    torch.cuda.synchronize()
    first = out.clone()
    ws.fill_(0xFF)
    out.fill_(float("nan"))
    assert call(*args) == 0
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), out.view(torch.int16))
    assert torch.count_nonzero(out[0].float()) == 0
    assert_close(out, oracle_outputs(c, range(len(lens))), f"workspace poison {codes}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_edge_lengths(dtype, d, bs):
    """Empty, single-token, block- and partition-aligned and ragged lengths, NaN in every unused slot."""
    w = synth.gqa8b()
    print(f"[case] edge dtype={dtype} d={d} bs={bs}", flush=True)
    c = make_case(w, EDGE_LENS, d=d, block_size=bs, dtype=dtype, hq=8, hkv=2, seed=300 + d + bs)
    out = run_decode(c)
    ref = oracle_outputs(c, range(len(EDGE_LENS)))
    assert torch.count_nonzero(out[0].float()) == 0  # S = 0 gives zeros
    tol = (1e-4, 1e-5) if dtype == torch.float32 else (1e-2, 5e-3)
    assert_close(out, ref, f"edge dtype={dtype} d={d} bs={bs}", *tol)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 1), (32, 2), (64, 4), (32, 1), (64, 1)])
def test_group_sizes(hq, hkv):
    """MHA (G = 1), MQA (Hkv = 1) and other group sizes, including G > 16 (generic kernel)."""
    w = synth.gqa8b()
    print(f"[case] group hq={hq} hkv={hkv}", flush=True)
    lens = [1, 100, 600, 1300]
    c = make_case(w, lens, hq=hq, hkv=hkv, seed=500 + hq + hkv)
    out = run_decode(c)
    ref = oracle_outputs(c, range(len(lens)))
    assert_close(out, ref, f"group hq={hq} hkv={hkv}")


def test_short_lengths_with_large_launch_bound():
    """max_context_len far above the real lengths: extra partitions exit, results unchanged."""
    c = make_case(synth.gqa8b(), [5, 40, 300], seed=700)
    c.max_blocks = 4096 // 16
    tables = np.zeros((3, c.max_blocks), dtype=np.int32)
    tables[:, : c.tables.shape[1]] = c.tables
    out = run_decode(c, tables_dev=torch.from_numpy(tables).cuda(), max_ctx=4096)
    ref = oracle_outputs(c, range(3))
    assert_close(out, ref, "short lengths, launch bound 4096")


def _run_partitioned(c, part=0):
    import paged_kv_cache_124_amd as pa
    out = torch.empty_like(c.q)
    pa.pa_decode_partitioned(out, c.q, c.k, c.v, c.tables_dev, c.lens_dev, c.scale, c.max_ctx, part)
    return out


def test_partitioned_path_gqa8b_and_edges():
    """The partitioned bf16 kernel + merge (the path for very large batches), on the 8B GQA layer at every partition
    size it takes and on edge lengths."""
    import paged_kv_cache_124_amd as pa
    print("[case] partitioned gqa8b", flush=True)
    c = make_case(synth.gqa8b())
    ref = oracle_outputs(c, range(len(c.lens)))
    for part in (0, 128, 256, 512, 1024):
        assert_close(_run_partitioned(c, part), ref, f"partitioned gqa8b part={part}")
    for bs in (8, 16, 32):
        e = make_case(synth.gqa8b(), EDGE_LENS, block_size=bs, seed=800 + bs)
        out = _run_partitioned(e)
        assert torch.count_nonzero(out[0].float()) == 0
        assert_close(out, oracle_outputs(e, range(len(EDGE_LENS))), f"partitioned edges bs={bs}")
    # partition sizes outside the documented set are refused before any launch
    for bad in (64, 100, 129, 64 * 16 + 128):
        with pytest.raises(pa.PAError):
            _run_partitioned(c, bad)


def test_many_sequences_take_partitioned_path():
    """More sequences than the persistent kernel's per-launch limit (3072): the partitioned kernel serves them."""
    import paged_kv_cache_124_amd as pa
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(0, 400, size=3100)]
    print("[case] 3100 sequences", flush=True)
    c = make_case(synth.gqa8b(), lens, seed=900)
    assert pa.pa_decode_partition_tokens(len(lens), c.hq, c.hkv, c.d, c.block_size, c.max_ctx, pa.PA_BF16) > 0
    out = run_decode(c)
    sample = sorted(set(rng.choice(len(lens), size=48, replace=False).tolist()) | {0, len(lens) - 1})
    assert_close(out[sample], oracle_outputs(c, sample), "3100 sequences")
    zero = [i for i, s in enumerate(lens) if s == 0]
    assert zero and torch.count_nonzero(out[zero].float()) == 0


@pytest.mark.parametrize("dtype,hq,hkv", [(torch.bfloat16, 8, 2), (torch.float32, 8, 2), (torch.bfloat16, 32, 1)])
def test_decode_leading_tile_outside_pool_is_left_out(dtype, hq, hkv):
    """Both blocks of a row's first 32 tokens outside [0, num_blocks): their tokens are left out of the softmax, with
    no NaN from a tile that holds no token before any other (persistent bf16 kernel; fp32 token-loop kernel; the
    partitioned MFMA kernel at 32 query heads per KV head)."""
    print(f"[case] leading tile out of pool {dtype} hq={hq} hkv={hkv}", flush=True)
    c = make_case(synth.gqa8b(), [100, 70], hq=hq, hkv=hkv, dtype=dtype, seed=1760)
    tables = c.tables.copy()
    tables[0, 0] = c.num_blocks + 3
    tables[0, 1] = c.num_blocks + 9  # tokens 0..31 of row 0
    out = run_decode(c, tables_dev=torch.from_numpy(tables).cuda())
    k_log = c.k.cpu().double().numpy()
    v_log = c.v.cpu().double().numpy()
    bs = c.block_size
    keep = range(2 * bs, 100)
    K = np.stack([k_log[int(c.tables[0][t // bs]), :, t % bs] for t in keep])
    V = np.stack([v_log[int(c.tables[0][t // bs]), :, t % bs] for t in keep])
    q = c.q.float().cpu().numpy().astype(np.float64)
    assert_close(out[0:1], OA.dense_attention(q[0], K, V, c.scale)[None], f"leading tile out of pool {dtype} g={hq // hkv}")
    assert_close(out[1:2], oracle_outputs(c, [1]), f"row 1 untouched {dtype} g={hq // hkv}")


@pytest.mark.parametrize("codes", ["", "e4m3", "int8"])
def test_decode_middle_block_outside_pool_between_full_tiles(codes):
    """One block in the middle of a 1,000-token row lies outside [0, num_blocks): the tile that holds it runs the
    masked tile math, the full tiles before and after it the unmasked instance, within one wave's range (forty
    3,000-token rows give every wave several tiles).  The row attends to every other token; the other rows are
    untouched."""
    print(f"[case] middle block out of pool {codes or 'bf16'}", flush=True)
    lens = [1000] + [3000] * 40
    c = make_case(synth.gqa8b(), lens, hq=8, hkv=2, seed=1790, fp8=codes == "e4m3", int8=codes == "int8")
    bs = c.block_size
    tables = c.tables.copy()
    tables[0, 20] = c.num_blocks + 5  # tokens 20 B .. 21 B - 1 of row 0
    out = run_decode(c, tables_dev=torch.from_numpy(tables).cuda())
    keep = [t for t in range(1000) if not 20 * bs <= t < 21 * bs]
    q = c.q.float().cpu().numpy().astype(np.float64)
    if codes:
        kc, vc, ks, vs = fp8_logical(c, [int(b) for b in c.tables[0][: -(-1000 // bs)]])
        # one "block" per kept token: codes [n][Hkv][1][D] with that token's block scale
        kb = np.stack([kc[t // bs, :, t % bs][:, None, :] for t in keep])
        vb = np.stack([vc[t // bs, :, t % bs][:, None, :] for t in keep])
        ksb = np.stack([ks[t // bs] for t in keep])
        vsb = np.stack([vs[t // bs] for t in keep])
        oracle = OI if codes == "int8" else OF
        ref = oracle.paged_decode(q[0:1], kb, vb, ksb, vsb, np.arange(len(keep))[None, :], [len(keep)], c.scale)
    else:
        k_log = c.k.cpu().double().numpy()
        v_log = c.v.cpu().double().numpy()
        K = np.stack([k_log[int(c.tables[0][t // bs]), :, t % bs] for t in keep])
        V = np.stack([v_log[int(c.tables[0][t // bs]), :, t % bs] for t in keep])
        ref = OA.dense_attention(q[0], K, V, c.scale)[None]
    assert_close(out[0:1], ref, f"middle block out of pool {codes or 'bf16'}")
    assert_close(out[[1, 40]], oracle_outputs(c, [1, 40]), f"other rows untouched {codes or 'bf16'}")
