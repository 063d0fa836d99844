"""GPU: the decode entry points captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

A serving loop replays one captured decode step per generated token instead of
launching kernels one by one.  The library allocates nothing and records no
memory fills inside these calls, so capture only has to see kernel launches on
the capturing stream.  Every replay runs with eager work and synchronisations
between replays, and is compared bit for bit with the same call made eagerly
(same sizes, so the same split and merge order), and with the oracle.
"""

import numpy as np
import pytest
import torch

import synth
from harness import assert_close, make_case, oracle_outputs
from oracle import attention as OA

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_graph_replays_match_eager(fp8):
    """pa_decode / pa_decode_fp8 captured once; each replay reads the q written into the captured buffer."""
    import paged_kv_cache_124_amd as pa
    print(f"[case] graph decode fp8={fp8}", flush=True)
    c = make_case(synth.gqa8b(), fp8=fp8)
    lib_call = pa.lib.pa_decode_fp8 if fp8 else pa.lib.pa_decode

    def make_args(out, q, ws=None, stream=None):
        if fp8:
            return pa.pa_decode_fp8_args(out, q, c.k, c.v, c.scales, c.tables_dev, c.lens_dev, c.scale,
                                         c.max_ctx, workspace=ws, stream=stream)
        return pa.pa_decode_args(out, q, c.k, c.v, c.tables_dev, c.lens_dev, c.scale, c.max_ctx, workspace=ws,
                                 stream=stream)

    q_buf = c.q.clone()
    out_buf = torch.empty_like(c.q)
    _, ws = make_args(out_buf, q_buf)  # the captured call's workspace, allocated outside the capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        args, _ = make_args(out_buf, q_buf, ws, torch.cuda.current_stream())
        assert lib_call(*args) == 0
    torch.cuda.synchronize()

    eager_out = torch.empty_like(c.q)
    for i in range(4):
        q_i = synth.randn(tuple(c.q.shape), c.q.dtype, 1.0 / np.sqrt(c.d), 9000 + i, "cuda")
        q_buf.copy_(q_i)
        out_buf.fill_(float("nan"))
        g.replay()
        # eager work between replays: the same call on its own buffers and workspace
        e_args, _ = make_args(eager_out, q_i)
        assert lib_call(*e_args) == 0
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_buf), _bits(eager_out)), f"replay {i} differs from the eager call"
        if i == 3:
            sample = [0, 17, 40, 63]
            assert_close(out_buf[sample], oracle_outputs(c, sample, q=q_i), f"graph replay fp8={fp8}")


def test_decode_step_graph_runs_a_decode_loop():
    """pa_decode_step captured once and replayed for 12 steps: the device tables and lengths advance inside the
    graph, the host block manager's slots reach it through a captured buffer written before each replay.  Every
    step's output, and the final pools, tables and lengths, equal an eager run of the same steps bit for bit."""
    import paged_kv_cache_124_amd as pa
    print("[case] graph decode_step loop", flush=True)
    steps = 12
    w = synth.gqa8b()
    lens = [43, 1, 15, 16, 300, 511, 2047, 1024] * 2  # most rows open a block within the 12 steps
    bs = w.block_size
    c = make_case(w, lens, num_blocks=sum(-(-(s + steps) // bs) for s in lens) + 64,
                  max_blocks=-(-(max(lens) + steps) // bs) + 1, seed=4242)
    n = len(lens)
    max_ctx = max(lens) + steps
    # two device states: A runs eagerly, B through the graph
    kA, vA, tA, lA = (t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev))
    kB, vB, tB, lB = (t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev))
    qB = torch.empty_like(c.q)
    knB = torch.empty((n, c.hkv, c.d), dtype=c.q.dtype, device="cuda")
    vnB = torch.empty_like(knB)
    slotsB = torch.zeros(n, dtype=torch.int32, device="cuda")
    outB = torch.empty_like(c.q)
    _, wsB = pa.pa_decode_step_args(outB, qB, knB, vnB, kB, vB, slotsB, tB, lB, c.scale, max_ctx)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # records the step; nothing runs until a replay
        args, _ = pa.pa_decode_step_args(outB, qB, knB, vnB, kB, vB, slotsB, tB, lB, c.scale, max_ctx,
                                         workspace=wsB, stream=torch.cuda.current_stream())
        assert pa.lib.pa_decode_step(*args) == 0
    torch.cuda.synchronize()
    assert torch.equal(lB, c.lens_dev)
    outA = torch.empty_like(c.q)
    seqs = list(range(n))
    for step in range(steps):
        st, slots, pairs, _ = c.bm.append_slots(seqs)
        assert st == 0 and len(pairs) == 0
        slots_t = torch.as_tensor(np.asarray(slots, dtype=np.int32), device="cuda")
        q = synth.randn(tuple(c.q.shape), c.q.dtype, w.value_scale, 7000 + step, "cuda")
        kn = synth.randn((n, c.hkv, c.d), c.q.dtype, w.value_scale, 7100 + step, "cuda")
        vn = synth.randn((n, c.hkv, c.d), c.q.dtype, w.value_scale, 7200 + step, "cuda")
        pa.pa_decode_step(outA, q, kn, vn, kA, vA, slots_t, tA, lA, c.scale, max_ctx)
        qB.copy_(q)
        knB.copy_(kn)
        vnB.copy_(vn)
        slotsB.copy_(slots_t)
        outB.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(outA), _bits(outB)), f"step {step}: replay differs from the eager step"
    for a, b, name in ((kA, kB, "K pool"), (vA, vB, "V pool"), (tA, tB, "tables"), (lA, lB, "lengths")):
        assert torch.equal(_bits(a), _bits(b)), f"{name} differ after {steps} steps"
    assert lB.cpu().numpy().tolist() == [s + steps for s in lens]
    st, tables, lens_bm = c.bm.build_batch(seqs, c.max_blocks)
    assert st == 0 and lens_bm.tolist() == lB.cpu().numpy().tolist()
    tb = tB.cpu().numpy()
    for r, s_r in enumerate(lens_bm.tolist()):  # the device rows moved exactly as the host manager's tables
        nb = -(-s_r // bs)
        assert tb[r, :nb].tolist() == tables[r, :nb].tolist()
    # the last step against the oracle over the final pool (it holds every appended token)
    k_log = kB.cpu().double().numpy()
    v_log = vB.cpu().double().numpy()
    ref = OA.paged_decode(qB.cpu().double().numpy(), k_log, v_log, tB.cpu().numpy(), lB.cpu().numpy().tolist(),
                          c.scale)
    assert_close(outB, ref, "graph step loop, last step")


@pytest.mark.parametrize("codes", ["e4m3", "int8"])
def test_decode_step_codes_graph_runs_a_decode_loop(codes):
    """pa_decode_step_fp8 / _int8 captured once and replayed for 8 steps over a cache of codes: every step's output,
    and the final codes, tables and lengths, equal an eager run of the same steps bit for bit.  Blocks a step opens
    get their scales before the step, as a caller sets them."""
    import paged_kv_cache_124_amd as pa
    print(f"[case] graph decode_step {codes} loop", flush=True)
    steps = 8
    w = synth.gqa8b()
    lens = [43, 1, 15, 16, 300, 511, 2047, 1024] * 2
    bs = w.block_size
    c = make_case(w, lens, num_blocks=sum(-(-(s + steps) // bs) for s in lens) + 64,
                  max_blocks=-(-(max(lens) + steps) // bs) + 1, seed=4343, fp8=codes == "e4m3", int8=codes == "int8")
    n = len(lens)
    max_ctx = max(lens) + steps
    args_of = pa.pa_decode_step_int8_args if codes == "int8" else pa.pa_decode_step_fp8_args
    call = pa.lib.pa_decode_step_int8 if codes == "int8" else pa.lib.pa_decode_step_fp8
    eager = pa.pa_decode_step_int8 if codes == "int8" else pa.pa_decode_step_fp8
    kA, vA, tA, lA = (t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev))
    kB, vB, tB, lB = (t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev))
    qB = torch.empty_like(c.q)
    knB = torch.empty((n, c.hkv, c.d), dtype=c.q.dtype, device="cuda")
    vnB = torch.empty_like(knB)
    slotsB = torch.zeros(n, dtype=torch.int32, device="cuda")
    outB = torch.empty_like(c.q)
    _, wsB = args_of(outB, qB, knB, vnB, kB, vB, c.scales, slotsB, tB, lB, c.scale, max_ctx)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        args, _ = args_of(outB, qB, knB, vnB, kB, vB, c.scales, slotsB, tB, lB, c.scale, max_ctx,
                          workspace=wsB, stream=torch.cuda.current_stream())
        assert call(*args) == 0
    torch.cuda.synchronize()
    outA = torch.empty_like(c.q)
    seqs = list(range(n))
    for step in range(steps):
        st, slots, pairs, _ = c.bm.append_slots(seqs)
        assert st == 0 and len(pairs) == 0
        for s in slots:  # a block the step opens carries the NaN scales of unused blocks: give it real ones
            b = int(s) // bs
            if torch.isnan(c.k_scale[b]).any():
                c.k_scale[b] = 0.0021 + 0.0001 * (b % 7)
                c.v_scale[b] = 0.0017 + 0.0001 * (b % 5)
        slots_t = torch.as_tensor(np.asarray(slots, dtype=np.int32), device="cuda")
        q = synth.randn(tuple(c.q.shape), c.q.dtype, w.value_scale, 7300 + step, "cuda")
        kn = synth.randn((n, c.hkv, c.d), c.q.dtype, 0.09, 7400 + step, "cuda")
        vn = synth.randn((n, c.hkv, c.d), c.q.dtype, 0.09, 7500 + step, "cuda")
        eager(outA, q, kn, vn, kA, vA, c.scales, slots_t, tA, lA, c.scale, max_ctx)
        qB.copy_(q)
        knB.copy_(kn)
        vnB.copy_(vn)
        slotsB.copy_(slots_t)
        outB.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(outA), _bits(outB)), f"step {step}: replay differs from the eager step"
    for a, b, name in ((kA, kB, "K codes"), (vA, vB, "V codes"), (tA, tB, "tables"), (lA, lB, "lengths")):
        assert torch.equal(a, b), f"{name} differ after {steps} steps"
    assert lB.cpu().numpy().tolist() == [s + steps for s in lens]
