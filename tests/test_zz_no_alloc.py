"""GPU: pa_decode_step_noalloc (the step with its workspace in the library's fixed device array) against
pa_decode_step with a caller workspace, on two calls in a row -- the 8B GQA batch, then a smaller one -- and its
size limit.

Both calls run the same kernels over the same split, so outputs, pools, tables and lengths must agree bit for bit;
the outputs are also held to the oracle's tolerance.  The second call is smaller and finds the array as the first
left it: nothing in it may need clearing.
"""

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import synth
from harness import assert_close, make_case, oracle_outputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _step_inputs(c, rows, seed):
    """Slots from the block manager for `rows`, seeded new tokens and queries for those rows."""
    st, slots, pairs, _ = c.bm.append_slots(rows)
    mst, mslots, mpairs, _ = c.model.append_slots(rows)
    assert st == mst == 0 and list(slots) == mslots and len(pairs) == len(mpairs) == 0
    n = len(rows)
    kn = synth.randn((n, c.hkv, c.d), torch.bfloat16, c.w.value_scale, seed + 1, "cuda")
    vn = synth.randn((n, c.hkv, c.d), torch.bfloat16, c.w.value_scale, seed + 2, "cuda")
    q = synth.randn((n, c.hq, c.d), torch.bfloat16, c.w.value_scale, seed + 3, "cuda")
    return torch.tensor(np.asarray(slots, dtype=np.int32), device="cuda"), kn, vn, q


def test_noalloc_step_matches_the_workspace_step_twice():
    import paged_kv_cache_124_amd as pa
    print("[case] noalloc step: gqa8b batch, then 16 rows", flush=True)
    c = make_case(synth.gqa8b(), max_blocks=4096 // 16 + 4)
    n = len(c.lens)
    A = [t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev)]
    B = [t.clone() for t in (c.k, c.v, c.tables_dev, c.lens_dev)]
    lens = list(c.lens)
    for call, rows in enumerate((list(range(n)), list(range(16)))):
        slots, kn, vn, q = _step_inputs(c, rows, 4100 + 10 * call)
        m = len(rows)
        max_ctx = max(lens[i] for i in rows) + 1
        outs = []
        for kk, vv, tt, ll in (A, B):
            out = torch.full((m, c.hq, c.d), float("nan"), dtype=torch.bfloat16, device="cuda")
            t_rows, l_rows = tt[:m].contiguous(), ll[:m].contiguous()
            if kk is A[0]:
                pa.pa_decode_step(out, q, kn, vn, kk, vv, slots, t_rows, l_rows, c.scale, max_ctx)
            else:
                pa.pa_decode_step_noalloc(out, q, kn, vn, kk, vv, slots, t_rows, l_rows, c.scale, max_ctx)
            tt[:m] = t_rows
            ll[:m] = l_rows
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(_bits(outs[0]), _bits(outs[1])), f"call {call}: outputs differ"
        for a, b in zip(A, B):
            assert torch.equal(_bits(a), _bits(b)), f"call {call}: pools, tables or lengths differ"
        for i in rows:
            lens[i] += 1
        st, tables, got_lens = c.bm.build_batch(list(range(n)), c.max_blocks)
        assert st == 0 and np.array_equal(B[2].cpu().numpy(), tables) and got_lens.tolist() == lens
        ref = oracle_outputs(dataclasses.replace(c, k=B[0], v=B[1]), rows, q=q, lens=lens, tables=tables)
        assert_close(outs[1], ref, f"noalloc call {call}")


def test_noalloc_step_refuses_sizes_beyond_its_array():
    """Hq / Hkv = 8 at d_head 128 needs more than PA_NOALLOC_SCRATCH_BYTES: refused before any launch."""
    import paged_kv_cache_124_amd as pa
    need = pa.pa_decode_workspace_bytes(64, 64, 8, 128, 16, 4096, pa.PA_BF16)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 4096, pa.PA_BF16) <= pa.PA_NOALLOC_SCRATCH_BYTES
    fake, nul = ctypes.c_void_p(0x1000), ctypes.c_void_p(0)  # never dereferenced: refused on the host
    st = pa.lib.pa_decode_step_noalloc(*([fake] * 9), 64, 64, 8, 128, 16, 0.1, 256, 4096, 1000, pa.PA_BF16, nul)
    assert st == pa.PA_ERR_WORKSPACE
    st = pa.lib.pa_decode_step_noalloc(*([fake] * 9), 64, 32, 8, 128, 16, 0.1, 256, 4096, 1000, pa.PA_F32, nul)
    assert st == pa.PA_ERR_UNSUPPORTED
