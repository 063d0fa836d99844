"""GPU: FP8 and INT8 decode against the fp64 oracle where the kernel's number ranges are stretched.

The kernel runs both products of a cache of codes as fp16 matrix-core
operations: each query row is scaled by a power of two before its fp16
conversion, P.V weighs the probabilities by value scales relative to the
largest value scale of the segment so far, and INT8 codes enter as
c + 1152 with the offset taken out per tile.  These cases push each of
those: 32K-token contexts (long accumulation), block scales spread over
2^-8 .. 2^8 (the reference rises many times along a segment), and query rows
from 2^-20 to 2^20 with a wide spread inside one row.  The oracle works in
fp64 on the values the codes and scales stand for ("PagedAttention in vLLM:
scattered memory, exact attention", sections 8 and 11: quantization changes
precision, not the attention rule).
"""

import numpy as np
import pytest
import torch

import synth
from harness import assert_close, make_case, oracle_outputs, run_decode

pytestmark = pytest.mark.gpu

CODES = ["e4m3", "int8"]


def _case(codes, lens, seed):
    return make_case(synth.gqa8b(), lens, seed=seed, fp8=codes == "e4m3", int8=codes == "int8")


@pytest.mark.parametrize("codes", CODES)
def test_long_contexts(codes):
    """Rows of 32768, 32768, 20001 and 1 tokens (Hq 32, Hkv 8, D 128, B 16)."""
    print(f"[case] {codes} long contexts", flush=True)
    lens = [32768, 32768, 20001, 1]
    c = _case(codes, lens, 3100)
    out = run_decode(c)
    assert_close(out, oracle_outputs(c, range(len(lens))), f"{codes} long contexts")


@pytest.mark.parametrize("codes", CODES)
def test_block_scales_spread_over_sixteen_octaves(codes):
    """Key and value scales of every block multiplied by 2^e, e uniform in -8 .. 8 (per block and head)."""
    print(f"[case] {codes} scale spread", flush=True)
    lens = [3000, 4096, 129, 700, 1, 2047]
    c = _case(codes, lens, 3200)
    g = torch.Generator().manual_seed(3201)
    e = torch.randint(-8, 9, tuple(c.scales.shape), generator=g).to(torch.float32)
    c.scales.mul_(torch.exp2(e).to(c.scales.device))
    out = run_decode(c)
    ref = oracle_outputs(c, range(len(lens)))
    # outputs now reach ~2^8 times the usual magnitude and bf16 output rounding alone is
    # up to 2^-9 of a value: elementwise, the usual absolute bound plus 4 half-ulps of the value
    assert_close(out, ref, f"{codes} scale spread", max_abs=float("inf"))
    err = np.abs(out.float().cpu().numpy() - ref)
    bound = 1e-2 + 2.0 ** -7 * np.abs(ref)
    assert np.all(err <= bound), f"{codes} scale spread: worst err / bound {float((err / bound).max()):.3f}"


@pytest.mark.parametrize("codes", CODES)
def test_query_rows_across_forty_octaves(codes):
    """Query rows scaled by 2^20, 2^-20 and 1, and rows whose elements span 2^-12 .. 2^12 inside the row."""
    print(f"[case] {codes} query range", flush=True)
    lens = [1500, 1500, 1500, 1500, 333]
    c = _case(codes, lens, 3300)
    q = c.q.float()
    q[0] *= 2.0 ** 20
    q[1] *= 2.0 ** -20
    g = torch.Generator().manual_seed(3301)
    spread = torch.exp2(torch.randint(-12, 13, tuple(q[3].shape), generator=g).to(torch.float32))
    q[3] = q[3] * spread.to(q.device) / 64.0
    q[4] = q[4] * spread.flip(-1).to(q.device) / 64.0
    c.q = q.to(torch.bfloat16)
    out = run_decode(c)
    # the oracle reads the bf16 queries the kernel got
    assert_close(out, oracle_outputs(c, range(len(lens))), f"{codes} query range")
