"""GPU: pa_check_batch against a plain count over the lengths and tables (integer work: exact).

A table entry names a physical block of the pool ("PagedAttention: Virtual
Memory for the KV Cache", sections 7-8): only the first ceil(S / B) entries of
a row are live.  The expected status is computed here by walking every row.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def expected_status(tables, lens, max_ctx, num_blocks, bs):
    n, maxb = tables.shape
    bad_rows, bad_entries, first_row, first_entry_row = 0, 0, -1, -1
    for r in range(n):
        s = int(lens[r])
        if s < 0 or s > max_ctx or -(-s // bs) > maxb:
            bad_rows += 1
            first_row = r if first_row < 0 else first_row
            continue
        live = tables[r, : -(-s // bs)]
        k = int(np.count_nonzero((live < 0) | (live >= num_blocks)))
        if k:
            bad_entries += k
            first_entry_row = r if first_entry_row < 0 else first_entry_row
    return [bad_rows, bad_entries, first_row, first_entry_row]


def run(tables, lens, max_ctx, num_blocks, bs, stale=None):
    import paged_kv_cache_124_amd as pa
    t = torch.from_numpy(tables).to("cuda")
    c = torch.from_numpy(lens).to("cuda")
    status = torch.full((4,), 12345, dtype=torch.int32, device="cuda") if stale is None else stale
    pa.pa_check_batch(t, c, max_ctx, num_blocks, bs, status=status)
    torch.cuda.synchronize()
    return status.cpu().tolist()


def valid_batch(n, maxb, bs, num_blocks, max_ctx, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_ctx + 1, n).astype(np.int32)
    tables = rng.integers(0, num_blocks, (n, maxb)).astype(np.int32)
    # entries past a row's live blocks may hold anything: they are never read
    for r in range(n):
        live = -(-int(lens[r]) // bs)
        tables[r, live:] = rng.integers(-(1 << 30), 1 << 30, maxb - live)
    return tables, lens


@pytest.mark.parametrize("n,maxb,bs", [(1, 1, 16), (64, 256, 16), (3072, 256, 16), (256, 512, 8), (1000, 128, 32)])
def test_valid_batches_report_nothing(n, maxb, bs):
    print(f"[case] valid n={n} maxb={maxb} bs={bs}", flush=True)
    num_blocks = 70000
    tables, lens = valid_batch(n, maxb, bs, num_blocks, maxb * bs, 11 + n)
    assert run(tables, lens, maxb * bs, num_blocks, bs) == [0, 0, -1, -1]


def test_bad_entries_and_rows_are_counted_exactly():
    print("[case] planted errors", flush=True)
    n, maxb, bs, num_blocks = 300, 64, 16, 5000
    tables, lens = valid_batch(n, maxb, bs, num_blocks, maxb * bs - 100, 5)
    lens[::7] = np.maximum(lens[::7], 40)   # rows 0, 7, ... hold at least 3 live blocks
    tables[::7, :3] = np.arange(3, dtype=np.int32)  # ... all valid before the errors below
    tables[7, 0] = -1                       # negative id
    tables[14, 2] = num_blocks              # one past the pool
    tables[14, 1] = 1 << 30
    tables[21, -(-int(lens[21]) // bs) - 1] = -5   # last live entry of row 21
    lens[100] = maxb * bs + 1               # needs one entry more than the table holds
    lens[150] = -3                          # negative length
    lens[200] = maxb * bs - 99              # over max_context_len (maxb * bs - 100), fits the table
    tables[100, 0] = -1                     # in a bad row: not counted as an entry
    want = expected_status(tables, lens, maxb * bs - 100, num_blocks, bs)
    assert want == [3, 4, 100, 7]
    assert run(tables, lens, maxb * bs - 100, num_blocks, bs) == want


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_planted_errors(seed):
    print(f"[case] random errors seed={seed}", flush=True)
    rng = np.random.default_rng(100 + seed)
    n, maxb, bs, num_blocks = 2048, 128, 16, 30000
    max_ctx = maxb * bs
    tables, lens = valid_batch(n, maxb, bs, num_blocks, max_ctx, 200 + seed)
    idx = rng.integers(0, n * maxb, 500)
    tables.reshape(-1)[idx] = rng.choice([-1, num_blocks, num_blocks + 7, -(1 << 31)], 500)
    rows = rng.integers(0, n, 20)
    lens[rows] = rng.choice([-1, max_ctx + 1, max_ctx + bs], 20)
    want = expected_status(tables, lens, max_ctx, num_blocks, bs)
    assert want[0] > 0 and want[1] > 0
    assert run(tables, lens, max_ctx, num_blocks, bs) == want


def test_empty_batch_writes_every_word():
    print("[case] empty batch", flush=True)
    tables = np.zeros((0, 4), dtype=np.int32)
    lens = np.zeros(0, dtype=np.int32)
    assert run(tables, lens, 64, 10, 16) == [0, 0, -1, -1]


def test_block_manager_tables_pass_and_a_smaller_pool_fails_them():
    """Tables the block manager builds for a seeded batch pass the check; a num_blocks below their ids flags them."""
    import synth
    from harness import make_case
    print("[case] block-manager tables", flush=True)
    c = make_case(synth.tiny())
    tables, lens = c.tables, np.asarray(c.lens, dtype=np.int32)
    assert run(tables, lens, c.max_ctx, c.num_blocks, c.block_size) == [0, 0, -1, -1]
    want = expected_status(tables, lens, c.max_ctx, 2, c.block_size)
    assert want[1] > 0
    assert run(tables, lens, c.max_ctx, 2, c.block_size) == want
