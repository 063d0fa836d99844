"""Builds seeded decode workloads for the GPU parity tests and ``smoke()``.

Both sides get the same inputs from ``synth``: the product side allocates with
the C++ block manager of libpa.so and runs the HIP kernels through the C ABI;
the oracle side allocates with ``oracle.block_manager`` and evaluates
``oracle.attention`` in fp64 on the CPU.  Block tables from the two managers
must agree exactly before any attention is compared.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

import synth
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import int8 as OI
from oracle.block_manager import BlockManagerModel

# Acceptance bar for attention against the fp64 oracle (bf16 inputs, fp32 accumulation).
MAX_ABS = 1e-2
REL_L2 = 5e-3


@dataclass
class DecodeCase:
    w: synth.Workload
    lens: List[int]
    hq: int
    hkv: int
    d: int
    block_size: int
    dtype: torch.dtype
    num_blocks: int
    max_blocks: int
    bm: object                  # product block manager
    model: BlockManagerModel    # oracle block manager
    tables: np.ndarray          # int32 [N][max_blocks] from the product manager
    k: torch.Tensor             # device, [L][nb][Hkv][B][D] or [nb][Hkv][B][D]
    v: torch.Tensor
    q: torch.Tensor             # device [N][Hq][D]
    tables_dev: torch.Tensor
    lens_dev: torch.Tensor
    scale: float
    scales: Optional[torch.Tensor] = None    # FP8 or INT8 cache: float32 [nb][Hkv][2] (key, value) device scales
    codes: str = ""                          # "e4m3" or "int8" for a cache of one-byte codes

    @property
    def fp8(self):
        """The cache holds one-byte codes with scales (E4M3 or INT8)."""
        return self.scales is not None

    @property
    def k_scale(self):
        """Key scales [nb][Hkv]: a view into ``scales`` (writes go through)."""
        return self.scales[..., 0]

    @property
    def v_scale(self):
        return self.scales[..., 1]

    @property
    def max_ctx(self):
        return max(self.lens) if self.lens else 0


def poison_unused_(k, v, tables, lens, block_size, value=float("nan")):
    """Fill every block no sequence uses, and every slot past a sequence's end, with `value` (pools [nb][Hkv][B][D]).

    The oracle never reads those slots, so the device output must not depend on them.
    """
    used = torch.zeros(k.shape[0], dtype=torch.bool)
    for row, s in zip(tables, lens):
        nb = -(-int(s) // block_size)
        used[torch.as_tensor(row[:nb], dtype=torch.long)] = True
    unused = (~used).nonzero().flatten().to(k.device)
    if unused.numel():
        k.index_fill_(0, unused, value)
        v.index_fill_(0, unused, value)
    for row, s in zip(tables, lens):
        s = int(s)
        off = s % block_size
        if s > 0 and off:
            pb = int(row[(s - 1) // block_size])
            k[pb, :, off:, :] = value
            v[pb, :, off:, :] = value


def make_case(w: synth.Workload, lens: Optional[Sequence[int]] = None, *, hq=None, hkv=None, d=None,
              block_size=None, dtype=None, num_blocks=None, max_blocks=None, layers=1, poison=True,
              device="cuda", seed=None, fp8=False, int8=False) -> DecodeCase:
    """A seeded decode batch on both block managers; ``fp8`` / ``int8`` give a cache of E4M3 / INT8 codes with
    scales and bf16 q."""
    import paged_kv_cache_124_amd as pa

    hq = hq or w.hq
    hkv = hkv or w.hkv
    d = d or w.d
    bs = block_size or w.block_size
    dtype = dtype or synth.torch_dtype(w)
    seed = w.seed if seed is None else seed
    lens = list(synth.seq_lengths(w) if lens is None else lens)
    if num_blocks is None:
        num_blocks = synth.pool_blocks(dataclasses.replace(w, block_size=bs), lens)
    order = synth.pop_order(num_blocks, seed)
    bm = pa.BlockManager(num_blocks, bs, order)
    model = BlockManagerModel(num_blocks, bs, order)
    ids = [n for n, s in enumerate(lens) if s > 0]
    for n in ids:
        assert bm.add_seq(n, lens[n]) == 0
        assert model.add_seq(n, lens[n]) == 0
    need = max([-(-s // bs) for s in lens] + [1])
    max_blocks = max_blocks or need
    st, t_ids, _ = bm.build_batch(ids, max_blocks)
    mst, m_ids, _ = model.build_batch(ids, max_blocks)
    assert st == 0 and mst == 0
    assert t_ids.tolist() == m_ids, "product and oracle block tables differ"
    tables = np.zeros((len(lens), max_blocks), dtype=np.int32)
    tables[ids] = t_ids

    if fp8 or int8:
        assert layers == 1 and not (fp8 and int8)
        fill = synth.fill_int8_codes_ if int8 else synth.fill_fp8_codes_
        scales = synth.int8_scales if int8 else synth.fp8_scales
        kshape, vshape = pa.pool_shapes(num_blocks, hkv, d, bs, 1)
        k = fill(torch.empty(kshape, dtype=torch.uint8, device=device), seed * 10 + 1)
        v = fill(torch.empty(vshape, dtype=torch.uint8, device=device), seed * 10 + 2)
        sc = torch.stack([scales(num_blocks, hkv, w.value_scale, seed * 10 + 4, device),
                          scales(num_blocks, hkv, w.value_scale, seed * 10 + 5, device)], -1).contiguous()
        if poison:  # NaN (E4M3) or -128 (INT8) codes in unused blocks and tail slots, NaN scales on unused blocks
            poison_unused_(k, v, tables, lens, bs, value=0x80 if int8 else 0x7F)
            used = torch.zeros(num_blocks, dtype=torch.bool)
            for row, s in zip(tables, lens):
                used[torch.as_tensor(row[: -(-int(s) // bs)], dtype=torch.long)] = True
            sc[~used.to(device)] = float("nan")
        q = synth.randn((len(lens), hq, d), torch.bfloat16, w.value_scale, seed * 10 + 3, device)
        return DecodeCase(w, lens, hq, hkv, d, bs, torch.uint8, num_blocks, max_blocks, bm, model, tables, k, v, q,
                          torch.from_numpy(tables).to(device), torch.tensor(lens, dtype=torch.int32, device=device),
                          1.0 / math.sqrt(d), sc, "int8" if int8 else "e4m3")
    elem = torch.tensor([], dtype=dtype).element_size()
    kshape, vshape = pa.pool_shapes(num_blocks, hkv, d, bs, elem)
    if layers > 1:
        kshape, vshape = (layers,) + kshape, (layers,) + vshape
    k = torch.empty(kshape, dtype=dtype, device=device)
    v = torch.empty(vshape, dtype=dtype, device=device)
    synth.fill_randn_(k, w.value_scale, seed * 10 + 1)
    synth.fill_randn_(v, w.value_scale, seed * 10 + 2)
    if poison:
        for layer in range(layers):
            kl, vl = (k[layer], v[layer]) if layers > 1 else (k, v)
            poison_unused_(kl, vl, tables, lens, bs)
    q = synth.randn((len(lens), hq, d), dtype, w.value_scale, seed * 10 + 3, device)
    return DecodeCase(w, lens, hq, hkv, d, bs, dtype, num_blocks, max_blocks, bm, model, tables, k, v, q,
                      torch.from_numpy(tables).to(device), torch.tensor(lens, dtype=torch.int32, device=device),
                      1.0 / math.sqrt(d))


def run_decode(case: DecodeCase, layer: Optional[int] = None, q=None, out=None, lens_dev=None, tables_dev=None,
               max_ctx=None):
    import paged_kv_cache_124_amd as pa
    k = case.k if layer is None else case.k[layer]
    v = case.v if layer is None else case.v[layer]
    q = case.q if q is None else q
    out = torch.empty_like(q) if out is None else out
    tables_dev = case.tables_dev if tables_dev is None else tables_dev
    lens_dev = case.lens_dev if lens_dev is None else lens_dev
    max_ctx = case.max_ctx if max_ctx is None else max_ctx
    if case.fp8:
        dec = pa.pa_decode_int8 if case.codes == "int8" else pa.pa_decode_fp8
        dec(out, q, k, v, case.scales, tables_dev, lens_dev, case.scale, max_ctx)
    else:
        pa.pa_decode(out, q, k, v, tables_dev, lens_dev, case.scale, max_ctx)
    return out


def logical_blocks(pool: torch.Tensor, blocks: Sequence[int], is_key: bool) -> np.ndarray:
    """Read some physical blocks back and return them in the oracle's logical layout, fp32 (exact for bf16)."""
    idx = torch.as_tensor(list(blocks), dtype=torch.long, device=pool.device)
    return pool.index_select(0, idx).cpu().float().numpy()


def oracle_outputs(case: DecodeCase, seqs: Sequence[int], layer: Optional[int] = None, q=None, lens=None,
                   tables=None) -> np.ndarray:
    """fp64 oracle outputs [len(seqs)][Hq][D] for the listed sequences.

    Each sequence's blocks are read back and handed to the oracle with the
    oracle manager's block table remapped onto the compact copy.
    """
    k = case.k if layer is None else case.k[layer]
    v = case.v if layer is None else case.v[layer]
    q = (case.q if q is None else q).float().cpu().numpy().astype(np.float64)
    lens = case.lens if lens is None else lens
    if case.fp8:
        return _oracle_outputs_fp8(case, seqs, q, lens, tables)
    outs = []
    for n in seqs:
        s = int(lens[n])
        nb = -(-s // case.block_size)
        if tables is None:
            row = list(case.model.tables.get(n, []))[:nb]
        else:
            row = list(tables[n][:nb])
        kl = logical_blocks(k, row, True) if nb else np.zeros((0, case.hkv, case.block_size, case.d), np.float32)
        vl = logical_blocks(v, row, False) if nb else np.zeros((0, case.hkv, case.block_size, case.d), np.float32)
        tab = np.arange(max(nb, 1)).reshape(1, -1)
        outs.append(OA.paged_decode(q[n:n + 1], kl, vl, tab, [s], case.scale)[0])
    return np.stack(outs)


def fp8_logical(case: DecodeCase, blocks: Sequence[int]):
    """Codes (uint8, logical [n][Hkv][B][D]) and scales (float64 [n][Hkv]) of some physical blocks of an FP8 case."""
    idx = torch.as_tensor(list(blocks), dtype=torch.long, device=case.k.device)
    kc = case.k.index_select(0, idx).cpu().numpy()
    vc = case.v.index_select(0, idx).cpu().numpy()
    ks = case.k_scale.index_select(0, idx).cpu().double().numpy()
    vs = case.v_scale.index_select(0, idx).cpu().double().numpy()
    return kc, vc, ks, vs


def _oracle_outputs_fp8(case: DecodeCase, seqs, q, lens, tables) -> np.ndarray:
    outs = []
    for n in seqs:
        s = int(lens[n])
        nb = -(-s // case.block_size)
        row = list(case.model.tables.get(n, []))[:nb] if tables is None else list(tables[n][:nb])
        if nb:
            kc, vc, ks, vs = fp8_logical(case, row)
        else:
            kc = vc = np.zeros((0, case.hkv, case.block_size, case.d), np.uint8)
            ks = vs = np.zeros((0, case.hkv))
        tab = np.arange(max(nb, 1)).reshape(1, -1)
        oracle = OI if case.codes == "int8" else OF
        outs.append(oracle.paged_decode(q[n:n + 1], kc, vc, ks, vs, tab, [s], case.scale)[0])
    return np.stack(outs)


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.float().cpu().numpy().astype(np.float64)
    diff = g - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got: torch.Tensor, ref: np.ndarray, what: str, max_abs=MAX_ABS, rel_l2=REL_L2):
    assert np.all(np.isfinite(got.float().cpu().numpy())), f"{what}: non-finite output"
    ma, rl = errors(got, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs {ma:.3e} rel_l2 {rl:.3e}"
    return ma, rl


def paired(k_scale: torch.Tensor, v_scale: torch.Tensor):
    """One contiguous float32 scale array [..][Hkv][2] (key, value), the layout the library reads, and views of its
    key and value halves (writes through the views land in the array)."""
    sc = torch.stack([k_scale, v_scale], -1).contiguous()
    return sc, sc[..., 0], sc[..., 1]
