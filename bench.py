#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode-step path over a batch of sequences:
  1. host block manager: one batch append (slot per sequence, copy-on-write
     pairs);
  2. the slots and pairs reach the GPU through pinned host memory that the
     kernels read directly (a ring of buffers);
  3. pa_copy_blocks (when the batch produced copy-on-write pairs);
  4. pa_decode_step: attention of every sequence over its context and its new
     token (taken from k_new / v_new), then the new token stored at its slot
     and the device-resident block tables and lengths moved forward as the
     block manager's were (decode kernel, then merge + append kernel).
The block tables and lengths are uploaded once, before the timed region, and
from then on follow the block manager through step 4.
Contexts grow by one token per step.  Inputs are resident in HBM before the
timed region starts.  `value` is the KV bytes the decode reads per step
(sum of context lengths x 2 x Hkv x d_head x 2 bytes) divided by the
wall-clock time of a step.

With --kv fp8 the cache holds FP8 (E4M3) codes with per-(block, KV head)
scales and steps 3-4 are pa_copy_blocks_fp8 (when there are pairs) and
pa_decode_step_fp8 (attention to the new tokens as codes, then the codes
stored and the rows moved forward); the KV bytes per step are then the codes (1 byte per element)
plus the 8 bytes of scales per (block, KV head) the contexts span.

With --kv int8 the cache holds INT8 codes with the same scales and layout and
the INT8 entry points (pa_copy_blocks_int8, pa_decode_step_int8) take their
places.

The default run (gqa8b, bf16) also measures the other workloads -- FP8 and
INT8 caches, the block-size sweep, the shared-prefix fork and the 32-layer
long context -- each in a child run of this script before this process
touches the GPU, and keeps their figures in its line under
"other_workloads" (--no-others skips them).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa8b] [--kv bf16|fp8|int8]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (KV read) + µs/step, 8B GQA shape"
HBM_PEAK_GBS = 8000.0
EVENT_EVERY = 10
EVENT_SPAN = 100  # steps per event pair on workloads whose steps launch nothing but the decode
RING = 512  # pinned staging buffers; the host records one event per half ring


# HBM traffic of the decode kernels, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a
# plain copy of known size; valid only while the kernel sources are those it was taken on.
TRAFFIC_FILES = {"bf16": os.path.join(ROOT, "profiles", "decode_stream_gqa8b_traffic.txt"),
                 "fp8": os.path.join(ROOT, "profiles", "decode_stream_gqa8b_fp8_traffic.txt"),
                 "int8": os.path.join(ROOT, "profiles", "decode_stream_gqa8b_int8_traffic.txt")}
KERNEL_SOURCES = ["decode_stream.hip", "decode_stream_kernel.h", "decode_stream_i8.hip", "decode_stream.h", "decode_tile.h",
                  "decode.hip", "common.h", "codes.h"]


def measured_traffic(workload_name, kv_kind="bf16"):
    """(fetched + written bytes per decode launch, algorithmic bytes of those launches), or None."""
    import hashlib
    path = TRAFFIC_FILES[kv_kind]
    if workload_name != "gqa8b" or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_124_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if kv.get("sources_sha256") != h.hexdigest():
        return None
    total = sum(float(kv[k]) for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                       "merge_fetch_bytes_per_launch", "merge_write_bytes_per_launch"))
    return total, float(kv["algorithmic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa8b",
                    choices=["gqa8b", "sweep_b8", "sweep_b16", "sweep_b32", "fork", "long"])
    ap.add_argument("--shared", action="store_true",
                    help="fork workload: decode with pa_decode_step_shared, each prompt's shared full blocks read "
                         "once per step for its samples (default: pa_decode_step)")
    ap.add_argument("--replicas", type=int, default=4,
                    help="pool copies rotated step to step so reads come from HBM, not the 256 MB Infinity Cache")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8", "int8"],
                    help="cache element type: bf16, or FP8 E4M3 / INT8 codes with per-(block, KV head) scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (known bytes) to scale HBM counters")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="run only pa_read_probe over 4 GiB: the achievable HBM read rate of this GPU")
    ap.add_argument("--no-others", action="store_true",
                    help="default run: skip the other workloads' lines (FP8, INT8, block-size sweep, fork, long)")
    return ap.parse_args()


# The other workloads, each measured by a child run of this script (its own
# process, started before this one touches the GPU) and summarised inside the
# default line under "other_workloads": name, arguments.
OTHER_WORKLOADS = [
    ("gqa8b-fp8", ["--kv", "fp8"]),
    ("gqa8b-int8", ["--kv", "int8"]),
    ("sweep_b8", ["--workload", "sweep_b8", "--steps", "50"]),
    ("sweep_b16", ["--workload", "sweep_b16", "--steps", "50"]),
    ("sweep_b32", ["--workload", "sweep_b32", "--steps", "50"]),
    ("fork-shared", ["--workload", "fork", "--shared", "--steps", "40", "--warmup", "5"]),
    ("long", ["--workload", "long", "--steps", "3", "--warmup", "1"]),
]


def summarize_line(line):
    """The figures of one bench line that the default line keeps for another workload."""
    d = json.loads(line)
    rf = d.get("roofline", {})
    return {"value": d["value"], "unit": d["unit"], "us_per_step": d["config"]["us_per_step"],
            "steps": d["steps"], "warmup": d["warmup"], "dtype": d["dtype"],
            "roofline_achieved": rf.get("achieved"), "roofline_frac": rf.get("frac"),
            "kernel_avg_us": rf.get("avg_us"), "tail_waste_slots": d["config"].get("tail_waste_slots"),
            "config": d["config"]["workload"]}


def other_workloads(timeout_s=300):
    """Run each of OTHER_WORKLOADS as a child `bench.py` and keep the figures of its line."""
    import subprocess
    rows = []
    for name, extra in OTHER_WORKLOADS:
        print(f"[bench] other workload {name}", file=sys.stderr, flush=True)
        cmd = [sys.executable, os.path.abspath(__file__), "--no-cpu-baseline", "--no-others"] + extra
        row = {"workload": name}
        try:
            cp = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s)
            lines = [ln for ln in cp.stdout.splitlines() if ln.startswith("{")]
            if cp.returncode != 0 or not lines:
                row["error"] = f"exit {cp.returncode}: {cp.stderr.strip().splitlines()[-1:] or ''}"
            else:
                row.update(summarize_line(lines[-1]))
        except subprocess.TimeoutExpired:
            row["error"] = f"no line within {timeout_s} s"
        rows.append(row)
    return rows


def workload(name):
    import synth
    if name == "gqa8b":
        return synth.gqa8b()
    if name == "fork":
        return synth.fork()
    if name == "long":
        return synth.long()
    return synth.sweep(int(name.split("_b")[1]))


class Runner:
    """Holds the resident state of one benchmark workload."""

    def __init__(self, w, steps_total, replicas, device="cuda", kv_kind="bf16", shared=False):
        import torch
        import synth
        import paged_kv_cache_124_amd as pa
        self.pa = pa
        self.torch = torch
        self.w = w
        self.fp8 = kv_kind in ("fp8", "int8")  # one-byte codes with scales
        self.int8 = kv_kind == "int8"
        self.fork = w.name == "fork"
        self.shared = shared
        bs = w.block_size
        if self.fork:
            # parallel sampling: each prompt forked into FORK_SAMPLES samples that share its blocks;
            # the first step copies the shared 7-token tails on write
            P, S = synth.FORK_PROMPTS, synth.FORK_SAMPLES
            prompt = w.fixed_lens[0]
            self.lens0 = [prompt] * (P * S)
            grown = [s + steps_total for s in self.lens0]
            extra = P * (S - 1) + P * S * (-(-grown[0] // bs) - (-(-prompt // bs)))
            self.num_blocks = synth.pool_blocks(w, list(w.fixed_lens), extra=extra)
        else:
            self.lens0 = synth.seq_lengths(w)
            grown = [s + steps_total for s in self.lens0]
            self.num_blocks = synth.pool_blocks(w, grown)
        self.n = len(self.lens0)
        self.max_blocks = max(-(-s // bs) for s in grown)
        self.max_ctx = max(grown)
        self.bm = pa.BlockManager(self.num_blocks, bs, synth.pop_order(self.num_blocks, w.seed))
        if self.fork:
            for p in range(P):
                assert self.bm.add_seq(p * S, prompt) == 0
                for j in range(1, S):
                    assert self.bm.fork(p * S, p * S + j) == 0
        else:
            for i, s in enumerate(self.lens0):
                assert self.bm.add_seq(i, s) == 0
        self.seqs = np.arange(self.n, dtype=np.int64)
        self.groups = None
        if self.shared:
            st, groups = self.bm.shared_groups(self.seqs, 32 // (w.hq // w.hkv))
            assert st == 0 and len(groups) > 0
            self.groups = torch.from_numpy(groups).to(device)
            # KV bytes a step needs once: each group's shared tokens once, every row's own tokens
            self.shared_tokens_saved = int(sum((c - 1) * p for _, c, p in groups.tolist()))
        dt = synth.torch_dtype(w)
        if self.fp8:
            kshape, vshape = pa.pool_shapes(self.num_blocks, w.hkv, w.d, bs, 1)
            fill = synth.fill_int8_codes_ if self.int8 else synth.fill_fp8_codes_
            scales = synth.int8_scales if self.int8 else synth.fp8_scales
            self.k = [fill(torch.empty(kshape, dtype=torch.uint8, device=device), w.seed * 10 + 1 + 7 * r)
                      for r in range(replicas)]
            self.v = [fill(torch.empty(vshape, dtype=torch.uint8, device=device), w.seed * 10 + 2 + 7 * r)
                      for r in range(replicas)]
            # one array [nb][Hkv][2] of (key scale, value scale) per replica
            self.sc = [torch.stack([scales(self.num_blocks, w.hkv, w.value_scale, w.seed * 10 + 8 + 7 * r, device),
                                    scales(self.num_blocks, w.hkv, w.value_scale, w.seed * 10 + 9 + 7 * r, device)],
                                   -1).contiguous() for r in range(replicas)]
        else:
            kshape, vshape = pa.pool_shapes(self.num_blocks, w.hkv, w.d, bs, torch.tensor([], dtype=dt).element_size())
            self.k = [synth.fill_randn_(torch.empty(kshape, dtype=dt, device=device), w.value_scale,
                                        w.seed * 10 + 1 + 7 * r) for r in range(replicas)]
            self.v = [synth.fill_randn_(torch.empty(vshape, dtype=dt, device=device), w.value_scale,
                                        w.seed * 10 + 2 + 7 * r) for r in range(replicas)]
        self.q = synth.randn((self.n, w.hq, w.d), dt, w.value_scale, w.seed * 10 + 3, device)
        self.k_new = synth.randn((self.n, w.hkv, w.d), dt, w.value_scale, w.seed * 10 + 4, device)
        self.v_new = synth.randn((self.n, w.hkv, w.d), dt, w.value_scale, w.seed * 10 + 5, device)
        self.out = torch.empty_like(self.q)
        if self.shared:
            ws = pa.pa_decode_shared_workspace_bytes(self.n, len(self.groups), w.hq, w.hkv, w.d, bs, self.max_ctx,
                                                     pa.PA_BF16)
        else:
            ws = pa.pa_decode_workspace_bytes(self.n, w.hq, w.hkv, w.d, bs, self.max_ctx,
                                              pa.PA_INT8 if self.int8 else pa.PA_FP8_E4M3 if self.fp8 else pa.PA_BF16)
        self.ws = torch.zeros(max(ws, 16), dtype=torch.uint8, device=device)  # zero before first use
        self.part = pa.pa_decode_partition_tokens(self.n, w.hq, w.hkv, w.d, bs, self.max_ctx, pa.PA_BF16)
        # Block tables and lengths live on the device; pa_append_step moves them forward.
        n, mb = self.n, self.max_blocks
        st, tables, lens = self.bm.build_batch(self.seqs, mb)
        assert st == 0
        self.d_tables = torch.from_numpy(tables).to(device)
        self.d_lens = torch.from_numpy(lens).to(device)
        # Host staging: a ring of RING pinned buffers [slots N | pairs 2N].  The block
        # manager writes a step's slots and copy-on-write pairs straight into one of them
        # and the kernels read them there through the buffer's device mapping, so a step
        # has no copy and no event of its own.  One event per half ring tells the host
        # when the GPU is done with a half before it is written again.  Where pinned
        # memory has no device mapping, the buffer is uploaded in-stream instead.
        import ctypes
        self.ct = ctypes
        self.words = 3 * n
        self.ring = RING
        # one pinned allocation, RING buffers of `words` int32 each (each 256-byte aligned)
        stride = -(-self.words // 64) * 64
        self.host_all = torch.empty(RING * stride, dtype=torch.int32, pin_memory=True)
        self.host = [self.host_all[b * stride:b * stride + self.words] for b in range(RING)]
        hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
        dp = ctypes.c_void_p()
        ok = hip.hipHostGetDevicePointer(ctypes.byref(dp), ctypes.c_void_p(self.host_all.data_ptr()), 0) == 0
        self.zero_copy = bool(ok and dp.value)
        self.mapped = [dp.value + 4 * b * stride if self.zero_copy else None for b in range(RING)]
        self.dev = None if self.zero_copy else [torch.empty(self.words, dtype=torch.int32, device=device)
                                                for _ in range(RING)]
        self.half_ev = [torch.cuda.Event(), torch.cuda.Event()]
        self.half_used = [False, False]
        self.replicas = replicas
        # pre-marshalled C calls per (replica, ring buffer)
        L = pa.lib
        self.lib = L
        self.seqs_p = self.seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        p32 = ctypes.POINTER(ctypes.c_int32)
        self.npairs = ctypes.c_int()
        self.append_slots_args = []
        for b in range(RING):
            base = self.host[b].data_ptr()
            self.append_slots_args.append((self.bm.handle, self.seqs_p, n, ctypes.cast(base, p32),
                                           ctypes.cast(base + 4 * n, p32), ctypes.byref(self.npairs)))
        check = torch.empty(self.words, dtype=torch.int32, device=device)  # shapes for validation only
        self.step_args, self.copy_args, self.append_args = {}, {}, {}
        for r in range(replicas):
            if self.fp8:
                cpy = pa.pa_copy_blocks_fp8_args(self.k[r], self.v[r], self.sc[r], check[n:3 * n].view(n, 2))
                step_codes_args = pa.pa_decode_step_int8_args if self.int8 else pa.pa_decode_step_fp8_args
            else:
                cpy = pa.pa_copy_blocks_args(self.k[r], self.v[r], check[n:3 * n].view(n, 2))
            for b in range(RING):
                base = self.mapped[b] if self.zero_copy else self.dev[b].data_ptr()
                pairs_at = 4 if self.fp8 else 2  # position of src_dst_pairs in the copy call
                self.copy_args[r, b] = (list(cpy[:pairs_at]) + [ctypes.c_void_p(base + 4 * n)] +
                                        list(cpy[pairs_at + 1:]))
                if self.fp8:
                    self.step_args[r, b], _ = step_codes_args(
                        self.out, self.q, self.k_new, self.v_new, self.k[r], self.v[r], self.sc[r],
                        check[:n], self.d_tables, self.d_lens, w.scale, self.max_ctx, workspace=self.ws,
                        slot_pointer=base)
                elif self.shared:
                    self.step_args[r, b], _ = pa.pa_decode_step_shared_args(
                        self.out, self.q, self.k_new, self.v_new, self.k[r], self.v[r], check[:n], self.d_tables,
                        self.d_lens, self.groups, w.scale, self.max_ctx, workspace=self.ws, slot_pointer=base)
                else:
                    self.step_args[r, b], _ = pa.pa_decode_step_args(
                        self.out, self.q, self.k_new, self.v_new, self.k[r], self.v[r], check[:n], self.d_tables,
                        self.d_lens, w.scale, self.max_ctx, workspace=self.ws, slot_pointer=base)
        self.step_i = 0
        # KV bytes the decode reads per token of context, and per (block, KV head) of it (FP8 scales)
        self.kv_bytes_per_token = 2 * w.hkv * w.d * (1 if self.fp8 else 2)
        self.scale_bytes_per_block = 2 * w.hkv * 4 if self.fp8 else 0
        self.lens = np.array(self.lens0, dtype=np.int64)
        self.host_s = 0.0

    def step(self, timing=None):
        t_host = time.perf_counter()
        L = self.lib
        k = self.step_i % self.ring
        half = RING // 2
        if k % half == 0 and self.half_used[k // half]:
            self.half_ev[k // half].synchronize()  # the GPU is done with this half of the ring
        st = L.pa_bm_append_slots(*self.append_slots_args[k])
        if st != 0:
            raise RuntimeError(f"block manager append failed: status {st}")
        npairs = self.npairs.value
        if not self.zero_copy:
            words = self.n + 2 * npairs
            self.dev[k][:words].copy_(self.host[k][:words], non_blocking=True)
        r = self.step_i % self.replicas
        if self.fp8:
            if npairs:
                ca = self.copy_args[r, k]
                ca[5] = npairs
                assert (L.pa_copy_blocks_int8 if self.int8 else L.pa_copy_blocks_fp8)(*ca) == 0
            if timing is not None and timing[0] is not None:
                timing[0].record()
            assert (L.pa_decode_step_int8 if self.int8 else L.pa_decode_step_fp8)(*self.step_args[r, k]) == 0
            if timing is not None and timing[1] is not None:
                timing[1].record()
        else:
            if npairs:
                ca = self.copy_args[r, k]
                ca[3] = npairs
                assert L.pa_copy_blocks(*ca) == 0
            if timing is not None and timing[0] is not None:
                timing[0].record()
            if self.shared:
                assert L.pa_decode_step_shared(*self.step_args[r, k]) == 0
            else:
                assert L.pa_decode_step(*self.step_args[r, k]) == 0
            if timing is not None and timing[1] is not None:
                timing[1].record()
        if k % half == half - 1:
            self.half_ev[k // half].record()
            self.half_used[k // half] = True
        self.step_i += 1
        self.lens += 1
        self.host_s += time.perf_counter() - t_host
        bs = self.w.block_size
        return int(self.lens.sum()) * self.kv_bytes_per_token + int((-(-self.lens // bs)).sum()) * self.scale_bytes_per_block

    def check_device_batch(self):
        """The device tables and lengths still equal the block manager's (after the timed steps)."""
        st, tables, lens = self.bm.build_batch(self.seqs, self.max_blocks)
        assert st == 0
        if not (np.array_equal(self.d_tables.cpu().numpy(), tables) and np.array_equal(self.d_lens.cpu().numpy(), lens)):
            raise RuntimeError("device block tables / lengths diverged from the block manager")


class LongRunner:
    """The 32-layer long-context step: 16 sequences of 32,768 tokens, 64 GiB of KV in one allocation per tensor.

    One step appends each sequence's new token in every layer (pa_append_step on layer 0 stores it and moves the
    device-resident rows forward; pa_append_kv stores it in layers 1..31 at the same slots) and then decodes every
    layer over S + 1 tokens.  The block manager's slots for all steps are computed before the timed region.
    """

    def __init__(self, w, steps_total, device="cuda"):
        import torch
        import synth
        import paged_kv_cache_124_amd as pa
        self.pa, self.w = pa, w
        self.lens0 = synth.seq_lengths(w)
        self.n = len(self.lens0)
        bs, L = w.block_size, w.layers
        extra = self.n * (steps_total // bs + 2)
        self.num_blocks = synth.pool_blocks(w, self.lens0, extra=extra)
        self.max_ctx = max(self.lens0) + steps_total
        self.max_blocks = -(-self.max_ctx // bs)
        bm = pa.BlockManager(self.num_blocks, bs, synth.pop_order(self.num_blocks, w.seed))
        self.bm = bm
        for i, s_ in enumerate(self.lens0):
            assert bm.add_seq(i, s_) == 0
        seqs = np.arange(self.n, dtype=np.int64)
        st, tables, lens = bm.build_batch(seqs, self.max_blocks)
        assert st == 0
        slots = []
        for _ in range(steps_total):
            st, sl, pairs, _ = bm.append_slots(seqs)
            assert st == 0 and len(pairs) == 0
            slots.append(sl.copy())
        self.slots = torch.from_numpy(np.stack(slots).astype(np.int32)).to(device)
        kshape, vshape = pa.pool_shapes(self.num_blocks, w.hkv, w.d, bs, 2)
        self.k = synth.fill_randn_(torch.empty((L,) + kshape, dtype=torch.bfloat16, device=device), w.value_scale,
                                   w.seed * 10 + 1)
        self.v = synth.fill_randn_(torch.empty((L,) + vshape, dtype=torch.bfloat16, device=device), w.value_scale,
                                   w.seed * 10 + 2)
        self.q = synth.randn((L, self.n, w.hq, w.d), torch.bfloat16, w.value_scale, w.seed * 10 + 3, device)
        self.kn = synth.randn((L, self.n, w.hkv, w.d), torch.bfloat16, w.value_scale, w.seed * 10 + 4, device)
        self.vn = synth.randn((L, self.n, w.hkv, w.d), torch.bfloat16, w.value_scale, w.seed * 10 + 5, device)
        self.out = torch.empty_like(self.q)
        self.d_tables = torch.from_numpy(tables).to(device)
        self.d_lens = torch.from_numpy(lens).to(device)
        ws = pa.pa_decode_workspace_bytes(self.n, w.hq, w.hkv, w.d, bs, self.max_ctx, pa.PA_BF16)
        self.ws = torch.zeros(max(ws, 16), dtype=torch.uint8, device=device)
        self.dec_args = [pa.pa_decode_args(self.out[l], self.q[l], self.k[l], self.v[l], self.d_tables, self.d_lens,
                                           w.scale, self.max_ctx, workspace=self.ws)[0] for l in range(L)]
        self.step_i = 0
        self.lens = np.array(self.lens0, dtype=np.int64)
        self.kv_bytes_per_token = 2 * w.hkv * w.d * 2 * L
        self.host_s = 0.0
        self.zero_copy = False
        self.fork = False
        self.part = pa.pa_decode_partition_tokens(self.n, w.hq, w.hkv, w.d, bs, self.max_ctx, pa.PA_BF16)

    def step(self, timing=None):
        pa, w, L = self.pa, self.w, self.w.layers
        sl = self.slots[self.step_i]
        pa.pa_append_step(self.k[0], self.v[0], self.kn[0], self.vn[0], sl, self.d_tables, self.d_lens)
        for l in range(1, L):
            pa.pa_append_kv(self.k[l], self.v[l], self.kn[l], self.vn[l], sl)
        if timing is not None:
            timing[0].record()
        for l in range(L):
            assert pa.lib.pa_decode(*self.dec_args[l]) == 0
        if timing is not None:
            timing[1].record()
        self.step_i += 1
        self.lens += 1
        return int(self.lens.sum()) * self.kv_bytes_per_token

    def check_device_batch(self):
        st, tables, lens = self.bm.build_batch(np.arange(self.n, dtype=np.int64), self.max_blocks)
        assert st == 0
        got_lens = self.d_lens.cpu().numpy()
        want = np.array(self.lens0) + self.step_i
        if not np.array_equal(got_lens, want):
            raise RuntimeError("device lengths diverged from the block manager's")


# Oracle inputs of the CPU baseline, set before the worker processes fork (they
# read them copy-on-write) and never touched by the GPU path.
_CPU_INPUTS = []
_CPU_ARGS = {}


def _oracle_over(idx):
    """The fp64 oracle over the listed sequences of _CPU_INPUTS (one BLAS thread in this process)."""
    from oracle import attention as OA
    from oracle import fp8 as OF
    from oracle import int8 as OI
    a = _CPU_ARGS
    OC = OI if a["kv"] == "int8" else OF
    for i in idx:
        q, kp, vp, ks, vs, table, s = _CPU_INPUTS[i]
        if a["codes"]:
            OC.paged_decode(q, kp, vp, ks, vs, table, [s], a["scale"])
        else:
            OA.paged_decode(q, kp, vp, table, [s], a["scale"])
    return len(idx)


def _limit_blas():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_baseline(w, seconds, kv_kind="bf16"):
    """The fp64 oracle on this host's cores over a bounded sample of the same workload.

    Inputs (one decode step of every sequence, values as stored in bf16, or
    FP8 / INT8 codes and scales) are built first and kept in host memory; then
    whole passes over all sequences are timed until `seconds` / 2 of wall time
    have accumulated, first on one core (one process, one BLAS thread), then on
    every core this process may use (capped at 16, the CPU share of one GPU on
    the measurement hosts): one worker process per core, one BLAS thread each,
    the sequences of a pass dealt round-robin to the workers.  Runs before the
    GPU is initialised, so the workers are plain forks of a CPU-only process.
    """
    import multiprocessing as mp
    import torch
    import synth
    from threadpoolctl import threadpool_limits
    fp8 = kv_kind in ("fp8", "int8")  # one-byte codes with scales
    fill = synth.fill_int8_codes_ if kv_kind == "int8" else synth.fill_fp8_codes_
    scales = synth.int8_scales if kv_kind == "int8" else synth.fp8_scales
    lens = synth.seq_lengths(w)
    if w.name == "long":
        lens = lens[:2]  # one layer of two 32,768-token sequences (the oracle holds them in host memory)
    rng = np.random.default_rng(0)
    bs, hkv, d = w.block_size, w.hkv, w.d
    _CPU_INPUTS.clear()
    _CPU_ARGS.update(kv=kv_kind, codes=fp8, scale=w.scale)
    for n, s in enumerate(lens):
        nb = -(-s // bs)
        if fp8:
            kp = fill(torch.empty((nb, hkv, bs, d), dtype=torch.uint8), 5000 + n).numpy()
            vp = fill(torch.empty((nb, hkv, bs, d), dtype=torch.uint8), 6000 + n).numpy()
            ks = scales(nb, hkv, w.value_scale, 8000 + n).double().numpy()
            vs = scales(nb, hkv, w.value_scale, 9000 + n).double().numpy()
        else:
            kp = synth.randn((nb, hkv, bs, d), torch.bfloat16, w.value_scale, 5000 + n).float().numpy()
            vp = synth.randn((nb, hkv, bs, d), torch.bfloat16, w.value_scale, 6000 + n).float().numpy()
            ks = vs = None
        q = synth.randn((1, w.hq, d), torch.bfloat16, w.value_scale, 7000 + n).double().numpy()
        table = rng.permutation(nb)[None]
        kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
        kp2[table[0]] = kp
        vp2[table[0]] = vp
        if fp8:
            ks2, vs2 = np.empty_like(ks), np.empty_like(vs)
            ks2[table[0]] = ks
            vs2[table[0]] = vs
            ks, vs = ks2, vs2
        _CPU_INPUTS.append((q, kp2, vp2, ks, vs, table, s))
    step_bytes = sum(lens) * 2 * hkv * d * (1 if fp8 else 2) + (sum(-(-s // bs) for s in lens) * 2 * hkv * 4 if fp8 else 0)
    every = list(range(len(lens)))

    def timed(run_pass):
        passes, t_total = 0, 0.0
        while t_total < seconds / 2:
            t0 = time.perf_counter()
            run_pass()
            t_total += time.perf_counter() - t0
            passes += 1
        return passes, t_total

    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        p1, t1 = timed(lambda: _oracle_over(every))
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    chunks = [every[c::cores] for c in range(cores)]
    with mp.get_context("fork").Pool(cores, initializer=_limit_blas) as pool:
        pool.map(_oracle_over, [[i] for i in range(min(cores, len(every)))])  # workers up
        pn, tn = timed(lambda: pool.map(_oracle_over, chunks))
    _CPU_INPUTS.clear()
    what = (f"one decode step of {'one layer of ' if w.name == 'long' else ''}"
            f"{'the first' if w.name == 'long' else 'all'} {len(lens)} sequences of the same workload "
            f"({kv_kind.upper() + ' cache, ' if fp8 else ''}all {w.hq} query heads; fp64 NumPy oracle)")
    return {"value": round(pn * step_bytes / tn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "blas_threads_per_process": 1,
            "sample": f"{pn} passes over {what} on {cores} worker processes, {tn:.1f} s wall",
            "us_per_step": round(tn / pn * 1e6, 1),
            "one_core": {"value": round(p1 * step_bytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "sample": f"{p1} passes over the same step in this process, one BLAS thread, "
                                   f"{t1:.1f} s of compute",
                         "us_per_step": round(t1 / p1 * 1e6, 1)}}


def synth_fork_prompts():
    import synth
    return synth.FORK_PROMPTS


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode path needs no inter-GPU exchange: sequences or KV heads shard with no collective).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return
    if args.read_ceiling:
        import ctypes
        import paged_kv_cache_124_amd as pa  # noqa: F401  (torch's HIP runtime first, as for libpa.so)
        probe = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_124_amd", "libpa_probe.so"))
        probe.pa_read_probe.restype = ctypes.c_int
        probe.pa_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
        buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")  # 4 GiB, 16x the Infinity Cache
        sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def read_probe(wgs, nt):
            st = probe.pa_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4, ctypes.c_void_p(sink.data_ptr()),
                                     wgs, nt, stream)
            if st != 0:
                raise RuntimeError(f"pa_read_probe: status {st}")
        rates = {"nontemporal": {}, "default_policy": {}}
        for nt, key in ((1, "nontemporal"), (0, "default_policy")):
            for wgs in (256, 512, 1024, 2048):  # 4, 8, 16, 32 waves per CU on 256 CUs
                for _ in range(3):
                    read_probe(wgs, nt)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(20):
                    read_probe(wgs, nt)
                b.record()
                torch.cuda.synchronize()
                rates[key][wgs] = round(buf.numel() * 4 * 20 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
        print(json.dumps({"read_ceiling_gb_s": max(rates["nontemporal"].values()),
                          "default_policy_gb_s": max(rates["default_policy"].values()), "by_workgroups": rates,
                          "bytes": buf.numel() * 4, "launches": 20, "peak_gb_s": HBM_PEAK_GBS}))
        return
    w = workload(args.workload)
    cpu = None
    if not args.no_cpu_baseline:  # before the GPU is initialised: its worker processes are plain forks
        print("[bench] oracle cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds, args.kv)
    others = None
    if not args.no_others and args.workload == "gqa8b" and args.kv == "bf16" and not args.shared:
        others = other_workloads()  # child processes, while this one has not touched the GPU
    total = args.steps + args.warmup + 1
    print(f"[bench] building workload {w.name}", file=sys.stderr, flush=True)
    if args.shared and (w.name != "fork" or args.kv != "bf16"):
        print("--shared applies to the bf16 fork workload", file=sys.stderr)
        sys.exit(2)
    if w.name == "long":
        if args.kv != "bf16" or args.shared:
            print("the long workload runs the bf16 decode", file=sys.stderr)
            sys.exit(2)
        run = LongRunner(w, total)
    else:
        run = Runner(w, total, args.replicas, kv_kind=args.kv, shared=args.shared)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps), timing {args.steps}", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # The decode is bracketed by events on the stream it is launched on.  An event
    # record costs the stream a few microseconds, part of it inside the bracket, so
    # where a step launches nothing but the decode step's two kernels (no
    # copy-on-write) one pair brackets EVENT_SPAN consecutive steps, placed between
    # the ring's own event records; elsewhere (the fork workload's copies, the long
    # workload's appends) one pair brackets the decode of every EVENT_EVERY-th step.
    long_ctx = w.name == "long"
    span = min(EVENT_SPAN, args.steps) if not (long_ctx or run.fork) else 1
    sampled = list(range(0, args.steps, 1 if long_ctx else EVENT_EVERY))  # a long step is ~12 ms: events every step
    timing = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
    spans, open_span = [], None  # [start event, end event, steps, bytes]
    torch.cuda.synchronize()
    run.host_s = 0.0
    t0 = time.perf_counter()
    e0.record()
    kv_bytes, sampled_bytes = 0, 0
    for i in range(args.steps):
        if span == 1:
            ev = timing.get(i)
        else:
            pos = run.step_i % (RING // 2)  # the ring's event is recorded after the step at pos RING / 2 - 1
            start = end = None
            # a span opens wherever it still ends before the ring's next record
            if open_span is None and pos + span <= RING // 2 and i + span <= args.steps:
                open_span = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), 0, 0]
                start = open_span[0]
            if open_span is not None and open_span[2] == span - 1:  # this step is the span's last
                end = open_span[1]
            ev = (start, end) if (start is not None or end is not None) else None
        step_bytes = run.step(ev)
        kv_bytes += step_bytes
        if span == 1 and ev is not None:
            sampled_bytes += step_bytes
        if open_span is not None:
            open_span[2] += 1
            open_span[3] += step_bytes
            if ev is not None and ev[1] is not None:
                spans.append(open_span)
                open_span = None
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    run.check_device_batch()
    gpu_ms = e0.elapsed_time(e1)
    ms_step = max(gpu_ms, wall * 1e3) / args.steps
    value = kv_bytes / args.steps / (ms_step * 1e-3) / 1e9
    if span == 1:
        dec_us = [1e3 * a.elapsed_time(b) for a, b in timing.values()]
    else:  # per-launch averages of the spans, each counted once per step it covers
        dec_us = [1e3 * a.elapsed_time(b) / n for a, b, n, _ in spans for _ in range(n)]
        sampled_bytes = sum(b for _, _, _, b in spans)
    if not dec_us:  # no span fitted between the ring's event records: the whole timed region instead
        dec_us = [gpu_ms * 1e3 / args.steps] * args.steps
        sampled_bytes = kv_bytes
    dec_avg_us = sum(dec_us) / len(dec_us)
    bytes_per_launch = kv_bytes / args.steps
    achieved = sampled_bytes / (sum(dec_us) * 1e-6) / 1e9
    traffic = measured_traffic(w.name, args.kv) if not args.shared else None
    fp8 = args.kv in ("fp8", "int8")  # one-byte codes with scales
    codes_name = {"fp8": "FP8 E4M3", "int8": "INT8"}.get(args.kv, "")
    if run.fork:
        # bytes a step needs from memory when each prompt's shared full blocks are read once
        st, groups = run.bm.shared_groups(run.seqs, 32 // (w.hq // w.hkv))
        assert st == 0
        saved = sum((c - 1) * p for _, c, p in groups.tolist()) * run.kv_bytes_per_token
        unique_per_step = bytes_per_launch - saved
        workload_desc = (f"fork: {synth_fork_prompts()} prompts of {run.lens0[0]} tokens, each forked into "
                         f"{run.n // synth_fork_prompts()} samples ({run.n} seqs sharing 128 full prefix blocks per "
                         f"prompt), Hq {w.hq}, Hkv {w.hkv}, d_head {w.d}, block {w.block_size}, bf16, copy-on-write "
                         f"of the tails on the first step, contexts growing 1/step; decode "
                         f"{'pa_decode_step_shared (shared blocks read once per group)' if args.shared else 'pa_decode_step (every row reads its own table)'}")
    elif long_ctx:
        workload_desc = (f"long: {w.layers} layers x {run.n} seqs of {run.lens0[0]} tokens (64 GiB of KV in one "
                         f"allocation per tensor), Hq {w.hq}, Hkv {w.hkv}, d_head {w.d}, block {w.block_size}, bf16, "
                         f"random placement; a step appends each sequence's new token in every layer and decodes every "
                         f"layer over S + 1 tokens, contexts growing 1/step")
    else:
        workload_desc = (f"{w.name}{'-' + args.kv if fp8 else ''}: {run.n} seqs, Hq {w.hq}, Hkv {w.hkv}, d_head {w.d}, "
                         f"block {w.block_size}, {codes_name + ' cache with per-(block, KV head) scales' if fp8 else 'bf16'}, "
                         f"contexts {min(run.lens0)}..{max(run.lens0)} growing 1/step")
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-e4m3 cache, bf16 q/out", "int8": "int8 cache, bf16 q/out"}.get(args.kv, "bf16"),
        "data": "synthetic",
        "config": {"workload": workload_desc,
                   "num_seqs": run.n, "block_size": w.block_size, "pool_blocks": run.num_blocks,
                   "pool_replicas": 1 if long_ctx else args.replicas, "partition_tokens": run.part,
                   "kv_bytes_per_step": int(bytes_per_launch), "us_per_step": round(ms_step * 1e3, 2),
                   "host_us_per_step": round(run.host_s / args.steps * 1e6, 2),
                   "staging": ("slots of every step on the device before the timed region" if long_ctx else
                               "pinned host ring read by the kernels" if run.zero_copy else "pinned ring, in-stream copy"),
                   "tail_waste_slots": run.bm.stats()["tail_waste_slots"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if traffic is None else int(traffic[0]),
                     "traffic_algorithmic": None if traffic is None else int(traffic[1]),
                     "kernel": f"pa_decode_step_{args.kv} (decode kernel + merge/append kernel)" if fp8 else
                               ("pa_decode_step_shared (shared-prefix decode kernel + merge/append kernel)"
                                if args.shared else
                                (f"pa_decode x {w.layers} layers (decode kernel + merge kernel each)" if long_ctx
                                 else "pa_decode_step (decode kernel + merge/append kernel)")),
                     "avg_us": round(dec_avg_us, 2), "launches_timed": len(dec_us)},
    }
    if run.fork:
        # value and roofline count the KV the attention consumes (every row's own context); with
        # sharing most of it is read once per group, so the bytes a step needs are given beside it
        res["config"]["unique_kv_bytes_per_step"] = int(unique_per_step)
        res["config"]["unique_gb_s"] = round(unique_per_step / (ms_step * 1e-3) / 1e9, 2)
        # the roofline counts the bytes a step needs from HBM (shared blocks once); the logical
        # figure (every row's context, re-reads served by the caches) is kept beside it
        res["roofline"]["achieved_logical"] = res["roofline"]["achieved"]
        res["roofline"]["achieved"] = round(achieved * unique_per_step / bytes_per_launch, 1)
        res["roofline"]["frac"] = round(res["roofline"]["achieved"] / HBM_PEAK_GBS, 4)
        res["roofline"]["bytes"] = "unique KV a step needs: each shared full block once, every row's own blocks"
    if cpu is not None:
        res["cpu_baseline"] = cpu
    if others is not None:
        res["other_workloads"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
