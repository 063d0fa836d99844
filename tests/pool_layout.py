"""Test-side conversion between the logical pool [nb][Hkv][B][D] and libpa's physical layout.

Written from the index formulas documented in include/pa.h (x = 16 / element size):
  K: k_pool[(((pb * Hkv + j) * (D / x) + d / x) * B + off) * x + d % x]
  V: v_pool[((pb * Hkv + j) * D + d) * B + off]
It is the tests' adapter for the device side; the oracle never sees it.
"""

import torch


def k_to_physical(k_log: torch.Tensor) -> torch.Tensor:
    nb, hkv, bs, d = k_log.shape
    x = 16 // k_log.element_size()
    return k_log.reshape(nb, hkv, bs, d // x, x).permute(0, 1, 3, 2, 4).contiguous()


def k_to_logical(k_phys: torch.Tensor) -> torch.Tensor:
    nb, hkv, dx, bs, x = k_phys.shape
    return k_phys.permute(0, 1, 3, 2, 4).reshape(nb, hkv, bs, dx * x)


def v_to_physical(v_log: torch.Tensor) -> torch.Tensor:
    return v_log.permute(0, 1, 3, 2).contiguous()


def v_to_logical(v_phys: torch.Tensor) -> torch.Tensor:
    return v_phys.permute(0, 1, 3, 2)


def poison_unused_(k_phys, v_phys, tables, lens, block_size, value=float("nan")):
    """Fill every block no sequence uses, and every slot past a sequence's end, with `value`.

    The oracle never reads those slots, so the device output must not depend on them.
    """
    used = torch.zeros(k_phys.shape[0], dtype=torch.bool)
    for row, s in zip(tables, lens):
        nb = -(-int(s) // block_size)
        used[torch.as_tensor(row[:nb], dtype=torch.long)] = True
    unused = (~used).nonzero().flatten().to(k_phys.device)
    if unused.numel():
        k_phys.index_fill_(0, unused, value)
        v_phys.index_fill_(0, unused, value)
    for row, s in zip(tables, lens):
        s = int(s)
        off = s % block_size
        if s > 0 and off:
            pb = int(row[(s - 1) // block_size])
            k_phys[pb, :, :, off:, :] = value
            v_phys[pb, :, :, off:] = value
