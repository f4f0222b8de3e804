"""Test helpers: marshal workload tensors into the NumPy arrays the oracle takes."""

import numpy as np
import torch

import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a bf16 tensor as uint16."""
    assert t.dtype == torch.bfloat16
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_cache(wl) -> "oracle.Cache":
    return oracle.Cache(
        bits(wl.k_cache),
        bits(wl.v_cache),
        wl.seq_lens.cpu().numpy(),
        layout=wl.layout,
        page_table=None if wl.page_table is None else wl.page_table.cpu().numpy(),
        page_size=wl.page_size,
    )


def bf16_from_float(x) -> np.ndarray:
    """bf16 bit patterns of float values via torch's rounding (round to nearest even)."""
    return bits(torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))
