"""Shared helpers for the GPU tests: moving seeded inputs to the device and
the parity bar."""
from __future__ import annotations

import numpy as np
import torch

# fp16 Q/K/V with fp32 accumulation against the fp64 oracle: a hard
# max |gpu - ref| <= ATOL over every compared element, and the relative part
# of the bar as a scale-aware check ||gpu - ref||_2 / ||ref||_2 <= REL_L2
# (outputs of long contexts are ~1e-3, where an elementwise relative bound
# would say little).
ATOL = 2e-3
REL_L2 = 1e-2


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev or device())


def dev_inputs(inp, dev=None):
    dev = dev or device()
    return dict(q=to_dev(inp.q, dev), k_cache=to_dev(inp.k_cache, dev),
                v_cache=to_dev(inp.v_cache, dev), block_tables=to_dev(inp.block_tables, dev),
                seq_lens=to_dev(inp.seq_lens, dev))


def assert_parity(gpu: np.ndarray, ref: np.ndarray, what: str = "", mask=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        gpu, ref = gpu[mask], ref[mask]
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert not err.size or err.max() <= ATOL, (
        f"{what}: max abs err {err.max():.3e} > {ATOL} at {worst} "
        f"(ref {ref[worst]:.4e}, gpu {gpu[worst]:.4e})")
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(gpu - ref) / nref
        assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e}"
    return float(err.max()) if err.size else 0.0
