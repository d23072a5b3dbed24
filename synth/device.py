"""Device-resident synthetic inputs (torch tensors filled by libsynth_gpu.so).

Input generation only: allocation and the seeded fill defined in synth_rng.h.
bf16 tensors hold exactly the bit patterns the CPU fill produces.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Workload, gpu_fill_kv, gpu_fill_weight, page_tables, host_tokens

WEIGHT_NAMES = ("embed", "norm", "w_qkv", "w_o", "w_router", "w_gate_up", "w_down")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def device_weights(wl: Workload, device="cuda") -> dict:
    out = {}
    for name, numel in wl.geom.tensor_numel().items():
        t = torch.empty(numel, dtype=torch.bfloat16, device=device)
        gpu_fill_weight(wl, name, t.data_ptr(), _stream())
        out[name] = t
    return out


def device_kv_pool(wl: Workload, device="cuda") -> torch.Tensor:
    n = wl.geom.n_layers * wl.geom.kv_layer_numel(wl.n_pages)
    t = torch.empty(n, dtype=torch.bfloat16, device=device)
    gpu_fill_kv(wl, t.data_ptr(), _stream())
    return t


def device_step_inputs(wl: Workload, step: int = 0, device="cuda") -> dict:
    """tokens, seq_lens, page_table (device int32) plus their host mirrors."""
    pt = page_tables(wl)
    toks = host_tokens(wl, step)
    sl = np.asarray(wl.seq_lens, dtype=np.int32)
    return {
        "tokens": torch.from_numpy(toks).to(device),
        "seq_lens": torch.from_numpy(sl).to(device),
        "page_table": torch.from_numpy(pt).to(device),
        "h_tokens": toks,
        "h_seq_lens": sl,
        "h_page_table": pt,
    }


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
