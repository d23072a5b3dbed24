"""Seeded synthetic inputs for the decode step: workload geometry, weights, cached
K/V, token ids and page tables.

This module makes inputs only and holds none of the decode arithmetic.  The
same values are produced on the CPU (libsynth_host.so, for the reference) and
on the GPU (libsynth_gpu.so, to fill device memory); the generator is defined
once in synth_rng.h.

Workloads follow the decode benchmarks of "Inside the megakernel serving engine
for North Mini Code" (section "Performance": synthetic KV cache, random weights
giving approximately uniform routing, 8K context, batch 1): a 30B-total /
~3B-active parallel-transformer MoE with 128 experts (top-8) and 4 KV groups.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# One stream per tensor; the flat element index inside the tensor is the counter.
STREAM = {
    "embed": 1,
    "norm": 2,
    "w_qkv": 3,
    "w_o": 4,
    "w_router": 5,
    "w_gate_up": 6,
    "w_down": 7,
    "kv": 8,
    "tokens": 9,
    "pages": 10,
}
WEIGHT_STD = 0.02
KV_STD = 1.0


@dataclasses.dataclass(frozen=True)
class Geometry:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    moe_inter: int
    vocab: int
    page_size: int = 16
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    # local-attention layers: layer l attends to the last attn_window positions unless
    # (l + 1) % full_every == 0 (attn_window 0: every layer full attention)
    attn_window: int = 0
    full_every: int = 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def tensor_numel(self) -> dict:
        L, H, E, I = self.n_layers, self.hidden, self.n_experts, self.moe_inter
        return {
            "embed": self.vocab * H,
            "norm": (L + 1) * H,
            "w_qkv": L * self.qkv_rows * H,
            "w_o": L * H * self.n_q_heads * self.head_dim,
            "w_router": L * E * H,
            "w_gate_up": L * E * 2 * I * H,
            "w_down": L * E * H * I,
        }

    def kv_layer_numel(self, n_pages: int) -> int:
        return 2 * n_pages * self.n_kv_heads * self.page_size * self.head_dim


TINY = Geometry(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, n_experts=8,
                top_k=2, moe_inter=128, vocab=1024)
FULL = Geometry(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
                n_experts=128, top_k=8, moe_inter=768, vocab=151552)
LAYER = dataclasses.replace(FULL, n_layers=1)


@dataclasses.dataclass
class Workload:
    """One decode-step input: geometry, batch lengths and KV pool size."""
    name: str
    geom: Geometry
    seq_lens: List[int]            # cached tokens per sequence (new token's position)
    n_pages: int                   # physical pages in the KV pool
    max_pages: int                 # page-table row length
    weight_seed: int = 0
    kv_seed: int = 1
    token_seed: int = 2

    @property
    def batch(self) -> int:
        return len(self.seq_lens)


def _pages_needed(seq_len: int, page: int) -> int:
    return (seq_len + 1 + page - 1) // page


def make_workload(name: str, geom: Geometry, seq_lens: Sequence[int], spare_pages: int = 0,
                  max_pages: Optional[int] = None, **seeds) -> Workload:
    need = [_pages_needed(s, geom.page_size) for s in seq_lens]
    mp = max_pages if max_pages is not None else max(need)
    return Workload(name, geom, list(seq_lens), n_pages=sum(need) + spare_pages, max_pages=mp,
                    **seeds)


def tiny_workload() -> Workload:
    """Tiny model, batch 1, 64 cached tokens: 4 cached pages plus the new token's
    page, drawn from a pool of 16 by a random permutation."""
    return make_workload("tiny-b1-ctx64", TINY, [64], spare_pages=11)


def layer_workload(ctx: int = 8192, batch: int = 1) -> Workload:
    """One full-size layer, batch 1, 8192 cached tokens in shuffled pages."""
    return make_workload(f"layer-b{batch}-ctx{ctx}", LAYER, [ctx] * batch, spare_pages=8)


def full_workload(ctx: int = 8192, batch: int = 1, steps: int = 128) -> Workload:
    """48-layer model, batch 1, 8K context; pages for `steps` further tokens."""
    extra = (steps + FULL.page_size - 1) // FULL.page_size + 1
    return make_workload(f"full-b{batch}-ctx{ctx}", FULL, [ctx] * batch,
                         spare_pages=extra * batch,
                         max_pages=_pages_needed(ctx + steps, FULL.page_size))


def ragged_workload(geom: Geometry, seq_lens: Sequence[int], spare_pages: int = 0) -> Workload:
    return make_workload(f"ragged-b{len(seq_lens)}", geom, list(seq_lens), spare_pages=spare_pages)


def continuous_sequences(n: int, vocab: int, seed: int = 11, cached=(512, 32768), new=(8, 64)):
    """A seeded stream of sequences for continuous batching: (id, cached tokens drawn
    uniform in [cached[0], cached[1]], first token uniform over the vocabulary, tokens to
    generate uniform in [new[0], new[1]])."""
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(cached[0], cached[1] + 1)), int(rng.integers(0, vocab)),
             int(rng.integers(new[0], new[1] + 1))) for i in range(n)]


def page_tables(wl: Workload) -> np.ndarray:
    """[batch][max_pages] int32 page table: every sequence's logical pages map to
    distinct physical pages of one randomly permuted pool (unused entries -1)."""
    rng = np.random.Generator(np.random.PCG64(wl.token_seed * 1000003 + STREAM["pages"]))
    perm = rng.permutation(wl.n_pages).astype(np.int32)
    pt = np.full((wl.batch, wl.max_pages), -1, dtype=np.int32)
    at = 0
    for b, s in enumerate(wl.seq_lens):
        n = _pages_needed(s, wl.geom.page_size)
        pt[b, :n] = perm[at:at + n]
        at += n
    # pages for future tokens come from the remaining pool, round robin
    rest = perm[at:]
    for b, s in enumerate(wl.seq_lens):
        n = _pages_needed(s, wl.geom.page_size)
        k = 0
        for p in range(n, wl.max_pages):
            idx = b + k * wl.batch
            if idx >= len(rest):
                break
            pt[b, p] = rest[idx]
            k += 1
    return pt


# ----------------------------------------------------------------------------------------
# CPU generation (libsynth_host.so)

_host_lib = None


def host_lib():
    global _host_lib
    if _host_lib is None:
        path = os.path.join(HERE, "libsynth_host.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build_host()
        lib = ctypes.CDLL(path)
        u64, f32 = ctypes.c_uint64, ctypes.c_float
        lib.synth_host_normal_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, f32, u64]
        lib.synth_host_normal_f32.argtypes = [ctypes.c_void_p, u64, u64, u64, f32, u64]
        lib.synth_host_gain_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, u64]
        lib.synth_host_uniform_int.argtypes = [ctypes.c_void_p, u64, u64, u64, ctypes.c_uint32,
                                               u64]
        _host_lib = lib
    return _host_lib


def host_normal_bf16(n: int, seed: int, stream: int, scale: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().synth_host_normal_bf16(out.ctypes.data, n, seed, stream, scale, offset)
    return out


def host_normal_f32(n: int, seed: int, stream: int, scale: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().synth_host_normal_f32(out.ctypes.data, n, seed, stream, scale, offset)
    return out


def host_tokens(wl: Workload, step: int = 0) -> np.ndarray:
    out = np.empty(wl.batch, dtype=np.int32)
    host_lib().synth_host_uniform_int(out.ctypes.data, wl.batch, wl.token_seed, STREAM["tokens"],
                                      wl.geom.vocab, step * 4096)
    return out


def host_gains(n: int, seed: int, offset: int = 0) -> np.ndarray:
    """bf16 bits of n RMSNorm gains 1 + 0.25 * N(0, 1) (counters offset .. offset+n-1)."""
    out = np.empty(n, dtype=np.uint16)
    host_lib().synth_host_gain_bf16(out.ctypes.data, n, seed, STREAM["norm"], offset)
    return out


def host_weight(wl: Workload, name: str, offset: int = 0, n: Optional[int] = None) -> np.ndarray:
    """bf16 bits of weight tensor `name` (elements [offset, offset+n)).  RMSNorm
    gains are 1 + 0.25 * N(0, 1), so that each layer's gains differ from one and from
    each other's."""
    numel = wl.geom.tensor_numel()[name]
    n = numel - offset if n is None else n
    if name == "norm":
        return host_gains(n, wl.weight_seed, offset)
    return host_normal_bf16(n, wl.weight_seed, STREAM[name], WEIGHT_STD, offset)


def host_weights(wl: Workload) -> dict:
    return {k: host_weight(wl, k) for k in wl.geom.tensor_numel()}


def host_kv_pool(wl: Workload) -> np.ndarray:
    n = wl.geom.n_layers * wl.geom.kv_layer_numel(wl.n_pages)
    return host_normal_bf16(n, wl.kv_seed, STREAM["kv"], KV_STD)


def host_kv_layer(wl: Workload, layer: int) -> np.ndarray:
    n = wl.geom.kv_layer_numel(wl.n_pages)
    return host_normal_bf16(n, wl.kv_seed, STREAM["kv"], KV_STD, offset=layer * n)


# ----------------------------------------------------------------------------------------
# GPU generation (libsynth_gpu.so): fills device memory in place.

_gpu_lib = None


def gpu_lib():
    global _gpu_lib
    if _gpu_lib is None:
        path = os.path.join(HERE, "libsynth_gpu.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build_gpu()
        lib = ctypes.CDLL(path)
        u64 = ctypes.c_uint64
        lib.synth_gpu_normal_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, ctypes.c_float, u64,
                                              ctypes.c_void_p]
        lib.synth_gpu_normal_bf16.restype = ctypes.c_int
        lib.synth_gpu_gain_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, u64, ctypes.c_void_p]
        lib.synth_gpu_gain_bf16.restype = ctypes.c_int
        lib.synth_gpu_fill_u16.argtypes = [ctypes.c_void_p, u64, ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_gpu_fill_u16.restype = ctypes.c_int
        _gpu_lib = lib
    return _gpu_lib


def gpu_fill_weight(wl: Workload, name: str, dev_ptr: int, stream_handle: int = 0) -> None:
    numel = wl.geom.tensor_numel()[name]
    if name == "norm":
        rc = gpu_lib().synth_gpu_gain_bf16(dev_ptr, numel, wl.weight_seed, STREAM["norm"], 0,
                                           stream_handle)
    else:
        rc = gpu_lib().synth_gpu_normal_bf16(dev_ptr, numel, wl.weight_seed, STREAM[name],
                                             WEIGHT_STD, 0, stream_handle)
    if rc != 0:
        raise RuntimeError(f"synth GPU fill of {name} failed: hip error {rc}")


def gpu_fill_kv(wl: Workload, dev_ptr: int, stream_handle: int = 0) -> None:
    n = wl.geom.n_layers * wl.geom.kv_layer_numel(wl.n_pages)
    rc = gpu_lib().synth_gpu_normal_bf16(dev_ptr, n, wl.kv_seed, STREAM["kv"], KV_STD, 0,
                                         stream_handle)
    if rc != 0:
        raise RuntimeError(f"synth GPU fill of kv pool failed: hip error {rc}")
