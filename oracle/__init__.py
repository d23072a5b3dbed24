"""ctypes binding of the CPU reference (liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the decode library never does.  Arrays are numpy:
bf16 tensors are uint16 bit patterns, activations float32, indices int32.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
F32 = ctypes.c_float


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "moe_inter", "vocab", "page_size")] + [("rms_eps", ctypes.c_float),
                                               ("rope_base", ctypes.c_float),
                                               ("attn_window", ctypes.c_int32),
                                               ("full_every", ctypes.c_int32)]


def layer_window(g, layer):
    """Attention window of layer `layer` in a decode step (0: every position)."""
    w, every = getattr(g, "attn_window", 0), getattr(g, "full_every", 1)
    return w if w > 0 and (every < 1 or (layer + 1) % every != 0) else 0


def dims_of(g, window=None) -> Dims:
    """Dims of geometry g; `window` overrides the attention window (per-layer calls)."""
    w = getattr(g, "attn_window", 0) if window is None else window
    return Dims(g.n_layers, g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.n_experts,
                g.top_k, g.moe_inter, g.vocab, g.page_size, g.rms_eps, g.rope_base,
                w, getattr(g, "full_every", 1))


def load(path):
    """Load a build of the reference from `path` and declare its signatures."""
    L = ctypes.CDLL(path)
    D = ctypes.POINTER(Dims)
    sig = {
        "orc_bf16_to_f32": ([ctypes.c_uint16], F32),
        "orc_f32_to_bf16": ([F32], ctypes.c_uint16),
        "orc_rmsnorm": ([I32, P, P, F32, P], None),
        "orc_matvec_bf16": ([I32, I32, P, P, P], None),
        "orc_rope": ([I32, F32, I64, P], None),
        "orc_kv_index": ([D, I32, I32, I32, I32, I32, I32], I64),
        "orc_qkv_rope_append": ([D, I64, P, P, P, P, I32, P], None),
        "orc_attention": ([D, I64, P, P, I32, P, P], None),
        "orc_topk_softmax": ([I32, I32, P, P, P], None),
        "orc_expert_act": ([I32, I32, P, P, P], None),
        "orc_expert_ffn": ([I32, I32, P, P, P, P], None),
        "orc_moe": ([D, P, P, P, P, P, P], None),
        "orc_layer": ([D, I32, P, P, I32, P, I32, P, P, P, P, P, P, P, P, P, P, P, P, P],
                      None),
        "orc_decode_step": ([D, I32, P, P, P, I32, P, I32, P, P, P, P, P, P, P, P, P, P, P],
                            None),
        "orc_lm_head": ([D, I32, P, P, P, P], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        _lib = load(path)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda v: lib().orc_f32_to_bf16(float(v)), otypes=[np.uint16])
    return f(np.asarray(x, dtype=np.float32))


def rmsnorm(v, gamma, eps):
    v, gamma = _f32(v), _u16(gamma)
    out = np.empty_like(v)
    lib().orc_rmsnorm(v.size, _p(v), _p(gamma), eps, _p(out))
    return out


def matvec(W, x):
    W, x = _u16(W), _f32(x)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float32)
    lib().orc_matvec_bf16(rows, cols, _p(W), _p(x), _p(y))
    return y


def rope(v, base, pos):
    v = _f32(v).copy()
    lib().orc_rope(v.size, base, pos, _p(v))
    return v


def kv_index(g, n_pages, kv, page, grp, t, dim):
    d = dims_of(g)
    return lib().orc_kv_index(ctypes.byref(d), n_pages, kv, page, grp, t, dim)


def qkv_rope_append(g, pos, page_row, x, w_qkv, kv_layer, n_pages):
    """Returns q [nq*hd]; writes k, v into kv_layer (modified in place)."""
    d = dims_of(g)
    page_row, x, w_qkv = _i32(page_row), _f32(x), _u16(w_qkv)
    assert kv_layer.dtype == np.uint16 and kv_layer.flags.c_contiguous
    q = np.empty(g.n_q_heads * g.head_dim, dtype=np.float32)
    lib().orc_qkv_rope_append(ctypes.byref(d), pos, _p(page_row), _p(x), _p(w_qkv),
                              _p(kv_layer), n_pages, _p(q))
    return q


def attention(g, pos, page_row, kv_layer, n_pages, q, window=0):
    """Attention of every q head over positions 0..pos (the last `window` of them when
    window > 0)."""
    d = dims_of(g, window)
    page_row, q, kv_layer = _i32(page_row), _f32(q), _u16(kv_layer)
    o = np.empty(g.n_q_heads * g.head_dim, dtype=np.float32)
    lib().orc_attention(ctypes.byref(d), pos, _p(page_row), _p(kv_layer), n_pages, _p(q), _p(o))
    return o


def topk_softmax(logits, k):
    logits = _f32(logits)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float32)
    lib().orc_topk_softmax(logits.size, k, _p(logits), _p(ids), _p(w))
    return ids, w


def expert_act(x, w_gate_up):
    """silu(gate rows . x) * (up rows . x); w_gate_up [2I][H] uint16."""
    x, w_gate_up = _f32(x), _u16(w_gate_up)
    I = w_gate_up.shape[0] // 2
    act = np.empty(I, dtype=np.float32)
    lib().orc_expert_act(w_gate_up.shape[1], I, _p(x), _p(w_gate_up), _p(act))
    return act


def expert_ffn(x, w_gate_up, w_down):
    x, w_gate_up, w_down = _f32(x), _u16(w_gate_up), _u16(w_down)
    H, I = w_down.shape
    y = np.empty(H, dtype=np.float32)
    lib().orc_expert_ffn(H, I, _p(x), _p(w_gate_up), _p(w_down), _p(y))
    return y


def moe(g, x, ids, w, gate_up, down):
    """gate_up: [E][2I][H] uint16, down: [E][H][I] uint16."""
    d = dims_of(g)
    x, ids, w = _f32(x), _i32(ids), _f32(w)
    gate_up, down = _u16(gate_up), _u16(down)
    E = gate_up.shape[0]
    gp = (ctypes.c_void_p * E)(*[gate_up[e].ctypes.data for e in range(E)])
    dp = (ctypes.c_void_p * E)(*[down[e].ctypes.data for e in range(E)])
    m = np.empty(g.hidden, dtype=np.float32)
    lib().orc_moe(ctypes.byref(d), _p(x), _p(ids), _p(w), ctypes.cast(gp, P), ctypes.cast(dp, P),
                  _p(m))
    return m


def layer(g, seq_lens, page_table, kv_layer, n_pages, gamma, w_qkv, w_o, w_router, w_gate_up,
          w_down, h, debug=False, layer_index=0):
    """One layer for a batch.  h [B][H] float32 is updated in place; kv_layer in
    place.  With debug=True returns a dict of intermediate values.  layer_index selects
    the attention window of a local-attention geometry."""
    d = dims_of(g, layer_window(g, layer_index))
    seq_lens, page_table = _i32(seq_lens), _i32(page_table)
    B = seq_lens.size
    assert h.dtype == np.float32 and h.flags.c_contiguous and h.shape == (B, g.hidden)
    assert kv_layer.dtype == np.uint16 and kv_layer.flags.c_contiguous
    outs = {}
    if debug:
        outs = dict(x=np.empty((B, g.hidden), np.float32),
                    q=np.empty((B, g.n_q_heads * g.head_dim), np.float32),
                    attn=np.empty((B, g.n_q_heads * g.head_dim), np.float32),
                    router=np.empty((B, g.n_experts), np.float32),
                    ids=np.empty((B, g.top_k), np.int32), w=np.empty((B, g.top_k), np.float32))
    lib().orc_layer(ctypes.byref(d), B, _p(seq_lens), _p(page_table), page_table.shape[1],
                    _p(kv_layer), n_pages, _p(_u16(gamma)), _p(_u16(w_qkv)), _p(_u16(w_o)),
                    _p(_u16(w_router)), _p(_u16(w_gate_up)), _p(_u16(w_down)), _p(h),
                    _p(outs.get("x")), _p(outs.get("q")), _p(outs.get("attn")),
                    _p(outs.get("router")), _p(outs.get("ids")), _p(outs.get("w")))
    return outs


def decode_step(g, tokens, seq_lens, page_table, kv_pool, n_pages, weights, want_layers=True):
    """Full step.  kv_pool (uint16, all layers) is updated in place.  Returns
    (logits [B][V], h_layers [L+1][B][H] or None, ids [L][B][k], w [L][B][k])."""
    d = dims_of(g)
    tokens, seq_lens, page_table = _i32(tokens), _i32(seq_lens), _i32(page_table)
    B = tokens.size
    assert kv_pool.dtype == np.uint16 and kv_pool.flags.c_contiguous
    logits = np.empty((B, g.vocab), np.float32)
    hl = np.empty((g.n_layers + 1, B, g.hidden), np.float32) if want_layers else None
    ids = np.empty((g.n_layers, B, g.top_k), np.int32)
    w = np.empty((g.n_layers, B, g.top_k), np.float32)
    W = {k: _u16(v) for k, v in weights.items()}
    lib().orc_decode_step(ctypes.byref(d), B, _p(tokens), _p(seq_lens), _p(page_table),
                          page_table.shape[1], _p(kv_pool), n_pages, _p(W["embed"]),
                          _p(W["norm"]), _p(W["w_qkv"]), _p(W["w_o"]), _p(W["w_router"]),
                          _p(W["w_gate_up"]), _p(W["w_down"]), _p(logits), _p(hl), _p(ids),
                          _p(w))
    return logits, hl, ids, w


def lm_head(g, h, gamma, embed):
    d = dims_of(g)
    h = _f32(h)
    B = h.shape[0]
    logits = np.empty((B, g.vocab), np.float32)
    lib().orc_lm_head(ctypes.byref(d), B, _p(h), _p(_u16(gamma)), _p(_u16(embed)), _p(logits))
    return logits
