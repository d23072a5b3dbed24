"""Python binding of libmkd.so, the persistent decode megakernel for MI355X (gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels behind
the C-ABI declared in include/mkd.h.  PyTorch provides device memory (the engine's
workspace is a torch tensor handed to mkd_set_workspace) and streams; tensors are
passed as raw device pointers.  There is no fallback: if the library is missing or
fails to load, creating an engine raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmkd.so")

MKD_OK = 0
MKD_ERR_ARG = -1
MKD_ERR_HIP = -2
MKD_ERR_CAPACITY = -3
MKD_ERR_DEADLOCK = -4
MKD_ERR_STATE = -5
MODE_MEGAKERNEL = 0
MODE_OP_PER_KERNEL = 1
DEBUG_HIDDEN = 0
DEBUG_TOPK_IDS = 1
DEBUG_TOPK_W = 2
DEBUG_ROUTER = 3
DEBUG_Q = 4
DEBUG_ATTN = 5
DEBUG_ROUTE = 6
DEBUG_ACT = 7
ORDER_DEFAULT, ORDER_ATTN_FIRST, ORDER_MOE_FIRST, ORDER_INTERLEAVED = 0, 1, 2, 3
PLACE_ROUND_ROBIN, PLACE_XCD = 0, 1
ROUTE_WORDS = 1548
DESC_WORDS = 32
D_WAVE = 6  # descriptor word holding the task's wave index
D_GIDX = 7  # descriptor word holding the task's position in the global order

# every symbol include/mkd.h declares
EXPORTS = ("mkd_create", "mkd_destroy", "mkd_workspace_bytes", "mkd_set_workspace",
           "mkd_load_weights", "mkd_set_mode", "mkd_decode_step", "mkd_decode_step_static",
           "mkd_sync_status",
           "mkd_set_watchdog", "mkd_set_attention_window", "mkd_last_error", "mkd_debug_read", "mkd_plan_inspect",
           "mkd_set_trace", "mkd_set_schedule",
           "mkd_server_create", "mkd_server_destroy", "mkd_server_buffer_bytes", "mkd_server_set_buffer",
           "mkd_server_join", "mkd_server_step", "mkd_server_last_step", "mkd_server_stats",
           "mkd_server_last_error", "mkd_protocol_litmus")


class MkdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mkd error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "moe_inter", "vocab", "page_size")] + [("rms_eps", ctypes.c_float),
                                               ("rope_base", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "embed", "norm", "w_qkv", "w_o", "w_router", "w_gate_up", "w_down")]


_lib = None


def lib():
    """Load libmkd.so; raises if it is absent (build it with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        # MKD_LIBRARY names another build of the same library (e.g. other tuning constants)
        path = os.environ.get("MKD_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
        sig = {
            "mkd_create": ([P(Config), I32, I32, I32, P(VP)], I32),
            "mkd_destroy": ([VP], None),
            "mkd_workspace_bytes": ([VP], ctypes.c_size_t),
            "mkd_set_workspace": ([VP, VP, ctypes.c_size_t], I32),
            "mkd_set_watchdog": ([VP, I32], I32),
            "mkd_set_attention_window": ([VP, I32, I32], I32),
            "mkd_load_weights": ([VP, P(Weights)], I32),
            "mkd_set_mode": ([VP, I32], I32),
            "mkd_decode_step": ([VP, VP, I32, VP, VP, VP, VP, VP, VP, I32, VP], I32),
            "mkd_decode_step_static": ([VP, VP, I32, VP, VP, VP, VP, VP, VP, I32, VP], I32),
            "mkd_sync_status": ([VP], I32),
            "mkd_last_error": ([VP], ctypes.c_char_p),
            "mkd_debug_read": ([VP, I32, VP, ctypes.c_size_t], I32),
            "mkd_plan_inspect": ([VP, I32, VP, I32, VP, P(I32)], I32),
            "mkd_set_schedule": ([VP, I32, I32], I32),
            "mkd_set_trace": ([VP, VP, ctypes.c_size_t], I32),
            "mkd_server_create": ([VP, I32, I32, P(VP)], I32),
            "mkd_server_destroy": ([VP], None),
            "mkd_server_buffer_bytes": ([VP], ctypes.c_size_t),
            "mkd_server_set_buffer": ([VP, VP, ctypes.c_size_t], I32),
            "mkd_server_join": ([VP, ctypes.c_int64, I32, I32, I32, VP, I32], I32),
            "mkd_server_step": ([VP, VP, VP, P(I32)], I32),
            "mkd_server_last_step": ([VP, VP, VP, VP, VP, VP, VP, I32, P(I32)], I32),
            "mkd_server_stats": ([VP, P(I32), P(I32), P(I32)], I32),
            "mkd_server_last_error": ([VP], ctypes.c_char_p),
            "mkd_protocol_litmus": ([I32, I32, I32, VP], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def config_of(g) -> Config:
    """mkd_config from any object with the geometry attribute names."""
    return Config(g.n_layers, g.hidden, g.n_q_heads, g.n_kv_heads, g.head_dim, g.n_experts,
                  g.top_k, g.moe_inter, g.vocab, g.page_size, g.rms_eps, g.rope_base)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


class Engine:
    """One mkd_engine.  device=-1 gives a host-only engine for plan inspection.  A device
    engine gets its workspace from torch (a uint8 tensor of mkd_workspace_bytes bytes on
    that device) unless `workspace=False`, in which case set_workspace() must be called."""

    def __init__(self, geom, device: int, max_batch: int, max_pages_per_seq: int, workspace=True):
        self.geom = geom
        self.device = device
        self.max_batch = max_batch
        self.max_pages = max_pages_per_seq
        self._cfg = config_of(geom)
        self._ws = None
        h = ctypes.c_void_p()
        rc = lib().mkd_create(ctypes.byref(self._cfg), device, max_batch, max_pages_per_seq,
                              ctypes.byref(h))
        if rc != MKD_OK:
            raise MkdError(rc, lib().mkd_last_error(None).decode())
        self._h = h
        self._weights = None
        if device >= 0 and workspace:
            import torch

            self.set_workspace(torch.empty(self.workspace_bytes(), dtype=torch.uint8,
                                           device=f"cuda:{device}"))

    def workspace_bytes(self) -> int:
        return int(lib().mkd_workspace_bytes(self._h))

    def set_workspace(self, buf):
        """buf: a device tensor of at least workspace_bytes() bytes, kept referenced."""
        self._check(lib().mkd_set_workspace(self._h, _ptr(buf), buf.numel() * buf.element_size()))
        self._ws = buf

    def set_watchdog(self, polls: int):
        self._check(lib().mkd_set_watchdog(self._h, int(polls)))

    def set_attention_window(self, window: int, full_every: int = 1):
        """Local-attention layers: layer l attends to its last `window` positions unless
        (l + 1) % full_every == 0; window 0 makes every layer full attention."""
        self._check(lib().mkd_set_attention_window(self._h, int(window), int(full_every)))

    def close(self):
        if getattr(self, "_h", None):
            lib().mkd_destroy(self._h)
            self._h = None
        self._ws = None
        self._weights = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc):
        if rc != MKD_OK:
            raise MkdError(rc, lib().mkd_last_error(self._h).decode())
        return rc

    def load_weights(self, w: dict):
        """w: dict of bf16 device tensors (embed, norm, w_qkv, w_o, w_router, w_gate_up,
        w_down), kept referenced by the engine."""
        self._weights = dict(w)
        st = Weights(*[_ptr(w[k]) for k in ("embed", "norm", "w_qkv", "w_o", "w_router",
                                           "w_gate_up", "w_down")])
        self._check(lib().mkd_load_weights(self._h, ctypes.byref(st)))

    def set_mode(self, mode: int):
        self._check(lib().mkd_set_mode(self._h, mode))

    def decode_step(self, tokens, seq_lens, h_seq_lens: np.ndarray, page_table, kv_pool, n_pages,
                    logits, h_page_table: Optional[np.ndarray] = None, stream=None, static=False):
        """Enqueue one step.  tokens, seq_lens, page_table: int32 device tensors; kv_pool
        bf16 device tensor; logits fp32 device tensor [batch][vocab].  static=True calls
        mkd_decode_step_static (the library's static scratch instead of the workspace)."""
        h_seq_lens = np.ascontiguousarray(h_seq_lens, dtype=np.int32)
        hpt = None if h_page_table is None else np.ascontiguousarray(h_page_table, dtype=np.int32)
        s = None if stream is None else ctypes.c_void_p(stream)
        fn = lib().mkd_decode_step_static if static else lib().mkd_decode_step
        self._check(fn(self._h, s, int(h_seq_lens.size), _ptr(tokens), _ptr(seq_lens), _ptr(h_seq_lens),
                       _ptr(page_table), _ptr(hpt), _ptr(kv_pool), int(n_pages), _ptr(logits)))

    def sync_status(self) -> int:
        return self._check(lib().mkd_sync_status(self._h))

    def debug_read(self, what: int, batch: int) -> np.ndarray:
        g = self.geom
        qd = g.n_q_heads * g.head_dim
        shapes = {DEBUG_HIDDEN: ((g.n_layers + 1, batch, g.hidden), np.float32),
                  DEBUG_TOPK_IDS: ((g.n_layers, batch, g.top_k), np.int32),
                  DEBUG_TOPK_W: ((g.n_layers, batch, g.top_k), np.float32),
                  DEBUG_ROUTER: ((g.n_layers, batch, g.n_experts), np.float32),
                  DEBUG_Q: ((g.n_layers, batch, qd), np.float32),
                  DEBUG_ATTN: ((g.n_layers, batch, qd), np.float32),
                  DEBUG_ROUTE: ((g.n_layers, ROUTE_WORDS), np.int32),
                  DEBUG_ACT: ((g.n_layers, batch * g.top_k, g.moe_inter), np.float32)}
        shape, dt = shapes[what]
        out = np.empty(shape, dtype=dt)
        self._check(lib().mkd_debug_read(self._h, what, out.ctypes.data, out.nbytes))
        return out

    def set_trace(self, buf):
        """buf: uint64/int64 device tensor of n_tasks * 4 entries, or None to disable."""
        if buf is None:
            self._check(lib().mkd_set_trace(self._h, None, 0))
        else:
            self._check(lib().mkd_set_trace(self._h, _ptr(buf), buf.numel() * buf.element_size()))
        self._trace = buf

    def set_schedule(self, order: int, placement: int = PLACE_ROUND_ROBIN):
        """Wave order (ORDER_*) and placement (PLACE_*) of the task lists."""
        self._check(lib().mkd_set_schedule(self._h, int(order), int(placement)))

    def plan(self, n_cu: int):
        """(descriptors [n_tasks][32] int32 grouped by CU, list offsets [n_cu + 1]); the
        list of CU c is desc[offs[c]:offs[c + 1]], in execution order."""
        n = ctypes.c_int32()
        rc = lib().mkd_plan_inspect(self._h, n_cu, None, 0, None, ctypes.byref(n))
        if rc not in (MKD_OK, MKD_ERR_CAPACITY):
            self._check(rc)
        desc = np.empty((n.value, DESC_WORDS), dtype=np.int32)
        offs = np.empty(n_cu + 1, dtype=np.int32)
        self._check(lib().mkd_plan_inspect(self._h, n_cu, desc.ctypes.data, n.value,
                                           offs.ctypes.data, ctypes.byref(n)))
        return desc, offs


class Server:
    """The continuous-decode loop (mkd_server_*) over an engine: sequences join with a
    cached length and a first token, each step feeds every scheduled sequence and samples
    greedily, finished sequences retire.  The device buffer is a torch uint8 tensor."""

    def __init__(self, engine: Engine, n_pages: int, max_live: int):
        import torch

        self.engine = engine
        h = ctypes.c_void_p()
        rc = lib().mkd_server_create(engine._h, int(n_pages), int(max_live), ctypes.byref(h))
        if rc != MKD_OK:
            raise MkdError(rc, "mkd_server_create failed")
        self._h = h.value
        self.max_batch = engine.max_batch
        self.max_pages = engine.max_pages
        self.vocab = engine.geom.vocab
        self._buf = None
        if engine.device >= 0:
            self._buf = torch.empty(lib().mkd_server_buffer_bytes(self._h), dtype=torch.uint8,
                                    device=f"cuda:{engine.device}")
            self._check(lib().mkd_server_set_buffer(self._h, _ptr(self._buf), self._buf.numel()))

    def _check(self, rc):
        if rc != MKD_OK:
            raise MkdError(rc, lib().mkd_server_last_error(self._h).decode())

    def join(self, seq_id: int, cached_len: int, first_token: int, max_new_tokens: int) -> np.ndarray:
        """Returns the physical pages given to the cached tokens (to be filled by the caller)."""
        pages = np.empty(max(1, self.max_pages), dtype=np.int32)
        self._check(lib().mkd_server_join(self._h, int(seq_id), int(cached_len), int(first_token),
                                          int(max_new_tokens), pages.ctypes.data, pages.size))
        return pages[:-(-int(cached_len) // self.engine.geom.page_size)] if cached_len > 0 else pages[:0]

    def try_join(self, *args) -> "np.ndarray | None":
        try:
            return self.join(*args)
        except MkdError as e:
            if e.code == MKD_ERR_CAPACITY:
                return None
            raise

    def step(self, kv_pool, stream=None) -> int:
        if stream is not None or kv_pool is None:
            s = stream or 0
        else:
            import torch

            s = torch.cuda.current_stream().cuda_stream
        n = ctypes.c_int32()
        self._check(lib().mkd_server_step(self._h, ctypes.c_void_p(s), _ptr(kv_pool), ctypes.byref(n)))
        return n.value

    def last_step(self, logits=False) -> dict:
        B, P = self.max_batch, self.max_pages
        ids = np.empty(B, np.int64)
        fed, smp, lens = (np.empty(B, np.int32) for _ in range(3))
        table = np.empty((B, P), np.int32)
        lg = np.empty((B, self.vocab), np.float32) if logits else None
        n = ctypes.c_int32()
        self._check(lib().mkd_server_last_step(self._h, ids.ctypes.data, fed.ctypes.data, smp.ctypes.data,
                                               lens.ctypes.data, table.ctypes.data,
                                               lg.ctypes.data if logits else None, B, ctypes.byref(n)))
        b = n.value
        out = dict(ids=ids[:b], fed=fed[:b], sampled=smp[:b], seq_lens=lens[:b], page_table=table[:b])
        if logits:
            out["logits"] = lg[:b]
        return out

    def stats(self) -> dict:
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(lib().mkd_server_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return dict(live=a.value, parked=b.value, free_pages=c.value)

    def close(self):
        if getattr(self, "_h", None):
            lib().mkd_server_destroy(self._h)
            self._h = None
        self._buf = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def protocol_litmus(device: int, n_pairs: int = 128, rounds: int = 2000) -> dict:
    """Message-passing litmus test of the inter-workgroup protocol (mkd_protocol_litmus)."""
    res = np.zeros(4, dtype=np.uint32)
    rc = lib().mkd_protocol_litmus(int(device), int(n_pairs), int(rounds), res.ctypes.data)
    if rc != MKD_OK:
        raise MkdError(rc, "mkd_protocol_litmus failed")
    return dict(torn_words=int(res[0]), stale_data=int(res[1]), timeouts=int(res[2]), rounds_done=int(res[3]))
