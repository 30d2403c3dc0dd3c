"""ctypes binding of libmk.so: the C ABI in include/mk.h, argument marshalling only.

Every step of the decode runs in the library's HIP kernels; this module turns
torch tensors into device pointers and status codes into exceptions. It never
computes anything of the decode step itself and has no fallback: if the
library is missing, importing the package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
STATUS = {0: "MK_OK", 1: "MK_ERR_INVALID_ARG", 2: "MK_ERR_UNSUPPORTED", 3: "MK_ERR_OOM", 4: "MK_ERR_HIP",
          5: "MK_ERR_DEVICE_TIMEOUT", 6: "MK_ERR_DEVICE_FAULT", 7: "MK_ERR_STATE"}
MODE_MEGAKERNEL = 0
MODE_KERNEL_PER_OP = 1
ORDER_SHIPPED, ORDER_QKV_FIRST, ORDER_ATTENTION_FIRST = 0, 1, 2
PLACE_TUNED, PLACE_ROUND_ROBIN, PLACE_AFFINITY, PLACE_COST_MODEL, PLACE_RANDOM = 0, 1, 2, 3, 4
STEP_ADVANCE = 1

# every function include/mk.h declares
EXPORTS = ("mk_create", "mk_create_host_only", "mk_load_layer", "mk_load_layer_dense", "mk_load_ffn_fp8", "mk_load_globals",
           "mk_load_weights",
           "mk_decode_step", "mk_set_mode", "mk_set_task_trace", "mk_set_routing_trace", "mk_set_wait_limit",
           "mk_set_debug_poison",
           "mk_set_schedule_options", "mk_set_placement_seed", "mk_decode_step_noalloc",
           "mk_service_create", "mk_service_pause", "mk_service_resume", "mk_service_alloc_pages",
           "mk_service_admit", "mk_service_evict", "mk_service_stats", "mk_service_last_error",
           "mk_service_destroy",
           "mk_sync_status", "mk_last_error", "mk_destroy", "mk_kv_cache", "mk_stream_read",
           "mk_litmus_message_passing",
           "mk_schedule_info_get", "mk_schedule_export", "mk_schedule_simulate", "mk_schedule_check",
           "mk_debug_read")


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class MkConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts",
                                              "top_k", "expert_ffn", "vocab", "n_layers")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("page_size", "window", "full_every", "max_batch", "max_seq_len",
                                      "max_pages_per_seq", "n_pages", "mode", "dense", "ffn_fp8")]


TOKEN_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32)


class MkServiceConfig(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("page0", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("on_token", TOKEN_FN), ("user", ctypes.c_void_p), ("stream", ctypes.c_void_p)]


class MkServiceInfo(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("tokens", ctypes.c_int64), ("active", ctypes.c_int32),
                ("free_pages", ctypes.c_int32), ("parked", ctypes.c_int32), ("status", ctypes.c_int32)]


class MkScheduleInfo(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int32), ("max_tasks_per_cu", ctypes.c_int32),
                ("n_counters", ctypes.c_int32), ("n_cus", ctypes.c_int32),
                ("weight_bytes_per_step", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run moe_persistent_decode_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64
    H = ctypes.c_void_p
    lib.mk_create.argtypes = [ctypes.POINTER(MkConfig), P, S, I, ctypes.POINTER(H)]
    lib.mk_create_host_only.argtypes = [ctypes.POINTER(MkConfig), I, ctypes.POINTER(H)]
    lib.mk_load_layer.argtypes = [H, I, P, P, P, P, P, P, P, P]
    lib.mk_load_layer_dense.argtypes = [H, I, P, P, P, P, P, P, P, P]
    lib.mk_load_globals.argtypes = [H, P, P, P, P]
    lib.mk_load_ffn_fp8.argtypes = [H, I, P, P, P, P, P, P, P]
    lib.mk_load_weights.argtypes = [H, P, P]
    lib.mk_decode_step.argtypes = [H, I, P, P, P, I, P, P, ctypes.c_uint32, P]
    lib.mk_decode_step_noalloc.argtypes = [H, I, P, P, P, I, P, P, ctypes.c_uint32, P]
    lib.mk_set_routing_trace.argtypes = [H, P]
    lib.mk_set_wait_limit.argtypes = [H, ctypes.c_uint32]
    lib.mk_set_debug_poison.argtypes = [H, I]
    lib.mk_set_placement_seed.argtypes = [H, ctypes.c_uint64]
    lib.mk_schedule_check.argtypes = [H, I, I, ctypes.c_uint32, P, S]
    lib.mk_set_schedule_options.argtypes = [H, I, I]
    lib.mk_kv_cache.argtypes = [H, I, ctypes.POINTER(P), ctypes.POINTER(S)]
    lib.mk_stream_read.argtypes = [P, S, P]
    lib.mk_litmus_message_passing.argtypes = [I, I, I, I, ctypes.POINTER(ctypes.c_uint32),
                                              ctypes.POINTER(ctypes.c_uint32)]
    lib.mk_set_mode.argtypes = [H, I]
    lib.mk_set_task_trace.argtypes = [H, P, S]
    lib.mk_debug_read.argtypes = [H, ctypes.c_char_p, P, S]
    lib.mk_sync_status.argtypes = [H, P]
    lib.mk_last_error.argtypes = [H]
    lib.mk_last_error.restype = ctypes.c_char_p
    lib.mk_destroy.argtypes = [H]
    lib.mk_destroy.restype = None
    lib.mk_schedule_info_get.argtypes = [H, I, I, ctypes.POINTER(MkScheduleInfo)]
    lib.mk_schedule_export.argtypes = [H, I, I, P, P]
    lib.mk_schedule_simulate.argtypes = [H, I, I, P, U64, ctypes.c_int32, ctypes.c_char_p, S]
    lib.mk_service_create.argtypes = [H, ctypes.POINTER(MkServiceConfig), ctypes.POINTER(H)]
    lib.mk_service_pause.argtypes = [H]
    lib.mk_service_resume.argtypes = [H]
    lib.mk_service_alloc_pages.argtypes = [H, ctypes.c_int32, P]
    lib.mk_service_admit.argtypes = [H, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32]
    lib.mk_service_evict.argtypes = [H, ctypes.c_int64]
    lib.mk_service_stats.argtypes = [H, ctypes.POINTER(MkServiceInfo)]
    lib.mk_service_last_error.argtypes = [H]
    lib.mk_service_last_error.restype = ctypes.c_char_p
    lib.mk_service_destroy.argtypes = [H]
    lib.mk_service_destroy.restype = None
    for name in EXPORTS:
        if name not in ("mk_last_error", "mk_destroy", "mk_service_last_error", "mk_service_destroy"):
            getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def stream_read(buf, stream=None) -> None:
    """mk_stream_read: read a device tensor once (the streaming-read ceiling
    diagnostic; also evicts the last-level cache when larger than it)."""
    nbytes = buf.numel() * buf.element_size()
    st = lib.mk_stream_read(_ptr(buf), nbytes, _stream_ptr(stream))
    if st != 0:
        raise MkError(st, lib.mk_last_error(None).decode())


def litmus_message_passing(pairs: int, rounds: int, coherent=True, device: int = 0):
    """mk_litmus_message_passing: (stale reads, timeouts) over `pairs` workgroup
    pairs on different XCDs passing `rounds` messages each; coherent: True,
    False (plain accesses) or "tagged" (the tagged-word hand-off)."""
    mode = 2 if coherent == "tagged" else (1 if coherent else 0)
    stale, timeouts = ctypes.c_uint32(0), ctypes.c_uint32(0)
    st = lib.mk_litmus_message_passing(device, pairs, rounds, mode, ctypes.byref(stale), ctypes.byref(timeouts))
    if st != 0:
        raise MkError(st, lib.mk_last_error(None).decode())
    return stale.value, timeouts.value


def make_config(model, max_batch: int, max_seq_len: int, n_pages: int, max_pages_per_seq: int,
                mode: int = MODE_MEGAKERNEL, ffn_fp8: bool = False) -> MkConfig:
    """MkConfig from a model-shape object (fields as in mkinputs.configs.ModelConfig)."""
    return MkConfig(hidden=model.hidden, n_q_heads=model.n_q_heads, n_kv_heads=model.n_kv_heads,
                    head_dim=model.head_dim, n_experts=model.n_experts, top_k=model.top_k,
                    expert_ffn=model.expert_ffn, vocab=model.vocab, n_layers=model.n_layers,
                    rope_theta=model.rope_theta, rms_eps=model.eps, page_size=model.page_size,
                    window=model.window, full_every=model.full_every, max_batch=max_batch,
                    max_seq_len=max_seq_len, max_pages_per_seq=max_pages_per_seq, n_pages=n_pages,
                    mode=mode, dense=1 if getattr(model, "dense", False) else 0, ffn_fp8=1 if ffn_fp8 else 0)


class Decoder:
    """One mk_handle. `kv_pool` is a caller-owned device bf16 tensor in the
    pool layout of include/mk.h (it must outlive the decoder), or None: the
    library allocates the pool (kv_cache gives each layer's address)."""

    def __init__(self, cfg: MkConfig, kv_pool=None, device: int = 0, host_only_cus: int = 0):
        self._h = ctypes.c_void_p()
        self.cfg = cfg
        self.kv_pool = kv_pool
        if host_only_cus:
            st = lib.mk_create_host_only(ctypes.byref(cfg), host_only_cus, ctypes.byref(self._h))
        else:
            nbytes = 0 if kv_pool is None else kv_pool.numel() * kv_pool.element_size()
            st = lib.mk_create(ctypes.byref(cfg), _ptr(kv_pool), nbytes, device, ctypes.byref(self._h))
        if st != MK_OK:
            raise MkError(st, lib.mk_last_error(None).decode())

    def _check(self, st: int):
        if st != MK_OK:
            raise MkError(st, lib.mk_last_error(self._h).decode())

    def close(self):
        if self._h:
            lib.mk_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- weights
    def load_layer(self, layer: int, gamma, wqkv, wo, wr, wg, wu, wd, stream=None):
        """A layer's tensors in the order of mk_load_layer; for a dense model
        (mk_load_layer_dense) the fourth is gamma2, the FFN's norm gain."""
        fn = lib.mk_load_layer_dense if self.cfg.dense else lib.mk_load_layer
        self._check(fn(self._h, layer, _ptr(gamma), _ptr(wqkv), _ptr(wo), _ptr(wr), _ptr(wg), _ptr(wu), _ptr(wd),
                       _stream_ptr(stream)))

    def load_ffn_fp8(self, layer: int, wg8, wu8, wd8, sg, su, sd, stream=None):
        """A layer's FP8 feed-forward codes (uint8) and scales (float32), in the
        order of mk_load_ffn_fp8."""
        self._check(lib.mk_load_ffn_fp8(self._h, layer, _ptr(wg8), _ptr(wu8), _ptr(wd8), _ptr(sg), _ptr(su),
                                        _ptr(sd), _stream_ptr(stream)))

    def load_globals(self, emb, gamma_f, wlm, stream=None):
        self._check(lib.mk_load_globals(self._h, _ptr(emb), _ptr(gamma_f), _ptr(wlm), _stream_ptr(stream)))

    def load_weights(self, w: Dict[str, "object"], stream=None):
        """Load canonical tensors named emb, gamma_f, wlm, gamma.{l}, wqkv.{l}, ..."""
        self.load_globals(w["emb"], w["gamma_f"], w["wlm"], stream)
        fp8 = bool(self.cfg.ffn_fp8)
        for l in range(self.cfg.n_layers):
            fourth = w[f"gamma2.{l}"] if self.cfg.dense else w[f"wr.{l}"]
            ffn = (None, None, None) if fp8 else (w[f"wg.{l}"], w[f"wu.{l}"], w[f"wd.{l}"])
            self.load_layer(l, w[f"gamma.{l}"], w[f"wqkv.{l}"], w[f"wo.{l}"], fourth, *ffn, stream)
            if fp8:
                self.load_ffn_fp8(l, *(w[f"{k}.{l}"] for k in ("wg8", "wu8", "wd8", "sg", "su", "sd")), stream)

    # ---- decode
    def step(self, tokens, block_tables, seq_lens, max_seq_len_hint: int, logits, next_tokens=None,
             advance: bool = False, stream=None):
        self._check(lib.mk_decode_step(self._h, tokens.shape[0], _ptr(tokens), _ptr(block_tables),
                                       _ptr(seq_lens), int(max_seq_len_hint), _ptr(logits), _ptr(next_tokens),
                                       STEP_ADVANCE if advance else 0, _stream_ptr(stream)))

    def step_noalloc(self, tokens, block_tables, seq_lens, max_seq_len_hint: int, logits, next_tokens=None,
                     advance: bool = False, stream=None):
        """The allocation-free step (static scratch; the schedule must be cached)."""
        self._check(lib.mk_decode_step_noalloc(self._h, tokens.shape[0], _ptr(tokens), _ptr(block_tables),
                                               _ptr(seq_lens), int(max_seq_len_hint), _ptr(logits),
                                               _ptr(next_tokens), STEP_ADVANCE if advance else 0,
                                               _stream_ptr(stream)))

    def set_mode(self, mode: int):
        self._check(lib.mk_set_mode(self._h, mode))

    def set_task_trace(self, trace, n_records: int = 0):
        self._check(lib.mk_set_task_trace(self._h, _ptr(trace), n_records))

    def set_routing_trace(self, trace):
        self._check(lib.mk_set_routing_trace(self._h, _ptr(trace)))

    def set_schedule_options(self, wave_order: int = 0, placement: int = 0):
        """Wave order (ORDER_*) and placement (PLACE_*) of later steps' schedules."""
        self._check(lib.mk_set_schedule_options(self._h, int(wave_order), int(placement)))

    def set_placement_seed(self, seed: int):
        """The seed of PLACE_RANDOM's candidate placement."""
        self._check(lib.mk_set_placement_seed(self._h, ctypes.c_uint64(int(seed))))

    def set_wait_limit(self, microseconds: int):
        self._check(lib.mk_set_wait_limit(self._h, int(microseconds)))

    def set_debug_poison(self, on: bool):
        """Fill the step's scratch with NaN before each step (read-before-write check)."""
        self._check(lib.mk_set_debug_poison(self._h, 1 if on else 0))

    def kv_cache(self, layer: int):
        """(device address, bytes) of layer `layer`'s part of the KV pool."""
        base, n = ctypes.c_void_p(), ctypes.c_size_t()
        self._check(lib.mk_kv_cache(self._h, layer, ctypes.byref(base), ctypes.byref(n)))
        return base.value, n.value

    def debug_read(self, name: str, shape, dtype="float32"):
        import numpy as np
        a = np.zeros(shape, dtype=dtype)
        self._check(lib.mk_debug_read(self._h, name.encode(), a.ctypes.data, a.nbytes))
        return a

    def sync(self, stream=None):
        self._check(lib.mk_sync_status(self._h, _stream_ptr(stream)))

    # ---- schedule (host only)
    def schedule_info(self, batch: int, hint: int) -> MkScheduleInfo:
        info = MkScheduleInfo()
        self._check(lib.mk_schedule_info_get(self._h, batch, hint, ctypes.byref(info)))
        return info

    def schedule_export(self, batch: int, hint: int):
        import numpy as np
        info = self.schedule_info(batch, hint)
        tasks = np.zeros((info.n_tasks, 32), dtype=np.int32)
        off = np.zeros(info.n_cus + 1, dtype=np.int32)
        self._check(lib.mk_schedule_export(self._h, batch, hint, tasks.ctypes.data, off.ctypes.data))
        return tasks, off

    def check_hazards(self, batch: int, hint: int, flags: int = 0):
        """mk_schedule_check: (status, report) of the read-before-arrive check."""
        buf = ctypes.create_string_buffer(2048)
        st = lib.mk_schedule_check(self._h, batch, hint, ctypes.c_uint32(flags), buf, 2048)
        return st, buf.value.decode()

    def simulate(self, batch: int, hint: int, n_active, seed: int = 0, corrupt_task: int = -1):
        import numpy as np
        na = np.ascontiguousarray(np.asarray(n_active, dtype=np.int32))
        buf = ctypes.create_string_buffer(256)
        st = lib.mk_schedule_simulate(self._h, batch, hint, na.ctypes.data, seed, corrupt_task, buf, 256)
        return st, buf.value.decode()


class DecodeService:
    """The host decode service (mk_service_*): a native thread decoding the
    admitted requests step after step on `decoder`, streaming greedy tokens.
    Tokens arrive through a callback into `tokens` (request id -> list) and
    `status` (request id -> 1 finished / -1 failed). It starts paused: admit
    requests (with pages from alloc_pages), then resume."""

    def __init__(self, decoder: Decoder, max_batch: int, page0: int, n_pages: int, stream=None):
        import threading
        self.decoder = decoder
        self.tokens: Dict[int, list] = {}
        self.status: Dict[int, int] = {}
        self._lock = threading.Lock()
        self._cb = TOKEN_FN(self._on_token)  # kept alive with the service
        cfg = MkServiceConfig(max_batch=max_batch, page0=page0, n_pages=n_pages, on_token=self._cb, user=None,
                              stream=_ptr_or_none(stream))
        self._s = ctypes.c_void_p()
        st = lib.mk_service_create(decoder._h, ctypes.byref(cfg), ctypes.byref(self._s))
        if st != MK_OK:
            raise MkError(st, "mk_service_create")

    def _on_token(self, user, request_id, token, status):
        with self._lock:
            self.tokens.setdefault(int(request_id), []).append(int(token))
            if status != 0:
                self.status[int(request_id)] = int(status)

    def _check(self, st: int):
        if st != MK_OK:
            raise MkError(st, lib.mk_service_last_error(self._s).decode())

    def pause(self):
        self._check(lib.mk_service_pause(self._s))

    def resume(self):
        self._check(lib.mk_service_resume(self._s))

    def alloc_pages(self, n: int):
        import numpy as np
        a = np.zeros(max(n, 1), dtype=np.int32)
        self._check(lib.mk_service_alloc_pages(self._s, n, a.ctypes.data))
        return a[:n].tolist()

    def admit(self, request_id: int, first_token: int, context_len: int, pages, max_new_tokens: int,
              stop_token: int = -1):
        import numpy as np
        a = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
        self._check(lib.mk_service_admit(self._s, request_id, first_token, context_len,
                                         a.ctypes.data if a.size else None, a.size, max_new_tokens, stop_token))

    def evict(self, request_id: int):
        self._check(lib.mk_service_evict(self._s, request_id))

    def stats(self) -> MkServiceInfo:
        info = MkServiceInfo()
        self._check(lib.mk_service_stats(self._s, ctypes.byref(info)))
        return info

    def snapshot(self):
        with self._lock:
            return {k: list(v) for k, v in self.tokens.items()}, dict(self.status)

    def close(self):
        if self._s:
            lib.mk_service_destroy(self._s)
            self._s = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr_or_none(stream):
    if stream is None:
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream
