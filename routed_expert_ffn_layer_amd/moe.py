"""Thin ctypes binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (device memory and streams are all
torch is used for); the default stream is torch's current stream.  The library
must be built (routed_expert_ffn_layer_amd/build.py); there is no fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY, MOE_EHIP, MOE_ENOMEM, MOE_ESTATE = range(7)
MOE_F32, MOE_BF16, MOE_MXFP4, MOE_MXFP4_A8 = 0, 1, 2, 3

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("n_experts", ctypes.c_int), ("n_slots", ctypes.c_int),
                ("expert_bytes", ctypes.c_size_t), ("slot_stride", ctypes.c_size_t),
                ("slot_pool", ctypes.c_void_p), ("host_pool_host", ctypes.c_void_p),
                ("host_expert_ptrs_host", ctypes.c_void_p), ("fill_stream", ctypes.c_void_p)]


class CacheStats(ctypes.Structure):
    _fields_ = [("accesses", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("cold_misses", ctypes.c_int64), ("fill_bytes", ctypes.c_int64), ("n_waves", ctypes.c_int32),
                ("wave_accesses", ctypes.c_int32), ("inplace", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Fill(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("layer", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("wave", ctypes.c_int32)]


class LayerStreamDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("layer_bytes", ctypes.c_size_t),
                ("host_layers_host", ctypes.c_void_p), ("host_layer_ptrs_host", ctypes.c_void_p),
                ("banks", ctypes.c_void_p * 2), ("fill_stream", ctypes.c_void_p)]


EXPORTS = ["moe_abi_version", "moe_status_str", "moe_last_error", "moe_expert_bytes", "moe_route_topk",
           "moe_permute", "moe_cache_create", "moe_cache_destroy", "moe_cache_lookup_fill",
           "moe_cache_lookup_host", "moe_cache_state", "moe_cache_inject_fill_failure",
           "moe_cache_lookup_fill_split", "moe_cache_wait_fills", "moe_cache_set_fill_fraction",
           "moe_cache_lookup_fill_inplace", "moe_cache_step_inplace", "moe_grouped_ffn_addr", "moe_route", "moe_cache_resize", "moe_route_project",
           "moe_grouped_ffn_workspace", "moe_grouped_ffn_kind", "moe_mx8_quantize", "moe_grouped_ffn", "moe_grouped_ffn_gate_up", "moe_grouped_ffn_down", "moe_grouped_ffn_noalloc",
           "moe_combine", "moe_layer_stream_create", "moe_layer_stream_destroy", "moe_layer_stream_fill",
           "moe_layer_stream_acquire", "moe_layer_stream_release"]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with routed_expert_ffn_layer_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_abi_version.restype = i
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [i]
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_expert_bytes.restype = sz
    L.moe_expert_bytes.argtypes = [i, i, i]
    L.moe_route_topk.argtypes = [P, i, i, i, P, P, P]
    L.moe_permute.argtypes = [P, i, i, i, P, P, P, P, P]
    L.moe_route.argtypes = [P, i, i, i, P, P, P, P, P, P, P]
    L.moe_route_project.argtypes = [P, P, i, i, i, i, P, P, P, P, P, P, P, P]
    L.moe_cache_create.argtypes = [ctypes.POINTER(CacheDesc), ctypes.POINTER(P)]
    L.moe_cache_destroy.argtypes = [P]
    L.moe_cache_lookup_fill.argtypes = [P, i, P, i, P, ctypes.POINTER(CacheStats), P]
    L.moe_cache_lookup_host.argtypes = [P, i, P, i, P, P, i, ctypes.POINTER(i), ctypes.POINTER(CacheStats)]
    L.moe_cache_lookup_fill_split.argtypes = [P, i, P, i, P, P, ctypes.POINTER(CacheStats), P]
    L.moe_cache_wait_fills.argtypes = [P, P]
    L.moe_cache_set_fill_fraction.argtypes = [P, i, i]
    L.moe_cache_lookup_fill_inplace.argtypes = [P, i, P, i, P, P, P, ctypes.POINTER(CacheStats), P]
    L.moe_cache_step_inplace.argtypes = [P, P, ctypes.POINTER(i)]
    L.moe_grouped_ffn_addr.argtypes = [i, P, P, i, P, P, P, i, i, i, i, i, P, P, P, sz, P]
    L.moe_cache_resize.argtypes = [P, i, P, sz, P, P]
    L.moe_cache_state.argtypes = [P, P, P]
    L.moe_cache_inject_fill_failure.argtypes = [P, ctypes.c_int64]
    L.moe_grouped_ffn_workspace.restype = sz
    L.moe_grouped_ffn_kind.argtypes = [i, i, i, i, i, i, i]
    L.moe_mx8_quantize.argtypes = [P, i, i, P, P, P]
    L.moe_grouped_ffn_workspace.argtypes = [i, i, i, i, i, i, i]
    ffn_args = [i, P, sz, P, P, i, P, P, P, i, i, i, i, i, P, P, P, sz, P]
    L.moe_grouped_ffn.argtypes = ffn_args
    L.moe_grouped_ffn_gate_up.argtypes = ffn_args
    L.moe_grouped_ffn_down.argtypes = ffn_args
    L.moe_grouped_ffn_noalloc.argtypes = [i, P, sz, P, P, i, P, P, P, i, i, i, i, i, P, P, P]
    L.moe_combine.argtypes = [P, P, P, P, i, i, i, P, i, P]
    L.moe_layer_stream_create.argtypes = [ctypes.POINTER(LayerStreamDesc), ctypes.POINTER(P)]
    L.moe_layer_stream_destroy.argtypes = [P]
    L.moe_layer_stream_fill.argtypes = [P, i, i]
    L.moe_layer_stream_acquire.argtypes = [P, i, P]
    L.moe_layer_stream_release.argtypes = [P, i, P]
    _lib = L
    return L


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def moe_abi_version():
    return lib().moe_abi_version()


def moe_expert_bytes(wdt, H, I):
    return int(lib().moe_expert_bytes(wdt, H, I))


def moe_route_topk(logits, k, topk_ids, topk_w, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_route(logits, k, topk_ids, topk_w, counts, offsets, sorted_rows, inv_rows, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                           _ptr(sorted_rows), _ptr(inv_rows), _stream(stream)))


def moe_route_project(x, w_router, k, logits, topk_ids, topk_w, counts, offsets, sorted_rows, inv_rows,
                      stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    _check(lib().moe_route_project(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(counts), _ptr(offsets), _ptr(sorted_rows), _ptr(inv_rows), _stream(stream)))


def moe_permute(topk_ids, E, counts, offsets, sorted_rows, inv_rows, stream=None):
    T, k = topk_ids.shape
    _check(lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_rows),
                             _ptr(inv_rows), _stream(stream)))


def moe_grouped_ffn_workspace(T, k, E, H, I, I_shared, wdt):
    return int(lib().moe_grouped_ffn_workspace(T, k, E, H, I, I_shared, wdt))


MOE_FFN_WEIGHT_STREAM, MOE_FFN_GROUPED_GEMM = 0, 1


def moe_mx8_quantize(x, codes, scales, stream=None):
    T, H = x.shape
    _check(lib().moe_mx8_quantize(_ptr(x), T, H, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_grouped_ffn_kind(T, k, E, H, I, I_shared, wdt):
    return int(lib().moe_grouped_ffn_kind(T, k, E, H, I, I_shared, wdt))


def _ffn(fn, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets, sorted_rows, T, k, E, H,
         I, out_rows, shared_out, workspace, stream):
    _check(fn(wdt, _ptr(slot_pool), slot_stride, _ptr(slot_of_expert), _ptr(shared_w), I_shared, _ptr(x),
              _ptr(offsets), _ptr(sorted_rows), T, k, E, H, I, _ptr(out_rows), _ptr(shared_out), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_ffn(wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets, sorted_rows, T, k,
                    E, H, I, out_rows, shared_out, workspace, stream=None):
    _ffn(lib().moe_grouped_ffn, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
         sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, stream)


def moe_grouped_ffn_gate_up(wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
                            sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, stream=None):
    _ffn(lib().moe_grouped_ffn_gate_up, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
         sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, stream)


def moe_grouped_ffn_down(wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets, sorted_rows,
                         T, k, E, H, I, out_rows, shared_out, workspace, stream=None):
    _ffn(lib().moe_grouped_ffn_down, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
         sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, stream)


def moe_grouped_ffn_addr(wdt, expert_addr, shared_w, I_shared, x, offsets, sorted_rows, T, k, E, H, I, out_rows,
                         shared_out, workspace, stream=None):
    _check(lib().moe_grouped_ffn_addr(wdt, _ptr(expert_addr), _ptr(shared_w), I_shared, _ptr(x), _ptr(offsets),
                                      _ptr(sorted_rows), T, k, E, H, I, _ptr(out_rows), _ptr(shared_out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_grouped_ffn_noalloc(wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets, sorted_rows,
                            T, k, E, H, I, out_rows, shared_out, stream=None):
    _check(lib().moe_grouped_ffn_noalloc(wdt, _ptr(slot_pool), slot_stride, _ptr(slot_of_expert), _ptr(shared_w),
                                         I_shared, _ptr(x), _ptr(offsets), _ptr(sorted_rows), T, k, E, H, I,
                                         _ptr(out_rows), _ptr(shared_out), _stream(stream)))


def moe_combine(out_rows, topk_w, inv_rows, shared_out, y, ydt, stream=None):
    T, k = topk_w.shape
    H = y.shape[-1]
    _check(lib().moe_combine(_ptr(out_rows), _ptr(topk_w), _ptr(inv_rows), _ptr(shared_out), T, k, H, _ptr(y), ydt,
                             _stream(stream)))


class MoeCache:
    """Handle of the global-LRU expert-slot cache (moe_cache_*)."""

    def __init__(self, n_layers, n_experts, n_slots, expert_bytes=0, slot_stride=0, slot_pool=None,
                 host_pool=None, host_expert_ptrs=None, fill_stream=None):
        self.n_experts, self.n_slots = n_experts, n_slots
        self._keep = (slot_pool, host_pool, host_expert_ptrs, fill_stream)
        d = CacheDesc(n_layers, n_experts, n_slots, expert_bytes, slot_stride,
                      None if slot_pool is None else slot_pool.data_ptr(),
                      None if host_pool is None else host_pool.data_ptr(),
                      None if host_expert_ptrs is None else ctypes.cast(host_expert_ptrs, ctypes.c_void_p).value,
                      None if fill_stream is None else _stream(fill_stream).value)
        h = ctypes.c_void_p()
        _check(lib().moe_cache_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().moe_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup_fill(self, layer, counts, wave, slot_of_expert, stream=None):
        st = CacheStats()
        _check(lib().moe_cache_lookup_fill(self._h, layer, _ptr(counts), wave, _ptr(slot_of_expert),
                                           ctypes.byref(st), _stream(stream)))
        return st.as_dict()

    def lookup_fill_split(self, layer, counts, wave, slot_hits, slot_misses, stream=None):
        st = CacheStats()
        _check(lib().moe_cache_lookup_fill_split(self._h, layer, _ptr(counts), wave, _ptr(slot_hits),
                                                 _ptr(slot_misses), ctypes.byref(st), _stream(stream)))
        return st.as_dict()

    def resize(self, n_slots, slot_pool=None, slot_stride=0, stream=None):
        """Elastic resize; returns moved_from (numpy int32 [n_slots]).  The handle keeps
        the new pool alive; the old one may be released once `stream` has run the copies."""
        import numpy as np
        moved = np.empty(n_slots, np.int32)
        st = ctypes.c_void_p(0) if slot_pool is None and stream is None else _stream(stream)
        _check(lib().moe_cache_resize(self._h, n_slots, _ptr(slot_pool), slot_stride,
                                      moved.ctypes.data_as(ctypes.c_void_p), st))
        self.n_slots = n_slots
        self._keep = (slot_pool,) + tuple(self._keep[1:])
        return moved

    def wait_fills(self, stream=None):
        _check(lib().moe_cache_wait_fills(self._h, _stream(stream)))

    def set_fill_fraction(self, num, den):
        _check(lib().moe_cache_set_fill_fraction(self._h, num, den))

    def lookup_fill_inplace(self, layer, counts, wave, slot_hits, slot_misses, addr_inplace, stream=None):
        st = CacheStats()
        _check(lib().moe_cache_lookup_fill_inplace(self._h, layer, _ptr(counts), wave, _ptr(slot_hits),
                                                   _ptr(slot_misses), _ptr(addr_inplace), ctypes.byref(st),
                                                   _stream(stream)))
        return st.as_dict()

    def step_inplace(self):
        import numpy as np
        out = np.empty(self.n_experts, np.int32)
        n = ctypes.c_int(0)
        _check(lib().moe_cache_step_inplace(self._h, out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)))
        return out[:n.value].copy()

    def lookup_host(self, layer, counts_host, wave):
        """counts_host: numpy int32 [E] (ignored for wave > 0).  Returns (slot table, fills, stats)."""
        import numpy as np
        table = np.empty(self.n_experts, np.int32)
        fills = (Fill * self.n_slots)()
        nf = ctypes.c_int(0)
        st = CacheStats()
        cp = None
        if counts_host is not None:
            counts_host = np.ascontiguousarray(counts_host, dtype=np.int32)
            cp = counts_host.ctypes.data_as(ctypes.c_void_p)
        _check(lib().moe_cache_lookup_host(self._h, layer, cp, wave, table.ctypes.data_as(ctypes.c_void_p), fills,
                                           self.n_slots, ctypes.byref(nf), ctypes.byref(st)))
        return table, [(f.slot, f.layer, f.expert, f.wave) for f in fills[:nf.value]], st.as_dict()

    def state(self):
        import numpy as np
        keys = np.empty(self.n_slots, np.int64)
        ticks = np.empty(self.n_slots, np.int64)
        _check(lib().moe_cache_state(self._h, keys.ctypes.data_as(ctypes.c_void_p),
                                     ticks.ctypes.data_as(ctypes.c_void_p)))
        return keys, ticks

    def inject_fill_failure(self, n):
        _check(lib().moe_cache_inject_fill_failure(self._h, n))


class LayerStream:
    """Two-bank whole-layer streamer for prefill (moe_layer_stream_*)."""

    def __init__(self, n_layers, layer_bytes, bank0, bank1, fill_stream, host_layers=None, host_layer_ptrs=None):
        self._keep = (bank0, bank1, host_layers, host_layer_ptrs, fill_stream)
        d = LayerStreamDesc()
        d.n_layers = n_layers
        d.layer_bytes = layer_bytes
        d.host_layers_host = None if host_layers is None else host_layers.data_ptr()
        d.host_layer_ptrs_host = None if host_layer_ptrs is None else ctypes.cast(host_layer_ptrs, ctypes.c_void_p).value
        d.banks[0] = bank0.data_ptr()
        d.banks[1] = bank1.data_ptr()
        d.fill_stream = _stream(fill_stream).value
        h = ctypes.c_void_p()
        _check(lib().moe_layer_stream_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            _check(lib().moe_layer_stream_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def fill(self, layer, bank):
        _check(lib().moe_layer_stream_fill(self._h, layer, bank))

    def acquire(self, bank, stream=None):
        _check(lib().moe_layer_stream_acquire(self._h, bank, _stream(stream)))

    def release(self, bank, stream=None):
        _check(lib().moe_layer_stream_release(self._h, bank, _stream(stream)))
