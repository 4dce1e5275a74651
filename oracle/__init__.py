"""Python access to the fp64 CPU oracle (``liboracle.so``, built from plain C by gcc).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
bench's CPU-baseline leg.  The product path never imports it.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "moe_oracle.c")]

F32, BF16, MXFP4, MXFP4_A8 = 0, 1, 2, 3

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (ISO C99, so no FMA contraction)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           *SOURCES, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or any(os.path.getmtime(s) > os.path.getmtime(LIB_PATH) for s in SOURCES):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.ora_bf16_value.restype = ctypes.c_double
        L.ora_bf16_value.argtypes = [ctypes.c_uint16]
        L.ora_e2m1_value.restype = ctypes.c_double
        L.ora_e2m1_value.argtypes = [ctypes.c_uint8]
        L.ora_e8m0_value.restype = ctypes.c_double
        L.ora_e8m0_value.argtypes = [ctypes.c_uint8]
        L.ora_e4m3_value.restype = ctypes.c_double
        L.ora_e4m3_value.argtypes = [ctypes.c_uint8]
        L.ora_mx8_quantize.argtypes = [P, i, i, P, P]
        L.ora_expert_bytes.restype = ctypes.c_size_t
        L.ora_expert_bytes.argtypes = [i, i, i]
        L.ora_decode_expert.argtypes = [i, P, i, i, P, P, P]
        L.ora_decode_x.argtypes = [i, P, i, i, P]
        L.ora_route_topk.argtypes = [P, i, i, i, P, P, P]
        L.ora_permute.argtypes = [P, i, i, i, P, P, P, P]
        L.ora_expert_ffn.restype = None
        L.ora_expert_ffn.argtypes = [P, P, P, i, i, P, P]
        L.ora_combine.restype = None
        L.ora_combine.argtypes = [P, P, P, i, i, i, P]
        L.ora_layer.argtypes = [i, P, P, i, P, P, i, i, i, i, i, P, P, P, P, P]
        L.ora_expert_rows.argtypes = [i, P, i, i, P, i, P, i, P]
        L.ora_lru_new.restype = P
        L.ora_lru_new.argtypes = [i, i, i]
        L.ora_lru_free.restype = None
        L.ora_lru_free.argtypes = [P]
        L.ora_lru_step.argtypes = [P, i, P, P, P, P, P, P, P, P]
        L.ora_lru_step_split.argtypes = [P, i, P, i, i, P, P, P, P, P, P, P, P, P, P]
        L.ora_lru_state.restype = None
        L.ora_lru_state.argtypes = [P, P, P]
        L.ora_router_logits.restype = i
        L.ora_router_logits.argtypes = [P, P, i, i, i, P]
        L.ora_lru_resize.restype = i
        L.ora_lru_resize.argtypes = [P, i, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with {rc}")


def bf16_value(bits: int) -> float:
    return lib().ora_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return lib().ora_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return float(lib().ora_e4m3_value(code))


def mx8_quantize(x_bits):
    """bf16 bits [T][H] -> (E4M3 codes uint8 [T][H], E8M0 scales uint8 [T][H/32])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    codes = np.empty((T, H), np.uint8)
    scales = np.empty((T, H // 32), np.uint8)
    _check(lib().ora_mx8_quantize(_p(x), T, H, _p(codes), _p(scales)), "mx8_quantize")
    return codes, scales


def e8m0_value(code: int) -> float:
    return lib().ora_e8m0_value(int(code))


def expert_bytes(dtype, H, I) -> int:
    return int(lib().ora_expert_bytes(dtype, H, I))


def decode_expert(dtype, slot_bytes, H, I):
    slot_bytes = np.ascontiguousarray(slot_bytes, dtype=np.uint8)
    wg = np.empty((I, H)); wu = np.empty((I, H)); wd = np.empty((H, I))
    _check(lib().ora_decode_expert(dtype, _p(slot_bytes), H, I, _p(wg), _p(wu), _p(wd)), "decode_expert")
    return wg, wu, wd


def decode_x(dtype, x, T, H):
    x = np.ascontiguousarray(x)
    out = np.empty((T, H))
    _check(lib().ora_decode_x(dtype, _p(x), T, H, _p(out)), "decode_x")
    return out


def route_topk(logits, k):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w32 = np.empty((T, k), dtype=np.float32)
    w64 = np.empty((T, k), dtype=np.float64)
    _check(lib().ora_route_topk(_p(logits), T, E, k, _p(ids), _p(w32), _p(w64)), "route_topk")
    return ids, w32, w64


def router_logits(x_bits, wr_bits):
    """x [T][H], wr [E][H] bf16 bits (uint16) -> fp64 logits [T][E]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wr = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E))
    _check(lib().ora_router_logits(_p(x), _p(wr), T, H, E, _p(out)), "router_logits")
    return out


def permute(ids, E):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_rows = np.empty(T * k, dtype=np.int32)
    inv_rows = np.empty(T * k, dtype=np.int32)
    _check(lib().ora_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_rows), _p(inv_rows)), "permute")
    return counts, offsets, sorted_rows, inv_rows


def expert_ffn(wg, wu, wd, x):
    wg = np.ascontiguousarray(wg, dtype=np.float64)
    wu = np.ascontiguousarray(wu, dtype=np.float64)
    wd = np.ascontiguousarray(wd, dtype=np.float64)
    x = np.ascontiguousarray(x, dtype=np.float64)
    I, H = wg.shape
    o = np.empty(H)
    lib().ora_expert_ffn(_p(wg), _p(wu), _p(wd), H, I, _p(x), _p(o))
    return o


def combine(rows, w, shared=None):
    rows = np.ascontiguousarray(rows, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = w.shape
    H = rows.shape[-1]
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.float64)
    y = np.empty((T, H))
    lib().ora_combine(_p(rows), _p(w), _p(sh), T, k, H, _p(y))
    return y


def expert_rows(dtype, slot_bytes, H, I, x, tokens):
    slot_bytes = np.ascontiguousarray(slot_bytes, dtype=np.uint8)
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    o = np.empty((tokens.size, H))
    _check(lib().ora_expert_rows(dtype, _p(slot_bytes), H, I, _p(x), T, _p(tokens), tokens.size, _p(o)),
           "expert_rows")
    return o


def layer(dtype, experts, x, logits, k, H, I, shared=None, I_shared=0):
    """experts: uint8 [E][expert_bytes] (or a list of per-expert byte arrays)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    bufs = [np.ascontiguousarray(experts[e], dtype=np.uint8) for e in range(E)]
    ptrs = (ctypes.c_void_p * E)(*[b.ctypes.data for b in bufs])
    x = np.ascontiguousarray(x)
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint8)
    y = np.empty((T, H))
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k))
    rows = np.empty((T * k, H))
    shared_out = np.empty((T, H)) if shared is not None else None
    _check(lib().ora_layer(dtype, ctypes.cast(ptrs, ctypes.c_void_p), _p(sh), I_shared, _p(x), _p(logits),
                           T, H, I, E, k, _p(y), _p(ids), _p(w), _p(rows), _p(shared_out)), "layer")
    return dict(y=y, ids=ids, w=w, rows=rows, shared_out=shared_out)


class LRU:
    """The oracle's global LRU expert cache."""

    def __init__(self, n_slots, n_layers, n_experts):
        self.S, self.L, self.E = n_slots, n_layers, n_experts
        self._h = lib().ora_lru_new(n_slots, n_layers, n_experts)
        if not self._h:
            raise OracleError("ora_lru_new failed")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().ora_lru_free(self._h)
            self._h = None

    def step(self, layer, counts, fill=None):
        """One (step, layer); fill = (num, den) splits the misses (the first
        floor(m num / den + 1/2) filled, the rest computed in place)."""
        counts = np.ascontiguousarray(counts, dtype=np.int32)
        E = self.E
        n = ctypes.c_int(0)
        ni = ctypes.c_int(0)
        ex = np.empty(E, np.int32); hit = np.empty(E, np.int32); slot = np.empty(E, np.int32)
        wave = np.empty(E, np.int32); cold = np.empty(E, np.int32); ev = np.empty(E, np.int64)
        inp = np.empty(E, np.int32); inp_cold = np.empty(E, np.int32)
        if fill is None:
            nw = lib().ora_lru_step(self._h, layer, _p(counts), ctypes.byref(n), _p(ex), _p(hit), _p(slot),
                                    _p(wave), _p(cold), _p(ev))
        else:
            nw = lib().ora_lru_step_split(self._h, layer, _p(counts), int(fill[0]), int(fill[1]), ctypes.byref(n),
                                          _p(ex), _p(hit), _p(slot), _p(wave), _p(cold), _p(ev), ctypes.byref(ni),
                                          _p(inp), _p(inp_cold))
        if nw < 0:
            raise OracleError(f"ora_lru_step failed with {nw}")
        m = n.value
        return dict(expert=ex[:m].copy(), hit=hit[:m].copy(), slot=slot[:m].copy(), wave=wave[:m].copy(),
                    cold=cold[:m].copy(), evicted=ev[:m].copy(), n_waves=nw,
                    inplace=inp[:ni.value].copy(), inplace_cold=inp_cold[:ni.value].copy())

    def state(self):
        keys = np.empty(self.S, np.int64)
        ticks = np.empty(self.S, np.int64)
        lib().ora_lru_state(self._h, _p(keys), _p(ticks))
        return keys, ticks

    def resize(self, new_S):
        """Elastic resize; returns moved_from [new_S] (old slot per new slot, -1 empty)."""
        moved = np.empty(new_S, np.int32)
        rc = lib().ora_lru_resize(self._h, new_S, _p(moved))
        if rc != 0:
            raise OracleError(f"ora_lru_resize failed with {rc}")
        self.S = new_S
        return moved
