"""Oracle for the batch-1 decode path: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  It holds:
  * ``oracle.cpp``  a plain double-precision C++ decoder step with its own
    int8/int4 quantisers (built to liboracle.so with g++, no HIP);
  * ``validator.py`` a brute-force reference of the schedule safety gate;
  * ``sim.py``      an abstract-machine simulator of the per-CU queue walk.
It shares no code with the product package.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

WFMT = {"bf16": 0, "int8": 1, "int4": 2}


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "max_ctx")] + [
        ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
        ("tied", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("act_bf16", ctypes.c_int32)]


def build():
    src = os.path.join(_HERE, "oracle.cpp")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["g++", "-O2", "-fopenmp", "-std=c++17", "-shared", "-fPIC",
                           "-ffp-contract=off", "-o", tmp, src])
    os.replace(tmp, _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        p, i32, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        sig = {
            "orc_bf16_to_double": ([ctypes.c_uint16], d),
            "orc_round_bf16": ([d], ctypes.c_uint16),
            "orc_f16_to_double": ([ctypes.c_uint16], d),
            "orc_f16_from_float": ([ctypes.c_float], ctypes.c_uint16),
            "orc_rmsnorm": ([p, p, i32, d, p], None),
            "orc_rope": ([p, i32, i32, d], None),
            "orc_silu": ([d], d),
            "orc_attention_head": ([p, p, p, i32, i32, p], None),
            "orc_gemv_bf16": ([p, i32, i32, p, p], None),
            "orc_gemv_int8": ([p, p, i32, i32, p, p], None),
            "orc_gemv_int4": ([p, p, p, i32, i32, p, p], None),
            "orc_quant_int8": ([p, i32, i32, p, p], None),
            "orc_quant_int4": ([p, i32, i32, p, p, p], None),
            "orc_model_new": ([ctypes.POINTER(OrcConfig), p], p),
            "orc_model_free": ([p], None),
            "orc_step": ([p, p, i32, i32, p], i32),
            "orc_set_jitter": ([d, ctypes.c_uint64], None),
            "orc_model_quant": ([p, i32, p, p, p], i32),
            "orc_set_threads": ([i32], None),
            "orc_get_threads": ([], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data if a is not None else None


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------- scalars --

def bf16_to_float(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v):
    return int(lib().orc_round_bf16(float(v)))


def f16_to_float(h):
    return float(lib().orc_f16_to_double(int(h)))


def f16_from_float(f):
    return int(lib().orc_f16_from_float(float(f)))


# -------------------------------------------------------------- operators --

def rmsnorm(x, g_bits, eps):
    x = _f64(x)
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(out))
    return out


def rope(v, pos, theta):
    v = _f64(v).copy()
    lib().orc_rope(_ptr(v), v.size, pos, theta)
    return v


def silu(z):
    return float(lib().orc_silu(float(z)))


def attention_head(q, K_bits, V_bits):
    q = _f64(q)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    n_pos, hd = K.shape
    o = np.empty(hd)
    lib().orc_attention_head(_ptr(q), _ptr(K), _ptr(V), hd, n_pos, _ptr(o))
    return o


def gemv_bf16(W_bits, x):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = _f64(x)
    y = np.empty(W.shape[0])
    lib().orc_gemv_bf16(_ptr(W), W.shape[0], W.shape[1], _ptr(x), _ptr(y))
    return y


def gemv_int8(q, s, x):
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    x = _f64(x)
    y = np.empty(q.shape[0])
    lib().orc_gemv_int8(_ptr(q), _ptr(s), q.shape[0], q.shape[1], _ptr(x), _ptr(y))
    return y


def gemv_int4(packed, scale, zero, cols, x):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    zero = np.ascontiguousarray(zero, dtype=np.uint16)
    x = _f64(x)
    rows = packed.shape[0]
    y = np.empty(rows)
    lib().orc_gemv_int4(_ptr(packed), _ptr(scale), _ptr(zero), rows, cols, _ptr(x), _ptr(y))
    return y


def quant_int8(W_bits):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    R, C = W.shape
    q = np.empty((R, C), dtype=np.int8)
    s = np.empty(R, dtype=np.float32)
    lib().orc_quant_int8(_ptr(W), R, C, _ptr(q), _ptr(s))
    return q, s


def quant_int4(W_bits):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    R, C = W.shape
    assert C % 128 == 0
    packed = np.zeros((R, C // 2), dtype=np.uint8)
    scale = np.empty((R, C // 128), dtype=np.uint16)
    zero = np.empty((R, C // 128), dtype=np.uint16)
    lib().orc_quant_int4(_ptr(W), R, C, _ptr(packed), _ptr(scale), _ptr(zero))
    return packed, scale, zero


# ------------------------------------------------------------------ model --

def config_of(wl):
    return OrcConfig(wl.n_layers, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.ffn,
                     wl.vocab, wl.max_ctx, wl.rms_eps, wl.rope_theta, int(wl.tied),
                     WFMT[wl.wfmt], int(wl.act_bf16))


def set_jitter(eps, seed=0):
    """Conditioning probe: multiply each value by 1 + eps*r (r uniform in
    [-1, 1)) right before every bf16 rounding decision of the decoder
    (activations of act_bf16 models, KV rows).  eps = 0 turns it off."""
    lib().orc_set_jitter(float(eps), int(seed))


class Model:
    """Oracle decoder over borrowed canonical bf16 tensors (dict id -> array)."""

    def __init__(self, wl, weights, threads=0):
        self.wl = wl
        self._keep = {k: np.ascontiguousarray(v, dtype=np.uint16) for k, v in weights.items()}
        n = 3 + 9 * wl.n_layers
        self._ptrs = (ctypes.c_void_p * n)()
        for k, v in self._keep.items():
            self._ptrs[k] = v.ctypes.data
        self._cfg = config_of(wl)
        if threads:
            lib().orc_set_threads(threads)
        self._h = lib().orc_model_new(ctypes.byref(self._cfg), self._ptrs)
        if not self._h:
            raise ValueError("oracle: unsupported model shape")

    def new_kv(self):
        wl = self.wl
        return np.zeros((wl.n_layers, 2, wl.n_kv_heads, wl.max_ctx, wl.head_dim), dtype=np.uint16)

    def step(self, kv, token, pos):
        assert kv.dtype == np.uint16 and kv.flags.c_contiguous
        logits = np.empty(self.wl.vocab)
        rc = lib().orc_step(self._h, kv.ctypes.data, int(token), int(pos), logits.ctypes.data)
        if rc != 0:
            raise ValueError("oracle step: bad token/pos")
        return logits

    def quantised(self, canon_id):
        q, s, z = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        rc = lib().orc_model_quant(self._h, canon_id, ctypes.byref(q), ctypes.byref(s),
                                   ctypes.byref(z))
        if rc != 0:
            raise KeyError(canon_id)
        return q.value, s.value, z.value

    def close(self):
        if self._h:
            lib().orc_model_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def threads():
    return int(lib().orc_get_threads())
