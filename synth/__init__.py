"""Seeded synthetic inputs (weights, tokens, KV prefixes) for the decode path.

This package is the one thing the oracle and the GPU path share: it produces
input bytes and nothing else.  It computes no step of the decoder.  The
generator is defined in ``gen.c`` (SplitMix64 counter stream + Box-Muller,
rounded to bf16).  ``workloads`` names the model shapes and run protocols.
"""
import ctypes
import os
import subprocess

import numpy as np

from .workloads import (CONFIGS, Workload, canonical_tensors, get,  # noqa: F401
                        tensor_shape)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream ids: weights use the canonical tensor id; these are far above any
# tensor id so they never collide with weight streams.
STREAM_TOKENS = 1 << 40
STREAM_KV = (1 << 40) + 1
STREAM_MISC = (1 << 40) + 2

BF16_ONE = 0x3F80


def build():
    """Compile libsynth.so (plain C, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fno-math-errno", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
    os.replace(tmp, _LIB_PATH)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [u64, u64, ctypes.c_double, u64, u64, p]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_mean_bf16.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double, u64, u64, p]
        lib.synth_normal_mean_bf16.restype = None
        lib.synth_tokens.argtypes = [u64, u64, ctypes.c_int64, u64, p]
        lib.synth_tokens.restype = None
        lib.synth_fill_u16.argtypes = [ctypes.c_uint16, u64, p]
        lib.synth_fill_u16.restype = None
        lib.synth_splitmix64.argtypes = [u64]
        lib.synth_splitmix64.restype = u64
        _lib = lib
    return _lib


def splitmix64(x):
    return int(_load().synth_splitmix64(ctypes.c_uint64(x & (2**64 - 1))))


def normal_bf16(seed, stream, n, std=0.02, first=0, out=None):
    """n samples of N(0, std^2) as bf16 bit patterns (uint16)."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    if n:
        _load().synth_normal_bf16(seed, stream, float(std), first, n, out.ctypes.data)
    return out


def normal_mean_bf16(seed, stream, n, mean, std, first=0):
    """n samples of N(mean, std^2) as bf16 bit patterns (uint16)."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_mean_bf16(seed, stream, float(mean), float(std), first, n, out.ctypes.data)
    return out


def fill_bf16(value_bits, n):
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_fill_u16(value_bits, n, out.ctypes.data)
    return out


def tokens(seed, n, vocab, stream=STREAM_TOKENS):
    out = np.empty(n, dtype=np.int32)
    if n:
        _load().synth_tokens(seed, stream, vocab, n, out.ctypes.data)
    return out


GAIN_STD = 0.25  # spread of the optional non-unit RMSNorm gains around 1


def model_weights(wl, seed=1, std=0.02, gains="unit"):
    """Canonical bf16 tensors of a workload, keyed by canonical tensor id.

    Projections and embeddings are N(0, std^2) rounded to bf16.  RMSNorm
    weights are 1.0 (gains="unit"), or with gains="random" N(1, GAIN_STD^2)
    rounded to bf16, drawn from the norm tensor's own stream, so that a
    gain read at the wrong index changes the result.  Tied-embedding models
    have no separate lm_head.
    """
    assert gains in ("unit", "random"), gains
    out = {}
    for tid, name, shape in canonical_tensors(wl):
        n = int(np.prod(shape))
        if name.endswith("norm") and gains == "random":
            out[tid] = random_gains(wl, seed)[tid]
        elif name.endswith("norm"):
            out[tid] = fill_bf16(BF16_ONE, n).reshape(shape)
        else:
            out[tid] = normal_bf16(seed, tid, n, std).reshape(shape)
    return out


def random_gains(wl, seed=1):
    """The non-unit RMSNorm gains of model_weights(gains="random"), keyed by
    canonical tensor id: N(1, GAIN_STD^2) rounded to bf16, each from its
    tensor's own stream.  Replacing the norms of a unit-gain weight set with
    these gives the random-gain weight set without regenerating the rest."""
    out = {}
    for tid, name, shape in canonical_tensors(wl):
        if name.endswith("norm"):
            out[tid] = normal_mean_bf16(seed, tid, int(np.prod(shape)), 1.0, GAIN_STD).reshape(shape)
    return out


def kv_prefix(wl, n_pos, seed=3, std=1.0):
    """A synthetic KV-cache state holding n_pos filled positions.

    Layout [L][2][n_kv][max_ctx][head_dim] bf16 (the cache layout both sides
    use); positions >= n_pos are zero.  Stands in for a prefill when only the
    decode steps after a long prompt are checked.
    """
    L, nkv, hd, mc = wl.n_layers, wl.n_kv_heads, wl.head_dim, wl.max_ctx
    kv = np.zeros((L, 2, nkv, mc, hd), dtype=np.uint16)
    per = n_pos * hd
    block = 0
    for l in range(L):
        for kvsel in range(2):
            for g in range(nkv):
                kv[l, kvsel, g, :n_pos, :] = normal_bf16(
                    seed, STREAM_KV, per, std, first=block * mc * hd).reshape(n_pos, hd)
                block += 1
    return kv
