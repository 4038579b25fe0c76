"""Pins for the oracle: closed forms, invariants, special cases and brute force.

Each test fixes a property the operator definitions force (Llama decoder
operators named by the AutoMegaKernel summary, "Methodology" layer 1, and the
Argus megakernel case study, "Workload and baselines"), so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails at
least one of them.  None of these tests calls the product library.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def f32_to_bf16_bits(a):
    """Float32 -> bf16 by the textbook round-half-even bit trick."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_vals(bits):
    return oracle.bf16_to_float(bits)


# ---------------------------------------------------------------- numbers --

def test_bf16_rounding_points():
    assert oracle.round_bf16(1.0) == 0x3F80
    assert oracle.round_bf16(-2.5) == 0xC020
    assert oracle.round_bf16(1.0 + 2**-8) == 0x3F80          # tie -> even (down)
    assert oracle.round_bf16(1.0 + 3 * 2**-8) == 0x3F82      # tie -> even (up)
    assert oracle.round_bf16(1.0 + 2**-8 + 2**-30) == 0x3F81  # just above the tie
    assert oracle.round_bf16(0.0) == 0 and oracle.round_bf16(-0.0) == 0x8000
    assert oracle.round_bf16(1e39) == 0x7F80
    assert oracle.round_bf16(2.0**-133) == 0x0001            # smallest subnormal
    assert oracle.round_bf16(2.0**-134) == 0x0000            # tie to even zero


def test_bf16_rounding_matches_float32_bit_trick():
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, rng.standard_normal(2000).astype(np.float32) * np.float32(1e-39)])
    want = f32_to_bf16_bits(x)
    got = np.array([oracle.round_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_f16_matches_numpy():
    x = np.concatenate([rng.standard_normal(5000) * 10, rng.standard_normal(2000) * 1e-6,
                        [65504.0, 65519.0, 65520.0, 7e4, 2.0**-24, 2.0**-25, 3 * 2.0**-26]])
    x = x.astype(np.float32)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f16_from_float(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)
    back = np.array([oracle.f16_to_float(int(b)) for b in want])
    assert np.array_equal(back, want.view(np.float16).astype(np.float64))


# -------------------------------------------------------------- operators --

ONES = lambda n: np.full(n, synth.BF16_ONE, dtype=np.uint16)  # noqa: E731


def test_rmsnorm_unit_rms():
    x = rng.standard_normal(4096) * 7.0
    y = oracle.rmsnorm(x, ONES(4096), 1e-5)
    assert abs(math.sqrt(np.mean(y**2)) - 1.0) < 1e-5
    # direction preserved
    assert np.allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), atol=1e-12)


def test_rmsnorm_constant_closed_form_and_gain():
    c, eps = 0.01, 1e-5
    y = oracle.rmsnorm(np.full(64, c), ONES(64), eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)
    g = np.full(64, 0x4000, dtype=np.uint16)  # bf16 2.0
    g[5] = 0xBF80                              # -1.0 on one channel
    y2 = oracle.rmsnorm(np.full(64, c), g, eps)
    assert np.allclose(y2[np.arange(64) != 5], 2 * c / math.sqrt(c * c + eps), rtol=1e-14)
    assert np.isclose(y2[5], -c / math.sqrt(c * c + eps), rtol=1e-14)
    assert np.all(oracle.rmsnorm(np.zeros(8), ONES(8), eps) == 0)


def test_rope_identity_at_pos0():
    v = rng.standard_normal(128)
    assert np.array_equal(oracle.rope(v, 0, 500000.0), v)


def test_rope_hd2_closed_form():
    # head_dim 2: one pair, frequency 1; (1, 0) rotates to (cos p, sin p)
    for p in (1, 2, 7):
        out = oracle.rope([1.0, 0.0], p, 10000.0)
        assert np.allclose(out, [math.cos(p), math.sin(p)], atol=1e-15)
        out = oracle.rope([0.0, 1.0], p, 10000.0)
        assert np.allclose(out, [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_hd4_pairing_and_frequencies():
    # pairs are (0, 2) and (1, 3); frequencies 1 and theta^(-1/2)
    theta, p = 100.0, 3
    out = oracle.rope([1.0, 0.0, 0.0, 0.0], p, theta)
    assert np.allclose(out, [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    out = oracle.rope([0.0, 1.0, 0.0, 0.0], p, theta)
    t = p * theta**-0.5
    assert np.allclose(out, [0, math.cos(t), 0, math.sin(t)], atol=1e-15)


def rope_complex(v, pos, theta):
    """RoPE as complex multiplication z_i * exp(i pos w_i), z_i = v_i + i v_{i+hd/2}."""
    hd = len(v)
    half = hd // 2
    w = theta ** (-np.arange(half) * 2.0 / hd)
    z = (np.asarray(v[:half]) + 1j * np.asarray(v[half:])) * np.exp(1j * pos * w)
    return np.concatenate([z.real, z.imag])


def test_rope_matches_complex_form_and_is_relative():
    theta = 500000.0
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for p in (1, 17, 1023, 8300):
        assert np.allclose(oracle.rope(q, p, theta), rope_complex(q, p, theta), atol=1e-12)
        # per-pair norm preserved
        r = oracle.rope(q, p, theta)
        assert np.allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    d1 = oracle.rope(q, 40, theta) @ oracle.rope(k, 30, theta)
    d2 = oracle.rope(q, 1010, theta) @ oracle.rope(k, 1000, theta)
    assert abs(d1 - d2) < 1e-10 * (abs(d1) + 1)


def test_silu_points():
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(oracle.silu(-2.0), -2.0 / (1.0 + math.exp(2.0)), rel_tol=1e-15)
    assert math.isclose(oracle.silu(40.0), 40.0, rel_tol=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_attention_single_position_returns_v():
    K = f32_to_bf16_bits(rng.standard_normal((1, 64)))
    V = f32_to_bf16_bits(rng.standard_normal((1, 64)))
    o = oracle.attention_head(rng.standard_normal(64) * 5, K, V)
    assert np.array_equal(o, bf16_vals(V[0]))


def test_attention_identical_keys_gives_mean():
    K = np.tile(f32_to_bf16_bits(rng.standard_normal(64)), (9, 1))
    V = f32_to_bf16_bits(rng.standard_normal((9, 64)))
    o = oracle.attention_head(rng.standard_normal(64), K, V)
    assert np.allclose(o, bf16_vals(V).mean(axis=0), atol=1e-14)


def test_attention_two_position_closed_form_and_rowsum():
    hd = 16
    q = np.zeros(hd)
    q[0] = 2.0
    K = np.zeros((2, hd), dtype=np.uint16)
    K[0, 0] = 0x3F80  # 1.0  -> score 2/sqrt(16) = 0.5
    K[1, 0] = 0xBF80  # -1.0 -> score -0.5
    V = np.zeros((2, hd), dtype=np.uint16)
    V[0, :] = 0x3F80
    V[1, :] = 0x4000  # 2.0
    o = oracle.attention_head(q, K, V)
    p0 = math.exp(0.5) / (math.exp(0.5) + math.exp(-0.5))
    assert np.allclose(o, p0 * 1.0 + (1 - p0) * 2.0, rtol=1e-14)
    # V = 1 everywhere: output 1 (probabilities sum to one)
    Kr = f32_to_bf16_bits(rng.standard_normal((37, hd)) * 4)
    o1 = oracle.attention_head(rng.standard_normal(hd) * 4, Kr, np.full((37, hd), 0x3F80, np.uint16))
    assert np.allclose(o1, 1.0, atol=1e-14)


def test_gemv_bf16_matches_numpy():
    W = f32_to_bf16_bits(rng.standard_normal((37, 200)) * 0.02)
    x = rng.standard_normal(200)
    assert np.allclose(oracle.gemv_bf16(W, x), bf16_vals(W) @ x, rtol=1e-13, atol=1e-15)


def unpack_int4(packed, cols):
    lo = packed & 0xF
    hi = packed >> 4
    q = np.empty((packed.shape[0], cols), dtype=np.int64)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def test_gemv_int8_int4_match_numpy_dequant():
    Wb = f32_to_bf16_bits(rng.standard_normal((24, 256)) * 0.02)
    x = rng.standard_normal(256)
    q, s = oracle.quant_int8(Wb)
    want = (q.astype(np.float64) * s.astype(np.float64)[:, None]) @ x
    assert np.allclose(oracle.gemv_int8(q, s, x), want, rtol=1e-13, atol=1e-15)
    packed, sc, zp = oracle.quant_int4(Wb)
    qq = unpack_int4(packed, 256)
    sv = sc.view(np.float16).astype(np.float64).repeat(128, axis=1)
    zv = zp.view(np.float16).astype(np.float64).repeat(128, axis=1)
    want4 = ((qq - zv) * sv) @ x
    assert np.allclose(oracle.gemv_int4(packed, sc, zp, 256, x), want4, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------ quantisers --

def test_quant_int8_golden():
    with open(os.path.join(GOLDEN, "quant_int8_rows.json")) as f:
        g = json.load(f)
    W = np.array([f32_to_bf16_bits(r["w"]) for r in g["rows"]])
    q, s = oracle.quant_int8(W)
    for i, r in enumerate(g["rows"]):
        assert q[i].tolist() == r["q"], r["why"]
        assert int(s[i:i + 1].view(np.uint32)[0]) == r["s_bits"], r["why"]


def test_quant_int8_bounds():
    W = f32_to_bf16_bits(rng.standard_normal((64, 512)) * 0.02)
    q, s = oracle.quant_int8(W)
    w = bf16_vals(W)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(w - q * s.astype(np.float64)[:, None])
    # half a step, plus the fp32 rounding of w/s (|w/s| <= 127.5 < 2^7)
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0**-16))
    # the largest magnitude of every row maps to +-127
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_quant_int4_golden():
    with open(os.path.join(GOLDEN, "quant_int4_group.json")) as f:
        g = json.load(f)
    vals = [g["pattern"][i % 6] for i in range(128)]
    W = f32_to_bf16_bits(np.array([vals, vals[::-1]]))
    packed, sc, zp = oracle.quant_int4(W)
    assert int(sc[0, 0]) == g["scale_bits"] and int(zp[0, 0]) == g["zero_bits"]
    qrow = unpack_int4(packed, 128)[0]
    assert qrow.tolist() == [g["q_pattern"][i % 6] for i in range(128)]
    assert packed[0, :3].tolist() == g["packed_pattern"]


def test_quant_int4_bounds():
    W = f32_to_bf16_bits(rng.standard_normal((16, 1024)) * 0.02)
    packed, sc, zp = oracle.quant_int4(W)
    q = unpack_int4(packed, 1024)
    s = sc.view(np.float16).astype(np.float64).repeat(128, axis=1)
    z = zp.view(np.float16).astype(np.float64).repeat(128, axis=1)
    w = bf16_vals(W)
    assert q.min() >= 0 and q.max() <= 15
    assert np.all((z >= 0) & (z <= 15) & (z == np.round(z)))
    unclamped = (np.round(w / s) + z >= 0) & (np.round(w / s) + z <= 15)
    err = np.abs(w - (q - z) * s)
    assert np.all(err[unclamped] <= s[unclamped] * (0.5 + 1e-3))


# ------------------------------------------------------------------ model --

TINY = Workload("pin", 2, 64, 4, 2, 16, 96, 300, 1e-5, 10000.0, False, "bf16", False, 6, 4, 16)


def rand_weights(wl, seed):
    return synth.model_weights(wl, seed=seed)


def zero_like(w, ids):
    out = dict(w)
    for i in ids:
        out[i] = np.zeros_like(w[i])
    return out


def lid(l, k):
    return 1 + 9 * l + k


def np_rms(x, g):
    return x / np.sqrt(np.mean(x * x) + 1e-5) * g


def test_model_zero_layers_reduces_to_norm_and_head():
    wl = TINY
    w = rand_weights(wl, 5)
    w = zero_like(w, [lid(l, k) for l in range(wl.n_layers) for k in (1, 2, 3, 4, 6, 7, 8)])
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    E, lm = bf16_vals(w[0]), bf16_vals(w[2 + 9 * wl.n_layers])
    for pos, tok in enumerate([3, 299, 0, 150]):
        want = lm @ np_rms(E[tok], 1.0)
        assert np.allclose(m.step(kv, tok, pos), want, rtol=1e-12, atol=1e-14)


def test_model_uniform_attention_is_causal_mean_of_v():
    """Wq = Wk = 0 makes every score 0, so each head's output is the mean of
    the cached V rows 0..pos (inclusive).  Wv and Wo are random; the MLP is
    zero.  Checks KV write position, causal extent, GQA group mapping and the
    attention residual, against a numpy evaluation of that closed form."""
    wl = TINY
    L, H, hd, nq, nkv = wl.n_layers, wl.hidden, wl.head_dim, wl.n_heads, wl.n_kv_heads
    w = rand_weights(wl, 6)
    w = zero_like(w, [lid(l, k) for l in range(L) for k in (1, 2, 6, 7, 8)])
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    E, lm = bf16_vals(w[0]), bf16_vals(w[2 + 9 * L])
    toks = [7, 100, 7, 250, 31]
    vhist = [[] for _ in range(L)]
    for pos, tok in enumerate(toks):
        x = E[tok].copy()
        for l in range(L):
            h = np_rms(x, 1.0)
            v = bf16_vals(w[lid(l, 3)]) @ h
            vhist[l].append(bf16_vals(f32_to_bf16_bits(v.astype(np.float32))))
            vm = np.mean(vhist[l], axis=0).reshape(nkv, hd)
            o = np.concatenate([vm[hq // (nq // nkv)] for hq in range(nq)])
            x = x + bf16_vals(w[lid(l, 4)]) @ o
        want = lm @ np_rms(x, 1.0)
        got = m.step(kv, tok, pos)
        # bf16 rounding of v: the oracle rounds the double, numpy the float32
        assert np.allclose(got, want, rtol=1e-5, atol=1e-6)


def test_model_mlp_only_matches_swiglu_closed_form():
    wl = TINY
    L = wl.n_layers
    w = rand_weights(wl, 7)
    w = zero_like(w, [lid(l, k) for l in range(L) for k in (1, 2, 3, 4)])
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    E, lm = bf16_vals(w[0]), bf16_vals(w[2 + 9 * L])
    x = E[42].copy()
    for l in range(L):
        h = np_rms(x, 1.0)
        g_ = bf16_vals(w[lid(l, 6)]) @ h
        u_ = bf16_vals(w[lid(l, 7)]) @ h
        a = g_ / (1 + np.exp(-g_)) * u_
        x = x + bf16_vals(w[lid(l, 8)]) @ a
    want = lm @ np_rms(x, 1.0)
    assert np.allclose(m.step(kv, 42, 0), want, rtol=1e-12, atol=1e-14)


def brute_force_decode(wl, w, toks):
    """Independent numpy float64 evaluation of the whole decoder on a tiny
    model: complex-number RoPE, matrix softmax, explicit GQA repeat."""
    L, H, hd, nq, nkv = wl.n_layers, wl.hidden, wl.head_dim, wl.n_heads, wl.n_kv_heads
    E = bf16_vals(w[0])
    lm = E if wl.tied else bf16_vals(w[2 + 9 * L])
    Kc = [[] for _ in range(L)]
    Vc = [[] for _ in range(L)]
    out = []
    for pos, tok in enumerate(toks):
        x = E[tok].copy()
        for l in range(L):
            Wl = {k: bf16_vals(w[lid(l, k)]) for k in (0, 1, 2, 3, 4, 5, 6, 7, 8)}
            h = np_rms(x, Wl[0])
            q = (Wl[1] @ h).reshape(nq, hd)
            k = (Wl[2] @ h).reshape(nkv, hd)
            v = (Wl[3] @ h).reshape(nkv, hd)
            q = np.stack([rope_complex(r, pos, wl.rope_theta) for r in q])
            k = np.stack([rope_complex(r, pos, wl.rope_theta) for r in k])
            Kc[l].append(bf16_vals(f32_to_bf16_bits(k.astype(np.float32))))
            Vc[l].append(bf16_vals(f32_to_bf16_bits(v.astype(np.float32))))
            K = np.stack(Kc[l], axis=1)  # [nkv][pos+1][hd]
            V = np.stack(Vc[l], axis=1)
            K = np.repeat(K, nq // nkv, axis=0)
            V = np.repeat(V, nq // nkv, axis=0)
            S = np.einsum("hd,hjd->hj", q, K) / math.sqrt(hd)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            o = np.einsum("hj,hjd->hd", P, V).reshape(-1)
            x = x + Wl[4] @ o
            h2 = np_rms(x, Wl[5])
            gg, uu = Wl[6] @ h2, Wl[7] @ h2
            x = x + Wl[8] @ (gg / (1 + np.exp(-gg)) * uu)
        out.append(lm @ np_rms(x, bf16_vals(w[1 + 9 * L])))
    return out


@pytest.mark.parametrize("tied", [False, True])
def test_model_brute_force_tiny(tied):
    wl = TINY.with_(tied=tied, n_layers=2)
    w = rand_weights(wl, 11)
    # non-trivial norm gains so a dropped gain is caught
    for l in range(wl.n_layers):
        for k in (0, 5):
            w[lid(l, k)] = f32_to_bf16_bits(1.0 + 0.25 * rng.standard_normal(wl.hidden))
    w[1 + 9 * wl.n_layers] = f32_to_bf16_bits(1.0 + 0.25 * rng.standard_normal(wl.hidden))
    toks = [5, 77, 5, 299, 0, 123, 64]
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    want = brute_force_decode(wl, w, toks)
    for pos, tok in enumerate(toks):
        got = m.step(kv, tok, pos)
        # the only difference is where each side rounds k, v to bf16
        rel = np.linalg.norm(got - want[pos]) / np.linalg.norm(want[pos])
        assert rel < 1e-5, (pos, rel)


def bf16_round_f64(x):
    """Round-to-nearest-even of float64 values to bf16 (8 significant bits),
    straight from the double (normal range): x = m * 2^e, m in [0.5, 1)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def np_dequant(wbits, fmt):
    """The stored weights of one projection as exact float64 values, from the
    format definitions (independent of the oracle's quantisers): bf16 as
    stored; int8 one fp32 scale per output row, s = amax / 127, q =
    clamp(rne(w / s), -127, 127) (all-zero rows: s = 1, q = 0); int4 groups of
    128 inputs, s = fp16((max - min) / 15) (1 if 0), z = clamp(rne(-min / s),
    0, 15), q = clamp(rne(w / s) + z, 0, 15), value (q - z) s.  The quantiser
    arithmetic is fp32, rounding half to even."""
    w = bf16_vals(wbits)
    if fmt == "bf16":
        return w
    w32 = w.astype(np.float32)
    if fmt == "int8":
        amax = np.max(np.abs(w32), axis=1)
        s = np.where(amax == 0, np.float32(1), amax / np.float32(127)).astype(np.float32)
        q = np.clip(np.rint(w32 / s[:, None]), -127, 127)
        q[amax == 0] = 0
        return q.astype(np.float64) * s.astype(np.float64)[:, None]
    rows, cols = w32.shape
    g = w32.reshape(rows, cols // 128, 128)
    mn, mx = g.min(axis=2), g.max(axis=2)
    s = ((mx - mn) / np.float32(15)).astype(np.float16).astype(np.float32)
    s = np.where(s == 0, np.float32(1), s)
    z = np.clip(np.rint(-mn / s), 0, 15).astype(np.float32)
    q = np.clip(np.rint(g / s[..., None]) + z[..., None], 0, 15)
    return ((q - z[..., None]).astype(np.float64) * s[..., None].astype(np.float64)).reshape(rows, cols)


def brute_force_decode_fmt(wl, w, toks):
    """brute_force_decode for any weight format and for bf16 projection
    inputs (act_bf16): the 7 projections of every layer and the LM head are
    quantised and dequantised by np_dequant; with act_bf16 the inputs of
    every projection (h, o, h2, a, the final normed x) are rounded to bf16;
    K and V rows are rounded to bf16 from the double."""
    L, H, hd, nq, nkv = wl.n_layers, wl.hidden, wl.head_dim, wl.n_heads, wl.n_kv_heads
    rb = bf16_round_f64 if wl.act_bf16 else (lambda v: v)
    E = bf16_vals(w[0])
    lm = np_dequant(w[0] if wl.tied else w[2 + 9 * L], "bf16" if wl.tied else wl.wfmt)
    Wl = [{k: (bf16_vals(w[lid(l, k)]) if k in (0, 5) else np_dequant(w[lid(l, k)], wl.wfmt)) for k in range(9)}
          for l in range(L)]
    Kc = [[] for _ in range(L)]
    Vc = [[] for _ in range(L)]
    out = []
    for pos, tok in enumerate(toks):
        x = E[tok].copy()
        for l in range(L):
            W = Wl[l]
            h = rb(np_rms(x, W[0]))
            q = (W[1] @ h).reshape(nq, hd)
            k = (W[2] @ h).reshape(nkv, hd)
            v = (W[3] @ h).reshape(nkv, hd)
            q = np.stack([rope_complex(r, pos, wl.rope_theta) for r in q])
            k = np.stack([rope_complex(r, pos, wl.rope_theta) for r in k])
            Kc[l].append(bf16_round_f64(k))
            Vc[l].append(bf16_round_f64(v))
            K = np.repeat(np.stack(Kc[l], axis=1), nq // nkv, axis=0)
            V = np.repeat(np.stack(Vc[l], axis=1), nq // nkv, axis=0)
            S = np.einsum("hd,hjd->hj", q, K) / math.sqrt(hd)
            Pm = np.exp(S - S.max(axis=1, keepdims=True))
            Pm /= Pm.sum(axis=1, keepdims=True)
            o = rb(np.einsum("hj,hjd->hd", Pm, V).reshape(-1))
            x = x + W[4] @ o
            h2 = rb(np_rms(x, W[5]))
            gg, uu = W[6] @ h2, W[7] @ h2
            x = x + W[8] @ rb(gg / (1 + np.exp(-gg)) * uu)
        out.append(lm @ rb(np_rms(x, bf16_vals(w[1 + 9 * L]))))
    return out


def test_bf16_round_f64_points():
    # halfway cases round to even, checked against the bit-level rounding
    for v in (1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 3.0 + 2.0**-7, 0.1, -7.3e-3, 0.0):
        assert bf16_round_f64(v) == bf16_vals(np.array([oracle.round_bf16(v)], dtype=np.uint16))[0], v


@pytest.mark.parametrize("fmt,act_bf16", [("bf16", True), ("int8", False), ("int8", True), ("int4", False),
                                          ("int4", True)])
def test_model_brute_force_quantised_and_act_bf16(fmt, act_bf16):
    """Every projection of every layer quantised (non-zero random layers and
    non-unit gains), with or without bf16 projection inputs: the oracle
    equals the float64 brute force built from the format definitions (a
    dropped or misplaced rounding of h, o, h2, a or the final normed x, or a
    wrong dequantisation in any layer, moves the logits by far more than the
    bound)."""
    wl = TINY.with_(hidden=128, head_dim=32, ffn=256, n_layers=2, wfmt=fmt, act_bf16=act_bf16)
    w = rand_weights(wl, 31)
    for l in range(wl.n_layers):
        for k in (0, 5):
            w[lid(l, k)] = f32_to_bf16_bits(1.0 + 0.25 * rng.standard_normal(wl.hidden))
    w[1 + 9 * wl.n_layers] = f32_to_bf16_bits(1.0 + 0.25 * rng.standard_normal(wl.hidden))
    toks = [5, 77, 5, 299, 0, 123]
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    want = brute_force_decode_fmt(wl, w, toks)
    for pos, tok in enumerate(toks):
        got = m.step(kv, tok, pos)
        rel = np.linalg.norm(got - want[pos]) / np.linalg.norm(want[pos])
        assert rel < 1e-9, (fmt, act_bf16, pos, rel)
    # the same weights without the activation rounding give clearly other
    # logits (the rounding is there), and the quantised model differs from
    # the bf16 one (the quantisation is applied)
    if act_bf16:
        other = brute_force_decode_fmt(wl.with_(act_bf16=False), w, toks)[-1]
        assert np.linalg.norm(other - want[-1]) / np.linalg.norm(want[-1]) > 1e-4
    if fmt != "bf16":
        other = brute_force_decode_fmt(wl.with_(wfmt="bf16"), w, toks)[-1]
        assert np.linalg.norm(other - want[-1]) / np.linalg.norm(want[-1]) > 1e-3


def test_model_quantised_uses_dequantised_weights():
    """An int8 (resp. int4) model equals the bf16 oracle run on the
    explicitly dequantised weights (written back as exact doubles via a
    float64 evaluation of the same zero-layer special case)."""
    for fmt in ("int8", "int4"):
        wl = TINY.with_(hidden=128, head_dim=32, ffn=256, wfmt=fmt)
        w = rand_weights(wl, 21)
        L = wl.n_layers
        w = zero_like(w, [lid(l, k) for l in range(L) for k in (1, 2, 3, 4, 6, 7, 8)])
        m = oracle.Model(wl, w)
        kv = m.new_kv()
        lmb = w[2 + 9 * L]
        if fmt == "int8":
            q, s = oracle.quant_int8(lmb)
            lm = q.astype(np.float64) * s.astype(np.float64)[:, None]
        else:
            p, sc, zp = oracle.quant_int4(lmb)
            lm = (unpack_int4(p, 128) - zp.view(np.float16).astype(np.float64).repeat(128, 1)) * \
                sc.view(np.float16).astype(np.float64).repeat(128, 1)
        E = bf16_vals(w[0])
        want = lm @ np_rms(E[9], 1.0)
        assert np.allclose(m.step(kv, 9, 0), want, rtol=1e-12, atol=1e-14)


def test_model_act_bf16_rounds_projection_inputs():
    wl = TINY.with_(act_bf16=True)
    w = rand_weights(wl, 8)
    L = wl.n_layers
    w = zero_like(w, [lid(l, k) for l in range(L) for k in (1, 2, 3, 4, 6, 7, 8)])
    m = oracle.Model(wl, w)
    kv = m.new_kv()
    E, lm = bf16_vals(w[0]), bf16_vals(w[2 + 9 * L])
    h = np_rms(E[1], 1.0)
    hb = bf16_vals(f32_to_bf16_bits(h.astype(np.float32)))
    got = m.step(kv, 1, 0)
    assert np.allclose(got, lm @ hb, rtol=1e-12, atol=1e-14)
    assert not np.allclose(got, lm @ h, rtol=1e-9, atol=0)


def test_model_rejects_bad_args():
    m = oracle.Model(TINY, rand_weights(TINY, 1))
    kv = m.new_kv()
    with pytest.raises(ValueError):
        m.step(kv, TINY.vocab, 0)
    with pytest.raises(ValueError):
        m.step(kv, 0, TINY.max_ctx)
