// Oracle: plain, slow CPU reference of one batch-1 decode step of a
// Llama-style decoder.  TEST INFRASTRUCTURE ONLY: the product path never
// links, loads or calls this file; only the tests, the smoke check and the
// bench's CPU-baseline leg do.
//
// What it computes follows the AutoMegaKernel summary pages ("AutoMegaKernel
// (AMK)" technical summary, section "Problem statement": single-stream
// batch-1 autoregressive decode of Hugging Face Llama-family models; section
// "Methodology", layer 1: GEMV, attention and RMSNorm micro-kernels) and the
// Argus page's megakernel case study (section "Workload and baselines": GEMM,
// attention, normalisation, KV-cache update and logits of one decode step).
// The pages give no formulas for these operators; the plain Llama
// definitions are used, read as follows:
//   * RMSNorm:  y_i = x_i / sqrt(mean(x^2) + eps) * g_i
//   * RoPE:     rotate-half pairs (i, i + hd/2), angle pos * theta^(-2i/hd)
//   * attention: causal over positions 0..pos inclusive, scale 1/sqrt(hd),
//                softmax, kv head of query head h = h / (n_heads / n_kv)
//   * SwiGLU:   a = silu(W_gate h) * (W_up h), silu(z) = z / (1 + e^-z)
//   * residual: x += W_o o ; x += W_down a
//   * the KV cache holds bf16 (rounded on write, read back as stored)
//   * weight-only quantised variants ("Quantised megakernels" contribution:
//     int8 and int4 weight-only) dequantise exactly: int8 q*s (per output
//     row), int4 (q - z)*s (groups of 128 along the input dimension)
//
// Arithmetic is double precision throughout; the only roundings are the ones
// the workload fixes: bf16 KV cache, and for act_bf16 models the bf16
// rounding of each projection's input vector.  Loops are sequential per
// output element (OpenMP only splits independent output rows / heads).
//
// Parity pins: tests/test_oracle_pins.py (closed forms, invariants, special
// cases and brute force on tiny inputs).

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, max_ctx;
  double rms_eps, rope_theta;
  int32_t tied;      // lm_head is the embedding matrix
  int32_t wfmt;      // 0 bf16, 1 int8 per output row, 2 int4 groups of 128
  int32_t act_bf16;  // round every projection input to bf16
} orc_config;

// ---------------------------------------------------------------- numbers --

double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// round a double to the nearest bf16 (ties to even), via exact bit work on
// the double (no intermediate float rounding)
uint16_t orc_round_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  // bf16 = 1 sign, 8 exponent, 7 mantissa bits; handle with frexp
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
  double a = std::fabs(v);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  int e;
  double m = std::frexp(a, &e);  // a = m * 2^e, m in [0.5, 1)
  // normal bf16 exponent range: value in [2^-126, 2^128)
  int ebias = e - 1 + 127;      // biased exponent of a = 1.f * 2^(e-1)
  if (ebias >= 255) return sign | 0x7F80;
  double scaled;                 // integer significand incl. hidden bit
  int exp_field;
  if (ebias >= 1) {
    scaled = std::ldexp(m, 8);   // in [128, 256)
    exp_field = ebias;
  } else {                       // subnormal: value = f * 2^-133
    scaled = std::ldexp(a, 133);
    exp_field = 0;
  }
  double r = std::nearbyint(scaled);  // default rounding mode: ties to even
  uint32_t sig = (uint32_t)r;
  if (exp_field >= 1) {
    if (sig == 256) { sig = 128; exp_field += 1; }
    if (exp_field >= 255) return sign | 0x7F80;
    return sign | (uint16_t)(exp_field << 7) | (uint16_t)(sig - 128);
  }
  // subnormal result (or rounds up into the smallest normal)
  if (sig >= 128) return sign | (uint16_t)(1 << 7) | (uint16_t)(sig - 128);
  return sign | (uint16_t)sig;
}

double orc_bf16_round_trip(double v) { return orc_bf16_to_double(orc_round_bf16(v)); }

// IEEE half (binary16) helpers, written from the format definition
double orc_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
  double v;
  if (ex == 0) v = std::ldexp((double)man, -24);
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = std::ldexp((double)(man + 1024), ex - 25);
  return sign ? -v : v;
}

uint16_t orc_f16_from_float(float f) {
  // round a float to the nearest binary16, ties to even
  if (std::isnan(f)) return 0x7E00;
  uint16_t sign = std::signbit(f) ? 0x8000 : 0;
  double a = std::fabs((double)f);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return sign | 0x7C00;  // rounds to inf
  int e;
  double m = std::frexp(a, &e);            // a = m 2^e
  int ebias = e - 1 + 15;
  if (ebias >= 1) {
    double r = std::nearbyint(std::ldexp(m, 11));  // [1024, 2048]
    uint32_t sig = (uint32_t)r;
    if (sig == 2048) { sig = 1024; ebias += 1; }
    if (ebias >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(ebias << 10) | (uint16_t)(sig - 1024);
  }
  double r = std::nearbyint(std::ldexp(a, 24));    // subnormal units of 2^-24
  uint32_t sig = (uint32_t)r;
  if (sig >= 1024) return sign | (uint16_t)(1 << 10) | (uint16_t)(sig - 1024);
  return sign | (uint16_t)sig;
}

// ------------------------------------------------------------- operators --

// RMSNorm with eps inside the square root, weight applied after normalising
void orc_rmsnorm(const double* x, const uint16_t* g, int n, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / std::sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv * orc_bf16_to_double(g[i]);
}

// rotary embedding of one head vector in place, rotate-half convention:
// for i < hd/2, (a, b) = (v[i], v[i + hd/2]) and angle t = pos * theta^(-2i/hd)
//   v[i]        = a cos t - b sin t
//   v[i + hd/2] = b cos t + a sin t
void orc_rope(double* v, int hd, int pos, double theta) {
  int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = std::pow(theta, -2.0 * i / hd);
    double t = (double)pos * inv_freq;
    double c = std::cos(t), s = std::sin(t);
    double a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

double orc_silu(double z) { return z / (1.0 + std::exp(-z)); }

// one query head against n_pos cached positions (rows of hd bf16 values)
void orc_attention_head(const double* q, const uint16_t* K, const uint16_t* V, int hd, int n_pos,
                        double* o) {
  std::vector<double> s(n_pos);
  double scale = 1.0 / std::sqrt((double)hd);
  double mx = -INFINITY;
  for (int j = 0; j < n_pos; ++j) {
    double d = 0.0;
    for (int i = 0; i < hd; ++i) d += q[i] * orc_bf16_to_double(K[(size_t)j * hd + i]);
    s[j] = d * scale;
    if (s[j] > mx) mx = s[j];
  }
  double sum = 0.0;
  for (int j = 0; j < n_pos; ++j) {
    s[j] = std::exp(s[j] - mx);
    sum += s[j];
  }
  for (int i = 0; i < hd; ++i) o[i] = 0.0;
  for (int j = 0; j < n_pos; ++j) {
    double p = s[j] / sum;
    for (int i = 0; i < hd; ++i) o[i] += p * orc_bf16_to_double(V[(size_t)j * hd + i]);
  }
}

// y = W x with W [rows][cols] row-major bf16
void orc_gemv_bf16(const uint16_t* W, int rows, int cols, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint16_t* w = W + (size_t)r * cols;
    double acc = 0.0;
    for (int c = 0; c < cols; ++c) acc += orc_bf16_to_double(w[c]) * x[c];
    y[r] = acc;
  }
}

// y = W x with W_rc = q_rc * s_r (exact product in double)
void orc_gemv_int8(const int8_t* q, const float* s, int rows, int cols, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const int8_t* w = q + (size_t)r * cols;
    double sr = (double)s[r], acc = 0.0;
    for (int c = 0; c < cols; ++c) acc += ((double)w[c] * sr) * x[c];
    y[r] = acc;
  }
}

// y = W x with W_rc = (q_rc - z_rg) * s_rg, g = c / 128; q nibbles packed two
// per byte, low nibble = even column
void orc_gemv_int4(const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, int rows,
                   int cols, const double* x, double* y) {
  const int ng = cols / 128;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint8_t* p = packed + (size_t)r * (cols / 2);
    double acc = 0.0;
    for (int c = 0; c < cols; ++c) {
      int qv = (c & 1) ? (p[c >> 1] >> 4) : (p[c >> 1] & 0xF);
      int g = c / 128;
      double s = orc_f16_to_double(scale[(size_t)r * ng + g]);
      double z = orc_f16_to_double(zero[(size_t)r * ng + g]);
      acc += (((double)qv - z) * s) * x[c];
    }
    y[r] = acc;
  }
}

// ------------------------------------------------------------ quantisers --

// int8, one scale per output row: s = amax / 127 (fp32), q = clamp(rne(w / s))
void orc_quant_int8(const uint16_t* w, int rows, int cols, int8_t* q, float* s) {
  for (int r = 0; r < rows; ++r) {
    const uint16_t* wr = w + (size_t)r * cols;
    float amax = 0.0f;
    for (int c = 0; c < cols; ++c) {
      float v = (float)orc_bf16_to_double(wr[c]);
      if (std::fabs(v) > amax) amax = std::fabs(v);
    }
    if (amax == 0.0f) {
      s[r] = 1.0f;
      for (int c = 0; c < cols; ++c) q[(size_t)r * cols + c] = 0;
      continue;
    }
    float sr = amax / 127.0f;
    s[r] = sr;
    for (int c = 0; c < cols; ++c) {
      float v = (float)orc_bf16_to_double(wr[c]);
      float t = std::nearbyint(v / sr);
      if (t > 127.0f) t = 127.0f;
      if (t < -127.0f) t = -127.0f;
      q[(size_t)r * cols + c] = (int8_t)t;
    }
  }
}

// int4, groups of 128 consecutive input columns:
//   s = fp16(rne((max - min) / 15)), 1 if that is 0
//   z = clamp(rne(-min / s), 0, 15)            (stored as fp16, exact)
//   q = clamp(rne(w / s) + z, 0, 15), packed low nibble = even column
void orc_quant_int4(const uint16_t* w, int rows, int cols, uint8_t* packed, uint16_t* scale,
                    uint16_t* zero) {
  const int ng = cols / 128;
  for (int r = 0; r < rows; ++r) {
    for (int g = 0; g < ng; ++g) {
      const uint16_t* wg = w + (size_t)r * cols + (size_t)g * 128;
      float mn = INFINITY, mx = -INFINITY;
      for (int i = 0; i < 128; ++i) {
        float v = (float)orc_bf16_to_double(wg[i]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
      }
      float range = mx - mn;
      uint16_t sh = orc_f16_from_float(range / 15.0f);
      float sf = (float)orc_f16_to_double(sh);
      if (sf == 0.0f) { sh = 0x3C00; sf = 1.0f; }
      float zf = std::nearbyint(-mn / sf);
      if (zf < 0.0f) zf = 0.0f;
      if (zf > 15.0f) zf = 15.0f;
      scale[(size_t)r * ng + g] = sh;
      zero[(size_t)r * ng + g] = orc_f16_from_float(zf);
      for (int i = 0; i < 128; ++i) {
        float v = (float)orc_bf16_to_double(wg[i]);
        float t = std::nearbyint(v / sf) + zf;
        if (t < 0.0f) t = 0.0f;
        if (t > 15.0f) t = 15.0f;
        int c = g * 128 + i;
        uint8_t* byte = packed + (size_t)r * (cols / 2) + (c >> 1);
        if ((c & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | (int)t);
        else *byte = (uint8_t)((*byte & 0x0F) | ((int)t << 4));
      }
    }
  }
}

// ------------------------------------------------------------------ model --

struct OrcProj {  // one projection matrix in the model's weight format
  int rows = 0, cols = 0;
  const uint16_t* bf16 = nullptr;
  std::vector<int8_t> q8;
  std::vector<float> s8;
  std::vector<uint8_t> q4;
  std::vector<uint16_t> s4, z4;
};

struct orc_model {
  orc_config cfg;
  const uint16_t* embed;
  const uint16_t* final_norm;
  std::vector<const uint16_t*> attn_norm, mlp_norm;
  std::vector<OrcProj> wq, wk, wv, wo, wg, wu, wd;
  OrcProj lm;
};

static void proj_init(OrcProj& p, const orc_config& c, const uint16_t* w, int rows, int cols) {
  p.rows = rows;
  p.cols = cols;
  if (c.wfmt == 0) {
    p.bf16 = w;
  } else if (c.wfmt == 1) {
    p.q8.resize((size_t)rows * cols);
    p.s8.resize(rows);
    orc_quant_int8(w, rows, cols, p.q8.data(), p.s8.data());
  } else {
    p.q4.assign((size_t)rows * cols / 2, 0);
    p.s4.resize((size_t)rows * (cols / 128));
    p.z4.resize((size_t)rows * (cols / 128));
    orc_quant_int4(w, rows, cols, p.q4.data(), p.s4.data(), p.z4.data());
  }
}

static void proj_apply(const OrcProj& p, int wfmt, const double* x, double* y) {
  if (wfmt == 0) orc_gemv_bf16(p.bf16, p.rows, p.cols, x, y);
  else if (wfmt == 1) orc_gemv_int8(p.q8.data(), p.s8.data(), p.rows, p.cols, x, y);
  else orc_gemv_int4(p.q4.data(), p.s4.data(), p.z4.data(), p.rows, p.cols, x, y);
}

// canon: pointers indexed by canonical tensor id (0 embed, 1+9l+k layer
// tensors, 1+9L final_norm, 2+9L lm_head).  Pointers are borrowed, not copied.
orc_model* orc_model_new(const orc_config* c, const uint16_t* const* canon) {
  const int qdim = c->n_heads * c->head_dim;
  if (c->n_layers < 1 || c->hidden < 1 || c->n_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || (c->head_dim & 1) || c->n_heads % c->n_kv_heads || c->ffn < 1 ||
      c->vocab < 1 || c->max_ctx < 1 || c->wfmt < 0 || c->wfmt > 2)
    return nullptr;
  if (c->wfmt == 2 && (c->hidden % 128 || c->ffn % 128 || qdim % 128)) return nullptr;
  orc_model* m = new orc_model();
  m->cfg = *c;
  const int L = c->n_layers, H = c->hidden, F = c->ffn;
  const int qd = c->n_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  m->embed = canon[0];
  m->final_norm = canon[1 + 9 * L];
  m->attn_norm.resize(L);
  m->mlp_norm.resize(L);
  m->wq.resize(L); m->wk.resize(L); m->wv.resize(L); m->wo.resize(L);
  m->wg.resize(L); m->wu.resize(L); m->wd.resize(L);
  for (int l = 0; l < L; ++l) {
    const uint16_t* const* t = canon + 1 + 9 * l;
    m->attn_norm[l] = t[0];
    proj_init(m->wq[l], *c, t[1], qd, H);
    proj_init(m->wk[l], *c, t[2], kvd, H);
    proj_init(m->wv[l], *c, t[3], kvd, H);
    proj_init(m->wo[l], *c, t[4], H, qd);
    m->mlp_norm[l] = t[5];
    proj_init(m->wg[l], *c, t[6], F, H);
    proj_init(m->wu[l], *c, t[7], F, H);
    proj_init(m->wd[l], *c, t[8], H, F);
  }
  proj_init(m->lm, *c, c->tied ? canon[0] : canon[2 + 9 * L], c->vocab, H);
  return m;
}

void orc_model_free(orc_model* m) { delete m; }

// Conditioning probe (off unless set): before each rounding decision the
// workload fixes (activation to bf16, KV row to bf16) every value is
// multiplied by 1 + eps*r, r uniform in [-1, 1) from a SplitMix64 counter
// stream.  With eps near the fp32 unit roundoff this shows how far the
// logits move when those decisions are taken on values carrying fp32-sized
// errors, which is the spread any fp32 implementation has against this
// oracle.
static double g_jitter_eps = 0.0;
static uint64_t g_jitter_ctr = 0;

void orc_set_jitter(double eps, uint64_t seed) {
  g_jitter_eps = eps;
  g_jitter_ctr = seed;
}

static double jitter(double v) {
  if (g_jitter_eps == 0.0) return v;
  uint64_t z = (g_jitter_ctr++) + 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  z ^= z >> 31;
  const double r = (double)(z >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
  return v * (1.0 + g_jitter_eps * r);
}

static void maybe_round(std::vector<double>& v, int act_bf16) {
  if (!act_bf16) return;
  for (double& e : v) e = orc_bf16_round_trip(jitter(e));
}

// One decode step at position pos for input token `token`.
// kv: [L][2][n_kv][max_ctx][head_dim] bf16, row pos is written, rows 0..pos read.
// logits: [vocab] doubles.  Returns 0, or -1 on a bad argument.
int orc_step(orc_model* m, uint16_t* kv, int token, int pos, double* logits) {
  const orc_config& c = m->cfg;
  if (token < 0 || token >= c.vocab || pos < 0 || pos >= c.max_ctx) return -1;
  const int L = c.n_layers, H = c.hidden, F = c.ffn, hd = c.head_dim;
  const int nq = c.n_heads, nkv = c.n_kv_heads, grp = nq / nkv, mc = c.max_ctx;
  std::vector<double> x(H), h(H), q(nq * hd), k(nkv * hd), v(nkv * hd), o(nq * hd), y(H);
  std::vector<double> gt(F), up(F), a(F);
  for (int i = 0; i < H; ++i) x[i] = orc_bf16_to_double(m->embed[(size_t)token * H + i]);
  for (int l = 0; l < L; ++l) {
    orc_rmsnorm(x.data(), m->attn_norm[l], H, c.rms_eps, h.data());
    maybe_round(h, c.act_bf16);
    proj_apply(m->wq[l], c.wfmt, h.data(), q.data());
    proj_apply(m->wk[l], c.wfmt, h.data(), k.data());
    proj_apply(m->wv[l], c.wfmt, h.data(), v.data());
    for (int hq = 0; hq < nq; ++hq) orc_rope(q.data() + hq * hd, hd, pos, c.rope_theta);
    for (int g = 0; g < nkv; ++g) orc_rope(k.data() + g * hd, hd, pos, c.rope_theta);
    for (int g = 0; g < nkv; ++g) {
      uint16_t* Kr = kv + ((((size_t)l * 2 + 0) * nkv + g) * mc + pos) * hd;
      uint16_t* Vr = kv + ((((size_t)l * 2 + 1) * nkv + g) * mc + pos) * hd;
      for (int i = 0; i < hd; ++i) {
        Kr[i] = orc_round_bf16(jitter(k[g * hd + i]));
        Vr[i] = orc_round_bf16(jitter(v[g * hd + i]));
      }
    }
#pragma omp parallel for schedule(static)
    for (int hq = 0; hq < nq; ++hq) {
      int g = hq / grp;
      const uint16_t* K0 = kv + (((size_t)l * 2 + 0) * nkv + g) * mc * hd;
      const uint16_t* V0 = kv + (((size_t)l * 2 + 1) * nkv + g) * mc * hd;
      orc_attention_head(q.data() + hq * hd, K0, V0, hd, pos + 1, o.data() + hq * hd);
    }
    maybe_round(o, c.act_bf16);
    proj_apply(m->wo[l], c.wfmt, o.data(), y.data());
    for (int i = 0; i < H; ++i) x[i] += y[i];
    orc_rmsnorm(x.data(), m->mlp_norm[l], H, c.rms_eps, h.data());
    maybe_round(h, c.act_bf16);
    proj_apply(m->wg[l], c.wfmt, h.data(), gt.data());
    proj_apply(m->wu[l], c.wfmt, h.data(), up.data());
    for (int i = 0; i < F; ++i) a[i] = orc_silu(gt[i]) * up[i];
    maybe_round(a, c.act_bf16);
    proj_apply(m->wd[l], c.wfmt, a.data(), y.data());
    for (int i = 0; i < H; ++i) x[i] += y[i];
  }
  orc_rmsnorm(x.data(), m->final_norm, H, c.rms_eps, h.data());
  maybe_round(h, c.act_bf16);
  proj_apply(m->lm, c.wfmt, h.data(), logits);
  return 0;
}

// quantised bytes the model holds for a canonical projection id (tests)
int orc_model_quant(orc_model* m, int canon_id, const void** q, const void** s, const void** z) {
  const int L = m->cfg.n_layers;
  OrcProj* p = nullptr;
  if (canon_id == 2 + 9 * L || (m->cfg.tied && canon_id == 0)) p = &m->lm;
  else if (canon_id >= 1 && canon_id < 1 + 9 * L) {
    int l = (canon_id - 1) / 9, k = (canon_id - 1) % 9;
    OrcProj* tbl[9] = {nullptr, &m->wq[l], &m->wk[l], &m->wv[l], &m->wo[l], nullptr,
                       &m->wg[l], &m->wu[l], &m->wd[l]};
    p = tbl[k];
  }
  if (!p) return -1;
  if (m->cfg.wfmt == 1) { *q = p->q8.data(); *s = p->s8.data(); *z = nullptr; }
  else if (m->cfg.wfmt == 2) { *q = p->q4.data(); *s = p->s4.data(); *z = p->z4.data(); }
  else { *q = p->bf16; *s = nullptr; *z = nullptr; }
  return 0;
}

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
