// Weight packing: canonical bf16 tensors -> device layouts, with the weight-only
// int8 / int4 quantisation of the AutoMegaKernel summary ("Quantised
// megakernels" contribution).  The pages fix neither format; this library
// uses (all arithmetic in fp32, round half to even):
//   int8, per output row:  s = amax / 127 (s = 1 for an all-zero row),
//                          q = clamp(round(w / s), -127, 127)
//   int4, per 128 inputs:  s = fp16(round((max - min) / 15)) (1 if that is 0),
//                          z = clamp(round(-min / s), 0, 15), stored as fp16,
//                          q = clamp(round(w / s) + z, 0, 15)
// Packed tensors (see ProjLayout): the fused QKV matrix stores each RoPE pair
// of rows (i, i + head_dim/2) of one head next to each other; the gate/up
// matrix stores gate row j next to up row j.
#include <cmath>
#include <cstring>

#include "amk_internal.h"

namespace amk {

namespace {

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // IEEE round to nearest even
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

inline float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}

// position of column c (0..7) of an 8-column chunk inside the 32-bit word:
// nibble j holds column 2j, nibble j + 4 holds column 2j + 1
inline int nibble_of_col(int c) { return (c & 1) ? (c >> 1) + 4 : (c >> 1); }

// quantise + store one row of a packed projection
void pack_row(const ProjLayout& p, int64_t r, const uint16_t* src, uint8_t* dst) {
  const int64_t K = p.cols;
  uint8_t* data = dst + r * p.data_row_bytes();
  uint8_t* meta = dst + p.meta_offset() + r * p.meta_row_bytes();
  if (p.fmt == AMK_W_BF16) {
    std::memcpy(data, src, K * 2);
    return;
  }
  if (p.fmt == AMK_W_INT8_ROW) {
    float amax = 0.0f;
    for (int64_t c = 0; c < K; ++c) amax = std::fmax(amax, std::fabs(bf16_to_f32(src[c])));
    float s = amax / 127.0f;
    if (amax == 0.0f) s = 1.0f;
    for (int64_t c = 0; c < K; ++c) {
      float q = amax == 0.0f ? 0.0f : std::nearbyintf(bf16_to_f32(src[c]) / s);
      q = std::fmin(127.0f, std::fmax(-127.0f, q));
      data[c] = (uint8_t)((int)q + 128);
    }
    std::memcpy(meta, &s, 4);
    return;
  }
  // int4
  for (int64_t g = 0; g < K / 128; ++g) {
    const uint16_t* w = src + g * 128;
    float mn = bf16_to_f32(w[0]), mx = mn;
    for (int i = 1; i < 128; ++i) {
      float v = bf16_to_f32(w[i]);
      mn = std::fmin(mn, v);
      mx = std::fmax(mx, v);
    }
    uint16_t sb = f32_to_f16_bits((mx - mn) / 15.0f);
    float s = f16_bits_to_f32(sb);
    if (s == 0.0f) { sb = 0x3C00; s = 1.0f; }
    float z = std::fmin(15.0f, std::fmax(0.0f, std::nearbyintf(-mn / s)));
    uint16_t zb = f32_to_f16_bits(z);
    std::memcpy(meta + g * 4, &sb, 2);
    std::memcpy(meta + g * 4 + 2, &zb, 2);
    for (int chunk = 0; chunk < 16; ++chunk) {
      uint32_t word = 0;
      for (int c = 0; c < 8; ++c) {
        float q = std::nearbyintf(bf16_to_f32(w[chunk * 8 + c]) / s) + z;
        q = std::fmin(15.0f, std::fmax(0.0f, q));
        word |= (uint32_t)(int)q << (4 * nibble_of_col(c));
      }
      std::memcpy(data + g * 64 + chunk * 4, &word, 4);
    }
  }
}

// decode one packed row back to canonical quantised values
void unpack_row(const ProjLayout& p, int64_t r, const uint8_t* src, int64_t out_row, void* q_out,
                void* s_out, void* z_out) {
  const int64_t K = p.cols;
  const uint8_t* data = src + r * p.data_row_bytes();
  const uint8_t* meta = src + p.meta_offset() + r * p.meta_row_bytes();
  if (p.fmt == AMK_W_BF16) {
    if (q_out) std::memcpy((uint16_t*)q_out + out_row * K, data, K * 2);
    return;
  }
  if (p.fmt == AMK_W_INT8_ROW) {
    if (q_out)
      for (int64_t c = 0; c < K; ++c) ((int8_t*)q_out)[out_row * K + c] = (int8_t)((int)data[c] - 128);
    if (s_out) std::memcpy((float*)s_out + out_row, meta, 4);
    return;
  }
  const int64_t G = K / 128;
  for (int64_t g = 0; g < G; ++g) {
    if (s_out) std::memcpy((uint16_t*)s_out + out_row * G + g, meta + g * 4, 2);
    if (z_out) std::memcpy((uint16_t*)z_out + out_row * G + g, meta + g * 4 + 2, 2);
    if (!q_out) continue;
    uint8_t* qo = (uint8_t*)q_out + out_row * (K / 2) + g * 64;
    for (int chunk = 0; chunk < 16; ++chunk) {
      uint32_t word;
      std::memcpy(&word, data + g * 64 + chunk * 4, 4);
      for (int c = 0; c < 8; c += 2) {
        uint32_t lo = (word >> (4 * nibble_of_col(c))) & 0xF;
        uint32_t hi = (word >> (4 * nibble_of_col(c + 1))) & 0xF;
        qo[chunk * 4 + c / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

struct RowSource { int32_t canon; int64_t row; };

// canonical source of packed row r of packed tensor k
RowSource source_row(const amk_model_config& m, int32_t k, int64_t r) {
  const int32_t L = m.n_layers;
  if (k == 0) return {0, r};
  if (k == 1) return {1 + 9 * L, 0};
  if (k == 2) return {m.tied_embeddings ? 0 : 2 + 9 * L, r};
  const int32_t l = (k - 3) / 6, sub = (k - 3) % 6, base = 1 + 9 * l;
  const int64_t hd = m.head_dim, half = hd / 2, nq = m.n_heads, nkv = m.n_kv_heads;
  switch (sub) {
    case LB_ATTN_NORM: return {base + 0, 0};
    case LB_MLP_NORM: return {base + 5, 0};
    case LB_O: return {base + 4, r};
    case LB_DOWN: return {base + 8, r};
    case LB_GATEUP: return {base + ((r & 1) ? 7 : 6), r >> 1};
    case LB_QKV: {
      const int64_t u = r >> 1, hs = u / half, i = u % half;
      const int64_t fused = hs * hd + i + ((r & 1) ? half : 0);
      if (hs < nq) return {base + 1, fused};
      if (hs < nq + nkv) return {base + 2, fused - nq * hd};
      return {base + 3, fused - (nq + nkv) * hd};
    }
  }
  return {-1, 0};
}

}  // namespace

amk_status pack_tensor(const amk_model_config& m, int32_t k, const uint16_t* const* canon, void* dst) {
  const ProjLayout p = packed_layout(m, k);
  uint8_t* out = (uint8_t*)dst;
  for (int64_t r = 0; r < p.rows; ++r) {
    RowSource src = source_row(m, k, r);
    const uint16_t* t = canon[src.canon];
    if (!t) return fail(AMK_ERR_INVALID_ARG, "canonical tensor " + std::to_string(src.canon) + " is null");
    pack_row(p, r, t + src.row * p.cols, out);
  }
  return AMK_OK;
}

amk_status unpack_tensor(const amk_model_config& m, int32_t k, int32_t canon_id, const void* packed,
                         void* q_out, void* s_out, void* z_out) {
  const ProjLayout p = packed_layout(m, k);
  bool any = false;
  for (int64_t r = 0; r < p.rows; ++r) {
    RowSource src = source_row(m, k, r);
    if (src.canon != canon_id) continue;
    any = true;
    unpack_row(p, r, (const uint8_t*)packed, src.row, q_out, s_out, z_out);
  }
  if (!any) return fail(AMK_ERR_INVALID_ARG, "canonical tensor not inside this packed tensor");
  return AMK_OK;
}

}  // namespace amk
