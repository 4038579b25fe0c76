// Model checks, ScheduleConfig resolution, packed weight layouts, the buffer
// table of a lowered schedule and the access footprint of every task type.
#include <algorithm>
#include <cstring>

#include "amk_internal.h"

namespace amk {

amk_status check_model(const amk_model_config& m) {
  if (m.n_layers < 1 || m.hidden < 1 || m.n_heads < 1 || m.n_kv_heads < 1 || m.head_dim < 1 ||
      m.ffn < 1 || m.vocab < 1 || m.max_ctx < 1)
    return fail(AMK_ERR_INVALID_ARG, "model sizes must be positive");
  if (!(m.rms_eps > 0.0f) || !(m.rope_theta > 0.0f))
    return fail(AMK_ERR_INVALID_ARG, "rms_eps and rope_theta must be positive");
  if (m.attn_bias || m.mlp_bias)
    return fail(AMK_ERR_UNSUPPORTED, "biased projections are not supported");
  if (m.n_heads % m.n_kv_heads)
    return fail(AMK_ERR_UNSUPPORTED, "n_heads must be a multiple of n_kv_heads");
  if (m.head_dim != 64 && m.head_dim != 128 && m.head_dim != 256)
    return fail(AMK_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (m.n_heads / m.n_kv_heads > 16)
    return fail(AMK_ERR_UNSUPPORTED, "at most 16 query heads per kv head");

  if (m.wfmt < AMK_W_BF16 || m.wfmt > AMK_W_INT4_G128)
    return fail(AMK_ERR_UNSUPPORTED, "unknown weight format");
  const int64_t qdim = (int64_t)m.n_heads * m.head_dim;
  const int64_t align = m.wfmt == AMK_W_BF16 ? 8 : (m.wfmt == AMK_W_INT8_ROW ? 16 : 128);
  if (m.hidden % align || qdim % align || m.ffn % align)
    return fail(AMK_ERR_UNSUPPORTED, "hidden, n_heads*head_dim and ffn must be multiples of " +
                                         std::to_string(align) + " for this weight format");
  if (m.hidden % 8) return fail(AMK_ERR_UNSUPPORTED, "hidden must be a multiple of 8");
  if ((int64_t)m.vocab * m.hidden > (int64_t)1 << 40)
    return fail(AMK_ERR_UNSUPPORTED, "embedding too large");
  if (m.hidden > 65536 || m.ffn > 65536)
    return fail(AMK_ERR_UNSUPPORTED, "hidden and ffn must be at most 65536");
  return AMK_OK;
}

static int32_t pick(int32_t v, int32_t dflt) { return v > 0 ? v : dflt; }

// Automatic split count: 3/4 of the queues run a split (8 per kv head for
// caches of at most 512 positions: short splits cost more in merging than
// they save).  Caches of more than 4096 positions take as many splits as
// leave one split-free queue per query head, where the merges go (on the
// 8192-position int4 workload, 28 splits per kv head: 2.457 ms; 24: 2.485;
// 30, two merges on some queues: 2.638; the position-major attention layout
// keeps such long splits fast).
int32_t default_attn_splits(const amk_model_config& m, int32_t num_cus) {
  if (m.max_ctx <= 512) return std::min(8, std::max(1, num_cus / m.n_kv_heads));
  if (m.max_ctx <= 4096) return std::max(1, 3 * num_cus / (4 * m.n_kv_heads));
  return std::max(1, (num_cus - m.n_heads) / m.n_kv_heads);
}

amk_status resolve_config(const amk_model_config& m, const amk_schedule_config& in,
                          amk_schedule_config* out) {
  amk_schedule_config c = in;
  if (c.num_cus < 1 || c.num_cus > 4096) return fail(AMK_ERR_INVALID_ARG, "num_cus out of range");
  if (c.wg_threads == 0) c.wg_threads = 512;
  if (c.wg_threads != 512) return fail(AMK_ERR_UNSUPPORTED, "wg_threads must be 512");
  const int32_t half = m.head_dim / 2;
  const int64_t qkv_units = (int64_t)(m.n_heads + 2 * m.n_kv_heads) * half;
  c.tiles_qkv = pick(c.tiles_qkv, c.num_cus);
  c.tiles_o = pick(c.tiles_o, c.num_cus);
  c.tiles_gateup = pick(c.tiles_gateup, c.num_cus);
  c.tiles_down = pick(c.tiles_down, c.num_cus);
  c.tiles_lm = pick(c.tiles_lm, c.num_cus);
  c.tiles_qkv = (int32_t)std::min<int64_t>(c.tiles_qkv, qkv_units);
  // O, down and LM-head tiles hold whole row pairs
  c.tiles_o = std::min(c.tiles_o, std::max(1, m.hidden / 2));
  c.tiles_gateup = std::min(c.tiles_gateup, m.ffn);
  c.tiles_down = std::min(c.tiles_down, std::max(1, m.hidden / 2));
  c.tiles_lm = std::min(c.tiles_lm, std::max(1, m.vocab / 2));
  if (c.attn_splits <= 0) c.attn_splits = default_attn_splits(m, c.num_cus);
  if (c.attn_splits > 256) return fail(AMK_ERR_UNSUPPORTED, "attn_splits must be at most 256");
  if (c.cu_policy != 0 && c.cu_policy != 1) return fail(AMK_ERR_UNSUPPORTED, "cu_policy must be 0 or 1");
  if (c.pipeline_depth == 0) c.pipeline_depth = 8;
  if (c.pipeline_depth != 4 && c.pipeline_depth != 8 && c.pipeline_depth != 16)
    return fail(AMK_ERR_UNSUPPORTED, "pipeline_depth must be 4, 8 or 16");
  if (c.poll_mode < 0 || c.poll_mode > 3) return fail(AMK_ERR_UNSUPPORTED, "poll_mode must be 0, 1, 2 or 3");
  if (c.release_mode != 0 && c.release_mode != 1)
    return fail(AMK_ERR_UNSUPPORTED, "release_mode must be 0 or 1");
  for (int32_t ph = 0; ph < 5; ++ph)
    for (int32_t x = 0; x < 8; ++x) {
      int32_t& w = c.xcd_weight[ph][x];
      if (w == 0) w = 1000;
      if (w < 100 || w > 10000)
        return fail(AMK_ERR_INVALID_ARG, "xcd_weight must be 0 (default) or 100..10000 permille");
    }
  if (c.merge_o_share == 0) c.merge_o_share = 1000;
  if (c.merge_o_share < 1 || c.merge_o_share > 1000)
    return fail(AMK_ERR_INVALID_ARG, "merge_o_share must be 0 (default) or 1..1000 permille");
  if (c.merge_place != 0 && c.merge_place != 1) return fail(AMK_ERR_UNSUPPORTED, "merge_place must be 0 or 1");
  if (c.sync_mode < 0 || c.sync_mode > 2) return fail(AMK_ERR_UNSUPPORTED, "sync_mode must be 0, 1 or 2");
  if (c.sync_mode != 0 && (c.attn_splits > 512 || (int64_t)c.attn_splits * m.head_dim > 8192))
    return fail(AMK_ERR_UNSUPPORTED, "sync_mode 1 and 2 need attn_splits <= 512 and attn_splits * head_dim <= 8192");
  // with DMA waves, 384 threads read a merge's tagged partials in one round
  if (c.sync_mode != 0 && c.poll_mode == 3 && (c.attn_splits > 384 || (int64_t)c.attn_splits * m.head_dim > 6144))
    return fail(AMK_ERR_UNSUPPORTED,
                "sync_mode 1 and 2 with poll_mode 3 need attn_splits <= 384 and attn_splits * head_dim <= 6144");
  // automatic prefetch: 64 KB for bf16 weights at hidden size >= 4096; off
  // for the quantised formats and smaller models, whose tasks gain less than
  // the copy delays the wake (the tuner's picks on those workloads)
  // (with DMA waves, poll_mode 3, the copy does not delay the wake: as much
  // as the two DMA waves and the LDS hold)
  if (c.prefetch_kb == 0)
    c.prefetch_kb = c.poll_mode == 3 ? 128 : (m.wfmt == AMK_W_BF16 && m.hidden >= 4096 ? 64 : -1);
  if (c.prefetch_kb != -1 && (c.prefetch_kb < 1 || c.prefetch_kb > 1024))
    return fail(AMK_ERR_INVALID_ARG, "prefetch_kb must be -1 (off) or 1..1024");
  // resolved: -1 = off, else a budget in KB
  if (c.prefetch_attn_kb == -1) c.prefetch_attn_kb = c.prefetch_kb;
  if (c.prefetch_attn_kb == 0) c.prefetch_attn_kb = 1024;
  if (c.prefetch_attn_kb != -1 && (c.prefetch_attn_kb < 1 || c.prefetch_attn_kb > 1024))
    return fail(AMK_ERR_INVALID_ARG, "prefetch_attn_kb must be -1 (as prefetch_kb), 0 (all that fits) or 1..1024");
  if (c.fuse_flags == 0) c.fuse_flags = AMK_FUSE_DEFAULT;
  if (c.fuse_flags != AMK_FUSE_DEFAULT)
    return fail(AMK_ERR_UNSUPPORTED, "only the fully fused task set (AMK_FUSE_DEFAULT) is built");
  *out = c;
  return AMK_OK;
}

ProjLayout packed_layout(const amk_model_config& m, int32_t k) {
  ProjLayout p;
  const int64_t H = m.hidden, F = m.ffn, qdim = (int64_t)m.n_heads * m.head_dim;
  const int64_t kvdim = (int64_t)m.n_kv_heads * m.head_dim;
  if (k == 0) { p.fmt = AMK_W_BF16; p.rows = m.vocab; p.cols = H; return p; }
  if (k == 1) { p.fmt = AMK_W_BF16; p.rows = 1; p.cols = H; return p; }
  if (k == 2) { p.fmt = m.wfmt; p.rows = m.vocab; p.cols = H; return p; }
  const int32_t sub = (k - 3) % 6;
  switch (sub) {
    case LB_ATTN_NORM: case LB_MLP_NORM: p.fmt = AMK_W_BF16; p.rows = 1; p.cols = H; break;
    case LB_QKV: p.fmt = m.wfmt; p.rows = qdim + 2 * kvdim; p.cols = H; break;
    case LB_O: p.fmt = m.wfmt; p.rows = H; p.cols = qdim; break;
    case LB_GATEUP: p.fmt = m.wfmt; p.rows = 2 * F; p.cols = H; break;
    case LB_DOWN: p.fmt = m.wfmt; p.rows = H; p.cols = F; break;
  }
  return p;
}

std::vector<Buffer> buffer_table(const amk_model_config& m, int32_t S) {
  const int64_t L = m.n_layers, H = m.hidden, F = m.ffn, hd = m.head_dim;
  const int64_t nq = m.n_heads, nkv = m.n_kv_heads, mc = m.max_ctx, V = m.vocab;
  std::vector<Buffer> b(n_buffers(m));
  for (int32_t k = 0; k < 3 + 6 * m.n_layers; ++k)
    b[packed_to_buffer(k)] = {packed_layout(m, k).total_bytes(), AMK_BUF_WEIGHT};
  b[B_KV_HIST] = {L * 2 * nkv * mc * hd * 2, AMK_BUF_HISTORY};
  b[B_KV_CUR] = {L * 2 * nkv * hd * 2, AMK_BUF_STATE};
  b[B_LOGITS] = {V * 4, AMK_BUF_OUTPUT};
  b[B_X] = {L * 2 * H * 4, AMK_BUF_SCRATCH};
  b[B_Q] = {L * nq * hd * 4, AMK_BUF_SCRATCH};
  b[B_PART] = {L * nq * (int64_t)S * (hd + 2) * 4, AMK_BUF_SCRATCH};
  b[B_O] = {L * nq * hd * 4, AMK_BUF_SCRATCH};
  b[B_A] = {L * F * 4, AMK_BUF_SCRATCH};
  return b;
}

static void push(std::vector<Access>* a, int32_t buf, int32_t mode, int64_t b, int64_t e) {
  a->push_back({buf, mode, b, e});
}

// rows [r0, r1) of a packed projection stored in buffer `buf`
static void proj_rows(std::vector<Access>* a, int32_t buf, const ProjLayout& p, int64_t r0,
                      int64_t r1) {
  push(a, buf, AMK_ACCESS_READ, r0 * p.data_row_bytes(), r1 * p.data_row_bytes());
  if (p.meta_row_bytes())
    push(a, buf, AMK_ACCESS_READ, p.meta_offset() + r0 * p.meta_row_bytes(),
         p.meta_offset() + r1 * p.meta_row_bytes());
}

bool derive_accesses(const amk_model_config& m, const Task& t, std::vector<Access>* out) {
  out->clear();
  const int64_t L = m.n_layers, H = m.hidden, F = m.ffn, hd = m.head_dim, half = hd / 2;
  const int64_t nq = m.n_heads, nkv = m.n_kv_heads, mc = m.max_ctx, V = m.vocab;
  const int64_t grp = nq / nkv;
  const int32_t* p = t.p;
  auto layer_ok = [&](int64_t l) { return l >= 0 && l < L; };
  // the residual stream a task of layer l reads: the embedding row at l = 0
  auto x_in = [&](int64_t l, int64_t r0, int64_t r1) {
    if (l == 0) push(out, B_EMBED, AMK_ACCESS_READ, 0, V * H * 2);
    else push(out, B_X, AMK_ACCESS_READ, (((l - 1) * 2 + 1) * H + r0) * 4, (((l - 1) * 2 + 1) * H + r1) * 4);
  };
  switch (t.type) {
    case AMK_TASK_QKV: {
      const int64_t l = p[0], u0 = p[1], u1 = p[2], U = (nq + 2 * nkv) * half;
      if (!layer_ok(l) || u0 < 0 || u1 <= u0 || u1 > U) return false;
      x_in(l, 0, H);
      push(out, layer_buf(l, LB_ATTN_NORM), AMK_ACCESS_READ, 0, H * 2);
      proj_rows(out, layer_buf(l, LB_QKV), packed_layout(m, 3 + 6 * l + LB_QKV), 2 * u0, 2 * u1);
      for (int64_t hs = u0 / half; hs * half < u1; ++hs) {
        const int64_t i0 = std::max(u0, hs * half) - hs * half;
        const int64_t i1 = std::min(u1, (hs + 1) * half) - hs * half;
        if (hs < nq) {
          const int64_t base = l * nq * hd + hs * hd;
          push(out, B_Q, AMK_ACCESS_WRITE, (base + i0) * 4, (base + i1) * 4);
          push(out, B_Q, AMK_ACCESS_WRITE, (base + half + i0) * 4, (base + half + i1) * 4);
        } else {
          const int64_t kv = hs < nq + nkv ? 0 : 1, g = hs - nq - kv * nkv;
          const int64_t base = ((l * 2 + kv) * nkv + g) * hd;
          push(out, B_KV_CUR, AMK_ACCESS_WRITE, (base + i0) * 2, (base + i1) * 2);
          push(out, B_KV_CUR, AMK_ACCESS_WRITE, (base + half + i0) * 2, (base + half + i1) * 2);
        }
      }
      return true;
    }
    case AMK_TASK_ATTN: {
      const int64_t l = p[0], g = p[1], s = p[2], S = p[3];
      if (!layer_ok(l) || g < 0 || g >= nkv || S < 1 || s < 0 || s >= S) return false;
      push(out, B_Q, AMK_ACCESS_READ, (l * nq * hd + g * grp * hd) * 4,
           (l * nq * hd + (g + 1) * grp * hd) * 4);
      for (int64_t kv = 0; kv < 2; ++kv) {
        const int64_t slot = (l * 2 + kv) * nkv + g;
        push(out, B_KV_HIST, AMK_ACCESS_READ, slot * mc * hd * 2, (slot + 1) * mc * hd * 2);
        push(out, B_KV_CUR, AMK_ACCESS_READ, slot * hd * 2, (slot + 1) * hd * 2);
      }
      for (int64_t h = g * grp; h < (g + 1) * grp; ++h) {
        const int64_t b = ((l * nq + h) * S + s) * (hd + 2) * 4;
        push(out, B_PART, AMK_ACCESS_WRITE, b, b + (hd + 2) * 4);
      }
      return true;
    }
    case AMK_TASK_MERGE: {
      const int64_t l = p[0], h = p[1], S = p[2];
      if (!layer_ok(l) || h < 0 || h >= nq || S < 1) return false;
      push(out, B_PART, AMK_ACCESS_READ, (l * nq + h) * S * (hd + 2) * 4,
           (l * nq + h + 1) * S * (hd + 2) * 4);
      push(out, B_O, AMK_ACCESS_WRITE, (l * nq * hd + h * hd) * 4, (l * nq * hd + (h + 1) * hd) * 4);
      return true;
    }
    case AMK_TASK_OPROJ: {
      const int64_t l = p[0], r0 = p[1], r1 = p[2];
      if (!layer_ok(l) || r0 < 0 || r1 <= r0 || r1 > H) return false;
      push(out, B_O, AMK_ACCESS_READ, l * nq * hd * 4, (l + 1) * nq * hd * 4);
      x_in(l, r0, r1);
      proj_rows(out, layer_buf(l, LB_O), packed_layout(m, 3 + 6 * l + LB_O), r0, r1);
      push(out, B_X, AMK_ACCESS_WRITE, (l * 2 * H + r0) * 4, (l * 2 * H + r1) * 4);
      return true;
    }
    case AMK_TASK_GATEUP: {
      const int64_t l = p[0], j0 = p[1], j1 = p[2];
      if (!layer_ok(l) || j0 < 0 || j1 <= j0 || j1 > F) return false;
      push(out, B_X, AMK_ACCESS_READ, l * 2 * H * 4, (l * 2 + 1) * H * 4);
      push(out, layer_buf(l, LB_MLP_NORM), AMK_ACCESS_READ, 0, H * 2);
      proj_rows(out, layer_buf(l, LB_GATEUP), packed_layout(m, 3 + 6 * l + LB_GATEUP), 2 * j0, 2 * j1);
      push(out, B_A, AMK_ACCESS_WRITE, (l * F + j0) * 4, (l * F + j1) * 4);
      return true;
    }
    case AMK_TASK_DOWN: {
      const int64_t l = p[0], r0 = p[1], r1 = p[2];
      if (!layer_ok(l) || r0 < 0 || r1 <= r0 || r1 > H) return false;
      push(out, B_A, AMK_ACCESS_READ, l * F * 4, (l + 1) * F * 4);
      push(out, B_X, AMK_ACCESS_READ, (l * 2 * H + r0) * 4, (l * 2 * H + r1) * 4);
      proj_rows(out, layer_buf(l, LB_DOWN), packed_layout(m, 3 + 6 * l + LB_DOWN), r0, r1);
      push(out, B_X, AMK_ACCESS_WRITE, ((l * 2 + 1) * H + r0) * 4, ((l * 2 + 1) * H + r1) * 4);
      return true;
    }
    case AMK_TASK_LMHEAD: {
      const int64_t r0 = p[0], r1 = p[1];
      if (r0 < 0 || r1 <= r0 || r1 > V) return false;
      push(out, B_X, AMK_ACCESS_READ, ((L - 1) * 2 + 1) * H * 4, (L - 1) * 2 * H * 4 + 2 * H * 4);
      push(out, B_FINAL_NORM, AMK_ACCESS_READ, 0, H * 2);
      proj_rows(out, B_LM, packed_layout(m, 2), r0, r1);
      push(out, B_LOGITS, AMK_ACCESS_WRITE, r0 * 4, r1 * 4);
      return true;
    }
    default:
      return false;
  }
}

void sort_accesses(std::vector<Access>* a) {
  std::sort(a->begin(), a->end(), [](const Access& x, const Access& y) {
    if (x.buf != y.buf) return x.buf < y.buf;
    if (x.begin != y.begin) return x.begin < y.begin;
    if (x.end != y.end) return x.end < y.end;
    return x.mode < y.mode;
  });
}

std::vector<uint32_t> counter_producers(const amk_schedule& s) {
  std::vector<uint32_t> P(std::max(0, s.n_counters), 0);
  for (const Task& t : s.tasks)
    for (int32_t c : t.sigs)
      if (c >= 0 && c < s.n_counters) P[c]++;
  return P;
}

}  // namespace amk
