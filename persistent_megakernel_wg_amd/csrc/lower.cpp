// Lowering of a Llama-style decoder to the typed Schedule DAG (the layer-2
// "Scheduler" of the AutoMegaKernel summary, section "Methodology": import the
// model, lower it to a task DAG synchronised by monotonic counters, under a
// ScheduleConfig of tiling, fusion, SM assignment and pipelining depth).
//
// Per layer l the fused task phases are
//   QKV    RMSNorm prologue, q/k/v rows, RoPE, K/V row written at pos
//   ATTN   one split of the positions of one kv head, for its query group
//   MERGE  log-sum-exp merge of the splits of one query head
//   OPROJ  o-projection rows + residual
//   GATEUP RMSNorm prologue, gate/up rows, silu(gate)*up
//   DOWN   down-projection rows + residual
// and one LMHEAD phase (final RMSNorm prologue + vocabulary rows) at the end.
// Each join is one counter whose waiters wait for all its producers:
//   QKV(l) <- DOWN(l-1);  ATTN(l) <- QKV(l);  MERGE(l,h) <- ATTN(l, group of h);
//   OPROJ(l) <- MERGE(l);  GATEUP(l) <- OPROJ(l);  DOWN(l) <- GATEUP(l);
//   LMHEAD <- DOWN(L-1).
// Task ids follow one global topological order (phase by phase) and every
// queue lists its tasks in that order.
#include <algorithm>

#include "amk_internal.h"

namespace amk {

namespace {

struct Builder {
  amk_schedule* s;
  const amk_model_config& m;
  const amk_schedule_config& c;

  int32_t counter() { return s->n_counters++; }

  int32_t cu_of(int64_t i, int64_t T) const {
    if (c.cu_policy == 1) return (int32_t)(i % c.num_cus);
    return (int32_t)((i * c.num_cus) / T);
  }

  // bounds of T tiles over n items (in groups of `grain`), each tile's share
  // proportional to the weight of the XCD its queue runs on
  std::vector<int64_t> bounds(int phase, int64_t n, int64_t T, int64_t grain,
                              const std::vector<char>* light = nullptr) const {
    std::vector<int64_t> w(T), b(T + 1);
    int64_t tot = 0;
    for (int64_t i = 0; i < T; ++i) {
      w[i] = c.xcd_weight[phase][cu_of(i, T) % 8];
      if (light && (*light)[cu_of(i, T)]) w[i] = w[i] * c.merge_o_share / 1000;
      tot += w[i];
    }
    const int64_t g = n / grain;  // whole groups; a remainder goes to the last tile
    int64_t acc = 0;
    for (int64_t i = 0; i <= T; ++i) {
      b[i] = i == T ? n : grain * ((g * acc) / tot);
      if (i < T) acc += w[i];
    }
    // at least one group per tile where possible
    for (int64_t i = 1; i < T; ++i) b[i] = std::max(b[i], std::min(b[i - 1] + grain, n - grain * (T - i)));
    return b;
  }

  int32_t add(int32_t type, int32_t cu, std::initializer_list<int32_t> params,
              std::initializer_list<Wait> waits, std::initializer_list<int32_t> sigs) {
    Task t;
    t.type = type;
    t.cu = cu;
    int k = 0;
    for (int32_t v : params) t.p[k++] = v;
    t.waits.assign(waits);
    t.sigs.assign(sigs);
    derive_accesses(m, t, &t.acc);
    sort_accesses(&t.acc);
    s->tasks.push_back(std::move(t));
    return (int32_t)s->tasks.size() - 1;
  }
};


}  // namespace

amk_status lower(const amk_model_config& m, const amk_schedule_config& c, amk_schedule* s) {
  Builder b{s, m, c};
  s->model = m;
  s->config = c;
  s->tasks.clear();
  s->n_counters = 0;
  const int32_t L = m.n_layers, nq = m.n_heads, nkv = m.n_kv_heads, grp = nq / nkv;
  const int64_t U = (int64_t)(nq + 2 * nkv) * (m.head_dim / 2);
  const int32_t S = c.attn_splits;
  const uint32_t Pq = c.tiles_qkv, Pattn = S, Pm = nq, Po = c.tiles_o, Pg = c.tiles_gateup,
                 Pd = c.tiles_down;
  int32_t prev_down = -1;
  for (int32_t l = 0; l < L; ++l) {
    const int32_t c_qkv = b.counter();
    std::vector<int32_t> c_attn(nkv);
    for (int32_t g = 0; g < nkv; ++g) c_attn[g] = b.counter();
    const int32_t c_merge = b.counter(), c_o = b.counter(), c_gu = b.counter(), c_down = b.counter();
    // MERGE queues: by default spread over the queues that run no attention
    // split (a merge queue then holds no attention loads when the splits of
    // its head land); queues that run a MERGE task of the layer get a
    // smaller O-projection tile
    const int64_t n_attn = (int64_t)nkv * S;
    std::vector<char> attn_q(c.num_cus, 0);
    for (int64_t i = 0; i < n_attn; ++i) attn_q[b.cu_of(i, n_attn)] = 1;
    std::vector<int32_t> free_q;
    for (int32_t q = 0; q < c.num_cus; ++q)
      if (!attn_q[q]) free_q.push_back(q);
    const bool spread_free = c.merge_place == 0 && !free_q.empty();
    auto merge_cu = [&](int32_t h) {
      return spread_free ? free_q[(size_t)(((int64_t)h * (int64_t)free_q.size()) / nq)] : b.cu_of(h, nq);
    };
    std::vector<char> merges(c.num_cus, 0);
    for (int32_t h = 0; h < nq; ++h) merges[merge_cu(h)] = 1;
    const std::vector<int64_t> bq = b.bounds(AMK_PHASE_QKV, U, c.tiles_qkv, 1),
                               bo = b.bounds(AMK_PHASE_O, m.hidden, c.tiles_o, 2, &merges),
                               bg = b.bounds(AMK_PHASE_GATEUP, m.ffn, c.tiles_gateup, 1),
                               bd = b.bounds(AMK_PHASE_DOWN, m.hidden, c.tiles_down, 2);
    for (int32_t i = 0; i < c.tiles_qkv; ++i) {
      const int32_t u0 = (int32_t)bq[i], u1 = (int32_t)bq[i + 1];
      if (l == 0) b.add(AMK_TASK_QKV, b.cu_of(i, c.tiles_qkv), {l, u0, u1}, {}, {c_qkv});
      else b.add(AMK_TASK_QKV, b.cu_of(i, c.tiles_qkv), {l, u0, u1}, {{prev_down, Pd}}, {c_qkv});
    }
    for (int32_t g = 0; g < nkv; ++g)
      for (int32_t sp = 0; sp < S; ++sp)
        b.add(AMK_TASK_ATTN, b.cu_of((int64_t)g * S + sp, n_attn), {l, g, sp, S}, {{c_qkv, Pq}},
              {c_attn[g]});
    for (int32_t h = 0; h < nq; ++h)
      b.add(AMK_TASK_MERGE, merge_cu(h), {l, h, S}, {{c_attn[h / grp], Pattn}}, {c_merge});
    for (int32_t i = 0; i < c.tiles_o; ++i)
      b.add(AMK_TASK_OPROJ, b.cu_of(i, c.tiles_o),
            {l, (int32_t)bo[i], (int32_t)bo[i + 1]},
            {{c_merge, Pm}}, {c_o});
    for (int32_t i = 0; i < c.tiles_gateup; ++i)
      b.add(AMK_TASK_GATEUP, b.cu_of(i, c.tiles_gateup),
            {l, (int32_t)bg[i], (int32_t)bg[i + 1]},
            {{c_o, Po}}, {c_gu});
    for (int32_t i = 0; i < c.tiles_down; ++i)
      b.add(AMK_TASK_DOWN, b.cu_of(i, c.tiles_down),
            {l, (int32_t)bd[i], (int32_t)bd[i + 1]},
            {{c_gu, Pg}}, {c_down});
    prev_down = c_down;
  }
  const int32_t c_lm = b.counter();
  const std::vector<int64_t> bl = b.bounds(AMK_PHASE_LM, m.vocab, c.tiles_lm, 2);
  for (int32_t i = 0; i < c.tiles_lm; ++i)
    b.add(AMK_TASK_LMHEAD, b.cu_of(i, c.tiles_lm), {(int32_t)bl[i], (int32_t)bl[i + 1]},
          {{prev_down, Pd}}, {c_lm});
  s->queues.assign(c.num_cus, {});
  for (int32_t t = 0; t < (int32_t)s->tasks.size(); ++t) s->queues[s->tasks[t].cu].push_back(t);
  s->buffers = buffer_table(m, S);
  return AMK_OK;
}

}  // namespace amk
