// The static safety gate (AutoMegaKernel summary, section "Methodology", "The
// safety gate": before any GPU launch, static graph checks on the Schedule IR
// certify deadlock freedom, race freedom and correctness, and a schedule that
// fails is rejected).  The pages list the checks, not their definitions; the
// rules below are this library's reading, checked in this order, returning the
// first failure with the smallest offending id:
//
//  V1 REF         ids in range; every task in exactly one queue, the queue of
//                 its cu; access ranges inside their buffers (0 <= begin <
//                 end <= size); typed tasks declare exactly the accesses their
//                 (type, params) perform.
//  V2 THRESHOLD   every wait (C, t) has 1 <= t <= P(C), P(C) = number of
//                 signal entries naming C.
//  V3 CYCLE       the producer -> waiter graph is acyclic.
//  V4 QUEUE_ORDER producer -> waiter edges plus queue-order edges are acyclic.
//  V5 UNDER_JOINED a partial wait (t < P(C)) by a task that reads memory a
//                 producer of C writes.
//  V6 RACE        two tasks whose accesses overlap, one of them a write, not
//                 ordered by happens-before (transitive closure of queue
//                 edges and full-join edges p -> w, w waiting (C, P(C))).
//  V7 OUTPUT      every OUTPUT buffer fully written, and every task reaches a
//                 task that writes an OUTPUT or STATE buffer through
//                 happens-before-ordered writer -> reader data flow.
// V2 + V3 + V4 make every wait satisfiable in a topological order of the
// combined graph (no deadlock for co-resident queues); V5 + V6 give race
// freedom.
#include <algorithm>
#include <numeric>

#include "amk_internal.h"

namespace amk {

namespace {

amk_verdict verdict(int32_t code, int32_t task = -1, int32_t counter = -1, int32_t aux = -1) {
  return amk_verdict{code, task, counter, aux};
}

// iterative Tarjan SCC; returns component id per node and component sizes
void scc(int32_t n, const std::vector<int32_t>& off, const std::vector<int32_t>& adj,
         std::vector<int32_t>* comp, std::vector<int32_t>* comp_size) {
  std::vector<int32_t> index(n, -1), low(n, 0), stack, it(n, 0);
  std::vector<char> on(n, 0);
  comp->assign(n, -1);
  comp_size->clear();
  int32_t idx = 0;
  std::vector<int32_t> call;
  for (int32_t root = 0; root < n; ++root) {
    if (index[root] >= 0) continue;
    call.push_back(root);
    index[root] = low[root] = idx++;
    stack.push_back(root);
    on[root] = 1;
    it[root] = off[root];
    while (!call.empty()) {
      int32_t v = call.back();
      if (it[v] < off[v + 1]) {
        int32_t w = adj[it[v]++];
        if (index[w] < 0) {
          index[w] = low[w] = idx++;
          stack.push_back(w);
          on[w] = 1;
          it[w] = off[w];
          call.push_back(w);
        } else if (on[w]) {
          low[v] = std::min(low[v], index[w]);
        }
      } else {
        call.pop_back();
        if (!call.empty()) low[call.back()] = std::min(low[call.back()], low[v]);
        if (low[v] == index[v]) {
          int32_t cid = (int32_t)comp_size->size(), cnt = 0;
          while (true) {
            int32_t w = stack.back();
            stack.pop_back();
            on[w] = 0;
            (*comp)[w] = cid;
            ++cnt;
            if (w == v) break;
          }
          comp_size->push_back(cnt);
        }
      }
    }
  }
}

struct Csr {
  std::vector<int32_t> off, adj;
  void build(int32_t n, std::vector<std::pair<int32_t, int32_t>>& edges) {
    off.assign(n + 1, 0);
    for (auto& e : edges) off[e.first + 1]++;
    for (int32_t i = 0; i < n; ++i) off[i + 1] += off[i];
    adj.resize(edges.size());
    std::vector<int32_t> pos(off.begin(), off.end() - 1);
    for (auto& e : edges) adj[pos[e.first]++] = e.second;
  }
};

// smallest task id lying on a cycle of the graph (tasks 0..nt-1, counters after)
int32_t smallest_on_cycle(int32_t nt, int32_t nc, std::vector<std::pair<int32_t, int32_t>>& edges) {
  Csr g;
  g.build(nt + nc, edges);
  std::vector<int32_t> comp, size;
  scc(nt + nc, g.off, g.adj, &comp, &size);
  for (int32_t t = 0; t < nt; ++t)
    if (size[comp[t]] >= 2) return t;
  return -1;
}

inline bool overlap(const Access& a, const Access& b) {
  return a.buf == b.buf && a.begin < b.end && b.begin < a.end;
}

}  // namespace

amk_verdict validate(const amk_schedule& s) {
  const int32_t nt = (int32_t)s.tasks.size(), nc = s.n_counters, ncu = (int32_t)s.queues.size();
  const int32_t nb = (int32_t)s.buffers.size();

  // ---- V1 REF
  std::vector<int32_t> occ(nt, 0), occ_cu(nt, -1), qpos(nt, -1);
  for (int32_t c = 0; c < ncu; ++c)
    for (size_t i = 0; i < s.queues[c].size(); ++i) {
      int32_t t = s.queues[c][i];
      if (t < 0 || t >= nt) return verdict(AMK_V_REF, -1, -1, c);
      occ[t]++;
      occ_cu[t] = c;
      qpos[t] = (int32_t)i;
    }
  std::vector<Access> derived, declared;
  for (int32_t i = 0; i < nt; ++i) {
    const Task& t = s.tasks[i];
    bool bad = t.cu < 0 || t.cu >= ncu || t.type < 0 || t.type >= AMK_TASK_NTYPES || occ[i] != 1 ||
               occ_cu[i] != t.cu;
    for (const Wait& w : t.waits) bad |= w.ctr < 0 || w.ctr >= nc;
    for (int32_t c : t.sigs) bad |= c < 0 || c >= nc;
    for (const Access& a : t.acc)
      bad |= a.buf < 0 || a.buf >= nb || (a.mode != AMK_ACCESS_READ && a.mode != AMK_ACCESS_WRITE) ||
             a.begin < 0 || a.end <= a.begin || (a.buf >= 0 && a.buf < nb && a.end > s.buffers[a.buf].size);
    if (!bad && t.type != AMK_TASK_NOP) {
      if (!derive_accesses(s.model, t, &derived)) {
        bad = true;
      } else {
        declared = t.acc;
        sort_accesses(&declared);
        sort_accesses(&derived);
        bad = declared.size() != derived.size();
        for (size_t k = 0; !bad && k < declared.size(); ++k)
          bad = declared[k].buf != derived[k].buf || declared[k].mode != derived[k].mode ||
                declared[k].begin != derived[k].begin || declared[k].end != derived[k].end;
      }
    }
    if (bad) return verdict(AMK_V_REF, i);
  }

  // ---- V2 THRESHOLD
  std::vector<uint32_t> P = counter_producers(s);
  for (int32_t i = 0; i < nt; ++i)
    for (size_t k = 0; k < s.tasks[i].waits.size(); ++k) {
      const Wait& w = s.tasks[i].waits[k];
      if (w.thr < 1 || w.thr > P[w.ctr]) return verdict(AMK_V_THRESHOLD, i, w.ctr, (int32_t)k);
    }

  // producers of each counter (ascending task ids, with multiplicity)
  std::vector<std::vector<int32_t>> prod(nc);
  for (int32_t i = 0; i < nt; ++i)
    for (int32_t c : s.tasks[i].sigs) prod[c].push_back(i);

  // ---- V3 CYCLE, V4 QUEUE_ORDER (counters as intermediate nodes)
  std::vector<std::pair<int32_t, int32_t>> edges;
  for (int32_t i = 0; i < nt; ++i) {
    for (int32_t c : s.tasks[i].sigs) edges.push_back({i, nt + c});
    for (const Wait& w : s.tasks[i].waits) edges.push_back({nt + w.ctr, i});
  }
  {
    auto e3 = edges;
    int32_t t = smallest_on_cycle(nt, nc, e3);
    if (t >= 0) return verdict(AMK_V_CYCLE, t);
  }
  for (int32_t c = 0; c < ncu; ++c)
    for (size_t i = 1; i < s.queues[c].size(); ++i) edges.push_back({s.queues[c][i - 1], s.queues[c][i]});
  {
    int32_t t = smallest_on_cycle(nt, nc, edges);
    if (t >= 0) return verdict(AMK_V_QUEUE_ORDER, t);
  }

  // ---- V5 UNDER_JOINED
  for (int32_t w = 0; w < nt; ++w) {
    const Task& tw = s.tasks[w];
    for (const Wait& wt : tw.waits) {
      if (wt.thr >= P[wt.ctr]) continue;
      for (int32_t p : prod[wt.ctr]) {
        const Task& tp = s.tasks[p];
        for (const Access& r : tw.acc) {
          if (r.mode != AMK_ACCESS_READ) continue;
          for (const Access& wr : tp.acc)
            if (wr.mode == AMK_ACCESS_WRITE && overlap(r, wr))
              return verdict(AMK_V_UNDER_JOINED, w, wt.ctr, p);
        }
      }
    }
  }

  // ---- happens-before as vector clocks over a topological order of the
  // queue + full-join graph (acyclic: it is a subgraph of the V4 graph)
  std::vector<std::pair<int32_t, int32_t>> hb;
  for (int32_t i = 0; i < nt; ++i) {
    for (int32_t c : s.tasks[i].sigs) hb.push_back({i, nt + c});
    for (const Wait& w : s.tasks[i].waits)
      if (w.thr == P[w.ctr]) hb.push_back({nt + w.ctr, i});
  }
  for (int32_t c = 0; c < ncu; ++c)
    for (size_t i = 1; i < s.queues[c].size(); ++i) hb.push_back({s.queues[c][i - 1], s.queues[c][i]});
  Csr g;
  g.build(nt + nc, hb);
  std::vector<int32_t> indeg(nt + nc, 0), order;
  for (int32_t v : g.adj) indeg[v]++;
  order.reserve(nt + nc);
  for (int32_t v = 0; v < nt + nc; ++v)
    if (!indeg[v]) order.push_back(v);
  for (size_t k = 0; k < order.size(); ++k) {
    int32_t v = order[k];
    for (int32_t e = g.off[v]; e < g.off[v + 1]; ++e)
      if (--indeg[g.adj[e]] == 0) order.push_back(g.adj[e]);
  }
  // vc[v][c] = largest queue position on cu c that happens-before-or-equals v
  std::vector<int32_t> vc((size_t)(nt + nc) * ncu, -1);
  for (int32_t v : order) {
    int32_t* row = &vc[(size_t)v * ncu];
    if (v < nt) row[s.tasks[v].cu] = std::max(row[s.tasks[v].cu], qpos[v]);
    for (int32_t e = g.off[v]; e < g.off[v + 1]; ++e) {
      int32_t* dst = &vc[(size_t)g.adj[e] * ncu];
      for (int32_t c = 0; c < ncu; ++c) dst[c] = std::max(dst[c], row[c]);
    }
  }
  auto happens_before = [&](int32_t a, int32_t b) {  // a HB b, a != b
    return vc[(size_t)b * ncu + s.tasks[a].cu] >= qpos[a];
  };

  // ---- V6 RACE and the data-flow edges of V7, from one sweep per buffer
  struct Acc { int64_t b, e; int32_t task, mode; };
  std::vector<std::vector<Acc>> per(nb);
  for (int32_t i = 0; i < nt; ++i)
    for (const Access& a : s.tasks[i].acc) per[a.buf].push_back({a.begin, a.end, i, a.mode});
  int64_t best_a = -1, best_b = -1;
  std::vector<std::pair<int32_t, int32_t>> flow;  // reader -> writer (reverse data flow)
  for (int32_t buf = 0; buf < nb; ++buf) {
    auto& v = per[buf];
    std::sort(v.begin(), v.end(), [](const Acc& x, const Acc& y) { return x.b < y.b; });
    for (size_t i = 0; i < v.size(); ++i)
      for (size_t j = i + 1; j < v.size() && v[j].b < v[i].e; ++j) {
        const Acc &x = v[i], &y = v[j];
        if (x.task == y.task) continue;
        if (x.mode != AMK_ACCESS_WRITE && y.mode != AMK_ACCESS_WRITE) continue;
        int32_t a = std::min(x.task, y.task), bt = std::max(x.task, y.task);
        bool ab = happens_before(a, bt), ba = happens_before(bt, a);
        if (!ab && !ba) {
          if (best_a < 0 || a < best_a || (a == best_a && bt < best_b)) { best_a = a; best_b = bt; }
          continue;
        }
        // writer -> reader data flow in happens-before order
        if (x.mode == AMK_ACCESS_WRITE && y.mode == AMK_ACCESS_READ && happens_before(x.task, y.task))
          flow.push_back({y.task, x.task});
        if (y.mode == AMK_ACCESS_WRITE && x.mode == AMK_ACCESS_READ && happens_before(y.task, x.task))
          flow.push_back({x.task, y.task});
      }
  }
  if (best_a >= 0) return verdict(AMK_V_RACE, (int32_t)best_a, -1, (int32_t)best_b);

  // ---- V7 OUTPUT
  bool any_output = false;
  for (int32_t buf = 0; buf < nb; ++buf) {
    if (s.buffers[buf].kind != AMK_BUF_OUTPUT) continue;
    any_output = true;
    std::vector<std::pair<int64_t, int64_t>> w;
    for (const Acc& a : per[buf])
      if (a.mode == AMK_ACCESS_WRITE) w.push_back({a.b, a.e});
    std::sort(w.begin(), w.end());
    int64_t covered = 0;
    for (auto& r : w) {
      if (r.first > covered) break;
      covered = std::max(covered, r.second);
    }
    if (covered < s.buffers[buf].size) return verdict(AMK_V_OUTPUT, -1, -1, buf);
  }
  if (!any_output) return verdict(AMK_V_OUTPUT);
  std::vector<char> live(nt, 0);
  std::vector<int32_t> work;
  for (int32_t i = 0; i < nt; ++i)
    for (const Access& a : s.tasks[i].acc)
      if (a.mode == AMK_ACCESS_WRITE &&
          (s.buffers[a.buf].kind == AMK_BUF_OUTPUT || s.buffers[a.buf].kind == AMK_BUF_STATE)) {
        if (!live[i]) { live[i] = 1; work.push_back(i); }
      }
  Csr rf;
  rf.build(nt, flow);
  while (!work.empty()) {
    int32_t r = work.back();
    work.pop_back();
    for (int32_t e = rf.off[r]; e < rf.off[r + 1]; ++e)
      if (!live[rf.adj[e]]) { live[rf.adj[e]] = 1; work.push_back(rf.adj[e]); }
  }
  for (int32_t i = 0; i < nt; ++i)
    if (!live[i]) return verdict(AMK_V_OUTPUT, i);
  return verdict(AMK_V_OK);
}

// Multi-step safety: the smallest task that is not a happens-before
// ancestor (queue edges and full-join wait edges, transitively) of any
// LM-head task, -1 when every task is one, -2 without LM-head tasks.
int32_t multistep_unsafe_task(const amk_schedule& s) {
  const int32_t nt = (int32_t)s.tasks.size(), nc = s.n_counters;
  const std::vector<uint32_t> P = counter_producers(s);
  // reverse edges of the happens-before graph: waiter -> counter -> producer,
  // queue successor -> predecessor
  std::vector<std::pair<int32_t, int32_t>> rev;
  for (int32_t i = 0; i < nt; ++i) {
    for (int32_t c : s.tasks[i].sigs)
      if (c >= 0 && c < nc) rev.push_back({nt + c, i});
    for (const Wait& w : s.tasks[i].waits)
      if (w.ctr >= 0 && w.ctr < nc && w.thr == P[w.ctr]) rev.push_back({i, nt + w.ctr});
  }
  for (const auto& q : s.queues)
    for (size_t i = 1; i < q.size(); ++i)
      if (q[i] >= 0 && q[i] < nt && q[i - 1] >= 0 && q[i - 1] < nt) rev.push_back({q[i], q[i - 1]});
  Csr g;
  g.build(nt + nc, rev);
  std::vector<char> anc(nt + nc, 0);
  std::vector<int32_t> work;
  for (int32_t i = 0; i < nt; ++i)
    if (s.tasks[i].type == AMK_TASK_LMHEAD) {
      anc[i] = 1;
      work.push_back(i);
    }
  if (work.empty()) return -2;
  while (!work.empty()) {
    const int32_t v = work.back();
    work.pop_back();
    for (int32_t e = g.off[v]; e < g.off[v + 1]; ++e)
      if (!anc[g.adj[e]]) {
        anc[g.adj[e]] = 1;
        work.push_back(g.adj[e]);
      }
  }
  for (int32_t i = 0; i < nt; ++i)
    if (!anc[i]) return i;
  return -1;
}

}  // namespace amk
