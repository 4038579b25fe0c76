// Internal declarations of the amk library: Schedule IR, buffer table,
// packed weight layouts and the device task record.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/amk.h"

namespace amk {

// ------------------------------------------------------------- errors --
void set_error(const std::string& msg);
amk_status fail(amk_status st, const std::string& msg);

// ------------------------------------------------------------ buffers --
// Fixed buffer enumeration of a lowered schedule.  KV_HIST / KV_CUR are the
// validator's two views of the one physical KV cache: rows before this
// step's position (read-only inside a step) and the row at the position
// (written by the QKV tasks).  Splitting them is sound because every task of
// one launch sees the same position and only that row is written.
enum BufferId : int32_t {
  B_EMBED = 0,
  B_FINAL_NORM = 1,
  B_LM = 2,
  B_KV_HIST = 3,
  B_KV_CUR = 4,
  B_LOGITS = 5,
  B_X = 6,     // fp32 [L][2][H]: slot 0 after attention, slot 1 after the MLP
  B_Q = 7,     // fp32 [L][nq*hd] rotated queries
  B_PART = 8,  // fp32 [L][nq][S][hd+2] attention partials (o[hd], max, sum)
  B_O = 9,     // fp32 [L][nq*hd] merged attention output
  B_A = 10,    // fp32 [L][F] silu(gate)*up
  B_LAYER0 = 11
};
enum LayerBuf : int32_t { LB_ATTN_NORM = 0, LB_QKV = 1, LB_O = 2, LB_MLP_NORM = 3, LB_GATEUP = 4, LB_DOWN = 5 };
inline int32_t layer_buf(int32_t l, int32_t k) { return B_LAYER0 + 6 * l + k; }
inline int32_t n_buffers(const amk_model_config& m) { return B_LAYER0 + 6 * m.n_layers; }

// packed tensor k <-> buffer id: 0 embed, 1 final norm, 2 lm head, then 6 per layer
inline int32_t packed_to_buffer(int32_t k) { return k < 3 ? k : B_LAYER0 + (k - 3); }

// -------------------------------------------------------- packed layout --
// A packed projection with R rows of K inputs is stored as
//   bf16: [R][K] bf16
//   int8: [R][K] bytes (q + 128, so a byte converts to float directly)
//         then [R] fp32 scales
//   int4: [R][K/2] bytes, nibble order permuted inside each 32-bit word so
//         that (w >> 4j) & 0x000F000F yields columns (2j, 2j+1) of an 8-column
//         chunk as the low nibbles of the two 16-bit halves,
//         then [R][K/128] {fp16 scale, fp16 zero}
struct ProjLayout {
  int32_t fmt = AMK_W_BF16;
  int64_t rows = 0, cols = 0;
  int64_t data_row_bytes() const {
    return fmt == AMK_W_BF16 ? cols * 2 : (fmt == AMK_W_INT8_ROW ? cols : cols / 2);
  }
  int64_t data_bytes() const { return rows * data_row_bytes(); }
  int64_t meta_row_bytes() const {
    return fmt == AMK_W_BF16 ? 0 : (fmt == AMK_W_INT8_ROW ? 4 : (cols / 128) * 4);
  }
  int64_t meta_offset() const { return data_bytes(); }
  int64_t total_bytes() const { return data_bytes() + rows * meta_row_bytes(); }
};

// layout of packed tensor k (norms and the embedding are plain bf16 vectors /
// matrices and are described as bf16 "projections" too)
ProjLayout packed_layout(const amk_model_config& m, int32_t k);

// ---------------------------------------------------------------- IR --
struct Wait { int32_t ctr; uint32_t thr; };
struct Access { int32_t buf, mode; int64_t begin, end; };
struct Task {
  int32_t type = AMK_TASK_NOP, cu = 0;
  int32_t p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  std::vector<Wait> waits;
  std::vector<int32_t> sigs;
  std::vector<Access> acc;
};
struct Buffer { int64_t size; int32_t kind; };

}  // namespace amk

struct amk_schedule {
  amk_model_config model{};
  amk_schedule_config config{};
  std::vector<amk::Task> tasks;
  std::vector<std::vector<int32_t>> queues;  // per CU, task ids in order
  int32_t n_counters = 0;
  std::vector<amk::Buffer> buffers;
  // flat view storage (filled by amk_schedule_view)
  mutable std::vector<amk_task_desc> v_tasks;
  mutable std::vector<int32_t> v_wait_off, v_sig_off, v_acc_off, v_queue_off, v_queue, v_sigs;
  mutable std::vector<amk_wait_desc> v_waits;
  mutable std::vector<amk_access_desc> v_acc;
  mutable std::vector<amk_buffer_desc> v_buffers;
};

namespace amk {

// model / config checks shared by lowering and engine
amk_status check_model(const amk_model_config& m);
amk_status resolve_config(const amk_model_config& m, const amk_schedule_config& in,
                          amk_schedule_config* out);
// the automatic attention split count (ScheduleConfig attn_splits = 0)
int32_t default_attn_splits(const amk_model_config& m, int32_t num_cus);

// standard buffer table of a lowered model
std::vector<Buffer> buffer_table(const amk_model_config& m, int32_t attn_splits);

// Accesses a typed task performs, derived from (type, params); false if the
// params are out of range for the model.  NOP tasks have no derivation.
bool derive_accesses(const amk_model_config& m, const Task& t, std::vector<Access>* out);

// canonical order of an access list (buffer, begin, end, mode)
void sort_accesses(std::vector<Access>* a);

amk_verdict validate(const amk_schedule& s);

// Greedy multi-step launches (amk_decode_steps) start step s + 1 on each
// queue once every LM-head task of step s has stored its argmax partial, so
// they are safe only if every task happens-before some LM-head task (then no
// step s + 1 store can overtake a step s read).  Returns the smallest task
// that is not such an ancestor, -1 if there is none, -2 if the schedule has
// no LM-head task.  Expects a schedule that passed validate().
int32_t multistep_unsafe_task(const amk_schedule& s);

// ----------------------------------------------------- device records --
constexpr int kMaxWaits = 4;
constexpr int kMaxSigs = 4;
constexpr int kCounterStride = 32;  // u32 per counter: one 128-byte line each

// One 128-byte line per task (the table is 128-byte aligned), with every
// field the wait and the signal read in it.
struct alignas(128) DevTask {
  int32_t type, id;
  int8_t nwait, nsig;
  int8_t qslot;    // parity of the task's position in its queue (wait-flag slot)
  int8_t pf_have;  // weight steps per wave already in LDS when the task starts (0: none)
  int32_t pf_lds;  // LDS byte offset of that prefetch area (wave w at + w*pf_have*step bytes)
  int32_t p[6];    // task params (typed tasks use at most 4)
  int32_t wctr[kMaxWaits];
  uint32_t wthr[kMaxWaits];
  uint32_t wprod[kMaxWaits];  // producers of the counter (epoch stride)
  int32_t sctr[kMaxSigs];
  // weights this task prefetches for the next task of its queue, after its
  // signal: packed tensor, rows per unit, steps per wave (0: none), inputs per
  // row, LDS byte offset, first row, units, rows of the whole tensor
  int16_t pfn_tensor;
  int8_t pfn_rpu, pfn_steps;
  int32_t pfn_K, pfn_lds, pfn_row0, pfn_nunits, pfn_rows_total;
};
static_assert(sizeof(DevTask) == 128, "device task record is 128 bytes");

// number of producers of every counter
std::vector<uint32_t> counter_producers(const amk_schedule& s);

}  // namespace amk
