/*
 * amk.h: C ABI of the MI355X persistent decode megakernel.
 *
 * The library runs one batch-1 autoregressive decode step of a Llama-style
 * decoder as ONE persistent cooperative HIP launch: one workgroup per queue
 * (one queue per compute unit), each walking its slice of a topologically
 * ordered task DAG with wait -> dispatch -> signal on monotonic counters.
 * This is the design the AutoMegaKernel summary pages describe ("AutoMegaKernel
 * (AMK)" technical summary, section "Methodology": layer 0 is a persistent
 * kernel with one cooperative block per multiprocessor and a local queue per
 * block over a global topological order, synchronised by monotonic counters
 * without locks; layer 1 holds the GEMV / attention / RMSNorm micro-kernels;
 * layer 2 lowers the model to a typed Schedule IR configured by a
 * ScheduleConfig with tiling, fusion, SM assignment and pipelining depth).
 * The problem it addresses is the one in that page's section "Problem
 * statement": single-stream batch-1 decode is bound by HBM bandwidth, with a
 * latency floor of weight bytes over bandwidth.
 *
 * Entry points, in the order a caller uses them: amk_default_schedule_config
 * -> amk_build_schedule -> amk_validate (the static safety gate) ->
 * amk_pack_tensor (weights into the device layout) -> amk_engine_create ->
 * amk_decode_step per token (or amk_decode_steps for n greedy tokens in one
 * launch) -> amk_engine_check; amk_engine_set_trace / read_trace /
 * region_stats time the tasks of a launch.  The dependency edges of the
 * schedule are carried either by the counters or, by default, by tagged
 * activation words (amk_schedule_config.sync_mode).
 *
 * Conventions (all entry points):
 *   - plain C types only; no exception crosses the ABI; every call that can
 *     fail returns amk_status and leaves a message in amk_last_error();
 *   - "host" pointers are CPU memory, "device" pointers are HIP device memory
 *     on the current device; the caller owns every buffer it passes in;
 *   - the library owns the opaque handles it returns and frees them in the
 *     matching *_free / *_destroy call.
 */
#ifndef AMK_H
#define AMK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AMK_OK = 0,
  AMK_ERR_INVALID_ARG = -1,      /* null pointer, bad size, gap in positions */
  AMK_ERR_UNSUPPORTED = -2,      /* model or schedule variant not supported */
  AMK_ERR_UNSAFE_SCHEDULE = -3,  /* the static safety gate rejected it */
  AMK_ERR_OUT_OF_RANGE = -4,     /* token / position / id out of range */
  AMK_ERR_HIP = -5,              /* a HIP runtime call failed */
  AMK_ERR_NOMEM = -6,            /* host or device allocation failed */
  AMK_ERR_TIMEOUT = -7           /* a device-side wait exceeded its budget */
} amk_status;

/* Weight storage formats ("Quantised megakernels" contribution of the AMK
 * summary: int8 and int4 weight-only kernels from the same IR path). */
typedef enum {
  AMK_W_BF16 = 0,       /* bf16 [out][in] */
  AMK_W_INT8_ROW = 1,   /* int8, one fp32 scale per output row */
  AMK_W_INT4_G128 = 2   /* int4, groups of 128 inputs, fp16 scale + fp16 zero */
} amk_wfmt;

/* Llama-family decoder shape.  Biased projections are not supported
 * (the AMK summary's "Automatic generation coverage" contribution: variants
 * with biased projections are rejected): attn_bias / mlp_bias must be 0, else
 * amk_build_schedule returns AMK_ERR_UNSUPPORTED. */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, max_ctx;
  float rms_eps, rope_theta;
  int32_t tied_embeddings; /* lm_head = token embedding */
  int32_t attn_bias, mlp_bias;
  int32_t wfmt;            /* amk_wfmt of the 7 projections per layer and lm_head */
  int32_t act_bf16;        /* 1: round every projection input vector to bf16 */
} amk_model_config;

/* The ScheduleConfig (AMK summary, "Methodology", layer 2): tiling, fusion,
 * compute-unit assignment and pipelining depth.  0 in a tiles_* / attn_splits
 * field means "automatic".  Tiles are tasks per phase; rows per task follow
 * (an even split of the phase's output rows). */
typedef struct {
  int32_t num_cus;         /* queues = workgroups of the persistent launch */
  int32_t wg_threads;      /* threads per workgroup: 512 */
  int32_t tiles_qkv, tiles_o, tiles_gateup, tiles_down, tiles_lm;
  int32_t attn_splits;     /* position splits per kv head (log-sum-exp merged);
                            * automatic: 3/4 of num_cus / n_kv_heads, so that
                            * a quarter of the queues run no attention split;
                            * (num_cus - n_heads) / n_kv_heads when max_ctx >
                            * 4096 (one split-free queue per query head, for
                            * its merge); min(8, num_cus / n_kv_heads) when
                            * max_ctx <= 512 */
  int32_t cu_policy;       /* 0: task i of T -> queue i*num_cus/T; 1: i % num_cus */
  int32_t pipeline_depth;  /* 16-byte weight loads in flight per lane: 4, 8, 16
                            * (amk_default_schedule_config: 4 for int4
                            * weights, 8 otherwise) */
  uint32_t fuse_flags;     /* AMK_FUSE_* bits; only AMK_FUSE_DEFAULT is built */
  /* Queue-walk knobs (no effect on the DAG the safety gate checks):
   * poll_mode 0: the polling wave issues its weight prologue before the
   *   wait like the others; 1: after the wait (its poll is then not queued
   *   behind its own loads); 2: every wave issues half of its ring before
   *   the wait and half once the wait is over, so that loads issued after
   *   the input arrived keep HBM busy while the input is staged.
   *   amk_default_schedule_config: 2 where the LDS prefetch runs (bf16
   *   weights, hidden >= 4096), 1 otherwise.
   * prefetch_kb: LDS kilobytes per task into which the end of the previous
   *   task of the queue copies the task's first weight slabs (LDS DMA), so
   *   streaming goes on through waits; 0 = 64 KB for bf16 weights with
   *   hidden >= 4096 (the measured best on the 8B shape) and off otherwise
   *   (the measured best on the int8 / int4 and 1B workloads), -1 = off.
   * release_mode 0: all waves wait for their stores, barrier, then the
   *   release; 1: the epilogue stores and the release are issued by the
   *   polling wave alone while the others start the next task. */
  int32_t poll_mode, release_mode, prefetch_kb;
  /* Relative work per XCD and GEMV phase (permille; 0 = 1000), indexed
   * [AMK_PHASE_*][xcd]: the rows of each phase are split over the queues in
   * proportion to the weight of the XCD that runs each queue (queue c runs
   * on XCD c % 8, the round-robin placement of workgroups over the 8 XCDs),
   * to even out XCD speed differences, which differ from phase to phase. */
  int32_t xcd_weight[5][8];
  /* Share (permille; 0 = default 1000) of an even O-projection tile given to
   * queues that also run a MERGE task of the layer: those queues reach the
   * O-projection late, so they get fewer of its rows. */
  int32_t merge_o_share;
  /* merge_place 0: MERGE tasks spread over the queues that run no attention
   * split of the layer (when there are such queues); 1: spread over all
   * queues like the other phases. */
  int32_t merge_place;
  /* LDS kilobytes prefetched for a GEMV task whose queue runs attention work
   * (ATTN or MERGE tasks) just before it: the O-projection.  HBM is mostly
   * idle during attention, so the default (0) takes all that fits; -1 uses
   * prefetch_kb (and is off when that is off); otherwise 1..1024.  A MERGE task between the two is
   * skipped: the task before it issues the copy, so that the merge does not
   * wait behind it. */
  int32_t prefetch_attn_kb;
  /* How a task learns that its inputs are written (the dependency edges of
   * the schedule stay the same):
   * 0: counters.  A producer waits for its stores, then adds 1 to each
   *    counter it signals; a consumer polls its counters, then reads.
   * 1: tagged activations.  Every value one task hands to another is stored
   *    as a 64-bit word {float, launch tag} in one single-copy-atomic store;
   *    a consumer reads the words it needs and re-reads those that do not
   *    yet carry this launch's tag.  No counter traffic, and the read is the
   *    wait.
   * 2: as 1, except the FFN activation (gate/up -> down, ffn values read in
   *    full by every down task): it keeps the counter, so that those reads
   *    move 4 bytes per value instead of 8.
   * 1 and 2 need attn_splits <= 512 and attn_splits * head_dim <= 8192. */
  int32_t sync_mode;
} amk_schedule_config;

enum { AMK_PHASE_QKV = 0, AMK_PHASE_O = 1, AMK_PHASE_GATEUP = 2, AMK_PHASE_DOWN = 3, AMK_PHASE_LM = 4 };

#define AMK_FUSE_NORM_PROLOGUE 0x1u  /* RMSNorm recomputed inside each GEMV task */
#define AMK_FUSE_ROPE_KV 0x2u        /* RoPE + KV append in the QKV task */
#define AMK_FUSE_SWIGLU 0x4u         /* silu(gate)*up in the gate/up task */
#define AMK_FUSE_RESIDUAL 0x8u       /* residual add in the O / down epilogue */
#define AMK_FUSE_DEFAULT 0xFu

/* ---- Schedule IR, flat view ------------------------------------------- */

typedef enum {
  AMK_TASK_NOP = 0,     /* waits and signals only; accesses as declared */
  AMK_TASK_QKV = 1,     /* p: layer, unit0, unit1 (rope pair units) */
  AMK_TASK_ATTN = 2,    /* p: layer, kv head, split, n_splits */
  AMK_TASK_MERGE = 3,   /* p: layer, q head, n_splits */
  AMK_TASK_OPROJ = 4,   /* p: layer, row0, row1 */
  AMK_TASK_GATEUP = 5,  /* p: layer, j0, j1 */
  AMK_TASK_DOWN = 6,    /* p: layer, row0, row1 */
  AMK_TASK_LMHEAD = 7,  /* p: row0, row1 */
  AMK_TASK_NTYPES = 8
} amk_task_type;

typedef enum {
  AMK_BUF_WEIGHT = 0,   /* read-only input */
  AMK_BUF_SCRATCH = 1,  /* activations inside one step */
  AMK_BUF_OUTPUT = 2,   /* logits */
  AMK_BUF_STATE = 3,    /* KV row written at this step's position */
  AMK_BUF_HISTORY = 4   /* KV rows before this step's position (read-only) */
} amk_buffer_kind;

#define AMK_ACCESS_READ 1
#define AMK_ACCESS_WRITE 2

/* Buffers of a schedule built by amk_build_schedule (ids in a schedule view):
 *   0 embedding (packed tensor 0)    1 final norm (packed 1)   2 LM head (packed 2)
 *   3 KV history [L][2][nkv][max_ctx][hd] bf16     4 KV row of this step [L][2][nkv][hd] bf16
 *   5 logits fp32 [V]     6 x fp32 [L][2][H] (after attention, after MLP of layer l)
 *   7 q fp32 [L][nq][hd]  8 attention partials fp32 [L][nq][S][hd + 2]
 *   9 o fp32 [L][nq][hd]  10 a fp32 [L][F]
 *   11 + 6l + {0 attn norm, 1 qkv, 2 o, 3 mlp norm, 4 gate/up, 5 down}: packed 3 + 6l + ...
 * Byte ranges [begin, end) that a typed task declares (and the safety gate
 * re-derives), with x_in(l, r0, r1) = all of buffer 0 when l = 0, else x of
 * layer l-1 "after MLP" rows [r0, r1); "rows [a, b) of packed tensor T" =
 * data bytes [a*rb, b*rb) plus, for int8 / int4, meta bytes [D + a*mb, D + b*mb)
 * (rb, mb = data and meta bytes per row, D = rows*rb):
 *   QKV (l, u0, u1): read x_in(l, 0, H), attn norm (all), rows [2u0, 2u1) of qkv;
 *     per head slot hs touched by units [u0, u1) (unit u = hs*hd/2 + i), with
 *     i in [i0, i1): write q[l][hs] (hs < nq) or the KV row of layer l, K for
 *     slot nq..nq+nkv-1, V after (slot g), elements [i0, i1) and
 *     [hd/2 + i0, hd/2 + i1), as two ranges.
 *   ATTN (l, g, s, S): read q[l][g*grp .. (g+1)*grp) (grp = nq/nkv), per
 *     K then V: history rows of (l, K/V, g) (all max_ctx) and the KV row of
 *     (l, K/V, g); write partial (l, h, s) for each h of the group.
 *   MERGE (l, h, S): read partials (l, h, 0..S); write o[l][h].
 *   OPROJ (l, r0, r1): read o[l] (all), x_in(l, r0, r1), rows [r0, r1) of o;
 *     write x[l][0] rows [r0, r1).
 *   GATEUP (l, j0, j1): read x[l][0] (all), mlp norm (all), rows [2j0, 2j1)
 *     of gate/up; write a[l] [j0, j1).
 *   DOWN (l, r0, r1): read a[l] (all), x[l][0] rows [r0, r1), rows [r0, r1)
 *     of down; write x[l][1] rows [r0, r1).
 *   LMHEAD (r0, r1): read x[L-1][1] (all), final norm (all), rows [r0, r1)
 *     of the LM head; write logits [r0, r1).
 * Params out of range (layer, head, split, rows) make the task invalid (REF). */

typedef struct { int32_t type, cu; int32_t p[8]; } amk_task_desc;
typedef struct { int32_t counter; uint32_t threshold; } amk_wait_desc;
typedef struct { int32_t buffer, mode; int64_t begin, end; } amk_access_desc; /* bytes [begin,end) */
typedef struct { int64_t size; int32_t kind; int32_t reserved; } amk_buffer_desc;

/* Flat, caller-readable view of a schedule.  CSR arrays: the waits of task i
 * are waits[wait_off[i] .. wait_off[i+1]), likewise signals and accesses;
 * queue c is queue[queue_off[c] .. queue_off[c+1]) in execution order. */
typedef struct {
  amk_model_config model;
  amk_schedule_config config;
  int32_t n_tasks, n_counters, n_buffers, n_cus;
  const amk_task_desc* tasks;
  const int32_t* wait_off; const amk_wait_desc* waits;
  const int32_t* sig_off;  const int32_t* sigs;
  const int32_t* acc_off;  const amk_access_desc* accesses;
  const int32_t* queue_off; const int32_t* queue;
  const amk_buffer_desc* buffers;
} amk_schedule_desc;

typedef struct amk_schedule amk_schedule;   /* opaque, host only */
typedef struct amk_engine amk_engine;       /* opaque, binds a schedule to device memory */

/* Validator verdict (AMK summary, "Methodology", the safety gate: deadlock
 * freedom = acyclic producer/consumer DAG, satisfiable thresholds
 * 1 <= t <= #producers, valid per-SM queue orders; race freedom = shared
 * multi-producer counters fully joined before a consumer waits, memory
 * accesses ordered by happens-before; correctness = output reachability and
 * referential integrity).  code 0 = safe, else the first failing rule:
 *   1 REF, 2 THRESHOLD, 3 CYCLE, 4 QUEUE_ORDER, 5 UNDER_JOINED, 6 RACE,
 *   7 OUTPUT.  task / counter / aux name the smallest offender (-1 if none;
 *   for RACE, task < aux is the racing pair; for OUTPUT with task -1, aux is
 *   the buffer that is not fully written). */
typedef struct { int32_t code, task, counter, aux; } amk_verdict;

enum { AMK_V_OK = 0, AMK_V_REF = 1, AMK_V_THRESHOLD = 2, AMK_V_CYCLE = 3, AMK_V_QUEUE_ORDER = 4,
       AMK_V_UNDER_JOINED = 5, AMK_V_RACE = 6, AMK_V_OUTPUT = 7 };

/* Device buffers, all owned by the caller.  weights[k] is the packed tensor k
 * (k < amk_packed_count), written with amk_pack_tensor and copied to the
 * device; kv_cache holds amk_kv_bytes bytes laid out
 * [n_layers][2 (K,V)][n_kv_heads][max_ctx][head_dim] bf16; logits holds
 * vocab fp32 values. */
typedef struct {
  const void* const* weights;
  int32_t n_weights;
  void* kv_cache;
  float* logits;
} amk_device_buffers;

/* ---- configuration ------------------------------------------------------ */

/* Default ScheduleConfig for a model on a device with device_cus compute
 * units (one queue per CU): every field resolved; sync_mode 1 where the
 * attention split count allows it, else 0.  (A zero-filled config passed to
 * amk_build_schedule resolves the same way except that its sync_mode 0
 * stays the counter protocol.) */
amk_status amk_default_schedule_config(const amk_model_config* model, int32_t device_cus,
                                       amk_schedule_config* out);

/* ---- lowering and the safety gate ---------------------------------------- */

/* Lower the model to a typed Schedule DAG (AMK summary, "Methodology",
 * layer 2): fused tasks, tiles, queue assignment, one counter per join, and
 * per-queue orders taken from one global topological order.  Host only.
 * AMK_ERR_UNSUPPORTED for biased projections, n_heads % n_kv_heads != 0, odd
 * head_dim, widths the weight format cannot tile, or an unbuilt fuse_flags
 * combination; AMK_ERR_INVALID_ARG for non-positive sizes. *out is owned by
 * the library (amk_schedule_free). */
amk_status amk_build_schedule(const amk_model_config* model, const amk_schedule_config* config,
                              amk_schedule** out);

/* The static safety gate (AMK summary, "Methodology", "The safety gate"),
 * rules checked in this order, the first failure reported:
 *   V1 REF: queue entries name tasks; each task sits in exactly one queue,
 *      that of its cu; counters, buffers, modes and byte ranges in range;
 *      a typed task declares exactly the accesses listed above.
 *   V2 THRESHOLD: every wait (C, t) has 1 <= t <= P(C), P(C) = number of
 *      signal entries naming C.
 *   V3 CYCLE: producer -> waiter edges are acyclic.
 *   V4 QUEUE_ORDER: producer -> waiter edges plus queue edges are acyclic.
 *   V5 UNDER_JOINED: a partial wait (t < P(C)) by a task that reads bytes a
 *      producer of C writes.
 *   V6 RACE: overlapping accesses of two tasks, one a write, not ordered by
 *      happens-before (queue edges and full-join producer -> waiter edges).
 *   V7 OUTPUT: each OUTPUT buffer fully written, and every task reaches,
 *      through happens-before-ordered writer -> reader data flow, a task
 *      writing an OUTPUT or STATE buffer.
 * AMK_OK iff the schedule is safe, else AMK_ERR_UNSAFE_SCHEDULE with *out
 * naming the first failure.  Host only, never touches a GPU. */
amk_status amk_validate(const amk_schedule* schedule, amk_verdict* out);

/* Whether a schedule may run greedy multi-step launches (amk_decode_steps).
 * Step s + 1 starts on a queue once that queue finished step s and every
 * LM-head task of step s stored its argmax partial; so every task must
 * happen-before some LM-head task (through queue order and full-join waits,
 * the gate's happens-before), else a step s + 1 store could overtake a read
 * of step s that is still running.  AMK_OK if that holds (*task = -1);
 * AMK_ERR_UNSUPPORTED with *task = the smallest task that is no such
 * ancestor (or -2: no LM-head task); AMK_ERR_UNSAFE_SCHEDULE if the gate
 * (amk_validate) rejects the schedule.  Host only. */
amk_status amk_multistep_check(const amk_schedule* schedule, int32_t* task);

/* Flat view of a schedule; the arrays stay valid until amk_schedule_free. */
amk_status amk_schedule_view(const amk_schedule* schedule, amk_schedule_desc* out);

/* Build a schedule from a caller-made description (hand-written or mutated
 * schedules for the validator).  Copies everything; nothing is checked
 * beyond array presence (that is amk_validate's job). */
amk_status amk_schedule_from_desc(const amk_schedule_desc* desc, amk_schedule** out);

void amk_schedule_free(amk_schedule* schedule);

/* ---- weights and KV cache ------------------------------------------------ */

/* Number of packed weight tensors of a model: 3 + 6 * n_layers
 * (0 embedding, 1 final norm, 2 lm_head, then per layer attn_norm, qkv, o,
 * mlp_norm, gate/up, down). */
amk_status amk_packed_count(const amk_model_config* model, int32_t* out);

/* Byte size of packed tensor k in device layout. */
amk_status amk_packed_bytes(const amk_model_config* model, int32_t k, size_t* bytes);

/* Pack (and for int8 / int4 models quantise) packed tensor k from canonical
 * bf16 host tensors.  canonical[id] points to canonical tensor id in Hugging
 * Face [out][in] order (0 embedding, 1 + 9l + {0 attn_norm, 1 wq, 2 wk, 3 wv,
 * 4 wo, 5 mlp_norm, 6 w_gate, 7 w_up, 8 w_down}, 1 + 9L final_norm,
 * 2 + 9L lm_head, unused when tied); only the ids packed tensor k needs are
 * read.  dst is host memory of amk_packed_bytes bytes.  Quantisation, in
 * fp32 with round-half-even: int8 per output row s = amax/127 (all-zero
 * row: s = 1), q = clamp(round(w/s), -127, 127); int4 per group of 128
 * input columns s = fp16((max - min)/15) (0 -> 1), z = clamp(round(-min/s),
 * 0, 15), q = clamp(round(w/s) + z, 0, 15). */
amk_status amk_pack_tensor(const amk_model_config* model, int32_t k,
                           const uint16_t* const* canonical, void* dst);

/* Inverse of the layout part of amk_pack_tensor for one canonical projection
 * inside packed tensor k (wq / wk / wv inside qkv, w_gate / w_up inside
 * gate/up; canonical_id picks which).  Writes the canonical quantised values:
 * bf16 bits (uint16 [rows][cols]); int8 q (int8 [rows][cols]) + fp32 scales;
 * int4 bytes (uint8 [rows][cols/2], low nibble = even column) + fp16 scales +
 * fp16 zeros ([rows][cols/128]).  Unused outputs may be null. */
amk_status amk_unpack_tensor(const amk_model_config* model, int32_t k, int32_t canonical_id,
                             const void* packed, void* q_out, void* scale_out, void* zero_out);

/* KV-cache bytes: n_layers * 2 * n_kv_heads * max_ctx * head_dim * 2. */
amk_status amk_kv_bytes(const amk_model_config* model, size_t* bytes);

/* ---- engine ---------------------------------------------------------------- */

/* Bind a schedule to caller device buffers on the current HIP device.
 * Calls amk_validate first and refuses unsafe schedules with
 * AMK_ERR_UNSAFE_SCHEDULE before anything reaches the GPU (AMK summary,
 * "Methodology": a schedule that fails the checks is rejected immediately).
 * Also refuses a schedule whose queues exceed the co-resident workgroups of
 * the device (AMK_ERR_UNSUPPORTED).  Allocates the library's sync region
 * (counters + activation scratch) and uploads the task table. */
amk_status amk_engine_create(const amk_schedule* schedule, const amk_device_buffers* buffers,
                             amk_engine** out);

/* Bytes of the static device scratch behind amk_engine_create_noalloc. */
#define AMK_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)

/* amk_engine_create without any device allocation, for callers that cannot
 * allocate device memory: code that runs under HIP graph capture, serving
 * loops that must not call hipMalloc, harnesses that forbid allocation.
 * Same checks, same engine and same results as amk_engine_create, but every
 * device region the engine needs (task table, queues, RoPE table,
 * activation scratch, counters, tagged words) is carved from one static
 * device array of AMK_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each device for the life of the process; no hipMalloc, hipFree or other
 * allocating routine is called (regions are zeroed and filled with
 * hipMemset / hipMemcpy).  A schedule whose regions exceed the array ->
 * AMK_ERR_UNSUPPORTED (the message gives both sizes) before anything is
 * written.  The array is shared by every such engine on a device: creating
 * one takes it over, after which an earlier engine from this call on that
 * device fails amk_decode_step / amk_decode_steps / amk_engine_check with
 * AMK_ERR_INVALID_ARG; using two such engines of one device concurrently,
 * or a creation while an earlier engine's launch is still running, races.
 * Tracing (amk_engine_set_trace) needs an allocation and is refused
 * (AMK_ERR_UNSUPPORTED) on these engines.  amk_engine_destroy frees only
 * the host object. */
amk_status amk_engine_create_noalloc(const amk_schedule* schedule, const amk_device_buffers* buffers,
                                     amk_engine** out);

/* One decode step: the logits of `token` at position `pos` (fp32[vocab] into
 * buffers->logits), the KV-cache row `pos` written.  Enqueues exactly one
 * cooperative launch on hip_stream (a hipStream_t, null = default stream) and
 * does not synchronise.  token outside [0, vocab) or pos outside
 * [0, max_ctx) -> AMK_ERR_OUT_OF_RANGE; pos greater than the number of
 * positions written so far -> AMK_ERR_INVALID_ARG; pos at or below it
 * rewinds (rows from pos on are overwritten).  One engine per stream. */
amk_status amk_decode_step(amk_engine* engine, int32_t token, int32_t pos, void* hip_stream);

/* Greedy decoding of n_steps tokens in ONE cooperative launch, the token fed
 * back on the device (the megakernel page's single kernel that also covers
 * the logits and sampling, section on the megakernel design): step s
 * decodes at position pos + s; step 0 consumes `token`, step s > 0 the
 * argmax of step s - 1's logits (lowest index on ties).  tokens_out is a
 * DEVICE int32[n_steps] (caller-owned) that receives the argmax of every
 * step's logits; buffers->logits holds the last step's logits.  Every
 * workgroup computes the argmax itself from one (max, index) partial per
 * LM-head task, so no extra join is added.  n_steps < 1 or pos + n_steps >
 * max_ctx -> AMK_ERR_OUT_OF_RANGE; null tokens_out -> AMK_ERR_INVALID_ARG;
 * otherwise as amk_decode_step. */
amk_status amk_decode_steps(amk_engine* engine, int32_t token, int32_t pos, int32_t n_steps,
                            int32_t* tokens_out, void* hip_stream);
/* (AMK_ERR_UNSUPPORTED, before anything is enqueued, when the engine's
 * schedule fails amk_multistep_check.) */

/* Declare that KV-cache rows 0..n_positions-1 already hold valid state the
 * caller wrote (a restored cache, or a prefix filled outside the library), so
 * the next decode step may use any pos <= n_positions.  0 <= n_positions <=
 * max_ctx, else AMK_ERR_OUT_OF_RANGE. */
amk_status amk_engine_set_kv_length(amk_engine* engine, int32_t n_positions);

/* After the caller synchronised the stream: AMK_ERR_TIMEOUT if a device-side
 * wait gave up (the sync region is then reset and the KV rows of that step
 * are undefined), AMK_OK otherwise. */
amk_status amk_engine_check(amk_engine* engine);

/* The cooperative-launch overhead of a decode step (the measurement the
 * scope table's evidence list asks for; the AMK summary, "Methodology",
 * layer 0, puts the whole forward pass in one launch so that this cost is
 * paid once per token): enqueue one launch of the engine's decode kernel
 * with the same grid, block, LDS and parameters as amk_decode_step, but
 * with every queue empty, so no task runs and nothing is read or written
 * beyond the kernel's own queue offsets.  Asynchronous on hip_stream; the
 * engine's state (positions, counters, tags) is unchanged.  AMK_ERR_INVALID_ARG
 * for a null engine or one whose static scratch was taken over. */
amk_status amk_engine_launch_empty(amk_engine* engine, void* hip_stream);

/* Per-launch spin budget in microseconds for device-side waits (default
 * 2,000,000).  Every wait of a launch gives up once the budget is spent and
 * the launch then drains; amk_engine_check reports it. */
amk_status amk_engine_set_spin_budget(amk_engine* engine, int64_t microseconds);

/* Per-task timing of the following launches (the region timing of the Argus
 * page's megakernel case study, section "Case 3": device-side timestamps of
 * the intervals between phases).  With tracing on, thread 0 of each
 * workgroup stores four wall-clock stamps per task: wait begin, wait end
 * (counters reached, acquire done), work end, signal end.  Off by default;
 * the stamps cost a few scalar instructions per task. */
amk_status amk_engine_set_trace(amk_engine* engine, int32_t enable);

/* Copy the stamps of the last traced launch: out[4*task + k], n_values =
 * 4 * n_tasks; *clock_khz receives the stamp clock rate. */
amk_status amk_engine_read_trace(amk_engine* engine, uint64_t* out, int64_t n_values,
                                 int32_t* clock_khz);

/* Region timing per task type of the last traced launch (device stamps
 * aggregated per region, as the Argus page's megakernel case study,
 * "Case 3", attributes a step's time to its phases).  out[type] for every
 * amk_task_type: tasks of that type, and over them the summed microseconds
 * from wait begin to inputs in hand (wait), to work end (work) and to signal
 * end (signal); span_us sums, over the layers, the time from the last signal
 * of the phase before it in the layer's order (QKV, ATTN, MERGE, OPROJ,
 * GATEUP, DOWN; the previous layer's DOWN before QKV, the launch start
 * before layer 0) to the type's own last signal, so the spans of all types
 * add up to the traced launch's length: each type's share of the critical
 * path.  AMK_ERR_INVALID_ARG if tracing was never enabled. */
typedef struct {
  int32_t n_tasks;
  double wait_us, work_us, signal_us, span_us;
} amk_region_stat;
amk_status amk_engine_region_stats(amk_engine* engine, amk_region_stat out[AMK_TASK_NTYPES]);

/* Host-side count of decode steps since creation (for the caller's bookkeeping). */
amk_status amk_engine_steps(const amk_engine* engine, int64_t* out);

amk_status amk_engine_destroy(amk_engine* engine);

/* Measurement utility, not part of the decode path: one streaming read of
 * `bytes` (a multiple of 16, below 2 GiB) of device memory `src` in the
 * pattern that reaches the highest read rate this device sustains (each of
 * `blocks` workgroups of 512 threads reads one contiguous share in 1 KB
 * slabs, 16 non-temporal 16-byte loads per lane in flight); one float per
 * workgroup may be written to device `out` (blocks floats).  Enqueued on
 * hip_stream; time it with events.  AMK_ERR_INVALID_ARG for null pointers,
 * blocks < 1 or a bad size. */
amk_status amk_stream_read_probe(const void* src, size_t bytes, float* out, int32_t blocks,
                                 void* hip_stream);

/* ---- errors ------------------------------------------------------------------ */

const char* amk_status_string(amk_status status);
const char* amk_last_error(void);  /* thread-local message of the last failure */

#ifdef __cplusplus
}
#endif
#endif /* AMK_H */
