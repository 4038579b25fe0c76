// The persistent decode megakernel for gfx950 (CDNA4) and its engine.
//
// One cooperative launch per decode step (or per n greedy steps); workgroup
// b (512 threads, 8 wave64s) walks queue b of the schedule: for every task it
// waits until its counters reach epoch*P + t, runs the task's micro-kernel,
// and signals its counters (AutoMegaKernel summary, section "Methodology",
// layer 0: one cooperative block per multiprocessor with a local queue over
// a global topological order, wait -> dispatch -> signal on monotonic
// counters, no locks).  With tagged activations (sync_mode 1, the default)
// the same edges are carried by the data: every value handed between tasks
// is a 64-bit {float, launch tag} word, a consumer's read of its inputs is
// its wait and a producer's stores are its signal.  Micro-kernels (layer 1 of the same section): fused RMSNorm
// prologue + GEMV for the projections, RoPE + KV append, split decode
// attention with a log-sum-exp merge, SwiGLU, residual epilogues, LM head.
//
// GEMV design (HBM-bound, batch 1): each wave owns whole output rows (or a
// RoPE / gate-up pair of rows), streams them with 16-byte buffer loads (64
// lanes read 1 KB contiguous per instruction), keeps `DEPTH` loads per lane
// in flight in a register ring, and multiplies against the activation vector
// staged in LDS.  The first DEPTH loads of a task are issued BEFORE its wait,
// so weight streaming continues while the workgroup waits on a counter (the
// "deeper pipelining" the AMK summary names as the remedy for per-tile sync
// cost on high-bandwidth GPUs, section "Experimental results", training-class
// GPUs).  Buffer loads whose offset is past the task's rows return zero
// without touching memory, so ring tails cost no bandwidth.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <cstring>
#include <vector>

#include "amk_internal.h"

namespace amk {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kHead = 16;  // LDS floats: block-reduction slots, wait flags, int8 sum of x
constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kOob = 0x80000000u;       // offset past every descriptor range

// Task records are read-only for the whole launch: reading them through the
// constant address space lets the compiler use scalar loads (scalar cache,
// counted apart from the vector loads that stream weights).
typedef const __attribute__((address_space(4))) DevTask CTask;
typedef CTask& TaskRef;

struct VmParams {
  const DevTask* tasks;
  const int32_t* queue_off;
  const int32_t* queue;
  const uint8_t* const* wptr;  // packed tensors [3 + 6L]
  uint16_t* kv;                // [L][2][nkv][mc][hd] bf16
  float* logits;
  float* x;     // [L][2][H]
  float* q;     // [L][nq*hd]
  float* part;  // [L][nq][S][hd+2]
  float* o;     // [L][nq*hd]
  float* a;     // [L][F]
  uint32_t* ctr;
  int32_t* err;
  uint64_t* trace;  // null, or 4 wall-clock stamps per task (see vm_wait / vm_signal)
  const float2* rope;  // [mc][hd/2] (cos, sin)
  uint64_t spin_ticks;
  int32_t token, pos;
  uint32_t epoch;
  int32_t L, H, nq, nkv, hd, F, V, mc, S, wfmt, act_bf16;
  float eps;
  // LDS offset (floats) of the attention scratch; GEMV tasks place x at
  // kHead and their partial tables right after (xs_floats)
  int32_t lds_att;
  // queue-walk knobs of the schedule configuration
  int32_t poll_late;  // the polling wave issues its weight prologue after the wait
  int32_t rel0;       // epilogue stores and release by wave 0 alone
  // tagged activations (sync_mode 1): every value one task hands to another
  // is a 64-bit word {float bits, launch tag}; a reader spins on the words
  // it needs instead of on counters, a writer only stores
  int32_t tagged;
  int32_t a_tagged;  // the FFN activation (gate/up -> down) is tagged too; else that edge keeps its counter
  uint32_t tag;
  uint64_t* tx;    // [L][2][H] as x
  uint64_t* tq;    // [L][nq*hd] as q
  uint64_t* tkv;   // [L][2][nkv*hd] K (roped) and V of this launch's position, bf16 values
  uint64_t* tpart; // [L][nq][S][hd+2] as part
  uint64_t* to;    // [L][nq*hd] as o
  uint64_t* ta;    // [L][F] as a
  // greedy multi-step decode: n_steps steps in one launch; step s decodes at
  // pos + s with tag + s and epoch + s, its token being the argmax of step
  // s - 1's logits.  LM-head task k stores its rows' (max, index) as two
  // tagged words targ[2k], targ[2k + 1] (its ordinal k is its p[2]).
  int32_t n_steps;
  int32_t n_lm;
  uint64_t* targ;        // [n_lm][2]
  int32_t* tokens_out;   // device int32[n_steps] or null: every step's argmax
};

// ------------------------------------------------------------- helpers --

// threadIdx.x through an opaque move: values derived from it cannot be
// hoisted out of one task into the queue loop, where the per-lane addresses
// of every inlined micro-kernel would otherwise stay live at once.
__device__ __forceinline__ int opaque_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to the nearest bf16 (ties to even); values are finite here
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(bf16_bits(f) << 16); }

// Cross-lane reductions on the VALU with DPP (no LDS crossbar round trips).
// dpp<CTRL, ROWMASK>(old, v): lanes of rows outside ROWMASK keep `old`.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWMASK, 0xF, false));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;
constexpr int kHalfMirror = 0x141, kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// every lane of each 16-lane row gets the row's sum
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kRowRor8>(0.0f, v);
  v += dpp<kRowRor4>(0.0f, v);
  v += dpp<kQuadSwap2>(0.0f, v);
  v += dpp<kQuadSwap1>(0.0f, v);
  return v;
}
// every lane of each 8-lane half row gets the half row's sum
__device__ __forceinline__ float row_sum8(float v) {
  v += dpp<kHalfMirror>(0.0f, v);
  v += dpp<kQuadSwap2>(0.0f, v);
  v += dpp<kQuadSwap1>(0.0f, v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kRowRor8>(v, v));
  v = fmaxf(v, dpp<kRowRor4>(v, v));
  v = fmaxf(v, dpp<kQuadSwap2>(v, v));
  v = fmaxf(v, dpp<kQuadSwap1>(v, v));
  return v;
}
// sum over the 64 lanes, returned uniformly (row sums, then the row
// broadcasts carry rows 0..2 into row 3, then lane 63 is read)
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += dpp<kRowBcast15, 0xA>(0.0f, v);
  v += dpp<kRowBcast31, 0xC>(0.0f, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  v = fmaxf(v, dpp<kRowBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp<kRowBcast31, 0xC>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// the value of lane (lane ^ OFF), OFF = 8, 16 or 32, on the VALU: a row
// rotation by 8 within each 16-lane row, or the row-pair / half-wave swaps
// (the swap returns the two operands with odd rows (upper half) of the first
// and even rows (lower half) of the second exchanged; each lane takes the
// one that holds its partner)
template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (OFF == 8) {
    return dpp<kRowRor8>(v, v);
  } else if constexpr (OFF == 16) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((opaque_tid() & 16) ? r[0] : r[1]);
  } else {
    static_assert(OFF == 32, "lane_xor: OFF is 8, 16 or 32");
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((opaque_tid() & 32) ? r[0] : r[1]);
  }
}

// sum over groups of LG consecutive lanes (LG = 8, 16, 32 or 64), every lane
// of a group gets its group's sum
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LG == 8) return row_sum8(v);
  if constexpr (LG == 16) return row_sum16(v);
  if constexpr (LG == 32) {
    v = row_sum16(v);
    return v + lane_xor<16>(v);
  }
  if constexpr (LG == 64) return wave_sum(v);
  return v;
}

// sum over the workgroup; `red` holds kWaves floats of LDS
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((opaque_tid() & 63) == 0) red[opaque_tid() >> 6] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

// true in every thread when `pred` holds in any thread; `red` holds kWaves
// floats of LDS
__device__ __forceinline__ bool block_any(bool pred, float* red) {
  const bool w = __builtin_amdgcn_ballot_w64(pred) != 0;
  if ((opaque_tid() & 63) == 0) reinterpret_cast<int*>(red)[opaque_tid() >> 6] = w ? 1 : 0;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) any |= reinterpret_cast<const int*>(red)[k];
  __syncthreads();
  return any != 0;
}

// (best, index) over the workgroup: the largest value, the lowest index among
// equal values; the result is in thread 0.  Uses the first 2*kWaves floats
// of `red`.
__device__ __forceinline__ void argmax_block(float& best, int& bi, float* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  __syncthreads();
  const int tid = opaque_tid();
  if ((tid & 63) == 0) {
    red[tid >> 6] = best;
    reinterpret_cast<int*>(red)[kWaves + (tid >> 6)] = bi;
  }
  __syncthreads();
  if (tid == 0)
    for (int w = 1; w < kWaves; ++w) {
      const float ob = red[w];
      const int oi = reinterpret_cast<const int*>(red)[kWaves + w];
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
  __syncthreads();
}

// Stores of data another workgroup reads in the same launch go through at
// agent scope (written through to the device coherence point), so that a
// signal only has to wait for its own stores to complete instead of writing
// back the whole L2 of its XCD.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged words: the value in the low half, the launch's tag in the high half,
// written and read as one aligned 64-bit agent-scope access (single-copy
// atomic), so a word that carries this launch's tag carries this launch's
// value.  Stores go through to the device coherence point; a reader's
// agent-scope loads see them without any fence.
__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tag_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Buffer descriptor over [base, base + bytes).  Base and size are the same in
// every lane; reading them through readfirstlane lets the compiler keep the
// descriptor in scalar registers (a descriptor it must assume divergent
// costs a loop over lanes around every buffer load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), (int)kBufFlags);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache policy of the streamed loads (weights, KV rows): they are read once
// per step, so they carry the non-temporal hint and do not displace what is
// reused from the L2: the kernel's code (an instruction fetch that misses
// the L2 waits behind the weight stream) and the activation vectors.  On
// the 8B shape this alone took a step from 3.34 to 3.15 ms.
#ifndef AMK_STREAM_NT
#define AMK_STREAM_NT 1
#endif
constexpr int kStreamPolicy = AMK_STREAM_NT ? 2 : 0;  // 2 = nt

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy);
}

// poll_mode 3 ("DMA waves"): waves kDmaWave0..7 copy the next task's first
// weight slabs into LDS (LDS DMA) at the end of each task and issue no other
// load before a wait; waves 0..kDmaWave0-1 read every input of a task
// (activations, q and K/V, attention partials).  A wave's loads complete in
// issue order, so an input read issued by a wave with a weight copy in
// flight is only usable after that copy: keeping the two in different
// waves lets a task take its input as soon as it is written.
constexpr int kDmaWave0 = 6;
__device__ __forceinline__ int input_threads(const VmParams& P) {
  return P.poll_late == 3 ? kDmaWave0 * 64 : kThreads;
}
// threads that store what a counter release covers (rel0: wave 0 alone)
__device__ __forceinline__ int epilogue_threads(const VmParams& P) { return P.rel0 ? 64 : input_threads(P); }

// ------------------------------------------------------- wait / signal --

// Thread 0 spins until every wait of the task holds, then performs the
// agent-scope acquire; the workgroup barrier passes the result to all
// threads.  Returns false when the spin budget ran out or another
// workgroup already reported an error (the launch then drains).  The flag
// slot alternates with the task's queue position: waves that run ahead into
// the next task cannot overwrite a flag a slower wave has yet to read.
template <typename Hook>
__device__ __forceinline__ bool vm_wait(const VmParams& P, TaskRef t, int* flags, Hook&& before_barrier) {
  if (P.tagged && (P.a_tagged || t.type != AMK_TASK_DOWN)) {  // the task's reads of tagged words are its wait
    if (P.trace && opaque_tid() == 0) P.trace[(size_t)t.id * 4 + 0] = wall_clock64();
    before_barrier();
    __syncthreads();
    return true;
  }
  int* flag = flags + t.qslot;
  if (opaque_tid() == 0) {
    if (P.trace) P.trace[(size_t)t.id * 4 + 0] = wall_clock64();
    int ok = 1;
    for (int k = 0; k < t.nwait && ok; ++k) {
      const uint32_t target = P.epoch * t.wprod[k] + t.wthr[k];
      uint32_t* c = P.ctr + (size_t)t.wctr[k] * kCounterStride;
      const uint64_t start = wall_clock64();
      uint32_t polls = 0;
      while ((int32_t)(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++polls & 63u) == 0u) {
          if (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
              wall_clock64() - start > P.spin_ticks) {
            ok = 0;
            break;
          }
        }
      }
    }
    if (!ok) __hip_atomic_store(P.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = ok;
    if (P.trace) P.trace[(size_t)t.id * 4 + 1] = wall_clock64();
  }
  before_barrier();
  __syncthreads();
  return *flag != 0;
}

__device__ __forceinline__ bool vm_wait(const VmParams& P, TaskRef t, int* flags) {
  return vm_wait(P, t, flags, [] {});
}

// Spin state of one thread's tagged reads.  again() is called while some
// word lacks the launch's tag: it backs off, and gives up (reporting the
// error to every workgroup) when the spin budget is spent or another
// workgroup already reported one.
struct TagSpin {
  uint64_t start = 0;
  uint32_t polls = 0;
  bool failed = false;
  __device__ __forceinline__ bool again(const VmParams& P) {
    if (start == 0) start = wall_clock64();
    __builtin_amdgcn_s_sleep(1);
    // every re-read is a memory round trip, so the clock is checked each time
    if (wall_clock64() - start > P.spin_ticks ||
        ((++polls & 15u) == 0u && __hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)) {
      __hip_atomic_store(P.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      failed = true;
      return false;
    }
    return true;
  }
};

// The tagged words p[idx(k)] for the k < N with use(k): issued together, then
// re-read until each carries the launch's tag.  v[k] = the value (0 where
// !use(k)).  False when the spin gave up.
template <int N, class Use, class Idx>
__device__ __forceinline__ bool ld_tagged(const VmParams& P, const uint64_t* p, Use&& use, Idx&& idx,
                                          float (&v)[N], TagSpin& sp) {
  const uint64_t ok = (uint64_t)P.tag << 32;
  uint64_t w[N];
#pragma unroll
  for (int k = 0; k < N; ++k) w[k] = use(k) ? ld_tag(p + idx(k)) : ok;
  while (true) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < N; ++k) all = all && (w[k] >> 32) == (ok >> 32);
    if (all) break;
    if (!sp.again(P)) return false;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((w[k] >> 32) != (ok >> 32)) w[k] = ld_tag(p + idx(k));
  }
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = tag_val(w[k]);
  return true;
}

__device__ __forceinline__ void trace_mark(const VmParams& P, TaskRef t, int k) {
  if (P.trace && opaque_tid() == 0) P.trace[(size_t)t.id * 4 + k] = wall_clock64();
}

// Release.  Every store another workgroup reads is a write-through
// agent-scope store, so its completion (vmcnt) means it is visible at the
// device coherence point; lane 0 of wave 0 then bumps each counter with a
// relaxed agent-scope add.  rel0 = 0: all waves wait for their stores and
// meet at a barrier first.  rel0 = 1: only wave 0 issued such stores (the
// epilogue ran on 64 threads), only it waits, and the other waves go on to
// issue the next task's weight loads.

__device__ __forceinline__ void vm_signal(const VmParams& P, TaskRef t) {
  const int tid = opaque_tid();
  if (P.tagged && (P.a_tagged || t.type != AMK_TASK_GATEUP)) {  // the stores were the signal
    if (P.trace && tid == 0) {
      const uint64_t now = wall_clock64();
      P.trace[(size_t)t.id * 4 + 2] = now;
      P.trace[(size_t)t.id * 4 + 3] = now;
    }
    return;
  }
  if (!P.rel0) {
    // (poll_mode 3: the DMA waves stored nothing here and may be copying the
    // next task's weights; they only meet the barrier)
    if (tid < input_threads(P)) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (tid < 64) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid == 0) {
      if (P.trace) P.trace[(size_t)t.id * 4 + 2] = wall_clock64();
      for (int k = 0; k < t.nsig; ++k)
        __hip_atomic_fetch_add(P.ctr + (size_t)t.sctr[k] * kCounterStride, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      if (P.trace) P.trace[(size_t)t.id * 4 + 3] = wall_clock64();
    }
  }
}

// --------------------------------------------------------------- GEMV ---
// Streaming GEMV over `nunits` units of RPU consecutive packed rows (a RoPE or
// gate/up pair when RPU = 2).  A step (unit, j) is one 16-byte load per lane
// and row: 64 lanes cover a 1 KB-wide slab of the row, J slabs per row.  Work
// split over the 8 waves:
//   rounds: while 8 whole units remain, wave w owns unit w of the round, so
//           the 8 waves stream 8 adjacent rows side by side (the workgroup's
//           reads stay within a few DRAM pages);
//   tail:   the R = nunits % 8 last units hold R*J steps; wave w takes the
//           contiguous steps [w*R*J/8, (w+1)*R*J/8) of them in unit-major
//           order, so every wave's share differs by at most one step (a
//           task's time then follows its row count in fine steps, which
//           lets the per-XCD row shares move work between queues).
// So a wave's steps form its round units plus at most one tail range, which
// spans at most two units (a range is shorter than J steps).  Each wave writes
// one partial per unit segment to an LDS table; the finalize pass adds, per
// row, the partials of the waves that covered its unit, in wave order
// (bit-reproducible).  Each
// wave keeps DS steps of loads in flight in a register ring; the first DS are
// issued before the task's wait (for wave 0, which polls, after it when
// poll_late is set: a poll then does not queue behind its own weight loads).
// Buffer loads whose offset lies past the task's rows return zero without
// memory traffic.
struct GemvSplit {
  int J, nr, R, TS;  // slabs per row, rounds, tail units, tail steps
  __device__ __forceinline__ GemvSplit(int nunits, int J_) : J(J_) {
    nr = nunits / kWaves;
    R = nunits - nr * kWaves;
    TS = R * J;
  }
  // tail steps [t0, t1) of wave w; tail step t is slab t % J of unit
  // nr * kWaves + t / J
  __device__ __forceinline__ void tail(int w, int* t0, int* t1) const {
    *t0 = (TS * w) / kWaves;
    *t1 = (TS * (w + 1)) / kWaves;
  }
};

// attention spreads positions over waves 1..7; wave 0 polls
constexpr int kAttnWaves = kWaves - 1;



// Attention splits of at least kAttnPmMin positions take the position-major
// lane layout (every 16-byte load brings distinct rows, so more bytes are in
// flight per register), shorter ones the head-major layout (the heads of a
// pass in parallel lane groups: a shorter chain per position, and q read
// straight into registers).
constexpr int kAttnPmMin = 128;

// Query heads one pass takes.  Head-major: the group size rounded up to a
// power of two, at most 64 lanes / (head_dim / 8 lanes per row).
// Position-major: the group size rounded up to a power of two, at most 4
// (every lane keeps q and the running sums of all heads of its pass in
// registers).  Larger groups take several passes.
__host__ __device__ constexpr int attn_pass_heads_hm(int grp, int hd) {
  return (grp == 1 ? 1 : grp == 2 ? 2 : grp <= 4 ? 4 : 8) < 512 / hd ? (grp == 1 ? 1 : grp == 2 ? 2 : grp <= 4 ? 4 : 8)
                                                                   : 512 / hd;
}
__host__ __device__ constexpr int attn_pass_heads_pm(int grp) { return grp == 1 ? 1 : grp == 2 ? 2 : 4; }

// LDS floats of an attention pass (the engine sizes the attention scratch
// for the larger of the two layouts).  Head-major: every lane's (acc[8],
// max, sum), then the merged heads.  Position-major: q, the row at pos, the
// waves' states and the merged heads.
__host__ __device__ constexpr int attn_lds_floats(int grp, int hd) {
  return (kWaves * 64 * 10 + attn_pass_heads_hm(grp, hd) * (hd + 2)) >
                 (attn_pass_heads_pm(grp) * hd + 2 * hd + (kWaves + 1) * attn_pass_heads_pm(grp) * (hd + 2))
             ? kWaves * 64 * 10 + attn_pass_heads_hm(grp, hd) * (hd + 2)
             : attn_pass_heads_pm(grp) * hd + 2 * hd + (kWaves + 1) * attn_pass_heads_pm(grp) * (hd + 2);
}

// x for 16-byte chunks of E elements, staged so lane l of wave-load j reads
// its E values as E/4 conflict-free float4s: element e (c = e/E, k = e%E,
// j = c/64) at ((j*(E/4) + k/4)*64 + c%64)*4 + k%4.
template <int E>
__device__ __forceinline__ int xperm_e(int e) {
  const int c = e / E, k = e % E;
  return (((c >> 6) * (E / 4) + (k >> 2)) * 64 + (c & 63)) * 4 + (k & 3);
}

__device__ __forceinline__ float f16_to_f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

struct FmtBf16 {
  static constexpr int E = 8;
  static constexpr bool kMeta = false;
  __device__ __forceinline__ static float dot(float t, u32x4 w, uint32_t, const float* xs, int cj, int lane,
                                              const float*) {
    const float4 xa = *reinterpret_cast<const float4*>(xs + ((cj * 2 + 0) * 64 + lane) * 4);
    const float4 xb = *reinterpret_cast<const float4*>(xs + ((cj * 2 + 1) * 64 + lane) * 4);
    t = fmaf(bf16_lo(w.x), xa.x, t);
    t = fmaf(bf16_hi(w.x), xa.y, t);
    t = fmaf(bf16_lo(w.y), xa.z, t);
    t = fmaf(bf16_hi(w.y), xa.w, t);
    t = fmaf(bf16_lo(w.z), xb.x, t);
    t = fmaf(bf16_hi(w.z), xb.y, t);
    t = fmaf(bf16_lo(w.w), xb.z, t);
    t = fmaf(bf16_hi(w.w), xb.w, t);
    return t;
  }
};

// int8 rows hold q + 128: row = s_r * (sum u x - 128 * sum x) (finalize)
struct FmtInt8 {
  static constexpr int E = 16;
  static constexpr bool kMeta = false;
  __device__ __forceinline__ static float dot(float t, u32x4 w, uint32_t, const float* xs, int cj, int lane,
                                              const float*) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(xs + ((cj * 4 + q) * 64 + lane) * 4);
      t = fmaf((float)((wd[q] >> 0) & 0xFFu), x.x, t);
      t = fmaf((float)((wd[q] >> 8) & 0xFFu), x.y, t);
      t = fmaf((float)((wd[q] >> 16) & 0xFFu), x.z, t);
      t = fmaf((float)((wd[q] >> 24) & 0xFFu), x.w, t);
    }
    return t;
  }
};

// int4 rows: a 16-byte chunk is 32 columns (a quarter group of 128) with the
// group's {fp16 scale, fp16 zero}; word q holds columns 8q..8q+7, nibble j
// column 2j and nibble j+4 column 2j+1, so (word >> 4j) & 0x000F000F holds
// the column pair (2j, 2j+1) in its two halves.  OR-ing in 0x4300 per half
// makes the exact bf16 values 128 + q, which meet the staged input (bf16
// high parts and bf16 remainders of x, packed in column pairs, see stage_x)
// in the bf16 dot2 instruction:
//   d = sum (128 + q) (xh + xl),  contribution s * (d - (z + 128) * sum (xh + xl)).
// Three shifts, four and-ors and eight dot2 per 8 columns, where a convert
// and an FMA per column cost 24.
struct FmtInt4 {
  static constexpr int E = 32;
  static constexpr bool kMeta = true;
  __device__ __forceinline__ static float dot2(uint32_t a, uint32_t b, float c) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
  }
  __device__ __forceinline__ static float dot(float acc, u32x4 w, uint32_t m, const float* xs, int cj, int lane,
                                              const float* csum) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    // the mask and the bias as wave-uniform values rather than literals:
    // the compiler then forms one three-operand and-or per pair (a VOP3
    // instruction takes no literal on this target)
    uint32_t kMask, kBias;
    asm("s_mov_b32 %0, 0x000f000f" : "=s"(kMask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(kBias));
    // four independent accumulation chains (the dot2 result latency is
    // several issue slots; one chain per row would leave the SIMD idle)
    float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // all eight input reads first, so their LDS latency overlaps
    u32x4 xv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) xv[k] = *reinterpret_cast<const u32x4*>(xs + ((cj * 8 + k) * 64 + lane) * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 xh = xv[2 * q], xl = xv[2 * q + 1];
      const uint32_t p0 = (wd[q] & kMask) | kBias;
      const uint32_t p1 = ((wd[q] >> 4) & kMask) | kBias;
      const uint32_t p2 = ((wd[q] >> 8) & kMask) | kBias;
      const uint32_t p3 = ((wd[q] >> 12) & kMask) | kBias;
      d[0] = dot2(p0, xh.x, d[0]);
      d[1] = dot2(p0, xl.x, d[1]);
      d[2] = dot2(p1, xh.y, d[2]);
      d[3] = dot2(p1, xl.y, d[3]);
      d[0] = dot2(p2, xh.z, d[0]);
      d[1] = dot2(p2, xl.z, d[1]);
      d[2] = dot2(p3, xh.w, d[2]);
      d[3] = dot2(p3, xl.w, d[3]);
    }
    const float cs = csum[cj * 64 + lane];
    const float dd = (d[0] + d[2]) + (d[1] + d[3]);
    return fmaf(f16_to_f(m & 0xFFFFu), dd - (f16_to_f(m >> 16) + 128.0f) * cs, acc);
  }
};

// x (fp32 or bf16 source, or tagged words when tsrc is set) -> optional
// RMSNorm with bf16 gain -> optional bf16 rounding -> LDS in the chunk
// layout of format F; int8 also gets sum x, int4 the per-chunk sums of x.
// n is a multiple of 8.  False when a tagged read gave up.
// Only the first `nr` threads read memory (the input, the gain); the others
// take part in the LDS passes and barriers.
template <class F>
__device__ __forceinline__ bool stage_x(const VmParams& P, const void* src, const uint64_t* tsrc, int n,
                                        const uint16_t* gain, bool src_bf16, float* xs, float* red, float* xsum,
                                        float* csum, int nr) {
  const bool NORM = gain != nullptr;
  const int tid = opaque_tid(), n4 = n >> 2;
  const bool reader = tid < nr;
  const float eps = P.eps;
  const int act_bf16 = P.act_bf16;
  float ss = 0.0f;
  // the gain of this thread's first two groups of 4 inputs (int4: of its
  // first group of 8), read now so that its round trip overlaps the input's
  constexpr bool G8 = F::E == 32;
  uint2 g2[2] = {{0u, 0u}, {0u, 0u}};
  if (NORM && reader)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int gi = G8 ? 2 * tid + k : tid + k * nr;
      if (gi < n4) g2[k] = reinterpret_cast<const uint2*>(gain)[gi];
    }
  if (tsrc) {  // up to 4 groups of 4 words per thread in flight at once
    TagSpin sp;
    for (int i0 = tid; reader && i0 < n4; i0 += nr * 4) {
      float v[16];
      if (!ld_tagged<16>(P, tsrc, [&](int k) { return i0 + (k >> 2) * nr < n4; },
                         [&](int k) { return 4 * (i0 + (k >> 2) * nr) + (k & 3); }, v, sp))
        break;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = i0 + g * nr;
        if (i < n4) {
          const float4 f = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
          if (NORM) ss += f.x * f.x + f.y * f.y + f.z * f.z + f.w * f.w;
          *reinterpret_cast<float4*>(xs + xperm_e<F::E>(i * 4)) = f;
        }
      }
    }
    if (block_any(sp.failed, red)) return false;
  } else
  for (int i = tid; reader && i < n4; i += nr) {
    float4 v;
    if (src_bf16) {
      const uint2 b = reinterpret_cast<const uint2*>(src)[i];
      v = make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
    } else {
      v = reinterpret_cast<const float4*>(src)[i];
    }
    if (NORM) ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    *reinterpret_cast<float4*>(xs + xperm_e<F::E>(i * 4)) = v;
  }
  constexpr int slab = F::E * 64;  // elements per wave-load
  const int padded = (n + slab - 1) / slab * slab;
  for (int e = n + tid * 4; e < padded; e += kThreads * 4)
    *reinterpret_cast<float4*>(xs + xperm_e<F::E>(e)) = make_float4(0.f, 0.f, 0.f, 0.f);
  float inv = 1.0f;
  if (NORM) inv = 1.0f / sqrtf(block_sum(ss, red) / (float)n + eps);
  else __syncthreads();
  float sx = 0.0f;
  if constexpr (G8) {
    // int4: per group of 8 inputs (one thread; the 4 groups of a chunk of 32
    // in 4 adjacent lanes) the norm, then the split into bf16 high parts xh
    // (4 column pairs, in the group's first slot) and the bf16 roundings xl
    // of the remainders x - xh (second slot): xh + xl is exact in fp32 and
    // within 2^-17 |x| of x.  csum is each chunk's sum of xh + xl, the
    // values the dot products see (chunks wholly in the padding get 0).
    const int n8 = n >> 3;
    for (int g = tid; reader && g < n8; g += nr) {
      float4* pa = reinterpret_cast<float4*>(xs + xperm_e<32>(8 * g));
      float4* pb = reinterpret_cast<float4*>(xs + xperm_e<32>(8 * g + 4));
      float4 a = *pa, b = *pb;
      if (NORM) {
        const uint2 ga = g == tid ? g2[0] : reinterpret_cast<const uint2*>(gain)[2 * g];
        const uint2 gb = g == tid ? g2[1] : reinterpret_cast<const uint2*>(gain)[2 * g + 1];
        a = make_float4(a.x * inv * bf16_lo(ga.x), a.y * inv * bf16_hi(ga.x), a.z * inv * bf16_lo(ga.y),
                        a.w * inv * bf16_hi(ga.y));
        b = make_float4(b.x * inv * bf16_lo(gb.x), b.y * inv * bf16_hi(gb.x), b.z * inv * bf16_lo(gb.y),
                        b.w * inv * bf16_hi(gb.y));
      }
      if (act_bf16) {
        a = make_float4(bf16_round(a.x), bf16_round(a.y), bf16_round(a.z), bf16_round(a.w));
        b = make_float4(bf16_round(b.x), bf16_round(b.y), bf16_round(b.z), bf16_round(b.w));
      }
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t hp[4], lp[4];
      float t = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          hb[e] = bf16_bits(v[2 * j + e]);
          const float xh = __uint_as_float(hb[e] << 16);
          lb[e] = bf16_bits(v[2 * j + e] - xh);
          t += xh + __uint_as_float(lb[e] << 16);
        }
        hp[j] = hb[0] | (hb[1] << 16);
        lp[j] = lb[0] | (lb[1] << 16);
      }
      *reinterpret_cast<u32x4*>(pa) = u32x4{hp[0], hp[1], hp[2], hp[3]};
      *reinterpret_cast<u32x4*>(pb) = u32x4{lp[0], lp[1], lp[2], lp[3]};
      t += __shfl_xor(t, 1);
      t += __shfl_xor(t, 2);
      if ((g & 3) == 0) csum[g >> 2] = t;
    }
    for (int c = (n >> 5) + tid; c < padded / 32; c += kThreads) csum[c] = 0.0f;
  } else
  for (int i = tid; reader && i < n4; i += nr) {
    float4* p = reinterpret_cast<float4*>(xs + xperm_e<F::E>(i * 4));
    float4 v = *p;
    if (NORM) {
      const uint2 g = i == tid ? g2[0] : (i == tid + nr ? g2[1] : reinterpret_cast<const uint2*>(gain)[i]);
      v.x = v.x * inv * bf16_lo(g.x);
      v.y = v.y * inv * bf16_hi(g.x);
      v.z = v.z * inv * bf16_lo(g.y);
      v.w = v.w * inv * bf16_hi(g.y);
    }
    if (act_bf16) v = make_float4(bf16_round(v.x), bf16_round(v.y), bf16_round(v.z), bf16_round(v.w));
    *p = v;
    sx += v.x + v.y + v.z + v.w;
  }
  if constexpr (F::E == 16) {
    const float tot = block_sum(sx, red);
    if (tid == 0) *xsum = tot;
  }
  __syncthreads();

  return true;
}

// Issue order of one wave's steps: its round units (sw, sw + 8, ...) slab by
// slab, then its tail piece.  ik counts steps, (iu, ij) is the next step.
struct StepIter {
  int J, nA, t_unit, t_j0, n;
  int ik, iu, ij;
  __device__ __forceinline__ void init(int sw, int nunits, int J_) {
    J = J_;
    const GemvSplit sp(nunits, J);
    int t0, t1;
    sp.tail(sw, &t0, &t1);
    t_unit = sp.nr * kWaves + t0 / J;
    t_j0 = t0 % J;
    nA = sp.nr * J;
    n = nA + (t1 - t0);
    ik = 0;
    iu = nA ? sw : t_unit;
    ij = nA ? 0 : t_j0;
  }
  // rounds: the next slab, then unit + 8; tail: the next slab, then the next unit
  __device__ __forceinline__ void advance() {
    ++ik;
    if (++ij == J) {
      ij = 0;
      iu += ik <= nA ? kWaves : 1;
    }
    if (ik == nA) {
      iu = t_unit;
      ij = t_j0;
    }
  }
};

// bytes of one row's slab in a prefetch area: 1 KB of weights, for int4 also
// the 64 lanes' group meta words
template <class F>
constexpr uint32_t pf_row_step() { return 1024u + (F::kMeta ? 256u : 0u); }

#if AMK_STREAM_NT
#define AMK_NT_SUFFIX " nt"
#else
#define AMK_NT_SUFFIX ""
#endif

// LDS DMA of 16 (4) bytes per lane from a buffer offset to LDS byte address
// `lds` + 16 (4) * lane.  The compiler does not see these loads: callers wait
// for them with explicit vmcnt waits.  M0 is saved and restored around the
// instruction.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen" AMK_NT_SUFFIX " lds\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds), "v"(off), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, 0 offen" AMK_NT_SUFFIX " lds\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "s"(lds), "v"(off), "s"(r)
               : "memory");
}

// The GEMV proper.  The first `pf_steps` steps of every wave (fewer if the
// wave has fewer) are already in LDS at `pf` (copied there by the end of the
// previous task, see issue_prefetch); the register ring starts after them.
template <class F, int DS, int RPU, typename StageFn, typename AfterFn>
__device__ __forceinline__ void gemv(const uint8_t* data, const uint8_t* meta, uint32_t row_bytes,
                                     uint32_t meta_row_bytes, int nunits, int K, const float* xs,
                                     const float* csum, float* tbl, int poll_late, int pf_steps,
                                     const uint8_t* pf, StageFn&& stage, AfterFn&& after_prologue) {
  const int tid = opaque_tid(), lane = tid & 63;
  const int sw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nchunk = K / F::E;
  const int J = (nchunk + 63) >> 6;
  const int jl = (nchunk - lane + 63) >> 6;  // slabs in which this lane has data
  StepIter it;
  it.init(sw, nunits, J);
  const int n = it.n;                // steps of this wave
  const int np = min(pf_steps, n);   // of which prefetched
  for (int k = 0; k < np; ++k) it.advance();
  const __amdgpu_buffer_rsrc_t rs = rsrc(data, (uint32_t)nunits * RPU * row_bytes);
  const __amdgpu_buffer_rsrc_t rm = rsrc(meta, F::kMeta ? (uint32_t)nunits * RPU * meta_row_bytes : 0u);
  u32x4 buf[DS][RPU];
  uint32_t mbuf[DS][RPU];
  auto issue = [&](u32x4 (&b)[RPU], uint32_t (&mb)[RPU]) {
    const bool valid = it.ik < n && it.ij < jl;
    const uint32_t off = (uint32_t)it.iu * RPU * row_bytes + (uint32_t)(it.ij * 64 + lane) * 16u;
    const uint32_t moff = (uint32_t)it.iu * RPU * meta_row_bytes + (uint32_t)(it.ij * 16 + (lane >> 2)) * 4u;
#pragma unroll
    for (int r = 0; r < RPU; ++r) {
      b[r] = bload(rs, valid ? off + (uint32_t)r * row_bytes : kOob);
      if constexpr (F::kMeta)
        mb[r] = __builtin_amdgcn_raw_buffer_load_b32(rm, valid ? moff + (uint32_t)r * meta_row_bytes : kOob, 0,
                                                     kStreamPolicy);
    }
    it.advance();
  };
  // ring slots [0, split) are loaded before the wait, the rest after it
  // (poll_late 1: none for the polling wave; 2: half of the ring for every
  // wave, so loads issued after the input has arrived keep streaming while
  // the input is staged; 3: none: the LDS copy alone streams through the
  // wait, and input reads queue behind no weight load)
  const int split = poll_late == 3 ? 0 : poll_late == 2 ? DS / 2 : (poll_late == 1 && sw == 0 ? 0 : DS);
  auto prologue = [&](bool first) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if ((s < split) == first) issue(buf[s], mbuf[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  prologue(true);
  stage();
  prologue(false);
  after_prologue();
  if (n > 0) {
    StepIter c;
    c.init(sw, nunits, J);
    int ck = 0;
    float acc[RPU];
#pragma unroll
    for (int r = 0; r < RPU; ++r) acc[r] = 0.0f;
    auto consume = [&](const u32x4 (&w)[RPU], const uint32_t (&m)[RPU]) {
#pragma unroll
      for (int r = 0; r < RPU; ++r) acc[r] = F::dot(acc[r], w[r], m[r], xs, c.ij, lane, csum);
      ++ck;
      if (ck <= n && (c.ij == J - 1 || ck == n)) {  // this wave's segment of unit c.iu is complete
#pragma unroll
        for (int r = 0; r < RPU; ++r) {
          const float v = wave_sum(acc[r]);
          if (lane == 0) tbl[(c.iu * RPU + r) * kWaves + sw] = v;
          acc[r] = 0.0f;
        }
      }
      c.advance();
    };
    if (np > 0) {
      const uint8_t* mine = pf + (uint32_t)sw * (uint32_t)pf_steps * RPU * pf_row_step<F>();
      for (int s = 0; s < np; ++s) {
        u32x4 w[RPU];
        uint32_t m[RPU];
#pragma unroll
        for (int r = 0; r < RPU; ++r) {
          const uint8_t* row = mine + (uint32_t)(s * RPU + r) * pf_row_step<F>();
          w[r] = *reinterpret_cast<const u32x4*>(row + lane * 16);
          m[r] = F::kMeta ? *reinterpret_cast<const uint32_t*>(row + 1024 + lane * 4) : 0u;
        }
        consume(w, m);
      }
    }
    // Past the wave's last step the ring issues nothing: loads past the
    // rows would return zeros without memory traffic, but each still takes
    // its turn in the compute unit's address pipeline, where the task's
    // epilogue stores and the next task's loads would queue behind it.
    // (The prologue always issues its DS slots: the LDS-copy waits count
    // them.)
    const int iters = (n - np + DS - 1) / DS;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        consume(buf[s], mbuf[s]);
        __builtin_amdgcn_sched_barrier(0);
        if (__builtin_amdgcn_readfirstlane(it.ik) < n) issue(buf[s], mbuf[s]);
      }
    }
  }
  __syncthreads();
}

// sum of the partials of output row i (unit u = i / RPU): its owner in the
// rounds, or the waves whose tail range overlaps unit u, in wave order
template <int RPU>
__device__ __forceinline__ float gemv_row(const float* tbl, int i, int nunits, int J) {
  const int u = i / RPU;
  const GemvSplit sp(nunits, J);
  if (u < sp.nr * kWaves) return tbl[i * kWaves + u % kWaves];
  const int q0 = (u - sp.nr * kWaves) * J, q1 = q0 + J;  // the unit's tail steps
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    int t0, t1;
    sp.tail(w, &t0, &t1);
    if (t1 > t0 && t0 < q1 && t1 > q0) v += tbl[i * kWaves + w];  // (empty ranges wrote nothing)
  }
  return v;
}

__device__ __forceinline__ int round4(int n) { return (n + 3) & ~3; }

// LDS floats of a GEMV task's staged input (padded to whole wave-loads) plus,
// for int4, the per-chunk sums; the partial table follows
template <int WFMT>
__device__ __forceinline__ int xs_floats(int K) {
  constexpr int E = WFMT == AMK_W_BF16 ? 8 : (WFMT == AMK_W_INT8_ROW ? 16 : 32);
  const int padded = (K + E * 64 - 1) / (E * 64) * (E * 64);
  return round4(padded + padded / 32);
}

// Runs the projection rows [row0, row0 + nunits*RPU) of packed tensor `ptr`
// (rows_total rows of K inputs) on the input vector `src` (RMSNorm'd with
// `gain` when NORM), waiting for the task's counters after the first weight
// loads are issued.  Results: res[i] for i < nunits*RPU (LDS).
template <int DEPTH, int WFMT, int RPU>
__device__ __forceinline__ bool project(const VmParams& P, TaskRef t, float* smem, const uint8_t* ptr,
                                        int64_t rows_total, int K, int row0, int nunits, const void* src,
                                        const uint64_t* tsrc, const uint16_t* gain, bool src_bf16) {
  using F = typename std::conditional<WFMT == AMK_W_BF16, FmtBf16,
            typename std::conditional<WFMT == AMK_W_INT8_ROW, FmtInt8, FmtInt4>::type>::type;
  float* red = smem;                                  // kWaves floats
  int* flag = reinterpret_cast<int*>(smem + kWaves);  // two wait-flag slots
  float* xsum = smem + kWaves + 2;                    // sum of x (int8)
  float* xs = smem + kHead;
  float* res = xs + xs_floats<WFMT>(K);
  float* tbl = res + round4(nunits * RPU);
  const int padded = (K + F::E * 64 - 1) / (F::E * 64) * (F::E * 64);
  float* csum = xs + padded;  // int4: per-chunk sums of x
  const uint32_t rb = WFMT == AMK_W_BF16 ? (uint32_t)K * 2u : (WFMT == AMK_W_INT8_ROW ? (uint32_t)K : (uint32_t)K / 2u);
  const uint32_t mb = WFMT == AMK_W_INT4_G128 ? (uint32_t)(K / 128) * 4u : (WFMT == AMK_W_INT8_ROW ? 4u : 0u);
  const uint8_t* meta = ptr + rows_total * (int64_t)rb + (int64_t)row0 * mb;
  bool ok = true;
  constexpr int DS = DEPTH / RPU;
  // waves 1..7 issued the LDS DMAs of this task's prefetched steps (for all
  // waves) before its ring prologue: waiting until only the prologue's loads
  // may be outstanding means those DMAs are done; the barrier after it shows
  // the data to every wave.
  // (poll_mode 2 issues only half of the ring before the wait.)
  // poll_mode 3: the DMA waves issued the copies and nothing else; they
  // wait for them after the input is staged and the ring issued, and the
  // barrier after that shows the data to every wave.
  constexpr int kPrologueLoads = DS * RPU * (F::kMeta ? 2 : 1);
  constexpr int kHalfPrologueLoads = (DS / 2) * RPU * (F::kMeta ? 2 : 1);
  const bool dma3 = P.poll_late == 3;
  const bool pf_wait = t.pf_have > 0 && (dma3 ? opaque_tid() >= kDmaWave0 * 64 : opaque_tid() >= 64);
  const bool half = P.poll_late == 2;
  gemv<F, DS, RPU>(ptr + (int64_t)row0 * rb, meta, rb, mb, nunits, K, xs, csum, tbl, P.poll_late,
                   t.pf_have, reinterpret_cast<const uint8_t*>(smem) + t.pf_lds, [&] {
    ok = vm_wait(P, t, flag, [&] {
      if (pf_wait && !dma3) {
        if (half) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kHalfPrologueLoads) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPrologueLoads) : "memory");
      }
    });
    if (ok) ok = stage_x<F>(P, src, tsrc, K, gain, src_bf16, xs, red, xsum, csum, input_threads(P));
    if (ok && P.tagged) trace_mark(P, t, 1);
  }, [&] {
    if (dma3 && t.pf_have > 0) {
      if (pf_wait) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPrologueLoads) : "memory");
      __syncthreads();
    }
  });
  if (!ok) return false;
  const int J = (K / F::E + 63) >> 6;
  const int nrows = nunits * RPU, tid = opaque_tid();
  for (int i = tid; i < nrows; i += kThreads) {
    float v = gemv_row<RPU>(tbl, i, nunits, J);
    if constexpr (WFMT == AMK_W_INT8_ROW)
      v = reinterpret_cast<const float*>(meta)[i] * (v - 128.0f * *xsum);
    res[i] = v;
  }
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------- tasks --

// The GEMV tasks (QKV, O, gate/up, down, LM head) share one body: the
// task's operand choice, one projection (row pairs when the row count is
// even), then the task's epilogue.  Every GEMV phase runs the same code, so
// the instruction cache keeps it between phases.
template <int DEPTH, int WFMT>
__device__ __forceinline__ bool task_gemv(const VmParams& P, TaskRef t, float* smem) {
  const int type = t.type;
  const int H = P.H, F = P.F, hd = P.hd, half = hd >> 1, nq = P.nq, nkv = P.nkv, qd = nq * hd;
  const int l = type == AMK_TASK_LMHEAD ? P.L - 1 : t.p[0];
  const int tid = opaque_tid();
  const uint8_t* w;
  const uint16_t* gain = nullptr;
  const void* src;
  const uint64_t* tsrc = nullptr;
  bool src_bf16 = false;
  int64_t rows_total;
  int K, row0, nrows;
  const int64_t xin = ((int64_t)(l - 1) * 2 + 1) * H;  // previous layer's output
  const int64_t xmid = (int64_t)l * 2 * H, xout = ((int64_t)l * 2 + 1) * H;
  int64_t resid_off = -1;  // O / down: where the residual rows are read
  switch (type) {
    case AMK_TASK_QKV:
      w = P.wptr[3 + 6 * l + LB_QKV];
      gain = reinterpret_cast<const uint16_t*>(P.wptr[3 + 6 * l + LB_ATTN_NORM]);
      rows_total = (int64_t)(nq + 2 * nkv) * hd;
      K = H;
      row0 = 2 * t.p[1];
      nrows = 2 * (t.p[2] - t.p[1]);
      if (l == 0) {
        src = P.wptr[0] + (int64_t)P.token * H * 2;
        src_bf16 = true;
      } else {
        src = P.x + xin;
        if (P.tagged) tsrc = P.tx + xin;
      }
      break;
    case AMK_TASK_OPROJ:
      w = P.wptr[3 + 6 * l + LB_O];
      rows_total = H;
      K = qd;
      row0 = t.p[1];
      nrows = t.p[2] - t.p[1];
      src = P.o + (int64_t)l * qd;
      if (P.tagged) tsrc = P.to + (int64_t)l * qd;
      if (l > 0) resid_off = xin;
      break;
    case AMK_TASK_GATEUP:
      w = P.wptr[3 + 6 * l + LB_GATEUP];
      gain = reinterpret_cast<const uint16_t*>(P.wptr[3 + 6 * l + LB_MLP_NORM]);
      rows_total = 2 * (int64_t)F;
      K = H;
      row0 = 2 * t.p[1];
      nrows = 2 * (t.p[2] - t.p[1]);
      src = P.x + xmid;
      if (P.tagged) tsrc = P.tx + xmid;
      break;
    case AMK_TASK_DOWN:
      w = P.wptr[3 + 6 * l + LB_DOWN];
      rows_total = H;
      K = F;
      row0 = t.p[1];
      nrows = t.p[2] - t.p[1];
      src = P.a + (int64_t)l * F;
      if (P.a_tagged) tsrc = P.ta + (int64_t)l * F;
      resid_off = xmid;
      break;
    default:  // AMK_TASK_LMHEAD
      w = P.wptr[2];
      gain = reinterpret_cast<const uint16_t*>(P.wptr[1]);
      rows_total = P.V;
      K = H;
      row0 = t.p[0];
      nrows = t.p[1] - t.p[0];
      src = P.x + xout;
      if (P.tagged) tsrc = P.tx + xout;
      break;
  }
  // tagged: the first residual row of each thread, read before the weight
  // stream so that it is not queued behind it (written by an earlier phase
  // whose output this queue's previous GEMV task staged in full; checked
  // anyway)
  uint64_t rres = 0;
  if (P.tagged && resid_off >= 0 && tid < nrows) rres = ld_tag(P.tx + resid_off + t.p[1] + tid);
  // QKV: the RoPE (cos, sin) of this thread's first pair unit, read now for the same reason
  float2 cs0 = make_float2(1.0f, 0.0f);
  if (type == AMK_TASK_QKV && tid < t.p[2] - t.p[1]) {
    const int u = t.p[1] + tid, hs = u / half;
    if (hs < nq + nkv) cs0 = P.rope[(int64_t)P.pos * half + (u - hs * half)];
  }
  const bool ok = nrows & 1 ? project<DEPTH, WFMT, 1>(P, t, smem, w, rows_total, K, row0, nrows, src, tsrc, gain, src_bf16)
                            : project<DEPTH, WFMT, 2>(P, t, smem, w, rows_total, K, row0, nrows / 2, src, tsrc, gain,
                                                      src_bf16);
  if (!ok) return false;
  const float* res = smem + kHead + xs_floats<WFMT>(K);
  const int EW = epilogue_threads(P);
  if (type == AMK_TASK_QKV) {
    const int u0 = t.p[1], u1 = t.p[2];
    if (tid < EW)
      for (int k = tid; k < u1 - u0; k += EW) {
        const int u = u0 + k, hs = u / half, i = u - hs * half;
        float a = res[2 * k], b = res[2 * k + 1];
        if (hs < nq + nkv) {
          const float2 cs = k == tid ? cs0 : P.rope[(int64_t)P.pos * half + i];
          const float ra = a * cs.x - b * cs.y, rb = b * cs.x + a * cs.y;
          a = ra;
          b = rb;
        }
        if (hs < nq) {
          const int64_t qo = (int64_t)l * nq * hd + (int64_t)hs * hd;
          if (P.tagged) {
            st_tag(P.tq + qo + i, a, P.tag);
            st_tag(P.tq + qo + i + half, b, P.tag);
          } else {
            st_agent(P.q + qo + i, a);
            st_agent(P.q + qo + i + half, b);
          }
        } else {
          const int kvsel = hs < nq + nkv ? 0 : 1, g = hs - nq - kvsel * nkv;
          uint16_t* row = P.kv + ((((int64_t)l * 2 + kvsel) * nkv + g) * P.mc + P.pos) * hd;
          const uint32_t ba = bf16_bits(a), bb = bf16_bits(b);
          st_agent(row + i, (uint16_t)ba);
          st_agent(row + i + half, (uint16_t)bb);
          // a multi-step launch reads this row from the cache in the next
          // step: the write-through stores complete (reach the device
          // coherence point) before the tagged copy, whose observation is
          // the next step's licence to read the cache, is stored
          if (P.tagged && P.tokens_out) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (P.tagged) {  // this launch's row for the attention tasks, as tagged bf16 values
            uint64_t* tr = P.tkv + (((int64_t)l * 2 + kvsel) * nkv + g) * hd;
            st_tag(tr + i, __uint_as_float(ba << 16), P.tag);
            st_tag(tr + i + half, __uint_as_float(bb << 16), P.tag);
          }
        }
      }
  } else if (type == AMK_TASK_OPROJ || type == AMK_TASK_DOWN) {
    // residual add: O adds the previous layer's output (the embedding row at
    // layer 0), down adds this layer's attention output
    const int r0 = t.p[1];
    const int64_t dst = type == AMK_TASK_OPROJ ? xmid : xout;
    if (P.tagged) {
      TagSpin sp;
      for (int k = tid; k < nrows && !sp.failed; k += kThreads) {
        const int r = r0 + k;
        float resid[1];
        if (resid_off < 0) resid[0] = bf16_to_f(reinterpret_cast<const uint16_t*>(P.wptr[0])[(int64_t)P.token * H + r]);
        else if (k == tid && (uint32_t)(rres >> 32) == P.tag) resid[0] = tag_val(rres);
        else if (!ld_tagged<1>(P, P.tx + resid_off, [](int) { return true; }, [&](int) { return r; }, resid, sp)) break;
        st_tag(P.tx + dst + r, resid[0] + res[k], P.tag);
      }
      if (block_any(sp.failed, smem)) return false;
    } else if (tid < EW) {
      for (int k = tid; k < nrows; k += EW) {
        const int r = r0 + k;
        const float resid = resid_off < 0 ? bf16_to_f(reinterpret_cast<const uint16_t*>(P.wptr[0])[(int64_t)P.token * H + r])
                                          : P.x[resid_off + r];
        st_agent(P.x + dst + r, resid + res[k]);
      }
    }
  } else if (type == AMK_TASK_GATEUP) {
    const int j0 = t.p[1], nj = t.p[2] - t.p[1];
    const int EWa = P.a_tagged ? kThreads : EW;
    if (tid < EWa)
      for (int k = tid; k < nj; k += EWa) {
        const float g = res[2 * k], u = res[2 * k + 1];
        const float h = g / (1.0f + expf(-g)) * u;
        if (P.a_tagged) st_tag(P.ta + (int64_t)l * F + j0 + k, h, P.tag);
        else st_agent(P.a + (int64_t)l * F + j0 + k, h);
      }
  } else {
    // logits, and this task's (max, lowest index of the max) for the greedy
    // token of the next step
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int k = tid; k < nrows; k += kThreads) {
      P.logits[row0 + k] = res[k];
      if (res[k] > best) {
        best = res[k];
        bi = row0 + k;
      }
    }
    if (P.tokens_out) {  // a multi-step launch: the partial feeds the next token
      argmax_block(best, bi, smem);
      if (tid == 0) {
        st_tag(P.targ + 2 * t.p[2], best, P.tag);
        st_tag(P.targ + 2 * t.p[2] + 1, __int_as_float(bi), P.tag);
      }
    }
  }
  vm_signal(P, t);
  return true;
}

// ------------------------------------------------------------ attention --
// Head-major layout (short splits): one split [p0, p1) of the positions of
// kv head g, for query heads
// h0..h0+nh-1 (nh <= GP).  Lane layout ("head rows"): LH = hd/8 lanes hold the
// 8-element chunks of one row; GP groups of LH lanes take GP query heads; the
// remaining factor PW = 64/(LH*GP) takes PW positions per wave step.  Chunk c
// of block b of wave w is position p0 + ((b*MAXC + c)*8 + w)*PW + lane/(LH*GP).
// A score needs one LH-lane DPP sum; the online softmax and sum p*V stay in
// each lane (every lane of a group holds its group's max and sum), and the
// (wave, position group) states are merged once through LDS.  Rows of
// earlier positions were written by previous launches, so block 0 is loaded
// before the wait; the row at `pos` (written by this launch) is re-read after.
// Output: part[(l*nq + h)*S + s] = {sum_j p_j V_j (hd values), max, sum p}.
template <int LH, int GP, int MAXC>
__device__ __forceinline__ bool attn_split_hm(const VmParams& P, TaskRef t, int l, int g, int h0,
                                           int nh, int s, int S, int p0, int p1, float* smem) {
  constexpr int PW = 64 / (LH * GP);
  const int hd = P.hd, pos = P.pos, tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int pw = lane / (LH * GP), hh = (lane / LH) % GP, li = lane % LH;
  int* flag = reinterpret_cast<int*>(smem + kWaves);
  // K / V rows of (l, g) through buffer descriptors: 32-bit offsets, and
  // positions past p1 read as zero without touching memory
  const uint32_t rows_bytes = (uint32_t)P.mc * hd * 2;
  const __amdgpu_buffer_rsrc_t rk = rsrc(P.kv + (((int64_t)l * 2 + 0) * P.nkv + g) * P.mc * hd, rows_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(P.kv + (((int64_t)l * 2 + 1) * P.nkv + g) * P.mc * hd, rows_bytes);
  const uint32_t lane_off = (uint32_t)li * 16u, row_b = (uint32_t)hd * 2u;
  // waves 1..7 take the positions; wave 0 polls and keeps no loads in flight
  // (poll_mode 3: waves 0..kDmaWave0-1 take them, the DMA waves none)
  const int wsc = __builtin_amdgcn_readfirstlane(wave);
  const int aw0 = P.poll_late == 3 ? 0 : 1;
  const int naw = P.poll_late == 3 ? kDmaWave0 : kAttnWaves;
  const bool aw = wsc >= aw0 && wsc < aw0 + naw;  // this wave takes positions
  const int wi = wsc - aw0;
  auto posof = [&](int blk, int c) {
    return p0 + ((blk * MAXC + c) * naw + wi) * PW + pw;
  };
  auto koff = [&](int j, bool ok) { return ok ? (uint32_t)j * row_b + lane_off : kOob; };
  // two register buffers of blocks: blocks 0 and 1 are loaded before the
  // wait (positions before pos only: rows of earlier launches); later blocks
  // are loaded into the buffer just consumed, two blocks ahead
  u32x4 ka[MAXC], va[MAXC], kb[MAXC], vb[MAXC];
  // a chunk whose first position (lane group 0) is past the split holds no
  // position of this wave: zeros, without a load (an out-of-range load
  // would still take a turn in the address pipeline)
  auto load_blk = [&](u32x4 (&k)[MAXC], u32x4 (&v)[MAXC], int blk, bool before_wait) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int j = posof(blk, c);
      if (__builtin_amdgcn_readfirstlane(j - pw) < p1) {
        const uint32_t o = koff(j, j < p1 && (!before_wait || j < pos));
        k[c] = bload(rk, o);
        v[c] = bload(rv, o);
      } else {
        k[c] = u32x4{0u, 0u, 0u, 0u};
        v[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (aw) {
    load_blk(ka, va, 0, true);
    load_blk(kb, vb, 1, true);
  }
  if (!vm_wait(P, t, flag)) return false;
  const bool hv = hh < nh;
  const float scale = 1.0f / sqrtf((float)hd);
  const bool tagged = P.tagged != 0;
  const int64_t qoff = (int64_t)l * P.nq * hd + (int64_t)(h0 + (hv ? hh : 0)) * hd + li * 8;
  float q[8];
  // tagged mode: the lane whose positions include pos takes that row's K and
  // V chunk from the launch's tagged copy (block pblk, chunk pc); no load of
  // the cache reaches row pos
  int pblk = -1, pc = 0;
  u32x4 kp = {0u, 0u, 0u, 0u}, vp = {0u, 0u, 0u, 0u};
  if (tagged) {
    const int d = pos - p0 - pw;
    if (aw && pos < p1 && d >= 0 && d % PW == 0 && (d / PW) % naw == wi) {
      const int bc = d / PW / naw;
      pblk = bc / MAXC;
      pc = bc % MAXC;
    }
    // q and, for the lane holding pos, that row's K and V chunks: one round
    // of reads (both live in the tagged arena, addressed from q's base)
    TagSpin sp;
    const int64_t kd = (P.tkv - P.tq) + (((int64_t)l * 2 + 0) * P.nkv + g) * hd + li * 8 - qoff;
    const int64_t vd = (P.tkv - P.tq) + (((int64_t)l * 2 + 1) * P.nkv + g) * hd + li * 8 - qoff;
    float v[24];
    if (ld_tagged<24>(P, P.tq + qoff, [&](int k) { return aw && (k < 8 || pblk >= 0); },
                      [&](int k) { return k < 8 ? (int64_t)k : (k < 16 ? kd + (k - 8) : vd + (k - 16)); }, v, sp)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = v[e] * scale;
      auto pack = [](float lo, float hi) { return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u); };
      kp = u32x4{pack(v[8], v[9]), pack(v[10], v[11]), pack(v[12], v[13]), pack(v[14], v[15])};
      vp = u32x4{pack(v[16], v[17]), pack(v[18], v[19]), pack(v[20], v[21]), pack(v[22], v[23])};
    }
    if (block_any(sp.failed, smem)) return false;
  } else {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (aw) {
      const float* qp = P.q + qoff;
      a = *reinterpret_cast<const float4*>(qp);
      b = *reinterpret_cast<const float4*>(qp + 4);
    }
    q[0] = a.x * scale; q[1] = a.y * scale; q[2] = a.z * scale; q[3] = a.w * scale;
    q[4] = b.x * scale; q[5] = b.y * scale; q[6] = b.z * scale; q[7] = b.w * scale;
  }
  if (tagged) trace_mark(P, t, 1);
  float M = -INFINITY, Ls = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const int len = p1 - p0;
  const int per_blk = MAXC * naw * PW;
  const int nblk = aw ? (len + per_blk - 1) / per_blk : 0;
  // the row at pos (written by this launch) in a block loaded before the wait
  auto patch_pos = [&](u32x4 (&k)[MAXC], u32x4 (&v)[MAXC], int blk) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (posof(blk, c) == pos) {
        k[c] = bload(rk, koff(pos, true));
        v[c] = bload(rv, koff(pos, true));
      }
  };
  auto compute = [&](const u32x4 (&kr)[MAXC], const u32x4 (&vr)[MAXC], int blk) {
    float sc[MAXC];
    float bm = -INFINITY;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const u32x4 k8 = kr[c];
      float d = q[0] * bf16_lo(k8.x);
      d = fmaf(q[1], bf16_hi(k8.x), d);
      d = fmaf(q[2], bf16_lo(k8.y), d);
      d = fmaf(q[3], bf16_hi(k8.y), d);
      d = fmaf(q[4], bf16_lo(k8.z), d);
      d = fmaf(q[5], bf16_hi(k8.z), d);
      d = fmaf(q[6], bf16_lo(k8.w), d);
      d = fmaf(q[7], bf16_hi(k8.w), d);
      d = group_sum<LH>(d);
      sc[c] = posof(blk, c) < p1 ? d : -INFINITY;
      bm = fmaxf(bm, sc[c]);
    }
    const float nm = fmaxf(M, bm);
    const float alpha = M == -INFINITY ? 0.0f : __expf(M - nm);
    Ls *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const float p = sc[c] == -INFINITY ? 0.0f : __expf(sc[c] - nm);
      Ls += p;
      const u32x4 v8 = vr[c];
      acc[0] = fmaf(p, bf16_lo(v8.x), acc[0]);
      acc[1] = fmaf(p, bf16_hi(v8.x), acc[1]);
      acc[2] = fmaf(p, bf16_lo(v8.y), acc[2]);
      acc[3] = fmaf(p, bf16_hi(v8.y), acc[3]);
      acc[4] = fmaf(p, bf16_lo(v8.z), acc[4]);
      acc[5] = fmaf(p, bf16_hi(v8.z), acc[5]);
      acc[6] = fmaf(p, bf16_lo(v8.w), acc[6]);
      acc[7] = fmaf(p, bf16_hi(v8.w), acc[7]);
    }
    M = nm;
  };
  auto patch_tag = [&](u32x4 (&k)[MAXC], u32x4 (&v)[MAXC], int blk) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (blk == pblk && c == pc) {
        k[c] = kp;
        v[c] = vp;
      }
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    if (tagged) patch_tag(ka, va, blk);
    else if (blk == 0) patch_pos(ka, va, 0);
    compute(ka, va, blk);
    if (blk + 2 < nblk) load_blk(ka, va, blk + 2, tagged);
    if (blk + 1 < nblk) {
      if (tagged) patch_tag(kb, vb, blk + 1);
      else if (blk == 0) patch_pos(kb, vb, 1);
      compute(kb, vb, blk + 1);
      if (blk + 3 < nblk) load_blk(kb, vb, blk + 3, tagged);
    }
  }
  // merge the (wave, position group) states of each head through LDS
  float* wacc = smem + P.lds_att;         // [kWaves*64][8]
  float* wst = wacc + kWaves * 64 * 8;    // [kWaves*64][2]
  *reinterpret_cast<float4*>(wacc + tid * 8) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(wacc + tid * 8 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  wst[tid * 2] = M;
  wst[tid * 2 + 1] = Ls;
  __syncthreads();
  float* wout = wst + kWaves * 64 * 2;  // [nh][hd] outputs, then [nh][2] stats
  for (int i = tid; i < nh * hd; i += kThreads) {
    const int hq = i / hd, e = i - hq * hd, ci = e >> 3, ee = e & 7;
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int q2 = 0; q2 < PW; ++q2) mt = fmaxf(mt, wst[(w * 64 + q2 * LH * GP + hq * LH) * 2]);
    float o = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int q2 = 0; q2 < PW; ++q2) {
        const int ln = w * 64 + q2 * LH * GP + hq * LH;
        const float mw = wst[ln * 2];
        const float f = mw == -INFINITY ? 0.0f : __expf(mw - mt);
        o = fmaf(f, wacc[(ln + ci) * 8 + ee], o);
        lsum = fmaf(f, wst[ln * 2 + 1], lsum);
      }
    wout[i] = o;
    if (e == 0) {
      wout[nh * hd + hq * 2] = mt;
      wout[nh * hd + hq * 2 + 1] = lsum;
    }
  }
  __syncthreads();
  const int EW = tagged ? kThreads : epilogue_threads(P);
  if (tid < EW) {  // the releasing threads store everything other workgroups read
    for (int i = tid; i < nh * (hd + 2); i += EW) {
      const int hq = i / (hd + 2), e = i - hq * (hd + 2);
      const float v = e < hd ? wout[hq * hd + e] : wout[nh * hd + hq * 2 + (e - hd)];
      const int64_t o = (((int64_t)l * P.nq + h0 + hq) * S + s) * (hd + 2) + e;
      if (tagged) st_tag(P.tpart + o, v, P.tag);
      else st_agent(P.part + o, v);
    }
  }
  return true;
}

template <int LH, int GP>
__device__ __forceinline__ bool attn_heads_hm(const VmParams& P, TaskRef t, int l, int g, int s, int S,
                                           int p0, int p1, float* smem) {
  const int grp = P.nq / P.nkv;
  constexpr int MAXC = 4;
  for (int h0 = 0; h0 < grp; h0 += GP) {  // later passes find the counters reached
    if (h0 > 0) __syncthreads();
    if (!attn_split_hm<LH, GP, MAXC>(P, t, l, g, g * grp + h0, min(GP, grp - h0), s, S, p0, p1, smem))
      return false;
  }
  return true;
}

// Position-major layout (long splits): one split [p0, p1) of the positions
// of kv head g, for query heads h0..h0+nh-1 (nh <= GP).  Lane layout: LH =
// hd/8 lanes hold the 8-element
// chunks of one K/V row, so a wave step covers PW = 64/LH positions, and
// every lane scores its row chunk against all GP query heads (a 16-byte load
// brings distinct rows into all 64 lanes).  Chunk c of block b of attention
// wave w is position p0 + ((b*MAXC + c)*naw + w)*PW + lane/LH.  A score needs
// one LH-lane DPP sum; the online softmax and sum p*V stay in each lane
// (every lane of a row group holds the group's max and sum per head); the
// PW position groups of a wave merge through cross-lane exchanges, then the
// waves once through LDS.  Rows of earlier positions were written by
// previous launches, so blocks 0 and 1 are loaded before the wait; the row
// at `pos` (written by this launch) is taken afterwards.  q (and, with
// tagged activations, the row at pos) is staged once in LDS.
// Output: part[(l*nq + h)*S + s] = {sum_j p_j V_j (hd values), max, sum p}.
template <int LH, int GP, int MAXC>
__device__ __forceinline__ bool attn_split_pm(const VmParams& P, TaskRef t, int l, int g, int h0,
                                           int nh, int s, int S, int p0, int p1, float* smem) {
  constexpr int PW = 64 / LH;
  const int hd = P.hd, pos = P.pos, tid = opaque_tid(), lane = tid & 63;
  const int pw = lane / LH, li = lane % LH;
  int* flag = reinterpret_cast<int*>(smem + kWaves);
  // K / V rows of (l, g) through buffer descriptors: 32-bit offsets, and
  // positions past p1 read as zero without touching memory
  const uint32_t rows_bytes = (uint32_t)P.mc * hd * 2;
  const __amdgpu_buffer_rsrc_t rk = rsrc(P.kv + (((int64_t)l * 2 + 0) * P.nkv + g) * P.mc * hd, rows_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(P.kv + (((int64_t)l * 2 + 1) * P.nkv + g) * P.mc * hd, rows_bytes);
  const uint32_t lane_off = (uint32_t)li * 16u, row_b = (uint32_t)hd * 2u;
  // waves 1..7 take the positions; wave 0 polls and keeps no loads in flight
  // (poll_mode 3: waves 0..kDmaWave0-1 take them, the DMA waves none)
  const int wsc = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int aw0 = P.poll_late == 3 ? 0 : 1;
  const int naw = P.poll_late == 3 ? kDmaWave0 : kAttnWaves;
  const bool aw = wsc >= aw0 && wsc < aw0 + naw;  // this wave takes positions
  const int wi = wsc - aw0;
  auto posof = [&](int blk, int c) {
    return p0 + ((blk * MAXC + c) * naw + wi) * PW + pw;
  };
  // first position of chunk c of block blk in this wave (the same in every lane)
  auto chunk0 = [&](int blk, int c) { return __builtin_amdgcn_readfirstlane(posof(blk, c) - pw); };
  auto koff = [&](int j, bool ok) { return ok ? (uint32_t)j * row_b + lane_off : kOob; };
  // two register buffers of blocks: blocks 0 and 1 are loaded before the
  // wait (positions before pos only: rows of earlier launches); later blocks
  // are loaded into the buffer just consumed, two blocks ahead
  u32x4 ka[MAXC], va[MAXC], kb[MAXC], vb[MAXC];
  // a chunk that holds no position of the split: zeros, without a load (an
  // out-of-range load would still take a turn in the address pipeline)
  auto load_blk = [&](u32x4 (&k)[MAXC], u32x4 (&v)[MAXC], int blk, bool before_wait) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int j = posof(blk, c);
      if (chunk0(blk, c) < p1) {
        const uint32_t o = koff(j, j < p1 && (!before_wait || j < pos));
        k[c] = bload(rk, o);
        v[c] = bload(rv, o);
      } else {
        k[c] = u32x4{0u, 0u, 0u, 0u};
        v[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if (aw) {
    load_blk(ka, va, 0, true);
    load_blk(kb, vb, 1, true);
  }
  if (!vm_wait(P, t, flag)) return false;
  // LDS: q of the pass [GP][hd] (scaled), the row at pos [2][hd] (tagged
  // mode), the waves' states [kWaves][GP][hd] + [kWaves][GP][2], and the
  // merged outputs [GP][hd] + [GP][2]
  float* qs = smem + P.lds_att;
  float* kvs = qs + GP * hd;
  float* wacc = kvs + 2 * hd;
  float* wst = wacc + kWaves * GP * hd;
  float* wout = wst + kWaves * GP * 2;
  const float scale = 1.0f / sqrtf((float)hd);
  const bool tagged = P.tagged != 0;
  const int64_t qbase = (int64_t)l * P.nq * hd + (int64_t)h0 * hd;  // heads h0.. are contiguous
  const bool has_pos = p0 <= pos && pos < p1;
  const int nq_w = nh * hd;
  if (tagged) {
    // one round of reads by the input threads: q of the pass and, when the
    // split holds pos, that row's K and V (the launch's tagged copy; no load
    // of the cache reaches row pos)
    const int nr = input_threads(P);
    const int nw = nq_w + (has_pos ? 2 * hd : 0);
    const int64_t kd = (P.tkv - P.tq) + (((int64_t)l * 2 + 0) * P.nkv + g) * hd - qbase;
    const int64_t vd = (P.tkv - P.tq) + (((int64_t)l * 2 + 1) * P.nkv + g) * hd - qbase;
    TagSpin sp;
    float v[4];
    auto idx = [&](int k) -> int64_t {
      const int i = tid + k * nr;
      return i < nq_w ? (int64_t)i : (i < nq_w + hd ? kd + (i - nq_w) : vd + (i - nq_w - hd));
    };
    if (tid < nr && ld_tagged<4>(P, P.tq + qbase, [&](int k) { return tid + k * nr < nw; }, idx, v, sp)) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = tid + k * nr;
        if (i < nq_w) qs[i] = v[k] * scale;
        else if (i < nw) kvs[i - nq_w] = v[k];
      }
    }
    if (block_any(sp.failed, smem)) return false;
    trace_mark(P, t, 1);
  } else {
    const int nr = input_threads(P);
    for (int i = tid; tid < nr && i < nq_w; i += nr) qs[i] = P.q[qbase + i] * scale;
    __syncthreads();
  }
  float q[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (h < nh) {
      a = *reinterpret_cast<const float4*>(qs + h * hd + li * 8);
      b = *reinterpret_cast<const float4*>(qs + h * hd + li * 8 + 4);
    }
    q[h][0] = a.x; q[h][1] = a.y; q[h][2] = a.z; q[h][3] = a.w;
    q[h][4] = b.x; q[h][5] = b.y; q[h][6] = b.z; q[h][7] = b.w;
  }
  // the chunk (block pblk, chunk pc) of this lane whose position is pos
  int pblk = -1, pc = 0;
  {
    const int d = pos - p0 - pw;
    if (aw && has_pos && d >= 0 && d % PW == 0 && (d / PW) % naw == wi) {
      const int bc = d / PW / naw;
      pblk = bc / MAXC;
      pc = bc % MAXC;
    }
  }
  // the row at pos: tagged mode from LDS (bf16 values carried as floats),
  // counter mode from the cache (visible after the acquire of the wait)
  auto patch = [&](u32x4 (&k)[MAXC], u32x4 (&v)[MAXC], int blk) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (blk == pblk && c == pc) {
        if (tagged) {
          auto pk = [](const float* f) {
            u32x4 r;
            r.x = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
            r.y = (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xFFFF0000u);
            r.z = (__float_as_uint(f[4]) >> 16) | (__float_as_uint(f[5]) & 0xFFFF0000u);
            r.w = (__float_as_uint(f[6]) >> 16) | (__float_as_uint(f[7]) & 0xFFFF0000u);
            return r;
          };
          k[c] = pk(kvs + li * 8);
          v[c] = pk(kvs + hd + li * 8);
        } else {
          k[c] = bload(rk, koff(pos, true));
          v[c] = bload(rv, koff(pos, true));
        }
      }
  };
  float M[GP], Ls[GP], acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    M[h] = -INFINITY;
    Ls[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }
  const int len = p1 - p0;
  const int per_blk = MAXC * naw * PW;
  const int nblk = aw ? (len + per_blk - 1) / per_blk : 0;
  auto compute = [&](const u32x4 (&kr)[MAXC], const u32x4 (&vr)[MAXC], int blk) {
    float sc[MAXC][GP];
    float bm[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) bm[h] = -INFINITY;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
#pragma unroll
      for (int h = 0; h < GP; ++h) sc[c][h] = -INFINITY;
      if (chunk0(blk, c) >= p1) continue;  // no position of the split in this chunk
      const u32x4 k8 = kr[c];
      const float kf[8] = {bf16_lo(k8.x), bf16_hi(k8.x), bf16_lo(k8.y), bf16_hi(k8.y),
                           bf16_lo(k8.z), bf16_hi(k8.z), bf16_lo(k8.w), bf16_hi(k8.w)};
      const bool valid = posof(blk, c) < p1;
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float d = q[h][0] * kf[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) d = fmaf(q[h][e], kf[e], d);
        d = group_sum<LH>(d);
        sc[c][h] = valid ? d : -INFINITY;
        bm[h] = fmaxf(bm[h], sc[c][h]);
      }
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float nm = fmaxf(M[h], bm[h]);
      const float alpha = M[h] == -INFINITY ? 0.0f : __expf(M[h] - nm);
      Ls[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      M[h] = nm;
    }
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (chunk0(blk, c) >= p1) continue;
      const u32x4 v8 = vr[c];
      const float vf[8] = {bf16_lo(v8.x), bf16_hi(v8.x), bf16_lo(v8.y), bf16_hi(v8.y),
                           bf16_lo(v8.z), bf16_hi(v8.z), bf16_lo(v8.w), bf16_hi(v8.w)};
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float p = sc[c][h] == -INFINITY ? 0.0f : __expf(sc[c][h] - M[h]);
        Ls[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    patch(ka, va, blk);
    compute(ka, va, blk);
    if (blk + 2 < nblk) load_blk(ka, va, blk + 2, tagged);
    if (blk + 1 < nblk) {
      patch(kb, vb, blk + 1);
      compute(kb, vb, blk + 1);
      if (blk + 3 < nblk) load_blk(kb, vb, blk + 3, tagged);
    }
  }
  // merge the PW position groups of the wave (lanes pw, pw ^ 1, ...): both
  // partners form the same sums, so every lane ends with the wave's state
  auto merge_lanes = [&](auto xr) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float mo = xr(M[h]);
      const float lo = xr(Ls[h]);
      const float nm = fmaxf(M[h], mo);
      const float fa = M[h] == -INFINITY ? 0.0f : __expf(M[h] - nm);
      const float fb = mo == -INFINITY ? 0.0f : __expf(mo - nm);
      Ls[h] = Ls[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * fa + xr(acc[h][e]) * fb;
      M[h] = nm;
    }
  };
  if constexpr (LH <= 8) merge_lanes([](float v) { return lane_xor<8>(v); });
  if constexpr (LH <= 16) merge_lanes([](float v) { return lane_xor<16>(v); });
  merge_lanes([](float v) { return lane_xor<32>(v); });
  // then the waves through LDS (lanes of position group 0 write)
  if (pw == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float* o = wacc + (wsc * GP + h) * hd + li * 8;
      *reinterpret_cast<float4*>(o) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      if (li == 0) {
        wst[(wsc * GP + h) * 2] = M[h];
        wst[(wsc * GP + h) * 2 + 1] = Ls[h];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < nh * hd; i += kThreads) {
    const int hq = i / hd, e = i - hq * hd;
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, wst[(w * GP + hq) * 2]);
    float o = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wst[(w * GP + hq) * 2];
      const float f = mw == -INFINITY ? 0.0f : __expf(mw - mt);
      o = fmaf(f, wacc[(w * GP + hq) * hd + e], o);
      lsum = fmaf(f, wst[(w * GP + hq) * 2 + 1], lsum);
    }
    wout[i] = o;
    if (e == 0) {
      wout[GP * hd + hq * 2] = mt;
      wout[GP * hd + hq * 2 + 1] = lsum;
    }
  }
  __syncthreads();
  const int EW = tagged ? kThreads : epilogue_threads(P);
  if (tid < EW) {  // the releasing threads store everything other workgroups read
    for (int i = tid; i < nh * (hd + 2); i += EW) {
      const int hq = i / (hd + 2), e = i - hq * (hd + 2);
      const float v = e < hd ? wout[hq * hd + e] : wout[GP * hd + hq * 2 + (e - hd)];
      const int64_t o = (((int64_t)l * P.nq + h0 + hq) * S + s) * (hd + 2) + e;
      if (tagged) st_tag(P.tpart + o, v, P.tag);
      else st_agent(P.part + o, v);
    }
  }
  return true;
}

template <int LH, int GP>
__device__ __forceinline__ bool attn_heads_pm(const VmParams& P, TaskRef t, int l, int g, int s, int S,
                                           int p0, int p1, float* smem) {
  const int grp = P.nq / P.nkv;
  constexpr int MAXC = 4;
  for (int h0 = 0; h0 < grp; h0 += GP) {  // later passes find the counters reached
    if (h0 > 0) __syncthreads();
    if (!attn_split_pm<LH, GP, MAXC>(P, t, l, g, g * grp + h0, min(GP, grp - h0), s, S, p0, p1, smem))
      return false;
  }
  return true;
}

__device__ __forceinline__ bool task_attn(const VmParams& P, TaskRef t, float* smem) {
  const int l = t.p[0], g = t.p[1], s = t.p[2], S = t.p[3];
  const int n = P.pos + 1;
  const int p0 = (int)(((int64_t)s * n) / S), p1 = (int)(((int64_t)(s + 1) * n) / S);
  const int grp = P.nq / P.nkv, hd = P.hd;
  if (p1 <= p0) {
    int* flag = reinterpret_cast<int*>(smem + kWaves);
    if (!vm_wait(P, t, flag)) return false;
    const int tid = opaque_tid();
    const int EW = P.tagged ? kThreads : epilogue_threads(P);
    if (tid < EW)
      for (int i = tid; i < grp * (hd + 2); i += EW) {
        const int hh = i / (hd + 2), e = i - hh * (hd + 2);
        const int64_t o = (((int64_t)l * P.nq + g * grp + hh) * S + s) * (hd + 2) + e;
        if (P.tagged) st_tag(P.tpart + o, e == hd ? -INFINITY : 0.0f, P.tag);
        else st_agent(P.part + o, e == hd ? -INFINITY : 0.0f);
      }
  } else {
    bool ok;
    if (p1 - p0 >= kAttnPmMin) {  // position-major, GP = attn_pass_heads_pm
      const int gp = attn_pass_heads_pm(grp);
      if (hd == 64) {
        ok = gp == 1 ? attn_heads_pm<8, 1>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 2 ? attn_heads_pm<8, 2>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_pm<8, 4>(P, t, l, g, s, S, p0, p1, smem);
      } else if (hd == 128) {
        ok = gp == 1 ? attn_heads_pm<16, 1>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 2 ? attn_heads_pm<16, 2>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_pm<16, 4>(P, t, l, g, s, S, p0, p1, smem);
      } else {
        ok = gp == 1 ? attn_heads_pm<32, 1>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 2 ? attn_heads_pm<32, 2>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_pm<32, 4>(P, t, l, g, s, S, p0, p1, smem);
      }
    } else {  // head-major, GP = attn_pass_heads_hm
      const int gp = attn_pass_heads_hm(grp, hd);
      if (hd == 64) {
        ok = gp == 1 ? attn_heads_hm<8, 1>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 2 ? attn_heads_hm<8, 2>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 4 ? attn_heads_hm<8, 4>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_hm<8, 8>(P, t, l, g, s, S, p0, p1, smem);
      } else if (hd == 128) {
        ok = gp == 1 ? attn_heads_hm<16, 1>(P, t, l, g, s, S, p0, p1, smem)
           : gp == 2 ? attn_heads_hm<16, 2>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_hm<16, 4>(P, t, l, g, s, S, p0, p1, smem);
      } else {
        ok = gp == 1 ? attn_heads_hm<32, 1>(P, t, l, g, s, S, p0, p1, smem)
                     : attn_heads_hm<32, 2>(P, t, l, g, s, S, p0, p1, smem);
      }
    }
    if (!ok) return false;
  }
  vm_signal(P, t);
  return true;
}

// Log-sum-exp merge of the S split partials of query head h: one round trip
// of loads (every thread its float4 chunks and, for threads below S, that
// split's (max, sum)), then LDS: weights w_s = exp(m_s - M), scaled chunks
// summed per output element in split order, o = sum / sum_s w_s l_s.
__device__ __forceinline__ bool task_merge(const VmParams& P, TaskRef t, float* smem) {
  const int l = t.p[0], h = t.p[1], S = t.p[2];
  int* flag = reinterpret_cast<int*>(smem + kWaves);
  float* red = smem;
  const int hd = P.hd, hq = hd >> 2, tid = opaque_tid();
  if (!vm_wait(P, t, flag)) return false;
  const int64_t pbase = ((int64_t)l * P.nq + h) * S * (hd + 2);
  const float* part = P.part + pbase;
  float* wsum = smem + P.lds_att;  // [S][hd] scaled chunks
  float* wts = wsum + S * hd;      // [S]
  float2 ml = make_float2(-INFINITY, 0.0f);
  const int items = S * hq;
  // the first nr threads read (poll_mode 3: not the DMA waves, which may be
  // copying the next task's weights)
  const int nr = input_threads(P);
  const bool reader = tid < nr;
  float4 ch[4];
  if (P.tagged) {
    // the partials are tagged words: one round of reads (this thread's four
    // chunks and its split's (max, sum)), then re-reads until tagged.  The
    // engine admits the tagged mode only where S <= nr and
    // S * hd / 4 <= 4 * nr, so these cover every item.
    const uint64_t* tp = P.tpart + pbase;
    TagSpin spn;
    float v[18];
    ld_tagged<18>(
        P, tp, [&](int k) { return reader && (k < 16 ? tid + (k >> 2) * nr < items : tid < S); },
        [&](int k) {
          if (k >= 16) return (int64_t)tid * (hd + 2) + hd + (k - 16);
          const int it = tid + (k >> 2) * nr, sp = it / hq, qd = it - sp * hq;
          return (int64_t)sp * (hd + 2) + qd * 4 + (k & 3);
        },
        v, spn);
    if (block_any(spn.failed, red)) return false;
    trace_mark(P, t, 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) ch[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    if (reader && tid < S) ml = make_float2(v[16], v[17]);
  } else if (reader) {
    if (tid < S) ml = *reinterpret_cast<const float2*>(part + (int64_t)tid * (hd + 2) + hd);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int it = tid + k * nr;
      if (it < items) {
        const int sp = it / hq, qd = it - sp * hq;
        ch[k] = *reinterpret_cast<const float4*>(part + (int64_t)sp * (hd + 2) + qd * 4);
      }
    }
  }
  float m = ml.x;
  for (int sp = tid + nr; reader && sp < S; sp += nr) m = fmaxf(m, part[(int64_t)sp * (hd + 2) + hd]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  float Mx = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, red[w]);
  __syncthreads();
  float lsum = 0.0f;
  if (reader && tid < S) {
    const float wgt = ml.x == -INFINITY ? 0.0f : __expf(ml.x - Mx);
    wts[tid] = wgt;
    lsum = wgt * ml.y;
  }
  for (int sp = tid + nr; reader && sp < S; sp += nr) {
    const float ms = part[(int64_t)sp * (hd + 2) + hd];
    const float wgt = ms == -INFINITY ? 0.0f : __expf(ms - Mx);
    wts[sp] = wgt;
    lsum += wgt * part[(int64_t)sp * (hd + 2) + hd + 1];
  }
  const float Ltot = block_sum(lsum, red);  // its barriers also publish wts
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int it = tid + k * nr;
    if (reader && it < items) {
      const int sp = it / hq, qd = it - sp * hq;
      const float wgt = wts[sp];
      *reinterpret_cast<float4*>(wsum + sp * hd + qd * 4) =
          make_float4(wgt * ch[k].x, wgt * ch[k].y, wgt * ch[k].z, wgt * ch[k].w);
    }
  }
  for (int it = tid + 4 * nr; reader && it < items; it += nr) {
    const int sp = it / hq, qd = it - sp * hq;
    const float4 c = *reinterpret_cast<const float4*>(part + (int64_t)sp * (hd + 2) + qd * 4);
    const float wgt = wts[sp];
    *reinterpret_cast<float4*>(wsum + sp * hd + qd * 4) = make_float4(wgt * c.x, wgt * c.y, wgt * c.z, wgt * c.w);
  }
  __syncthreads();
  const float inv = 1.0f / Ltot;
  // the sum over splits: Q = kThreads / hd threads per output element each
  // add every Q-th split (Q dependent LDS reads in flight instead of one
  // chain of S), then the Q partial sums are added in a fixed order
  const int Q = kThreads / hd, e0 = tid % hd, q0 = tid / hd;
  float v = 0.0f;
  for (int sp = q0; sp < S; sp += Q) v += wsum[sp * hd + e0];
  __syncthreads();
  wsum[q0 * hd + e0] = v;  // rows 0..Q-1 (inside the attention scratch also when S < Q)
  __syncthreads();
  const int EW = epilogue_threads(P);
  if (tid < EW)
    for (int e = tid; e < hd; e += EW) {
      float tot = 0.0f;
      for (int k = 0; k < Q; ++k) tot += wsum[k * hd + e];
      const int64_t o = (int64_t)l * P.nq * hd + (int64_t)h * hd + e;
      if (P.tagged) st_tag(P.to + o, tot * inv, P.tag);
      else st_agent(P.o + o, tot * inv);
    }
  vm_signal(P, t);
  return true;
}

__device__ __forceinline__ bool task_nop(const VmParams& P, TaskRef t, float* smem) {
  int* flag = reinterpret_cast<int*>(smem + kWaves);
  if (!vm_wait(P, t, flag)) return false;
  vm_signal(P, t);
  return true;
}

// After a task has signalled, waves 1..7 copy the first slabs of the next
// task's weights into LDS with DMA (`t.pfn_*`, planned by the engine so the
// area is untouched by both tasks): the slabs each wave of the next task
// will consume first, in its own order; wave 0's slabs are issued by waves
// 1..7 in turn, so wave 0, which polls, keeps no loads outstanding.  The
// loads run through the next task's wait; that task waits for them before
// its barrier (see project).
// the prefetch fields of a task, read when the task starts so that they are
// in registers (not a memory round trip away) when the task ends
struct PfNext {
  int tensor, rpu, steps, K, lds, row0, nunits, rows_total;
  __device__ __forceinline__ explicit PfNext(TaskRef t) {
    steps = __builtin_amdgcn_readfirstlane(t.pfn_steps);
    tensor = __builtin_amdgcn_readfirstlane(t.pfn_tensor);
    rpu = __builtin_amdgcn_readfirstlane(t.pfn_rpu);
    K = __builtin_amdgcn_readfirstlane(t.pfn_K);
    lds = __builtin_amdgcn_readfirstlane(t.pfn_lds);
    row0 = __builtin_amdgcn_readfirstlane(t.pfn_row0);
    nunits = __builtin_amdgcn_readfirstlane(t.pfn_nunits);
    rows_total = __builtin_amdgcn_readfirstlane(t.pfn_rows_total);
  }
};

template <int WFMT, int RPU>
__device__ __forceinline__ void issue_prefetch_rpu(const VmParams& P, const PfNext& t, float* smem, int sw) {
  using F = typename std::conditional<WFMT == AMK_W_BF16, FmtBf16,
            typename std::conditional<WFMT == AMK_W_INT8_ROW, FmtInt8, FmtInt4>::type>::type;
  const int lane = opaque_tid() & 63;
  const int K = t.K, nunits = t.nunits, steps = t.steps;
  const uint32_t rb = WFMT == AMK_W_BF16 ? (uint32_t)K * 2u : (WFMT == AMK_W_INT8_ROW ? (uint32_t)K : (uint32_t)K / 2u);
  const uint32_t mb = WFMT == AMK_W_INT4_G128 ? (uint32_t)(K / 128) * 4u : 0u;
  const uint8_t* tensor = P.wptr[t.tensor];
  const uint8_t* data = tensor + (int64_t)t.row0 * rb;
  const uint8_t* meta = tensor + (int64_t)t.rows_total * rb + (int64_t)t.row0 * mb;
  const __amdgpu_buffer_rsrc_t rs = rsrc(data, (uint32_t)nunits * RPU * rb);
  const __amdgpu_buffer_rsrc_t rm = rsrc(meta, F::kMeta ? (uint32_t)nunits * RPU * mb : 0u);
  const int nchunk = K / F::E, J = (nchunk + 63) >> 6;
  const int jl = (nchunk - lane + 63) >> 6;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)t.lds);
  constexpr uint32_t kStep = pf_row_step<F>();
  // poll_mode 3: DMA wave kDmaWave0 + i copies all slabs of waves
  // i*per .. i*per + per - 1; otherwise waves 1..7 copy their own slabs
  // and a share of wave 0's (which polls)
  const bool dma3 = P.poll_late == 3;
  constexpr int per = kWaves / (kWaves - kDmaWave0);
  const int npass = dma3 ? per : 2;
  for (int pass = 0; pass < npass; ++pass) {
    const int v = dma3 ? (sw - kDmaWave0) * per + pass : (pass == 0 ? sw : 0);
    StepIter it;
    it.init(v, nunits, J);
    const int np = min(steps, it.n);
    const uint32_t area = lds0 + (uint32_t)v * (uint32_t)steps * RPU * kStep;
    for (int k = 0; k < np; ++k) {
      if (dma3 || v == sw || k % (kWaves - 1) == sw - 1) {
        const bool valid = it.ij < jl;
        const uint32_t off = (uint32_t)it.iu * RPU * rb + (uint32_t)(it.ij * 64 + lane) * 16u;
        const uint32_t moff = (uint32_t)it.iu * RPU * mb + (uint32_t)(it.ij * 16 + (lane >> 2)) * 4u;
#pragma unroll
        for (int r = 0; r < RPU; ++r) {
          const uint32_t dst = area + (uint32_t)(k * RPU + r) * kStep;
          dma16(rs, valid ? off + (uint32_t)r * rb : kOob, dst);
          if constexpr (F::kMeta) dma4(rm, valid ? moff + (uint32_t)r * mb : kOob, dst + 1024u);
        }
      }
      it.advance();
    }
  }
}

template <int WFMT>
__device__ __forceinline__ void issue_prefetch(const VmParams& P, const PfNext& t, float* smem) {
  if (t.steps <= 0) return;
  const int sw = __builtin_amdgcn_readfirstlane(opaque_tid() >> 6);
  if (P.poll_late == 3 ? sw < kDmaWave0 : sw == 0) return;
  if (t.rpu == 2) issue_prefetch_rpu<WFMT, 2>(P, t, smem, sw);
  else issue_prefetch_rpu<WFMT, 1>(P, t, smem, sw);
}

template <int DEPTH, int WFMT>
__device__ __forceinline__ bool run_task(const VmParams& P, TaskRef t, float* smem) {
  switch (t.type) {
    case AMK_TASK_QKV:
    case AMK_TASK_OPROJ:
    case AMK_TASK_GATEUP:
    case AMK_TASK_DOWN:
    case AMK_TASK_LMHEAD: return task_gemv<DEPTH, WFMT>(P, t, smem);
    case AMK_TASK_ATTN: return task_attn(P, t, smem);
    case AMK_TASK_MERGE: return task_merge(P, t, smem);
    default: return task_nop(P, t, smem);
  }
}

template <int DEPTH, int WFMT>
__device__ __forceinline__ bool run_one(const VmParams& P, TaskRef t, float* smem) {
  const PfNext pf(t);
  const bool ok = run_task<DEPTH, WFMT>(P, t, smem);
  if (ok) issue_prefetch<WFMT>(P, pf, smem);
  return ok;
}


// Argmax of the last step's logits from the LM-head tasks' tagged (max,
// index) partials, lowest index on ties; the same value in every thread.
__device__ __forceinline__ bool greedy_token(const VmParams& P, float* smem, int* tok) {
  const int tid = opaque_tid();
  TagSpin sp;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int k = tid; k < P.n_lm && !sp.failed; k += kThreads) {
    float v[2];
    if (!ld_tagged<2>(P, P.targ + 2 * k, [](int) { return true; }, [](int j) { return j; }, v, sp)) break;
    const int i = __float_as_int(v[1]);
    if (v[0] > best || (v[0] == best && i < bi)) {
      best = v[0];
      bi = i;
    }
  }
  if (block_any(sp.failed, smem)) return false;
  argmax_block(best, bi, smem);
  if (bi < 0 || bi >= P.V) bi = 0;  // all logits NaN: keep the embedding gather in range
  if (tid == 0) reinterpret_cast<int*>(smem)[0] = bi;
  __syncthreads();
  *tok = reinterpret_cast<const int*>(smem)[0];
  __syncthreads();
  return true;
}

// Workgroup b walks queue b in order.  A task that fails its wait (spin
// budget spent, or another workgroup reported an error) ends the walk; the
// error word tells every other workgroup to stop at its next wait.
template <int DEPTH, int WFMT, bool MULTI>
__global__ void __launch_bounds__(kThreads) amk_vm(VmParams P0) {
  extern __shared__ __align__(16) float smem[];
  const int q0 = P0.queue_off[blockIdx.x], q1 = P0.queue_off[blockIdx.x + 1];
  if constexpr (!MULTI) {  // one step: the parameters stay in the kernel-argument segment
    for (int qi = q0; qi < q1; ++qi) {
      const int ti = ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)P0.queue)[qi];
      if (!run_one<DEPTH, WFMT>(P0, ((CTask*)(uintptr_t)P0.tasks)[ti], smem)) return;
    }
    return;
  }
  VmParams P = P0;
  for (int s = 0; s < P0.n_steps; ++s) {
    if (s > 0) {
      // the next token: argmax over the LM-head tasks' partials of step s - 1
      // (every workgroup computes it); then an acquire, so that plain loads
      // of KV rows written in step s - 1 by other workgroups see them
      int tok;
      if (!greedy_token(P, smem, &tok)) return;
      if (blockIdx.x == 0 && opaque_tid() == 0 && P.tokens_out) P.tokens_out[s - 1] = tok;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      P.token = tok;
      P.pos += 1;
      P.tag += 1;
      P.epoch += 1;
    }
    for (int qi = q0; qi < q1; ++qi) {
      const int ti = ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)P.queue)[qi];
      if (!run_one<DEPTH, WFMT>(P, ((CTask*)(uintptr_t)P.tasks)[ti], smem)) return;
    }
  }
  if (blockIdx.x == 0 && P.tokens_out) {  // the last step's token
    int tok;
    if (!greedy_token(P, smem, &tok)) return;
    if (opaque_tid() == 0) P.tokens_out[P0.n_steps - 1] = tok;
  }
}


// Host-visible launch handle of the kernel instance for (pipeline depth,
// weight format); multi selects the greedy multi-step instance.  Each
// (depth, format) pair is instantiated in its own object (vm_inst.hip).
template <int DEPTH, int WFMT>
const void* vm_kernel(bool multi);
#define AMK_DECLARE_VM(D, W) template <> const void* vm_kernel<D, W>(bool multi);
AMK_DECLARE_VM(4, AMK_W_BF16) AMK_DECLARE_VM(4, AMK_W_INT8_ROW) AMK_DECLARE_VM(4, AMK_W_INT4_G128)
AMK_DECLARE_VM(8, AMK_W_BF16) AMK_DECLARE_VM(8, AMK_W_INT8_ROW) AMK_DECLARE_VM(8, AMK_W_INT4_G128)
AMK_DECLARE_VM(16, AMK_W_BF16) AMK_DECLARE_VM(16, AMK_W_INT8_ROW) AMK_DECLARE_VM(16, AMK_W_INT4_G128)
#undef AMK_DECLARE_VM

}  // namespace amk
