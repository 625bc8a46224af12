// Device-side synchronisation and copy helpers shared by the persistent
// kernels: flag waits and publishes, pull-copy tasks, ticket counters and the
// XCD tile queues.
//
// Memory-model contract (agent scope, all 8 XCDs). Data that another
// workgroup consumes inside the same launch (gathered rows, GEMM-RS partial
// tiles) is written with agent-coherent stores (cache policy SC1, the
// encoding of a relaxed agent-scope atomic store on this chip family), which
// complete at the agent's point of coherence instead of staying dirty in one
// XCD's L2. A producer therefore publishes by waiting for its own stores to
// complete (vmcnt 0), a workgroup barrier, then one relaxed agent-scope atomic
// on the counter / flag -- no L2 writeback, which measured ~20 us per publish
// on a busy XCD. A consumer polls the flag with relaxed loads, bounded in
// time, then issues one acquire fence (drops stale cache lines) before its
// loads of the published data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.h"
#include "ocg_internal.h"

namespace ocg {

typedef __attribute__((address_space(1))) const u32x4_t* gcptr16;
typedef __attribute__((address_space(1))) u32x4_t* gptr16;

__device__ __forceinline__ u32x4_t gload16(const void* p) { return *(gcptr16)p; }
__device__ __forceinline__ void gstore16(void* p, u32x4_t v) { *(gptr16)p = v; }
// Store of a final output, written once and read only after the kernel:
// non-temporal (streaming) cache policy, so the output does not crowd the
// L2 lines the kernel's loads reuse (measured: 70B AG-GEMM launch 417.3 ->
// 415.3 us, 8B 83.6 -> 82.0 us).
__device__ __forceinline__ void gstore16_out(void* p, u32x4_t v) { __builtin_nontemporal_store(v, (gptr16)p); }

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }
// Shader-clock cycle counter (its rate follows the compute-unit clock).
__device__ __forceinline__ uint64_t now_cycles() { return __builtin_amdgcn_s_memtime(); }

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ---------------------------------------------------------------- flags

// consume_tile_wait over all the flags a task depends on, run by one whole
// wave: the k-th flag the task enumerates belongs to lane k % 64 (relaxed
// loads, bounded by the timeout); every lane loads its flags together, so a
// round of polls over up to 64 * N flags costs one memory round trip (a
// load per call, awaited before the next call, made a GEMM-RS strip's 128
// pushed-tile flags cost ~23 us), and one acquire fence after the polls
// covers every flag (an agent-scope acquire invalidates the non-coherent
// cache lines, which costs about a microsecond, too much to pay per flag).
// A timed-out wait sets the error word and proceeds, so the grid always
// drains.
template <int N>
struct FlagWaitT {
  uint64_t t0, timeout;
  int k, lane, n;
  bool ok;
  uint32_t seen;
  const uint32_t* ptr[N > 0 ? N : 1];
  uint32_t want[N > 0 ? N : 1];
  __device__ explicit FlagWaitT(uint64_t timeout_ticks)
      : t0(now_ticks()), timeout(timeout_ticks), k(0), lane(threadIdx.x & 63), n(0), ok(true), seen(0) {}
  // The next flag the task depends on, and the value that means "ready":
  // the task's k-th flag goes to lane k % 64.
  __device__ void operator()(const uint32_t* flag, uint32_t value) {
    if ((k++ & 63) == lane) take(flag, value);
  }
  // A flag of this lane's own: the caller computes each lane's flags (flag
  // i on lane i % 64) instead of walking every flag on every lane -- a wave
  // walking 128 flags spent ~18 us on the loop's control flow alone.
  __device__ void add(const uint32_t* flag, uint32_t value) { take(flag, value); }

 private:
  // With N slots a lane records its first N flags and polls them all at
  // once in finish(); a flag beyond them (or every flag, N = 0) is polled
  // here, one load after the other.
  __device__ void take(const uint32_t* flag, uint32_t value) {
    if constexpr (N > 0) {
      if (n < N) {
#pragma unroll
        for (int i = 0; i < N; ++i)
          if (i == n) {
            ptr[i] = flag;
            want[i] = value;
          }
        ++n;
        return;
      }
    }
    uint32_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (v != value && ok) {
      if (now_ticks() - t0 > timeout) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    seen = v;
  }

 public:
  // After the last flag: the recorded flags (their loads issued together,
  // so a round of polls costs one memory round trip, not one per flag), the
  // fence and the error word; returns the number of flags and (in
  // *seen_out) a value lane 0 observed.
  __device__ int finish(const Common& cm, uint32_t* seen_out) {
    if constexpr (N > 0) {
      if (n > 0) {
        for (;;) {
          uint32_t v[N];
          bool done = true;
#pragma unroll
          for (int i = 0; i < N; ++i)
            if (i < n) v[i] = __hip_atomic_load(ptr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int i = 0; i < N; ++i)
            if (i < n && v[i] != want[i]) done = false;
          seen = v[0];
          if (done || !ok) break;
          if (now_ticks() - t0 > timeout) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (!ok) __hip_atomic_fetch_or(&cm.hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *seen_out = __shfl(seen, 0);
    return k;
  }
};
// Flags polled one after the other: for waits on a flag or two (a tile's
// start), where recorded flags would cost registers. Waits on many flags
// (a GEMM-RS strip: 16 tile flags pulled, 128 pushed) use FlagWaitT<2>.
using FlagWait = FlagWaitT<0>;

// Wait until every store this thread issued has completed (for the
// agent-coherent stores below: is visible at agent scope).
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache-policy immediate of buffer stores: SC1 = agent-scope coherent.
constexpr int kAgentCoherent = 16;

__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)byte_off, 0, kAgentCoherent);
}

// produce_tile_notify for copy tasks: called by every thread after its
// agent-coherent stores; returns (to thread 0) whether this task published
// flag `f` (the last of its copy tasks does).
__device__ __forceinline__ bool publish_slab(uint32_t* cnt, uint32_t* flag, int f, int target, uint32_t epoch,
                             const Common& cm) {
  drain_stores();
  __syncthreads();
  bool published = false;
  if (threadIdx.x == 0) {
    uint32_t old = __hip_atomic_fetch_add(&cnt[f], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)old + 1 == target) {
      __hip_atomic_store(&cnt[f], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f != cm.fault_skip_slab)
        __hip_atomic_store(&flag[f], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      published = true;
    }
  }
  return published;
}

// Test hook: hold a copy task back by `rounds` x s_sleep 127 (64 x 127
// shader cycles each) before it moves any data, so the flags it completes
// are published late and dependent tiles really wait.
__device__ __forceinline__ void copy_delay(uint32_t rounds) {
  for (uint32_t i = 0; i < rounds; ++i) __builtin_amdgcn_s_sleep(127);
}

// ---------------------------------------------------------------- copy

// Pull `n16` 16-byte granules from src to dst (agent-coherent stores) with
// all NT threads of the workgroup, 16 granules in flight per thread.
// n16 * 16 < 2^31.
template <int NT = kThreads, int U = 16>
__device__ __forceinline__ void copy_granules(const uint16_t* src, uint16_t* dst, uint32_t n16) {
  const u32x4_t* s = (const u32x4_t*)src;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, n16 * 16u);
  uint32_t i = threadIdx.x;
  for (; i + (uint32_t)(U - 1) * NT < n16; i += (uint32_t)U * NT) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = gload16(s + i + u * NT);
#pragma unroll
    for (int u = 0; u < U; ++u) store16_agent(rs, (i + u * NT) * 16u, v[u]);
  }
  for (; i < n16; i += NT) store16_agent(rs, i * 16u, gload16(s + i));
}

// Pull a rows x (gpr granules) block: row i of src (row stride `stride`
// elements) to row i of dst (same stride), agent-coherent stores, U granules
// in flight per thread, consecutive threads on consecutive granules of a row.
// The block spans ((rows - 1) * stride + gpr * 8) * 2 < 2^31 bytes.
template <int NT, int U>
__device__ __forceinline__ void copy_block(const uint16_t* src, uint16_t* dst, uint32_t rows, uint32_t gpr,
                                           uint32_t stride) {
  const uint32_t n16 = rows * gpr;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, ((rows - 1) * stride + gpr * 8) * 2u);
  // every round issues all of its (up to U) loads before its stores, the
  // last, partial round included
  for (uint32_t i = threadIdx.x; i < n16; i += (uint32_t)U * NT) {
    u32x4_t v[U];
    uint32_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = i + u * NT, r = j / gpr;
      off[u] = r * stride + (j - r * gpr) * 8;
      if (j < n16) v[u] = gload16(src + off[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u * NT < n16) store16_agent(rs, off[u] * 2u, v[u]);
  }
}

// The same rectangle with few registers, for the side producer: source and
// destination through buffer descriptors (32-bit lane offsets), lane
// positions stepped without division, and the descriptors' range checks in
// place of per-granule bounds tests (a position past the last row lies past
// the rectangle's last byte: loads return zeros, stores are dropped).
// gpr * 8 <= stride; offsets stay below 2^32.
template <int NT, int U>
__device__ __forceinline__ void copy_rect(const uint16_t* src, uint16_t* dst, uint32_t rows, uint32_t gpr,
                                          uint32_t stride) {
  const uint32_t ext = ((rows - 1) * stride + gpr * 8) * 2u;
  const __amdgpu_buffer_rsrc_t ss = make_rsrc(src, ext), ds = make_rsrc(dst, ext);
  const uint32_t n16 = rows * gpr, dr = NT / gpr, dg = NT % gpr;
  uint32_t r = threadIdx.x / gpr, g = threadIdx.x % gpr;
  for (uint32_t base = 0; base < n16; base += (uint32_t)U * NT) {
    uint32_t off[U];
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      off[u] = (r * stride + g * 8) * 2u;
      v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ss, (int)off[u], 0, 0));
      r += dr;
      g += dg;
      if (g >= gpr) {
        g -= gpr;
        ++r;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) store16_agent(ds, off[u], v[u]);
  }
}

// One copy task of the AllGather (pull mode): rows [row0, row1) x columns
// [k0, k1) of the gathered matrix come from rank `chunk`'s shard; the last of
// the tasks of a (slab, K-slab) publishes its flag.
// LEAN: the side producer's form (copy_rect, few registers).
template <int NT = kThreads, int U = 16, bool LEAN = false>
__device__ __forceinline__ void run_copy_task(const AgPlan& p, const uint16_t* const* chunks, uint16_t* a_gathered,
                              uint32_t* slab_cnt, uint32_t* slab_flag, int u, uint32_t epoch,
                              const Common& cm) {
  const uint64_t t0 = now_ticks(), c0 = now_cycles();
  const CopyDesc d = copy_desc(p, u);
  copy_delay(cm.copy_delay * (uint32_t)(d.kslab + 1));   // later K-slabs land later
  const uint16_t* src = chunks[d.chunk] + (size_t)(d.row0 - d.chunk * p.m) * p.K + d.k0;
  uint16_t* dst = a_gathered + (size_t)d.row0 * p.K + d.k0;
  if constexpr (LEAN)
    copy_rect<NT, U>(src, dst, (uint32_t)(d.row1 - d.row0), (uint32_t)(d.k1 - d.k0) / 8, (uint32_t)p.K);
  else if (d.k1 - d.k0 == p.K)
    copy_granules<NT, U>(src, dst, (uint32_t)((size_t)(d.row1 - d.row0) * p.K / 8));
  else
    copy_block<NT, U>(src, dst, (uint32_t)(d.row1 - d.row0), (uint32_t)(d.k1 - d.k0) / 8, (uint32_t)p.K);
  const int target = slab_target(p.m, p.S, p.CT, p.bpr, d.slab);
  const bool pub = publish_slab(slab_cnt, slab_flag, d.flag, target, epoch, cm);
  if (threadIdx.x == 0 && cm.trace && (uint32_t)u < cm.trace_cap) {
    ocg_trace_rec* r = cm.trace + u;
    const uint64_t t1 = now_ticks();
    r->ticket = u; r->kind = 1; r->a = d.chunk; r->b = d.piece; r->c = d.flag; r->d = (pub ? 1u : 0u) | (LEAN ? 2u : 0u);
    r->hw = (xcc_id() << 16) | blockIdx.x; r->epoch = epoch;
    r->t_start = t0; r->t_ready = t1; r->t_end = t1; r->flag_seen = 0; r->queue = d.kslab;
    r->cycles = now_cycles() - c0; r->wait_ticks = 0; r->pad = 0;
  }
}

// ---------------------------------------------------------------- scheduling helpers

__device__ __forceinline__ uint32_t read_epoch(WsHeader* hdr, uint32_t* s_bcast) {
  if (threadIdx.x == 0) {
    uint32_t e = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    s_bcast[1] = e ? e : 1u;
    s_bcast[3] = xcc_id();
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_bcast[1]);   // uniform: kept in a scalar register
}

__device__ __forceinline__ uint32_t next_ticket(uint32_t* counter, uint32_t* s_bcast) {
  __syncthreads();
  if (threadIdx.x == 0)
    s_bcast[0] = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_bcast[0]);
}

// Next tile from the XCD queues: own XCD first, then the others. `*q` is the
// queue being drained (starts at the XCD id). When it runs dry, one relaxed
// load per queue (all eight in parallel) finds the queues that may still hold
// tiles -- a queue whose ticket is past its last tile is empty for good, since
// tickets only grow within a launch -- and the search moves to the next of
// them; -1 once none is left. `*tried` is unused (kept for the call sites).
__device__ __forceinline__ int next_tile(WsHeader* hdr, int n_tiles, int* q, int* tried, uint32_t* s_bcast,
                                         uint32_t* t_out, int xcd_remap = 1) {
  (void)tried;
  if (!xcd_remap) {
    // ablation: one queue (queue 0's ticket) in plain tile order
    const uint32_t t = next_ticket(&hdr->xtick[0], s_bcast);
    *q = 0;
    *t_out = t;
    return (int)t < n_tiles ? (int)t : -1;
  }
  for (;;) {
    const uint32_t t = next_ticket(&hdr->xtick[*q * kHdrWords], s_bcast);
    const int v = xcd_tile(*q, (int)t, n_tiles);
    if (v >= 0) {
      *t_out = t;
      return v;
    }
    if (threadIdx.x < 64) {
      bool open = false;
      if (threadIdx.x < kXcds) {
        const uint32_t x = __hip_atomic_load(&hdr->xtick[threadIdx.x * kHdrWords], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        open = xcd_tile((int)threadIdx.x, (int)x, n_tiles) >= 0;
      }
      const uint64_t m = __ballot(open);
      if (threadIdx.x == 0) s_bcast[5] = (uint32_t)m;
    }
    __syncthreads();
    const uint32_t mask = __builtin_amdgcn_readfirstlane(s_bcast[5]);
    if (mask == 0) return -1;
    // next open queue after *q, cyclically
    const uint32_t rot = ((mask >> ((*q + 1) % kXcds)) | (mask << (kXcds - (*q + 1) % kXcds))) & 0xFFu;
    *q = (*q + 1 + __builtin_ctz(rot)) % kXcds;
  }
}

// Last workgroup out resets the counters and records the epoch. Relaxed
// atomics suffice: a workgroup arrives here only after its last ticket
// fetch returned (its value decided the exit), and the next launch on the
// stream is ordered after this one by the kernel boundary. When a call runs
// two kernels at once (GEMM + side producer), `total` counts the workgroups
// of both: the last of them resets, after every workgroup of either kernel
// has read the call's epoch at its start.
__device__ __forceinline__ void finish(WsHeader* hdr, uint32_t epoch, int total = 0) {
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t d = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d + 1 == (total > 0 ? (uint32_t)total : gridDim.x)) {
      __hip_atomic_store(&hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->side_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int q = 0; q < kXcds; ++q)
        __hip_atomic_store(&hdr->xtick[q * kHdrWords], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// c0: shader-clock cycle count at t0 (0 = not measured); wait: ticks spent in
// flag waits after t1.
__device__ __forceinline__ void trace_task(const Common& cm, uint32_t slot, uint32_t kind, uint32_t a, uint32_t b,
                                           uint32_t c, uint32_t d, uint32_t epoch, uint64_t t0, uint64_t t1,
                                           uint32_t seen, uint32_t queue_ticket, uint64_t c0 = 0,
                                           uint32_t wait = 0) {
  if (threadIdx.x == 0 && cm.trace && slot < cm.trace_cap) {
    ocg_trace_rec* r = cm.trace + slot;
    r->ticket = slot; r->kind = kind; r->a = a; r->b = b; r->c = c; r->d = d;
    r->hw = (xcc_id() << 16) | blockIdx.x; r->epoch = epoch;
    r->t_start = t0; r->t_ready = t1; r->t_end = now_ticks(); r->flag_seen = seen; r->queue = queue_ticket;
    r->cycles = c0 ? now_cycles() - c0 : 0; r->wait_ticks = wait; r->pad = 0;
  }
}

}  // namespace ocg
