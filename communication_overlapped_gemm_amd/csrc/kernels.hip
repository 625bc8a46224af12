// gfx950 kernels of the communication-overlapped GEMM library.
//
// One persistent kernel per operation. Each workgroup (4 waves of 64) first
// takes copy tasks from a global ticket counter -- pull one piece of a peer's
// shard into the gathered buffer, then publish the slab's flag
// ("produce_tile_notify") -- and then GEMM tiles from its XCD's queue, each
// tile waiting on the flags of the slabs it reads ("consume_tile_wait")
// before the MFMA main loop of gemm_core.h. The primitives follow "TileLink:
// Generating Efficient Compute-Communication Overlapping Kernels using
// Tile-Centric Primitives" (MLSys 2025 talk summary), "Technical Deep Dive":
// signal primitives between producer and consumer tiles; a notify lowered to
// a synchronisation, the tile id and an atomic; pull transfers whose
// "transfer complete" barrier is the slab flag; lookup tables for the
// dynamic (MoE) dependencies.
//
// The memory-model contract of the flags and copies is stated in sync.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gemm_core.h"
#include "ocg_internal.h"
#include "sync.h"

namespace ocg {

// ---------------------------------------------------------------- AG-GEMM

// Direct-to-LDS 4-byte load of *g (agent-coherent: SC1, as a relaxed
// agent-scope atomic load) into LDS address lds + 4 * lane.
__device__ __forceinline__ void dma_flag(uint32_t lds, const uint32_t* g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off sc1" ::"s"(lds), "v"(g) : "memory", "m0");
}

// consume_tile_wait per K-slab inside an AG-GEMM tile's K loop. The tile
// depends on `ndeps` peer slabs (lane i of wave 0 holds the flag row of dep
// i). K-slabs are confirmed in groups that double in size (kgroup_first):
// pair k of the loop loads stages up to min(k + S, nk - 1), so before the
// first pair that loads a stage of group g, wave 0 confirms the flags of
// every (dep, K-slab of g), one lane each, and all waves then pass the
// pair's barrier. The flags are read one or two pairs early (PD) by a
// direct-to-LDS load, which the loop's vmcnt waits count: it has landed by
// the check, so the check costs no memory round trip. A flag not yet set
// (or a group of more than 64 flags) is polled by wave 0 before the barrier,
// bounded as FlagWait. After seeing the flags, wave 0 invalidates the
// non-coherent cache lines (buffer_inv sc1, the acquire half of the
// agent-scope handshake; the load that observed the flags has completed) --
// without the vmcnt(0) a compiler acquire fence adds, which would drain the
// ring's loads in flight. The invalidate is not free (it drops the XCD L2's
// non-coherent lines that the other tiles reuse), hence the doubling groups.
template <int S, int PD>
struct KslabHook {
  OCG_LDS const uint64_t* rows;   // LDS: address of slab_flag + dep_i * nks, i < ndeps (kept in
                                  // LDS, not registers, for the whole K loop)
  OCG_LDS uint32_t* land;         // 64 words of LDS the prefetched flags land in
  const Common* cm;
  uint32_t epoch, wait_ticks;
  int wave, ndeps, spk, nks, nk;
  int g, j0, j1, check_k, prefetch_k;   // next group: K-slabs [j0, j1)
  bool prefetched;

  // flag of lane L in the group: dep L / gs, K-slab j0 + L % gs (lanes past
  // the last pair repeat pair 0)
  __device__ __forceinline__ const uint32_t* lane_flag(int L) const {
    const int gs = j1 - j0;
    const int i = (L / gs < ndeps) ? L / gs : 0;
    const int j = (L / gs < ndeps) ? j0 + L % gs : j0;
    return (const uint32_t*)rows[i] + j;
  }
  __device__ void schedule() {
    prefetched = false;
    j0 = kgroup_first(g);
    if (j0 >= nks || j0 * spk > nk - 1) {
      check_k = prefetch_k = 1 << 30;
      return;
    }
    j1 = min(kgroup_first(g + 1), nks);
    int kc = j0 * spk - S;
    kc = kc < 0 ? 0 : (kc + 1) & ~1;
    check_k = kc;
    prefetch_k = (ndeps * (j1 - j0) <= 64) ? kc - 2 * PD : -1;
  }
  __device__ __forceinline__ void prefetch(int k) {
    if (k == prefetch_k) {
      if (wave == 0) dma_flag(lds_u32(land), lane_flag(threadIdx.x & 63));
      prefetched = true;
    }
  }
  __device__ __forceinline__ void check(int k) {
    if (k != check_k) return;
    if (wave == 0) {
      bool ok = false;
      if (prefetched) ok = __ballot(land[threadIdx.x & 63] != epoch) == 0;
      if (ok) {
        asm volatile("buffer_inv sc1" ::: "memory");
      } else {
        const uint64_t t0 = now_ticks();
        FlagWait w(cm->timeout_ticks);
        const int gs = j1 - j0;
        for (int L = threadIdx.x & 63; L < ndeps * gs; L += 64) w.add((const uint32_t*)rows[L / gs] + j0 + L % gs, epoch);
        uint32_t seen;
        w.finish(*cm, &seen);
        wait_ticks += (uint32_t)(now_ticks() - t0);
      }
    }
    ++g;
    schedule();
  }
};

// Split K, the combine of a tile's two K halves (called by every thread after
// the half's K loop). The half that arrives first stores its fp32 sums (each
// thread's 16-byte accumulator blocks at (block * NT + thread) * 16 bytes of
// the tile's slot, agent-coherent) and publishes the tile's flag; it returns
// false (nothing more to do). The second resets the arrival count, waits for
// the flag -- the first half is already past its K loop, so the wait ends --
// and adds the stored sums to its own: a + b rounds the same whichever half
// came first, so C does not depend on the order. Returns true: the caller
// writes the tile.
template <int BM, int BN>
__device__ bool combine_halves(const AgArgs& args, int v, AccTile<BM, BN>& acc, uint32_t epoch, uint32_t* s_bcast,
                               uint32_t* seen) {
  using G = Gemm<BM, BN>;
  if (threadIdx.x == 0)
    s_bcast[6] = __hip_atomic_fetch_add(&args.sk_cnt[v], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t before = __builtin_amdgcn_readfirstlane(s_bcast[6]);
  float* slot = args.sk_part + (size_t)v * (BM * BN);
  if (before == 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(slot, (uint32_t)(BM * BN * 4));
#pragma unroll
    for (int f = 0; f < G::FM; ++f)
#pragma unroll
      for (int g = 0; g < G::FN; ++g)
        store16_agent(rs, (uint32_t)(((f * G::FN + g) * G::NT + threadIdx.x) * 16),
                      __builtin_bit_cast(u32x4_t, acc.v[f][g]));
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(&args.sk_flag[v], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  if (threadIdx.x == 0) __hip_atomic_store(&args.sk_cnt[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x < 64) {
    FlagWait w(args.cm.timeout_ticks);
    if (threadIdx.x == 0) w.add(&args.sk_flag[v], epoch);
    w.finish(args.cm, seen);
  }
  __syncthreads();
  const f32x4_t* src = (const f32x4_t*)slot;
#pragma unroll
  for (int f = 0; f < G::FM; ++f) {
    f32x4_t x[G::FN];
#pragma unroll
    for (int g = 0; g < G::FN; ++g) x[g] = src[(f * G::FN + g) * G::NT + threadIdx.x];
#pragma unroll
    for (int g = 0; g < G::FN; ++g) acc.v[f][g] += x[g];
    __builtin_amdgcn_sched_barrier(0);
  }
  return true;
}

// SPLIT: work units are K halves of tiles (plan.sk == 2); otherwise tiles.
template <int BM, int BN, bool SPLIT>
__global__ __launch_bounds__((Gemm<BM, BN>::NT), 1) void ag_gemm_kernel(AgArgs args) {
  using G = Gemm<BM, BN>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[G::LDS_BYTES + 256];
  __shared__ uint64_t s_deprow[64];   // flag rows of the tile's dependency slabs
  __shared__ uint32_t s_bcast[8];
  OCG_LDS char* smem = (OCG_LDS char*)smem_raw;
  const AgPlan& p = args.plan;
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  // copy tasks: all of them, or (SIDE transfer) the first K-slab of the
  // first phase, so the first tiles need not wait for the side producer to
  // start; the producer takes the rest (none: no ticket to take)
  while (p.n_inline > 0) {
    const uint32_t u = next_ticket(&cm.hdr->ticket, s_bcast);
    if ((int)u >= p.n_inline) break;
    run_copy_task<G::NT>(p, args.chunks, args.a_gathered, args.slab_cnt, args.slab_flag, (int)u, epoch, cm);
  }
  // GEMM tiles
  int q = (int)__builtin_amdgcn_readfirstlane(s_bcast[3]) % kXcds, tried = 0;
  uint32_t qt = 0;
  TileCtx<BM, BN> t;
  const int kl = SPLIT ? p.K / 2 : p.K;             // K columns of one work unit
  t.N = p.N;
  t.nk = kl / BKS;
  const int spk = p.KS / BKS;                       // stages per K-slab (>= 8)
  for (;;) {
    const int vu = next_tile(cm.hdr, SPLIT ? 2 * p.n_tiles : p.n_tiles, &q, &tried, s_bcast, &qt, cm.xcd_remap);
    if (vu < 0) break;
    const int v = SPLIT ? vu >> 1 : vu, half = SPLIT ? vu & 1 : 0;
    const size_t k0 = (size_t)half * kl;           // first K column of the unit
    t.brs = make_rsrc(args.b + k0 * p.N, (uint32_t)((size_t)kl * p.N * 2));
    const uint64_t t0 = now_ticks(), c0 = now_cycles();
    int rb, cb;
    tile_of(p.n_rb, p.n_cb, p.rb0, v, &rb, &cb);
    const int r0 = rb * BM, r1 = min(r0 + BM, p.M);
    // peer slabs the tile reads; wave 0 lane i keeps the flag row of dep i
    int ndeps = 0;
    uint64_t myrow = (uint64_t)args.slab_flag;
    if (p.mode == 0)
      for_each_dep_slab(p.m, p.S, p.bpr, p.local, r0, r1, [&](int sl) {
        if (ndeps == 0 || ndeps == lane) myrow = (uint64_t)(args.slab_flag + (size_t)sl * p.nks);
        ++ndeps;
      });
    uint32_t seen = 0;
    if (ndeps > 0 && wave == 0) {
      // consume_tile_wait on K-slab 0 (group 0), which holds every stage the
      // prologue loads: lane i polls dep i's flag
      FlagWait w(cm.timeout_ticks);
      if (lane < ndeps) w.add((const uint32_t*)myrow, epoch);
      w.finish(cm, &seen);
      seen = __builtin_amdgcn_readfirstlane(seen);
      s_deprow[lane] = myrow;
    }
    const uint64_t t1 = now_ticks();
    __syncthreads();
    // Rows of the local chunk come from the local shard; all others from the
    // gathered buffer filled by the copy tasks.
#pragma unroll
    for (int i = 0; i < G::A_PER_WAVE; ++i) {
      const int row = min(r0 + dma_row<BM, BN>(wave, i, lane), p.M - 1);
      const int c = row / p.m;
      t.rowp[i] = (const char*)(((c == p.local) ? args.chunks[c] + (size_t)(row - c * p.m) * p.K
                                                : args.a_gathered + (size_t)row * p.K) + k0);
    }
    const int n0 = cb * BN;
    t.n0 = n0;
    AccTile<BM, BN> acc;
    uint32_t d = 0, wait_ticks = 0;
    if constexpr (SPLIT) {
      // one K-slab, which the start wait covered: nothing to check in the loop
      mainloop<BM, BN>(smem, t, acc);
      uint32_t seen2 = 0;
      const uint64_t tc = now_ticks();
      const bool writes = combine_halves<BM, BN>(args, v, acc, epoch, s_bcast, &seen2);
      d = (uint32_t)half | (writes ? 2u : 0u);
      if (!writes) {
        trace_task(cm, (uint32_t)(p.n_copy + vu), 2, rb, cb, ndeps, d, epoch, t0, t1, seen,
                   ((uint32_t)q << 16) | qt, c0, 0);
        continue;
      }
      wait_ticks = (uint32_t)(now_ticks() - tc);
    } else {
      KslabHook<G::S, (G::S >= 6 ? 2 : 1)> hook;
      hook.rows = (OCG_LDS const uint64_t*)s_deprow;
      hook.land = (OCG_LDS uint32_t*)(smem + G::LDS_BYTES);
      hook.cm = &cm;
      hook.epoch = epoch;
      hook.wait_ticks = 0;
      hook.wave = wave;
      hook.ndeps = ndeps;
      hook.spk = spk;
      hook.nks = ndeps > 0 ? p.nks : 0;   // no dependency: nothing to check
      hook.nk = t.nk;
      hook.g = 1;
      hook.schedule();
      mainloop<BM, BN>(smem, t, acc, hook);
      wait_ticks = hook.wait_ticks;
    }
    stage_c<BM, BN>(smem, acc);
    for_each_c_chunk<BM, BN>(smem, [&](int row, int col, u32x4_t val) {
      if (r0 + row < p.M && n0 + col < p.N) gstore16_out(args.c + (size_t)(r0 + row) * p.N + n0 + col, val);
    });
    trace_task(cm, (uint32_t)(p.n_copy + vu), 2, rb, cb, ndeps, d, epoch, t0, t1, seen, ((uint32_t)q << 16) | qt, c0,
               wait_ticks);
  }
  finish(cm.hdr, epoch, cm.total_wgs);
}

// Side producer of the AllGather (transfer mode SIDE): the copy tasks of an
// ocg_ag_gemm call, run by a small kernel on a second stream while the GEMM
// kernel's tiles compute on the same compute units. It uses no LDS beyond
// the ticket broadcast and at most 40 registers per lane (the GEMM wave of a
// SIMD leaves that many of the 512 free), so one of its workgroups fits on
// every compute unit next to a GEMM workgroup; its copies never wait.
__global__ __launch_bounds__(kSideThreads) void ag_side_copy_kernel(AgArgs args) {
  __shared__ uint32_t s_bcast[8];
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  for (;;) {
    const int u = args.plan.n_inline + (int)next_ticket(&cm.hdr->side_ticket, s_bcast);
    if (u >= args.plan.n_copy) break;
    run_copy_task<kSideThreads, 4, true>(args.plan, args.chunks, args.a_gathered, args.slab_cnt, args.slab_flag, u,
                                         epoch, cm);
  }
  finish(cm.hdr, epoch, cm.total_wgs);
}

// ---------------------------------------------------------------- GEMM-RS

// Reduce strip: out rows [r0, r1) = bf16( sum over ranks s = 0..R-1, in
// that order, of the bf16 partials P_s ), fp32 accumulation, one rounding.
// Every 16-byte chunk issues the loads of all ranks before adding, U chunks
// per round, so each thread keeps up to U * R loads in flight.
template <int NT>
__device__ void run_reduce_strip(const RsArgs& a, int r0, int r1) {
  constexpr int U = 2;
  const RsPlan& p = a.plan;
  const int lo = p.local * p.blk;
  const size_t first = (size_t)r0 * p.N / 8, n16 = (size_t)(r1 - r0) * p.N / 8;
  for (size_t base = threadIdx.x; base < n16; base += (size_t)U * NT) {
    u32x4_t v[U][kMaxRanks];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * NT;
      if (i >= n16) continue;
#pragma unroll
      for (int s = 0; s < kMaxRanks; ++s) {
        if (s < p.R) v[u][s] = gload16(a.src[s] + (first + i) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * NT;
      if (i >= n16) continue;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = bf16_to_f32((v[u][0][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
#pragma unroll
      for (int s = 1; s < kMaxRanks; ++s) {
        if (s < p.R) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += bf16_to_f32((v[u][s][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
        }
      }
      u32x4_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7])};
      gstore16_out(a.out + (first + i) * 8 - (size_t)lo * p.N, o);
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__((Gemm<BM, BN>::NT), 1) void gemm_rs_kernel(RsArgs args) {
  using G = Gemm<BM, BN>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[G::LDS_BYTES];
  __shared__ uint32_t s_bcast[8];
  OCG_LDS char* smem = (OCG_LDS char*)smem_raw;
  const RsPlan& p = args.plan;
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  int q = (int)__builtin_amdgcn_readfirstlane(s_bcast[3]) % kXcds, tried = 0;
  uint32_t qt = 0;
  TileCtx<BM, BN> t;
  t.brs = make_rsrc(args.b, (uint32_t)((size_t)p.K * p.N * 2));
  t.N = p.N;
  t.nk = p.K / BKS;
  for (;;) {
    const int v = next_tile(cm.hdr, p.n_tiles, &q, &tried, s_bcast, &qt, cm.xcd_remap);
    if (v < 0) break;
    const uint64_t t0 = now_ticks();
    int rb, cb;
    tile_of(p.n_rb, p.n_cb, p.rb0, v, &rb, &cb);
    const int r0 = rb * BM;
#pragma unroll
    for (int i = 0; i < G::A_PER_WAVE; ++i) {
      const int row = min(r0 + dma_row<BM, BN>(wave, i, lane), p.M - 1);
      t.rowp[i] = (const char*)(args.a + (size_t)row * p.K);
    }
    const int n0 = cb * BN;
    t.n0 = n0;
    AccTile<BM, BN> acc;
    mainloop<BM, BN>(smem, t, acc);
    stage_c<BM, BN>(smem, acc);
    // The bf16 partial tile is consumed by reduce strips of this launch (or,
    // pushed, by the rank that owns its row block): agent-coherent stores.
    const int rows = min(BM, p.M - r0);
    const int sblk = r0 / p.blk;   // row block (rank) the tile belongs to
    const __amdgpu_buffer_rsrc_t prs =
        make_rsrc(args.dst[sblk] + (size_t)r0 * p.N, (uint32_t)((size_t)rows * p.N * 2));
    for_each_c_chunk<BM, BN>(smem, [&](int row, int col, u32x4_t val) {
      if (row < rows && n0 + col < p.N) store16_agent(prs, (uint32_t)(((size_t)row * p.N + n0 + col) * 2), val);
    });
    // produce_tile_notify (pull: our tile flag; push: the owner's receive flag)
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
      if (args.push)
        __hip_atomic_store(&args.rflag[sblk][p.local * args.tpb + (rb - sblk * args.local_nrb) * p.n_cb + cb],
                           args.flag_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store(&args.tile_flag[rb * p.n_cb + cb], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    trace_task(cm, (uint32_t)v, 3, rb, cb, rs_tile_touches_local(p, rb) ? 1u : 0u, 0, epoch, t0, t0, 0,
               ((uint32_t)q << 16) | qt);
  }
  // reduce strips, once every tile has been claimed
  for (;;) {
    const uint32_t j = next_ticket(&cm.hdr->ticket, s_bcast);
    if ((int)j >= p.n_red) break;
    const uint64_t t0 = now_ticks();
    // consume_tile_wait on the local tiles of the strip, peer_tile_wait on
    // the peers' tiles, then the fixed-order reduce.
    int r0, r1;
    rs_strip(p, (int)j, &r0, &r1);
    // The first strip of each row block (the lowest ticket among its strips,
    // so it is claimed first) polls the flags of the block's tiles and then
    // sets the block's summary word; every other strip of the block polls
    // that one word. (Every strip polling every flag of its block put
    // ~32K loads on a few flag lines at once: ~18 us per poll round.)
    uint32_t seen = 0, designated = 0;
    int nwait = 0;
    uint64_t t_own = 0;
    if (wave == 0) {
      const int lo = p.local * p.blk;
      for (int rb = r0 / BM; rb <= (r1 - 1) / BM; ++rb) {
        const int first = rb * BM > lo ? rb * BM : lo;   // the block's first local row
        if (first < r0 || first >= r1) continue;
        // flag f of the block on lane f % 64: f = cb * per_tile + q, q = 0 the
        // tile's own flag (pull) or rank 0's push, q > 0 a peer's
        FlagWaitT<2> w(cm.timeout_ticks);
        const int per_tile = args.push ? p.R : 1 + (args.peer_flags ? p.R - 1 : 0);
        const int nf = p.n_cb * per_tile;
        for (int f = lane; f < nf; f += 64) {
          const int cb = f / per_tile, q = f - cb * per_tile;
          const int t_local = (rb - args.local_rb0) * p.n_cb + cb;
          if (args.push) {
            // every rank's pushed tile in our receive buffer, ours included
            w.add(&args.rflag[p.local][q * args.tpb + t_local], args.flag_value);
          } else if (q == 0) {
            w.add(&args.tile_flag[rb * p.n_cb + cb], epoch);
          } else {
            const int s = q - 1 < p.local ? q - 1 : q;   // the peers, skipping the local rank
            w.add(&args.peer_flags[s * args.local_nrb * p.n_cb + t_local], args.peer_flag_value);
          }
        }
        const uint64_t tw = now_ticks();
        w.finish(cm, &seen);   // ends with the acquire fence
        nwait += nf;
        t_own += now_ticks() - tw;
        ++designated;
        // set even after a timeout (the error word is set): the block's other
        // strips must not wait on it for a second bound
        if (lane == 0)
          __hip_atomic_store(&args.rs_sum[rb - args.local_rb0], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      FlagWait ws(cm.timeout_ticks);
      int nsum = 0;
      for (int rb = r0 / BM; rb <= (r1 - 1) / BM; ++rb) {
        const int first = rb * BM > lo ? rb * BM : lo;
        if (first >= r0 && first < r1) continue;
        ws(&args.rs_sum[rb - args.local_rb0], epoch);
        ++nsum;
      }
      if (nsum) {
        uint32_t seen_sum;
        nwait += ws.finish(cm, &seen_sum);
        if (!seen) seen = seen_sum;
      }
    }
    // trace: the flags the strip depends on (polled by it or by its blocks'
    // first strips), and in the next field the flags it polled itself
    const int per_tile = args.push ? p.R : 1 + (args.peer_flags ? p.R - 1 : 0);
    const int ndeps = ((r1 - 1) / BM - r0 / BM + 1) * p.n_cb * per_tile;
    const uint64_t t1 = now_ticks();
    __syncthreads();
    run_reduce_strip<G::NT>(args, r0, r1);
    // queue: row blocks this strip polled the tile flags of; wait ticks: time in those polls
    trace_task(cm, (uint32_t)(p.n_tiles + j), 5, r0, r1, ndeps, nwait, epoch, t0, t1, seen, designated, 0,
               (uint32_t)t_own);
  }
  finish(cm.hdr, epoch);
}

// ---------------------------------------------------------------- MoE routing

// Routing runs as two kernels over blocks of kRouteBlock tokens, so every
// step is spread over the chip: (1) per token top-k of the fp32 logits (ties
// -> lower expert, slot 0 = larger logit) and softmax weights, one lane per
// expert, plus a per-block expert histogram; (2) per block, the expert
// bases of the block (histograms of the blocks before it) and the expert
// offsets (totals, scanned across the wave), then a stable rank of the
// block's token slots within each expert gives the expert-sorted slot list
// perm (stable in expert, then token, then slot). Block 0 also writes the
// offsets and the grouped-tile lookup table (the dynamic dependency table:
// expert, first row, rows, column block per tile).

// Wave-wide maximum / sum of one value per lane: DPP within rows of 16
// lanes, then the lane swaps across rows (no LDS round trips).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float wave_reduce(float x) {
  auto op = [](float u, float v) { return MAX ? fmaxf(u, v) : u + v; };
  x = op(x, dpp_f<0xB1>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp_f<0x4E>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp_f<0x141>(x));   // row_half_mirror
  x = op(x, dpp_f<0x140>(x));   // row_mirror
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Top-k of each token with one lane per expert: a routing block of
// kRouteBlock tokens per workgroup, kRouteTokW consecutive tokens per wave,
// all their logit rows loaded at once (coalesced). Per token: the wave
// maximum and softmax denominator, then k rounds of "largest remaining
// logit, lowest expert among equals" (a wave maximum, then the lowest lane
// holding it), each pick's weight and a count in the block histogram.
constexpr int kRouteWaves = 16;
constexpr int kRouteTokW = kRouteBlock / kRouteWaves;

__global__ __launch_bounds__(64 * kRouteWaves) void moe_topk_kernel(RouteArgs a) {
  __shared__ int s_cnt[kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, E = a.E, K = a.topk;
  if (threadIdx.x < kMaxExperts) s_cnt[threadIdx.x] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kRouteBlock + wave * kRouteTokW;
  float v[kRouteTokW];
#pragma unroll
  for (int i = 0; i < kRouteTokW; ++i)
    v[i] = (t0 + i < a.T && lane < E) ? a.logits[(size_t)(t0 + i) * E + lane] : -INFINITY;
#pragma unroll
  for (int i = 0; i < kRouteTokW; ++i) {
    const int t = t0 + i;
    if (t >= a.T) break;
    const float mx = wave_reduce<true>(v[i]);
    const float sum = wave_reduce<false>(lane < E ? __expf(v[i] - mx) : 0.f);
    float y = v[i];
    for (int j = 0; j < K; ++j) {
      const float m = wave_reduce<true>(y);
      const int e = __builtin_ctzll(__ballot(lane < E && y == m));
      if (lane == 0) {
        a.topk_ids[t * K + j] = e;
        a.topk_w[t * K + j] = __expf(m - mx) / sum;
        atomicAdd(&s_cnt[e], 1);
      }
      if (lane == e) y = -INFINITY;
    }
  }
  __syncthreads();
  if (threadIdx.x < E) a.blk_cnt[blockIdx.x * E + threadIdx.x] = s_cnt[threadIdx.x];
}

// Exclusive prefix sum across the wave; *total gets the wave's sum.
__device__ __forceinline__ int wave_excl_scan(int x, int* total) {
  const int lane = threadIdx.x & 63;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  *total = __shfl(incl, 63);
  return incl - x;
}

__global__ __launch_bounds__(kRouteBlock) void moe_scatter_kernel(RouteArgs a) {
  __shared__ int s_run[kMaxExperts];
  const int lane = threadIdx.x;
  const int E = a.E, K = a.topk, S = a.T * K;
  const int nb = cdiv(a.T, kRouteBlock);
  // expert totals, and the slots of each expert in the blocks before this
  // one (all histograms of a round of 64 blocks loaded at once)
  int tot = 0, before = 0;
  if (lane < E) {
    for (int b0 = 0; b0 < nb; b0 += 64) {
      int c[64];
#pragma unroll
      for (int i = 0; i < 64; ++i) c[i] = (b0 + i < nb) ? a.blk_cnt[(b0 + i) * E + lane] : 0;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        if (b0 + i < (int)blockIdx.x) before += c[i];
        tot += c[i];
      }
    }
  }
  // expert offsets: exclusive scan of the totals (lanes >= E hold 0)
  int n_slots;
  const int off = wave_excl_scan(tot, &n_slots);
  if (lane < E) s_run[lane] = off + before;
  if (blockIdx.x == 0) {
    // E + 1 entries (E may be 64: the last one comes from lane 0)
    if (lane < E) {
      a.offsets[lane] = off;
      if (a.user_offsets) a.user_offsets[lane] = off;
    }
    if (lane == 0) {
      a.offsets[E] = n_slots;
      if (a.user_offsets) a.user_offsets[E] = n_slots;
    }
    // lookup table: one entry per (expert, column block, row tile), in that
    // nesting order; lane e writes its expert's entries from its base
    const int nrt = lane < E ? cdiv(tot, a.BM) : 0;
    int n_ent;
    const int tb = wave_excl_scan(nrt * a.n_cb, &n_ent);
    if (lane == 0) a.hdr->n_tiles = (uint32_t)min(n_ent, a.max_tiles);
    if (lane < E) a.lut_base[lane] = tb;
    for (int j = 0; j < nrt * a.n_cb; ++j) {
      const int i = tb + j;
      if (i >= a.max_tiles) break;
      const int cb = j / nrt, rt = j - cb * nrt;
      const int r0 = off + rt * a.BM;
      int4* L = reinterpret_cast<int4*>(a.lut + (size_t)i * 8);
      L[0] = make_int4(lane, r0, min(a.BM, off + tot - r0), cb);
      L[1] = make_int4(0, 0, 0, 0);
    }
  }
  __syncthreads();
  // the block's slots in index order, one wave-wide round at a time: the
  // lanes holding the same expert are found by matching its index bit by
  // bit (E <= 64: six ballots), the lower lanes among them give the rank
  const int s0 = blockIdx.x * kRouteBlock * K;
  for (int c = 0; c < K; ++c) {
    const int s = s0 + c * kRouteBlock + lane;
    const int e = s < S ? a.topk_ids[s] : -1;
    uint64_t same = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t ones = __ballot(e >= 0 && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? ones : ~ones;
    }
    if (e >= 0) {
      const int base = s_run[e];
      const int pos = base + __builtin_popcountll(same & ((1ull << lane) - 1ull));
      a.perm[pos] = s;
      a.inv[s] = pos;
    }
    __syncthreads();
    // the highest lane of each expert's group advances that expert's base
    if (e >= 0 && lane == 63 - __builtin_clzll(same)) s_run[e] += __builtin_popcountll(same);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- TopK-Reduce + ReduceScatter

// Rows [r0, r1) of the token order rotated to start at the local block
// (row t = (r + local*m) mod T): each row's 16-byte column chunks summed over
// its top-k slot rows in slot order, weight times value in fp32, rounded
// once to bf16 and stored to the partial. LOCAL rows (r < m) also finish the
// ReduceScatter on the spot: the R ranks' bf16 rows summed in ascending rank
// order in fp32 (the local one as just rounded) and rounded once into out.
// U chunks per thread in flight per round.
template <bool LOCAL, int U, int K, int NT = kThreads>
__device__ void combine_rows(const CombArgs& a, int r0, int r1) {
  const int T = a.T, N = a.N, n8 = N / 8, base = a.local * a.m;
  const int n16 = (r1 - r0) * n8;
  for (int b0 = threadIdx.x; b0 < n16; b0 += U * NT) {
    u32x4_t v[U][K];
    u32x4_t pv[U][LOCAL ? kMaxRanks : 1];
    float wt[U][K];
    int row[U], c8[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int i = b0 + q * NT;
      row[q] = -1;
      if (i >= n16) continue;
      const int rr = r0 + i / n8;
      const int t = rr + base < T ? rr + base : rr + base - T;
      row[q] = t;
      c8[q] = i - (i / n8) * n8;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        v[q][j] = gload16(a.y + ((size_t)t * K + j) * N + (size_t)c8[q] * 8);
        wt[q][j] = a.w[(size_t)t * K + j];
      }
      if constexpr (LOCAL) {
#pragma unroll
        for (int s = 0; s < kMaxRanks; ++s)
          if (s < a.R && s != a.local) pv[q][s] = gload16(a.peers[s] + (size_t)t * N + (size_t)c8[q] * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (row[q] < 0) continue;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = wt[q][0] * bf16_to_f32((v[q][0][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
#pragma unroll
      for (int j = 1; j < K; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_fmaf(wt[q][j], bf16_to_f32((v[q][j][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu), acc[e]);
      }
      const u32x4_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7])};
      gstore16(a.partial + (size_t)row[q] * N + (size_t)c8[q] * 8, o);
      if constexpr (LOCAL) {
        // rank order; the local rank's term is `o` (selected per unrolled
        // rank, so the register arrays are never indexed at run time)
        float r[8];
#pragma unroll
        for (int s = 0; s < kMaxRanks; ++s)
          if (s < a.R) {
            const u32x4_t x = (s == a.local) ? o : pv[q][s];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float f = bf16_to_f32((x[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
              r[e] = (s == 0) ? f : r[e] + f;
            }
          }
        const u32x4_t ro = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                            pack_bf16x2(r[6], r[7])};
        gstore16(a.out + (size_t)(row[q] - base) * N + (size_t)c8[q] * 8, ro);
      }
    }
  }
}

// ---------------------------------------------------------------- AG + grouped GEMM

// consume_tile_wait of a TopK-Reduce task of the MoE layer chain (wave 0):
// every grouped tile that wrote a slot row of the task's tokens (rotated
// rows [r0, r1)) must have published. A dependency (token, slot j, column
// block cb) resolves through the routing tables -- the slot's position in
// the expert-sorted order, its expert's row tile, the lookup-table entry of
// (expert, cb, row tile) -- the dynamic-dependency lookup the pages describe
// for MoE. 64 dependencies per round, one lane each, polled in parallel,
// then one acquire fence. Returns the number of dependencies.
__device__ int wait_combine_deps(const MoeArgs& a, const Common& cm, int r0, int r1, uint32_t epoch,
                                 uint32_t* seen_out) {
  const int lane = threadIdx.x & 63;
  const CombArgs& c = a.comb;
  const int K = a.topk, base = c.local * c.m, T = c.T;
  const int n = (r1 - r0) * K * a.n_cb;
  const uint64_t t0 = now_ticks();
  bool ok = true;
  uint32_t v = epoch;
  for (int b = 0; b < n; b += 64) {
    const int it = b + lane;
    if (it >= n) continue;
    const int cb = it % a.n_cb, q = it / a.n_cb, j = q % K, rr = r0 + q / K;
    const int t = rr + base < T ? rr + base : rr + base - T;
    const int slot = t * K + j;
    const int e = a.topk_ids[slot], pos = a.inv[slot];
    const int off = a.offsets[e], nrt = cdiv(a.offsets[e + 1] - off, a.BM);
    const int tile = min(a.lut_base[e] + cb * nrt + (pos - off) / a.BM, a.comb.max_tiles - 1);
    const uint32_t* f = a.tflag + tile;
    v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (v != epoch && ok) {
      if (now_ticks() - t0 > cm.timeout_ticks) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (__ballot(!ok)) {
    if (lane == 0) __hip_atomic_fetch_or(&cm.hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  *seen_out = __shfl(v, 0);
  return n;
}

template <int NT, int K>
__device__ __forceinline__ void combine_task(const CombArgs& c, bool local, int r0, int r1) {
  if (local)
    combine_rows<true, kCombineChunksLocal, K, NT>(c, r0, r1);
  else
    combine_rows<false, kCombineChunks, K, NT>(c, r0, r1);
}

template <int BM, int BN>
__global__ __launch_bounds__((Gemm<BM, BN>::NT), 1) void moe_gemm_kernel(MoeArgs args) {
  using G = Gemm<BM, BN>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[G::LDS_BYTES];
  __shared__ uint32_t s_bcast[8];
  OCG_LDS char* smem = (OCG_LDS char*)smem_raw;
  const AgPlan& p = args.plan;
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  if (threadIdx.x == 0) s_bcast[2] = __hip_atomic_load(&cm.hdr->n_tiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int n_tiles = p.mode == 2 ? 0 : (int)s_bcast[2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const size_t wstride = (size_t)p.K * p.N;

  while (p.n_copy > 0) {
    const uint32_t u = next_ticket(&cm.hdr->ticket, s_bcast);
    if ((int)u >= p.n_copy) break;
    run_copy_task<G::NT>(p, args.chunks, args.a_gathered, args.slab_cnt, args.slab_flag, (int)u, epoch, cm);
  }
  int q = (int)__builtin_amdgcn_readfirstlane(s_bcast[3]) % kXcds, tried = 0;
  uint32_t qt = 0;
  TileCtx<BM, BN> t;
  t.N = p.N;
  t.nk = p.K / BKS;
  for (;;) {
    const int v = next_tile(cm.hdr, n_tiles, &q, &tried, s_bcast, &qt, cm.xcd_remap);
    if (v < 0) break;
    const uint64_t t0 = now_ticks();
    const int32_t* L = args.lut + (size_t)v * 8;
    const int e = L[0], r0 = L[1], nrows = L[2], cb = L[3];
    uint32_t seen = 0;
    int nwait = 0;
    if (p.mode == 0 && wave == 0) {
      // consume_tile_wait on every non-local slab between the slabs of the
      // tile's first and last token (tokens ascend within an expert)
      const int tf = args.perm[r0] / args.topk, tl = args.perm[r0 + nrows - 1] / args.topk;
      const int s_lo = (tf / p.m) * p.bpr + (tf % p.m) / p.S;
      const int s_hi = (tl / p.m) * p.bpr + (tl % p.m) / p.S;
      FlagWait w(cm.timeout_ticks);
      for (int s = s_lo + lane; s <= s_hi; s += 64)
        if (s / p.bpr != p.local) w.add(&args.slab_flag[s], epoch);
      w.finish(cm, &seen);
      nwait = s_hi - s_lo + 1 - (p.local * p.bpr + p.bpr - 1 >= s_lo && p.local * p.bpr <= s_hi
                                   ? min(s_hi, p.local * p.bpr + p.bpr - 1) - max(s_lo, p.local * p.bpr) + 1
                                   : 0);
    }
    const uint64_t t1 = now_ticks();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < G::A_PER_WAVE; ++i) {
      const int rr = min(dma_row<BM, BN>(wave, i, lane), nrows - 1);
      const int tok = args.perm[r0 + rr] / args.topk;
      const int c = tok / p.m;
      t.rowp[i] = (const char*)((c == p.local) ? args.chunks[c] + (size_t)(tok - c * p.m) * p.K
                                               : args.a_gathered + (size_t)tok * p.K);
    }
    t.brs = make_rsrc(args.w + (size_t)e * wstride, (uint32_t)(wstride * 2));
    const int n0 = cb * BN;
    t.n0 = n0;
    AccTile<BM, BN> acc;
    mainloop<BM, BN>(smem, t, acc);
    stage_c<BM, BN>(smem, acc);
    // local scatter: row rr of the tile is token-slot perm[r0 + rr]
    if (args.combine) {
      // read by this launch's TopK-Reduce tasks: agent-coherent stores, then
      // produce_tile_notify
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(args.out, (uint32_t)((size_t)args.comb.T * args.topk * p.N * 2));
      for_each_c_chunk<BM, BN>(smem, [&](int rr, int col, u32x4_t val) {
        if (rr < nrows && n0 + col < p.N) {
          const int slot = args.perm[r0 + rr];
          store16_agent(ors, (uint32_t)(((size_t)slot * p.N + n0 + col) * 2), val);
        }
      });
      drain_stores();
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(&args.tflag[v], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      for_each_c_chunk<BM, BN>(smem, [&](int rr, int col, u32x4_t val) {
        if (rr < nrows && n0 + col < p.N) {
          const int slot = args.perm[r0 + rr];
          gstore16_out(args.out + (size_t)slot * p.N + n0 + col, val);
        }
      });
    }
    trace_task(cm, (uint32_t)(p.n_copy + v), 4, e, r0, nrows, cb | ((uint32_t)nwait << 16), epoch, t0, t1, seen,
               ((uint32_t)q << 16) | qt);
  }
  // The layer chain's TopK-Reduce + ReduceScatter tasks, once every tile has
  // been claimed: local block first; each waits on the tiles that wrote its
  // tokens' slot rows (trace slot n_copy + #tiles + task).
  if (args.combine) {
    const CombArgs& c = args.comb;
    for (;;) {
      const uint32_t u = next_ticket(&cm.hdr->side_ticket, s_bcast);
      if ((int)u >= c.n_comb) break;
      const uint64_t t0 = now_ticks();
      const bool local = (int)u < c.n_lt;
      const int r0 = local ? (int)u * c.CRL : c.m + ((int)u - c.n_lt) * c.CR;
      const int r1 = local ? min(r0 + c.CRL, c.m) : min(r0 + c.CR, c.T);
      uint32_t seen = 0;
      int nd = 0;
      if (wave == 0) nd = wait_combine_deps(args, cm, r0, r1, epoch, &seen);
      const uint64_t t1 = now_ticks();
      __syncthreads();
      switch (args.topk) {
        case 1: combine_task<G::NT, 1>(c, local, r0, r1); break;
        case 2: combine_task<G::NT, 2>(c, local, r0, r1); break;
        case 3: combine_task<G::NT, 3>(c, local, r0, r1); break;
        default: combine_task<G::NT, 4>(c, local, r0, r1); break;
      }
      trace_task(cm, (uint32_t)(p.n_copy + n_tiles) + u, 6, (uint32_t)r0, (uint32_t)r1,
                 local ? (uint32_t)(r1 - r0) : 0u, (uint32_t)nd, epoch, t0, t1, seen, 0);
    }
  }
  finish(cm.hdr, epoch);
}

// Tasks: first the local block's rows (rotated rows [0, m)) in tasks of CRL
// rows, then the others in tasks of CR rows; a local row moves (topk + R + 1)
// rows of data against topk + 1 for the others, hence the smaller tasks. The
// local rows' reduce needs only the peers' rows (inputs of the call) and the
// row's own combined value, so no task waits on another, and the tasks are
// dealt round-robin (task u to workgroup u mod grid): the tasks are short
// and alike, and a shared ticket counter became the bottleneck at this rate.
template <int K>
__global__ __launch_bounds__(kThreads) void moe_combine_rs_kernel(CombArgs args) {
  __shared__ uint32_t s_bcast[8];
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  for (uint32_t u = blockIdx.x; (int)u < args.n_comb; u += gridDim.x) {
    const uint64_t t0 = now_ticks();
    const bool local = (int)u < args.n_lt;
    const int r0 = local ? (int)u * args.CRL : args.m + ((int)u - args.n_lt) * args.CR;
    const int r1 = local ? min(r0 + args.CRL, args.m) : min(r0 + args.CR, args.T);
    if (local)
      combine_rows<true, kCombineChunksLocal, K>(args, r0, r1);
    else
      combine_rows<false, kCombineChunks, K>(args, r0, r1);
    trace_task(cm, u, 6, (uint32_t)r0, (uint32_t)r1, local ? (uint32_t)(r1 - r0) : 0u, 0, epoch, t0, t0, 0, 0);
  }
  finish(cm.hdr, epoch);
}

// ---------------------------------------------------------------- fill

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v, int release) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (size_t)gridDim.x * blockDim.x) {
    if (release)
      __hip_atomic_store(p + i, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    else
      p[i] = v;
  }
}

// ---------------------------------------------------------------- no-allocation scratch

// Workspace of ocg_ag_gemm_noalloc, the entry point for callers that cannot
// allocate: a file-scope device array, one copy per GPU the library runs on,
// held until the process ends. Every call on a GPU shares that GPU's copy
// (the header's counters return to zero at the end of each call and the
// flags carry the call's epoch, so it is cleared once, at set-up).
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, null until set up
}

// Set-up, from ocg_create with `device` current: look up the array's device
// address (in host code its name is only a host-side stand-in) and clear the
// array, once per device.
hipError_t noalloc_scratch_setup(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    e = launch_fill_u32((uint32_t*)ptr, kNoAllocScratchBytes / 4, 0u, 0, nullptr);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

// ---------------------------------------------------------------- launchers

static_assert(gemm_waves<256, 224>() == 4 && gemm_waves<128, 224>() == 4 && gemm_waves<128, 256>() == 4 &&
                  gemm_waves<128, 128>() == 4 && gemm_waves<256, 256>() == 4 && gemm_waves<288, 224>() == 4 &&
                  gemm_waves<320, 224>() == 8,
              "tile_waves (host planning) must match the engine");

template <int BM, int BN>
static hipError_t ag_launch(const AgArgs& a, int grid, hipStream_t s) {
  if (a.plan.sk == 2)
    hipLaunchKernelGGL((ag_gemm_kernel<BM, BN, true>), dim3(grid), dim3(Gemm<BM, BN>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((ag_gemm_kernel<BM, BN, false>), dim3(grid), dim3(Gemm<BM, BN>::NT), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t rs_launch(const RsArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_rs_kernel<BM, BN>), dim3(grid), dim3(Gemm<BM, BN>::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ag_gemm(const AgArgs& a, int tile, int grid, hipStream_t s) {
  switch (tile) {
    case OCG_TILE_256x224: return ag_launch<256, 224>(a, grid, s);
    case OCG_TILE_128x224: return ag_launch<128, 224>(a, grid, s);
    case OCG_TILE_128x256: return ag_launch<128, 256>(a, grid, s);
    case OCG_TILE_128x128: return ag_launch<128, 128>(a, grid, s);
    case OCG_TILE_256x256: return ag_launch<256, 256>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ag_side_copy(const AgArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ag_side_copy_kernel, dim3(grid), dim3(kSideThreads), 0, s, a);
  return hipGetLastError();
}

template <class K>
static bool attrs(K kern, int* vgprs, int* lds) {
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern)) != hipSuccess) return false;
  *vgprs = fa.numRegs;
  *lds = (int)fa.sharedSizeBytes;
  return true;
}

// op < 0: the side producer kernel; else the AG-GEMM kernel of `tile`.
bool kernel_resources(int op, int tile, int* vgprs, int* lds) {
  if (op < 0) return attrs(ag_side_copy_kernel, vgprs, lds);
  switch (tile) {
    case OCG_TILE_256x224: return attrs(ag_gemm_kernel<256, 224, false>, vgprs, lds);
    case OCG_TILE_128x224: return attrs(ag_gemm_kernel<128, 224, false>, vgprs, lds);
    case OCG_TILE_128x256: return attrs(ag_gemm_kernel<128, 256, false>, vgprs, lds);
    case OCG_TILE_128x128: return attrs(ag_gemm_kernel<128, 128, false>, vgprs, lds);
    case OCG_TILE_256x256: return attrs(ag_gemm_kernel<256, 256, false>, vgprs, lds);
  }
  return false;
}

hipError_t launch_gemm_rs(const RsArgs& a, int tile, int grid, hipStream_t s) {
  switch (tile) {
    case OCG_TILE_256x224: return rs_launch<256, 224>(a, grid, s);
    case OCG_TILE_128x224: return rs_launch<128, 224>(a, grid, s);
    case OCG_TILE_128x256: return rs_launch<128, 256>(a, grid, s);
    case OCG_TILE_128x128: return rs_launch<128, 128>(a, grid, s);
    case OCG_TILE_256x256: return rs_launch<256, 256>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_moe(const RouteArgs& r, const MoeArgs& a, int tile, int grid, hipStream_t s) {
  const int nb = cdiv(r.T, kRouteBlock);
  hipLaunchKernelGGL(moe_topk_kernel, dim3(nb), dim3(64 * kRouteWaves), 0, s, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nb), dim3(kRouteBlock), 0, s, r);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (tile) {
    case OCG_TILE_128x224: hipLaunchKernelGGL((moe_gemm_kernel<128, 224>), dim3(grid), dim3(Gemm<128, 224>::NT), 0, s, a); break;
    case OCG_TILE_256x224: hipLaunchKernelGGL((moe_gemm_kernel<256, 224>), dim3(grid), dim3(Gemm<256, 224>::NT), 0, s, a); break;
    case OCG_TILE_288x224: hipLaunchKernelGGL((moe_gemm_kernel<288, 224>), dim3(grid), dim3(Gemm<288, 224>::NT), 0, s, a); break;
    case OCG_TILE_320x224: hipLaunchKernelGGL((moe_gemm_kernel<320, 224>), dim3(grid), dim3(Gemm<320, 224>::NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One kernel per slot count, so registers are sized for exactly topk rows.
hipError_t launch_moe_combine_rs(const CombArgs& a, int grid, hipStream_t s) {
  switch (a.topk) {
    case 1: hipLaunchKernelGGL((moe_combine_rs_kernel<1>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((moe_combine_rs_kernel<2>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((moe_combine_rs_kernel<3>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((moe_combine_rs_kernel<4>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, int release, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v, release);
  return hipGetLastError();
}

template <class K>
static int occ(K kern, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

int resident_per_cu(int op, int tile, int sk) {
  if (op == OCG_OP_AG_GROUPED_GEMM) {
    switch (tile) {
      case OCG_TILE_128x224: return occ(moe_gemm_kernel<128, 224>, Gemm<128, 224>::NT);
      case OCG_TILE_256x224: return occ(moe_gemm_kernel<256, 224>, Gemm<256, 224>::NT);
      case OCG_TILE_288x224: return occ(moe_gemm_kernel<288, 224>, Gemm<288, 224>::NT);
      case OCG_TILE_320x224: return occ(moe_gemm_kernel<320, 224>, Gemm<320, 224>::NT);
    }
    return 1;
  }
  if (op == OCG_OP_AG_GEMM) {
    switch (tile) {
      case OCG_TILE_256x224: return sk == 2 ? occ(ag_gemm_kernel<256, 224, true>, Gemm<256, 224>::NT)
                                           : occ(ag_gemm_kernel<256, 224, false>, Gemm<256, 224>::NT);
      case OCG_TILE_128x224: return sk == 2 ? occ(ag_gemm_kernel<128, 224, true>, Gemm<128, 224>::NT)
                                           : occ(ag_gemm_kernel<128, 224, false>, Gemm<128, 224>::NT);
      case OCG_TILE_128x256: return sk == 2 ? occ(ag_gemm_kernel<128, 256, true>, Gemm<128, 256>::NT)
                                           : occ(ag_gemm_kernel<128, 256, false>, Gemm<128, 256>::NT);
      case OCG_TILE_128x128: return sk == 2 ? occ(ag_gemm_kernel<128, 128, true>, Gemm<128, 128>::NT)
                                           : occ(ag_gemm_kernel<128, 128, false>, Gemm<128, 128>::NT);
      case OCG_TILE_256x256: return sk == 2 ? occ(ag_gemm_kernel<256, 256, true>, Gemm<256, 256>::NT)
                                           : occ(ag_gemm_kernel<256, 256, false>, Gemm<256, 256>::NT);
    }
  } else {
    switch (tile) {
      case OCG_TILE_256x224: return occ(gemm_rs_kernel<256, 224>, Gemm<256, 224>::NT);
      case OCG_TILE_128x224: return occ(gemm_rs_kernel<128, 224>, Gemm<128, 224>::NT);
      case OCG_TILE_128x256: return occ(gemm_rs_kernel<128, 256>, Gemm<128, 256>::NT);
      case OCG_TILE_128x128: return occ(gemm_rs_kernel<128, 128>, Gemm<128, 128>::NT);
      case OCG_TILE_256x256: return occ(gemm_rs_kernel<256, 256>, Gemm<256, 256>::NT);
    }
  }
  return 1;
}

}  // namespace ocg
