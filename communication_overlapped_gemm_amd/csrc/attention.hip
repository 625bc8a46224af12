// AllGather-KV attention on gfx950: the gather of the keys and values of R
// context-parallel ranks overlapped with the attention of the local queries
// over the gathered sequence ("TileLink: Generating Efficient
// Compute-Communication Overlapping Kernels using Tile-Centric Primitives",
// MLSys 2025 talk summary, section "Experimental Setup & Results": the
// AllGather-KV attention, overlapped with the attention computation itself).
//
// One persistent kernel. Workgroups first take copy tasks (pull a piece of a
// peer's key or value chunk into the gathered buffers, publish the slab flag
// once its key and value pieces have landed), then attention tiles from the
// XCD queues. A tile holds 256 query rows (query, head) that share one kv
// head; its 8 waves (two per SIMD) take 32 rows each and stream the keys and
// values in blocks of 64 through a 4-slot LDS ring filled by direct-to-LDS
// loads, starting with the local chunk (read from the local shard, never
// waited on); before its first load of a peer chunk each wave waits on that
// chunk's slab flags.
//
// Per wave and key block (flash-attention style online softmax, fp32):
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, A = key rows from LDS
//                    (16-byte reads), B = the wave's query fragments, held in
//                    registers for the whole tile;
//   softmax          lane (l & 15) of every 16-lane row owns one query of a
//                    16-query column block and 4 of its keys per 16-key tile,
//                    so a row maximum is an in-lane maximum plus two lane
//                    swaps (v_permlane16/32_swap); the exponentials are taken
//                    against a reference that only moves when a block's
//                    maximum passes it by 2^8, so the accumulators are
//                    rarely rescaled;
//   O^T += V^T P^T   A = value columns from LDS with the transposing read
//                    ds_read_b64_tr_b16, B = the probabilities converted to
//                    bf16 in registers. Each lane's 8 probabilities of a
//                    32-key step are keys {4q..4q+3, 16+4q..16+4q+3}
//                    (q = lane >> 4), the order the S^T accumulators leave
//                    them in; the value reads fetch the same keys, so the
//                    contraction pairs them up;
//   row sums         one more MFMA per 32-key step against a 0/1 key
//                    validity operand, so keys past a chunk's end (whose
//                    value rows load as zeros) drop out without masking the
//                    scores, and no VALU adds are spent on the sums.
// On this chip the MFMA and VALU work of a SIMD mostly add up rather than
// overlap (measured), so the loop is built to spend few VALU instructions per
// score: an FMA, an exponential, half a conversion and part of a maximum.
// The output accumulators hold O^T: lane (q, j) has O[query j][d = 16t + 4q
// .. +3] of each 16x16 block; the epilogue divides by the row sums and
// stores 8-byte pieces.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.h"
#include "ocg_internal.h"
#include "sync.h"

namespace ocg {
namespace {

constexpr int kWaves = 8;                   // waves per workgroup (two per SIMD)
constexpr int kAThreads = 64 * kWaves;
constexpr int kD = kAttnD;                  // head dimension (128)
constexpr int kKB = kAttnKB;                // keys per block (64)
constexpr int kSlots = 4;                   // LDS ring slots
constexpr int kRowBytes = kD * 2;           // one head's key or value row (256 B)
constexpr int kPart = kKB * kRowBytes;      // keys (or values) of one block: 16 KiB
constexpr int kStage = 2 * kPart;           // keys, then values
constexpr int kLoads = kPart / 1024 / kWaves;   // 1 KiB loads per wave per tensor per block
constexpr int kNdma = 2 * kLoads;           // loads per wave per block
constexpr int kRowsW = kAttnRows / kWaves;  // query rows per wave
constexpr int kQTiles = kRowsW / 16;        // 16-row query blocks per wave
constexpr int kDSteps = kD / 32;            // MFMA k steps over the head dimension
constexpr int kDTiles = kD / 16;            // 16-column blocks of the output
constexpr float kLazy = 8.0f;               // reference lag of the online softmax (log2 units)

static_assert(kSlots * kStage <= 160 * 1024 - 64, "ring fits the LDS");
static_assert(kKB == 64 && kD == 128, "fragment maps below assume 64-key blocks of 128-wide heads");

// LDS slot layout: keys [64][256 B] then values [64][256 B]. The 16-byte
// chunk c of key row r sits at chunk position c ^ (r & 15): the 16 lanes of a
// key-fragment read (16 rows, one chunk) hit 16 distinct positions. The
// 32-byte chunk pair c2 of value row r sits at pair position c2 ^ (r & 7):
// a transposing read touches 4 rows x 32 bytes per 16 lanes, and rows
// 8n..8n+7 land on 8 distinct pairs (all 64 banks for 32 lanes).
__device__ __forceinline__ int key_src_chunk(int pos, int r) { return pos ^ (r & 15); }
__device__ __forceinline__ int val_src_chunk(int pos, int r) { return (((pos >> 1) ^ (r & 7)) << 1) | (pos & 1); }

__device__ __forceinline__ float swap_max16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// One copy task: piece u >> 1 of the AG copy order of tensor u & 1.
__device__ void run_kv_copy(const AttnArgs& a, int u, uint32_t epoch) {
  const AgPlan& p = a.plan.cp;
  const uint64_t t0 = now_ticks();
  const int tensor = u & 1;
  const CopyDesc d = copy_desc(p, u >> 1);
  copy_delay(a.cm.copy_delay);   // test hook: publish late
  const uint16_t* src = (tensor ? a.v_chunks[d.chunk] : a.k_chunks[d.chunk]) + (size_t)(d.row0 - d.chunk * p.m) * p.K;
  uint16_t* dst = (tensor ? a.v_gathered : a.k_gathered) + (size_t)d.row0 * p.K;
  copy_granules<kAThreads>(src, dst, (uint32_t)((size_t)(d.row1 - d.row0) * p.K / 8));
  const int target = 2 * slab_target(p.m, p.S, p.CT, p.bpr, d.slab);
  const bool pub = publish_slab(a.slab_cnt, a.slab_flag, d.slab, target, epoch, a.cm);
  trace_task(a.cm, (uint32_t)u, 1, d.chunk, (uint32_t)d.piece | ((uint32_t)tensor << 16), d.slab, pub ? 1u : 0u,
             epoch, t0, now_ticks(), 0, 0);
}

// Per-lane constants of a tile's block loads: load ii of this wave fills
// rows 4*i .. 4*i+3 (i = wave + 4*ii) of the slot's key and value parts;
// lane L takes row 4*i + L/16, LDS chunk position L & 15, whose source chunk
// is given by the swizzles above.
struct BlockLoads {
  uint32_t kofs[kLoads], vofs[kLoads];   // byte offset of the lane's source chunk from the block's first row
  uint32_t koff[kLoads], voff[kLoads];   // ... within its head row
  int row[kLoads];                       // row within the block
};

// Direct-to-LDS 16-byte load of buffer bytes soff + voff (the lane's
// offset; out-of-range voff reads zeros, soff is not range-checked).
__device__ __forceinline__ void dma_buffer_so(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

struct TileState {
  bf16x8_t qf[kQTiles][kDSteps];   // query fragments: row (lane & 15) of block qt, d = 32u + 8(lane >> 4) ..
  f32x4_t o[kDTiles][kQTiles];     // O^T accumulators
  f32x4_t l[kQTiles];              // row sums, from an MFMA against the key validity (all 4 entries equal)
  float mrun[kQTiles];             // softmax reference of the query (log2 units)
};

// Key block j: issue this wave's 8 loads into `slot` (LDS byte address).
// Key rows past the chunk's end re-read its last row (a duplicate score,
// harmless to the running maximum); value rows past it read zeros (buffer
// loads bounded to the chunk's rows of this head), and the row sums leave
// those keys out, so they add nothing.
__device__ __forceinline__ void issue_block(const AttnArgs& a, const BlockLoads& bl, int g, int j, uint32_t slot) {
  const AttnPlan& p = a.plan;
  const int c = attn_block_chunk(p, j);
  const int m = p.cp.m;
  const int key0 = (j % p.nbc) * kKB;
  const uint32_t row_bytes = (uint32_t)p.Hkv * kRowBytes;
  const uint16_t* kb;
  const uint16_t* vb;
  if (c == p.cp.local) {
    kb = a.k_chunks[c] + (size_t)g * kD;
    vb = a.v_chunks[c] + (size_t)g * kD;
  } else {
    kb = a.k_gathered + (size_t)c * m * p.Hkv * kD + (size_t)g * kD;
    vb = a.v_gathered + (size_t)c * m * p.Hkv * kD + (size_t)g * kD;
  }
  const uint32_t bound = (uint32_t)(m - 1) * row_bytes + kRowBytes;   // the chunk's rows of head g
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb, bound);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vb, bound);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (key0 + kKB <= m) {
    // every row inside the chunk: the block's first row as the scalar offset
    const uint32_t so = (uint32_t)key0 * row_bytes;
#pragma unroll
    for (int ii = 0; ii < kLoads; ++ii) {
      const int i = wave + kWaves * ii;
      dma_buffer_so(slot + i * 1024, krs, bl.kofs[ii], so);
      dma_buffer_so(slot + kPart + i * 1024, vrs, bl.vofs[ii], so);
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < kLoads; ++ii) {
      const int i = wave + kWaves * ii;
      const int key = key0 + bl.row[ii];
      dma_buffer_so(slot + i * 1024, krs, (uint32_t)min(key, m - 1) * row_bytes + bl.koff[ii], 0u);
      dma_buffer_so(slot + kPart + i * 1024, vrs, (uint32_t)key * row_bytes + bl.voff[ii], 0u);
    }
  }
}

// Wait (this wave) for every slab flag of every peer chunk, lane-parallel;
// returns the flag count. Called once per wave, before its first load of a
// peer chunk: the acquire that ends a wait drains the wave's loads in flight
// and invalidates the XCD L2's non-coherent lines (keys and values the
// head's other tiles reuse), so one wait for all peers replaces one per peer
// chunk: 536.3 -> 519.3 us per fused launch at the 16K share (one process,
// alternating; attention alone 494.0 / 489.0). The copies have landed long
// before a tile leaves its local chunk, so the single wait costs no time.
__device__ __forceinline__ int wait_peers(const AttnArgs& a, uint32_t epoch, uint32_t* seen) {
  const AgPlan& p = a.plan.cp;
  FlagWait w(a.cm.timeout_ticks);
  const int n = p.R * p.bpr;
  for (int s = threadIdx.x & 63; s < n; s += 64)
    if (s / p.bpr != p.local) w.add(&a.slab_flag[s], epoch);
  w.finish(a.cm, seen);
  return (p.R - 1) * p.bpr;
}

// A half step covers 32 keys (key tiles 2h, 2h+1 of a block, one MFMA k
// step of the value product). Scores of a half: s[tile][qt] = K_tile Q_qt^T.
constexpr int kHalfTiles = 2;

__device__ __forceinline__ void read_key_frags(OCG_LDS const char* st, const uint32_t (&kfa)[kDSteps], int t,
                                               bf16x8_t (&kf)[kDSteps]) {
#pragma unroll
  for (int u = 0; u < kDSteps; ++u) kf[u] = *(OCG_LDS const bf16x8_t*)(st + t * 16 * kRowBytes + kfa[u]);
}

__device__ __forceinline__ void tile_scores(const TileState& ts, const bf16x8_t (&kf)[kDSteps],
                                            f32x4_t (&sn)[kQTiles]) {
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int qt = 0; qt < kQTiles; ++qt) {
    sn[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], ts.qf[qt][0], zero, 0, 0, 0);
#pragma unroll
    for (int u = 1; u < kDSteps; ++u) sn[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u], ts.qf[qt][u], sn[qt], 0, 0, 0);
  }
}

// Exponentials of query block qt of a half's scores against the reference,
// as the bf16 MFMA B operand of the half's 32 keys.
__device__ __forceinline__ bf16x8_t half_probs(const TileState& ts, const f32x4_t (&s)[kHalfTiles][kQTiles], int qt,
                                               float scale) {
  const float mref = ts.mrun[qt];
  float p[kHalfTiles][4];
#pragma unroll
  for (int t = 0; t < kHalfTiles; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) p[t][i] = __builtin_amdgcn_exp2f(fmaf(s[t][qt][i], scale, -mref));
  return bf16x8_t{(__bf16)p[0][0], (__bf16)p[0][1], (__bf16)p[0][2], (__bf16)p[0][3],
                  (__bf16)p[1][0], (__bf16)p[1][1], (__bf16)p[1][2], (__bf16)p[1][3]};
}

// In-lane maxima of a half's scores, one per query block (the lane's 8 keys).
__device__ __forceinline__ void half_lane_max(const f32x4_t (&s)[kHalfTiles][kQTiles], float (&mx)[kQTiles]) {
#pragma unroll
  for (int qt = 0; qt < kQTiles; ++qt)
    mx[qt] = fmaxf(fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3])),
                   fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3])));
}

// Row maximum over the 4 lanes sharing a query, scaled to log2 units.
__device__ __forceinline__ float row_max(float v, float scale) { return swap_max32(swap_max16(v)) * scale; }

// Online softmax with a lazily moved reference: the exponentials are taken
// against mrun, which moves (rescaling the output accumulators and the row
// sums) only when a half's maximum exceeds it by more than kLazy (log2
// units), so every p <= 2^kLazy; the offset cancels in the final division.
__device__ __forceinline__ void lazy_rescale(TileState& ts, const float (&mx)[kQTiles]) {
  bool up = false;
#pragma unroll
  for (int qt = 0; qt < kQTiles; ++qt) up |= mx[qt] > ts.mrun[qt] + kLazy;
  if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
    for (int qt = 0; qt < kQTiles; ++qt) {
      const float mnew = mx[qt] > ts.mrun[qt] + kLazy ? mx[qt] : ts.mrun[qt];
      const float alpha = __builtin_amdgcn_exp2f(ts.mrun[qt] - mnew);
      ts.mrun[qt] = mnew;
      ts.l[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) ts.o[dt][qt] *= alpha;
    }
  }
}

// Value fragment of output column block dt, 32-key step sp.
__device__ __forceinline__ bf16x8_t read_val_frag(OCG_LDS const char* sv, uint32_t vfa, int vx, int dt, int sp) {
  OCG_LDS const char* pa = sv + vfa + sp * 32 * kRowBytes + ((dt ^ vx) << 5);
  bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((OCG_LDS bf16x4_t*)pa);
  bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((OCG_LDS bf16x4_t*)(pa + 16 * kRowBytes));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The lane's 8 key slots of a 32-key step as the MFMA A operand of the row
// sums: 1 for keys below `valid` (counted from the step's first key), else 0.
// Slot s of lane (q, j) is key 4q + s (s < 4) or 16 + 4q + s - 4.
__device__ __forceinline__ bf16x8_t key_validity(int valid) {
  const int qg = (threadIdx.x & 63) >> 4;
  bf16x8_t v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = (__bf16)((s < 4 ? 4 * qg + s : 16 + 4 * qg + s - 4) < valid ? 1.0f : 0.0f);
  return v;
}

// Instruction classes of sched_group_barrier masks.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008;

struct StepCtx {
  OCG_LDS char* smem;
  uint32_t kfa[kDSteps];
  uint32_t vfa;
  int vx;
  float scale;
};

// One attention tile v: kv head g, query rows [256 rb, 256 rb + 256).
__device__ void attention_tile(const AttnArgs& a, OCG_LDS char* smem, int v, uint32_t epoch, uint32_t queue) {
  const AttnPlan& p = a.plan;
  const AgPlan& cp = p.cp;
  const uint64_t t0 = now_ticks();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int qg = lane >> 4, qj = lane & 15;
  const int g = v / p.n_rb, rb = v - g * p.n_rb;
  const int nrows = p.G * cp.m;

  // query rows of this lane (one per 16-row block) and their element offsets
  TileState ts;
  size_t qoff[kQTiles];
  bool qok[kQTiles];
#pragma unroll
  for (int qt = 0; qt < kQTiles; ++qt) {
    const int r = rb * kAttnRows + wave * kRowsW + qt * 16 + qj;
    qok[qt] = r < nrows;
    const int rc = min(r, nrows - 1);
    const int i = rc / p.G, h = g * p.G + (rc - (rc / p.G) * p.G);
    qoff[qt] = ((size_t)i * p.Hq + h) * kD;
#pragma unroll
    for (int u = 0; u < kDSteps; ++u) ts.qf[qt][u] = *(const bf16x8_t*)(a.q + qoff[qt] + 32 * u + 8 * qg);
    ts.mrun[qt] = -INFINITY;
    ts.l[qt] = f32x4_t{};
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) ts.o[dt][qt] = f32x4_t{};
  }
  // The query loads are the only loads the compiler tracks; waiting for them
  // here (as a builtin, so its wait insertion knows) keeps it from adding a
  // whole-queue wait inside the key loop, whose direct-to-LDS loads it does
  // not see.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt open
  BlockLoads bl;
#pragma unroll
  for (int ii = 0; ii < kLoads; ++ii) {
    const int r = 4 * (wave + kWaves * ii) + (lane >> 4);
    bl.row[ii] = r;
    bl.koff[ii] = (uint32_t)key_src_chunk(lane & 15, r) * 16u;
    bl.voff[ii] = (uint32_t)val_src_chunk(lane & 15, r) * 16u;
    bl.kofs[ii] = (uint32_t)r * (uint32_t)p.Hkv * kRowBytes + bl.koff[ii];
    bl.vofs[ii] = (uint32_t)r * (uint32_t)p.Hkv * kRowBytes + bl.voff[ii];
  }
  // fragment read offsets within a slot
  uint32_t kfa[kDSteps];
#pragma unroll
  for (int u = 0; u < kDSteps; ++u) kfa[u] = (uint32_t)(qj * kRowBytes + (((4 * u + qg) ^ qj) << 4));
  const int vrow = 4 * qg + (qj >> 2);           // value row of the low transposing read (+32 per k step)
  const uint32_t vfa = (uint32_t)(vrow * kRowBytes + (((qj >> 1) & 1) << 4) + ((qj & 1) << 3));
  const int vx = vrow & 7;                       // pair swizzle of that row (same for +16, +32)

  const uint32_t base = lds_u32(smem);
  const int nblk = cp.R * p.nbc;
  const bool fused = cp.mode == 0;
  int nwait = 0;
  uint32_t seen = 0;
  uint64_t t_ready = t0;
  // Block j's loads, preceded, before the first block of the first peer
  // chunk, by the wait on every peer chunk's flags. Past the end the last
  // block is loaded again into the free slot (never used), so every step
  // issues kNdma loads.
  bool waited = false;
  auto issue = [&](int j) {
    const uint32_t slot = base + (uint32_t)(j % kSlots) * kStage;
    const int jj = j < nblk ? j : nblk - 1;
    if (fused && !waited && j < nblk && jj % p.nbc == 0 && attn_block_chunk(p, jj) != cp.local) {
      nwait = wait_peers(a, epoch, &seen);
      waited = true;
      t_ready = now_ticks();
    }
    issue_block(a, bl, g, jj, slot);
  };
  auto valid_keys = [&](int j) { return min(kKB, cp.m - (j % p.nbc) * kKB); };
  StepCtx c;
  c.smem = smem;
#pragma unroll
  for (int u = 0; u < kDSteps; ++u) c.kfa[u] = kfa[u];
  c.vfa = vfa;
  c.vx = vx;
  c.scale = a.scale_log2;
  bf16x8_t all_valid;
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) all_valid[s8] = (__bf16)1.0f;
#pragma unroll
  for (int j = 0; j < kSlots - 1; ++j) issue(j);
  // One block per step. The scores of the second 32-key half are computed
  // under the maxima of the first; the value product of the first half runs
  // under the exponentials of the second (the scheduling groups interleave
  // them: an MFMA only overlaps VALU work of its own wave that follows it in
  // program order).
  for (int k = 0; k < nblk; ++k) {
    vm_wait<(kSlots - 2) * kNdma>();   // block k has landed (this wave's loads)
    lds_barrier();                     // ... everyone's; slot (k-1) % kSlots is free
    issue(k + kSlots - 1);
    OCG_LDS const char* st = smem + (k % kSlots) * kStage;
    OCG_LDS const char* sv = st + kPart;
    f32x4_t sh[2][kHalfTiles][kQTiles];
    float m0[kQTiles], m1[kQTiles];
    bf16x8_t vf[kDTiles];
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t) {
      bf16x8_t kf[kDSteps];
      read_key_frags(st, kfa, t, kf);
      tile_scores(ts, kf, sh[0][t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // second half's scores || first half's maxima; the first half's value
    // fragments are read meanwhile
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t) {
      bf16x8_t kf[kDSteps];
      read_key_frags(st, kfa, 2 + t, kf);
      tile_scores(ts, kf, sh[1][t]);
    }
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) vf[dt] = read_val_frag(sv, vfa, vx, dt, 0);
    half_lane_max(sh[0], m0);
#pragma unroll
    for (int i = 0; i < kHalfTiles * kQTiles * kDSteps; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    half_lane_max(sh[1], m1);
#pragma unroll
    for (int qt = 0; qt < kQTiles; ++qt) m0[qt] = row_max(fmaxf(m0[qt], m1[qt]), c.scale);
    lazy_rescale(ts, m0);
    const int vk = valid_keys(k);
    bf16x8_t vv0 = all_valid, vv1 = all_valid;
    if (vk < kKB) {
      vv0 = key_validity(vk);
      vv1 = key_validity(vk - 32);
    }
    bf16x8_t pf0[kQTiles], pf1[kQTiles];
#pragma unroll
    for (int qt = 0; qt < kQTiles; ++qt) pf0[qt] = half_probs(ts, sh[0], qt, c.scale);
    __builtin_amdgcn_sched_barrier(0);
    // first half's value product || second half's exponentials
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQTiles; ++qt)
        ts.o[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf0[qt], ts.o[dt][qt], 0, 0, 0);
#pragma unroll
    for (int qt = 0; qt < kQTiles; ++qt) {
      ts.l[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv0, pf0[qt], ts.l[qt], 0, 0, 0);
      pf1[qt] = half_probs(ts, sh[1], qt, c.scale);
    }
#pragma unroll
    for (int i = 0; i < kDTiles * kQTiles + kQTiles; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) vf[dt] = read_val_frag(sv, vfa, vx, dt, 1);
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQTiles; ++qt)
        ts.o[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf1[qt], ts.o[dt][qt], 0, 0, 0);
#pragma unroll
    for (int qt = 0; qt < kQTiles; ++qt)
      ts.l[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv1, pf1[qt], ts.l[qt], 0, 0, 0);
  }
  vm_wait<0>();
  lds_barrier();

  // epilogue: O / l, rounded to bf16, 8-byte stores
#pragma unroll
  for (int qt = 0; qt < kQTiles; ++qt) {
    const float inv = 1.0f / ts.l[qt][0];
    if (!qok[qt]) continue;
    uint16_t* orow = a.out + qoff[qt] + 4 * qg;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const f32x4_t x = ts.o[dt][qt] * inv;
      u32x2_t w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *(u32x2_t*)(orow + 16 * dt) = w;
    }
  }
  trace_task(a.cm, (uint32_t)(p.n_copy + v), 7, (uint32_t)g, (uint32_t)rb, (uint32_t)nwait, 0, epoch, t0, t_ready,
             seen, queue);
}

}  // namespace

__global__ __launch_bounds__(kAThreads, 1) void ag_attention_kernel(AttnArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kSlots * kStage];
  __shared__ uint32_t s_bcast[8];
  OCG_LDS char* smem = (OCG_LDS char*)smem_raw;
  const AttnPlan& p = args.plan;
  const Common& cm = args.cm;
  const uint32_t epoch = read_epoch(cm.hdr, s_bcast);
  while (p.n_copy > 0) {
    const uint32_t u = next_ticket(&cm.hdr->ticket, s_bcast);
    if ((int)u >= p.n_copy) break;
    run_kv_copy(args, (int)u, epoch);
  }
  int q = (int)s_bcast[3] % kXcds, tried = 0;
  uint32_t qt = 0;
  for (;;) {
    const int v = next_tile(cm.hdr, p.n_tiles, &q, &tried, s_bcast, &qt, cm.xcd_remap);
    if (v < 0) break;
    attention_tile(args, smem, v, epoch, ((uint32_t)q << 16) | qt);
  }
  finish(cm.hdr, epoch);
}

hipError_t launch_ag_attention(const AttnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ag_attention_kernel, dim3(grid), dim3(kAThreads), 0, s, a);
  return hipGetLastError();
}

int resident_attention() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ag_attention_kernel, kAThreads, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

}  // namespace ocg
