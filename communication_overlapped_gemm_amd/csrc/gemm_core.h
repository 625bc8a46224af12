// bf16 MFMA tile engine for gfx950 (one workgroup = 4 or 8 waves, one tile).
//
// Tile BM x BN, K consumed in stages of 32. The NW waves (4 or 8, see
// gemm_waves) form an NW/2 x 2 grid: wave w = 2*wm + wn owns rows
// [wm*WM, +WM) (WM = 2*BM/NW) and columns [wn*BN/2, +BN/2),
// computed with v_mfma_f32_16x16x32_bf16 (one 16x16 accumulator per (16-row,
// 16-col) block; one MFMA covers the whole 32-deep stage). Compared with four
// waves stacked along M, every wave reads half of B instead of all of it, which
// halves the transposing LDS reads (the slowest LDS read form on gfx950).
//
// Stage s of the K loop lives in slot s % S of an S-slot LDS ring (S = 4..6):
//   A part [BM][32] bf16, 64-byte rows; the 16-byte chunk c of row r is stored
//     at chunk position c ^ swz_a(r) (conflict-free 16-lane row reads);
//   B part [BN/32 blocks][32 k][32 n] bf16, 64-byte rows, kept k-major as in
//     memory; the 32-byte halves of row k swap when bit 3 of k is set. The MFMA
//     operand (8 consecutive k of one column per lane) is read with the gfx950
//     transposing LDS read ds_read_b64_tr_b16.
// Slots are filled by direct-to-LDS 16-byte loads (global_load_lds_dwordx4 for
// A rows, buffer_load_dwordx4 ... lds for B with out-of-range reads returning
// zero), S-1 stages ahead. They are issued from inline assembly so the
// compiler does not add its own whole-queue waits before every LDS read; the
// explicit vmcnt waits plus one barrier per pair of stages order them. Every
// wave issues the same number of loads per stage, so the waits are constants
// and the K loop has no branches. With one wave per SIMD an instruction only
// overlaps an MFMA if it sits between MFMAs in program order, so the fragment
// reads of stage k+1 and the loads of stage k+S-1 are interleaved with stage
// k's MFMAs.
//
// The MFMA's A operand carries B (rows = n) and its B operand carries A
// (columns = m), so each lane ends with 4 consecutive output columns of one
// row: acc.v[f][g][r] = C[m = wm*BM/2 + 16f + (lane & 15)]
//                        [n = wn*BN/2 + 16g + 4*(lane >> 4) + r].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ocg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define OCG_LDS __attribute__((address_space(3)))

constexpr int BKS = 32;   // K per stage

// Waves per workgroup of a tile: 8 for the 320-row grouped-GEMM tile (a 4 x 2
// wave grid, two waves per SIMD: 140 accumulators per wave instead of 280,
// which the 256-entry accumulator file cannot hold), else 4 (2 x 2). Eight
// waves (4 x 2, two per SIMD) hide each wave's LDS reads and barrier waits
// behind the other's MFMAs: at the 70B share a tile took 9 % fewer shader
// cycles (319k vs 350k), but the clock under the chip's power limit fell by
// as much (1.78 vs 2.00 GHz; 369 vs 372 us GEMM-only, 435 vs 412 us fused,
// same process, alternating) -- the 4 x 2 grid reads 47 % more LDS bytes
// per stage -- so the other tiles keep 4.
template <int BM, int BN>
constexpr int gemm_waves() {
  return BM == 320 ? 8 : 4;
}

template <int BM, int BN>
struct Gemm {
  static constexpr int NW = gemm_waves<BM, BN>();   // waves per workgroup
  static constexpr int NT = 64 * NW;                // threads per workgroup
  static constexpr int WM = BM / (NW / 2), WN = BN / 2;   // rows / columns per wave
  static constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 blocks per wave
  static constexpr int A_BYTES = BM * BKS * 2;
  static constexpr int B_BYTES = BN * BKS * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // LDS ring slots: as deep as ~150 KiB allows (loads of S-1 stages in flight
  // hide HBM latency when a tile streams operands with little reuse), at most
  // 6; the 128x128 tile keeps 4 so two workgroups fit on a CU.
  static constexpr int S = (BM == 128 && BN == 128) ? 4 : ((150 * 1024 / STAGE) < 6 ? 150 * 1024 / STAGE : 6);
  static constexpr int A_INST = A_BYTES / 1024;     // 1 KiB DMA instructions per stage
  static constexpr int B_INST = B_BYTES / 1024;
  static constexpr int A_PER_WAVE = (A_INST + NW - 1) / NW;  // A instruction of wave w: see a_block
  // JOINT: the A blocks do not split evenly over the waves but A and B
  // blocks together do (288x224: 18 + 14 = 32). The stage's loads are then
  // numbered A blocks first, then B blocks, and load I of wave w is number
  // w + NW*I: every wave issues the same count and none repeats a load.
  // Otherwise A and B split separately and a wave past the last block of
  // either repeats its previous load.
  static constexpr bool JOINT = (A_INST % NW != 0) && ((A_INST + B_INST) % NW == 0);
  static constexpr int A_MIN = JOINT ? A_INST / NW : A_PER_WAVE;  // loads I < A_MIN are A loads in every wave
  static constexpr int NDMA = JOINT ? (A_INST + B_INST) / NW
                                    : A_PER_WAVE + (B_INST + NW - 1) / NW;  // loads per wave per stage
  static constexpr int B_PER_WAVE = NDMA - A_MIN;   // loads I >= A_MIN that may be B loads
  static constexpr int RING = S * STAGE;
  // Tiles with more accumulators than the 256-entry accumulator file keep
  // one set of B fragments instead of two (block g of the next stage is read
  // into b[g] right after MFMA group g used it): it lowers the register
  // pressure of the 320x224 tile (280 accumulators per lane) and measured
  // faster there, slower for tiles that fit.
  static constexpr bool SINGLE_B = FM * FN * 4 > 256 / (NW / 4);
  // 4-wave tiles that fill (nearly) the whole accumulator file: the MFMAs
  // are issued with each accumulator tied to one register (inline assembly),
  // since the compiler otherwise rotates accumulators through spare
  // registers (a move between dependent MFMAs) once fewer than 8 are free.
  static constexpr bool TIED_ACC = NW == 4 && FM * FN * 4 > 248;
  // With SINGLE_B a fragment read overwrites the B registers right after the
  // group's MFMAs read them, a hazard the compiler pads only for MFMAs it
  // can see, so the two are never combined.
  static_assert(!(TIED_ACC && SINGLE_B), "tied accumulators need double-buffered B fragments");
  static constexpr int LD_C = BN + 8;               // epilogue staging row (elements)
  static constexpr int LDS_BYTES = (RING > BM * LD_C * 2) ? RING : BM * LD_C * 2;
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BN % 32 == 0, "whole 16x16 blocks per wave, 32-column B blocks");
  static_assert(A_INST >= NW, "every wave has A loads");
  static_assert(NDMA <= 2 * FN, "at most two loads behind each MFMA group");
  static_assert(S >= 4 && (S - 2) * NDMA <= 63, "vmcnt waits fit the 6-bit counter");
  static_assert(LDS_BYTES <= 160 * 1024 - 64, "fits the 160 KiB LDS of a gfx950 CU");
};

// fp32 accumulators of one wave's part of the tile.
template <int BM, int BN>
struct AccTile {
  f32x4_t v[Gemm<BM, BN>::FM][Gemm<BM, BN>::FN];
};

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int k) { return (k >> 3) & 1; }

__device__ __forceinline__ uint32_t lds_u32(OCG_LDS const void* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ void dma_global(uint32_t lds, const void* g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma_buffer(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int BM, int BN>
struct Frags {
  bf16x8_t a[Gemm<BM, BN>::FM];   // [16-row block]: 8 k of row (lane & 15), k group lane >> 4
  bf16x8_t b[Gemm<BM, BN>::FN];   // [16-col block]: 8 k of column (lane & 15), k group lane >> 4
};

template <int BM, int BN>
struct TileCtx {
  const char* rowp[Gemm<BM, BN>::A_PER_WAVE];  // A row of DMA instruction i for this lane, at k = 0
  __amdgpu_buffer_rsrc_t brs;                   // B [K][N] (out-of-range reads return 0)
  int N, n0, nk;
};

// 1 KiB block of the slot's A part (rows 16b..16b+15) that A instruction i
// of wave `wave` loads: consecutive blocks per wave when they split evenly,
// else block wave + NW*i, a wave past the last block repeating its previous
// one (same source, same LDS bytes), so every wave issues A_PER_WAVE loads.
template <int BM, int BN>
__device__ __forceinline__ int a_block(int wave, int i) {
  using G = Gemm<BM, BN>;
  if constexpr (G::A_INST % G::NW == 0) {
    return wave * G::A_PER_WAVE + i;
  } else {
    const int j = wave + G::NW * i;
    return j < G::A_INST ? j : j - G::NW;
  }
}

// Row of the tile that lane `lane` of DMA instruction i (of wave `wave`) loads.
template <int BM, int BN>
__device__ __forceinline__ int dma_row(int wave, int i, int lane) {
  return a_block<BM, BN>(wave, i) * 16 + (lane >> 2);
}

// Whether load I of wave `wave` is an A load (wave-uniform).
template <int BM, int BN>
__device__ __forceinline__ bool load_is_a(int wave, int I) {
  using G = Gemm<BM, BN>;
  if constexpr (G::JOINT) return wave + G::NW * I < G::A_INST;
  return I < G::A_PER_WAVE;
}

// 1 KiB B block that B-capable load A_MIN + i of wave `wave` fetches (any
// valid block where that load is an A load of this wave).
template <int BM, int BN>
__device__ __forceinline__ int b_block(int wave, int i) {
  using G = Gemm<BM, BN>;
  if constexpr (G::JOINT) {
    const int j = wave + G::NW * (G::A_MIN + i) - G::A_INST;
    return j < 0 ? 0 : j;
  } else {
    const int j = wave + G::NW * i;
    return j >= G::B_INST ? j - G::NW : j;
  }
}

// Per-tile constants of this wave's loads: the A instruction i loads rows
// 16*b + lane/4 (b = a_block(wave, i)), chunk (lane & 3) ^ swz_a(row), into
// the slot's 1 KiB block b; B-capable load i (j = b_block(wave, i)) loads k
// row (j & 1)*16 + lane/4 of column block j/2, chunk pair
// (lane & 3) ^ 2*swz_b(k), into block j of the slot's B part. Every wave
// issues NDMA loads per stage.
template <int BM, int BN>
struct DmaPlan {
  const char* a[Gemm<BM, BN>::A_PER_WAVE];     // per lane, stage 0
  uint32_t b_off[Gemm<BM, BN>::B_PER_WAVE];    // per lane byte offset in B, stage 0
  uint32_t b_dst[Gemm<BM, BN>::B_PER_WAVE];    // LDS offset within a slot (wave-uniform)
  uint32_t b_step;                             // bytes of B per stage (32 rows)
};

template <int BM, int BN>
__device__ __forceinline__ DmaPlan<BM, BN> make_dma_plan(const TileCtx<BM, BN>& t, int wave) {
  using G = Gemm<BM, BN>;
  const int lane = threadIdx.x & 63;
  DmaPlan<BM, BN> d;
#pragma unroll
  for (int i = 0; i < G::A_PER_WAVE; ++i) {
    const int r = a_block<BM, BN>(wave, i) * 16 + (lane >> 2);
    d.a[i] = t.rowp[i] + ((lane & 3) ^ swz_a(r)) * 16;
  }
#pragma unroll
  for (int i = 0; i < G::B_PER_WAVE; ++i) {
    const int j = b_block<BM, BN>(wave, i);
    const int nb = j >> 1, k = (j & 1) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ (2 * swz_b(k));
    // byte offset of B[k][n0 + 32*nb + 8*c]; K*N*2 < 2^32 (unsigned math)
    d.b_off[i] = ((uint32_t)k * (uint32_t)t.N + (uint32_t)(t.n0 + nb * 32 + c * 8)) * 2u;
    d.b_dst[i] = (uint32_t)(G::A_BYTES + j * 1024);
  }
  d.b_step = (uint32_t)BKS * (uint32_t)t.N * 2u;
  return d;
}

// Load number `I` (0 <= I < NDMA) of this wave for stage `s` into `slot`.
template <int BM, int BN, int I>
__device__ __forceinline__ void dma_one(uint32_t slot, const DmaPlan<BM, BN>& d, const __amdgpu_buffer_rsrc_t& brs,
                                        int s, int wave) {
  using G = Gemm<BM, BN>;
  if constexpr (I < G::A_MIN) {
    dma_global(slot + a_block<BM, BN>(wave, I) * 1024, d.a[I] + s * (BKS * 2));
  } else if constexpr (I >= G::A_PER_WAVE) {
    constexpr int i = I - G::A_MIN;
    dma_buffer(slot + d.b_dst[i], brs, d.b_off[i] + (uint32_t)s * d.b_step);
  } else {
    // JOINT: A load in the first waves, B load in the others
    constexpr int i = I - G::A_MIN;
    if (load_is_a<BM, BN>(wave, I))
      dma_global(slot + a_block<BM, BN>(wave, I) * 1024, d.a[I] + s * (BKS * 2));
    else
      dma_buffer(slot + d.b_dst[i], brs, d.b_off[i] + (uint32_t)s * d.b_step);
  }
}

template <int BM, int BN, int I = 0>
__device__ __forceinline__ void dma_stage(uint32_t slot, const DmaPlan<BM, BN>& d, const __amdgpu_buffer_rsrc_t& brs,
                                          int s, int wave) {
  if constexpr (I < Gemm<BM, BN>::NDMA) {
    dma_one<BM, BN, I>(slot, d, brs, s, wave);
    dma_stage<BM, BN, I + 1>(slot, d, brs, s, wave);
  }
}

struct FragAddr {
  uint32_t a;        // A block f = 0 (block f adds f*1024: 16 rows of 64 bytes)
  uint32_t b[2];     // B block g, low 4 k rows: b[g & 1] + (g >> 1)*2048; high 4 rows +256
};

// Per-lane LDS byte offsets (within a slot) of this wave's fragments. Lane
// l = 16q + j reads A row wm*BM/2 + j, k chunk q (8 k), and, for the 16-column
// block c, the transposing reads of k rows 8q + j/4 (+4), columns 4(j & 3)..+3
// of the block, which leave column j, k rows 8q..8q+3 (+4..7) in lane l.
template <int BM, int BN>
__device__ __forceinline__ FragAddr frag_addr(int wave) {
  using G = Gemm<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, j = lane & 15;
  FragAddr fa;
  const int r = wm * G::WM + j;
  fa.a = r * 64 + ((q ^ swz_a(r)) * 16);
  const int kk = 8 * q + (j >> 2);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = wn * G::FN + t;   // 16-column block of g = t
    fa.b[t] = G::A_BYTES + (c >> 1) * 2048 + kk * 64 + (((c & 1) ^ swz_b(kk)) * 32) + (j & 3) * 8;
  }
  return fa;
}

template <int BM, int BN>
__device__ __forceinline__ bf16x8_t read_b_frag(OCG_LDS const char* st, const FragAddr& fa, int g) {
  OCG_LDS const char* p = st + fa.b[g & 1] + (g >> 1) * 2048;
  bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((OCG_LDS bf16x4_t*)p);
  bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((OCG_LDS bf16x4_t*)(p + 256));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int BM, int BN>
__device__ __forceinline__ void read_frags(OCG_LDS const char* st, const FragAddr& fa, Frags<BM, BN>& fr) {
  using G = Gemm<BM, BN>;
#pragma unroll
  for (int g = 0; g < G::FN; ++g) fr.b[g] = read_b_frag<BM, BN>(st, fa, g);
#pragma unroll
  for (int f = 0; f < G::FM; ++f) fr.a[f] = *(OCG_LDS const bf16x8_t*)(st + fa.a + f * 1024);
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left open (gfx9 encoding), as a
// builtin so the compiler's own wait insertion knows every LDS read is done.
// The scheduling fences keep it from being hoisted above the MFMAs.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_sched_barrier(0);
}

// The loads I of stage `s` with I * FN / NDMA == GI (spread evenly over the
// FN MFMA groups, which keeps the per-CU memory pipe from queueing up behind
// a burst).
template <int BM, int BN, int GI, int I = 0>
__device__ __forceinline__ void dma_after_group(uint32_t slot, const DmaPlan<BM, BN>& d,
                                                const __amdgpu_buffer_rsrc_t& brs, int s, int wave) {
  using G = Gemm<BM, BN>;
  if constexpr (I < G::NDMA) {
    if constexpr ((I * G::FN) / G::NDMA == GI) dma_one<BM, BN, I>(slot, d, brs, s, wave);
    dma_after_group<BM, BN, GI, I + 1>(slot, d, brs, s, wave);
  }
}

// acc += a x b on one 16x16 block: the builtin, or with TIED the same
// instruction with the accumulator in one fixed accumulator register tuple.
template <bool TIED>
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t b, bf16x8_t a, f32x4_t acc) {
  if constexpr (TIED) {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    return acc;
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc, 0, 0, 0);
  }
}

// MFMA group GI (column block GI) of `cur`, preceded by the two transposing
// reads of the same block of `nxt` and followed by its share of the loads.
// With SINGLE_B the B fragments live in `bs` only and the reads follow the
// group's MFMAs.
template <int BM, int BN, int GI = 0>
__device__ __forceinline__ void mfma_groups(const Frags<BM, BN>& cur, Frags<BM, BN>& nxt, OCG_LDS const char* st,
                                            const FragAddr& fa, AccTile<BM, BN>& acc, uint32_t slot,
                                            const DmaPlan<BM, BN>& d, const __amdgpu_buffer_rsrc_t& brs, int s,
                                            int wave, bf16x8_t (&bs)[Gemm<BM, BN>::FN]) {
  using G = Gemm<BM, BN>;
  if constexpr (GI < G::FN) {
    if constexpr (G::SINGLE_B) {
#pragma unroll
      for (int f = 0; f < G::FM; ++f)
        acc.v[f][GI] = mfma16<G::TIED_ACC>(bs[GI], cur.a[f], acc.v[f][GI]);
      bs[GI] = read_b_frag<BM, BN>(st, fa, GI);
    } else {
      nxt.b[GI] = read_b_frag<BM, BN>(st, fa, GI);
#pragma unroll
      for (int f = 0; f < G::FM; ++f)
        acc.v[f][GI] = mfma16<G::TIED_ACC>(cur.b[GI], cur.a[f], acc.v[f][GI]);
    }
    dma_after_group<BM, BN, GI>(slot, d, brs, s, wave);
    __builtin_amdgcn_sched_barrier(0);
    mfma_groups<BM, BN, GI + 1>(cur, nxt, st, fa, acc, slot, d, brs, s, wave, bs);
  }
}

// One K stage: MFMAs of `cur`, with the fragment reads of the next stage from
// `st` (into `nxt`) and the loads of stage `s` into `slot` spread between
// them. No MFMA depends on a read issued in the same stage.
template <int BM, int BN>
__device__ __forceinline__ void stage_body(const Frags<BM, BN>& cur, Frags<BM, BN>& nxt, OCG_LDS const char* st,
                                           const FragAddr& fa, AccTile<BM, BN>& acc, uint32_t slot,
                                           const DmaPlan<BM, BN>& d, const __amdgpu_buffer_rsrc_t& brs, int s,
                                           int wave, bf16x8_t (&bs)[Gemm<BM, BN>::FN]) {
  using G = Gemm<BM, BN>;
#pragma unroll
  for (int f = 0; f < G::FM; ++f) nxt.a[f] = *(OCG_LDS const bf16x8_t*)(st + fa.a + f * 1024);
  mfma_groups<BM, BN>(cur, nxt, st, fa, acc, slot, d, brs, s, wave, bs);
  // The reads of `nxt` had the whole MFMA block to land.
  lds_reads_done();
}

// Per-pair hook of the K loop: prefetch(k) runs at the start of pair k, before
// its wait; check(k) after the wait and before the barrier that releases the
// pair's loads (stages k+S-1 and k+S). NoHook does nothing; the AG-GEMM tiles
// use them to wait on the flags of the K-slabs they are about to load.
struct NoHook {
  __device__ __forceinline__ void prefetch(int) {}
  __device__ __forceinline__ void check(int) {}
};

// C tile += A[rows of t.rowp][0:K] x B[0:K][n0:n0+BN], K = 32 * t.nk (nk even).
// Starts and ends with every wave past a barrier; LDS is free afterwards.
//
// Stage j lives in slot j % S. Step k computes stage k while reading stage
// k+1 and loading stage k+S-1 into slot (k+S-1) % S = (k-1) % S. Steps come
// in pairs (k even, k+1) with one wait + barrier per pair, at step k: wait
// until at most S-4 stages of this wave's loads are in flight (stages k+1 and
// k+2 have landed), then barrier (everyone's have, and every wave finished
// reading stage k-1 (in step k-2) and stage k (in step k-1), the slots the
// pair overwrites). A 4-slot ring waits and syncs before every step instead
// (stage k+1 landed, stage k+2 may still be in flight; the barrier also
// covers the slot of stage k-1 that step k overwrites). Past the end the
// loads repeat stage nk-1 into the free
// slot, which is never read again, so the per-step load count and the wait
// are constants; in the last step the fragment reads fetch a stale slot whose
// values are never used.
template <int BM, int BN, class Hook>
__device__ __forceinline__ void mainloop(OCG_LDS char* smem, const TileCtx<BM, BN>& t, AccTile<BM, BN>& acc,
                                         Hook& hook) {
  using G = Gemm<BM, BN>;
  constexpr int S = G::S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t base = lds_u32(smem);
  const FragAddr fa = frag_addr<BM, BN>(wave);
  const DmaPlan<BM, BN> d = make_dma_plan<BM, BN>(t, wave);
  const int nk = t.nk;
#pragma unroll
  for (int f = 0; f < G::FM; ++f)
#pragma unroll
    for (int g = 0; g < G::FN; ++g) acc.v[f][g] = f32x4_t{};
  // Tied MFMAs: each zeroed accumulator passes through a 2-wait-state nop
  // of its own before any MFMA can read it (the compiler pads only the
  // MFMAs it sees).
  if constexpr (G::TIED_ACC) {
#pragma unroll
    for (int f = 0; f < G::FM; ++f)
#pragma unroll
      for (int g = 0; g < G::FN; ++g) asm volatile("s_nop 1" : "+a"(acc.v[f][g]));
  }
  // prologue: stages 0 .. S-2 (repeating stage nk-1 past the end)
#pragma unroll
  for (int j = 0; j < S - 1; ++j) dma_stage<BM, BN>(base + j * G::STAGE, d, t.brs, j < nk ? j : nk - 1, wave);
  vm_wait<(S - 2) * G::NDMA>();
  lds_barrier();
  Frags<BM, BN> f0, f1;
  read_frags<BM, BN>(smem, fa, f0);
  lds_reads_done();
  // SINGLE_B: the one set of B fragments (unused otherwise)
  bf16x8_t bs[G::FN];
  if constexpr (G::SINGLE_B) {
#pragma unroll
    for (int g = 0; g < G::FN; ++g) bs[g] = f0.b[g];
  }
  uint32_t rd = G::STAGE, wr = (S - 1) * G::STAGE;   // slot offsets of stages k+1 and k+S-1
  auto step = [&](int k, Frags<BM, BN>& cur, Frags<BM, BN>& nxt) {
    stage_body<BM, BN>(cur, nxt, smem + rd, fa, acc, base + wr, d, t.brs, k + S - 1 < nk ? k + S - 1 : nk - 1, wave,
                       bs);
    rd = (rd + G::STAGE == S * G::STAGE) ? 0u : rd + G::STAGE;
    wr = (wr + G::STAGE == S * G::STAGE) ? 0u : wr + G::STAGE;
  };
  for (int k = 0; k < nk; k += 2) {
    hook.prefetch(k);
    if constexpr (S >= 5) {
      vm_wait<(S - 4) * G::NDMA>();
      hook.check(k);
      lds_barrier();
      step(k, f0, f1);
      step(k + 1, f1, f0);
    } else {
      // A 4-slot ring would leave no load in flight at a pair's wait (stage
      // k+2 is issued in step k-1): wait and barrier before every step
      // instead, for stage k+1 only, so the loads of stage k+2 stay in
      // flight and each stage has two steps to land, as with 5 slots.
      vm_wait<(S - 3) * G::NDMA>();
      hook.check(k);
      lds_barrier();
      step(k, f0, f1);
      vm_wait<(S - 3) * G::NDMA>();
      lds_barrier();
      step(k + 1, f1, f0);
    }
    // The compiler does not see the tied MFMAs as MFMAs, so it does not pad
    // a read of their results: 20 wait states (at least the 19 these 8-pass
    // MFMAs need) end every pair of steps, before anything can read an
    // accumulator (the copies the compiler places at the loop exit
    // included). They overlap the last MFMA, which still occupies the pipe.
    if constexpr (G::TIED_ACC) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  }
  vm_wait<0>();   // no load may still target LDS when the tile's LDS is reused
  lds_barrier();
  if constexpr (G::TIED_ACC) {
    // each accumulator leaves the loop in the register it was tied to
#pragma unroll
    for (int f = 0; f < G::FM; ++f)
#pragma unroll
      for (int g = 0; g < G::FN; ++g) asm volatile("" : "+a"(acc.v[f][g]));
  }
}

template <int BM, int BN>
__device__ __forceinline__ void mainloop(OCG_LDS char* smem, const TileCtx<BM, BN>& t, AccTile<BM, BN>& acc) {
  NoHook h;
  mainloop<BM, BN, NoHook>(smem, t, acc, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Round the tile to bf16 (nearest-even, v_cvt_pk_bf16_f32) and stage it in
// LDS as [BM][BN + 8]; ends with a barrier.
template <int BM, int BN>
__device__ __forceinline__ void stage_c(OCG_LDS char* smem, const AccTile<BM, BN>& acc) {
  using G = Gemm<BM, BN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  OCG_LDS uint16_t* cst = (OCG_LDS uint16_t*)smem;
#pragma unroll
  for (int f = 0; f < G::FM; ++f) {
    const int row = wm * G::WM + 16 * f + (lane & 15);
#pragma unroll
    for (int g = 0; g < G::FN; ++g) {
      const int col = wn * G::WN + 16 * g + 4 * (lane >> 4);
      u32x2_t v = {pack_bf16x2(acc.v[f][g][0], acc.v[f][g][1]), pack_bf16x2(acc.v[f][g][2], acc.v[f][g][3])};
      *(OCG_LDS u32x2_t*)(cst + row * G::LD_C + col) = v;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
}

// f(row_in_tile, col_in_tile, 16-byte value) over every 16-byte chunk of the
// staged tile, consecutive threads on consecutive chunks of a row.
template <int BM, int BN, class F>
__device__ __forceinline__ void for_each_c_chunk(OCG_LDS const char* smem, F f) {
  using G = Gemm<BM, BN>;
  constexpr int CPR = BN / 8;
  OCG_LDS const uint16_t* cst = (OCG_LDS const uint16_t*)smem;
  for (int i = threadIdx.x; i < BM * CPR; i += G::NT) {
    const int row = i / CPR, c8 = i - row * CPR;
    f(row, c8 * 8, *(OCG_LDS const u32x4_t*)(cst + row * G::LD_C + c8 * 8));
  }
}

}  // namespace ocg
