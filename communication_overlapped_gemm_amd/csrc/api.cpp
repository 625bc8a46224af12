// C-ABI layer: argument checks, tile/slab plan resolution, workspace layout
// and launches. Every entry point returns an OCG_* status and enqueues
// nothing when it returns an error.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "ocg_internal.h"

using namespace ocg;

struct ocg_handle_s {
  int device;
  int cus;
  int resident[3][OCG_TILE_COUNT];  // per op and tile preset, 0 = not queried yet
  int resident_split[OCG_TILE_COUNT];   // AG-GEMM kernel of split-K units, per preset
  int resident_attn;                // attention kernel, 0 = not queried yet
  int side_fits[OCG_TILE_COUNT];    // AG-GEMM kernel + side producer fit on a CU: 0 unknown, 1 yes, -1 no
  hipStream_t side;                 // side stream of the SIDE transfer mode (default priority)
  hipEvent_t fork, join;            // caller stream -> side stream -> caller stream
  void* scratch;                    // device address of the no-allocation scratch on `device`
};

namespace {

constexpr uint64_t kTicksPerUs = 100;  // s_memrealtime runs at 100 MHz

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMinKslabCols = 256;    // K-slab widths are multiples of this
constexpr int kSideKslabCols = 512;   // default K-slab width of the SIDE transfer mode

// Workspace sections, sized for the worst plan a call of this shape can pick
// (smallest slab, K-slab, tile and strip sizes). max_slabs counts flags:
// (slab, K-slab) pairs for AG-GEMM, slabs for the other gathers.
// sk_tiles > 0: an AG-GEMM plan that splits K, with tiles of sk_area
// elements (per tile an arrival count, a flag and the first half's fp32 sums).
WsLayout layout(int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk, int64_t sk_tiles = 0,
                int64_t sk_area = 0) {
  WsLayout L{};
  size_t off = sizeof(WsHeader);
  int64_t rows = (op == OCG_OP_GEMM_RS) ? m : (int64_t)R * m;
  const int nks = (op == OCG_OP_AG_GEMM) ? cdiv((int)K, kMinKslabCols) : 1;
  L.max_slabs = (op == OCG_OP_GEMM_RS) ? 0 : (int)(R * cdiv((int)m, kMinSlabRows)) * nks;
  L.max_rs_tiles = (op == OCG_OP_GEMM_RS) ? cdiv((int)rows, 128) * cdiv((int)N, 128) : 0;
  L.slab_cnt = off;
  off = align256(off + sizeof(uint32_t) * L.max_slabs);
  L.slab_flag = off;
  off = align256(off + sizeof(uint32_t) * L.max_slabs);
  L.rs_flag = off;
  off = align256(off + sizeof(uint32_t) * L.max_rs_tiles);
  L.rs_sum = off;   // one word per row block of the local block (blocks of >= 128 rows)
  off = align256(off + sizeof(uint32_t) * (op == OCG_OP_GEMM_RS ? cdiv((int)(rows / R), 128) + 1 : 0));
  L.moe_off = L.moe_lut = L.moe_perm = L.moe_bcnt = L.moe_inv = L.moe_lbase = L.moe_tflag = off;
  L.max_moe_tiles = 0;
  if (op == OCG_OP_AG_GROUPED_GEMM) {
    int slots = (int)(rows * topk);
    // sized for the preset with the most tiles (128-row)
    L.max_moe_tiles = (cdiv(slots, tile_bm(kMoeTileSmall)) + E) * cdiv((int)N, tile_bn(kMoeTileSmall));
    L.moe_off = off;
    off = align256(off + sizeof(int32_t) * (E + 1));
    L.moe_lut = off;
    off = align256(off + sizeof(int32_t) * 8 * (size_t)L.max_moe_tiles);
    L.moe_perm = off;
    off = align256(off + sizeof(int32_t) * (size_t)slots);
    const int nb = cdiv((int)rows, kRouteBlock);
    L.moe_bcnt = off;
    off = align256(off + sizeof(int32_t) * (size_t)nb * E);
    L.moe_inv = off;       // position of each token-slot in the sorted order
    off = align256(off + sizeof(int32_t) * (size_t)slots);
    L.moe_lbase = off;     // first lookup-table entry of each expert
    off = align256(off + sizeof(int32_t) * (size_t)E);
    L.moe_tflag = off;     // per grouped tile: epoch once its rows are stored
    off = align256(off + sizeof(uint32_t) * (size_t)L.max_moe_tiles);
  }
  L.sk_cnt = L.sk_flag = L.sk_part = off;
  if (op == OCG_OP_AG_GEMM && sk_tiles > 0) {
    L.sk_cnt = off;
    off = align256(off + sizeof(uint32_t) * (size_t)sk_tiles);
    L.sk_flag = off;
    off = align256(off + sizeof(uint32_t) * (size_t)sk_tiles);
    L.sk_part = off;
    off = align256(off + sizeof(float) * (size_t)sk_tiles * (size_t)sk_area);
  }
  (void)K;
  L.total = off;
  return L;
}

bool shape_ok(int R, int64_t m, int64_t K, int64_t N) {
  if (R < 1 || R > kMaxRanks || m < 1 || K < 64 || N < 8) return false;
  if (K % 64 != 0 || N % 8 != 0) return false;
  // 32-bit element/byte offsets inside buffer descriptors and tile math
  if ((int64_t)R * m > (1 << 30) || K > (1 << 20) || N > (1 << 20)) return false;
  if (K * N * 2 > 0xFFFFFFFFll) return false;
  return true;
}

// Estimated cost of a tile preset split in sk K parts: rounds of the
// persistent grid (of units, tiles x sk) times the tile area over the
// preset's relative speed per output element, times the share of K a unit
// runs plus, when split, a fixed cost worth the K loop over 1800 columns
// (fitted: at the 8B share 256x224 halves ran their loops in 60 us against
// 54 us for whole 128x224 tiles of the same MFMA work, and the combine --
// one half's fp32 sums stored, then read and added -- took the other 12 us:
// 85.3 against 72.0 us GEMM-only; on 512-1024-row shares with K 8192, whose
// whole tiles fill under half the CUs, split 128x128 tiles were 8-10 %
// faster).
// Speeds from GEMM-only launches at the 8B AllGather share (M 4096, K 4096,
// N 1792; one MI355X): 256x224 tiles 93.6 us for 128 tiles (one round, half
// the CUs idle) = 1; 128x256 74.6 us for 224 tiles -> 0.717; 256x256 104.2
// us for 112 -> 1.03; 128x128 94.0 us for 448 (two rounds) -> 0.57. 128x224
// (256 tiles, one per CU) measured 74.8 us then (0.626); since the workspace
// counters got cache lines of their own it runs 61.9 us against 66.2 us for
// 128x256 (same process, alternating): 0.935 of 128x256's speed per output
// element -> 0.670.
double tile_cost(int t, int64_t M, int64_t N, int64_t K, int cus, int sk) {
  static const double eff[OCG_TILE_COUNT] = {1.0, 0.670, 0.717, 0.57, 1.03, 0.0, 0.0};
  if (t < 0 || t >= OCG_TILE_COUNT || eff[t] <= 0) return 1e300;   // grouped-GEMM-only presets
  const int64_t units = cdiv((int)M, tile_bm(t)) * (int64_t)cdiv((int)N, tile_bn(t)) * sk;
  const int64_t rounds = (units + cus - 1) / cus;
  const double part = 1.0 / sk + (sk > 1 ? 1800.0 / (double)K : 0.0);
  return (double)rounds * tile_bm(t) * tile_bn(t) / eff[t] * part;
}

// The cheapest (preset, K parts): `tile` >= 0 fixes the preset; sk 2 is
// considered only if `can_split`.
void choose_tile(int64_t M, int64_t N, int64_t K, int cus, int tile, bool can_split, int* tile_out, int* sk_out) {
  int best = tile >= 0 ? tile : OCG_TILE_128x128, best_sk = 1;
  double best_cost = 1e300;
  for (int t = 0; t < OCG_TILE_COUNT; ++t) {
    if (tile >= 0 && t != tile) continue;
    for (int sk = 1; sk <= (can_split ? 2 : 1); ++sk) {
      const double cost = tile_cost(t, M, N, K, cus, sk);
      if (cost < best_cost * (1.0 - 1e-9)) {
        best_cost = cost;
        best = t;
        best_sk = sk;
      }
    }
  }
  *tile_out = best;
  *sk_out = best_sk;
}

// Grouped GEMM: one row tile per expert where the rows an expert gets fit
// in a preset -- the count is binomial (T tokens, each picking the expert
// with probability topk/E); its mean plus two standard deviations is taken
// as the rows to hold -- the smallest such preset; 256-row tiles when experts
// are larger. A second row tile for the few rows past a tile boundary would
// cost as much as a full one; an expert past the estimate still gets one.
int choose_moe_tile(int64_t T, int E, int topk) {
  if (E < 1) return OCG_TILE_256x224;
  const double p = (double)topk / E;
  const double avg = (double)T * p;
  const double hi = avg + 2.0 * sqrt(avg * (1.0 - p));
  if (hi <= 128) return OCG_TILE_128x224;
  if (hi <= 256) return OCG_TILE_256x224;
  if (hi <= 288) return OCG_TILE_288x224;
  if (hi <= 320) return OCG_TILE_320x224;
  return OCG_TILE_256x224;
}

struct Resolved {
  int tile, BM, BN, S, CT, KS, transfer, SK;
};

// split_room: the caller's workspace can hold split-K sums (AG-GEMM; the
// automatic choice splits only then).
int resolve(int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk, const ocg_config& c, int cus,
            Resolved* r, bool split_room = true) {
  int64_t M = (op == OCG_OP_GEMM_RS) ? m : R * m;
  // transfer mode and K-slab width (AG-GEMM; the other ops copy whole rows)
  r->transfer = OCG_TRANSFER_INLINE;
  r->KS = (int)K;
  r->SK = 1;
  if (op == OCG_OP_AG_GEMM) {
    if (c.transfer < OCG_TRANSFER_AUTO || c.transfer > OCG_TRANSFER_SIDE) return OCG_ERR_INVALID_ARG;
    // AUTO: INLINE. SIDE measures 1-3 % faster per fused call at the 70B
    // share (two builds in one process, alternating: 391-412 against
    // 402-416 us) and 12 % slower at the 8B share (one round of tiles), but
    // its GEMM tiles wait on a second kernel: under a tool that runs
    // dispatches one at a time they can wait out their bound. Guarding that
    // (the producer marks itself started; a tile that finds it not started
    // runs its copy tickets) was correct but cost ~10 us per 70B call, more
    // than SIDE gains, so one kernel stays the default.
    r->transfer = c.transfer == OCG_TRANSFER_AUTO ? OCG_TRANSFER_INLINE : c.transfer;
    if (c.mode == OCG_MODE_GEMM_ONLY) r->transfer = OCG_TRANSFER_INLINE;   // no copies to place
    if (c.kslab_cols < 0 || c.kslab_cols % kMinKslabCols) return OCG_ERR_INVALID_ARG;
    if (c.kslab_cols > 0)
      r->KS = c.kslab_cols;
    else if (r->transfer == OCG_TRANSFER_SIDE)
      r->KS = kSideKslabCols;
    if (r->KS > K) r->KS = (int)K;
    if (c.split_k < 0 || c.split_k > 2) return OCG_ERR_INVALID_ARG;
  }
  // split K: AG-GEMM, inline copies, one K-slab, and halves of whole MFMA
  // stage pairs (K % 128 == 0)
  const bool can_split = op == OCG_OP_AG_GEMM && r->transfer == OCG_TRANSFER_INLINE && r->KS == K && K % 128 == 0 &&
                         c.mode != OCG_MODE_COPY_ONLY;
  if (op == OCG_OP_AG_GROUPED_GEMM) {
    r->tile = c.tile < 0 ? choose_moe_tile(M, E, topk) : c.tile;
  } else if (op == OCG_OP_AG_GEMM && c.split_k == 2) {
    if (!can_split) return OCG_ERR_INVALID_ARG;
    r->SK = 2;
    r->tile = c.tile;
    if (r->tile < 0) {   // the cheapest preset for halves
      double best = 1e300;
      for (int t = 0; t < OCG_TILE_COUNT; ++t) {
        const double cost = tile_cost(t, M, N, K, cus, 2);
        if (cost < best * (1.0 - 1e-9)) {
          best = cost;
          r->tile = t;
        }
      }
    }
  } else {
    const bool auto_split = op == OCG_OP_AG_GEMM && c.split_k == 0 && can_split && split_room;
    choose_tile(M, N, K, cus, c.tile, auto_split, &r->tile, &r->SK);
  }
  if (r->tile < 0 || r->tile >= OCG_TILE_COUNT) return OCG_ERR_INVALID_ARG;
  if (op == OCG_OP_AG_GROUPED_GEMM ? !moe_tile_ok(r->tile) : (r->tile == OCG_TILE_320x224 || r->tile == OCG_TILE_288x224))
    return OCG_ERR_INVALID_ARG;
  r->BM = tile_bm(r->tile);
  r->BN = tile_bn(r->tile);
  r->S = c.slab_rows > 0 ? c.slab_rows : r->BM;
  if (r->S < kMinSlabRows) return OCG_ERR_INVALID_ARG;
  if (c.copy_rows > 0) {
    r->CT = c.copy_rows;
  } else {
    // a power of two dividing the slab, about 256 KiB per copy task -- 32 KiB
    // for the side producer, whose workgroups keep 16 KiB in flight: small
    // tasks spread each K-slab over many of them
    int64_t ct = (r->transfer == OCG_TRANSFER_SIDE ? 16 * 1024 : 128 * 1024) / (r->KS > 0 ? r->KS : 1);
    // at least one task per workgroup, so the copies spread over all of
    // them: the grouped GEMM's tiles hold tokens of every rank, so none
    // starts before the whole gather has landed (MoE share: 16-row tasks,
    // 169 vs 175 us per step); the AllGather-GEMM's tiles wait for their
    // own rows' slabs, fed sooner the same way (8B share: 16-row tasks,
    // 80.6-80.8 vs 82.3-82.8 us per fused launch; the 70B share keeps 16),
    // but no task under 64 KiB, whose fixed cost (ticket, drain, publish)
    // would outweigh its copy
    const bool spread = op == OCG_OP_AG_GROUPED_GEMM || (op == OCG_OP_AG_GEMM && r->transfer == OCG_TRANSFER_INLINE);
    if (spread && cus > 0) {
      int64_t per_wg = (int64_t)R * m / cus;
      const int64_t floor_rows = (32 * 1024) / (K > 0 ? K : 1);
      if (per_wg < floor_rows) per_wg = floor_rows;
      if (per_wg < ct) ct = per_wg;
    }
    int p2 = 1;
    while ((int64_t)p2 * 2 <= ct) p2 *= 2;
    r->CT = p2 < r->S ? p2 : r->S;
    while (r->S % r->CT) r->CT /= 2;
  }
  if (r->CT < 1 || r->S % r->CT) return OCG_ERR_INVALID_ARG;
  if ((int64_t)r->CT * K * 2 >= ((int64_t)1 << 31)) return OCG_ERR_INVALID_ARG;  // one copy task < 2 GiB
  return OCG_OK;
}

// Whether the AG-GEMM kernel of `tile` (at its resident count per CU) and
// one side producer workgroup fit on a compute unit together: per SIMD the
// registers of the GEMM waves plus a producer wave within 512, LDS within
// 160 KiB. Queried once per handle and tile.
bool side_fits(ocg_handle h, int tile) {
  if (!h || tile < 0 || tile >= OCG_TILE_COUNT) return false;
  int& f = h->side_fits[tile];
  if (f == 0) {
    int vg = 0, lg = 0, vs = 0, ls = 0;
    f = -1;
    if (kernel_resources(OCG_OP_AG_GEMM, tile, &vg, &lg) && kernel_resources(-1, 0, &vs, &ls)) {
      int& r = h->resident[OCG_OP_AG_GEMM][tile];
      if (r == 0) r = resident_per_cu(OCG_OP_AG_GEMM, tile);
      const int waves_per_simd = r * tile_waves(tile) / 4;
      const int regs = waves_per_simd * ((vg + 7) & ~7) + ((vs + 7) & ~7);
      if (regs <= 512 && r * lg + ls <= 160 * 1024) f = 1;
    }
  }
  return f == 1;
}

// Rows per reduce strip: at most ~32 KiB of each partial, and few enough
// that every CU gets a strip (the strips run once the tiles are done).
// TopK-Reduce task sizes: about two tasks per CU, all running at once,
// with equal bytes each -- a local row moves topk + R + 1 rows of data (the
// slot rows, the peers' rows, the partial and out), another row topk + 1.
// At the MoE share (R = 8, m = 512, top-2): 3 local rows or 11 other rows per
// task, 497 tasks.
void combine_rows(int R, int64_t m, int topk, int cus, int* crl, int* cr) {
  const double bl = topk + R + 1.0, bo = topk + 1.0;
  const double T = (double)R * (double)m;
  const double per_task = ((double)m * bl + (T - (double)m) * bo) / (2.0 * (cus > 0 ? cus : 1));
  const long l = llround(per_task / bl), o = llround(per_task / bo);
  *crl = l < 1 ? 1 : (int)l;
  *cr = o < 1 ? 1 : (int)o;
}

bool combine_shape_ok(int R, int64_t m, int64_t N, int topk) {
  if (R < 1 || R > kMaxRanks || m < 1 || N < 8 || N % 8 || topk < 1 || topk > kMaxTopk) return false;
  const int64_t T = (int64_t)R * m;
  if (T > (1 << 24) || N > (1 << 20)) return false;
  if (T * N * 2 >= ((int64_t)1 << 31)) return false;   // 32-bit offsets of the partial's stores
  return true;
}

// AllGather-KV attention shapes: d = 128, Hq a multiple of Hkv, 32-bit
// element offsets into every buffer.
bool attn_shape_ok(int R, int64_t m, int64_t Hq, int64_t Hkv) {
  if (R < 1 || R > kMaxRanks || m < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv) return false;
  if ((int64_t)R * m * Hkv * kAttnD >= ((int64_t)1 << 31)) return false;
  if (m * Hq * kAttnD >= ((int64_t)1 << 31)) return false;
  return true;
}

// Slab rows default to the whole chunk (one flag per chunk: a tile waits per
// chunk); copy tasks of about 128 KiB, a power of two dividing the slab.
int resolve_attn(int64_t m, int64_t Hkv, const ocg_config& c, int* S, int* CT) {
  *S = c.slab_rows > 0 ? c.slab_rows : (int)m;
  if (*S > m) *S = (int)m;
  if (*S < kMinSlabRows && *S < m) return OCG_ERR_INVALID_ARG;
  const int64_t row_bytes = Hkv * kAttnD * 2;
  if (c.copy_rows > 0) {
    *CT = c.copy_rows;
  } else {
    // about 512 KiB per copy task: at the 16K-context share (2 x 64 tasks)
    // half the workgroups gather first while the rest start on the local
    // chunk's keys. Per fused launch (one process, alternating): 1 MiB
    // tasks 530.3 us, 512 KiB 517.5, 256 KiB 520.7, 128 KiB 519.4, 2 MiB
    // 540.5; attention alone 491.2, copies alone 35.6
    int64_t ct = (512 * 1024) / row_bytes;
    int p2 = 1;
    while ((int64_t)p2 * 2 <= ct) p2 *= 2;
    *CT = p2 < *S ? p2 : *S;
    while (*S % *CT) *CT /= 2;
  }
  if (*CT < 1 || *S % *CT) return OCG_ERR_INVALID_ARG;
  if ((int64_t)*CT * row_bytes >= ((int64_t)1 << 31)) return OCG_ERR_INVALID_ARG;
  return OCG_OK;
}

int reduce_rows(int64_t M, int R, int64_t N, int cus) {
  int64_t rr = (32 * 1024) / (2 * N);
  const int64_t spread = (M / R) / (cus > 0 ? cus : 1);
  if (spread < rr) rr = spread;
  return rr < 1 ? 1 : (int)rr;
}

ocg_config cfg_or_default(const ocg_config* c) {
  ocg_config d;
  ocg_config_default(&d);
  return c ? *c : d;
}

// Persistent workgroups for `tasks` tickets of which `units` are GEMM tiles:
// the kernel's resident capacity, except that a preset with two workgroups
// per CU keeps one per CU when its tiles fit in one round -- a second
// workgroup on a CU shares that CU's MFMA pipe, so tiles doubled up on some
// CUs end late (128x128 tiles, 8 ranks x 256 rows, K 8192, N 1792: 224 tiles
// plus 112 copy tasks on 336 workgroups took 150.6 us fused against 89.3 us
// GEMM-only).
int cap_grid(int resident, int cus, int tasks, int units) {
  int g = resident * cus;
  if (resident > 1 && units <= cus) g = cus;
  if (tasks < g) g = tasks;
  return g < 1 ? 1 : g;
}

int grid_for(ocg_handle h, int op, int tile, int tasks, int units, const ocg_config& c) {
  if (c.grid > 0) return c.grid;
  int& r = h->resident[op][tile];
  if (r == 0) r = resident_per_cu(op, tile);
  return cap_grid(r, h->cus, tasks, units);
}

Common make_common(void* ws, const ocg_config& c) {
  Common cm;
  cm.hdr = (WsHeader*)ws;
  uint64_t us = c.spin_timeout_us ? c.spin_timeout_us : 1000000u;
  cm.timeout_ticks = us * kTicksPerUs;
  cm.trace = (ocg_trace_rec*)c.trace;
  cm.trace_cap = c.trace ? c.trace_capacity : 0;
  cm.fault_skip_slab = c.fault_skip_slab;
  cm.copy_delay = c.copy_delay;
  cm.xcd_remap = c.xcd_remap ? 1 : 0;
  cm.total_wgs = 0;
  return cm;
}

bool device_matches(ocg_handle h) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == h->device;
}

// h = NULL plans for a 256-CU MI355X on which the producer fits.
struct AgSetup {
  Resolved rv;
  AgPlan plan;
  WsLayout L;   // the workspace this plan uses
  int ggrid, pgrid;
};

int ag_setup(ocg_handle h, int R, int local_rank, int64_t m, int64_t K, int64_t N, const ocg_config& cfg,
             AgSetup* o, size_t ws_bytes = SIZE_MAX) {
  const int cus = h ? h->cus : 256;
  int st = resolve(OCG_OP_AG_GEMM, R, m, K, N, 0, 0, cfg, cus, &o->rv, true);
  if (st) return st;
  auto need = [&](const Resolved& rv) {
    const int64_t tiles = rv.SK > 1 ? (int64_t)cdiv((int)(R * m), rv.BM) * cdiv((int)N, rv.BN) : 0;
    return layout(OCG_OP_AG_GEMM, R, m, K, N, 0, 0, tiles, (int64_t)rv.BM * rv.BN);
  };
  o->L = need(o->rv);
  if (o->L.total > ws_bytes && o->rv.SK > 1) {
    if (cfg.split_k == 2) return OCG_ERR_WORKSPACE_TOO_SMALL;
    // the automatic choice splits only where the workspace holds the sums
    st = resolve(OCG_OP_AG_GEMM, R, m, K, N, 0, 0, cfg, cus, &o->rv, false);
    if (st) return st;
    o->L = need(o->rv);
  }
  if (h && o->rv.transfer == OCG_TRANSFER_SIDE && !side_fits(h, o->rv.tile)) return OCG_ERR_UNSUPPORTED_SHAPE;
  int resident = 1;
  if (h) {
    int& r = o->rv.SK > 1 ? h->resident_split[o->rv.tile] : h->resident[OCG_OP_AG_GEMM][o->rv.tile];
    if (r == 0) r = resident_per_cu(OCG_OP_AG_GEMM, o->rv.tile, o->rv.SK);
    resident = r;
  } else if (o->rv.tile == OCG_TILE_128x128) {
    resident = 2;   // no handle: two 128x128 workgroups fit on a CU, one of every other preset
  }
  const int tpr = cfg.grid > 0 ? cfg.grid : resident * cus;
  AgPlan& p = o->plan;
  p = make_ag_plan(R, local_rank, (int)m, (int)K, (int)N, o->rv.BM, o->rv.BN, o->rv.S, o->rv.CT,
                   cfg.swizzle ? 1 : 0, cfg.mode, o->rv.KS, tpr, o->rv.SK);
  const bool side = o->rv.transfer == OCG_TRANSFER_SIDE;
  if (side) {
    const int first = first_kslab_tickets(p);
    p.n_inline = first < p.n_copy ? first : p.n_copy;
  }
  const int gtasks = p.n_inline + p.n_tiles * p.sk;
  o->ggrid = cfg.grid > 0 ? (gtasks < tpr ? gtasks : tpr) : cap_grid(resident, cus, gtasks, p.n_tiles * p.sk);
  o->pgrid = 0;
  if (p.n_copy > p.n_inline) {
    const int pg = cfg.side_grid > 0 ? cfg.side_grid : cus;
    o->pgrid = pg < p.n_copy - p.n_inline ? pg : p.n_copy - p.n_inline;
  }
  return OCG_OK;
}

}  // namespace


extern "C" {

void ocg_config_default(ocg_config* c) {
  if (!c) return;
  memset(c, 0, sizeof(*c));
  c->tile = OCG_TILE_AUTO;
  c->swizzle = 1;
  c->mode = OCG_MODE_FUSED;
  c->fault_skip_slab = -1;
  c->transfer = OCG_TRANSFER_AUTO;
  c->xcd_remap = 1;
}

int ocg_create(int device, ocg_handle* out) {
  if (!out) return OCG_ERR_INVALID_ARG;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return OCG_ERR_NO_DEVICE;
  if (device < 0 || device >= n) return OCG_ERR_NO_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return OCG_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return OCG_ERR_UNSUPPORTED_SHAPE;
  ocg_handle h = new (std::nothrow) ocg_handle_s();
  if (!h) return OCG_ERR_HIP;
  h->device = device;
  h->cus = prop.multiProcessorCount;
  // the side stream and its events live on `device`
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) prev = -1;
  bool ok = hipSetDevice(device) == hipSuccess && hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&h->join, hipEventDisableTiming) == hipSuccess &&
            noalloc_scratch_setup(device, &h->scratch) == hipSuccess;
  if (prev >= 0) (void)hipSetDevice(prev);
  if (!ok) {
    ocg_destroy(h);
    return OCG_ERR_HIP;
  }
  *out = h;
  return OCG_OK;
}

void ocg_destroy(ocg_handle h) {
  if (!h) return;
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->side) (void)hipStreamDestroy(h->side);
  delete h;
}

size_t ocg_workspace_bytes(ocg_handle h, int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk) {
  return ocg_workspace_bytes_for(h, op, R, m, K, N, E, topk, nullptr);
}

size_t ocg_workspace_bytes_for(ocg_handle h, int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk,
                               const ocg_config* cfgp) {
  if (op < 0 || op > 4) return 0;
  if (op == OCG_OP_AG_ATTENTION) return attn_shape_ok(R, m, K, N) ? layout(op, R, m, 0, 0, 0, 0).total : 0;
  if (op == OCG_OP_MOE_COMBINE_RS) return combine_shape_ok(R, m, N, topk) ? layout(op, R, m, 0, N, 0, topk).total : 0;
  if (op == OCG_OP_GEMM_RS) {
    if (R < 1 || R > kMaxRanks || m < R || m % R) return 0;
    if (!shape_ok(1, m, K, N)) return 0;
  } else if (!shape_ok(R, m, K, N)) {
    return 0;
  }
  if (op == OCG_OP_AG_GROUPED_GEMM &&
      (E < 1 || E > kMaxExperts || topk < 1 || topk > kMaxTopk || topk > E || (int64_t)R * m * topk > kMaxRouteSlots))
    return 0;
  if (op == OCG_OP_AG_GEMM) {
    // with room for split-K sums where the plan splits
    AgSetup su;
    if (ag_setup(h, R, 0, m, K, N, cfg_or_default(cfgp), &su) != OCG_OK) return 0;
    return su.L.total;
  }
  return layout(op, R, m, K, N, E, topk).total;
}

int ocg_workspace_init(ocg_handle h, void* ws, size_t bytes, void* stream) {
  if (!h || !ws || bytes < sizeof(WsHeader) || (bytes & 3) || !aligned16(ws)) return OCG_ERR_INVALID_ARG;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  hipError_t e = launch_fill_u32((uint32_t*)ws, bytes / 4, 0u, 0, (hipStream_t)stream);
  return e == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

// The AG-GEMM plan of a call: tile, slabs, K-slabs and transfer (resolve),
// the rounds of tiles of the persistent grid (copy phases), the copy tickets
// the GEMM kernel runs itself, and the two grids (producer 0 unless SIDE).
int ocg_ag_gemm(ocg_handle h, const void* const* a_chunks, int R, int local_rank, int64_t m, int64_t K,
                const void* b, int64_t N, void* a_gathered, void* c, void* ws, size_t ws_bytes,
                const ocg_config* cfgp, void* stream) {
  if (!h || !a_chunks || !b || !a_gathered || !c || !ws) return OCG_ERR_INVALID_ARG;
  if (!shape_ok(R, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  for (int r = 0; r < R; ++r)
    if (!a_chunks[r] || !aligned16(a_chunks[r])) return OCG_ERR_INVALID_ARG;
  if (!aligned16(b) || !aligned16(a_gathered) || !aligned16(c) || !aligned16(ws)) return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  if (cfg.mode < 0 || cfg.mode > 2) return OCG_ERR_INVALID_ARG;
  if (ws_bytes < layout(OCG_OP_AG_GEMM, R, m, K, N, 0, 0).total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  AgSetup su;
  int st = ag_setup(h, R, local_rank, m, K, N, cfg, &su, ws_bytes);
  if (st) return st;
  const WsLayout& L = su.L;
  if (ws_bytes < L.total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  AgArgs a{};
  for (int r = 0; r < R; ++r) a.chunks[r] = (const uint16_t*)a_chunks[r];
  a.b = (const uint16_t*)b;
  a.a_gathered = (uint16_t*)a_gathered;
  a.c = (uint16_t*)c;
  a.slab_cnt = (uint32_t*)((char*)ws + L.slab_cnt);
  a.slab_flag = (uint32_t*)((char*)ws + L.slab_flag);
  a.sk_cnt = (uint32_t*)((char*)ws + L.sk_cnt);
  a.sk_flag = (uint32_t*)((char*)ws + L.sk_flag);
  a.sk_part = (float*)((char*)ws + L.sk_part);
  a.plan = su.plan;
  if (a.plan.R * a.plan.bpr * a.plan.nks > L.max_slabs) return OCG_ERR_INVALID_ARG;
  a.cm = make_common(ws, cfg);
  hipStream_t s = (hipStream_t)stream;
  if (su.pgrid == 0)
    return launch_ag_gemm(a, su.rv.tile, su.ggrid < 1 ? 1 : su.ggrid, s) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
  // SIDE: the producer on the side stream, then the GEMM kernel on the
  // caller's stream, both after the caller's earlier work; the caller's
  // stream then waits for the producer. The two kernels start a few
  // microseconds apart, either one first; with the producer submitted first,
  // a tool that runs dispatches one at a time (counter collection) mostly
  // runs the copies before the tiles that wait on them (the other way round
  // the tiles wait out their bound). The last workgroup of either kernel
  // resets the workspace counters.
  a.cm.total_wgs = su.ggrid + su.pgrid;
  if (hipEventRecord(h->fork, s) != hipSuccess || hipStreamWaitEvent(h->side, h->fork, 0) != hipSuccess)
    return OCG_ERR_HIP;
  if (launch_ag_side_copy(a, su.pgrid, h->side) != hipSuccess) return OCG_ERR_HIP;
  if (su.ggrid > 0 && launch_ag_gemm(a, su.rv.tile, su.ggrid, s) != hipSuccess) return OCG_ERR_HIP;
  if (hipEventRecord(h->join, h->side) != hipSuccess || hipStreamWaitEvent(s, h->join, 0) != hipSuccess)
    return OCG_ERR_HIP;
  return OCG_OK;
}

int ocg_ag_gemm_noalloc(ocg_handle h, const void* const* a_chunks, int R, int local_rank, int64_t m, int64_t K,
                        const void* b, int64_t N, void* a_gathered, void* c, const ocg_config* cfg, void* stream) {
  if (!h || !h->scratch) return OCG_ERR_INVALID_ARG;
  if (!shape_ok(R, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  // the shape's workspace must fit the fixed scratch (nothing is allocated)
  if (layout(OCG_OP_AG_GEMM, R, m, K, N, 0, 0).total > kNoAllocScratchBytes) return OCG_ERR_WORKSPACE_TOO_SMALL;
  return ocg_ag_gemm(h, a_chunks, R, local_rank, m, K, b, N, a_gathered, c, h->scratch, kNoAllocScratchBytes, cfg,
                     stream);
}

}  // extern "C"

namespace {

// Shared part of the pull and push GEMM-ReduceScatter calls: checks, plan,
// launch. `fill` sets the mode-specific fields of the arguments.
template <class Fill>
int gemm_rs_call(ocg_handle h, const void* A, const void* B, int64_t M, int64_t K, int64_t N, int R, int local_rank,
                 void* out, void* ws, size_t ws_bytes, const ocg_config* cfgp, void* stream, bool push, Fill fill) {
  if (!h || !A || !B || !out || !ws) return OCG_ERR_INVALID_ARG;
  if (R < 1 || R > kMaxRanks || M < R || M % R) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (!shape_ok(1, M, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(out) || !aligned16(ws)) return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  WsLayout L = layout(OCG_OP_GEMM_RS, R, M, K, N, 0, 0);
  if (ws_bytes < L.total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  Resolved rv;
  int st = resolve(OCG_OP_GEMM_RS, R, M, K, N, 0, 0, cfg, h->cus, &rv);
  if (st) return st;
  RsArgs a{};
  a.a = (const uint16_t*)A;
  a.b = (const uint16_t*)B;
  a.out = (uint16_t*)out;
  a.tile_flag = (uint32_t*)((char*)ws + L.rs_flag);
  a.plan = make_rs_plan(R, local_rank, (int)M, (int)K, (int)N, rv.BM, rv.BN, reduce_rows(M, R, N, h->cus),
                        cfg.swizzle ? 1 : 0, push ? 1 : 0);
  if (a.plan.n_tiles > L.max_rs_tiles) return OCG_ERR_INVALID_ARG;
  a.rs_sum = (uint32_t*)((char*)ws + L.rs_sum);
  a.local_rb0 = (local_rank * a.plan.blk) / rv.BM;
  a.local_nrb = cdiv(a.plan.blk, rv.BM);
  a.tpb = a.local_nrb * a.plan.n_cb;
  a.push = push ? 1 : 0;
  st = fill(a, cfg, rv);
  if (st) return st;
  a.cm = make_common(ws, cfg);
  int grid = grid_for(h, OCG_OP_GEMM_RS, rv.tile, a.plan.n_tiles + a.plan.n_red, a.plan.n_tiles, cfg);
  return launch_gemm_rs(a, rv.tile, grid, (hipStream_t)stream) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

}  // namespace

extern "C" {

int ocg_gemm_rs(ocg_handle h, const void* A, const void* B, int64_t M, int64_t K, int64_t N, int R, int local_rank,
                const void* const* peer_partials, void* partial, void* out, void* ws, size_t ws_bytes,
                const ocg_config* cfgp, void* stream) {
  if (!peer_partials || !partial) return OCG_ERR_INVALID_ARG;
  if (R >= 1 && R <= kMaxRanks && local_rank >= 0 && local_rank < R)
    for (int s = 0; s < R; ++s)
      if (s != local_rank && (!peer_partials[s] || !aligned16(peer_partials[s]))) return OCG_ERR_INVALID_ARG;
  if (!aligned16(partial)) return OCG_ERR_INVALID_ARG;
  return gemm_rs_call(h, A, B, M, K, N, R, local_rank, out, ws, ws_bytes, cfgp, stream, false,
                      [&](RsArgs& a, const ocg_config& cfg, const Resolved& rv) {
                        for (int s = 0; s < R; ++s) {
                          a.dst[s] = (uint16_t*)partial;
                          a.src[s] = (s == local_rank) ? (const uint16_t*)partial : (const uint16_t*)peer_partials[s];
                        }
                        a.peer_flags = cfg.peer_flags;
                        a.peer_flag_value = cfg.peer_flag_value;
                        if (cfg.peer_flags && a.plan.blk % rv.BM) return OCG_ERR_UNSUPPORTED_SHAPE;
                        return OCG_OK;
                      });
}

int ocg_gemm_rs_push(ocg_handle h, const void* A, const void* B, int64_t M, int64_t K, int64_t N, int R,
                     int local_rank, void* const* recv, uint32_t* const* recv_flags, uint32_t flag_value, void* out,
                     void* ws, size_t ws_bytes, const ocg_config* cfgp, void* stream) {
  if (!recv || !recv_flags) return OCG_ERR_INVALID_ARG;
  if (R < 1 || R > kMaxRanks) return OCG_ERR_UNSUPPORTED_SHAPE;
  for (int s = 0; s < R; ++s)
    if (!recv[s] || !aligned16(recv[s]) || !recv_flags[s] || ((uintptr_t)recv_flags[s] & 3)) return OCG_ERR_INVALID_ARG;
  return gemm_rs_call(h, A, B, M, K, N, R, local_rank, out, ws, ws_bytes, cfgp, stream, true,
                      [&](RsArgs& a, const ocg_config& cfg, const Resolved& rv) {
                        (void)cfg;
                        if (a.plan.blk % rv.BM) return OCG_ERR_UNSUPPORTED_SHAPE;   // a tile in one row block
                        const int64_t blk = a.plan.blk;
                        for (int s = 0; s < R; ++s) {
                          // rank s's slot `local` holds rows [s*blk, (s+1)*blk) of our partial:
                          // global row r -> slot row r - s*blk
                          a.dst[s] = (uint16_t*)recv[s] + (local_rank - s) * blk * N;
                          // our slot s holds rank s's rows of our block: row r -> r - local*blk
                          a.src[s] = (const uint16_t*)recv[local_rank] + (s - local_rank) * blk * N;
                          a.rflag[s] = recv_flags[s];
                        }
                        a.flag_value = flag_value;
                        return OCG_OK;
                      });
}

}  // extern "C"

namespace {

// AllGather + routing + grouped GEMM, and (layer != NULL) the TopK-Reduce +
// ReduceScatter tasks of the layer chain in the same persistent kernel.
struct LayerOut {
  const void* const* peer_partials;
  void* partial;
  void* out;
};

int grouped_call(ocg_handle h, const void* const* a_chunks, int R, int local_rank, int64_t m, int64_t K,
                 const float* logits, int E, int topk, const void* w, int64_t N, void* a_gathered, int32_t* topk_ids,
                 float* topk_w, int32_t* perm, int32_t* expert_offsets, void* out, void* ws, size_t ws_bytes,
                 const ocg_config* cfgp, void* stream, const LayerOut* layer) {
  if (!h || !a_chunks || !logits || !w || !a_gathered || !topk_ids || !topk_w || !out || !ws)
    return OCG_ERR_INVALID_ARG;
  if (!shape_ok(R, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (E < 1 || E > kMaxExperts || topk < 1 || topk > kMaxTopk || topk > E) return OCG_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)R * m * topk > kMaxRouteSlots) return OCG_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)E * K * N * 2 > (int64_t)1 << 40) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  for (int r = 0; r < R; ++r)
    if (!a_chunks[r] || !aligned16(a_chunks[r])) return OCG_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(a_gathered) || !aligned16(out) || !aligned16(ws)) return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  if (cfg.mode < 0 || cfg.mode > 2) return OCG_ERR_INVALID_ARG;
  WsLayout L = layout(OCG_OP_AG_GROUPED_GEMM, R, m, K, N, E, topk);
  if (ws_bytes < L.total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  Resolved rv;
  int st = resolve(OCG_OP_AG_GROUPED_GEMM, R, m, K, N, E, topk, cfg, h->cus, &rv);
  if (st) return st;
  int32_t* perm_buf = perm ? perm : (int32_t*)((char*)ws + L.moe_perm);
  MoeArgs a{};
  for (int r = 0; r < R; ++r) a.chunks[r] = (const uint16_t*)a_chunks[r];
  a.w = (const uint16_t*)w;
  a.a_gathered = (uint16_t*)a_gathered;
  a.out = (uint16_t*)out;
  a.perm = perm_buf;
  a.lut = (const int32_t*)((char*)ws + L.moe_lut);
  a.slab_cnt = (uint32_t*)((char*)ws + L.slab_cnt);
  a.slab_flag = (uint32_t*)((char*)ws + L.slab_flag);
  a.topk = topk;
  a.E = E;
  a.plan = make_ag_plan(R, local_rank, (int)m, (int)K, (int)N, rv.BM, rv.BN, rv.S, rv.CT, cfg.swizzle ? 1 : 0,
                        cfg.mode);
  if (a.plan.R * a.plan.bpr > L.max_slabs) return OCG_ERR_INVALID_ARG;
  a.cm = make_common(ws, cfg);
  RouteArgs r{};
  r.logits = logits;
  r.topk_ids = topk_ids;
  r.topk_w = topk_w;
  r.perm = perm_buf;
  r.offsets = (int32_t*)((char*)ws + L.moe_off);
  r.user_offsets = expert_offsets;
  r.lut = (int32_t*)((char*)ws + L.moe_lut);
  r.blk_cnt = (int32_t*)((char*)ws + L.moe_bcnt);
  r.inv = (int32_t*)((char*)ws + L.moe_inv);
  r.lut_base = (int32_t*)((char*)ws + L.moe_lbase);
  r.hdr = (WsHeader*)ws;
  r.T = (int)(R * m);
  r.E = E;
  r.topk = topk;
  r.BM = rv.BM;
  r.n_cb = cdiv((int)N, rv.BN);
  r.max_tiles = L.max_moe_tiles;
  if (layer) {
    const int64_t T = (int64_t)R * m;
    if (!combine_shape_ok(R, m, N, topk) || T * topk * N * 2 >= ((int64_t)1 << 31)) return OCG_ERR_UNSUPPORTED_SHAPE;
    a.combine = 1;
    a.BM = rv.BM;
    a.n_cb = cdiv((int)N, rv.BN);
    a.tflag = (uint32_t*)((char*)ws + L.moe_tflag);
    a.inv = r.inv;
    a.lut_base = r.lut_base;
    a.offsets = r.offsets;
    a.topk_ids = topk_ids;
    CombArgs& c = a.comb;
    c.y = (const uint16_t*)out;
    c.w = topk_w;
    for (int s = 0; s < R; ++s)
      c.peers[s] = (s == local_rank) ? nullptr : (const uint16_t*)layer->peer_partials[s];
    c.partial = (uint16_t*)layer->partial;
    c.out = (uint16_t*)layer->out;
    c.topk = topk;
    combine_rows(R, m, topk, h->cus, &c.CRL, &c.CR);
    c.n_lt = cdiv((int)m, c.CRL);
    c.n_comb = c.n_lt + cdiv((int)(T - m), c.CR);
    c.R = R;
    c.local = local_rank;
    c.m = (int)m;
    c.T = (int)T;
    c.N = (int)N;
    c.max_tiles = L.max_moe_tiles;
  }
  int grid = grid_for(h, OCG_OP_AG_GROUPED_GEMM, rv.tile, a.plan.n_copy + L.max_moe_tiles, L.max_moe_tiles, cfg);
  return launch_moe(r, a, rv.tile, grid, (hipStream_t)stream) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

}  // namespace

extern "C" {

int ocg_ag_grouped_gemm(ocg_handle h, const void* const* a_chunks, int R, int local_rank, int64_t m, int64_t K,
                        const float* logits, int E, int topk, const void* w, int64_t N, void* a_gathered,
                        int32_t* topk_ids, float* topk_w, int32_t* perm, int32_t* expert_offsets, void* out,
                        void* ws, size_t ws_bytes, const ocg_config* cfgp, void* stream) {
  return grouped_call(h, a_chunks, R, local_rank, m, K, logits, E, topk, w, N, a_gathered, topk_ids, topk_w, perm,
                      expert_offsets, out, ws, ws_bytes, cfgp, stream, nullptr);
}

int ocg_ag_moe_layer(ocg_handle h, const void* const* a_chunks, int R, int local_rank, int64_t m, int64_t K,
                     const float* logits, int E, int topk, const void* w, int64_t N,
                     const void* const* peer_partials, void* a_gathered, int32_t* topk_ids, float* topk_w,
                     int32_t* perm, int32_t* expert_offsets, void* y, void* partial, void* out, void* ws,
                     size_t ws_bytes, const ocg_config* cfgp, void* stream) {
  if (!peer_partials || !partial || !out || !y) return OCG_ERR_INVALID_ARG;
  if (R < 1 || R > kMaxRanks || local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  for (int s = 0; s < R; ++s)
    if (s != local_rank && (!peer_partials[s] || !aligned16(peer_partials[s]))) return OCG_ERR_INVALID_ARG;
  if (!aligned16(partial) || !aligned16(out) || ((uintptr_t)topk_w & 3)) return OCG_ERR_INVALID_ARG;
  LayerOut lo{peer_partials, partial, out};
  return grouped_call(h, a_chunks, R, local_rank, m, K, logits, E, topk, w, N, a_gathered, topk_ids, topk_w, perm,
                      expert_offsets, y, ws, ws_bytes, cfgp, stream, &lo);
}

int ocg_signal(uint32_t* flags, int count, uint32_t value, void* stream) {
  if (!flags || count < 0 || ((uintptr_t)flags & 3)) return OCG_ERR_INVALID_ARG;
  return launch_fill_u32(flags, (size_t)count, value, 1, (hipStream_t)stream) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

int ocg_moe_combine_rs(ocg_handle h, const void* y, const float* topk_w, int R, int local_rank, int64_t m,
                       int64_t N, int topk, const void* const* peer_partials, void* partial, void* out, void* ws,
                       size_t ws_bytes, const ocg_config* cfgp, void* stream) {
  if (!h || !y || !topk_w || !peer_partials || !partial || !out || !ws) return OCG_ERR_INVALID_ARG;
  if (!combine_shape_ok(R, m, N, topk)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  for (int s = 0; s < R; ++s)
    if (s != local_rank && (!peer_partials[s] || !aligned16(peer_partials[s]))) return OCG_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(partial) || !aligned16(out) || !aligned16(ws) || ((uintptr_t)topk_w & 3))
    return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  WsLayout L = layout(OCG_OP_MOE_COMBINE_RS, R, m, 0, N, 0, topk);
  if (ws_bytes < L.total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  const int64_t T = (int64_t)R * m;
  CombArgs a{};
  a.y = (const uint16_t*)y;
  a.w = topk_w;
  for (int s = 0; s < R; ++s) a.peers[s] = (s == local_rank) ? nullptr : (const uint16_t*)peer_partials[s];
  a.partial = (uint16_t*)partial;
  a.out = (uint16_t*)out;
  a.topk = topk;
  combine_rows(R, m, topk, h->cus, &a.CRL, &a.CR);
  a.n_lt = cdiv((int)m, a.CRL);
  a.n_comb = a.n_lt + cdiv((int)(T - m), a.CR);
  a.R = R;
  a.local = local_rank;
  a.m = (int)m;
  a.T = (int)T;
  a.N = (int)N;
  a.cm = make_common(ws, cfg);
  int grid = cfg.grid > 0 ? cfg.grid : 2 * h->cus;   // no LDS: two workgroups per CU
  if (grid > a.n_comb) grid = a.n_comb;
  return launch_moe_combine_rs(a, grid, (hipStream_t)stream) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

int ocg_ag_attention(ocg_handle h, const void* q, const void* const* k_chunks, const void* const* v_chunks, int R,
                     int local_rank, int64_t m, int64_t Hq, int64_t Hkv, int64_t d, void* k_gathered,
                     void* v_gathered, void* out, void* ws, size_t ws_bytes, const ocg_config* cfgp, void* stream) {
  if (!h || !q || !k_chunks || !v_chunks || !k_gathered || !v_gathered || !out || !ws) return OCG_ERR_INVALID_ARG;
  if (d != kAttnD || !attn_shape_ok(R, m, Hq, Hkv)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  for (int r = 0; r < R; ++r)
    if (!k_chunks[r] || !v_chunks[r] || !aligned16(k_chunks[r]) || !aligned16(v_chunks[r])) return OCG_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_gathered) || !aligned16(v_gathered) || !aligned16(out) || !aligned16(ws))
    return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  if (cfg.mode < 0 || cfg.mode > 2) return OCG_ERR_INVALID_ARG;
  WsLayout L = layout(OCG_OP_AG_ATTENTION, R, m, 0, 0, 0, 0);
  if (ws_bytes < L.total) return OCG_ERR_WORKSPACE_TOO_SMALL;
  if (!device_matches(h)) return OCG_ERR_INVALID_ARG;
  int S, CT;
  int st = resolve_attn(m, Hkv, cfg, &S, &CT);
  if (st) return st;
  AttnArgs a{};
  a.q = (const uint16_t*)q;
  for (int r = 0; r < R; ++r) {
    a.k_chunks[r] = (const uint16_t*)k_chunks[r];
    a.v_chunks[r] = (const uint16_t*)v_chunks[r];
  }
  a.k_gathered = (uint16_t*)k_gathered;
  a.v_gathered = (uint16_t*)v_gathered;
  a.out = (uint16_t*)out;
  a.slab_cnt = (uint32_t*)((char*)ws + L.slab_cnt);
  a.slab_flag = (uint32_t*)((char*)ws + L.slab_flag);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  a.plan = make_attn_plan(R, local_rank, (int)m, (int)Hq, (int)Hkv, S, CT, cfg.swizzle ? 1 : 0, cfg.mode);
  if (a.plan.cp.R * a.plan.cp.bpr > L.max_slabs) return OCG_ERR_INVALID_ARG;
  a.cm = make_common(ws, cfg);
  int grid = cfg.grid;
  if (grid <= 0) {
    if (h->resident_attn == 0) h->resident_attn = resident_attention();
    grid = h->resident_attn * h->cus;
    const int tasks = a.plan.n_copy + a.plan.n_tiles;
    if (tasks < grid) grid = tasks;
    if (grid < 1) grid = 1;
  }
  return launch_ag_attention(a, grid, (hipStream_t)stream) == hipSuccess ? OCG_OK : OCG_ERR_HIP;
}

int ocg_check(ocg_handle h, void* ws) {
  if (!h || !ws) return OCG_ERR_INVALID_ARG;
  WsHeader* hdr = (WsHeader*)ws;
  uint32_t err = 0;
  if (hipMemcpy(&err, &hdr->error, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return OCG_ERR_HIP;
  if (err) {
    uint32_t zero = 0;
    if (hipMemcpy(&hdr->error, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return OCG_ERR_HIP;
    return OCG_ERR_TIMEOUT;
  }
  return OCG_OK;
}

const char* ocg_status_string(int s) {
  switch (s) {
    case OCG_OK: return "ok";
    case OCG_ERR_INVALID_ARG: return "invalid argument";
    case OCG_ERR_UNSUPPORTED_SHAPE: return "unsupported shape or device";
    case OCG_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case OCG_ERR_HIP: return "HIP runtime error";
    case OCG_ERR_TIMEOUT: return "a flag wait timed out";
    case OCG_ERR_NO_DEVICE: return "no such device";
  }
  return "unknown status";
}

int ocg_plan_info(ocg_handle h, int op, int R, int local_rank, int64_t m, int64_t K, int64_t N, int E, int topk,
                  const ocg_config* cfgp, int64_t out[8]) {
  if (!out || op < 0 || op > 4) return OCG_ERR_INVALID_ARG;
  const int cus = h ? h->cus : 256;   // no handle: a full MI355X
  if (op == OCG_OP_AG_ATTENTION) {
    if (!attn_shape_ok(R, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
    if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
    ocg_config cfg = cfg_or_default(cfgp);
    int S, CT;
    int st = resolve_attn(m, N, cfg, &S, &CT);
    if (st) return st;
    AttnPlan p = make_attn_plan(R, local_rank, (int)m, (int)K, (int)N, S, CT, cfg.swizzle ? 1 : 0, cfg.mode);
    out[0] = -1;
    out[1] = kAttnRows;
    out[2] = kAttnKB;
    out[3] = S;
    out[4] = CT;
    out[5] = p.n_copy;
    out[6] = p.n_tiles;
    out[7] = (int64_t)R * p.cp.bpr;
    return OCG_OK;
  }
  if (op == OCG_OP_MOE_COMBINE_RS) {
    if (!combine_shape_ok(R, m, N, topk)) return OCG_ERR_UNSUPPORTED_SHAPE;
    if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
    const int64_t T = (int64_t)R * m;
    int cr, crl;
    combine_rows(R, m, topk, cus, &crl, &cr);
    const int n_lt = cdiv((int)m, crl);
    out[0] = -1;
    out[1] = out[2] = out[7] = 0;
    out[3] = cr;
    out[4] = crl;
    out[5] = n_lt + cdiv((int)(T - m), cr);
    out[6] = n_lt;
    return OCG_OK;
  }
  if (op == OCG_OP_GEMM_RS) {
    if (R < 1 || R > kMaxRanks || m < R || m % R || !shape_ok(1, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  } else if (!shape_ok(R, m, K, N)) {
    return OCG_ERR_UNSUPPORTED_SHAPE;
  }
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  Resolved rv;
  AgSetup su;
  if (op == OCG_OP_AG_GEMM) {
    int st = ag_setup(h, R, local_rank, m, K, N, cfg, &su);
    if (st) return st;
    rv = su.rv;
  } else {
    int st = resolve(op, R, m, K, N, E, topk, cfg, cus, &rv);
    if (st) return st;
  }
  out[0] = rv.tile;
  out[1] = rv.BM;
  out[2] = rv.BN;
  out[3] = rv.S;
  out[4] = rv.CT;
  if (op == OCG_OP_GEMM_RS) {
    RsPlan p = make_rs_plan(R, local_rank, (int)m, (int)K, (int)N, rv.BM, rv.BN, reduce_rows(m, R, N, cus), cfg.swizzle);
    out[5] = p.n_red;
    out[6] = p.n_tiles;
    out[7] = p.RR;
  } else if (op == OCG_OP_AG_GEMM) {
    out[5] = su.plan.n_copy;
    out[6] = su.plan.n_tiles;
    out[7] = (int64_t)R * su.plan.bpr * su.plan.nks;
  } else {
    AgPlan p = make_ag_plan(R, local_rank, (int)m, (int)K, (int)N, rv.BM, rv.BN, rv.S, rv.CT, cfg.swizzle,
                            cfg.mode);
    out[5] = p.n_copy;
    out[6] = p.n_tiles;
    out[7] = (int64_t)R * p.bpr;
  }
  return OCG_OK;
}

int ocg_plan_ag(ocg_handle h, int R, int local_rank, int64_t m, int64_t K, int64_t N, const ocg_config* cfgp,
                int64_t out[8]) {
  if (!out) return OCG_ERR_INVALID_ARG;
  if (!shape_ok(R, m, K, N)) return OCG_ERR_UNSUPPORTED_SHAPE;
  if (local_rank < 0 || local_rank >= R) return OCG_ERR_INVALID_ARG;
  ocg_config cfg = cfg_or_default(cfgp);
  AgSetup su;
  int st = ag_setup(h, R, local_rank, m, K, N, cfg, &su);
  if (st) return st;
  for (int i = 0; i < 8; ++i) out[i] = 0;
  out[0] = su.plan.KS;
  out[1] = su.plan.nks;
  out[2] = su.rv.transfer;
  out[3] = su.ggrid;
  out[4] = su.pgrid;
  out[5] = su.plan.n_inline;
  out[6] = su.plan.rpr;
  out[7] = su.plan.sk;
  return OCG_OK;
}

int ocg_plan_task(ocg_handle h, int op, int R, int local_rank, int64_t m, int64_t K, int64_t N, const ocg_config* cfgp,
                  int64_t ticket, int64_t desc[8]) {
  if (!desc) return OCG_ERR_INVALID_ARG;
  for (int i = 0; i < 8; ++i) desc[i] = -1;
  desc[0] = 0;
  int64_t info[8];
  int st = ocg_plan_info(h, op, R, local_rank, m, K, N, 0, 0, cfgp, info);
  if (st) return st;
  ocg_config cfg = cfg_or_default(cfgp);
  if (op == OCG_OP_AG_ATTENTION) {
    AttnPlan p = make_attn_plan(R, local_rank, (int)m, (int)K, (int)N, (int)info[3], (int)info[4], cfg.swizzle ? 1 : 0,
                                cfg.mode);
    if (ticket < 0 || ticket >= p.n_copy + p.n_tiles) return OCG_OK;
    if (ticket < p.n_copy) {
      CopyDesc d = copy_desc(p.cp, (int)(ticket >> 1));
      desc[0] = 1;
      desc[1] = d.chunk;
      desc[2] = d.piece;
      desc[3] = d.row0;
      desc[4] = d.row1;
      desc[5] = d.slab;
      desc[6] = ticket & 1;
      return OCG_OK;
    }
    const int v = (int)(ticket - p.n_copy);
    desc[0] = 7;
    desc[1] = v / p.n_rb;
    desc[2] = v % p.n_rb;
    desc[3] = p.cp.mode == 0 ? (int64_t)(R - 1) * p.cp.bpr : 0;
    int q, t;
    tile_queue(v, &q, &t);
    desc[4] = q;
    desc[5] = t;
    return OCG_OK;
  }
  if (op == OCG_OP_GEMM_RS) {
    RsPlan p = make_rs_plan(R, local_rank, (int)m, (int)K, (int)N, (int)info[1], (int)info[2], (int)info[7],
                            cfg.swizzle);
    if (ticket < 0 || ticket >= p.n_tiles + p.n_red) return OCG_OK;
    if (ticket < p.n_tiles) {
      int rb, cb;
      tile_of(p.n_rb, p.n_cb, p.rb0, (int)ticket, &rb, &cb);
      desc[0] = 3;
      desc[1] = rb;
      desc[2] = cb;
      desc[3] = rs_tile_touches_local(p, rb) ? 1 : 0;
      int q, t;
      tile_queue((int)ticket, &q, &t);
      desc[4] = q;
      desc[5] = t;
    } else {
      int r0, r1;
      rs_strip(p, (int)(ticket - p.n_tiles), &r0, &r1);
      desc[0] = 5;
      desc[1] = r0;
      desc[2] = r1;
    }
    return OCG_OK;
  }
  AgPlan p;
  if (op == OCG_OP_AG_GEMM) {
    AgSetup su;
    st = ag_setup(h, R, local_rank, m, K, N, cfg, &su);
    if (st) return st;
    p = su.plan;
  } else {
    p = make_ag_plan(R, local_rank, (int)m, (int)K, (int)N, (int)info[1], (int)info[2], (int)info[3], (int)info[4],
                     cfg.swizzle, cfg.mode);
  }
  if (ticket < 0 || ticket >= p.n_copy + (op == OCG_OP_AG_GEMM ? p.n_tiles * p.sk : 0)) return OCG_OK;
  if (ticket < p.n_copy) {
    CopyDesc d = copy_desc(p, (int)ticket);
    desc[0] = 1;
    desc[1] = d.chunk;
    desc[2] = d.piece;
    desc[3] = d.row0;
    desc[4] = d.row1;
    desc[5] = d.slab;
    desc[6] = d.kslab;
    return OCG_OK;
  }
  int rb, cb;
  const int u = (int)(ticket - p.n_copy);
  tile_of(p.n_rb, p.n_cb, p.rb0, u / p.sk, &rb, &cb);
  desc[0] = 2;
  desc[1] = rb;
  desc[2] = cb;
  int r0 = rb * p.BM, r1 = r0 + p.BM < p.M ? r0 + p.BM : p.M;
  int k = 0;
  int n = for_each_dep_slab(p.m, p.S, p.bpr, p.local, r0, r1, [&](int s) {
    if (k < 3) desc[4 + k] = s;
    ++k;
  });
  desc[3] = p.mode == 0 ? n : 0;
  if (p.mode != 0)
    for (int i = 4; i < 7; ++i) desc[i] = -1;
  desc[7] = u % p.sk;
  return OCG_OK;
}

}  // extern "C"
