// Internal launch parameters shared by the C-ABI layer (api.cpp) and the
// kernels (kernels.hip). Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ocg.h"
#include "sched.h"

namespace ocg {

constexpr int kMaxRanks = 16;
constexpr int kThreads = 256;         // every persistent kernel: 4 waves of 64
constexpr int kRouteBlock = 64;       // tokens per routing block
constexpr int kMaxRouteSlots = 16384; // token slots (T * topk) per call
constexpr int kMaxExperts = 64;
constexpr int kMaxTopk = 4;
constexpr int kCombineChunks = 8;        // 16-byte chunks per thread and round of a TopK-Reduce task
constexpr int kCombineChunksLocal = 2;   // the same for the local block's rows (R + topk loads each)
constexpr int kMinSlabRows = 16;
// grouped GEMM presets: 128x224, 256x224, 288x224, 320x224 (the smallest is
// used to size the tile lookup table)
constexpr int kMoeTileSmall = OCG_TILE_128x224;
inline bool moe_tile_ok(int t) {
  return t == OCG_TILE_128x224 || t == OCG_TILE_256x224 || t == OCG_TILE_288x224 || t == OCG_TILE_320x224;
}

// Workspace header (the first 1536 bytes of every workspace).
// Every counter the workgroups update sits in a 128-byte line of its own:
// agent-scope atomics on one line are served one after the other, and with
// all of them in one line the 224-256 workgroups of a launch took their
// first ticket over ~10 us (the last XCD's tiles started that late).
constexpr int kHdrWords = 32;    // uint32 words per 128-byte line
struct WsHeader {
  uint32_t ticket;               // next ticket of the running persistent kernel
  uint32_t pad_ticket[kHdrWords - 1];
  uint32_t done;                 // workgroups (of every kernel of the call) that finished
  uint32_t pad_done[kHdrWords - 1];
  uint32_t side_ticket;          // next copy ticket of the side producer kernel
  uint32_t pad_side[kHdrWords - 1];
  uint32_t epoch;                // epoch of the last completed call (flags carry epochs)
  uint32_t error;                // bit 0: a flag wait timed out
  uint32_t n_tiles;              // MoE: grouped tiles of the current routing
  uint32_t pad_misc[kHdrWords - 3];
  uint32_t xtick[8 * kHdrWords]; // next ticket of XCD queue q at xtick[q * kHdrWords]
};
static_assert(sizeof(WsHeader) == 12 * 128, "header is twelve 128-byte lines");

// Byte offsets of the workspace sections for one call shape.
struct WsLayout {
  size_t slab_cnt, slab_flag, rs_flag, rs_sum, moe_off, moe_lut, moe_perm, moe_bcnt, moe_inv, moe_lbase, moe_tflag;
  size_t sk_cnt, sk_flag, sk_part;   // AG-GEMM split K: per tile arrivals, flag, fp32 half (0 when unsplit)
  size_t total;
  int max_slabs, max_rs_tiles, max_moe_tiles;
};

struct Common {
  WsHeader* hdr;
  uint64_t timeout_ticks;   // bound on each wait, 100 MHz ticks
  ocg_trace_rec* trace;
  uint32_t trace_cap;
  int fault_skip_slab;      // flag index never published (test hook), -1 = off
  uint32_t copy_delay;      // s_sleep 127 rounds before each copy task (test hook)
  int xcd_remap;            // 1 = per-XCD tile queues, 0 = one queue
  int total_wgs;            // workgroups of every kernel of the call (finish counter)
};

struct AgArgs {
  const uint16_t* chunks[kMaxRanks];
  const uint16_t* b;
  uint16_t* a_gathered;
  uint16_t* c;
  uint32_t* slab_cnt;           // [flags]: copy tasks done per (slab, K-slab)
  uint32_t* slab_flag;          // [flags]: epoch once the (slab, K-slab) has landed
  uint32_t* sk_cnt;             // split K, [tiles]: halves finished (back to 0 by the second)
  uint32_t* sk_flag;            // split K, [tiles]: epoch once the first half's sums are stored
  float* sk_part;               // split K, [tiles][BM * BN]: the first half's fp32 sums
  AgPlan plan;                  // copy tickets >= plan.n_inline: the side producer's
  Common cm;
};

// GEMM-ReduceScatter. Pull (push = 0): tiles store the partial into
// `partial` and notify tile_flag[rb * n_cb + cb] = epoch; the reduce reads
// every rank's partial where it lives. Push (push = 1): the tile of row
// block s goes straight to rank s's receive buffer, slot `local`, and sets
// that rank's flag rflag[s][local * tpb + t] = flag_value (t: the tile
// within the block); the reduce reads our own receive buffer's R slots.
// Addressing by global row r and column c, for both:
//   tile store      dst[s] + r * N + c      (s = block of r)
//   reduce operand  src[s] + r * N + c      (r in the local block)
struct RsArgs {
  const uint16_t* a;
  const uint16_t* b;
  const uint16_t* src[kMaxRanks];
  uint16_t* dst[kMaxRanks];
  uint16_t* out;
  uint32_t* tile_flag;          // pull: notify flag per tile (row-major rb*n_cb+cb)
  const uint32_t* peer_flags;   // pull: [R][local-block tiles] or null (local block aligned to BM)
  uint32_t peer_flag_value;
  uint32_t* rflag[kMaxRanks];   // push: rank s's receive flags [R][tpb]
  uint32_t flag_value;          // push: value of a set flag (this call's)
  int push, tpb;                // tpb: tiles per row block (push)
  int local_rb0, local_nrb;     // row blocks of the local block (peer flag indexing)
  uint32_t* rs_sum;             // [local row blocks]: epoch once the row block's first reduce strip
                                // has seen every flag of the block's tiles
  RsPlan plan;
  Common cm;
};

// TopK-Reduce + ReduceScatter: tasks of CR rows of the token order rotated
// to start at the local block; every row's combined value goes to the
// partial, and the local block's rows are also reduced over the ranks.
struct CombArgs {
  const uint16_t* y;            // [T*topk][N], token-slot order
  const float* w;               // [T][topk]
  const uint16_t* peers[kMaxRanks];
  uint16_t* partial;            // [T][N]
  uint16_t* out;                // [m][N]
  int topk, CR, CRL, n_lt, n_comb;   // rows per task (other / local rows), #local tasks, #tasks
  int R, local, m, T, N;
  int max_tiles;                // MoE layer chain: entries of the grouped-tile flag array
  Common cm;
};

struct MoeArgs {
  const uint16_t* chunks[kMaxRanks];
  const uint16_t* w;            // [E][K][N]
  uint16_t* a_gathered;
  uint16_t* out;
  const int32_t* perm;          // expert-sorted token-slot list
  const int32_t* lut;           // [tiles][8]: e, r0, nrows, cb, 0, 0, 0, 0
  uint32_t* slab_cnt;
  uint32_t* slab_flag;
  int topk, E;
  AgPlan plan;                  // copy plan (tiles come from the lookup table)
  Common cm;
  // The MoE layer chain (combine = 1): after its tiles the kernel runs the
  // TopK-Reduce + ReduceScatter tasks of `comb` on `out`, each waiting on the
  // flags of the grouped tiles that wrote its tokens' slot rows.
  int combine;
  int BM, n_cb;
  uint32_t* tflag;              // [tiles]: epoch once the grouped tile has stored its rows
  const int32_t* inv;           // [slots]: position of each token-slot in the expert-sorted order
  const int32_t* lut_base;      // [E]: first lookup-table entry of each expert
  const int32_t* offsets;       // [E+1]: expert offsets in the sorted order
  const int32_t* topk_ids;      // [T][topk]
  CombArgs comb;
};

// AllGather-KV attention: copy tasks of both tensors, then attention tiles.
struct AttnArgs {
  const uint16_t* q;                      // [m][Hq][d], the local queries
  const uint16_t* k_chunks[kMaxRanks];    // [m][Hkv][d] per rank
  const uint16_t* v_chunks[kMaxRanks];
  uint16_t* k_gathered;                   // [R*m][Hkv][d]
  uint16_t* v_gathered;
  uint16_t* out;                          // [m][Hq][d]
  uint32_t* slab_cnt;
  uint32_t* slab_flag;
  float scale_log2;                       // log2(e) / sqrt(d)
  AttnPlan plan;
  Common cm;
};

struct RouteArgs {
  const float* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* perm;
  int32_t* offsets;             // workspace copy [E+1]
  int32_t* user_offsets;        // optional
  int32_t* lut;
  int32_t* blk_cnt;             // [blocks][E] slots per expert in each routing block
  int32_t* inv;                 // [slots]: inverse of perm
  int32_t* lut_base;            // [E]: first lookup-table entry of each expert
  WsHeader* hdr;
  int T, E, topk, BM, n_cb, max_tiles;
};

// Launchers (kernels.hip). Return hipSuccess or the launch error.
hipError_t launch_ag_gemm(const AgArgs& a, int tile, int grid, hipStream_t s);
// Side producer of ocg_ag_gemm's copy tasks (co-resident with the GEMM kernel).
hipError_t launch_ag_side_copy(const AgArgs& a, int grid, hipStream_t s);
constexpr int kSideThreads = 256;     // 4 waves: one per SIMD of a compute unit
// Registers (VGPRs incl. accumulation registers) and LDS bytes of a kernel
// per workgroup; false if the query fails.
bool kernel_resources(int op, int tile, int* vgprs, int* lds_bytes);
hipError_t launch_gemm_rs(const RsArgs& a, int tile, int grid, hipStream_t s);
hipError_t launch_moe(const RouteArgs& r, const MoeArgs& a, int tile, int grid, hipStream_t s);
hipError_t launch_moe_combine_rs(const CombArgs& a, int grid, hipStream_t s);
hipError_t launch_ag_attention(const AttnArgs& a, int grid, hipStream_t s);
int resident_attention();
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, int release, hipStream_t s);
// No-allocation entry point: the device address of the file-scope scratch
// array on `device` (which must be current), cleared on first use.
constexpr size_t kNoAllocScratchBytes = (size_t)1 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch_setup(int device, void** out);
// Resident workgroups per CU of each persistent kernel (op, tile preset; sk:
// the AG-GEMM kernel for tiles split in sk K parts).
int resident_per_cu(int op, int tile, int sk = 1);

}  // namespace ocg
