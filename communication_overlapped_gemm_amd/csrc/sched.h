// Closed-form ticket -> task maps of the persistent kernels (host and device).
//
// Tile-centric scheduling after "TileLink: Generating Efficient
// Compute-Communication Overlapping Kernels using Tile-Centric Primitives"
// (MLSys 2025 talk summary), section "Technical Deep Dive": a wait names only
// a tile; its rank, barrier (slab), tiles per rank and barriers per rank
// follow from affine maps for static workloads; swizzling reorders tile
// access and transfers so transfers line up with compute.
//
// AG-GEMM plan. Gathered rows M = R*m; rank chunk c owns rows [c*m, (c+1)*m).
// A chunk is cut into slabs of S rows and its columns into K-slabs of KS
// columns (the last one may be shorter); one flag is published per (slab,
// K-slab), at index slab * nks + kslab. Copy tasks move CT rows (S % CT == 0)
// of one K-slab. The chunk sequence is local+1, local+2, ..., local+R-1,
// local (swizzled) or 0..R-1 (natural); when swizzled its peer chunks are cut
// into phases by the round of tiles that first reads them (rows per round
// rpr: the persistent grid's tiles cover rpr gathered rows of the rotated
// order per round), and the local chunk, which no tile waits on, comes last.
// Copy tickets run phase by phase, K-slab by K-slab within a phase, and over
// the phase's chunks and their pieces within a K-slab. Tickets below
// n_inline are taken by the GEMM kernel's own workgroups before their tiles;
// the rest by the side producer kernel (SIDE transfer; n_inline = n_copy
// otherwise). With one K-slab (KS = K) this is the plain per-slab plan; with
// several, a tile can start on the first columns of a peer's rows while
// later columns are still being copied, and it waits on each K-slab's flag
// before its loads of that K-slab. GEMM tiles are
// numbered 0..n_tiles-1 in grouped order: row blocks rotated to start at the
// block holding the local chunk's first row, taken in groups of kGroup, each
// group walked column block by column block. Tiles are cut into batches of
// kBatch consecutive tiles dealt round-robin to kXcds queues; a workgroup
// drains the queue of the XCD it runs on, then the others. Concurrent tiles of
// one XCD thereby share A and B panels in that XCD's L2. A workgroup takes
// tiles only once every copy ticket has been claimed, tiles wait only on copy
// tasks, and copy tasks never wait: the schedule cannot deadlock.
//
// Split K (sk = 2): when the tiles would leave compute units idle for a
// round, each tile becomes two units, its K halves, queued as consecutive
// work items u = 2v, 2v + 1 of one XCD batch (the tile queues then hand out
// units). The half that finishes first stores its fp32 accumulators; the
// other adds them and writes the tile. Neither waits on a unit that has not
// started, so this adds no deadlock either.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define OCG_HD __host__ __device__ __forceinline__
#else
#define OCG_HD inline
#endif

namespace ocg {

OCG_HD int cdiv(int a, int b) { return (a + b - 1) / b; }

struct AgPlan {
  int R, local, m, M, K, N;
  int BM, BN, S, CT, KS;
  int swizzle, mode;
  int n_rb, n_cb, bpr, n_tpc, nks, n_copy, n_tiles, rb0;
  int rpr;        // gathered rows per round of tiles (copy phases)
  int n_inline;   // copy tickets the GEMM kernel runs itself (the rest: side producer)
  int sk;         // K parts per tile (1, or 2 = split K); work units = n_tiles * sk
};

// Copy phase of position q of the chunk sequence: swizzled, the peers by the
// round whose tiles first read them (the rotated order starts at the local
// chunk), the local chunk last; natural order, one phase.
OCG_HD int copy_phase(const AgPlan& p, int q) {
  if (!p.swizzle) return 0;
  if (q == p.R - 1) return 1 << 20;
  return (int)(((long long)(q + 1) * p.m) / p.rpr);
}

// mode: 0 fused, 1 gemm only, 2 copy only. KS <= 0 or KS >= K: one K-slab.
// tpr: work units per round (the persistent grid); 0 = all tiles in one round.
// sk: K parts per tile (2 needs one K-slab and K % 128 == 0).
OCG_HD AgPlan make_ag_plan(int R, int local, int m, int K, int N, int BM, int BN, int S, int CT,
                           int swizzle, int mode, int KS = 0, int tpr = 0, int sk = 1) {
  AgPlan p;
  p.R = R; p.local = local; p.m = m; p.M = R * m; p.K = K; p.N = N;
  p.BM = BM; p.BN = BN; p.S = S; p.CT = CT; p.swizzle = swizzle; p.mode = mode;
  p.KS = (KS <= 0 || KS > K) ? K : KS;
  p.n_rb = cdiv(p.M, BM);
  p.n_cb = cdiv(N, BN);
  p.bpr = cdiv(m, S);
  p.n_tpc = cdiv(m, CT);
  p.nks = cdiv(K, p.KS);
  p.n_copy = (mode == 1) ? 0 : R * p.n_tpc * p.nks;
  p.n_tiles = (mode == 2) ? 0 : p.n_rb * p.n_cb;
  p.rb0 = swizzle ? (int)(((long long)local * m) / BM) : 0;
  p.sk = sk > 1 ? sk : 1;
  const int rb_per_round = tpr > 0 ? tpr / (p.n_cb * p.sk) : p.n_rb;
  p.rpr = (rb_per_round > 0 ? rb_per_round : 1) * BM;
  p.n_inline = p.n_copy;
  return p;
}

// Copy tickets of the first phase's first K-slab (what the GEMM kernel
// copies itself under the SIDE transfer before its tiles start).
OCG_HD int first_kslab_tickets(const AgPlan& p) {
  int q1 = 0;
  while (q1 < p.R && copy_phase(p, q1) == copy_phase(p, 0)) ++q1;
  return q1 * p.n_tpc;
}

// Chunk copied at position q of the copy sequence.
OCG_HD int copy_chunk(const AgPlan& p, int q) {
  if (!p.swizzle) return q;
  return (q < p.R - 1) ? (p.local + 1 + q) % p.R : p.local;
}

// Copy task: gathered rows [row0, row1) x columns [k0, k1) of one chunk;
// completes part of flag `flag` = slab * nks + kslab.
struct CopyDesc {
  int chunk, piece, row0, row1, slab, kslab, k0, k1, flag;
};

OCG_HD CopyDesc copy_desc(const AgPlan& p, int u) {
  CopyDesc d;
  // the phase holding ticket u: sequence positions [q0, q1)
  int q0 = 0, base = 0;
  for (;;) {
    int q1 = q0 + 1;
    while (q1 < p.R && copy_phase(p, q1) == copy_phase(p, q0)) ++q1;
    const int n = (q1 - q0) * p.n_tpc * p.nks;
    if (u < base + n || q1 >= p.R) {
      const int per_ks = (q1 - q0) * p.n_tpc;
      const int w = u - base;
      d.kslab = w / per_ks;
      const int r = w - d.kslab * per_ks;
      const int q = q0 + r / p.n_tpc;
      d.piece = r - (q - q0) * p.n_tpc;
      d.chunk = copy_chunk(p, q);
      break;
    }
    base += n;
    q0 = q1;
  }
  int r0 = d.piece * p.CT;
  int r1 = r0 + p.CT < p.m ? r0 + p.CT : p.m;
  d.row0 = d.chunk * p.m + r0;
  d.row1 = d.chunk * p.m + r1;
  d.slab = d.chunk * p.bpr + r0 / p.S;
  d.k0 = d.kslab * p.KS;
  d.k1 = d.k0 + p.KS < p.K ? d.k0 + p.KS : p.K;
  d.flag = d.slab * p.nks + d.kslab;
  return d;
}

// K-slabs are confirmed by the tiles in groups that double in size: group g
// holds K-slabs [2^g - 1, 2^(g+1) - 1) (clipped to nks), so a tile that
// streams K pays one acquire per group instead of one per K-slab; the copy
// front keeps ahead because the copies run K-slab by K-slab from the start.
OCG_HD int kgroup_first(int g) { return (1 << g) - 1; }

// Copy tasks that complete slab `slab` (global id chunk*bpr + s) in one
// K-slab.
OCG_HD int slab_target(int m, int S, int CT, int bpr, int slab) {
  int s = slab % bpr;
  int per = S / CT;
  int n_tpc = cdiv(m, CT);
  int first = s * per;
  int left = n_tpc - first;
  return left < per ? left : per;
}

constexpr int kGroup = 4;    // row blocks per group of the tile order
constexpr int kBatch = 32;   // consecutive tiles per XCD batch (one per CU of an XCD)
constexpr int kXcds = 8;     // XCDs of an MI355X (hardware queue id range of XCC_ID)

// Tile v (0-based, grouped order) -> (rb, cb).
OCG_HD void tile_of(int n_rb, int n_cb, int rb0, int v, int* rb, int* cb) {
  const int per_group = kGroup * n_cb;
  const int grp = v / per_group;
  const int rho0 = grp * kGroup;
  const int gsz = n_rb - rho0 < kGroup ? n_rb - rho0 : kGroup;
  const int w = v - grp * per_group;
  *cb = w / gsz;
  const int r = rb0 + rho0 + (w - *cb * gsz);
  *rb = r >= n_rb ? r - n_rb : r;
}

// Ticket t of XCD queue q -> tile index, or -1 once the queue is exhausted.
OCG_HD int xcd_tile(int q, int t, int n_tiles) {
  const int beta = (t / kBatch) * kXcds + q;
  const int v = beta * kBatch + (t % kBatch);
  return v < n_tiles ? v : -1;
}

// Tile index -> (queue, ticket).
OCG_HD void tile_queue(int v, int* q, int* t) {
  const int beta = v / kBatch;
  *q = beta % kXcds;
  *t = (beta / kXcds) * kBatch + v % kBatch;
}

// Slabs (excluding the local chunk) overlapping gathered rows [r0, r1):
// visits them in ascending order, calling f(slab).
template <class F>
OCG_HD int for_each_dep_slab(int m, int S, int bpr, int local, int r0, int r1, F f) {
  int n = 0;
  if (r1 <= r0) return 0;
  int c0 = r0 / m, c1 = (r1 - 1) / m;
  for (int c = c0; c <= c1; ++c) {
    if (c == local) continue;
    int lo = (c == c0) ? r0 - c * m : 0;
    int hi = (c == c1) ? r1 - c * m : m;  // exclusive
    int s0 = lo / S, s1 = (hi - 1) / S;
    for (int s = s0; s <= s1; ++s) {
      f(c * bpr + s);
      ++n;
    }
  }
  return n;
}

// GEMM-RS plan: tiles 0..n_tiles-1 of the full partial in the grouped order
// above (local row block first when swizzled), handed out by the XCD queues;
// then reduce strips 0..n_red-1 of RR rows of the local block
// [local*blk, (local+1)*blk), handed out by the global counter once every tile
// has been claimed.
struct RsPlan {
  int R, local, M, K, N, BM, BN, blk, RR;
  int n_rb, n_cb, n_tiles, n_red, rb0;
};

// push: the partials are pushed to their owners, so the tiles start at the
// block after the local one (local + 1, local + 2, ..., local last): every
// peer's data leaves as early as possible and the local block, reduced here,
// comes last.
OCG_HD RsPlan make_rs_plan(int R, int local, int M, int K, int N, int BM, int BN, int RR, int swizzle,
                           int push = 0) {
  RsPlan p;
  p.R = R; p.local = local; p.M = M; p.K = K; p.N = N; p.BM = BM; p.BN = BN; p.RR = RR;
  p.blk = M / R;
  p.n_rb = cdiv(M, BM);
  p.n_cb = cdiv(N, BN);
  p.n_tiles = p.n_rb * p.n_cb;
  p.n_red = cdiv(p.blk, RR);
  const int first = push ? (local + 1) % R : local;
  p.rb0 = swizzle ? (int)(((long long)first * p.blk) / BM) : 0;
  return p;
}

// Reduce strip j -> gathered rows [*r0, *r1).
OCG_HD void rs_strip(const RsPlan& p, int j, int* r0, int* r1) {
  int lo = p.local * p.blk;
  *r0 = lo + j * p.RR;
  int e = *r0 + p.RR;
  *r1 = e < lo + p.blk ? e : lo + p.blk;
}

OCG_HD bool rs_tile_touches_local(const RsPlan& p, int rb) {
  int lo = rb * p.BM;
  int hi = lo + p.BM < p.M ? lo + p.BM : p.M;
  return lo < (p.local + 1) * p.blk && hi > p.local * p.blk;
}

// AllGather-KV attention plan. The gathered keys / values are R chunks of m
// tokens; a token row holds Hkv heads of d elements. Copy tasks are the AG
// copy plan of one tensor (rows = tokens, K = Hkv * d) run for both tensors:
// ticket u copies piece u >> 1 of that order for tensor u & 1 (0 keys, 1
// values), so a slab's flag is published after 2 * slab_target tasks.
// Attention tiles: the query rows of kv head g are the pairs (i, h), i < m,
// h in [g*G, (g+1)*G), G = Hq / Hkv, numbered i-major (row r -> i = r / G,
// h = g*G + r % G) and cut into blocks of kAttnRows; tile v -> (g = v / n_rb,
// rb = v % n_rb), in the XCD queues of the GEMM tiles, so one XCD's tiles
// share the keys and values of one head in its L2. A tile visits the keys in
// blocks of kAttnKB, chunk by chunk, starting at the local chunk when swizzled
// (its keys need no wait) and walking up the ranks from there.
constexpr int kAttnRows = 256;   // query rows per tile (64 per wave)
constexpr int kAttnKB = 64;      // keys per block
constexpr int kAttnD = 128;      // head dimension

struct AttnPlan {
  AgPlan cp;                     // copy plan of one tensor
  int Hq, Hkv, G, n_rb, n_tiles, nbc, n_copy;   // n_copy: tickets of both tensors
};

OCG_HD AttnPlan make_attn_plan(int R, int local, int m, int Hq, int Hkv, int S, int CT, int swizzle, int mode) {
  AttnPlan p;
  p.cp = make_ag_plan(R, local, m, Hkv * kAttnD, kAttnD, kAttnRows, kAttnKB, S, CT, swizzle, mode);
  p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
  p.n_rb = cdiv(p.G * m, kAttnRows);
  p.n_tiles = (mode == 2) ? 0 : Hkv * p.n_rb;
  p.nbc = cdiv(m, kAttnKB);
  p.n_copy = 2 * p.cp.n_copy;
  return p;
}

// Chunk whose keys key block j (0 .. R*nbc-1) of a tile holds.
OCG_HD int attn_block_chunk(const AttnPlan& p, int j) {
  const int pos = j / p.nbc;
  return p.cp.swizzle ? (p.cp.local + pos) % p.cp.R : pos;
}

// Tile presets: {BM, BN} = {256,224}, {128,224}, {128,256}, {128,128}.
OCG_HD int tile_bm(int t) { return t == 6 ? 288 : t == 5 ? 320 : ((t == 0 || t == 4) ? 256 : 128); }
OCG_HD int tile_bn(int t) { return (t == 2 || t == 4) ? 256 : (t == 3 ? 128 : 224); }
// Waves per workgroup of a preset's GEMM kernels (the engine's gemm_waves).
OCG_HD int tile_waves(int t) { return tile_bm(t) == 320 ? 8 : 4; }

}  // namespace ocg
