/*
 * ocg.h -- communication-overlapped GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the fused tile-centric AllGather-GEMM, GEMM-ReduceScatter,
 * AllGather + MoE grouped GEMM, MoE TopK-Reduce + ReduceScatter and
 * AllGather-KV attention, each computing one GPU's share of a tensor- or
 * context-parallel LLM layer. The operations are the ones named in
 * "TileLink: Generating Efficient Compute-Communication Overlapping Kernels
 * using Tile-Centric Primitives" (MLSys 2025 talk summary), sections "Key
 * Findings" (AllGather-GEMM, GEMM-ReduceScatter), "Technical Deep Dive"
 * (tile signals, pull transfers, swizzled tile order, lookup tables for
 * dynamic dependencies) and "Experimental Setup & Results" (MoE:
 * AllGather -> GroupGEMM -> ... -> local scatter).
 *
 * Conventions (every entry point):
 *   - Matrices are row-major. "bf16" buffers hold raw bfloat16 bit patterns
 *     (uint16). Every matrix pointer is a DEVICE pointer owned by the caller;
 *     the library never frees or retains it past the call.
 *   - Peer ranks are given as an array of R device pointers (a host array,
 *     read during the call only). On one GPU they point at local stand-in
 *     buffers; across GPUs they would be IPC-mapped peer buffers.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     means the default stream) and allocate no device memory: every scratch
 *     word (tickets, flags, counters, routing tables, error word) lives in the
 *     caller's workspace, sized by ocg_workspace_bytes() and cleared once by
 *     ocg_workspace_init(). Calls that share a workspace must be ordered on
 *     one stream; concurrent calls on one workspace race.
 *   - Return value: OCG_OK or a negative OCG_ERR_* code. On an error return
 *     nothing has been enqueued. No C++ exception or abort crosses the ABI.
 *     A flag wait that exceeds its time bound is recorded in the workspace's
 *     error word and reported by ocg_check() after the stream has drained.
 *   - GEMM shapes: K must be a multiple of 64, N a multiple of 8, 1 <= R <= 16.
 *     M, N and the per-rank rows m may leave ragged tiles. Pointers to bf16
 *     matrices must be 16-byte aligned.
 */
#ifndef OCG_H_
#define OCG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OCG_OK 0
#define OCG_ERR_INVALID_ARG (-1)
#define OCG_ERR_UNSUPPORTED_SHAPE (-2)
#define OCG_ERR_WORKSPACE_TOO_SMALL (-3)
#define OCG_ERR_HIP (-4)
#define OCG_ERR_TIMEOUT (-5)
#define OCG_ERR_NO_DEVICE (-6)

#define OCG_OP_AG_GEMM 0
#define OCG_OP_GEMM_RS 1
#define OCG_OP_AG_GROUPED_GEMM 2
#define OCG_OP_MOE_COMBINE_RS 3
#define OCG_OP_AG_ATTENTION 4

/* Fused (default), GEMM tiles only with every flag treated as published
 * (measurement of the GEMM part; expects the gathered buffer filled), or
 * copy tasks only (measurement of the gather part). */
#define OCG_MODE_FUSED 0
#define OCG_MODE_GEMM_ONLY 1
#define OCG_MODE_COPY_ONLY 2

/* How the AllGather part of ocg_ag_gemm moves the peers' rows (ocg_config.transfer):
 *   INLINE -- copy tasks run in the GEMM's own persistent kernel: every
 *             workgroup takes copy tickets first, then tiles;
 *   SIDE   -- the copy tasks run in a small producer kernel on a side stream
 *             owned by the handle, co-resident with the GEMM kernel on every
 *             compute unit (it uses no LDS and few registers), so copies
 *             proceed while the tiles compute. The caller's stream waits for
 *             the producer before the call's later work; the GEMM tiles wait
 *             on the per-(slab, K-slab) flags it publishes.
 *   AUTO   -- INLINE (SIDE measures 1-3 % faster per call at the 70B share
 *             and slower at the 8B one; one kernel stays safe under
 *             profilers that serialise dispatches, where SIDE's tiles may
 *             wait out their bound for a producer that has not run:
 *             ocg_check then reports the timeout). SIDE is refused
 *             (OCG_ERR_UNSUPPORTED_SHAPE) if the producer does not fit next
 *             to the GEMM kernel's workgroup.
 * (Pull transfers with a "transfer complete" flag per slab: "TileLink ..."
 * (MLSys 2025 talk summary), "Technical Deep Dive".) */
#define OCG_TRANSFER_AUTO (-1)
#define OCG_TRANSFER_INLINE 0
#define OCG_TRANSFER_SIDE 1

/* Tile presets (rows x columns of C per workgroup tile, K step 64);
 * OCG_TILE_288x224 and OCG_TILE_320x224 are for the grouped GEMM only. */
#define OCG_TILE_AUTO (-1)
#define OCG_TILE_256x224 0
#define OCG_TILE_128x224 1
#define OCG_TILE_128x256 2
#define OCG_TILE_128x128 3
#define OCG_TILE_256x256 4
#define OCG_TILE_320x224 5
#define OCG_TILE_288x224 6
#define OCG_TILE_COUNT 7

/* Trace record written per executed task when ocg_config.trace is set
 * (80 bytes), at slot: AG-GEMM / MoE copy task u -> u, tile v -> n_copy + v;
 * GEMM-RS tile v -> v, reduce strip j -> n_tiles + j (v = tile index in the
 * grouped tile order; TopK-Reduce: task u -> u).
 * kind: 1 copy task, 2 AG-GEMM tile, 3 GEMM-RS tile, 4 MoE tile, 5 GEMM-RS
 * reduce strip, 6 TopK-Reduce task, 7 attention tile (AllGather-KV
 * attention: copy ticket u -> u, tile v -> #copy tickets + v). Times are the
 * GPU's constant 100 MHz clock; `cycles` counts shader-clock cycles over the
 * same interval (s_memtime), so cycles / (t_end - t_start) * 100 MHz is the
 * compute-unit clock while the task ran. */
typedef struct ocg_trace_rec {
  uint32_t ticket, kind;
  uint32_t a, b, c, d;   /* copy: chunk, piece, flag index (slab * #K-slabs + K-slab), published(0/1)
                            AG tile: rb, cb, #slabs waited, 0
                            RS tile: rb, cb, local-block(0/1), 0
                            MoE tile: expert, row start, rows, cb | (#slabs waited << 16)
                            RS strip: row0, row1, #flags waited, 0
                            KV copy: chunk, piece | (tensor << 16), slab, published
                            attention tile: kv head, row block, #flags waited, 0 */
  uint32_t hw;           /* (XCC id << 16) | workgroup id */
  uint32_t epoch;        /* epoch of the call */
  uint64_t t_start, t_ready, t_end; /* ready = dependencies satisfied (tiles)
                                       or flag published (copy) */
  uint32_t flag_seen;
  uint32_t queue;        /* tiles: (XCD queue << 16) | ticket within that queue;
                            AG copy: K-slab index */
  uint64_t cycles;       /* shader-clock cycles from t_start to t_end */
  uint32_t wait_ticks;   /* AG tile: 100 MHz ticks spent waiting on K-slab flags inside the
                            K loop (after t_ready); 0 otherwise */
  uint32_t pad;
} ocg_trace_rec;

typedef struct ocg_config {
  int32_t tile;             /* OCG_TILE_* preset, or OCG_TILE_AUTO */
  int32_t slab_rows;        /* rows of a rank chunk per published flag; 0 = tile rows */
  int32_t copy_rows;        /* rows per copy task (must divide slab_rows;
                               rows * K * 2 < 2 GiB); 0 = auto */
  int32_t swizzle;          /* 1 = tiles and copies start at the local rank and rotate
                               (default); 0 = natural rank order */
  int32_t mode;             /* OCG_MODE_* */
  int32_t grid;             /* persistent workgroups; 0 = resident capacity */
  uint32_t spin_timeout_us; /* bound on every flag wait, microseconds; 0 = 1 s */
  int32_t fault_skip_slab;  /* test hook: this slab's flag is never published; -1 = off */
  void* trace;              /* device array of ocg_trace_rec indexed by ticket, or NULL */
  uint32_t trace_capacity;  /* records in `trace` */
  const uint32_t* peer_flags; /* GEMM-RS: device array [R][tiles of the local row block],
                                 written by peers when their partial tile has landed;
                                 NULL = all peer partials are complete */
  uint32_t peer_flag_value;   /* value meaning "landed" in peer_flags */
  int32_t transfer;         /* OCG_TRANSFER_* (ocg_ag_gemm only); default AUTO */
  int32_t kslab_cols;       /* ocg_ag_gemm: columns of A per published flag (a multiple of 256);
                               0 = auto: the whole K for INLINE, 512 for SIDE */
  uint32_t copy_delay;      /* test hook: a copy task of K-slab j first sleeps (j + 1) x this many
                               rounds of s_sleep 127 (~8k cycles each) -- forces late publishes,
                               later K-slabs later (copy tasks of the AG-GEMM, the grouped GEMM and
                               the MoE layer; the attention's copy tasks, which have no K-slabs,
                               sleep this many rounds); 0 = off */
  int32_t xcd_remap;        /* 1 = tiles dealt in batches to per-XCD queues (default);
                               0 = one queue in plain tile order (ablation) */
  int32_t side_grid;        /* SIDE transfer: producer workgroups (one per compute unit at most
                               counts); 0 = auto */
  int32_t split_k;          /* ocg_ag_gemm: 0 = auto (split where the cost estimate favours it
                               and the workspace holds the sums), 1 = off, 2 = every tile as two
                               K halves (needs the INLINE transfer, one K-slab and K % 128 == 0:
                               OCG_ERR_INVALID_ARG otherwise; OCG_ERR_WORKSPACE_TOO_SMALL if
                               the workspace lacks room for the sums) */
} ocg_config;

/* Opaque per-device handle: device id, compute-unit count and the resident
 * capacity of each persistent kernel. */
typedef struct ocg_handle_s* ocg_handle;

/* Fill `cfg` with defaults (auto tile, swizzled, fused, 1 s timeout, no
 * trace, no fault injection, auto transfer and K-slab width, XCD queues). */
void ocg_config_default(ocg_config* cfg);

/* Create a handle for `device` (HIP ordinal). Returns OCG_ERR_NO_DEVICE if no
 * such device exists and OCG_ERR_UNSUPPORTED_SHAPE if it is not gfx950. */
int ocg_create(int device, ocg_handle* out);
void ocg_destroy(ocg_handle h);

/* Workspace bytes for `op` with the default configuration: AG_GEMM (R,
 * m = rows per rank, K, N), GEMM_RS (R, m = M total rows, K, N),
 * AG_GROUPED_GEMM (R, m, K, N, E, topk), MOE_COMBINE_RS (R, m, 0, N, 0,
 * topk), AG_ATTENTION (R, m = tokens per rank, K = Hq, N = Hkv). For AG_GEMM
 * this includes room for the fp32 sums of split-K tiles (BM x BN x 4 bytes
 * per tile) where the default plan splits, which depends on the device's
 * compute units (`h`; NULL = a 256-CU MI355X); the other sizes do not depend
 * on the device. Unused arguments are ignored. Returns 0 on invalid
 * arguments. */
size_t ocg_workspace_bytes(ocg_handle h, int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk);

/* As ocg_workspace_bytes, for calls made with configuration `cfg` (NULL =
 * default), e.g. ocg_ag_gemm with split_k = 2. Returns 0 on invalid
 * arguments or configurations. */
size_t ocg_workspace_bytes_for(ocg_handle h, int op, int R, int64_t m, int64_t K, int64_t N, int E, int topk,
                               const ocg_config* cfg);

/* Clear a workspace once before its first use (a fill kernel on `stream`). */
int ocg_workspace_init(ocg_handle h, void* workspace, size_t ws_bytes, void* stream);

/*
 * AllGather-GEMM: a_gathered = concat_r a_chunks[r] (row block r = rank r),
 * C = a_gathered x B, fp32 accumulation, C rounded to bf16 (nearest-even).
 *   a_chunks[r] : bf16 [m, K] of rank r (r = 0..R-1), read
 *   b           : bf16 [K, N], read
 *   a_gathered  : bf16 [R*m, K], written (every row, the local one included)
 *   c           : bf16 [R*m, N], written
 * Copy tasks pull each peer chunk into a_gathered slab by slab and publish a
 * per-slab flag; GEMM tiles wait on the flags of the slabs they read (the
 * local rank's rows are read from its own shard and never wait).
 * Split K (cfg->split_k; chosen automatically when the tiles would leave
 * compute units idle, e.g. 128 tiles on 256 CUs): each tile runs as two
 * work units, one per K half; the half that finishes first stores its fp32
 * sums in the workspace, and the other adds them to its own and writes the
 * tile. C is then fp32(first half) + fp32(second half) rounded once --
 * the same bits whichever half finishes first, but not always the same
 * bits as the unsplit sum (another fp32 summation order).
 */
int ocg_ag_gemm(ocg_handle h, const void* const* a_chunks, int R, int local_rank,
                int64_t m, int64_t K, const void* b, int64_t N, void* a_gathered, void* c,
                void* workspace, size_t ws_bytes, const ocg_config* cfg, void* stream);

/*
 * ocg_ag_gemm without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, semantics and errors as
 * ocg_ag_gemm minus the workspace: it uses a fixed 1 MiB scratch array that
 * the library keeps on each GPU (a file-scope device array, set up and
 * cleared once by ocg_create, held until the process ends), and allocates
 * nothing itself. Limit: shapes whose AG-GEMM workspace
 * (ocg_workspace_bytes(h, OCG_OP_AG_GEMM, R, m, K, N, 0, 0)) exceeds 1 MiB
 * return OCG_ERR_WORKSPACE_TOO_SMALL and enqueue nothing (the 70B-class
 * share needs about 130 KiB). K is split (cfg->split_k) only where the
 * split-K sums fit the scratch too: where ocg_ag_gemm would split and this
 * entry point cannot, C can differ from ocg_ag_gemm's in the last bit (another
 * fp32 summation order, the same error bound), and split_k = 2 returns
 * OCG_ERR_WORKSPACE_TOO_SMALL. All calls on one GPU share the scratch, which
 * keeps the last call's state: calls that overlap on one GPU (on different
 * streams, or from different handles or threads) race and must not be
 * issued; calls ordered on one stream are fine. A timed-out flag wait is
 * recorded in the scratch, not reported.
 */
int ocg_ag_gemm_noalloc(ocg_handle h, const void* const* a_chunks, int R, int local_rank,
                        int64_t m, int64_t K, const void* b, int64_t N, void* a_gathered, void* c,
                        const ocg_config* cfg, void* stream);

/*
 * GEMM-ReduceScatter (one rank's share):
 *   partial = A x B rounded to bf16 (this rank's send buffer, every row);
 *   out     = bf16( sum_{s=0..R-1} P_s[rows local*M/R .. (local+1)*M/R) )
 * where P_local is `partial` and P_s (s != local) are peer_partials[s]. The
 * sum runs in fp32 over the bf16 partials in ascending rank order s = 0..R-1
 * with a single rounding at the end, so it is reproducible bit for bit.
 *   a                : bf16 [M, K];  b: bf16 [K, N]   (M % R == 0)
 *   peer_partials[s] : bf16 [M, N] for s != local_rank (entry local ignored)
 *   partial          : bf16 [M, N], written
 *   out              : bf16 [M/R, N], written
 * Tiles outside the local row block publish a per-tile flag after storing
 * their partial (the signal a peer would wait on).
 */
int ocg_gemm_rs(ocg_handle h, const void* a, const void* b, int64_t M, int64_t K, int64_t N,
                int R, int local_rank, const void* const* peer_partials, void* partial, void* out,
                void* workspace, size_t ws_bytes, const ocg_config* cfg, void* stream);

/*
 * GEMM-ReduceScatter with push transfers (the one-barrier protocol: the
 * producer writes the data and the flag into the consumer's memory, so no
 * "ready to receive" handshake is needed -- every sender owns a slot; "TileLink
 * ..." (MLSys 2025 talk summary), "Technical Deep Dive", push versus pull).
 * Each rank s has a receive buffer recv[s], bf16 [R][M/R][N] (slot q holds
 * rank q's partial of row block s), and receive flags recv_flags[s], uint32
 * [R][T] (T = tiles per row block: (M/R / BM) * ceil(N / BN) for the
 * resolved tile). This call computes partial = A x B tile by tile; the tile
 * of row block s is rounded to bf16 and stored into recv[s] slot local_rank,
 * then recv_flags[s][local_rank * T + t] = flag_value (t = the tile's index
 * within the block, row-major); row block local_rank goes to our own slot.
 * Tiles run blocks local+1, local+2, ..., local last (peers' data first).
 * Then, waiting on recv_flags[local_rank][q * T + t] == flag_value for every
 * rank q (peers' pushes, and our own), the reduce
 *   out = bf16( sum over q = 0..R-1, in that order, of recv[local_rank][q] )
 * runs in fp32 with one rounding, as ocg_gemm_rs (identical results).
 *   a, b, M, K, N, R, local_rank, out, workspace: as ocg_gemm_rs
 *   recv        : R device pointers (rank r's receive buffer; on one GPU,
 *                 stand-ins in this GPU's memory), 16-byte aligned
 *   recv_flags  : R device pointers (rank r's receive flags), 4-byte aligned
 *   flag_value  : the value this call's pushes write; it must differ from
 *                 every value those flags held before (e.g. a call counter)
 * Requires M/R to be a multiple of the tile's rows (OCG_ERR_UNSUPPORTED_SHAPE
 * otherwise); tile rows: ocg_plan_info(h, OCG_OP_GEMM_RS, ...) out[1]. Errors
 * as for the other calls. */
int ocg_gemm_rs_push(ocg_handle h, const void* a, const void* b, int64_t M, int64_t K, int64_t N,
                     int R, int local_rank, void* const* recv, uint32_t* const* recv_flags,
                     uint32_t flag_value, void* out, void* workspace, size_t ws_bytes,
                     const ocg_config* cfg, void* stream);

/*
 * AllGather + MoE grouped GEMM: tokens t = 0..R*m-1 of the gathered
 * activations are routed to the top-k experts of their fp32 logits (equal
 * logits: lower expert first; slot 0 = largest), grouped by expert (stable
 * in token, slot) and multiplied by the expert's weight:
 *   out[t*topk + j] = a_gathered[t] x W[topk_ids[t][j]]     (token-slot order)
 *   logits      : fp32 [R*m, E], read (E <= 64, topk in 1..4)
 *   w           : bf16 [E, K, N] contiguous, read
 *   a_gathered  : bf16 [R*m, K], written
 *   topk_ids    : int32 [R*m, topk], written
 *   topk_w      : fp32 [R*m, topk], written (softmax probability of each pick)
 *   perm        : int32 [R*m*topk], written: token-slot indices sorted by expert
 *   expert_offsets : int32 [E+1], written (may be NULL): row offsets of each
 *                    expert in `perm`
 *   out         : bf16 [R*m*topk, N], written
 * The grouped tiles wait on the flags of every peer slab their tokens come
 * from (a per-tile lookup table built on the device after routing). Tile
 * presets: OCG_TILE_128x224, OCG_TILE_256x224, OCG_TILE_288x224 or
 * OCG_TILE_320x224 (the last two only here); OCG_TILE_AUTO takes the
 * smallest whose rows hold the rows an expert is expected to get at most
 * (mean R*m*topk/E plus two standard deviations of the binomial count),
 * else 256x224. An expert with more rows than a tile gets further row tiles,
 * so every preset gives the same results. Any other preset is
 * OCG_ERR_INVALID_ARG.
 */
int ocg_ag_grouped_gemm(ocg_handle h, const void* const* a_chunks, int R, int local_rank,
                        int64_t m, int64_t K, const float* logits, int E, int topk,
                        const void* w, int64_t N, void* a_gathered, int32_t* topk_ids,
                        float* topk_w, int32_t* perm, int32_t* expert_offsets, void* out,
                        void* workspace, size_t ws_bytes, const ocg_config* cfg, void* stream);

/* The MoE layer chain in one call: ocg_ag_grouped_gemm (AllGather, routing,
 * grouped GEMM, local scatter into y) followed by ocg_moe_combine_rs on its
 * output (TopK-Reduce of y into `partial`, ReduceScatter of the ranks'
 * partials into `out`), the operators "TileLink ..." (MLSys 2025 talk
 * summary), "Experimental Setup & Results", overlaps in its MoE layer. The
 * TopK-Reduce tasks run in the grouped GEMM's persistent kernel after its
 * tiles: each grouped tile stores its rows and publishes a flag, and each
 * task waits on the flags of exactly the tiles that wrote its tokens' slot
 * rows -- found through the routing tables (the slot's position in the
 * expert-sorted order, its expert's row tile, every column block), the
 * dynamic dependencies resolved by lookup tables of "Technical Deep Dive" --
 * so the tail of the grouped GEMM overlaps the first TopK-Reduce tasks.
 * Arguments as ocg_ag_grouped_gemm (y = its `out`, bf16 [R*m*topk, N], here
 * also an input of the combine) and ocg_moe_combine_rs (peer_partials,
 * partial bf16 [R*m, N], out bf16 [m, N]; topk_w are the routing's gate
 * weights). Results equal the two calls made in sequence. Requires the shapes
 * of both calls and R*m*topk*N*2 < 2^31; workspace from
 * ocg_workspace_bytes(h, OCG_OP_AG_GROUPED_GEMM, R, m, K, N, E, topk). Trace:
 * copies and tiles as ocg_ag_grouped_gemm, then TopK-Reduce task u at slot
 * n_copy + #tiles + u (kind 6; d = #dependencies waited on). */
int ocg_ag_moe_layer(ocg_handle h, const void* const* a_chunks, int R, int local_rank,
                     int64_t m, int64_t K, const float* logits, int E, int topk, const void* w,
                     int64_t N, const void* const* peer_partials, void* a_gathered, int32_t* topk_ids,
                     float* topk_w, int32_t* perm, int32_t* expert_offsets, void* y, void* partial,
                     void* out, void* workspace, size_t ws_bytes, const ocg_config* cfg, void* stream);

/* MoE TopK-Reduce + ReduceScatter, the tail of the MoE layer ("TileLink ...
 * (MLSys 2025 talk summary)", section "Experimental Setup & Results", lists
 * TopK-Reduce and ReduceScatter among the MoE operators it overlaps; the
 * formula is the plain reading of a gate-weighted top-k combine followed by
 * the ReduceScatter of the GEMM-ReduceScatter call):
 *   P_l[t] = sum over j < topk of topk_w[t][j] * y[t*topk + j]   (t < T = R*m)
 *   out    = sum over ranks s = 0..R-1 of P_s[rows local*m .. (local+1)*m)
 * P_l is computed in fp32 (slot order, fma), rounded once to bf16 and stored
 * in `partial` (the send buffer); the reduce sums the R bf16 partials in
 * ascending rank order in fp32 with one rounding (as ocg_gemm_rs). Tasks of
 * rows cover the local block's rows first (smaller tasks: a local row also
 * reads the R-1 peer rows and writes out); a local row is reduced by the
 * task that combines it (its inputs are the peers' rows and its own rounded
 * value), so no task waits on another.
 *   y             : bf16 [R*m*topk, N], token-slot order (row t*topk + j)
 *   topk_w        : fp32 [R*m, topk] gate weights (4-byte aligned)
 *   peer_partials : R device pointers, bf16 [R*m, N] each; entry local_rank
 *                   is ignored (the local partial is computed here)
 *   partial       : bf16 [R*m, N], written
 *   out           : bf16 [m, N], written
 * Requires N % 8 == 0, 1 <= topk <= 4, R*m*N*2 < 2^31, 16-byte aligned
 * bf16 pointers; workspace from ocg_workspace_bytes(OCG_OP_MOE_COMBINE_RS,
 * R, m, 0, N, 0, topk). Trace: kind 6 per task (a, b = rows [a, b) of the
 * order rotated to start at the local block, c = b - a for a local task,
 * else 0). Errors as for the other calls. */
int ocg_moe_combine_rs(ocg_handle h, const void* y, const float* topk_w, int R, int local_rank,
                       int64_t m, int64_t N, int topk, const void* const* peer_partials,
                       void* partial, void* out, void* ws, size_t ws_bytes,
                       const ocg_config* cfg, void* stream);

/* AllGather-KV attention (one context-parallel rank's share): "TileLink ...
 * (MLSys 2025 talk summary)", section "Experimental Setup & Results", names
 * an attention whose KV AllGather is overlapped with the attention itself;
 * the formula is the plain reading of unmasked softmax attention of the local
 * queries over the whole gathered sequence, with grouped kv heads:
 *   k_gathered = concat_r k_chunks[r],  v_gathered = concat_r v_chunks[r]
 *   out[i][h] = sum_j softmax_j( q[i][h] . k_gathered[j][h / G] / sqrt(d) )
 *               * v_gathered[j][h / G]                  (G = Hq / Hkv)
 * Scores and the softmax run in fp32 (running maximum and sum over key
 * blocks of 64), the probabilities enter the value product as bf16, and out
 * is rounded to bf16 (nearest-even).
 *   q            : bf16 [m, Hq, d], the local queries, read
 *   k_chunks[r], v_chunks[r] : bf16 [m, Hkv, d] of rank r (r = 0..R-1), read
 *   k_gathered, v_gathered   : bf16 [R*m, Hkv, d], written (every chunk, the
 *                  local one included)
 *   out          : bf16 [m, Hq, d], written
 * Copy tasks pull each peer chunk of keys and values into the gathered
 * buffers slab by slab (slab_rows tokens, default the whole chunk; tasks of
 * copy_rows tokens, default about 512 KiB of one tensor) and publish a flag
 * per slab; each tile (256 query rows of one kv head) starts
 * on the local chunk, read from its own shard, and before its first load of
 * a peer chunk waits on the flags of every peer chunk. Requires d == 128, Hq % Hkv == 0,
 * R*m*Hkv*d < 2^31, m*Hq*d < 2^31, 16-byte aligned pointers; workspace from
 * ocg_workspace_bytes(OCG_OP_AG_ATTENTION, R, m, Hq, Hkv, 0, 0). cfg.tile is
 * ignored; cfg.mode GEMM_ONLY runs the attention with every flag treated as
 * published (expects the gathered buffers filled), COPY_ONLY the copies.
 * Errors as for the other calls. */
int ocg_ag_attention(ocg_handle h, const void* q, const void* const* k_chunks, const void* const* v_chunks,
                     int R, int local_rank, int64_t m, int64_t Hq, int64_t Hkv, int64_t d,
                     void* k_gathered, void* v_gathered, void* out, void* ws, size_t ws_bytes,
                     const ocg_config* cfg, void* stream);

/* Stand-in for a peer's remote notify: writes `value` into `count` uint32
 * flags at `flags` (device) with release semantics, on `stream`. */
int ocg_signal(uint32_t* flags, int count, uint32_t value, void* stream);

/* After the stream has drained: returns OCG_ERR_TIMEOUT if any flag wait of
 * an earlier call on `workspace` exceeded its bound (and clears the record),
 * OCG_OK otherwise. Synchronous (reads one word). */
int ocg_check(ocg_handle h, void* workspace);

const char* ocg_status_string(int status);

/* ---- host-only planning queries (no GPU needed; used by tests/tools) ---- */

/* Resolved plan parameters for a call with config `cfg` (NULL = defaults) on
 * the device of `h` (its compute-unit count sizes the automatic choices;
 * h = NULL plans for a full 256-CU MI355X without touching any device): 
 * out[0]=tile preset, out[1]=BM, out[2]=BN, out[3]=slab rows,
 * out[4]=copy rows, out[5]=#copy tasks, out[6]=#tiles (static ops),
 * out[7]=#slabs. For OCG_OP_MOE_COMBINE_RS: out[0]=-1, out[3]=rows per
 * task outside the local block, out[4]=rows per local task, out[5]=#tasks,
 * out[6]=#local tasks (the first ones), the rest 0. For OCG_OP_AG_ATTENTION
 * (K = Hq, N = Hkv): out[0]=-1, out[1]=query rows per tile, out[2]=keys per
 * block, out[3]=slab tokens, out[4]=copy tokens, out[5]=#copy tickets (both
 * tensors), out[6]=#tiles, out[7]=#slabs. For GEMM_RS pass m = M. E and topk are the grouped GEMM's
 * expert count and picks per token (they choose its default tile; ignored
 * by the other ops). For OCG_OP_AG_GEMM, out[7] counts flags (slabs x
 * K-slabs) and the K-slab width and transfer mode are returned by
 * ocg_plan_ag(). Returns OCG_OK or an error. */
int ocg_plan_info(ocg_handle h, int op, int R, int local_rank, int64_t m, int64_t K, int64_t N, int E,
                  int topk, const ocg_config* cfg, int64_t out[8]);

/* AG-GEMM plan details: out[0] = K-slab columns, out[1] = #K-slabs,
 * out[2] = transfer mode the call would use (OCG_TRANSFER_INLINE or _SIDE),
 * out[3] = persistent GEMM workgroups, out[4] = producer workgroups (SIDE)
 * or 0, out[5] = copy tickets the GEMM kernel runs itself (the first K-slab
 * of the first copy phase under SIDE, all of them otherwise), out[6] =
 * gathered rows per round of tiles (copy phases), out[7] = K parts per tile
 * (1, or 2 when split). `h` as for ocg_plan_info. */
int ocg_plan_ag(ocg_handle h, int R, int local_rank, int64_t m, int64_t K, int64_t N, const ocg_config* cfg,
                int64_t out[8]);

/* Task at trace slot `ticket` of the AG-GEMM / GEMM-RS plan (slots as for
 * ocg_trace_rec: AG copies, then AG tiles; RS tiles, then RS strips):
 * desc[0]=kind (1 copy, 2 AG tile, 3 RS tile, 5 RS strip, 0 none),
 * copy: desc[1]=chunk, [2]=piece, [3]=row0, [4]=row1, [5]=slab, [6]=K-slab;
 * AG tile (a work unit: a tile, or one K half of it when split):
 *          desc[1]=rb, [2]=cb, [3]=#dependency slabs, [4..6]=first three
 *          dependency slab ids (-1 if none), [7]=K part (0, or 0/1 when split);
 * RS tile: desc[1]=rb, [2]=cb, [3]=local-block (0/1), [4]=XCD queue,
 *          [5]=ticket within the queue;
 * RS strip: desc[1]=row0, [2]=row1;
 * AG_ATTENTION (K = Hq, N = Hkv): copy ticket: desc[0]=1, [1..5] as for a
 *          copy, [6]=tensor (0 keys, 1 values); tile: desc[0]=7, [1]=kv
 *          head, [2]=row block, [3]=#flags each wave waits on, [4]=XCD
 *          queue, [5]=ticket within the queue. */
int ocg_plan_task(ocg_handle h, int op, int R, int local_rank, int64_t m, int64_t K, int64_t N,
                  const ocg_config* cfg, int64_t ticket, int64_t desc[8]);

#ifdef __cplusplus
}
#endif

#endif /* OCG_H_ */
