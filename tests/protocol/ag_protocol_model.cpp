// CPU model of the AG-GEMM copy / flag protocol, for ThreadSanitizer.
//
// Each std::thread plays one persistent workgroup and runs the same
// protocol as the kernels, on the same closed-form schedule (sched.h):
//   * copy tasks taken from the ticket counters (GEMM "kernel": tickets below
//     n_inline; side producer "kernel": the rest), each moving its rows x
//     K-slab columns of a rank chunk into the gathered buffer with plain
//     stores, then produce_tile_notify: bump the (slab, K-slab) counter and,
//     as the last task of that flag, reset it and store flag = epoch;
//   * tiles from the per-XCD queues, each waiting (bounded) on the K-slab
//     flags of the peer slabs it reads before reading those columns -- the
//     reads are plain loads, so a read not ordered after its publish is a
//     data race that TSan reports;
//   * the last workgroup of every "kernel" of the call resets the counters
//     and records the epoch; calls repeat on one workspace (epoch-tagged
//     flags, no clearing);
//   * --split: tiles run as two K-half units (split K). Each half sums the
//     values it reads; the half that arrives first at the tile's counter
//     stores its sum with a plain store and publishes the tile's flag, the
//     other resets the counter, waits (bounded) on the flag and adds the
//     stored sum to its own, which must equal the tile's exact sum.
// The flag store/load use release/acquire (the HIP memory model's form of
// the kernels' agent-coherent stores + vmcnt(0) + flag, and poll + acquire
// fence). --relaxed plants the mistake of a relaxed publish: TSan must then
// report a race; --relaxed-split plants it in the split-K combine only. --skip-flag F never publishes flag F (a dead producer):
// every wait on it must time out, the error word must be set, and every
// thread must still finish. Exit status: 0 when the run checks out (every
// tile read the right bytes, every flag published once per call, the error
// word as expected), 1 otherwise.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../communication_overlapped_gemm_amd/csrc/sched.h"

using namespace ocg;

struct Opts {
  int R = 4, local = 1, m = 96, K = 1024, N = 256, BM = 64, BN = 64, S = 32, CT = 16, KS = 256;
  int gemm_wgs = 8, side_wgs = 4, calls = 3, swizzle = 1, side = 1, skip_flag = -1, tpr = 8, sk = 1;
  bool relaxed = false, relaxed_split = false;
  int timeout_ms = 200;
};

struct Workspace {
  std::atomic<uint32_t> ticket{0}, side_ticket{0}, done{0}, epoch{0}, error{0};
  std::atomic<uint32_t> xtick[kXcds];
  std::vector<std::atomic<uint32_t>> cnt, flag;
  std::vector<std::atomic<uint32_t>> published;   // per call: flags published (checked: exactly once)
  std::vector<std::atomic<uint32_t>> sk_cnt, sk_flag;   // split K, per tile: halves arrived, first half stored
  std::vector<uint64_t> sk_part;                        // split K, per tile: the first half's sum (plain data)
  Workspace(int nflags, int ntiles)
      : cnt(nflags), flag(nflags), published(nflags), sk_cnt(ntiles), sk_flag(ntiles), sk_part(ntiles, 0) {
    for (auto& q : xtick) q = 0;
    for (auto& c : cnt) c = 0;
    for (auto& f : flag) f = 0;
    for (auto& c : sk_cnt) c = 0;
    for (auto& f : sk_flag) f = 0;
  }
};

struct Call {
  const Opts& o;
  AgPlan p;
  Workspace& ws;
  const std::vector<std::vector<uint16_t>>& chunks;
  std::vector<uint16_t>& gathered;
  std::atomic<int> bad_reads{0};
  std::atomic<int> bad_sums{0}, combined{0};   // split K: tiles combined, wrong combined sums
  int total_wgs;

  Call(const Opts& o_, const AgPlan& p_, Workspace& w, const std::vector<std::vector<uint16_t>>& c,
       std::vector<uint16_t>& g, int total)
      : o(o_), p(p_), ws(w), chunks(c), gathered(g), total_wgs(total) {}

  void copy_task(int u, uint32_t epoch) {
    const CopyDesc d = copy_desc(p, u);
    for (int r = d.row0; r < d.row1; ++r) {
      const uint16_t* src = chunks[d.chunk].data() + (size_t)(r - d.chunk * p.m) * p.K;
      std::memcpy(&gathered[(size_t)r * p.K + d.k0], src + d.k0, (size_t)(d.k1 - d.k0) * 2);
    }
    const uint32_t target = (uint32_t)slab_target(p.m, p.S, p.CT, p.bpr, d.slab);
    const uint32_t old = ws.cnt[d.flag].fetch_add(1, std::memory_order_acq_rel);
    if (old + 1 == target) {
      ws.cnt[d.flag].store(0, std::memory_order_relaxed);
      if (d.flag != o.skip_flag) {
        ws.flag[d.flag].store(epoch, o.relaxed ? std::memory_order_relaxed : std::memory_order_release);
        ws.published[d.flag].fetch_add(1, std::memory_order_relaxed);
      }
    }
  }

  // consume_tile_wait: bounded poll; on timeout record the error and go on
  void wait_flag(int f, uint32_t epoch) { wait_on(ws.flag[f], epoch, o.relaxed); }

  void wait_on(std::atomic<uint32_t>& flag, uint32_t epoch, bool relaxed) {
    const auto t0 = std::chrono::steady_clock::now();
    const auto mo = relaxed ? std::memory_order_relaxed : std::memory_order_acquire;
    while (flag.load(mo) != epoch) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(o.timeout_ms)) {
        ws.error.fetch_or(1, std::memory_order_relaxed);
        return;
      }
      std::this_thread::yield();
    }
  }

  // next work unit: a tile, or (split K) one K half of a tile
  int next_tile(int* q) {
    const int n = p.n_tiles * p.sk;
    for (;;) {
      const int t = (int)ws.xtick[*q].fetch_add(1, std::memory_order_relaxed);
      const int v = xcd_tile(*q, t, n);
      if (v >= 0) return v;
      uint32_t mask = 0;
      for (int x = 0; x < kXcds; ++x)
        if (xcd_tile(x, (int)ws.xtick[x].load(std::memory_order_relaxed), n) >= 0) mask |= 1u << x;
      if (!mask) return -1;
      int n = (*q + 1) % kXcds;
      while (!(mask >> n & 1)) n = (n + 1) % kXcds;
      *q = n;
    }
  }

  // Sum of the tile's rows over columns [k0, k1) from the chunks themselves.
  uint64_t exact_sum(int r0, int r1, int k0, int k1) const {
    uint64_t s = 0;
    for (int r = r0; r < r1; ++r) {
      const int c = r / p.m;
      const uint16_t* want = chunks[c].data() + (size_t)(r - c * p.m) * p.K;
      for (int k = k0; k < k1; ++k) s += want[k];
    }
    return s;
  }

  // A work unit u: tile u / sk, K part u % sk (columns of that part only).
  void tile(int u, uint32_t epoch) {
    const int v = u / p.sk, part = u % p.sk;
    int rb, cb;
    tile_of(p.n_rb, p.n_cb, p.rb0, v, &rb, &cb);
    (void)cb;
    const int r0 = rb * p.BM, r1 = std::min(r0 + p.BM, p.M);
    const int kp0 = part * (p.K / p.sk), kp1 = kp0 + p.K / p.sk;
    std::vector<int> deps;
    if (p.mode == 0) for_each_dep_slab(p.m, p.S, p.bpr, p.local, r0, r1, [&](int s) { deps.push_back(s); });
    uint64_t sum = 0;
    for (int j = 0; j < p.nks; ++j) {
      const int k0 = std::max(j * p.KS, kp0), k1 = std::min(std::min((j + 1) * p.KS, p.K), kp1);
      if (k0 >= k1) continue;
      for (int s : deps) wait_flag(s * p.nks + j, epoch);
      // the unit's loads of this K-slab: local rows from the shard, the
      // others from the gathered buffer (plain loads)
      for (int r = r0; r < r1; ++r) {
        const int c = r / p.m;
        const uint16_t* want = chunks[c].data() + (size_t)(r - c * p.m) * p.K;
        const uint16_t* got = (c == p.local) ? want : &gathered[(size_t)r * p.K];
        for (int k = k0; k < k1; ++k) {
          if (p.sk == 1 && (k - k0) % 37) continue;   // whole tiles: a sample of the columns
          if (got[k] != want[k]) bad_reads.fetch_add(1, std::memory_order_relaxed);
          sum += got[k];
        }
      }
    }
    if (p.sk == 1) return;
    // combine the halves: the first stores its sum and publishes, the second adds it
    const uint32_t before = ws.sk_cnt[v].fetch_add(1, std::memory_order_relaxed);
    if (before == 0) {
      ws.sk_part[v] = sum;
      const bool rx = o.relaxed || o.relaxed_split;
      ws.sk_flag[v].store(epoch, rx ? std::memory_order_relaxed : std::memory_order_release);
      return;
    }
    ws.sk_cnt[v].store(0, std::memory_order_relaxed);
    wait_on(ws.sk_flag[v], epoch, o.relaxed || o.relaxed_split);
    if (sum + ws.sk_part[v] != exact_sum(r0, r1, 0, p.K)) bad_sums.fetch_add(1, std::memory_order_relaxed);
    combined.fetch_add(1, std::memory_order_relaxed);
  }

  void finish(uint32_t epoch) {
    const uint32_t d = ws.done.fetch_add(1, std::memory_order_acq_rel);
    if ((int)d + 1 == total_wgs) {
      ws.ticket.store(0, std::memory_order_relaxed);
      ws.side_ticket.store(0, std::memory_order_relaxed);
      for (auto& q : ws.xtick) q.store(0, std::memory_order_relaxed);
      ws.done.store(0, std::memory_order_relaxed);
      ws.epoch.store(epoch, std::memory_order_release);
    }
  }

  uint32_t read_epoch() {
    const uint32_t e = ws.epoch.load(std::memory_order_acquire) + 1;
    return e ? e : 1;
  }

  void gemm_wg(int id) {
    const uint32_t epoch = read_epoch();
    for (;;) {
      const int u = (int)ws.ticket.fetch_add(1, std::memory_order_relaxed);
      if (u >= p.n_inline) break;
      copy_task(u, epoch);
    }
    int q = id % kXcds;
    for (int v; (v = next_tile(&q)) >= 0;) tile(v, epoch);
    finish(epoch);
  }

  void side_wg() {
    const uint32_t epoch = read_epoch();
    for (;;) {
      const int u = p.n_inline + (int)ws.side_ticket.fetch_add(1, std::memory_order_relaxed);
      if (u >= p.n_copy) break;
      copy_task(u, epoch);
    }
    finish(epoch);
  }
};

int main(int argc, char** argv) {
  Opts o;
  for (int i = 1; i < argc; ++i) {
    const std::string a = argv[i];
    auto next = [&]() { return std::atoi(argv[++i]); };
    if (a == "--relaxed") o.relaxed = true;
    else if (a == "--inline") o.side = 0;
    else if (a == "--natural") o.swizzle = 0;
    else if (a == "--skip-flag") o.skip_flag = next();
    else if (a == "--local") o.local = next();
    else if (a == "--calls") o.calls = next();
    else if (a == "--kslab") o.KS = next();
    else if (a == "--split") o.sk = 2;
    else if (a == "--relaxed-split") o.relaxed_split = true;
    else if (a == "--timeout-ms") o.timeout_ms = next();
    else { std::fprintf(stderr, "unknown option %s\n", a.c_str()); return 2; }
  }
  if (o.sk == 2) {   // split K: inline copies, one K-slab
    o.side = 0;
    o.KS = o.K;
  }
  AgPlan p = make_ag_plan(o.R, o.local, o.m, o.K, o.N, o.BM, o.BN, o.S, o.CT, o.swizzle, 0, o.KS, o.tpr, o.sk);
  if (o.side) p.n_inline = std::min(first_kslab_tickets(p), p.n_copy);
  const int nflags = p.R * p.bpr * p.nks;
  std::vector<std::vector<uint16_t>> chunks(o.R, std::vector<uint16_t>((size_t)o.m * o.K));
  Workspace ws(nflags, p.n_tiles);
  int failures = 0;
  for (int call = 0; call < o.calls; ++call) {
    // fresh data every call: a stale gathered row from the previous call
    // would be read as a bad value if a wait were skipped
    for (int r = 0; r < o.R; ++r)
      for (size_t i = 0; i < chunks[r].size(); ++i) chunks[r][i] = (uint16_t)(1 + (i * 7 + r * 131 + call * 977) % 60000);
    std::vector<uint16_t> gathered((size_t)p.M * o.K, 0);
    for (auto& x : ws.published) x = 0;
    const int side_wgs = (o.side && p.n_copy > p.n_inline) ? o.side_wgs : 0;
    Call c(o, p, ws, chunks, gathered, o.gemm_wgs + side_wgs);
    std::vector<std::thread> th;
    for (int g = 0; g < o.gemm_wgs; ++g) th.emplace_back([&c, g] { c.gemm_wg(g); });
    for (int s = 0; s < side_wgs; ++s) th.emplace_back([&c] { c.side_wg(); });
    for (auto& t : th) t.join();   // kernel boundary
    // every peer row of the gathered buffer landed; every flag once
    int missing = 0, dup = 0;
    for (int f = 0; f < nflags; ++f) {
      const uint32_t n = ws.published[f].load();
      if (f == o.skip_flag ? n != 0 : n != 1) ++dup;
    }
    for (int r = 0; r < p.M; ++r) {
      const int ch = r / p.m;
      if (std::memcmp(&gathered[(size_t)r * o.K], chunks[ch].data() + (size_t)(r - ch * p.m) * o.K, (size_t)o.K * 2))
        ++missing;
    }
    const uint32_t err = ws.error.exchange(0);
    // a skipped flag of a peer's slab is waited on by tiles (timeout expected);
    // one of the local chunk is waited on by nobody
    const bool want_err = o.skip_flag >= 0 && (o.skip_flag / p.nks) / p.bpr != p.local;
    std::printf("call %d: epoch %u, copies %d (inline %d), tiles %d x %d parts, flags %d, bad reads %d, rows wrong %d, "
                "flag publish counts off %d, split tiles combined %d (wrong sums %d), error word %u\n",
                call, ws.epoch.load(), p.n_copy, p.n_inline, p.n_tiles, p.sk, nflags, c.bad_reads.load(), missing, dup,
                c.combined.load(), c.bad_sums.load(), err);
    if (missing || dup || (!want_err && c.bad_reads.load()) || (err != 0) != want_err) ++failures;
    if (p.sk == 2 && !want_err && (c.combined.load() != p.n_tiles || c.bad_sums.load())) ++failures;
    if (ws.epoch.load() != (uint32_t)(call + 1)) ++failures;
  }
  std::printf(failures ? "FAILED\n" : "ok\n");
  return failures ? 1 : 0;
}
