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
//     flags, no clearing).
// The flag store/load use release/acquire (the HIP memory model's form of
// the kernels' agent-coherent stores + vmcnt(0) + flag, and poll + acquire
// fence). --relaxed plants the mistake of a relaxed publish: TSan must then
// report a race. --skip-flag F never publishes flag F (a dead producer):
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
  int gemm_wgs = 8, side_wgs = 4, calls = 3, swizzle = 1, side = 1, skip_flag = -1, tpr = 8;
  bool relaxed = false;
  int timeout_ms = 200;
};

struct Workspace {
  std::atomic<uint32_t> ticket{0}, side_ticket{0}, done{0}, epoch{0}, error{0};
  std::atomic<uint32_t> xtick[kXcds];
  std::vector<std::atomic<uint32_t>> cnt, flag;
  std::vector<std::atomic<uint32_t>> published;   // per call: flags published (checked: exactly once)
  explicit Workspace(int nflags) : cnt(nflags), flag(nflags), published(nflags) {
    for (auto& q : xtick) q = 0;
    for (auto& c : cnt) c = 0;
    for (auto& f : flag) f = 0;
  }
};

struct Call {
  const Opts& o;
  AgPlan p;
  Workspace& ws;
  const std::vector<std::vector<uint16_t>>& chunks;
  std::vector<uint16_t>& gathered;
  std::atomic<int> bad_reads{0};
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
  void wait_flag(int f, uint32_t epoch) {
    const auto t0 = std::chrono::steady_clock::now();
    const auto mo = o.relaxed ? std::memory_order_relaxed : std::memory_order_acquire;
    while (ws.flag[f].load(mo) != epoch) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(o.timeout_ms)) {
        ws.error.fetch_or(1, std::memory_order_relaxed);
        return;
      }
      std::this_thread::yield();
    }
  }

  int next_tile(int* q) {
    for (;;) {
      const int t = (int)ws.xtick[*q].fetch_add(1, std::memory_order_relaxed);
      const int v = xcd_tile(*q, t, p.n_tiles);
      if (v >= 0) return v;
      uint32_t mask = 0;
      for (int x = 0; x < kXcds; ++x)
        if (xcd_tile(x, (int)ws.xtick[x].load(std::memory_order_relaxed), p.n_tiles) >= 0) mask |= 1u << x;
      if (!mask) return -1;
      int n = (*q + 1) % kXcds;
      while (!(mask >> n & 1)) n = (n + 1) % kXcds;
      *q = n;
    }
  }

  void tile(int v, uint32_t epoch) {
    int rb, cb;
    tile_of(p.n_rb, p.n_cb, p.rb0, v, &rb, &cb);
    (void)cb;
    const int r0 = rb * p.BM, r1 = std::min(r0 + p.BM, p.M);
    std::vector<int> deps;
    if (p.mode == 0) for_each_dep_slab(p.m, p.S, p.bpr, p.local, r0, r1, [&](int s) { deps.push_back(s); });
    for (int j = 0; j < p.nks; ++j) {
      for (int s : deps) wait_flag(s * p.nks + j, epoch);
      const int k0 = j * p.KS, k1 = std::min(k0 + p.KS, p.K);
      // the tile's loads of this K-slab: local rows from the shard, the
      // others from the gathered buffer (plain loads)
      for (int r = r0; r < r1; ++r) {
        const int c = r / p.m;
        const uint16_t* want = chunks[c].data() + (size_t)(r - c * p.m) * p.K;
        const uint16_t* got = (c == p.local) ? want : &gathered[(size_t)r * p.K];
        for (int k = k0; k < k1; k += 37)
          if (got[k] != want[k]) bad_reads.fetch_add(1, std::memory_order_relaxed);
      }
    }
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
    else if (a == "--timeout-ms") o.timeout_ms = next();
    else { std::fprintf(stderr, "unknown option %s\n", a.c_str()); return 2; }
  }
  AgPlan p = make_ag_plan(o.R, o.local, o.m, o.K, o.N, o.BM, o.BN, o.S, o.CT, o.swizzle, 0, o.KS, o.tpr);
  if (o.side) p.n_inline = std::min(first_kslab_tickets(p), p.n_copy);
  const int nflags = p.R * p.bpr * p.nks;
  std::vector<std::vector<uint16_t>> chunks(o.R, std::vector<uint16_t>((size_t)o.m * o.K));
  Workspace ws(nflags);
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
    std::printf("call %d: epoch %u, copies %d (inline %d), tiles %d, flags %d, bad reads %d, rows wrong %d, "
                "flag publish counts off %d, error word %u\n",
                call, ws.epoch.load(), p.n_copy, p.n_inline, p.n_tiles, nflags, c.bad_reads.load(), missing, dup, err);
    if (missing || dup || (!want_err && c.bad_reads.load()) || (err != 0) != want_err) ++failures;
    if (ws.epoch.load() != (uint32_t)(call + 1)) ++failures;
  }
  std::printf(failures ? "FAILED\n" : "ok\n");
  return failures ? 1 : 0;
}
