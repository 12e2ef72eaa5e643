// Randomised bookkeeping driver for libkvc's host allocator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only; the
// device launchers are stubbed out and never reached).  Every operation of
// the public C ABI that touches the allocator -- add, fork, free, reserve
// (the append's slot reservation with copy-on-write), truncate, batched
// truncate, evict -- runs in random order on small pools, and after each one
// the invariants of a refcounted block table are checked from the outside:
//   - a block's refcount is the number of live tables that hold it, so the
//     blocks in use and the shared ones match the library's statistics, and
//     free + used = all blocks;
//   - every slot a reservation returns lies in a block only its sequence holds;
//   - a call that fails changes nothing (tables and statistics as before).
// Prints "ok <operations>" and exits 0, or names the first broken invariant.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "kvc.h"
#include "../../paged_kv_cache_split_amd/csrc/kvc_internal.h"

namespace kvc {
hipError_t launch_copy_blocks(const PoolDesc&, const CowPair*, int32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_append(const PoolDesc&, const AppendSegment*, const InlineSegments*, int32_t, const void*,
                         const void*, kvc_dtype, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const PoolDesc&, int32_t, const DecodePlan&, const void*, kvc_dtype, const int32_t*, int32_t,
                         const int32_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t, float, void*, void*,
                         const void*, const void*, hipEvent_t, hipEvent_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_stream_copy(void*, const void*, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_stream_read(const void*, size_t, uint32_t*, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t static_scratch(void**) { return hipErrorNotSupported; }
}  // namespace kvc

namespace {

struct Snapshot {
  std::map<int64_t, std::vector<int32_t>> tables;
  std::map<int64_t, int32_t> lens;
  kvc_stats_t stats;
  bool operator==(const Snapshot& o) const {
    return tables == o.tables && lens == o.lens && stats.used_blocks == o.stats.used_blocks &&
           stats.free_blocks == o.stats.free_blocks && stats.shared_blocks == o.stats.shared_blocks &&
           stats.num_seqs == o.stats.num_seqs;
  }
};

[[noreturn]] void die(const char* what, int trial, long op) {
  std::printf("FAIL trial %d op %ld: %s (%s)\n", trial, op, what, kvc_last_error());
  std::exit(1);
}

Snapshot snap(kvc_cache* c, const std::vector<int64_t>& live, int nb) {
  Snapshot s;
  std::vector<int32_t> buf(nb + 64);
  for (int64_t id : live) {
    int32_t n = 0, len = 0;
    if (kvc_get_table(c, id, buf.data(), (int32_t)buf.size(), &n, &len) != KVC_OK) die("get_table", -1, -1);
    s.tables[id].assign(buf.begin(), buf.begin() + n);
    s.lens[id] = len;
  }
  if (kvc_stats(c, &s.stats) != KVC_OK) die("stats", -1, -1);
  return s;
}

void check(const Snapshot& s, int nb, int bs, int trial, long op) {
  std::vector<int> ref(nb, 0);
  for (const auto& [id, t] : s.tables) {
    const int32_t len = s.lens.at(id);
    if ((int64_t)t.size() * bs < len) die("table shorter than the length", trial, op);
    std::vector<char> seen(nb, 0);
    for (int32_t b : t) {
      if (b == -1) continue;
      if (b < 0 || b >= nb) die("block id out of range", trial, op);
      if (seen[b]) die("a block twice in one table", trial, op);
      seen[b] = 1;
      ++ref[b];
    }
  }
  int used = 0, shared = 0;
  for (int r : ref) used += r >= 1, shared += r >= 2;
  if (used != s.stats.used_blocks) die("used blocks differ from the tables", trial, op);
  if (shared != s.stats.shared_blocks) die("shared blocks differ from the tables", trial, op);
  if (s.stats.used_blocks + s.stats.free_blocks != nb) die("free + used != all blocks", trial, op);
  if ((int64_t)s.tables.size() != s.stats.num_seqs) die("sequence count", trial, op);
}

}  // namespace

int main() {
  long ops = 0;
  for (int trial = 0; trial < 60; ++trial) {
    std::mt19937_64 rng(1000 + trial);
    auto uni = [&](int lo, int hi) { return (int)std::uniform_int_distribution<int>(lo, hi)(rng); };
    const int bs = (trial % 3 == 0) ? 16 : (trial % 3 == 1 ? 4 : 1);
    const int nb = uni(8, 90);
    std::vector<int32_t> order(nb);
    for (int i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    kvc_config cfg{};
    cfg.num_layers = 1;
    cfg.num_kv_heads = 2;
    cfg.head_dim = 64;
    cfg.block_size = bs;
    cfg.num_blocks = nb;
    cfg.kv_dtype = KVC_BF16;
    cfg.free_order = (trial & 1) ? order.data() : nullptr;
    kvc_cache* c = nullptr;
    if (kvc_create(&cfg, &c) != KVC_OK) die("create", trial, 0);
    std::vector<int64_t> live;
    int64_t next_id = 0;
    for (int step = 0; step < 400; ++step, ++ops) {
      const Snapshot before = snap(c, live, nb);
      const int op = uni(0, 99);
      kvc_status st = KVC_OK;
      bool may_fail_quietly = true;   // a failure must leave everything unchanged
      if (op < 18 || live.empty()) {
        st = kvc_add_seq(c, next_id, uni(0, 3 * bs + 5));
        if (st == KVC_OK) live.push_back(next_id);
        ++next_id;
      } else if (op < 28) {
        const int64_t p = live[uni(0, (int)live.size() - 1)];
        st = kvc_fork(c, p, next_id);
        if (st == KVC_OK) live.push_back(next_id);
        ++next_id;
      } else if (op < 38) {
        const int i = uni(0, (int)live.size() - 1);
        st = kvc_free_seq(c, live[i]);
        if (st == KVC_OK) live.erase(live.begin() + i);
      } else if (op < 70) {
        // reservation for a random subset (distinct ids), several rows each
        std::vector<int64_t> ids;
        std::vector<int32_t> n_new;
        for (int64_t id : live)
          if (uni(0, 2) == 0) ids.push_back(id), n_new.push_back(uni(0, 2 * bs + 3));
        if (ids.empty()) continue;
        int64_t total = 0;
        for (int32_t x : n_new) total += x;
        std::vector<int32_t> slots(total + 1), src(ids.size() + total + 1), dst(ids.size() + total + 1);
        int32_t ncow = 0;
        st = kvc_reserve_host(c, (int32_t)ids.size(), ids.data(), n_new.data(), slots.data(), src.data(), dst.data(),
                              (int32_t)src.size(), &ncow);
        if (st == KVC_OK) {
          const Snapshot after = snap(c, live, nb);
          std::vector<int> ref(nb, 0);
          for (const auto& [id, t] : after.tables)
            for (int32_t b : t)
              if (b >= 0) ++ref[b];
          for (int64_t k = 0; k < total; ++k) {
            const int32_t b = slots[k] / bs;
            if (b < 0 || b >= nb || ref[b] != 1) die("a reserved slot in a shared or foreign block", trial, step);
          }
        }
      } else if (op < 80) {
        const int64_t id = live[uni(0, (int)live.size() - 1)];
        const int32_t len = before.lens.at(id);
        st = kvc_truncate(c, id, uni(0, len));
      } else if (op < 90) {
        std::vector<int64_t> ids;
        std::vector<int32_t> to;
        for (int64_t id : live)
          if (uni(0, 1)) ids.push_back(id), to.push_back(uni(0, before.lens.at(id)));
        if (uni(0, 9) == 0 && !ids.empty()) ids.push_back(ids[0]), to.push_back(0);   // a repeated id: rejected
        st = kvc_truncate_many(c, (int32_t)ids.size(), ids.data(), to.data());
      } else {
        const int64_t id = live[uni(0, (int)live.size() - 1)];
        st = kvc_evict(c, id, uni(0, before.lens.at(id)));
      }
      const Snapshot after = snap(c, live, nb);
      if (st != KVC_OK && may_fail_quietly && !(after == before)) die("a failed call changed the state", trial, step);
      check(after, nb, bs, trial, step);
    }
    for (int64_t id : live)
      if (kvc_free_seq(c, id) != KVC_OK) die("final free", trial, -1);
    kvc_stats_t s;
    kvc_stats(c, &s);
    if (s.used_blocks != 0 || s.free_blocks != nb) die("blocks left after freeing everything", trial, -1);
    kvc_destroy(c);
  }
  std::printf("ok %ld\n", ops);
  return 0;
}
