// Host half of libkvc: configuration, validation, the block allocator
// (free list, per-sequence block tables, refcounts, copy-on-write), append
// planning, device uploads and kernel dispatch.
//
// Allocator semantics follow the BlockTable class of
// "大模型推理加速核心KV Cache 复用机制与内存布局优化" §三 (allocate / fork / free with
// refcounts; allocation fails as a whole when the free list is short, which
// is where a scheduler would preempt) and the RequestBlockTable of
// "LLM推理优化实战：从KV-Cache到Continuous Batching的技术演进与代码实现" §2.2 (position p
// lives in logical block p / block_size).  Copy-on-write on the first write
// into a shared block follows the same pages and "大模型推理加速——KV Cache篇" §6.1.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "kvc_internal.h"

using kvc::AppendSegment;
using kvc::CowPair;

namespace {

thread_local std::string g_last_error;

kvc_status fail(kvc_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvc_status fail(kvc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvc_status ok() {
  g_last_error.clear();
  return KVC_OK;
}

bool valid_dtype(int t) { return t >= KVC_F32 && t <= KVC_INT8; }

// Caches of one-byte codes with per-(block, KV head) scales.
bool is_quantised(kvc_dtype t) { return t == KVC_FP8_E4M3 || t == KVC_INT8; }

constexpr int kDeviceBlockSize = 16;

using kvc::align256;

// Upper bound on the segments (and copy pairs) an append of `tokens` rows over
// `batch` sequences produces with 16-token blocks: each sequence's run of n
// rows touches at most n / 16 + 2 blocks.
int64_t max_segments(int64_t batch, int64_t tokens) { return tokens / kDeviceBlockSize + 2 * batch + 1; }

}  // namespace

struct kvc_cache {
  kvc_config cfg;
  std::mutex mu;

  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
  };
  std::vector<int32_t> free_list;  // blocks are taken from the back
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t used = 0;
  int64_t peak_used = 0;
  int64_t cow_copies = 0;

  // Pinned staging for host->device uploads; `staging_free` is recorded
  // after the last copy that reads it.
  void* staging = nullptr;
  size_t staging_bytes = 0;
  hipEvent_t staging_free = nullptr;

  kvc::PoolDesc pool() const {
    kvc::PoolDesc p;
    p.k = static_cast<char*>(cfg.k_pool);
    p.v = static_cast<char*>(cfg.v_pool);
    p.k_scale = cfg.k_scale;
    p.v_scale = cfg.v_scale;
    p.num_layers = cfg.num_layers;
    p.num_blocks = cfg.num_blocks;
    p.num_kv_heads = cfg.num_kv_heads;
    p.head_dim = cfg.head_dim;
    p.block_size = cfg.block_size;
    p.dtype = cfg.kv_dtype;
    return p;
  }

  int32_t pop_block() {
    int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    ++used;
    peak_used = std::max(peak_used, used);
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] == 0) {
      free_list.push_back(b);
      --used;
    }
  }
};

namespace {

// Waits until the previous upload has consumed the staging buffer, then
// makes it at least `bytes` long.
kvc_status staging_acquire(kvc_cache* c, size_t bytes) {
  if (c->staging_free) {
    hipError_t e = hipEventSynchronize(c->staging_free);
    if (e != hipSuccess) return fail(KVC_E_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
  } else {
    hipError_t e = hipEventCreateWithFlags(&c->staging_free, hipEventDisableTiming);
    if (e != hipSuccess) {
      c->staging_free = nullptr;
      return fail(KVC_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  if (c->staging_bytes < bytes) {
    if (c->staging) (void)hipHostFree(c->staging);
    c->staging = nullptr;
    c->staging_bytes = 0;
    size_t want = std::max(bytes, size_t(1) << 16);
    hipError_t e = hipHostMalloc(&c->staging, want, hipHostMallocDefault);
    if (e != hipSuccess) {
      c->staging = nullptr;
      return fail(KVC_E_HIP, "hipHostMalloc(%zu): %s", want, hipGetErrorString(e));
    }
    c->staging_bytes = want;
  }
  return KVC_OK;
}

kvc_status staging_upload(kvc_cache* c, void* dst_dev, size_t bytes, hipStream_t s) {
  hipError_t e = hipMemcpyAsync(dst_dev, c->staging, bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(KVC_E_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  e = hipEventRecord(c->staging_free, s);
  if (e != hipSuccess) return fail(KVC_E_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  return KVC_OK;
}

struct AppendPlan {
  std::vector<int32_t> slots;
  std::vector<CowPair> cow;
  std::vector<AppendSegment> segs;
};

// The bookkeeping of an append.  Validates, counts the blocks it needs
// (fresh blocks past a table's end plus private copies of shared blocks), and
// only then takes them, so a failing call changes nothing.
kvc_status plan_append(kvc_cache* c, int32_t batch, const int64_t* ids, const int32_t* n_new, bool want_slots,
                       int64_t cow_capacity, AppendPlan* plan) {
  if (batch < 0) return fail(KVC_E_INVALID, "batch must be >= 0");
  if (batch > 0 && !ids) return fail(KVC_E_INVALID, "seq_ids is NULL");
  const int32_t bs = c->cfg.block_size;
  std::vector<kvc_cache::Seq*> seqs(batch);
  {
    std::unordered_set<int64_t> seen;
    seen.reserve(batch * 2 + 1);
    for (int32_t i = 0; i < batch; ++i) {
      if (!seen.insert(ids[i]).second) return fail(KVC_E_INVALID, "sequence %lld listed twice", (long long)ids[i]);
      auto it = c->seqs.find(ids[i]);
      if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)ids[i]);
      seqs[i] = &it->second;
      int32_t n = n_new ? n_new[i] : 1;
      if (n < 0) return fail(KVC_E_INVALID, "n_new[%d] < 0", i);
      if ((int64_t)seqs[i]->len + n > (int64_t)INT32_MAX - bs)
        return fail(KVC_E_INVALID, "sequence %lld would exceed the maximum length", (long long)ids[i]);
    }
  }
  // Dry run: how many blocks will be popped, and how many copy pairs issued.
  int64_t need = 0, pairs = 0;
  std::unordered_map<int32_t, int32_t> drop;  // references a copy-on-write already released, per block
  for (int32_t i = 0; i < batch; ++i) {
    const kvc_cache::Seq& s = *seqs[i];
    int32_t n = n_new ? n_new[i] : 1;
    if (n == 0) continue;
    int64_t first = s.len / bs, last = ((int64_t)s.len + n - 1) / bs;
    for (int64_t idx = first; idx <= last; ++idx) {
      if (idx >= (int64_t)s.blocks.size()) {
        ++need;
      } else {
        int32_t b = s.blocks[idx];
        if (b < 0)
          return fail(KVC_E_INVALID, "sequence %lld would write into a released block", (long long)ids[i]);
        int32_t r = c->ref[b] - drop[b];
        if (r > 1) {
          ++need;
          ++drop[b];
          int64_t first_pos = std::max<int64_t>(s.len, idx * bs);
          if (first_pos % bs != 0) ++pairs;
        }
      }
    }
  }
  if (need > (int64_t)c->free_list.size())
    return fail(KVC_E_NO_BLOCKS, "append needs %lld free blocks, %zu available", (long long)need,
                c->free_list.size());
  if (pairs > cow_capacity)
    return fail(KVC_E_INVALID, "append needs %lld copy pairs, capacity %lld", (long long)pairs,
                (long long)cow_capacity);
  // Commit, in the same order as the dry run.
  int64_t total = 0;
  for (int32_t i = 0; i < batch; ++i) total += n_new ? n_new[i] : 1;
  if (want_slots) plan->slots.reserve(total);
  int32_t row = 0;
  for (int32_t i = 0; i < batch; ++i) {
    kvc_cache::Seq& s = *seqs[i];
    int32_t n = n_new ? n_new[i] : 1;
    int32_t p = s.len, end = s.len + n;
    while (p < end) {
      int32_t idx = p / bs, off = p % bs;
      int32_t run = std::min(end - p, bs - off);
      if (idx == (int32_t)s.blocks.size()) {
        s.blocks.push_back(c->pop_block());
      } else if (c->ref[s.blocks[idx]] > 1) {
        int32_t old = s.blocks[idx];
        int32_t fresh = c->pop_block();
        c->release(old);
        s.blocks[idx] = fresh;
        if (off > 0) {
          plan->cow.push_back({old, fresh});
          ++c->cow_copies;
        }
      }
      int32_t blk = s.blocks[idx];
      plan->segs.push_back({blk, off, run, row});
      if (want_slots)
        for (int32_t k = 0; k < run; ++k) plan->slots.push_back(blk * bs + off + k);
      row += run;
      p += run;
    }
    s.len = end;
  }
  return KVC_OK;
}

kvc_status check_device_ready(const kvc_cache* c) {
  const kvc_config& f = c->cfg;
  if (f.block_size != kDeviceBlockSize)
    return fail(KVC_E_UNSUPPORTED, "device work needs block_size 16 (cache has %d)", f.block_size);
  if (!f.k_pool || !f.v_pool) return fail(KVC_E_INVALID, "pools are NULL (bookkeeping-only cache)");
  if (is_quantised(f.kv_dtype) && (!f.k_scale || !f.v_scale))
    return fail(KVC_E_INVALID, "an fp8 or int8 cache needs k_scale and v_scale");
  return KVC_OK;
}

int32_t auto_partition_tokens(int32_t batch, int32_t num_kv_heads, int32_t max_context_len) {
  // Enough partitions to give the chip many waves, few enough to keep the
  // merge small: start at 256 tokens and grow while there are over ~8 waves
  // per CU-SIMD slot's worth of work items (2048 slots on 256 CUs).
  int64_t pt = 256;
  while (pt < 1024) {
    int64_t parts = (max_context_len + pt - 1) / pt;
    if ((int64_t)batch * num_kv_heads * parts <= 16384) break;
    pt *= 2;
  }
  return (int32_t)pt;
}

// kv: the cache dtype, or -1 when unknown (workspace sizing without a cache:
// then the larger default wave count is assumed).
bool plan_decode(int32_t batch, int32_t num_kv_heads, int32_t max_context_len, int32_t kernel, int kv,
                 const kvc_decode_opts* opts, kvc::DecodePlan* plan) {
  int32_t pt = (opts && opts->partition_tokens > 0) ? opts->partition_tokens
                                                    : auto_partition_tokens(batch, num_kv_heads, max_context_len);
  if (pt % kDeviceBlockSize != 0 || pt > 1024) return false;
  if (opts && opts->work_items < 0) return false;
  if (opts && (opts->pool_shift < 0 || opts->pool_shift > 6 || opts->pool_pieces > 64)) return false;
  plan->kernel = kernel;
  plan->split_steps = 0;
  plan->max_pieces = 1;
  plan->skip_blocks = 0;
  plan->pre_groups = 0;
  plan->pre_split_steps = 0;
  plan->pre_pieces = 0;
  plan->partition_tokens = pt;
  plan->num_partitions = std::max(1, (max_context_len + pt - 1) / pt);
  const int32_t waves = kv < 0 ? kvc::kMaxDefaultWaves : kvc::default_waves(static_cast<kvc_dtype>(kv));
  plan->work_items = (opts && opts->work_items > 0) ? opts->work_items
                                                    : std::max(1, waves / std::max(1, num_kv_heads));
  plan->pool_pieces = (opts && opts->pool_pieces > 0) ? opts->pool_pieces : 0;
  plan->pool_shift = (opts && opts->pool_shift > 0) ? opts->pool_shift : kvc::kDefaultPoolShift;
  plan->tile_groups = 0;
  plan->waves_per_group = 1;
  plan->tiles_per_wave = 1;
  plan->max_q = 1;
  if (opts && opts->window < 0) return false;
  plan->window = opts ? opts->window : 0;
  return plan->chunk_slots() <= (1 << 28);   // chunk ids stay far inside int32
}

// Several query tokens per sequence (MFMA kernel).  A sequence's columns are
// ceil(max_q * G / 16) tiles of 16 (query token, head) pairs.  A wave holds up
// to 4 of them (tiles_per_wave) and reuses every K/V block it loads for all of
// them; up to 4 waves share a work-group (side by side on one chunk of blocks,
// so the chunk is read from HBM once and served to the others from cache),
// the rest go to grid.z.  A wave uses the whole register file of its
// SIMD, so a CU holds 4 / waves_per_group work-groups; with several waves per
// group the default launches two such rounds over the chip, divided among the
// KV heads and tile groups (measured on the verify and prefill workloads: one
// round leaves too few blocks in flight, more rounds gain nothing), with one
// wave per group one round, as decode; capped so the partials stay within
// kExtendRowBudget rows per query head.
constexpr int64_t kExtendRowBudget = 1 << 16;
constexpr int64_t kExtendCUs = 256;   // fixed (not queried), so results do not depend on the device
constexpr int32_t kMaxQueryTokens = 4096;
// From this many new tokens in a sequence on, several-token calls take the
// kernel without a row split by default (enough column tiles to fill the chip).
constexpr int32_t kFlashMinQueryTokens = 64;
// Cutting its rows: about this many waves in all, pieces of at least this many
// steps (two blocks each), at most this many pieces per column tile.  (The
// 2048-token prompt, kernel / step us: no cut 59 / 71, 4096 waves 35-37 /
// 55-57, 8192 37 / 60, 16384 40 / 68: longer pieces leave fewer partials to
// write and merge, shorter ones balance the causal tail.)  With 16-bit codes
// and head_dim 64 the kernel holds three waves per SIMD, so one round is 3072
// waves (same prompt: 2048 waves 54 us, 3072 32, 4096 34, 6144 37).
constexpr int64_t kFlashWaves = 4096;
constexpr int64_t kFlashWaves16D64 = 3072;
int64_t flash_waves_target(int kv, int32_t head_dim) {
  return ((kv == KVC_F16 || kv == KVC_BF16) && head_dim == 64) ? kFlashWaves16D64 : kFlashWaves;
}
constexpr int64_t kFlashMinSteps = 4;
constexpr int64_t kFlashMaxPieces = 64;
constexpr int32_t kFlashWavesPerGroup = 4;   // column tiles (waves) per work-group
// 16-bit caches at head_dim 128: eight, each step's staged K/V shared by twice
// the tiles at the same two waves per SIMD (chunk workload 406-409 us against
// 411-416); at head_dim 64 a group of eight would leave two waves per SIMD
// instead of three (the prompt took 40 us against 32)
int32_t flash_waves_per_group(int kv, int32_t head_dim) {
  return ((kv == KVC_F16 || kv == KVC_BF16) && head_dim == 128) ? 8 : kFlashWavesPerGroup;
}

// kv: the cache's dtype, or -1 for a one-byte cache's plan (the largest cut)
bool plan_extend(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_q,
                 int32_t max_context_len, int kv, const kvc_decode_opts* opts, kvc::DecodePlan* plan) {
  if (opts && (opts->work_items < 0 || (opts->kernel != 0 && opts->kernel != 2 && opts->kernel != 3) ||
               opts->window < 0 || opts->tiles_per_wave < 0 || opts->tiles_per_wave > 4))
    return false;
  if (max_q < 1 || max_q > kMaxQueryTokens) return false;
  plan->window = opts ? opts->window : 0;
  const int32_t G = num_heads / num_kv_heads;
  const int32_t tiles = (max_q * G + 15) / 16;
  plan->partition_tokens = 0;
  plan->num_partitions = 1;
  plan->pool_pieces = 0;
  plan->pool_shift = kvc::kDefaultPoolShift;
  plan->max_q = max_q;
  plan->kernel = (opts && opts->kernel != 0) ? opts->kernel : (max_q >= kFlashMinQueryTokens ? 3 : 2);
  plan->split_steps = 0;
  plan->max_pieces = 1;
  if (plan->kernel == 3) {
    // one wave per 32 (token, head) columns, every row its columns see, four
    // or eight column tiles per work-group sharing the K/V steps; groups of
    // tiles on grid.z (work_items and tiles_per_wave do not apply)
    const int32_t wpg = flash_waves_per_group(kv, head_dim);
    plan->tiles_per_wave = 1;
    plan->waves_per_group = wpg;
    plan->tile_groups = ((max_q * G + 31) / 32 + wpg - 1) / wpg;
    plan->work_items = 1;
    // Too few tiles to fill the chip (a single prompt): each group's steps of
    // two blocks are cut into pieces, so the groups holding the causal
    // diagonal's far end do not run alone; about flash_waves_target() waves in all.
    const int64_t waves = (int64_t)batch * num_kv_heads * plan->tile_groups * wpg;
    const int64_t max_steps = ((int64_t)(max_context_len + 15) / 16 + 1) / 2 + 1;
    const int64_t target = flash_waves_target(kv, head_dim);
    if (waves < target / 2 && max_steps > kFlashMinSteps) {
      int64_t S = std::max<int64_t>(kFlashMinSteps, (max_steps * waves + target - 1) / target);
      int64_t pieces = (max_steps + S - 1) / S;
      const int64_t cap = std::min<int64_t>(kFlashMaxPieces, 65535 / plan->tile_groups);
      if (pieces > cap) {
        S = (max_steps + cap - 1) / cap;
        pieces = (max_steps + S - 1) / S;
      }
      if (pieces > 1) {
        plan->split_steps = (int32_t)S;
        plan->max_pieces = (int32_t)pieces;
      }
    }
    return true;
  }
  // A wave walks the union of its tiles' block ranges.  When the new tokens
  // are most of what is attended (a prompt with little or no cached history),
  // those ranges differ tile to tile along the causal diagonal, so one tile
  // per wave is cheaper (measured on a 2048-token prompt: 56 us against 66 us
  // for four); with a long history they nearly coincide and four tiles share
  // every block load.
  const bool mostly_new = max_context_len > 0 && (int64_t)max_context_len <= 2 * (int64_t)max_q;
  plan->tiles_per_wave = (opts && opts->tiles_per_wave > 0) ? opts->tiles_per_wave
                                                            : (mostly_new && tiles > 4 ? 1 : std::min(4, tiles));
  plan->tiles_per_wave = std::min(plan->tiles_per_wave, tiles);
  const int32_t wave_slots = (tiles + plan->tiles_per_wave - 1) / plan->tiles_per_wave;
  plan->waves_per_group = std::min(4, wave_slots);
  plan->tile_groups = (wave_slots + plan->waves_per_group - 1) / plan->waves_per_group;
  (void)kv;
  const int64_t groups_per_round = (int64_t)kExtendCUs * std::max(1, 4 / plan->waves_per_group);
  const int64_t rounds = plan->waves_per_group == 1 ? 1 : 2;   // one tile: shaped like decode, one round
  int64_t w = rounds * groups_per_round / ((int64_t)num_kv_heads * plan->tile_groups);
  w = std::min<int64_t>(w, kExtendRowBudget / max_q - batch);
  if (opts && opts->work_items > 0) w = opts->work_items;
  plan->work_items = (int32_t)std::max<int64_t>(1, w);
  return plan->chunk_slots() <= (1 << 28);
}

// Shared-prefix (cascade) decode on top of a kernel-2 decode plan: the
// prefix's blocks are skipped by every sequence's decode list and attended
// once by a prefix pass, the several-token kernel without the causal mask
// over one virtual sequence (sequence 0's first prefix_tokens rows, the
// batch's queries as its columns, four 32-column tiles per work-group), cut
// into pieces like a prompt when its groups are too few to fill the chip.
bool plan_shared_prefix(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t prefix_tokens,
                        const kvc_decode_opts* opts, kvc::DecodePlan* plan) {
  if (plan->kernel != 2 || prefix_tokens <= 0 || prefix_tokens % kDeviceBlockSize != 0) return false;
  if (opts && (opts->window != 0 || opts->pool_pieces > 0)) return false;
  const int32_t G = num_heads / num_kv_heads;
  const int64_t tiles = ((int64_t)batch * G + 31) / 32;
  const int64_t groups = (tiles + kFlashWavesPerGroup - 1) / kFlashWavesPerGroup;
  if (groups > 65535) return false;
  const int64_t steps = ((int64_t)prefix_tokens / kDeviceBlockSize + 1) / 2;   // as the kernel counts them
  const int64_t waves = (int64_t)num_kv_heads * groups * kFlashWavesPerGroup;
  int64_t S = 0, pieces = 1;
  if (waves < kFlashWaves / 2 && steps > kFlashMinSteps) {
    S = std::max<int64_t>(kFlashMinSteps, (steps * waves + kFlashWaves - 1) / kFlashWaves);
    pieces = (steps + S - 1) / S;
    const int64_t cap = std::min<int64_t>(kFlashMaxPieces, 65535 / groups);
    if (pieces > cap) {
      S = (steps + cap - 1) / cap;
      pieces = (steps + S - 1) / S;
    }
    if (pieces <= 1) S = 0, pieces = 1;
  }
  plan->skip_blocks = prefix_tokens / kDeviceBlockSize;
  plan->pre_groups = (int32_t)groups;
  plan->pre_split_steps = (int32_t)S;
  plan->pre_pieces = (int32_t)pieces;
  return true;
}

size_t workspace_bytes_for(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           const kvc::DecodePlan& p) {
  return kvc::workspace_layout(p, batch, num_heads, num_kv_heads, head_dim).bytes;
}

// The shared-prefix decode's preconditions, from the tables the handle owns:
// every listed sequence exists, holds more than prefix_tokens tokens, and its
// first prefix_tokens / block_size table entries are the first sequence's.
// The caller holds the handle's lock.
kvc_status check_prefix_tables(kvc_cache* c, int32_t batch, const int64_t* seq_ids, int32_t prefix_tokens) {
  const int32_t bs = c->cfg.block_size;
  if (batch < 1 || !seq_ids) return fail(KVC_E_INVALID, "shared prefix check: batch >= 1 and seq_ids needed");
  if (prefix_tokens <= 0 || prefix_tokens % bs != 0)
    return fail(KVC_E_INVALID, "shared prefix %d is not a positive multiple of the block size", prefix_tokens);
  const int32_t nb = prefix_tokens / bs;
  const kvc_cache::Seq* first = nullptr;
  for (int32_t i = 0; i < batch; ++i) {
    auto it = c->seqs.find(seq_ids[i]);
    if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    const kvc_cache::Seq& s = it->second;
    if (s.len <= prefix_tokens)
      return fail(KVC_E_INVALID, "sequence %lld holds %d tokens, not more than the shared prefix %d",
                  (long long)seq_ids[i], s.len, prefix_tokens);
    if (!first) {
      first = &s;
      for (int32_t j = 0; j < nb; ++j)
        if (s.blocks[j] < 0)
          return fail(KVC_E_INVALID, "sequence %lld released block %d of the prefix", (long long)seq_ids[i], j);
      continue;
    }
    if (!std::equal(s.blocks.begin(), s.blocks.begin() + nb, first->blocks.begin()))
      return fail(KVC_E_INVALID, "sequence %lld does not share the first %d blocks of sequence %lld",
                  (long long)seq_ids[i], nb, (long long)seq_ids[0]);
  }
  return KVC_OK;
}

}  // namespace

namespace kvc {
kvc_status host_fail(kvc_status st, const char* msg) { return fail(st, "%s", msg); }
int32_t cache_block_size(const kvc_cache* c) { return c->cfg.block_size; }
}  // namespace kvc

extern "C" {

size_t kvc_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim, kvc_dtype dtype) {
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || !valid_dtype(dtype)) return 0;
  return (size_t)2 * num_layers * num_kv_heads * head_dim * kvc::dtype_bytes(dtype);
}

size_t kvc_pool_bytes(int32_t num_layers, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, kvc_dtype dtype) {
  if (num_layers < 0 || num_blocks < 0 || num_kv_heads < 0 || head_dim < 0 || block_size < 0 || !valid_dtype(dtype))
    return 0;
  return (size_t)num_layers * num_blocks * num_kv_heads * block_size * head_dim * kvc::dtype_bytes(dtype);
}

size_t kvc_scale_bytes(int32_t num_layers, int32_t num_blocks, int32_t num_kv_heads) {
  if (num_layers < 0 || num_blocks < 0 || num_kv_heads < 0) return 0;
  return (size_t)num_layers * num_blocks * num_kv_heads * sizeof(float);
}

size_t kvc_scratch_bytes(int32_t max_batch, int64_t max_tokens) {
  if (max_batch < 0 || max_tokens < 0) return 0;
  int64_t s = max_segments(max_batch, max_tokens);
  return align256((size_t)s * sizeof(AppendSegment)) + align256((size_t)s * sizeof(CowPair));
}

kvc_status kvc_create(const kvc_config* cfg, kvc_cache** out) {
  if (!cfg || !out) return fail(KVC_E_INVALID, "cfg and out must be non-NULL");
  *out = nullptr;
  if (cfg->num_layers < 1) return fail(KVC_E_INVALID, "num_layers must be >= 1");
  if (cfg->num_kv_heads < 1) return fail(KVC_E_INVALID, "num_kv_heads must be >= 1");
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return fail(KVC_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (cfg->block_size < 1 || cfg->block_size > 256) return fail(KVC_E_INVALID, "block_size must be in 1..256");
  if (cfg->num_blocks < 1) return fail(KVC_E_INVALID, "num_blocks must be >= 1");
  if (!valid_dtype(cfg->kv_dtype)) return fail(KVC_E_INVALID, "unknown kv_dtype %d", (int)cfg->kv_dtype);
  if ((int64_t)cfg->num_blocks * cfg->block_size > INT32_MAX)
    return fail(KVC_E_INVALID, "num_blocks * block_size must fit int32 slot numbers");
  // the kernels form a block's offset as a 32 x 32-bit product of its id and
  // the bytes of one block of one layer (all KV heads)
  if ((int64_t)cfg->num_kv_heads * cfg->block_size * cfg->head_dim * (int64_t)kvc::dtype_bytes(cfg->kv_dtype) >
      (int64_t)UINT32_MAX)
    return fail(KVC_E_UNSUPPORTED, "one block of one layer (num_kv_heads * block_size * head_dim * dtype bytes) "
                                   "must be below 4 GiB");
  kvc_cache* c = new (std::nothrow) kvc_cache();
  if (!c) return fail(KVC_E_INVALID, "out of host memory");
  c->cfg = *cfg;
  c->cfg.free_order = nullptr;
  c->ref.assign(cfg->num_blocks, 0);
  c->free_list.resize(cfg->num_blocks);
  if (cfg->free_order) {
    std::vector<char> seen(cfg->num_blocks, 0);
    for (int32_t i = 0; i < cfg->num_blocks; ++i) {
      int32_t b = cfg->free_order[i];
      if (b < 0 || b >= cfg->num_blocks || seen[b]) {
        delete c;
        return fail(KVC_E_INVALID, "free_order is not a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      c->free_list[i] = b;
    }
  } else {
    for (int32_t i = 0; i < cfg->num_blocks; ++i) c->free_list[i] = i;
  }
  *out = c;
  return ok();
}

void kvc_destroy(kvc_cache* c) {
  if (!c) return;
  if (c->staging_free) {
    (void)hipEventSynchronize(c->staging_free);
    (void)hipEventDestroy(c->staging_free);
  }
  if (c->staging) (void)hipHostFree(c->staging);
  delete c;
}

kvc_status kvc_set_scratch(kvc_cache* c, void* dev_scratch, size_t dev_scratch_bytes) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  c->cfg.dev_scratch = dev_scratch;
  c->cfg.dev_scratch_bytes = dev_scratch ? dev_scratch_bytes : 0;
  return ok();
}

kvc_status kvc_add_seq(kvc_cache* c, int64_t seq_id, int32_t num_tokens) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  if (num_tokens < 0) return fail(KVC_E_INVALID, "num_tokens must be >= 0");
  if (c->seqs.count(seq_id)) return fail(KVC_E_SEQ_EXISTS, "sequence %lld exists", (long long)seq_id);
  int64_t needed = ((int64_t)num_tokens + c->cfg.block_size - 1) / c->cfg.block_size;
  if (needed > (int64_t)c->free_list.size())
    return fail(KVC_E_NO_BLOCKS, "need %lld blocks, %zu free", (long long)needed, c->free_list.size());
  kvc_cache::Seq s;
  s.blocks.reserve(needed);
  for (int64_t i = 0; i < needed; ++i) s.blocks.push_back(c->pop_block());
  c->seqs.emplace(seq_id, std::move(s));
  return ok();
}

kvc_status kvc_fork(kvc_cache* c, int64_t parent_id, int64_t child_id) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  auto it = c->seqs.find(parent_id);
  if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown parent %lld", (long long)parent_id);
  if (c->seqs.count(child_id)) return fail(KVC_E_SEQ_EXISTS, "sequence %lld exists", (long long)child_id);
  kvc_cache::Seq child = it->second;
  for (int32_t b : child.blocks)
    if (b >= 0) ++c->ref[b];
  c->seqs.emplace(child_id, std::move(child));
  return ok();
}

kvc_status kvc_free_seq(kvc_cache* c, int64_t seq_id) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.blocks)
    if (b >= 0) c->release(b);
  c->seqs.erase(it);
  return ok();
}

kvc_status kvc_truncate(kvc_cache* c, int64_t seq_id, int32_t num_tokens) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_id);
  kvc_cache::Seq& s = it->second;
  if (num_tokens < 0 || num_tokens > s.len)
    return fail(KVC_E_INVALID, "truncate to %d outside 0..%d", num_tokens, s.len);
  const int32_t bs = c->cfg.block_size;
  if (num_tokens % bs != 0 && s.blocks[num_tokens / bs] < 0)
    return fail(KVC_E_INVALID, "truncate to %d would end inside a released block", num_tokens);
  size_t keep = ((int64_t)num_tokens + bs - 1) / bs;
  while (s.blocks.size() > keep) {
    if (s.blocks.back() >= 0) c->release(s.blocks.back());
    s.blocks.pop_back();
  }
  s.len = num_tokens;
  return ok();
}

kvc_status kvc_truncate_many(kvc_cache* c, int32_t n, const int64_t* seq_ids, const int32_t* num_tokens) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  if (n < 0) return fail(KVC_E_INVALID, "n must be >= 0");
  if (n == 0) return ok();
  if (!seq_ids || !num_tokens) return fail(KVC_E_INVALID, "NULL host array");
  std::lock_guard<std::mutex> lock(c->mu);
  const int32_t bs = c->cfg.block_size;
  std::vector<kvc_cache::Seq*> seqs((size_t)n);
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    if (!seen.insert(seq_ids[i]).second)
      return fail(KVC_E_INVALID, "sequence %lld appears twice", (long long)seq_ids[i]);
    auto it = c->seqs.find(seq_ids[i]);
    if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    kvc_cache::Seq& s = it->second;
    const int32_t t = num_tokens[i];
    if (t < 0 || t > s.len)
      return fail(KVC_E_INVALID, "sequence %lld: truncate to %d outside 0..%d", (long long)seq_ids[i], t, s.len);
    if (t % bs != 0 && s.blocks[t / bs] < 0)
      return fail(KVC_E_INVALID, "sequence %lld: truncate to %d would end inside a released block",
                  (long long)seq_ids[i], t);
    seqs[(size_t)i] = &s;
  }
  for (int32_t i = n - 1; i >= 0; --i) {   // last entry first: blocks return in reverse order of taking
    kvc_cache::Seq& s = *seqs[(size_t)i];
    const size_t keep = ((int64_t)num_tokens[i] + bs - 1) / bs;
    while (s.blocks.size() > keep) {
      if (s.blocks.back() >= 0) c->release(s.blocks.back());
      s.blocks.pop_back();
    }
    s.len = num_tokens[i];
  }
  return ok();
}

kvc_status kvc_evict(kvc_cache* c, int64_t seq_id, int32_t keep_from) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_id);
  kvc_cache::Seq& s = it->second;
  if (keep_from < 0 || keep_from > s.len)
    return fail(KVC_E_INVALID, "keep_from %d outside 0..%d", keep_from, s.len);
  const int32_t whole = keep_from / c->cfg.block_size;   // blocks holding only positions < keep_from
  for (int32_t j = 0; j < whole; ++j) {
    if (s.blocks[j] < 0) continue;
    c->release(s.blocks[j]);
    s.blocks[j] = -1;
  }
  return ok();
}

kvc_status kvc_reserve_host(kvc_cache* c, int32_t batch, const int64_t* seq_ids, const int32_t* n_new,
                            int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst, int32_t cow_capacity,
                            int32_t* num_cow) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  AppendPlan plan;
  int64_t cap = (cow_src && cow_dst) ? std::max(cow_capacity, 0) : INT64_MAX;
  kvc_status st = plan_append(c, batch, seq_ids, n_new, slots_out != nullptr, cap, &plan);
  if (st != KVC_OK) return st;
  if (slots_out) std::copy(plan.slots.begin(), plan.slots.end(), slots_out);
  if (cow_src && cow_dst)
    for (size_t i = 0; i < plan.cow.size(); ++i) {
      cow_src[i] = plan.cow[i].src;
      cow_dst[i] = plan.cow[i].dst;
    }
  if (num_cow) *num_cow = (int32_t)plan.cow.size();
  return ok();
}

kvc_status kvc_get_table(const kvc_cache* cc, int64_t seq_id, int32_t* blocks_out, int32_t max_blocks,
                         int32_t* num_blocks, int32_t* length) {
  kvc_cache* c = const_cast<kvc_cache*>(cc);
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  auto it = c->seqs.find(seq_id);
  if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_id);
  const auto& s = it->second;
  if (blocks_out) {
    int32_t n = std::min<int32_t>(max_blocks, (int32_t)s.blocks.size());
    std::copy(s.blocks.begin(), s.blocks.begin() + std::max(n, 0), blocks_out);
  }
  if (num_blocks) *num_blocks = (int32_t)s.blocks.size();
  if (length) *length = s.len;
  return ok();
}

kvc_status kvc_check_shared_prefix(const kvc_cache* cc, int32_t batch, const int64_t* seq_ids,
                                   int32_t prefix_tokens) {
  kvc_cache* c = const_cast<kvc_cache*>(cc);
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  return check_prefix_tables(c, batch, seq_ids, prefix_tokens);
}

kvc_status kvc_stats(const kvc_cache* cc, kvc_stats_t* out) {
  kvc_cache* c = const_cast<kvc_cache*>(cc);
  if (!c || !out) return fail(KVC_E_INVALID, "cache and out must be non-NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  out->total_blocks = c->cfg.num_blocks;
  out->free_blocks = (int64_t)c->free_list.size();
  out->used_blocks = c->used;
  int64_t shared = 0;
  for (int32_t r : c->ref) shared += (r >= 2);
  out->shared_blocks = shared;
  out->peak_used_blocks = c->peak_used;
  out->cow_copies = c->cow_copies;
  out->num_seqs = (int64_t)c->seqs.size();
  return ok();
}

kvc_status kvc_append(kvc_cache* c, int32_t batch, const int64_t* seq_ids, const int32_t* n_new,
                      const void* k_new, const void* v_new, kvc_dtype in_dtype, kvc_stream_t stream) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  kvc_status st = check_device_ready(c);
  if (st != KVC_OK) return st;
  const kvc_dtype kv = c->cfg.kv_dtype;
  // No rows at all: reserve the slots (and copy shared blocks) only; a
  // decode call writes each sequence's newest row (kvc_decode_opts.k_new).
  const bool rows_later = !k_new && !v_new;
  if (!rows_later) {
    if (!valid_dtype(in_dtype)) return fail(KVC_E_INVALID, "unknown in_dtype");
    if (is_quantised(kv) ? is_quantised(in_dtype) : in_dtype != kv)
      return fail(KVC_E_UNSUPPORTED, "append rows of dtype %d into a cache of dtype %d", (int)in_dtype, (int)kv);
  }
  if (batch < 0) return fail(KVC_E_INVALID, "batch must be >= 0");
  int64_t total = 0, seg_bound = 0;
  int32_t active = 0;
  for (int32_t i = 0; i < batch; ++i) {
    int32_t n = n_new ? n_new[i] : 1;
    if (n < 0) return fail(KVC_E_INVALID, "n_new[%d] < 0", i);
    total += n;
    active += (n > 0);
    // n rows starting anywhere inside a 16-token block span at most (n + 30) / 16 blocks
    if (n > 0) seg_bound += ((int64_t)n + 2 * kDeviceBlockSize - 2) / kDeviceBlockSize;
  }
  if (total > 0 && !rows_later && (!k_new || !v_new)) return fail(KVC_E_INVALID, "one of k_new / v_new is NULL");
  if (rows_later)
    for (int32_t i = 0; i < batch; ++i)
      if (n_new && n_new[i] > 1)
        return fail(KVC_E_INVALID, "an append without rows reserves at most one token per sequence");
  if (total > INT32_MAX) return fail(KVC_E_INVALID, "too many rows in one append");
  size_t need = kvc_scratch_bytes(active, total);
  if (!c->cfg.dev_scratch || c->cfg.dev_scratch_bytes < need)
    return fail(KVC_E_WORKSPACE, "dev_scratch has %zu bytes, this append needs %zu", c->cfg.dev_scratch_bytes, need);
  const kvc::PoolDesc pool = c->pool();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // A plan that fits the kernel arguments needs no upload (the usual decode
  // step); larger ones, and any copy-on-write list, go through dev_scratch.
  const int64_t smax = max_segments(active, total);
  const bool may_inline = seg_bound <= kvc::kInlineSegments;
  const size_t seg_bytes = align256((size_t)smax * sizeof(AppendSegment));
  // Get the staging buffer before touching the bookkeeping so that a HIP
  // failure here leaves the allocator unchanged.
  if (!may_inline) {
    st = staging_acquire(c, need);
    if (st != KVC_OK) return st;
  }
  AppendPlan plan;
  st = plan_append(c, batch, seq_ids, n_new, false, INT64_MAX, &plan);
  if (st != KVC_OK) return st;
  if (plan.segs.empty()) return ok();
  // The bookkeeping is committed at this point; device failures below are
  // reported but the blocks stay reserved (the caller frees the sequences).
  char* scratch = static_cast<char*>(c->cfg.dev_scratch);
  const bool inline_plan = may_inline && plan.cow.empty();
  if (!inline_plan) {
    if (may_inline) {
      st = staging_acquire(c, need);
      if (st != KVC_OK) return st;
    }
    char* stg = static_cast<char*>(c->staging);
    std::memcpy(stg, plan.segs.data(), plan.segs.size() * sizeof(AppendSegment));
    if (!plan.cow.empty()) std::memcpy(stg + seg_bytes, plan.cow.data(), plan.cow.size() * sizeof(CowPair));
    size_t upload = plan.cow.empty() ? plan.segs.size() * sizeof(AppendSegment)
                                     : seg_bytes + plan.cow.size() * sizeof(CowPair);
    st = staging_upload(c, c->cfg.dev_scratch, upload, s);
    if (st != KVC_OK) return st;
  }
  if (!plan.cow.empty()) {
    hipError_t e = kvc::launch_copy_blocks(pool, reinterpret_cast<const CowPair*>(scratch + seg_bytes),
                                           (int32_t)plan.cow.size(), s);
    if (e != hipSuccess) return fail(KVC_E_HIP, "copy-on-write launch: %s", hipGetErrorString(e));
  }
  if (rows_later) return ok();
  hipError_t e;
  if (inline_plan) {
    kvc::InlineSegments segs;
    std::memcpy(segs.s, plan.segs.data(), plan.segs.size() * sizeof(AppendSegment));
    e = kvc::launch_append(pool, nullptr, &segs, (int32_t)plan.segs.size(), k_new, v_new, in_dtype, total, s);
  } else {
    e = kvc::launch_append(pool, reinterpret_cast<const AppendSegment*>(scratch), nullptr, (int32_t)plan.segs.size(),
                           k_new, v_new, in_dtype, total, s);
  }
  if (e != hipSuccess) return fail(KVC_E_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

kvc_status kvc_export_tables(kvc_cache* c, int32_t batch, const int64_t* seq_ids, int32_t* block_table,
                             int32_t max_blocks, int32_t* context_lens, kvc_stream_t stream) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  if (batch < 0 || max_blocks < 1) return fail(KVC_E_INVALID, "batch must be >= 0 and max_blocks >= 1");
  if (batch == 0) return ok();
  if (!seq_ids || !block_table || !context_lens) return fail(KVC_E_INVALID, "NULL argument");
  std::vector<const kvc_cache::Seq*> rows(batch);
  for (int32_t i = 0; i < batch; ++i) {
    auto it = c->seqs.find(seq_ids[i]);
    if (it == c->seqs.end()) return fail(KVC_E_NO_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return fail(KVC_E_INVALID, "sequence %lld has %zu blocks > max_blocks %d", (long long)seq_ids[i],
                  it->second.blocks.size(), max_blocks);
    rows[i] = &it->second;
  }
  size_t table_bytes = (size_t)batch * max_blocks * sizeof(int32_t);
  size_t lens_off = align256(table_bytes);
  kvc_status st = staging_acquire(c, lens_off + (size_t)batch * sizeof(int32_t));
  if (st != KVC_OK) return st;
  int32_t* t = static_cast<int32_t*>(c->staging);
  int32_t* l = reinterpret_cast<int32_t*>(static_cast<char*>(c->staging) + lens_off);
  for (int32_t i = 0; i < batch; ++i) {
    const auto& b = rows[i]->blocks;
    std::copy(b.begin(), b.end(), t + (size_t)i * max_blocks);
    std::fill(t + (size_t)i * max_blocks + b.size(), t + (size_t)(i + 1) * max_blocks, -1);
    l[i] = rows[i]->len;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(block_table, t, table_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(context_lens, l, batch * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(c->staging_free, s);
  if (e != hipSuccess) return fail(KVC_E_HIP, "table upload: %s", hipGetErrorString(e));
  return ok();
}

size_t kvc_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, const kvc_decode_opts* opts) {
  if (batch < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || max_context_len < 1) return 0;
  const int32_t kernel = opts ? opts->kernel : 0;
  const int32_t prefix = opts ? opts->shared_prefix : 0;
  if (prefix < 0 || num_heads % num_kv_heads != 0) return 0;
  size_t need = 0;
  for (int32_t k = 1; k <= 2; ++k) {
    if (kernel != 0 && kernel != k) continue;
    if (prefix > 0 && k != 2) continue;   // the shared-prefix decode runs the MFMA kernel
    kvc::DecodePlan p;
    if (!plan_decode(batch, num_kv_heads, max_context_len, k, -1, opts, &p)) return 0;
    if (prefix > 0 && !plan_shared_prefix(batch, num_heads, num_kv_heads, prefix, opts, &p)) return 0;
    need = std::max(need, workspace_bytes_for(batch, num_heads, num_kv_heads, head_dim, p));
  }
  return need;
}

}  // extern "C"

namespace {

// Checks shared by the decode and the multi-token call, in order: cache,
// layer, shape against the cache, head grouping, pointers, dtypes, scale,
// batch.  Returns KVC_OK or the failure (already recorded).
kvc_status check_attention_args(const kvc_cache* c, int32_t layer, const void* q, kvc_dtype q_dtype,
                                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, float scale, const void* out) {
  if (!c) return fail(KVC_E_INVALID, "cache is NULL");
  kvc_status st = check_device_ready(c);
  if (st != KVC_OK) return st;
  const kvc_config& f = c->cfg;
  if (layer < 0 || layer >= f.num_layers) return fail(KVC_E_INVALID, "layer %d outside 0..%d", layer, f.num_layers - 1);
  if (batch < 0) return fail(KVC_E_INVALID, "batch must be >= 0");
  if (num_kv_heads != f.num_kv_heads) return fail(KVC_E_INVALID, "num_kv_heads %d != cache's %d", num_kv_heads, f.num_kv_heads);
  if (head_dim != f.head_dim) return fail(KVC_E_INVALID, "head_dim %d != cache's %d", head_dim, f.head_dim);
  if (block_size != f.block_size) return fail(KVC_E_INVALID, "block_size %d != cache's %d", block_size, f.block_size);
  if (num_heads < 1 || num_heads % num_kv_heads != 0)
    return fail(KVC_E_INVALID, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
  if (num_heads / num_kv_heads > 16) return fail(KVC_E_UNSUPPORTED, "more than 16 query heads per KV head");
  if (batch == 0) return KVC_OK;
  if (!q || !block_table || !context_lens || !out) return fail(KVC_E_INVALID, "NULL device argument");
  if (max_blocks_per_seq < 1) return fail(KVC_E_INVALID, "max_blocks_per_seq must be >= 1");
  if (max_context_len < 1) return fail(KVC_E_INVALID, "max_context_len must be >= 1");
  const kvc_dtype kv = f.kv_dtype;
  bool dt_ok = is_quantised(kv) ? (q_dtype == KVC_BF16) : (q_dtype == kv);
  if (!dt_ok) return fail(KVC_E_UNSUPPORTED, "q dtype %d with a cache of dtype %d", (int)q_dtype, (int)kv);
  // the split kernel takes the block max of the raw scores and scales it, so
  // the scale must not flip the order of the scores
  if (!(scale >= 0.0f) || scale > 3.0e38f) return fail(KVC_E_INVALID, "scale must be finite and >= 0");
  if (batch > kvc::kMaxBatch) return fail(KVC_E_UNSUPPORTED, "batch %d > %d", batch, kvc::kMaxBatch);
  // the kernels cap a length at max_blocks_per_seq x block_size in 32 bits
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(KVC_E_UNSUPPORTED, "max_blocks_per_seq * block_size must fit int32");
  // the kernels read the block table through 32-bit byte offsets: every list
  // position of a head's blocks (at most batch x blocks per sequence) < 2^30
  const int64_t per_seq = std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  if ((int64_t)batch * ((per_seq + 15) / 16) >= ((int64_t)1 << 30))
    return fail(KVC_E_UNSUPPORTED, "batch * blocks per sequence must be below 2^30");
  return KVC_OK;
}

}  // namespace

extern "C" {

kvc_status kvc_decode_attention(kvc_cache* c, int32_t layer, const void* q, kvc_dtype q_dtype,
                                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, float scale, void* out, void* workspace,
                                size_t workspace_bytes, const kvc_decode_opts* opts, kvc_stream_t stream) {
  kvc_status st = check_attention_args(c, layer, q, q_dtype, block_table, max_blocks_per_seq, context_lens,
                                       max_context_len, batch, num_heads, num_kv_heads, head_dim, block_size, scale,
                                       out);
  if (st != KVC_OK) return st;
  if (batch == 0) return ok();
  const kvc_dtype kv = c->cfg.kv_dtype;
  int32_t kernel = opts ? opts->kernel : 0;
  if (kernel == 0) kernel = (kv == KVC_F32) ? 1 : 2;
  if (kernel == 2 && kv == KVC_F32) return fail(KVC_E_UNSUPPORTED, "the MFMA kernel needs a 16-bit or fp8 cache");
  if (kernel != 1 && kernel != 2) return fail(KVC_E_INVALID, "unknown kernel %d", kernel);
  kvc::DecodePlan plan;
  if (!plan_decode(batch, num_kv_heads, std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size),
                   kernel, (int)kv, opts, &plan))
    return fail(KVC_E_INVALID,
                "partition_tokens must be a multiple of 16 and at most 1024, work_items >= 0, "
                "pool_pieces <= 64, pool_shift in 0..6, window >= 0");
  if (opts && opts->shared_prefix != 0) {
    const int32_t P = opts->shared_prefix;
    if (P < 0 || !plan_shared_prefix(batch, num_heads, num_kv_heads, P, opts, &plan) ||
        P / block_size >= max_blocks_per_seq)
      return fail(KVC_E_INVALID,
                  "shared_prefix must be a positive multiple of the block size below the table length, with "
                  "the MFMA kernel, window 0 and no pool");
    if (opts->seq_ids) {
      std::lock_guard<std::mutex> lock(c->mu);
      kvc_status pst = check_prefix_tables(c, batch, opts->seq_ids, P);
      if (pst != KVC_OK) return pst;
    }
  }
  const void* k_new = opts ? opts->k_new : nullptr;
  const void* v_new = opts ? opts->v_new : nullptr;
  if (!k_new != !v_new) return fail(KVC_E_INVALID, "opts: k_new and v_new must both be set or both be NULL");
  size_t need = workspace_bytes_for(batch, num_heads, num_kv_heads, head_dim, plan);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVC_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipError_t e = kvc::launch_decode(c->pool(), layer, plan, q, q_dtype, nullptr, batch, block_table,
                                    max_blocks_per_seq, context_lens, max_context_len, batch, num_heads, scale, out,
                                    workspace, k_new, v_new,
                                    opts ? static_cast<hipEvent_t>(opts->split_start) : nullptr,
                                    opts ? static_cast<hipEvent_t>(opts->split_end) : nullptr,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVC_E_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

kvc_status kvc_decode_attention_static(kvc_cache* c, int32_t layer, const void* q, kvc_dtype q_dtype,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       float scale, void* out, const kvc_decode_opts* opts, kvc_stream_t stream) {
  // The workspace is the library's static array of the current device;
  // kvc_decode_attention makes every check, the size this plan needs against
  // the array's included, before it launches anything.
  void* ws = nullptr;
  hipError_t e = kvc::static_scratch(&ws);
  if (e != hipSuccess) return fail(KVC_E_HIP, "static workspace: %s", hipGetErrorString(e));
  kvc_status st = kvc_decode_attention(c, layer, q, q_dtype, block_table, max_blocks_per_seq, context_lens,
                                       max_context_len, batch, num_heads, num_kv_heads, head_dim, block_size, scale,
                                       out, ws, KVC_STATIC_SCRATCH_BYTES, opts, stream);
  if (st == KVC_E_WORKSPACE) {
    const std::string why = g_last_error;
    return fail(KVC_E_WORKSPACE, "%s: beyond the static workspace (%u bytes); use kvc_decode_attention with a "
                "workspace of its own", why.c_str(), (unsigned)KVC_STATIC_SCRATCH_BYTES);
  }
  return st;
}

size_t kvc_extend_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_query_len, int32_t max_context_len, const kvc_decode_opts* opts) {
  if (batch < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || num_heads % num_kv_heads != 0) return 0;
  // the plan depends on the cache's dtype (work-group size, cut): the larger
  // of the 16-bit plan and the one-byte one
  size_t need = 0;
  for (int kv : {(int)KVC_BF16, -1}) {
    kvc::DecodePlan p;
    if (!plan_extend(batch, num_heads, num_kv_heads, head_dim, max_query_len, max_context_len, kv, opts, &p)) return 0;
    need = std::max(need, workspace_bytes_for(batch, num_heads, num_kv_heads, head_dim, p));
  }
  return need;
}

kvc_status kvc_extend_attention(kvc_cache* c, int32_t layer, const void* q, kvc_dtype q_dtype,
                                const int32_t* query_start, int32_t total_query, int32_t max_query_len,
                                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, float scale, void* out, void* workspace,
                                size_t workspace_bytes, const kvc_decode_opts* opts, kvc_stream_t stream) {
  kvc_status st = check_attention_args(c, layer, q, q_dtype, block_table, max_blocks_per_seq, context_lens,
                                       max_context_len, batch, num_heads, num_kv_heads, head_dim, block_size, scale,
                                       out);
  if (st != KVC_OK) return st;
  if (batch == 0) return ok();
  if (!query_start) return fail(KVC_E_INVALID, "NULL device argument");
  if (total_query < 0) return fail(KVC_E_INVALID, "total_query must be >= 0");
  if (total_query == 0) return ok();
  if (max_query_len < 1 || max_query_len > kMaxQueryTokens)
    return fail(KVC_E_INVALID, "max_query_len must be in 1..%d", kMaxQueryTokens);
  const kvc_dtype kv = c->cfg.kv_dtype;
  if (kv == KVC_F32) return fail(KVC_E_UNSUPPORTED, "several query tokens need a 16-bit or fp8 cache");
  kvc::DecodePlan plan;
  if (!plan_extend(batch, num_heads, num_kv_heads, head_dim, max_query_len,
                   std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size), (int)kv, opts, &plan))
    return fail(KVC_E_INVALID, "opts: kernel must be 0, 2 or 3, work_items >= 0, window >= 0");
  size_t need = workspace_bytes_for(batch, num_heads, num_kv_heads, head_dim, plan);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVC_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipError_t e = kvc::launch_decode(c->pool(), layer, plan, q, q_dtype, query_start, total_query, block_table,
                                    max_blocks_per_seq, context_lens, max_context_len, batch, num_heads, scale, out,
                                    workspace, nullptr, nullptr,
                                    opts ? static_cast<hipEvent_t>(opts->split_start) : nullptr,
                                    opts ? static_cast<hipEvent_t>(opts->split_end) : nullptr,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVC_E_HIP, "extend launch: %s", hipGetErrorString(e));
  return ok();
}

kvc_status kvc_stream_copy(void* dst, const void* src, size_t bytes, kvc_stream_t stream) {
  if (!dst || !src) return fail(KVC_E_INVALID, "NULL pointer");
  if (bytes % 16 != 0) return fail(KVC_E_INVALID, "bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  hipError_t e = kvc::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVC_E_HIP, "copy launch: %s", hipGetErrorString(e));
  return ok();
}

kvc_status kvc_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, kvc_stream_t stream) {
  if (!src || !sink) return fail(KVC_E_INVALID, "NULL pointer");
  if (bytes % 16 != 0) return fail(KVC_E_INVALID, "bytes must be a multiple of 16");
  if (sink_words < 1) return fail(KVC_E_INVALID, "sink_words must be >= 1");
  if (bytes == 0) return ok();
  hipError_t e = kvc::launch_stream_read(src, bytes, sink, sink_words, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVC_E_HIP, "read launch: %s", hipGetErrorString(e));
  return ok();
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
