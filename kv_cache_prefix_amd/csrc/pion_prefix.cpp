// C ABI of the prefix-attention library: argument validation, the resident slot table
// and the launch plan. Declarations and the contract of every entry point are in
// include/pion_prefix.h; this file only implements them.
//
// Slot table: one entry per (sid, layer) as the ATTEND.PREFIX.STORE wire form keys it
// ("Shared KV Cache Serving", Stage 2 wire forms). Each entry owns one device
// allocation holding the resident K/V in the store layout [H, N, D] (fp16), or the
// mlx4g32 arrays (codes [H, N, D/8] and (scale, bias) pairs [H, N, D/32], per side),
// plus the per-B block-mean cache of the sparse-auto query.
//
// Capacity and cold tier ("Shared KV Cache Serving", Cold-tier state machine): the
// table holds at most a number of slots and, optionally, a budget of resident K/V
// bytes. A store that would exceed either first demotes the least recently used
// slots (last access = a logical clock advanced by every store and successful query):
// their device memory is released and their shape kept in a bounded cold registry.
// A query of a cold key answers PION_ERR_COLDMISS, a lookup answers 2 (+COLD); a store
// of a cold key makes it warm again (a rehydrate) and the most recent.
//
// Launch plan of an attention call: one split-KV kernel (fp16 or mlx4g32 prefix; an
// mlx4g32 prefix with an fp16 suffix takes one launch of each) over workgroups (key
// span, q-head group sharing one kv-head, query index); each writes (acc, m, l) per (row,
// span) into a per-stream workspace, and the last workgroup of each row group merges
// them into out and lse. The sparse-auto call runs block_mean (first use per slot and B)
// and block_select first, and the split-KV kernel reads the picked block
// list on the device.
#include "pion_prefix.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "attn_gqa.h"
#include "kernels.h"
#include "mlx4g32.h"
#include "sparse.h"

namespace {

using namespace pion;

constexpr int kMaxSplitsTotal = 8192;  // spans per row: the in-kernel merge limit
constexpr int kDenseSpans = 512;        // a dense key range is cut into at most this many
constexpr int kMaxKTop = 1024;

struct KMean {
  float *ptr = nullptr;
  int nb = 0;
  hipEvent_t ready = nullptr;
  hipStream_t stream = nullptr;
  bool done = false;
};

struct Slot {
  int H = 0, N = 0, D = 0, fmt = 0;
  void *mem = nullptr;
  size_t bytes = 0;
  uint64_t last = 0;  // logical clock of the last store or successful query
  KVView view{};
  hipEvent_t ready = nullptr;
  hipStream_t stream = nullptr;
  bool done = false;
  std::map<int, KMean> kmeans;
};

struct Workspace {
  void *ptr = nullptr;
  size_t cap = 0;
  int *counters = nullptr;  // ticket counters of the split merge, kMaxCounters ints
};


// A demoted slot: its shape and last access (the K/V bytes are gone).
struct ColdEntry {
  int H = 0, N = 0, D = 0, fmt = 0;
  uint64_t last = 0;
};

std::mutex g_mu;
std::unordered_map<std::string, Slot> g_slots;
std::unordered_map<std::string, ColdEntry> g_cold;
std::unordered_map<hipStream_t, Workspace> g_ws;      // split partials
std::unordered_map<hipStream_t, Workspace> g_sel_ws;  // sparse-auto scores and picks

std::string key_of(const char *sid, int layer) {
  std::string k(sid);
  k.push_back('\0');
  k.append(std::to_string(layer));
  return k;
}

bool sid_ok(const char *sid) {
  if (!sid) return false;
  const size_t n = strnlen(sid, 256);
  return n >= 1 && n <= 255;
}

bool d_supported(int D) { return head_dim_supported(D); }
// Head dims of the MFMA kernels; a query at another head dim runs on the split kernels.
// Batched-Q prefill: every served D but 512 (its accumulators exceed the registers).
// Grouped-query decode: the power-of-two dims its LDS layout is written for.
bool prefill_dim(int D) { return D != 512; }
bool gqa_dim(int D) { return D == 64 || D == 128 || D == 256; }

// Capacity (env PION_MAX_SLOTS, PION_MAX_BYTES, PION_COLD_SLOTS at load; then
// pion_prefix_set_capacity) and the cold-tier counters; all under g_mu.
long long env_ll(const char *name, long long dflt, long long lo) {
  const char *e = getenv(name);
  const long long x = e ? atoll(e) : dflt;
  return x >= lo ? x : dflt;
}
struct Tier {
  long long max_slots = env_ll("PION_MAX_SLOTS", 4096, 1);
  long long max_bytes = env_ll("PION_MAX_BYTES", 0, 0);  // 0: no byte budget
  long long cold_slots = env_ll("PION_COLD_SLOTS", 1024, 0);
  uint64_t clock = 0;
  long long demotions = 0, rehydrates = 0;
  size_t resident = 0;  // K/V bytes of the warm slots
} g_tier;

// Workgroups a launch aims for when it splits keys. fp16 prefix: two per CU of the
// MI355X (512): the kernel holds few bytes in flight per wave, and cold-HBM bandwidth
// needs more waves per CU (measured on the 32-layer decode launch). mlx4g32 prefix: one
// per CU (256): its workgroups are larger and its merge dearer per span. Env
// PION_SPLIT_TARGET overrides both for tuning.
int split_target(bool mlx4) {
  static int v = [] {
    const char *e = getenv("PION_SPLIT_TARGET");
    int x = e ? atoi(e) : 0;
    return x > 0 ? x : 0;
  }();
  return v ? v : (mlx4 ? 256 : 512);
}

// A row group whose keys fit in this many tile passes of the fp16 kernel (4 waves, each
// 4 x 64 / LPR keys per pass, LPR lanes per key row) runs as one span: the serial passes
// cost less than the store, ticket and merge of a split.
int one_span_keys(int D) {
  static int iters = [] {
    const char *e = getenv("PION_ONE_SPAN_ITERS");
    return e ? std::max(0, atoi(e)) : 3;
  }();
  return iters * 4 * (256 / fp16_row_lanes(D));
}

bool getenv_flag(const char *name) {
  const char *e = getenv(name);
  return e && e[0] && e[0] != '0';
}

// Memory that a kernel may read or write: device (or managed) allocations only.
bool on_device(const void *p) {
  if (!p) return false;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged ||
         a.type == hipMemoryTypeUnified;
}

// fp16 tensors are read with 16-byte vector loads; fp32 / int32 with 4-byte accesses.
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

void free_slot(Slot &s) {
  for (auto &kv : s.kmeans) {
    if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    if (kv.second.ready) (void)hipEventDestroy(kv.second.ready);
  }
  s.kmeans.clear();
  if (s.mem) (void)hipFree(s.mem);  // hipFree waits for queued device work
  if (s.ready) (void)hipEventDestroy(s.ready);
  s.mem = nullptr;
  s.ready = nullptr;
}

void trim_cold() {
  while ((long long)g_cold.size() > g_tier.cold_slots) {
    auto old = g_cold.begin();
    for (auto it = g_cold.begin(); it != g_cold.end(); ++it)
      if (it->second.last < old->second.last) old = it;
    g_cold.erase(old);
  }
}

// Demote the least recently used warm slot other than `keep`: free its memory, keep its
// shape in the cold registry. False when there is none.
bool demote_lru(const std::string &keep) {
  auto lru = g_slots.end();
  for (auto it = g_slots.begin(); it != g_slots.end(); ++it)
    if (it->first != keep && (lru == g_slots.end() || it->second.last < lru->second.last)) lru = it;
  if (lru == g_slots.end()) return false;
  Slot &s = lru->second;
  ColdEntry c;
  c.H = s.H;
  c.N = s.N;
  c.D = s.D;
  c.fmt = s.fmt;
  c.last = s.last;
  g_tier.resident -= s.bytes;
  free_slot(s);
  g_cold[lru->first] = c;
  g_slots.erase(lru);
  ++g_tier.demotions;
  trim_cold();
  return true;
}

// Status of a query whose key has no warm slot.
int absent_status(const char *sid, int layer) {
  return g_cold.count(key_of(sid, layer)) ? PION_ERR_COLDMISS : PION_ERR_NOT_FOUND;
}

void touch(Slot *s) { s->last = ++g_tier.clock; }

// Make `st` wait for work recorded on another stream (store or block-mean build).
hipError_t order_after(hipEvent_t ev, hipStream_t src, bool &done, hipStream_t st) {
  if (done || !ev) return hipSuccess;
  hipError_t q = hipEventQuery(ev);
  if (q == hipSuccess) {
    done = true;
    return hipSuccess;
  }
  if (q != hipErrorNotReady) return q;
  if (src == st) return hipSuccess;
  return hipStreamWaitEvent(st, ev, 0);
}

// Set by pion_prefix_query_noalloc for the duration of its call (under g_mu): the launch
// plan's workspace then comes from the fixed scratch area, never from hipMalloc.
struct FixedScratch {
  char *base = nullptr;     // split partials
  size_t bytes = 0;
  int *counters = nullptr;  // kMaxCounters zeroed ticket counters
  bool too_small = false;   // a request exceeded `bytes`
};
FixedScratch *g_fixed = nullptr;

// Per-stream scratch for the split partials, plus the zeroed ticket counters (the
// merging workgroup resets its counter, so they stay zero between calls). Grows by
// reallocating after the stream has drained; never shrinks.
hipError_t get_counters(hipStream_t st, int **out) {
  if (g_fixed) {
    *out = g_fixed->counters;
    return hipSuccess;
  }
  Workspace &w = g_ws[st];
  if (!w.counters) {
    hipError_t e = hipMalloc(&w.counters, kMaxCounters * sizeof(int));
    if (e == hipSuccess) e = launch_zero_counters(w.counters, kMaxCounters, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      if (w.counters) (void)hipFree(w.counters);
      w.counters = nullptr;
      return e;
    }
  }
  *out = w.counters;
  return hipSuccess;
}

hipError_t get_ws(hipStream_t st, size_t bytes, void **out) {
  if (g_fixed) {
    if (bytes > g_fixed->bytes) {
      g_fixed->too_small = true;
      return hipErrorOutOfMemory;
    }
    *out = g_fixed->base;
    return hipSuccess;
  }
  Workspace &w = g_ws[st];
  int *cnt;
  if (hipError_t e = get_counters(st, &cnt); e != hipSuccess) return e;
  if (w.cap < bytes) {
    if (w.ptr) {
      hipError_t e = hipStreamSynchronize(st);
      if (e != hipSuccess) return e;
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.cap = 0;
    }
    size_t cap = std::max(bytes, (size_t)1 << 20);
    cap = align256(cap + cap / 4);
    hipError_t e = hipMalloc(&w.ptr, cap);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      w.ptr = nullptr;
      return e;
    }
    w.cap = cap;
  }
  *out = w.ptr;
  return hipSuccess;
}

// head_map (host, may be null) -> vector; returns false when out of range or when the
// default map is undefined.
bool resolve_map(const int32_t *head_map, int H_q, int H_kv, std::vector<int> &hm) {
  hm.resize(H_q);
  if (!head_map) {
    if (H_kv < 1 || H_q % H_kv) return false;
    const int r = H_q / H_kv;
    for (int h = 0; h < H_q; ++h) hm[h] = h / r;
    return true;
  }
  for (int h = 0; h < H_q; ++h) {
    if (head_map[h] < 0 || head_map[h] >= H_kv) return false;
    hm[h] = head_map[h];
  }
  return true;
}

// Group the q-heads of each kv-head into chunks of at most `cap` (<= kRowsPerGroup)
// rows; returns the largest group size.
int build_groups(const std::vector<int> &hm, int H_kv, int cap, RowGroups &rg) {
  memset(&rg, 0, sizeof(rg));
  int maxcnt = 0;
  for (int g = 0; g < H_kv; ++g) {
    int cur = -1, cnt = 0;
    for (int h = 0; h < (int)hm.size(); ++h) {
      if (hm[h] != g) continue;
      if (cur < 0 || cnt == cap) {
        cur = rg.n++;
        cnt = 0;
      }
      rg.heads[cur] |= (uint64_t)h << (8 * cnt);  // row cnt of the group
      ++cnt;
      rg.gc[cur] = (uint32_t)g | (uint32_t)cnt << 8;
      maxcnt = std::max(maxcnt, cnt);
    }
  }
  return maxcnt;
}

// The per-problem segment and span counts the kernels read (p.spans), once
// seg_per_span and the prefix chunking are set: a problem's prefix segments are its
// selected blocks, or its token-list positions or keys in chunks of pre_chunk.
void fill_spans(PartialParams &p) {
  for (int z = 0; z < p.n_prob; ++z) {
    const int keys = p.gidx ? p.gmax : p.N[z];
    const int pre = p.blocks ? p.n_sel : (keys + p.pre_chunk - 1) / p.pre_chunk;
    const int total = (pre + p.suf_splits + p.seg_per_span - 1) / p.seg_per_span;
    p.spans[z] = (uint32_t)pre | (uint32_t)total << 16;
  }
}

int pow2_at_least(int n) {
  int R = 1;
  while (R < n) R <<= 1;
  return R;
}

// Whether a decode over row groups of `grp_rows` q-heads (4 to 8) runs faster on the MFMA
// kernel than on the vector split kernel, from timings of single-layer and 32-layer
// launches at N = 2048 to 8192 and D = 64, 128 and 256. Groups of 5 or more rows, which
// the vector kernel pads to 8: at D = 64 always, else for 64 or more row groups (+25-45%)
// or prefixes of at most 2048 keys. Groups of 4 rows: at D = 64 unless long prefixes
// fill the chip (N > 4096 over 64 or more row groups), at D = 128 for prefixes of at
// most 2048 keys, never at D = 256. The 8-wave split kernel is ahead elsewhere, by up
// to 30% (4 rows at D = 256, N = 4096).
bool prefer_gqa(int grp_rows, int D, int N_max, long long units) {
  if (grp_rows >= 5) return D == 64 || units >= 64 || N_max <= 2048;
  if (grp_rows == 4) return D == 64 ? !(units >= 64 && N_max > 4096) : D == 128 && N_max <= 2048;
  return false;
}

int pick_chunk(long long keys, long long work_rows, int granule, bool mlx4, int waves = 4) {
  if (keys <= 0) return granule;
  const long long target = split_target(mlx4) * 4 / waves;  // the same waves in total
  long long c = (keys * work_rows + target - 1) / target;
  c = std::max<long long>(c, granule);
  c = (c + granule - 1) / granule * granule;
  // keep the span count of a dense range at most kDenseSpans
  while ((keys + c - 1) / c > kDenseSpans) c *= 2;
  return (int)std::min<long long>(c, 1LL << 30);
}

struct AttnCall {
  const void *Q;          // fp16, or fp32 for an fp32 slot
  size_t q_stride;        // elements between problems
  int H_q, M, D;
  const std::vector<int> *hm;
  int H_kv;
  const void *Ksuf, *Vsuf;  // the slot's precision (fp16 for an mlx4g32 slot)
  int S_suf;
  const int32_t *blocks;  // device [H_kv, K_top] or null
  int n_sel, K_top, B;
  const int32_t *gidx, *gcount;  // device [H, gmax], [H] or null
  int gmax;
  float *out, *lse;
  size_t out_stride, lse_stride;
};

// Query rows at or above which an fp16 query runs on the MFMA kernel.
constexpr int kMfmaMinRows = 32;

// Batched-Q on the MFMA kernel: one fp16 slot, no block list. Splits the key range so
// that row blocks x splits gives about two workgroups per CU.
int run_prefill(const Slot &sl, const AttnCall &c, hipStream_t st) {
  PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.Q = (const uint16_t *)c.Q;
  p.K = (const uint16_t *)sl.view.K;
  p.V = (const uint16_t *)sl.view.V;
  p.Ksuf = c.S_suf > 0 ? (const uint16_t *)c.Ksuf : nullptr;
  p.Vsuf = c.S_suf > 0 ? (const uint16_t *)c.Vsuf : nullptr;
  p.H_q = c.H_q;
  p.M = c.M;
  p.D = c.D;
  p.H_kv = sl.H;
  p.N = sl.N;
  p.S_suf = c.S_suf;
  p.qscale = (float)(1.4426950408889634 / std::sqrt((double)c.D));
  p.n_iblk = (c.M + 127) / 128;
  const long long tiles = (long long)c.H_q * p.n_iblk;
  if (tiles * (c.D / 32) > 0x7fffffffLL) return PION_ERR_UNSUPPORTED;  // merge grid
  const long long total = (long long)sl.N + c.S_suf;
  // splits: as many as keep every workgroup resident at once (two fit on a CU for
  // D <= 128, one above: 512 or 256 on 256 CUs), at most 16; a second kernel merges
  // them. env PION_PREFILL_SPLITS overrides
  const long long slots = c.D <= 128 ? 512 : 256;
  long long ns = std::max<long long>(1, slots / tiles);
  if (const char *e = getenv("PION_PREFILL_SPLITS")) ns = std::max(1, atoi(e));
  ns = std::min<long long>(ns, std::min<long long>(16, (total + 31) / 32));
  long long sk = (total + ns - 1) / ns;
  sk = (sk + 31) / 32 * 32;
  if (sk > (1LL << 30)) return PION_ERR_UNSUPPORTED;
  p.split_keys = (int)sk;
  p.n_splits = (int)((total + sk - 1) / sk);
  p.out = c.out;
  p.lse = c.lse;
  p.hm.H_q = c.H_q;
  for (int h = 0; h < c.H_q; ++h) p.hm.m[h] = (uint8_t)(*c.hm)[h];
  {
    int n = 0;
    for (int g = 0; g < c.H_kv; ++g)
      for (int h = 0; h < c.H_q; ++h)
        if ((*c.hm)[h] == g) p.order[n++] = (uint8_t)h;
  }
  if (p.n_splits > 1) {
    const size_t rows = (size_t)c.H_q * c.M;
    // fp16 partials per (tile, split): 128 rows x D in the kernel's register layout;
    // one fp32 log-sum-exp per (row, split)
    const size_t acc_bytes = align256((size_t)tiles * 128 * p.n_splits * c.D * sizeof(uint16_t));
    const size_t lse_bytes = align256(rows * p.n_splits * sizeof(float));
    void *ws = nullptr;
    if (get_ws(st, acc_bytes + lse_bytes, &ws) != hipSuccess) return PION_ERR_NOMEM;
    p.part_acc = (uint16_t *)ws;
    p.part_lse = (float *)((char *)ws + acc_bytes);
  }
  return launch_prefill(p, st) == hipSuccess ? PION_OK : PION_ERR_HIP;
}

// One launch (two for an mlx4g32 prefix with an fp16 suffix) over `slots`, which share
// H, D and format.
int run_attention(const std::vector<const Slot *> &slots, const AttnCall &c, hipStream_t st) {
  // (the MFMA kernel addresses a kv-head's K, V and suffix through 32-bit buffer ranges)
  const long long row_bytes = 2LL * c.D;
  if (slots.size() == 1 && slots[0]->fmt == PION_KV_FP16 && !c.blocks && c.M >= kMfmaMinRows &&
      prefill_dim(c.D) &&
      slots[0]->N * row_bytes < (1LL << 31) && c.S_suf * row_bytes < (1LL << 31) &&
      !getenv_flag("PION_NO_MFMA"))
    return run_prefill(*slots[0], c, st);
  static PartialParams p;  // large; the library lock serializes callers
  memset(&p, 0, sizeof(p));
  const int n_prob = (int)slots.size();
  const Slot &s0 = *slots[0];
  const bool mlx4 = s0.fmt == PION_KV_MLX4G32;
  // the mlx4g32 kernel holds up to kMlx4Rows rows; both launches of a call share groups
  const int grp_rows = build_groups(*c.hm, c.H_kv, mlx4 ? kMlx4Rows : kRowsPerGroup, p.rg);
  const int R = pow2_at_least(grp_rows);
  const int Y = p.rg.n * c.M;
  if (Y > 65535 || (long long)Y * n_prob > kMaxCounters) return PION_ERR_UNSUPPORTED;
  p.H_q = c.H_q;
  p.M = c.M;
  p.D = c.D;
  p.H_kv = s0.H;
  p.fmt = s0.fmt;
  p.esz = s0.fmt == PION_KV_FP32 ? 4 : 2;
  p.qscale = (float)(1.4426950408889634 / std::sqrt((double)c.D));
  p.n_prob = n_prob;
  int N_max = 0;
  for (int z = 0; z < n_prob; ++z) {
    p.kv_base[z] = slots[z]->mem;
    p.N[z] = slots[z]->N;
    N_max = std::max(N_max, slots[z]->N);
  }
  // 8-wave workgroups (fp16 prefix, groups of at most 4 rows, dense keys): the same
  // waves in half as many workgroups. Taken when that leaves every row group one span,
  // so no split merge runs at all, and there are at least 256 of them to fill the chip
  // (measured +5% on the 32-layer decode launch; single layers keep 4-wave splits).
  // PION_SPLIT_WAVES=4 or 8 forces the choice where 8 is allowed.
  static const int waves_env = [] {
    const char *e = getenv("PION_SPLIT_WAVES");
    return e ? atoi(e) : 0;
  }();
  {
    const bool can8 = s0.fmt == PION_KV_FP16 && !c.gidx && !c.blocks && R <= 4;
    const long long units = (long long)Y * n_prob;
    bool use8 = can8 && units >= 256 &&
                pick_chunk(N_max, units, 64, false, 8) >= N_max;  // one span per row group
    if (waves_env == 4 || waves_env == 8) use8 = can8 && waves_env == 8;
    p.waves = use8 ? 8 : 4;
  }
  p.Q = c.Q;
  p.q_stride = c.q_stride;
  p.out = c.out;
  p.out_stride = c.out_stride;
  p.lse = c.lse;
  p.lse_stride = c.lse_stride;
  int pre_max;
  if (c.gidx) {  // a caller's token list per head: chunks of list positions
    p.gidx = c.gidx;
    p.gcount = c.gcount;
    p.gmax = c.gmax;
    p.pre_chunk = std::min(pick_chunk(c.gmax, (long long)Y, 64, false), kGatherChunk);
    pre_max = (c.gmax + p.pre_chunk - 1) / p.pre_chunk;
  } else if (c.blocks) {
    p.blocks = c.blocks;
    p.K_top = c.K_top;
    p.B = c.B;
    p.n_sel = c.n_sel;
    p.pre_chunk = c.B;
    pre_max = c.n_sel;
  } else {
    // at least 128 keys per span: below that the store, ticket and merge of a split cost
    // more than the keys save (measured on single M = 1 calls at N = 2048)
    p.pre_chunk = pick_chunk(N_max, (long long)Y * n_prob, 128, mlx4, p.waves);
    pre_max = (N_max + p.pre_chunk - 1) / p.pre_chunk;
  }
  if (c.S_suf > 0) {
    p.Ksuf = c.Ksuf;
    p.Vsuf = c.Vsuf;
    p.S_suf = c.S_suf;
    p.suf_chunk = pick_chunk(c.S_suf, Y, 64, false);
    p.suf_splits = (c.S_suf + p.suf_chunk - 1) / p.suf_chunk;
  }
  p.S_max = pre_max + p.suf_splits;
  if (p.S_max > kMaxSplitsTotal) return PION_ERR_UNSUPPORTED;
  // the kernels address one query index's partials (H_q x S_max x D fp32) with 32-bit
  // byte offsets
  if ((long long)c.H_q * p.S_max * c.D * 4 > 0x7fffffffLL) return PION_ERR_UNSUPPORTED;
  p.y_groups = Y;

  const size_t rows = (size_t)c.H_q * c.M;
  p.part_stride = rows * p.S_max * c.D;
  p.ml_stride = rows * p.S_max;
  const size_t acc_bytes = align256(n_prob * p.part_stride * sizeof(float));
  const size_t ml_bytes = align256(n_prob * p.ml_stride * sizeof(float));
  void *ws = nullptr;
  if (get_ws(st, acc_bytes + 2 * ml_bytes, &ws) != hipSuccess) return PION_ERR_NOMEM;
  p.part_acc = (float *)ws;
  p.part_m = (float *)((char *)ws + acc_bytes);
  p.part_l = (float *)((char *)ws + acc_bytes + ml_bytes);
  if (get_counters(st, &p.counters) != hipSuccess) return PION_ERR_NOMEM;

  hipError_t e;
  if (mlx4) {
    p.x_begin = 0;
    p.seg_per_span = 1;
    fill_spans(p);
    // head dim 128: the MFMA kernel (PION_NO_MLX4_MFMA keeps the vector kernel)
    const bool mm = c.D == 128 && !getenv_flag("PION_NO_MLX4_MFMA");
    e = mm ? launch_mlx4_mfma(p, grp_rows, pre_max, st) : launch_partial_mlx4(p, grp_rows, pre_max, st);
    if (e == hipSuccess && p.suf_splits > 0) {
      p.x_begin = pre_max;  // single problem: its prefix spans are exactly pre_max
      e = launch_partial(p, R, p.suf_splits, st);
    }
  } else {
    p.x_begin = 0;
    const long long keys =
        (c.gidx ? (long long)c.gmax : c.blocks ? (long long)c.n_sel * c.B : N_max) + c.S_suf;
    // Row groups of 4 to 8 q-heads at M = 1 may run on the MFMA kernel, whose key work
    // does not grow with the rows; the vector kernel pads a group of 5 to 8 rows to 8.
    // PION_GQA_MFMA forces it for any group of 4 or more rows, PION_NO_GQA_MFMA turns
    // it off. It addresses a kv-head's K, V and suffix through 32-bit buffer ranges.
    const long long row_bytes = 2LL * c.D;
    const bool gqa_ok = c.M == 1 && grp_rows >= 4 && !c.gidx && gqa_dim(c.D) &&
                        s0.fmt == PION_KV_FP16 &&
                        N_max * row_bytes < (1LL << 31) &&
                        (long long)c.S_suf * row_bytes < (1LL << 31) &&
                        !getenv_flag("PION_NO_GQA_MFMA");
    const bool gqa = gqa_ok && (getenv_flag("PION_GQA_MFMA") ||
                                prefer_gqa(grp_rows, c.D, N_max, (long long)Y * n_prob));
    if (gqa) {
      // one span when each wave gets at most PION_GQA_ONE_SPAN (default 2) sub-tiles of
      // 32 keys: a wave keeps one sub-tile in flight ahead, which does not cover the load
      // latency, so more keys are better spread over workgroups and merged
      static const int one_span_sub = [] {
        const char *e = getenv("PION_GQA_ONE_SPAN");
        return e ? std::max(0, atoi(e)) : 2;
      }();
      const long long one_span = (long long)(c.D == 256 ? 2 : 4) * 32 * one_span_sub;
      p.seg_per_span = keys <= one_span && p.S_max <= kGqaMaxSegs ? p.S_max : 1;
      fill_spans(p);
      e = launch_gqa_mfma(p, (p.S_max + p.seg_per_span - 1) / p.seg_per_span, st);
    } else {
      p.seg_per_span = keys <= one_span_keys(c.D) && !c.gidx ? p.S_max : 1;
      fill_spans(p);
      e = launch_partial(p, R, (p.S_max + p.seg_per_span - 1) / p.seg_per_span, st);
    }
  }
  return e == hipSuccess ? PION_OK : PION_ERR_HIP;
}

// Shape checks shared by STORE and WARM.
int check_slot_shape(const char *sid, int H, int N, int D, int kv_format) {
  if (!sid_ok(sid) || H < 1 || H > 255 || N < 1 || D <= 0) return PION_ERR_INVALID;
  if (kv_format != PION_KV_FP16 && kv_format != PION_KV_MLX4G32 && kv_format != PION_KV_FP32)
    return PION_ERR_INVALID;
  if (kv_format == PION_KV_MLX4G32 && D % 32) return PION_ERR_INVALID;
  if (!d_supported(D)) return PION_ERR_UNSUPPORTED;
  if ((size_t)N * D > ((size_t)1 << 40)) return PION_ERR_INVALID;
  // the mlx4g32 kernel addresses a kv-head's codes (N * D / 2 bytes) through a 32-bit
  // buffer range
  if (kv_format == PION_KV_MLX4G32 && (size_t)N * D >= ((size_t)1 << 33)) return PION_ERR_UNSUPPORTED;
  return PION_OK;
}

// Write a slot's arrays from K, V [H, N, D] (fp32 for an fp32 slot, else fp16): copies,
// or the mlx4g32 encoder with scale and bias interleaved as (scale | bias << 16) words.
hipError_t fill_from_fp16(char *base, const SlotLayout &L, int kv_format, const void *K,
                          const void *V, size_t elems, int D, hipStream_t st) {
  if (kv_format != PION_KV_MLX4G32) {
    const size_t bytes = elems * (kv_format == PION_KV_FP32 ? 4 : 2);
    hipError_t e = hipMemcpyAsync(base + L.off[0], K, bytes, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(base + L.off[1], V, bytes, hipMemcpyDeviceToDevice, st);
  }
  // K and V in one launch
  const int64_t rows = (int64_t)(elems / D);
  return launch_quantize_mlx4g32_pair(
      (const uint16_t *)K, (uint32_t *)(base + L.off[0]), (uint32_t *)(base + L.off[1]),
      (const uint16_t *)V, (uint32_t *)(base + L.off[2]), (uint32_t *)(base + L.off[3]), rows, D, st);
}

// Allocate the slot (sid, layer), let `fill` write its arrays on stream `st`, and install
// it under the capacity rules: least recently used slots are demoted first when the
// count or the byte budget would be exceeded, or when device memory is short; a
// replaced slot is freed after the new one is ready; a cold key is rehydrated.
template <typename Fill>
int install_slot(const char *sid, int layer, int H, int N, int D, int kv_format, hipStream_t st,
                 const Fill &fill) {
  const SlotLayout L = slot_layout(kv_format, H, N, D);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_tier.max_bytes > 0 && L.bytes > (size_t)g_tier.max_bytes) return PION_ERR_NOMEM;
  const std::string key = key_of(sid, layer);
  auto old = g_slots.find(key);
  const bool replacing = old != g_slots.end();
  const size_t old_bytes = replacing ? old->second.bytes : 0;
  // a cold key leaves the registry now (so that demotions below cannot drop it); it is
  // put back if the store fails
  ColdEntry was_cold;
  auto ci = g_cold.find(key);
  const bool rehydrate = ci != g_cold.end();
  if (rehydrate) {
    was_cold = ci->second;
    g_cold.erase(ci);
  }
  auto fail = [&](int rc) {
    if (rehydrate) {
      g_cold[key] = was_cold;
      trim_cold();
    }
    return rc;
  };
  // room: demote least recently used slots until the count and the byte budget hold
  // (a replaced slot's bytes count as freed)
  while ((long long)(g_slots.size() - (replacing ? 1 : 0) + 1) > g_tier.max_slots ||
         (g_tier.max_bytes > 0 &&
          g_tier.resident - old_bytes + L.bytes > (size_t)g_tier.max_bytes))
    if (!demote_lru(key)) break;

  Slot sl;
  sl.H = H;
  sl.N = N;
  sl.D = D;
  sl.fmt = kv_format;
  sl.bytes = L.bytes;
  // device memory short: demote further, least recently used first
  while (hipMalloc(&sl.mem, sl.bytes) != hipSuccess) {
    (void)hipGetLastError();
    sl.mem = nullptr;
    if (!demote_lru(key)) return fail(PION_ERR_NOMEM);
  }
  sl.view = make_view(sl.mem, kv_format, H, N, D);
  hipError_t e = fill((char *)sl.mem, L, st);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&sl.ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(sl.ready, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free_slot(sl);
    return fail(PION_ERR_HIP);
  }
  sl.stream = st;
  if (replacing) {
    g_tier.resident -= old_bytes;
    free_slot(g_slots[key]);
  }
  if (rehydrate) ++g_tier.rehydrates;
  g_tier.resident += sl.bytes;
  sl.last = ++g_tier.clock;
  g_slots[key] = sl;
  return PION_OK;
}

Slot *find_slot(const char *sid, int layer) {
  auto it = g_slots.find(key_of(sid, layer));
  return it == g_slots.end() ? nullptr : &it->second;
}

// Common checks of the query entry points that need no slot. Returns PION_OK or an error.
int check_query_args(const char *sid, int H_q, int D, int M, const void *Q, const float *out) {
  if (!sid_ok(sid) || !Q || !out) return PION_ERR_INVALID;
  if (!aligned(Q, 16) || !aligned(out, 4)) return PION_ERR_INVALID;
  if (H_q < 1 || H_q > kMaxHeads || M < 1 || D <= 0) return PION_ERR_INVALID;
  if (!d_supported(D)) return PION_ERR_UNSUPPORTED;
  return PION_OK;
}

// Kernel names of the current call's launches, on the calling thread.
thread_local std::string g_plan;
void plan_begin() { g_plan.clear(); }

// pion_prefix_query, with the plan's workspace from the fixed scratch when `fixed`.
int query_one(const char *sid, int layer, int H_q, int D, int M, const void *Q,
              const int32_t *head_map, float *out, float *lse, void *stream, bool fixed) {
  plan_begin();
  int rc = check_query_args(sid, H_q, D, M, Q, out);
  if (rc != PION_OK) return rc;
  if (lse && !aligned(lse, 4)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  Slot *sl = find_slot(sid, layer);
  if (!sl) return absent_status(sid, layer);
  if (sl->D != D) return PION_ERR_INVALID;
  std::vector<int> hm;
  if (!resolve_map(head_map, H_q, sl->H, hm)) return PION_ERR_INVALID;
  if (!on_device(Q) || !on_device(out) || (lse && !on_device(lse))) return PION_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (order_after(sl->ready, sl->stream, sl->done, st) != hipSuccess) return PION_ERR_HIP;
  AttnCall c{};
  c.Q = Q;
  c.H_q = H_q;
  c.M = M;
  c.D = D;
  c.hm = &hm;
  c.H_kv = sl->H;
  c.out = out;
  c.lse = lse;
  FixedScratch fx;
  if (fixed) {
    void *scr = nullptr;
    if (noalloc_scratch(st, &scr) != hipSuccess) return PION_ERR_HIP;
    fx.counters = (int *)scr;
    fx.base = (char *)scr + kNoallocCounterBytes;
    fx.bytes = kNoallocScratchBytes - kNoallocCounterBytes;
    g_fixed = &fx;
  }
  rc = run_attention({sl}, c, st);
  g_fixed = nullptr;
  if (fx.too_small) return PION_ERR_SCRATCH;
  if (rc == PION_OK) touch(sl);
  return rc;
}

}  // namespace

namespace pion {
void note_launch(const char *fmt, ...) {
  char buf[160];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (!g_plan.empty()) g_plan += " + ";
  g_plan += buf;
}
}  // namespace pion

extern "C" {

const char *pion_prefix_last_plan(void) { return g_plan.c_str(); }

int pion_bench_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  plan_begin();
  if (bytes < 0 || bytes % 16) return PION_ERR_INVALID;
  if (bytes == 0) return PION_OK;
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4)) return PION_ERR_INVALID;
  if (!on_device(buf) || !on_device(sink)) return PION_ERR_INVALID;
  return launch_stream_read(buf, bytes, sink, (hipStream_t)stream) == hipSuccess ? PION_OK
                                                                                 : PION_ERR_HIP;
}

int pion_bench_mfma_peak(int iters, double *flops, uint32_t *sink, void *stream) {
  plan_begin();
  if (iters < 1 || !flops || !sink || !aligned(sink, 4)) return PION_ERR_INVALID;
  if (!on_device(sink)) return PION_ERR_INVALID;
  return launch_mfma_peak(iters, flops, sink, (hipStream_t)stream) == hipSuccess ? PION_OK
                                                                                : PION_ERR_HIP;
}

const char *pion_status_str(int status) {
  switch (status) {
    case PION_OK: return "ok";
    case PION_ERR_NOT_FOUND: return "session not found";
    case PION_ERR_INVALID: return "invalid argument";
    case PION_ERR_UNSUPPORTED: return "unsupported";
    case PION_ERR_NOMEM: return "out of memory";
    case PION_ERR_HIP: return "HIP error";
    case PION_ERR_COLDMISS: return "cold miss";
    case PION_ERR_SCRATCH: return "exceeds the fixed scratch area";
    default: return "unknown status";
  }
}

int pion_kv_quantize_mlx4g32(const void *x, int64_t rows, int D, uint32_t *codes, void *scales,
                             void *biases, void *stream) {
  plan_begin();
  if (rows < 0 || D <= 0 || D % 32) return PION_ERR_INVALID;
  if (rows == 0) return PION_OK;
  if (!x || !codes || !scales || !biases) return PION_ERR_INVALID;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(scales, 2) || !aligned(biases, 2))
    return PION_ERR_INVALID;
  if (!on_device(x) || !on_device(codes) || !on_device(scales) || !on_device(biases))
    return PION_ERR_INVALID;
  if (launch_quantize_mlx4g32((const uint16_t *)x, rows, D, codes, (uint16_t *)scales,
                              (uint16_t *)biases, 1, (hipStream_t)stream) != hipSuccess)
    return PION_ERR_HIP;
  return PION_OK;
}

int pion_prefix_store(const char *sid, int layer, int H, int N, int D, const void *K,
                      const void *V, int kv_format, void *stream) {
  plan_begin();
  int rc = check_slot_shape(sid, H, N, D, kv_format);
  if (rc != PION_OK) return rc;
  if (!K || !V || !aligned(K, 16) || !aligned(V, 16)) return PION_ERR_INVALID;
  if (!on_device(K) || !on_device(V)) return PION_ERR_INVALID;
  const size_t elems = (size_t)H * N * D;
  return install_slot(sid, layer, H, N, D, kv_format, (hipStream_t)stream,
                      [&](char *base, const SlotLayout &L, hipStream_t st) {
                        return fill_from_fp16(base, L, kv_format, K, V, elems, D, st);
                      });
}

int pion_prefix_warm(const char *sid, int layer, int H, int N, int D, int src_format,
                     const void *K_rows, const void *V_rows, int kv_format, void *stream) {
  plan_begin();
  int rc = check_slot_shape(sid, H, N, D, kv_format);
  if (rc != PION_OK) return rc;
  if (src_format != PION_KV_FP16 && src_format != PION_KV_MLX4G32) return PION_ERR_INVALID;
  if (src_format == PION_KV_MLX4G32 && D % 32) return PION_ERR_INVALID;
  const uintptr_t al = src_format == PION_KV_FP16 ? 16 : 4;
  if (!K_rows || !V_rows || !aligned(K_rows, al) || !aligned(V_rows, al)) return PION_ERR_INVALID;
  if (!on_device(K_rows) || !on_device(V_rows)) return PION_ERR_INVALID;
  return install_slot(
      sid, layer, H, N, D, kv_format, (hipStream_t)stream,
      [&](char *base, const SlotLayout &L, hipStream_t st) -> hipError_t {
        if (kv_format == PION_KV_FP16) {  // dequantized (if need be) and transposed
          hipError_t e = launch_rows_to_fp16_slot(K_rows, src_format, N, H, D,
                                                  (uint16_t *)(base + L.off[0]), st);
          if (e != hipSuccess) return e;
          return launch_rows_to_fp16_slot(V_rows, src_format, N, H, D,
                                          (uint16_t *)(base + L.off[1]), st);
        }
        if (kv_format == PION_KV_FP32) {  // dequantized to fp32 and transposed
          hipError_t e = launch_rows_to_fp32_slot(K_rows, src_format, N, H, D,
                                                  (float *)(base + L.off[0]), st);
          if (e != hipSuccess) return e;
          return launch_rows_to_fp32_slot(V_rows, src_format, N, H, D,
                                          (float *)(base + L.off[1]), st);
        }
        if (src_format == PION_KV_MLX4G32) {  // codes, scales and biases move unchanged
          hipError_t e = launch_rows_to_mlx4_slot(K_rows, N, H, D, (uint32_t *)(base + L.off[0]),
                                                  (uint32_t *)(base + L.off[1]), st);
          if (e != hipSuccess) return e;
          return launch_rows_to_mlx4_slot(V_rows, N, H, D, (uint32_t *)(base + L.off[2]),
                                          (uint32_t *)(base + L.off[3]), st);
        }
        // fp16 rows into an mlx4g32 slot: transpose into a scratch [H, N, D], then encode
        const size_t elems = (size_t)H * N * D;
        void *tmp[2] = {nullptr, nullptr};
        hipError_t e = hipSuccess;
        for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipMalloc(&tmp[i], elems * 2);
        if (e == hipSuccess)
          e = launch_rows_to_fp16_slot(K_rows, PION_KV_FP16, N, H, D, (uint16_t *)tmp[0], st);
        if (e == hipSuccess)
          e = launch_rows_to_fp16_slot(V_rows, PION_KV_FP16, N, H, D, (uint16_t *)tmp[1], st);
        if (e == hipSuccess) e = fill_from_fp16(base, L, kv_format, tmp[0], tmp[1], elems, D, st);
        for (void *t : tmp)
          if (t) (void)hipFree(t);  // waits for the encoder
        return e;
      });
}

int pion_vstore_fetch_f32(const void *rows, int fmt, int64_t n_rows, int kv_dim, int64_t start,
                          int64_t end, float *out, void *stream) {
  plan_begin();
  if (n_rows < 0 || kv_dim <= 0) return PION_ERR_INVALID;
  if (fmt != PION_KV_FP16 && fmt != PION_KV_MLX4G32) return PION_ERR_INVALID;
  if (kv_dim % 32) return PION_ERR_INVALID;  // whole groups of 32 values
  if (start < 0 || end < start || end > n_rows) return PION_ERR_INVALID;
  if (end == start) return PION_OK;  // nothing read or written
  if (!rows || !out) return PION_ERR_INVALID;
  if (!aligned(rows, fmt == PION_KV_FP16 ? 16 : 4) || !aligned(out, 16)) return PION_ERR_INVALID;
  if (!on_device(rows) || !on_device(out)) return PION_ERR_INVALID;
  return launch_vstore_fetch(rows, fmt, kv_dim, start, end - start, out, (hipStream_t)stream) ==
                 hipSuccess
             ? PION_OK
             : PION_ERR_HIP;
}

int pion_prefix_lookup(const char *sid, int layer) {
  if (!sid_ok(sid)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  return find_slot(sid, layer) ? 1 : g_cold.count(key_of(sid, layer)) ? 2 : 0;
}

int pion_prefix_drop(const char *sid, int layer) {
  if (!sid_ok(sid)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  int n = 0;
  if (layer >= 0) {
    const std::string key = key_of(sid, layer);
    auto it = g_slots.find(key);
    if (it != g_slots.end()) {
      g_tier.resident -= it->second.bytes;
      free_slot(it->second);
      g_slots.erase(it);
      n = 1;
    }
    return n + (int)g_cold.erase(key);
  }
  const std::string prefix = std::string(sid) + '\0';
  for (auto it = g_slots.begin(); it != g_slots.end();) {
    if (it->first.compare(0, prefix.size(), prefix) == 0) {
      g_tier.resident -= it->second.bytes;
      free_slot(it->second);
      it = g_slots.erase(it);
      ++n;
    } else {
      ++it;
    }
  }
  for (auto it = g_cold.begin(); it != g_cold.end();) {
    if (it->first.compare(0, prefix.size(), prefix) == 0) {
      it = g_cold.erase(it);
      ++n;
    } else {
      ++it;
    }
  }
  return n;
}

int pion_prefix_info(const char *sid, int layer, int *H, int *N, int *D, int *kv_format) {
  if (!sid_ok(sid)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  const Slot *s = find_slot(sid, layer);
  if (!s) {
    auto c = g_cold.find(key_of(sid, layer));
    if (c == g_cold.end()) return PION_ERR_NOT_FOUND;
    if (H) *H = c->second.H;  // the shape the demoted slot had
    if (N) *N = c->second.N;
    if (D) *D = c->second.D;
    if (kv_format) *kv_format = c->second.fmt;
    return PION_ERR_COLDMISS;
  }
  if (H) *H = s->H;
  if (N) *N = s->N;
  if (D) *D = s->D;
  if (kv_format) *kv_format = s->fmt;
  return PION_OK;
}

int pion_prefix_stats(pion_prefix_stats_t *out) {
  if (!out) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  out->warm_slots = (int64_t)g_slots.size();
  out->cold_slots = (int64_t)g_cold.size();
  out->demotions = g_tier.demotions;
  out->rehydrates = g_tier.rehydrates;
  out->resident_bytes = (int64_t)g_tier.resident;
  out->max_slots = g_tier.max_slots;
  out->max_bytes = g_tier.max_bytes;
  out->cold_capacity = g_tier.cold_slots;
  return PION_OK;
}

int pion_prefix_set_capacity(int64_t max_slots, int64_t max_bytes, int64_t cold_slots) {
  if (max_slots < 1 || max_bytes < 0 || cold_slots < 0) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  g_tier.max_slots = max_slots;
  g_tier.max_bytes = max_bytes;
  g_tier.cold_slots = cold_slots;
  while ((long long)g_slots.size() > g_tier.max_slots ||
         (g_tier.max_bytes > 0 && g_tier.resident > (size_t)g_tier.max_bytes))
    if (!demote_lru(std::string())) break;
  trim_cold();
  return PION_OK;
}

int pion_prefix_query(const char *sid, int layer, int H_q, int D, int M, const void *Q,
                      const int32_t *head_map, float *out, float *lse, void *stream) {
  return query_one(sid, layer, H_q, D, M, Q, head_map, out, lse, stream, false);
}

int pion_prefix_query_noalloc(const char *sid, int layer, int H_q, int D, int M, const void *Q,
                              const int32_t *head_map, float *out, float *lse, void *stream) {
  return query_one(sid, layer, H_q, D, M, Q, head_map, out, lse, stream, true);
}

int pion_prefix_query_layers(const char *sid, int layer0, int n_layers, int H_q, int D, int M,
                             const void *Q, const int32_t *head_map, float *out, float *lse,
                             void *stream) {
  plan_begin();
  int rc = check_query_args(sid, H_q, D, M, Q, out);
  if (rc != PION_OK) return rc;
  if (n_layers < 1 || n_layers > kMaxBatch) return PION_ERR_INVALID;
  if (lse && !aligned(lse, 4)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<const Slot *> slots(n_layers);
  for (int i = 0; i < n_layers; ++i) {
    Slot *sl = find_slot(sid, layer0 + i);
    if (!sl) return absent_status(sid, layer0 + i);
    slots[i] = sl;
  }
  const Slot &s0 = *slots[0];
  for (const Slot *sl : slots)
    if (sl->D != D || sl->H != s0.H || sl->fmt != s0.fmt) return PION_ERR_INVALID;
  std::vector<int> hm;
  if (!resolve_map(head_map, H_q, s0.H, hm)) return PION_ERR_INVALID;
  if (!on_device(Q) || !on_device(out) || (lse && !on_device(lse))) return PION_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  for (int i = 0; i < n_layers; ++i) {
    Slot *sl = find_slot(sid, layer0 + i);
    if (order_after(sl->ready, sl->stream, sl->done, st) != hipSuccess) return PION_ERR_HIP;
  }
  AttnCall c{};
  c.Q = Q;
  c.q_stride = (size_t)H_q * M * D;
  c.H_q = H_q;
  c.M = M;
  c.D = D;
  c.hm = &hm;
  c.H_kv = s0.H;
  c.out = out;
  c.out_stride = (size_t)H_q * M * D;
  c.lse = lse;
  c.lse_stride = (size_t)H_q * M;
  rc = run_attention(slots, c, st);
  if (rc == PION_OK)
    for (int i = 0; i < n_layers; ++i) touch(find_slot(sid, layer0 + i));
  return rc;
}

int pion_prefix_query_fused(const char *sid, int layer, int H_q, int D, int M, int S_suf,
                            int H_kv, const void *Q, const void *K_suf, const void *V_suf,
                            const int32_t *head_map, float *out, float *lse, void *stream) {
  plan_begin();
  int rc = check_query_args(sid, H_q, D, M, Q, out);
  if (rc != PION_OK) return rc;
  if (S_suf < 0 || H_kv < 1 || H_kv > 255) return PION_ERR_INVALID;
  if (S_suf > 0 && (M > S_suf || !K_suf || !V_suf)) return PION_ERR_INVALID;
  if (S_suf > 0 && (!aligned(K_suf, 16) || !aligned(V_suf, 16))) return PION_ERR_INVALID;
  if (lse && !aligned(lse, 4)) return PION_ERR_INVALID;
  std::vector<int> hm;
  if (!resolve_map(head_map, H_q, H_kv, hm)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  Slot *sl = find_slot(sid, layer);
  if (!sl) return absent_status(sid, layer);
  if (sl->D != D || sl->H != H_kv) return PION_ERR_INVALID;
  if (!on_device(Q) || !on_device(out) || (lse && !on_device(lse))) return PION_ERR_INVALID;
  if (S_suf > 0 && (!on_device(K_suf) || !on_device(V_suf))) return PION_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (order_after(sl->ready, sl->stream, sl->done, st) != hipSuccess) return PION_ERR_HIP;
  AttnCall c{};
  c.Q = Q;
  c.H_q = H_q;
  c.M = M;
  c.D = D;
  c.hm = &hm;
  c.H_kv = H_kv;
  c.Ksuf = K_suf;
  c.Vsuf = V_suf;
  c.S_suf = S_suf;
  c.out = out;
  c.lse = lse;
  rc = run_attention({sl}, c, st);
  if (rc == PION_OK) touch(sl);
  return rc;
}

int pion_prefix_query_sparse_auto(const char *sid, int layer, int H_q, int D, int B, int K_top,
                                  int H_kv, int S_suf, const void *Q, const void *K_suf,
                                  const void *V_suf, const int32_t *head_map, float *out,
                                  float *lse, int32_t *blocks_out, void *stream) {
  plan_begin();
  int rc = check_query_args(sid, H_q, D, 1, Q, out);
  if (rc != PION_OK) return rc;
  if (B < 1 || K_top < 1 || K_top > kMaxKTop || S_suf < 0 || H_kv < 1 || H_kv > 255)
    return PION_ERR_INVALID;
  if (S_suf > 0 && (!K_suf || !V_suf)) return PION_ERR_INVALID;
  if (S_suf > 0 && (!aligned(K_suf, 16) || !aligned(V_suf, 16))) return PION_ERR_INVALID;
  if ((lse && !aligned(lse, 4)) || (blocks_out && !aligned(blocks_out, 4)))
    return PION_ERR_INVALID;
  std::vector<int> hm;
  if (!resolve_map(head_map, H_q, H_kv, hm)) return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  Slot *sl = find_slot(sid, layer);
  if (!sl) return absent_status(sid, layer);
  if (sl->D != D || sl->H != H_kv) return PION_ERR_INVALID;
  if (!on_device(Q) || !on_device(out) || (lse && !on_device(lse))) return PION_ERR_INVALID;
  if (S_suf > 0 && (!on_device(K_suf) || !on_device(V_suf))) return PION_ERR_INVALID;
  if (blocks_out && !on_device(blocks_out)) return PION_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (order_after(sl->ready, sl->stream, sl->done, st) != hipSuccess) return PION_ERR_HIP;

  const int nb = (sl->N + B - 1) / B;
  const int n_sel = std::min(K_top, nb);
  // block means: cached per (slot, B), built on first use
  auto it = sl->kmeans.find(B);
  if (it == sl->kmeans.end()) {
    KMean km;
    km.nb = nb;
    if (hipMalloc(&km.ptr, (size_t)H_kv * nb * D * sizeof(float)) != hipSuccess) {
      (void)hipGetLastError();
      return PION_ERR_NOMEM;
    }
    hipError_t e = launch_block_mean(sl->view, B, km.ptr, st);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&km.ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(km.ready, st);
    if (e != hipSuccess) {
      (void)hipFree(km.ptr);
      if (km.ready) (void)hipEventDestroy(km.ready);
      return PION_ERR_HIP;
    }
    km.stream = st;
    it = sl->kmeans.emplace(B, km).first;
  } else if (order_after(it->second.ready, it->second.stream, it->second.done, st) !=
             hipSuccess) {
    return PION_ERR_HIP;
  }
  // score and block buffers: a per-stream allocation separate from the partials'
  // workspace (run_attention may grow and move that one)
  const size_t score_bytes = align256((size_t)H_kv * nb * sizeof(uint32_t));
  const size_t cand_bytes =
      align256((size_t)H_kv * ((nb + 63) / 64) * std::min(K_top, 64) * sizeof(uint64_t));
  const size_t blk_bytes = align256((size_t)H_kv * K_top * sizeof(int32_t));
  Workspace &w = g_sel_ws[st];
  if (w.cap < score_bytes + cand_bytes + blk_bytes) {
    if (w.ptr) {
      if (hipStreamSynchronize(st) != hipSuccess) return PION_ERR_HIP;
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.cap = 0;
    }
    const size_t cap = align256(score_bytes + cand_bytes + blk_bytes + (1 << 16));
    if (hipMalloc(&w.ptr, cap) != hipSuccess) {
      (void)hipGetLastError();
      return PION_ERR_NOMEM;
    }
    w.cap = cap;
  }
  uint32_t *keys = (uint32_t *)w.ptr;
  uint64_t *cand = (uint64_t *)((char *)w.ptr + score_bytes);
  int32_t *blocks =
      blocks_out ? blocks_out : (int32_t *)((char *)w.ptr + score_bytes + cand_bytes);

  HeadMap hmap;
  memset(&hmap, 0, sizeof(hmap));
  hmap.H_q = H_q;
  for (int h = 0; h < H_q; ++h) hmap.m[h] = (uint8_t)hm[h];
  // the selection's tickets use the stream's split counters (zero between launches)
  int *counters;
  if (get_counters(st, &counters) != hipSuccess) return PION_ERR_NOMEM;
  if (launch_block_select(Q, sl->fmt == PION_KV_FP32, hmap, it->second.ptr, H_kv, nb, D, K_top,
                          keys, cand, counters, blocks, st) != hipSuccess)
    return PION_ERR_HIP;

  AttnCall c{};
  c.Q = Q;
  c.H_q = H_q;
  c.M = 1;
  c.D = D;
  c.hm = &hm;
  c.H_kv = H_kv;
  c.Ksuf = K_suf;
  c.Vsuf = V_suf;
  c.S_suf = S_suf;
  c.blocks = blocks;
  c.n_sel = n_sel;
  c.K_top = K_top;
  c.B = B;
  c.out = out;
  c.lse = lse;
  rc = run_attention({sl}, c, st);
  if (rc == PION_OK) touch(sl);
  return rc;
}

int pion_prefix_query_sparse(const char *sid, int layer, int H, int D, int K_sparse_max,
                             const void *Q, const int32_t *indices, const int32_t *counts,
                             float *out, float *lse, void *stream) {
  plan_begin();
  int rc = check_query_args(sid, H, D, 1, Q, out);
  if (rc != PION_OK) return rc;
  if (K_sparse_max < 1 || K_sparse_max > (1 << 24) || !indices || !counts) return PION_ERR_INVALID;
  if (!aligned(indices, 4) || !aligned(counts, 4) || (lse && !aligned(lse, 4)))
    return PION_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  Slot *sl = find_slot(sid, layer);
  if (!sl) return absent_status(sid, layer);
  if (sl->D != D || sl->H != H) return PION_ERR_INVALID;
  if (sl->fmt == PION_KV_MLX4G32) return PION_ERR_UNSUPPORTED;
  if (!on_device(Q) || !on_device(out) || (lse && !on_device(lse)) || !on_device(indices) ||
      !on_device(counts))
    return PION_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (order_after(sl->ready, sl->stream, sl->done, st) != hipSuccess) return PION_ERR_HIP;
  std::vector<int> hm(H);
  for (int h = 0; h < H; ++h) hm[h] = h;
  AttnCall c{};
  c.Q = Q;
  c.H_q = H;
  c.M = 1;
  c.D = D;
  c.hm = &hm;
  c.H_kv = H;
  c.gidx = indices;
  c.gcount = counts;
  c.gmax = K_sparse_max;
  c.out = out;
  c.lse = lse;
  rc = run_attention({sl}, c, st);
  if (rc == PION_OK) touch(sl);
  return rc;
}

}  // extern "C"
