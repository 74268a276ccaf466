// Host runtime of the fused LongFlow decode step: argument validation, the
// layout of the caller's device state buffer, the split-KV work list and the
// C ABI entry points declared in include/lf.h.
//
// The cache is static: its slots are fixed at init and every step overwrites
// one of them in place (the statically pre-allocated KV cache of the LongFlow
// summary, section 2.C).  This file only plans work and launches it; every
// arithmetic step of the decode runs in lf_kernel.hip.
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>
#include <vector>

#include "../../include/lf.h"
#include "lf_internal.h"

struct lf_cache {
  uint64_t magic;
  lf_config cfg;
  int group;
  lf::StateLayout lay;
  void* k_cache;
  void* v_cache;
  char* state;
  size_t state_bytes;  // capacity of the caller's state buffer
  float scale_log2;
  uint32_t wait_ticks;  // split chunks' wait for their pair's statistics (s_memrealtime ticks)
  int32_t u_budget;  // the common budget when every sequence has the same one, else 0
  std::vector<int32_t> budgets;  // per sequence, as validated at init
};

namespace {

thread_local char g_err[512] = "";

lf_status fail(lf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

size_t align_up(size_t x) { return (x + lf::kAlign - 1) / lf::kAlign * lf::kAlign; }

// Default wait of a split chunk for its pair's statistics: 100 us (100 MHz ticks).
constexpr uint32_t kDefaultWaitTicks = 10000;

lf_status validate_config(const lf_config* cfg) {
  if (!cfg) return fail(LF_ERR_ARG, "cfg is NULL");
  if (cfg->batch < 1) return fail(LF_ERR_ARG, "batch must be >= 1 (got %d)", cfg->batch);
  if (cfg->n_kv_heads < 1) return fail(LF_ERR_ARG, "n_kv_heads must be >= 1 (got %d)", cfg->n_kv_heads);
  if (cfg->n_q_heads < cfg->n_kv_heads || cfg->n_q_heads % cfg->n_kv_heads)
    return fail(LF_ERR_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", cfg->n_q_heads,
                cfg->n_kv_heads);
  const int group = cfg->n_q_heads / cfg->n_kv_heads;
  if (group > lf::kMaxGroup)
    return fail(LF_ERR_UNSUPPORTED, "group size n_q_heads/n_kv_heads = %d; supported 1..%d", group, lf::kMaxGroup);
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(LF_ERR_UNSUPPORTED, "head_dim %d; supported 64 and 128", cfg->head_dim);
  if (cfg->dtype != LF_F32 && cfg->dtype != LF_BF16)
    return fail(LF_ERR_UNSUPPORTED, "dtype %d; supported LF_F32 and LF_BF16", cfg->dtype);
  if (cfg->score != LF_SCORE_ATTN && cfg->score != LF_SCORE_VL1 && cfg->score != LF_SCORE_NONE)
    return fail(LF_ERR_ARG, "score mode %d; expected LF_SCORE_ATTN, LF_SCORE_VL1 or LF_SCORE_NONE", cfg->score);
  if (cfg->max_budget < 1 || cfg->max_budget > lf::kMaxBudget)
    return fail(LF_ERR_ARG, "max_budget %d outside [1, %d]", cfg->max_budget, lf::kMaxBudget);
  if (cfg->sink < 0 || cfg->recent < 0) return fail(LF_ERR_ARG, "sink and recent must be >= 0");
  if (cfg->reserved != 0) return fail(LF_ERR_ARG, "reserved must be 0");
  if (!(cfg->softmax_scale == cfg->softmax_scale) || std::isinf(cfg->softmax_scale))
    return fail(LF_ERR_ARG, "softmax_scale must be finite");
  if (cfg->chunk_slots < 0) return fail(LF_ERR_ARG, "chunk_slots must be >= 0");
  if (cfg->chunk_slots > 0) {
    const int tile = lf::tile_rows(cfg->dtype, cfg->head_dim, group);
    if (cfg->chunk_slots % tile)
      return fail(LF_ERR_ARG, "chunk_slots %d must be a multiple of the kernel tile (%d rows)", cfg->chunk_slots,
                  tile);
  }
  const double cache_elems = (double)cfg->batch * cfg->n_kv_heads * cfg->max_budget * cfg->head_dim;
  if (cache_elems > 9.0e15) return fail(LF_ERR_ARG, "cache too large");
  return LF_OK;
}

// Metadata and ring of sequence b's pairs for a cache holding `t` tokens laid
// out as lf_init_cache describes (meta and ring indexed by pair, the other
// PairMeta fields already set by the layout).
void start_sequence(const lf_config& cfg, int b, int64_t t, int32_t budget, lf::PairMeta* meta, int32_t* ring) {
  const int R = cfg.recent;
  const int64_t len = t < budget ? t : budget;
  for (int g = 0; g < cfg.n_kv_heads; ++g) {
    const int p = b * cfg.n_kv_heads + g;
    meta[p].t = (int32_t)t;
    meta[p].len = (int32_t)len;
    for (int j = 0; j < R; ++j) ring[(size_t)p * R + j] = -1;
    // The R newest cached positions [t - R, t): slot = position while the
    // prefill fits, else they are the last R slots (layout contract).
    for (int64_t pos = t - R < 0 ? 0 : t - R; pos < t; ++pos) {
      const int64_t slot = t <= budget ? pos : budget - (t - pos);
      ring[(size_t)p * R + pos % R] = (int32_t)slot;
    }
  }
}

lf_status validate_budgets(const lf_config* cfg, const int32_t* budgets, std::vector<int32_t>& out) {
  out.assign(cfg->batch, cfg->max_budget);
  if (budgets)
    for (int b = 0; b < cfg->batch; ++b) out[b] = budgets[b];
  for (int b = 0; b < cfg->batch; ++b) {
    if (out[b] < 1 || out[b] > cfg->max_budget)
      return fail(LF_ERR_ARG, "budget[%d] = %d outside [1, max_budget = %d]", b, out[b], cfg->max_budget);
    if ((int64_t)out[b] <= (int64_t)cfg->sink + cfg->recent)
      return fail(LF_ERR_ARG, "budget[%d] = %d must exceed sink + recent = %d", b, out[b], cfg->sink + cfg->recent);
  }
  return LF_OK;
}

// Chunk length: a multiple of the kernel tile.  Pairs are split only when
// there are too few of them to give about kTargetItems workgroups; a pair never
// has more than kMaxChunks chunks.
int choose_chunk(const lf_config* cfg, int group, int max_b) {
  const int tile = lf::tile_rows(cfg->dtype, cfg->head_dim, group);
  if (cfg->chunk_slots > 0) return cfg->chunk_slots;  // explicit: make_layout checks the chunk count
  const int64_t pairs = (int64_t)cfg->batch * cfg->n_kv_heads;
  int64_t want = (lf::kTargetItems + pairs - 1) / pairs;  // chunks per pair
  if (want < 1) want = 1;
  int chunk = (int)((max_b + want - 1) / want);
  const int min_chunk = (max_b + lf::kMaxChunks - 1) / lf::kMaxChunks;
  if (chunk < min_chunk) chunk = min_chunk;
  return (chunk + tile - 1) / tile * tile;
}

lf_status make_layout(const lf_config* cfg, const std::vector<int32_t>& bud, lf::StateLayout& L,
                      std::vector<lf::WorkItem>* items, std::vector<lf::PairMeta>* meta) {
  const int group = cfg->n_q_heads / cfg->n_kv_heads;
  int max_b = 0;
  for (int x : bud) max_b = x > max_b ? x : max_b;
  const int chunk = choose_chunk(cfg, group, max_b);
  const int64_t P = (int64_t)cfg->batch * cfg->n_kv_heads;
  int64_t W = 0, S = 0;
  int max_nchunk = 0;
  for (int b = 0; b < cfg->batch; ++b) {
    const int nch = (bud[b] + chunk - 1) / chunk;
    max_nchunk = nch > max_nchunk ? nch : max_nchunk;
    W += (int64_t)nch * cfg->n_kv_heads;
    S += (int64_t)(bud[b] + lf::kSlotPad - 1) / lf::kSlotPad * lf::kSlotPad * cfg->n_kv_heads;
  }
  if (max_nchunk > lf::kMaxChunks) return fail(LF_ERR_ARG, "chunk_slots too small: %d chunks per pair", max_nchunk);
  if (W > 0x7FFFFFFF || P > 0x7FFFFFFF || S > 0x7FFFFFFF) return fail(LF_ERR_ARG, "batch too large");
  L.n_pairs = (int32_t)P;
  L.n_items = (int32_t)W;
  L.total_slots = (int32_t)S;
  L.chunk = chunk;
  L.max_nchunk = max_nchunk;
  size_t off = 0;
  L.header = off;
  off = align_up(off + sizeof(lf::StateHeader));
  L.meta = off;
  off = align_up(off + sizeof(lf::PairMeta) * P);
  L.ring = off;
  off = align_up(off + sizeof(int32_t) * P * (size_t)cfg->recent);
  L.count = off;
  off = align_up(off + sizeof(uint32_t) * P);
  L.items = off;
  off = align_up(off + sizeof(lf::WorkItem) * W);
  L.xcell = off;
  off = align_up(off + sizeof(uint64_t) * (size_t)group * (cfg->head_dim + 2) * W);
  L.xcand = off;
  off = align_up(off + sizeof(uint64_t) * 2 * W);
  L.logits = off;  // none without importance (LF_SCORE_NONE)
  if (cfg->score != LF_SCORE_NONE) off = align_up(off + sizeof(float) * (size_t)group * S);
  L.total = off;
  if (items || meta) {
    // Workspace offsets follow pair order; work items follow sequences in
    // decreasing budget (longest first, so the dispatcher's greedy placement
    // balances ragged budgets), the chunks of one pair contiguous.
    if (items) items->clear();
    if (meta) meta->assign(P, lf::PairMeta{});
    int32_t slot = 0;
    for (int b = 0; b < cfg->batch; ++b) {
      const int lstride = (bud[b] + lf::kSlotPad - 1) / lf::kSlotPad * lf::kSlotPad;
      for (int g = 0; g < cfg->n_kv_heads; ++g) {
        if (meta) {
          lf::PairMeta& m = (*meta)[b * cfg->n_kv_heads + g];
          m.budget = bud[b];
          m.nchunk = (bud[b] + chunk - 1) / chunk;
          m.slot0 = slot;
          m.lstride = lstride;
          m.epoch = 1;
        }
        slot += lstride;
      }
    }
    std::vector<int> order(cfg->batch);
    for (int b = 0; b < cfg->batch; ++b) order[b] = b;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return bud[x] > bud[y]; });
    int32_t item = 0;
    for (int b : order) {
      const int nch = (bud[b] + chunk - 1) / chunk;
      for (int g = 0; g < cfg->n_kv_heads; ++g) {
        const int32_t p = b * cfg->n_kv_heads + g;
        if (meta) (*meta)[p].item0 = item;
        for (int c = 0; c < nch; ++c) {
          const int start = c * chunk;
          const int cnt = bud[b] - start < chunk ? bud[b] - start : chunk;
          if (items) items->push_back(lf::WorkItem{p, start, cnt, c});
        }
        item += nch;
      }
    }
  }
  return LF_OK;
}

lf_status check_handle(const lf_cache* c) {
  if (!c) return fail(LF_ERR_ARG, "cache handle is NULL");
  if (c->magic != lf::kHandleMagic) return fail(LF_ERR_STATE, "cache handle is not a live lf_cache");
  return LF_OK;
}

// Arguments shared by lf_reset_sequences and lf_reset_sequences_budget.
lf_status check_reset_args(const lf_cache* cache, int32_t n, const int32_t* seqs, const int64_t* seq_len) {
  lf_status st = check_handle(cache);
  if (st != LF_OK) return st;
  if (n < 0) return fail(LF_ERR_ARG, "n must be >= 0");
  if (n == 0) return LF_OK;
  if (!seqs || !seq_len) return fail(LF_ERR_ARG, "seqs and seq_len must be non-NULL");
  const lf_config& cfg = cache->cfg;
  std::vector<char> seen(cfg.batch, 0);
  for (int i = 0; i < n; ++i) {
    if (seqs[i] < 0 || seqs[i] >= cfg.batch) return fail(LF_ERR_ARG, "seqs[%d] = %d outside [0, %d)", i, seqs[i], cfg.batch);
    if (seen[seqs[i]]) return fail(LF_ERR_ARG, "sequence %d listed twice", seqs[i]);
    seen[seqs[i]] = 1;
    if (seq_len[i] < 0 || seq_len[i] > 0x7FFFFFFFll - 0x10000000ll)
      return fail(LF_ERR_ARG, "seq_len[%d] = %lld out of range", i, (long long)seq_len[i]);
  }
  return LF_OK;
}

lf_status step_impl(const void* q, const void* k_new, const void* v_new, lf_cache* cache, void* out,
                    int32_t* evict_idx, float* scores, float* lse, void* stream) {
  lf_status st = check_handle(cache);
  if (st != LF_OK) return st;
  if (!q || !k_new || !v_new || !out || !evict_idx)
    return fail(LF_ERR_ARG, "q, k_new, v_new, out and evict_idx must be non-NULL");
  const lf_config& cfg = cache->cfg;
  lf::StepArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.out = out;
  a.evict_idx = evict_idx;
  a.dbg_scores = scores;
  a.dbg_lse = lse;
  char* s = cache->state;
  const lf::StateLayout& L = cache->lay;
  a.meta = reinterpret_cast<lf::PairMeta*>(s + L.meta);
  a.ring = reinterpret_cast<int32_t*>(s + L.ring);
  a.items = reinterpret_cast<const lf::WorkItem*>(s + L.items);
  a.xcell = reinterpret_cast<uint64_t*>(s + L.xcell);
  a.xcand = reinterpret_cast<uint64_t*>(s + L.xcand);
  a.count = reinterpret_cast<uint32_t*>(s + L.count);
  a.deferred = reinterpret_cast<uint32_t*>(s + L.header + offsetof(lf::StateHeader, deferred));
  a.fault = reinterpret_cast<uint32_t*>(s + L.header + offsetof(lf::StateHeader, fault));
  a.logits = reinterpret_cast<float*>(s + L.logits);
  a.wait_ticks = cache->wait_ticks;
  a.n_items = L.n_items;
  a.n_pairs = cfg.batch * cfg.n_kv_heads;
  a.n_q_heads = cfg.n_q_heads;
  a.n_kv_heads = cfg.n_kv_heads;
  a.max_budget = cfg.max_budget;
  a.sink = cfg.sink;
  a.recent = cfg.recent;
  a.scale_log2 = cache->scale_log2;
  a.vl1 = cfg.score == LF_SCORE_VL1;
  a.score_none = cfg.score == LF_SCORE_NONE;
  a.u_budget = cache->u_budget;
  a.u_chunk = L.chunk;
  a.u_nchunk = cache->u_budget > 0 ? (cache->u_budget + L.chunk - 1) / L.chunk : 0;
  if (lf::launch_step(cfg.dtype, cfg.head_dim, cache->group, a, stream, g_err, sizeof(g_err)))
    return LF_ERR_HIP;
  return LF_OK;
}

// Prefill compression with the scratch `work` (work_bytes >= need, the size
// lf_prefill_work_bytes gives): shared by lf_prefill_compress (caller's
// workspace) and lf_prefill_compress_noalloc (the library's static scratch).
lf_status prefill_impl(const lf_config* cfg, const int32_t* budgets, const int32_t* prefill, int32_t max_prefill,
                       const void* q_last, const void* k_pre, const void* v_pre, void* k_cache, void* v_cache,
                       int32_t* kept, void* work, size_t work_bytes, size_t need, void* stream) {
  std::vector<int32_t> bud;
  lf_status st = validate_budgets(cfg, budgets, bud);
  if (st != LF_OK) return st;
  if (!prefill) return fail(LF_ERR_ARG, "prefill is NULL");
  for (int b = 0; b < cfg->batch; ++b)
    if (prefill[b] < 1 || prefill[b] > max_prefill)
      return fail(LF_ERR_ARG, "prefill[%d] = %d outside [1, max_prefill = %d]", b, prefill[b], max_prefill);
  const void* dev[] = {q_last, k_pre, v_pre, k_cache, v_cache, kept, work};
  const char* names[] = {"q_last", "k_pre", "v_pre", "k_cache", "v_cache", "kept", "work"};
  for (int i = 0; i < 7; ++i) {
    if (!dev[i]) return fail(LF_ERR_ARG, "%s is NULL", names[i]);
    if (reinterpret_cast<uintptr_t>(dev[i]) % 16) return fail(LF_ERR_ARG, "%s is not 16-byte aligned", names[i]);
  }
  if (work_bytes < need) return fail(LF_ERR_ARG, "work_bytes %zu < %zu (lf_prefill_work_bytes)", work_bytes, need);
  const size_t pairs = (size_t)cfg->batch * cfg->n_kv_heads;
  const int nck = (max_prefill + lf::kPrefillChunk - 1) / lf::kPrefillChunk;
  char* w = static_cast<char*>(work);
  float* stats = reinterpret_cast<float*>(w + align_up(sizeof(float) * pairs * (size_t)max_prefill));
  int32_t* dlen = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(stats) + align_up(sizeof(float) * pairs * nck * 16));
  float* logits = reinterpret_cast<float*>(reinterpret_cast<char*>(dlen) + align_up(sizeof(int32_t) * 2 * cfg->batch));
  std::vector<int32_t> host(2 * cfg->batch);
  for (int b = 0; b < cfg->batch; ++b) {
    host[b] = prefill[b];
    host[cfg->batch + b] = bud[b];
  }
  char err[256];
  if (lf::upload_and_wait(dlen, host.data(), sizeof(int32_t) * host.size(), stream, err, sizeof(err)))
    return fail(LF_ERR_HIP, "%s", err);
  lf::PrefillArgs a{};
  a.q_last = q_last;
  a.k_pre = k_pre;
  a.v_pre = v_pre;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kept = kept;
  a.work = reinterpret_cast<float*>(w);
  a.stats = stats;
  a.logits = logits;
  a.n_chunks = nck;
  a.n_copy = (cfg->max_budget + lf::kPrefillCopyRows - 1) / lf::kPrefillCopyRows;
  a.prefill = dlen;
  a.budget = dlen + cfg->batch;
  a.n_kv_heads = cfg->n_kv_heads;
  a.n_q_heads = cfg->n_q_heads;
  a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.max_prefill = max_prefill;
  a.max_budget = cfg->max_budget;
  a.sink = cfg->sink;
  a.recent = cfg->recent;
  const double scale = cfg->softmax_scale > 0 ? cfg->softmax_scale : 1.0 / std::sqrt((double)cfg->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  if (lf::launch_prefill(cfg->dtype, cfg->head_dim, a, (int)pairs, stream, err, sizeof(err)))
    return fail(LF_ERR_HIP, "%s", err);
  g_err[0] = 0;
  return LF_OK;
}

}  // namespace

extern "C" {

int32_t lf_abi_version(void) { return LF_ABI_VERSION; }

const char* lf_last_error(void) { return g_err; }

lf_status lf_state_bytes(const lf_config* cfg, const int32_t* budgets, size_t* bytes) {
  lf_status st = validate_config(cfg);
  if (st != LF_OK) return st;
  if (!bytes) return fail(LF_ERR_ARG, "bytes is NULL");
  std::vector<int32_t> bud;
  if ((st = validate_budgets(cfg, budgets, bud)) != LF_OK) return st;
  lf::StateLayout L{};
  if ((st = make_layout(cfg, bud, L, nullptr, nullptr)) != LF_OK) return st;
  *bytes = L.total;
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_init_cache(const lf_config* cfg, const int32_t* budgets, const int64_t* seq_len, void* k_cache,
                        void* v_cache, void* state, size_t state_bytes, int32_t flags, void* stream,
                        lf_cache** out) {
  lf_status st = validate_config(cfg);
  if (st != LF_OK) return st;
  if (!out) return fail(LF_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!seq_len || !k_cache || !v_cache || !state)
    return fail(LF_ERR_ARG, "seq_len, k_cache, v_cache and state must be non-NULL");
  if (flags & ~LF_INIT_ATTACH) return fail(LF_ERR_ARG, "unknown flags 0x%x", (unsigned)flags);
  if (reinterpret_cast<uintptr_t>(state) % lf::kAlign) return fail(LF_ERR_ARG, "state must be 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 || reinterpret_cast<uintptr_t>(v_cache) % 16)
    return fail(LF_ERR_ARG, "k_cache and v_cache must be 16-byte aligned");
  std::vector<int32_t> bud;
  if ((st = validate_budgets(cfg, budgets, bud)) != LF_OK) return st;
  for (int b = 0; b < cfg->batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > 0x7FFFFFFFll - 0x10000000ll)
      return fail(LF_ERR_ARG, "seq_len[%d] = %lld out of range", b, (long long)seq_len[b]);
  lf::StateLayout L{};
  std::vector<lf::WorkItem> items;
  std::vector<lf::PairMeta> meta;
  if ((st = make_layout(cfg, bud, L, &items, &meta)) != LF_OK) return st;
  if (state_bytes < L.total)
    return fail(LF_ERR_ARG, "state_bytes %zu < required %zu (see lf_state_bytes)", state_bytes, L.total);

  if (!(flags & LF_INIT_ATTACH)) {
    // Host image of header, meta, ring, work list and the zeroed exchange
    // cells (no stale epoch tag may survive), uploaded in one copy.
    std::vector<char> img(L.logits, 0);
    lf::StateHeader h{lf::kStateMagic, L.n_pairs, L.n_items, L.total_slots, 0, 0, {0, 0}};
    std::memcpy(img.data() + L.header, &h, sizeof(h));
    int32_t* ring = reinterpret_cast<int32_t*>(img.data() + L.ring);
    for (int b = 0; b < cfg->batch; ++b) start_sequence(*cfg, b, seq_len[b], bud[b], meta.data(), ring);
    std::memcpy(img.data() + L.meta, meta.data(), sizeof(lf::PairMeta) * meta.size());
    std::memcpy(img.data() + L.items, items.data(), sizeof(lf::WorkItem) * items.size());
    if (lf::upload_and_wait(state, img.data(), img.size(), stream, g_err, sizeof(g_err))) return LF_ERR_HIP;
  }

  lf_cache* c = new (std::nothrow) lf_cache;
  if (!c) return fail(LF_ERR_ARG, "out of host memory");
  c->magic = lf::kHandleMagic;
  c->cfg = *cfg;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  c->lay = L;
  c->u_budget = bud[0];
  for (int b = 1; b < cfg->batch; ++b)
    if (bud[b] != bud[0]) c->u_budget = 0;
  c->budgets = bud;
  c->k_cache = k_cache;
  c->v_cache = v_cache;
  c->state = static_cast<char*>(state);
  c->state_bytes = state_bytes;
  c->wait_ticks = kDefaultWaitTicks;
  const double scale = cfg->softmax_scale > 0 ? cfg->softmax_scale : 1.0 / std::sqrt((double)cfg->head_dim);
  c->scale_log2 = (float)(scale * 1.4426950408889634);
  *out = c;
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_decode_step(const void* q, const void* k_new, const void* v_new, lf_cache* cache, void* out,
                         int32_t* evict_idx, void* stream) {
  return step_impl(q, k_new, v_new, cache, out, evict_idx, nullptr, nullptr, stream);
}

lf_status lf_decode_step_dbg(const void* q, const void* k_new, const void* v_new, lf_cache* cache, void* out,
                             int32_t* evict_idx, float* scores, float* lse, void* stream) {
  return step_impl(q, k_new, v_new, cache, out, evict_idx, scores, lse, stream);
}

void lf_free(lf_cache* cache) {
  if (!cache || cache->magic != lf::kHandleMagic) return;
  cache->magic = 0;
  delete cache;
}

lf_status lf_set_split_wait(lf_cache* cache, int32_t max_wait_us) {
  lf_status st = check_handle(cache);
  if (st != LF_OK) return st;
  if (max_wait_us < 0 || max_wait_us > 1000000)
    return fail(LF_ERR_ARG, "max_wait_us %d outside [0, 1000000]", max_wait_us);
  cache->wait_ticks = (uint32_t)max_wait_us * 100u;  // s_memrealtime runs at 100 MHz
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_check_state(const lf_cache* cache, void* stream, lf_state_report* report) {
  lf_status st = check_handle(cache);
  if (st != LF_OK) return st;
  if (!report) return fail(LF_ERR_ARG, "report is NULL");
  const lf_config& cfg = cache->cfg;
  const lf::StateLayout& L = cache->lay;
  std::vector<char> img(L.items);
  if (lf::download_and_wait(img.data(), cache->state, L.items, stream, g_err, sizeof(g_err))) return LF_ERR_HIP;
  const lf::StateHeader* h = reinterpret_cast<const lf::StateHeader*>(img.data() + L.header);
  report->deferred = h->deferred;
  report->n_pairs = L.n_pairs;
  report->bad_pair = -1;
  report->reserved = 0;
  if (h->magic != lf::kStateMagic || h->n_pairs != L.n_pairs || h->n_items != L.n_items)
    return fail(LF_ERR_STATE, "state header does not match the handle (magic 0x%08x, %d pairs, %d items)", h->magic,
                h->n_pairs, h->n_items);
  if (h->fault)
    return fail(LF_ERR_STATE, "a step's wait for another workgroup's published words hit its safety bound "
                "(fault bits 0x%x: 1 statistics, 2 value sums, 4 candidates); results since are not valid", h->fault);
  lf::StateLayout L2{};
  std::vector<lf::PairMeta> want;
  if ((st = make_layout(&cfg, cache->budgets, L2, nullptr, &want)) != LF_OK) return st;
  const lf::PairMeta* meta = reinterpret_cast<const lf::PairMeta*>(img.data() + L.meta);
  const int32_t* ring = reinterpret_cast<const int32_t*>(img.data() + L.ring);
  const uint32_t* count = reinterpret_cast<const uint32_t*>(img.data() + L.count);
  const int R = cfg.recent;
  std::vector<char> seen;
  for (int p = 0; p < L.n_pairs; ++p) {
    const lf::PairMeta& m = meta[p];
    const lf::PairMeta& w = want[p];
    const char* why = nullptr;
    if (m.budget != w.budget || m.nchunk != w.nchunk || m.item0 != w.item0 || m.slot0 != w.slot0 ||
        m.lstride != w.lstride)
      why = "layout fields differ from the handle's";
    else if (m.t < 0 || m.len != (m.t < m.budget ? m.t : m.budget))
      why = "fill level is not min(position, budget)";
    else if (m.epoch == 0)
      why = "epoch is 0";
    else if (count[p] != 0)
      why = "chunk counter is not 0 between steps";
    if (!why && R > 0) {
      seen.assign(m.budget, 0);
      for (int64_t pos = m.t - R < 0 ? 0 : m.t - R; pos < m.t && !why; ++pos) {
        const int32_t sl = ring[(size_t)p * R + pos % R];
        if (sl < 0 || sl >= m.len)
          why = "a recent position's slot is outside the filled slots";
        else if (seen[sl]++)
          why = "two recent positions share a slot";
      }
    }
    if (why) {
      report->bad_pair = p;
      return fail(LF_ERR_STATE, "pair %d (sequence %d, KV head %d): %s", p, p / cfg.n_kv_heads, p % cfg.n_kv_heads,
                  why);
    }
  }
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_reset_sequences(lf_cache* cache, int32_t n, const int32_t* seqs, const int64_t* seq_len,
                             void* stream) {
  lf_status st = check_reset_args(cache, n, seqs, seq_len);
  if (st != LF_OK || n == 0) return st;
  const lf_config& cfg = cache->cfg;
  lf::StateLayout L{};
  std::vector<lf::PairMeta> meta;
  if ((st = make_layout(&cfg, cache->budgets, L, nullptr, &meta)) != LF_OK) return st;
  const int H = cfg.n_kv_heads, R = cfg.recent;
  std::vector<int32_t> ring((size_t)L.n_pairs * (R > 0 ? R : 1));
  for (int i = 0; i < n; ++i) {
    const int b = seqs[i];
    // The pairs' epochs tag their exchange cells: read the metadata back so
    // they carry on (a restarted epoch could match a stale tag).
    if (lf::download_and_wait(meta.data() + (size_t)b * H, cache->state + L.meta + sizeof(lf::PairMeta) * (size_t)b * H,
                              sizeof(lf::PairMeta) * H, stream, g_err, sizeof(g_err)))
      return LF_ERR_HIP;
    start_sequence(cfg, b, seq_len[i], cache->budgets[b], meta.data(), ring.data());
    // A sequence's pairs are contiguous in the metadata and in the ring.
    if (lf::upload_and_wait(cache->state + L.meta + sizeof(lf::PairMeta) * (size_t)b * H, meta.data() + (size_t)b * H,
                            sizeof(lf::PairMeta) * H, stream, g_err, sizeof(g_err)))
      return LF_ERR_HIP;
    if (R > 0 && lf::upload_and_wait(cache->state + L.ring + sizeof(int32_t) * (size_t)b * H * R,
                                     ring.data() + (size_t)b * H * R, sizeof(int32_t) * H * R, stream, g_err,
                                     sizeof(g_err)))
      return LF_ERR_HIP;
  }
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_reset_sequences_budget(lf_cache* cache, int32_t n, const int32_t* seqs, const int64_t* seq_len,
                                    const int32_t* budgets, void* stream) {
  lf_status st = check_reset_args(cache, n, seqs, seq_len);
  if (st != LF_OK || n == 0) return st;
  if (!budgets) return fail(LF_ERR_ARG, "budgets must be non-NULL");
  const lf_config& cfg = cache->cfg;
  std::vector<int32_t> nb = cache->budgets;
  for (int i = 0; i < n; ++i) nb[seqs[i]] = budgets[i];
  std::vector<int32_t> checked;
  if ((st = validate_budgets(&cfg, nb.data(), checked)) != LF_OK) return st;
  lf::StateLayout L{};
  std::vector<lf::WorkItem> items;
  std::vector<lf::PairMeta> meta;
  if ((st = make_layout(&cfg, nb, L, &items, &meta)) != LF_OK) return st;
  if (L.total > cache->state_bytes)
    return fail(LF_ERR_ARG, "the new budgets need %zu state bytes, the buffer holds %zu", L.total,
                cache->state_bytes);
  // Header, metadata and rings lie before the work list at offsets that depend
  // only on the numbers of pairs and ring entries, so the old and the new
  // layout place them alike.  Read them back (after the queued steps), keep
  // every other sequence's position, fill level and ring, restart the listed
  // ones, and write header, metadata, rings and the new work list back.
  const lf::StateLayout& old = cache->lay;
  // The new work list moves the exchange cells: they are zeroed (no stale
  // epoch tag may survive); the pairs' epochs and the chunk counters carry on.
  std::vector<char> img(L.logits, 0);
  if (lf::download_and_wait(img.data(), cache->state, old.items, stream, g_err, sizeof(g_err))) return LF_ERR_HIP;
  const lf::PairMeta* cur = reinterpret_cast<const lf::PairMeta*>(img.data() + L.meta);
  for (int p = 0; p < L.n_pairs; ++p) {
    meta[p].t = cur[p].t;
    meta[p].len = cur[p].len;
    meta[p].epoch = cur[p].epoch;
  }
  int32_t* ring = reinterpret_cast<int32_t*>(img.data() + L.ring);
  for (int i = 0; i < n; ++i) start_sequence(cfg, seqs[i], seq_len[i], nb[seqs[i]], meta.data(), ring);
  const lf::StateHeader* oldh = reinterpret_cast<const lf::StateHeader*>(img.data() + L.header);
  lf::StateHeader h{lf::kStateMagic, L.n_pairs, L.n_items, L.total_slots, oldh->deferred, oldh->fault, {0, 0}};
  std::memcpy(img.data() + L.header, &h, sizeof(h));
  std::memcpy(img.data() + L.meta, meta.data(), sizeof(lf::PairMeta) * meta.size());
  std::memcpy(img.data() + L.items, items.data(), sizeof(lf::WorkItem) * items.size());
  if (lf::upload_and_wait(cache->state, img.data(), img.size(), stream, g_err, sizeof(g_err))) return LF_ERR_HIP;
  cache->lay = L;
  cache->budgets = nb;
  cache->u_budget = nb[0];
  for (int b = 1; b < cfg.batch; ++b)
    if (nb[b] != nb[0]) cache->u_budget = 0;
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_prefill_work_bytes(const lf_config* cfg, int32_t max_prefill, size_t* bytes) {
  lf_status st = validate_config(cfg);
  if (st != LF_OK) return st;
  if (!bytes) return fail(LF_ERR_ARG, "bytes is NULL");
  if (max_prefill < 1 || max_prefill > lf::kMaxPrefill)
    return fail(LF_ERR_ARG, "max_prefill %d outside [1, %d]", max_prefill, lf::kMaxPrefill);
  const size_t pairs = (size_t)cfg->batch * cfg->n_kv_heads;
  const size_t nck = (max_prefill + lf::kPrefillChunk - 1) / lf::kPrefillChunk;
  const size_t group = cfg->n_q_heads / cfg->n_kv_heads;
  *bytes = align_up(sizeof(float) * pairs * (size_t)max_prefill) + align_up(sizeof(float) * pairs * nck * 16) +
           align_up(sizeof(int32_t) * 2 * cfg->batch) + align_up(sizeof(float) * pairs * (size_t)max_prefill * group);
  g_err[0] = 0;
  return LF_OK;
}

lf_status lf_prefill_compress(const lf_config* cfg, const int32_t* budgets, const int32_t* prefill,
                              int32_t max_prefill, const void* q_last, const void* k_pre, const void* v_pre,
                              void* k_cache, void* v_cache, int32_t* kept, void* work, size_t work_bytes,
                              void* stream) {
  size_t need = 0;
  lf_status st = lf_prefill_work_bytes(cfg, max_prefill, &need);
  if (st != LF_OK) return st;
  if (!work) return fail(LF_ERR_ARG, "work is NULL");
  return prefill_impl(cfg, budgets, prefill, max_prefill, q_last, k_pre, v_pre, k_cache, v_cache, kept, work,
                      work_bytes, need, stream);
}

lf_status lf_prefill_compress_noalloc(const lf_config* cfg, const int32_t* budgets, const int32_t* prefill,
                                      int32_t max_prefill, const void* q_last, const void* k_pre,
                                      const void* v_pre, void* k_cache, void* v_cache, int32_t* kept,
                                      void* stream) {
  size_t need = 0;
  lf_status st = lf_prefill_work_bytes(cfg, max_prefill, &need);
  if (st != LF_OK) return st;
  if (need > lf::kPrefillScratchBytes)
    return fail(LF_ERR_ARG,
                "this batch needs %zu bytes of prefill scratch, the static scratch holds %zu: use "
                "lf_prefill_compress with a workspace",
                need, lf::kPrefillScratchBytes);
  void* work = nullptr;
  char err[256];
  if (lf::prefill_scratch(&work, err, sizeof(err))) return fail(LF_ERR_HIP, "%s", err);
  return prefill_impl(cfg, budgets, prefill, max_prefill, q_last, k_pre, v_pre, k_cache, v_cache, kept, work,
                      lf::kPrefillScratchBytes, need, stream);
}

}  // extern "C"
