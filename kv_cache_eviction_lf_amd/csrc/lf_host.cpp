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
  int32_t n_layers;
  lf::StateLayout lay;            // the layout of every layer's state
  std::vector<void*> k_cache;     // per layer
  std::vector<void*> v_cache;
  char* state;                    // layer l's state at state + l * layer_stride
  size_t state_bytes;             // capacity of the caller's state buffer
  size_t layer_stride;            // state_bytes / n_layers, rounded down to the state alignment
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

// Metadata and ring of one sequence's pairs for a cache holding `t` tokens
// laid out as lf_init_cache describes: meta_b and ring_b point at the
// sequence's first pair (the other PairMeta fields already set by the layout).
void start_sequence(const lf_config& cfg, int64_t t, int32_t budget, lf::PairMeta* meta_b, int32_t* ring_b) {
  const int R = cfg.recent;
  const int64_t len = t < budget ? t : budget;
  for (int g = 0; g < cfg.n_kv_heads; ++g) {
    meta_b[g].t = (int32_t)t;
    meta_b[g].len = (int32_t)len;
    int32_t* ring = ring_b + (size_t)g * R;
    for (int j = 0; j < R; ++j) ring[j] = -1;
    // The R newest cached positions [t - R, t): slot = position while the
    // prefill fits, else they are the last R slots (layout contract).
    for (int64_t pos = t - R < 0 ? 0 : t - R; pos < t; ++pos) {
      const int64_t slot = t <= budget ? pos : budget - (t - pos);
      ring[pos % R] = (int32_t)slot;
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
  off = align_up(off + sizeof(uint64_t) * (size_t)group * cfg->head_dim * W);
  L.xcand = off;
  off = align_up(off + sizeof(uint64_t) * 2 * W);
  L.xstat = off;
  off = align_up(off + sizeof(uint64_t) * 2 * (lf::kThreads / 64) * (size_t)group * W);
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

lf_status step_impl(const void* q, const void* k_new, const void* v_new, lf_cache* cache, int32_t layer,
                    void* out, int32_t* evict_idx, float* scores, float* lse, void* stream) {
  lf_status st = check_handle(cache);
  if (st != LF_OK) return st;
  if (layer < 0 || layer >= cache->n_layers)
    return fail(LF_ERR_ARG, "layer %d outside [0, %d)", layer, cache->n_layers);
  if (!q || !k_new || !v_new || !out || !evict_idx)
    return fail(LF_ERR_ARG, "q, k_new, v_new, out and evict_idx must be non-NULL");
  const lf_config& cfg = cache->cfg;
  lf::StepArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = cache->k_cache[layer];
  a.v_cache = cache->v_cache[layer];
  a.out = out;
  a.evict_idx = evict_idx;
  a.dbg_scores = scores;
  a.dbg_lse = lse;
  char* s = cache->state + (size_t)layer * cache->layer_stride;
  const lf::StateLayout& L = cache->lay;
  a.meta = reinterpret_cast<lf::PairMeta*>(s + L.meta);
  a.ring = reinterpret_cast<int32_t*>(s + L.ring);
  a.items = reinterpret_cast<const lf::WorkItem*>(s + L.items);
  a.xcell = reinterpret_cast<uint64_t*>(s + L.xcell);
  a.xcand = reinterpret_cast<uint64_t*>(s + L.xcand);
  a.xstat = reinterpret_cast<uint64_t*>(s + L.xstat);
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
  float* logits = reinterpret_cast<float*>(reinterpret_cast<char*>(dlen) + align_up(sizeof(int32_t) * 3 * cfg->batch));
  // prefill lengths, budgets, and the sequences by decreasing prefill length
  // (the selection pass starts its longest pairs first)
  std::vector<int32_t> host(3 * cfg->batch);
  for (int b = 0; b < cfg->batch; ++b) {
    host[b] = prefill[b];
    host[cfg->batch + b] = bud[b];
    host[2 * cfg->batch + b] = b;
  }
  std::stable_sort(host.begin() + 2 * cfg->batch, host.end(),
                   [&](int32_t x, int32_t y) { return prefill[x] > prefill[y]; });
  char err[256];
  lf::PrefillArgs a{};
  if (cfg->batch <= lf::kPrefillArgBatch) {
    a.n_inline = cfg->batch;
    std::copy(host.begin(), host.end(), a.lens);
  } else if (lf::upload_and_wait(dlen, host.data(), sizeof(int32_t) * host.size(), stream, err, sizeof(err))) {
    return fail(LF_ERR_HIP, "%s", err);
  }
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
  a.order = dlen + 2 * cfg->batch;
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

constexpr int32_t kMaxLayers = 4096;

// lf_init_cache over n_layers layer caches sharing the configuration and the
// budgets: every layer's state has the same layout, layer l's at
// state + l * stride with stride = state_bytes / n_layers rounded down to
// the state alignment (so a later budget change never moves a layer).
lf_status init_impl(const lf_config* cfg, int32_t n_layers, const int32_t* budgets, const int64_t* seq_len,
                    void* const* k_caches, void* const* v_caches, void* state, size_t state_bytes, int32_t flags,
                    void* stream, lf_cache** out) {
  lf_status st = validate_config(cfg);
  if (st != LF_OK) return st;
  if (!out) return fail(LF_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(LF_ERR_ARG, "n_layers %d outside [1, %d]", n_layers, kMaxLayers);
  if (!seq_len || !state) return fail(LF_ERR_ARG, "seq_len and state must be non-NULL");
  for (int l = 0; l < n_layers; ++l) {
    if (!k_caches[l] || !v_caches[l])
      return fail(LF_ERR_ARG, n_layers == 1 ? "k_cache and v_cache must be non-NULL"
                                            : "k_caches[%d] and v_caches[%d] must be non-NULL", l, l);
    if (reinterpret_cast<uintptr_t>(k_caches[l]) % 16 || reinterpret_cast<uintptr_t>(v_caches[l]) % 16)
      return fail(LF_ERR_ARG, "k_cache and v_cache must be 16-byte aligned (layer %d)", l);
  }
  if (flags & ~LF_INIT_ATTACH) return fail(LF_ERR_ARG, "unknown flags 0x%x", (unsigned)flags);
  if (reinterpret_cast<uintptr_t>(state) % lf::kAlign) return fail(LF_ERR_ARG, "state must be 256-byte aligned");
  std::vector<int32_t> bud;
  if ((st = validate_budgets(cfg, budgets, bud)) != LF_OK) return st;
  for (int b = 0; b < cfg->batch; ++b)
    if (seq_len[b] < 0 || seq_len[b] > 0x7FFFFFFFll - 0x10000000ll)
      return fail(LF_ERR_ARG, "seq_len[%d] = %lld out of range", b, (long long)seq_len[b]);
  lf::StateLayout L{};
  std::vector<lf::WorkItem> items;
  std::vector<lf::PairMeta> meta;
  if ((st = make_layout(cfg, bud, L, &items, &meta)) != LF_OK) return st;
  const size_t stride = state_bytes / (size_t)n_layers / lf::kAlign * lf::kAlign;
  if (stride < L.total)
    return fail(LF_ERR_ARG, "state_bytes %zu < %d layer(s) x %zu (see lf_state_bytes / lf_state_bytes_layers)",
                state_bytes, n_layers, L.total);

  if (!(flags & LF_INIT_ATTACH)) {
    // Host image of header, meta, ring, work list and the zeroed exchange
    // cells (no stale epoch tag may survive), the same for every layer.
    std::vector<char> img(L.logits, 0);
    lf::StateHeader h{lf::kStateMagic, L.n_pairs, L.n_items, L.total_slots, 0, 0, {0, 0}};
    std::memcpy(img.data() + L.header, &h, sizeof(h));
    int32_t* ring = reinterpret_cast<int32_t*>(img.data() + L.ring);
    const int H = cfg->n_kv_heads;
    for (int b = 0; b < cfg->batch; ++b)
      start_sequence(*cfg, seq_len[b], bud[b], meta.data() + (size_t)b * H, ring + (size_t)b * H * cfg->recent);
    std::memcpy(img.data() + L.meta, meta.data(), sizeof(lf::PairMeta) * meta.size());
    std::memcpy(img.data() + L.items, items.data(), sizeof(lf::WorkItem) * items.size());
    for (int l = 0; l < n_layers; ++l)
      if (lf::upload_and_wait(static_cast<char*>(state) + (size_t)l * stride, img.data(), img.size(), stream, g_err,
                              sizeof(g_err)))
        return LF_ERR_HIP;
  }

  lf_cache* c = new (std::nothrow) lf_cache;
  if (!c) return fail(LF_ERR_ARG, "out of host memory");
  c->magic = lf::kHandleMagic;
  c->cfg = *cfg;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  c->n_layers = n_layers;
  c->lay = L;
  c->u_budget = bud[0];
  for (int b = 1; b < cfg->batch; ++b)
    if (bud[b] != bud[0]) c->u_budget = 0;
  c->budgets = bud;
  c->k_cache.assign(k_caches, k_caches + n_layers);
  c->v_cache.assign(v_caches, v_caches + n_layers);
  c->state = static_cast<char*>(state);
  c->state_bytes = state_bytes;
  c->layer_stride = stride;
  c->wait_ticks = kDefaultWaitTicks;
  const double scale = cfg->softmax_scale > 0 ? cfg->softmax_scale : 1.0 / std::sqrt((double)cfg->head_dim);
  c->scale_log2 = (float)(scale * 1.4426950408889634);
  *out = c;
  g_err[0] = 0;
  return LF_OK;
}

// lf_decode_step(_dbg) take single-layer handles only.
lf_status check_single_layer(const lf_cache* c) {
  lf_status st = check_handle(c);
  if (st != LF_OK) return st;
  if (c->n_layers != 1)
    return fail(LF_ERR_ARG, "the handle spans %d layers: use lf_decode_step_layer", c->n_layers);
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

lf_status lf_state_bytes_layers(const lf_config* cfg, const int32_t* budgets, int32_t n_layers, size_t* bytes) {
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(LF_ERR_ARG, "n_layers %d outside [1, %d]", n_layers, kMaxLayers);
  size_t one = 0;
  lf_status st = lf_state_bytes(cfg, budgets, &one);
  if (st != LF_OK) return st;
  *bytes = one * (size_t)n_layers;  // each layer's state is a multiple of the alignment
  return LF_OK;
}

lf_status lf_init_cache(const lf_config* cfg, const int32_t* budgets, const int64_t* seq_len, void* k_cache,
                        void* v_cache, void* state, size_t state_bytes, int32_t flags, void* stream,
                        lf_cache** out) {
  return init_impl(cfg, 1, budgets, seq_len, &k_cache, &v_cache, state, state_bytes, flags, stream, out);
}

lf_status lf_init_layers(const lf_config* cfg, int32_t n_layers, const int32_t* budgets, const int64_t* seq_len,
                         void* const* k_caches, void* const* v_caches, void* state, size_t state_bytes,
                         int32_t flags, void* stream, lf_cache** out) {
  if (out) *out = nullptr;
  if (!k_caches || !v_caches) return fail(LF_ERR_ARG, "k_caches and v_caches must be non-NULL");
  return init_impl(cfg, n_layers, budgets, seq_len, k_caches, v_caches, state, state_bytes, flags, stream, out);
}

lf_status lf_decode_step(const void* q, const void* k_new, const void* v_new, lf_cache* cache, void* out,
                         int32_t* evict_idx, void* stream) {
  lf_status st = check_single_layer(cache);
  if (st != LF_OK) return st;
  return step_impl(q, k_new, v_new, cache, 0, out, evict_idx, nullptr, nullptr, stream);
}

lf_status lf_decode_step_dbg(const void* q, const void* k_new, const void* v_new, lf_cache* cache, void* out,
                             int32_t* evict_idx, float* scores, float* lse, void* stream) {
  lf_status st = check_single_layer(cache);
  if (st != LF_OK) return st;
  return step_impl(q, k_new, v_new, cache, 0, out, evict_idx, scores, lse, stream);
}

lf_status lf_decode_step_layer(const void* q, const void* k_new, const void* v_new, lf_cache* cache, int32_t layer,
                               void* out, int32_t* evict_idx, void* stream) {
  return step_impl(q, k_new, v_new, cache, layer, out, evict_idx, nullptr, nullptr, stream);
}

lf_status lf_decode_step_layer_dbg(const void* q, const void* k_new, const void* v_new, lf_cache* cache,
                                   int32_t layer, void* out, int32_t* evict_idx, float* scores, float* lse,
                                   void* stream) {
  return step_impl(q, k_new, v_new, cache, layer, out, evict_idx, scores, lse, stream);
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
  const int NL = cache->n_layers;
  // Everything before the work list, of every layer.
  std::vector<char> all((size_t)NL * L.items);
  if (lf::copy_rows_and_wait(all.data(), L.items, cache->state, cache->layer_stride, L.items, NL, false, stream, g_err,
                             sizeof(g_err)))
    return LF_ERR_HIP;
  report->deferred = 0;
  report->n_pairs = L.n_pairs;
  report->bad_pair = -1;
  report->bad_layer = -1;
  for (int l = 0; l < NL; ++l)
    report->deferred += reinterpret_cast<const lf::StateHeader*>(all.data() + (size_t)l * L.items + L.header)->deferred;
  lf::StateLayout L2{};
  std::vector<lf::PairMeta> want;
  if ((st = make_layout(&cfg, cache->budgets, L2, nullptr, &want)) != LF_OK) return st;
  const int R = cfg.recent;
  std::vector<char> seen;
  for (int l = 0; l < NL; ++l) {
    const char* img = all.data() + (size_t)l * L.items;
    const lf::StateHeader* h = reinterpret_cast<const lf::StateHeader*>(img + L.header);
    if (h->magic != lf::kStateMagic || h->n_pairs != L.n_pairs || h->n_items != L.n_items) {
      report->bad_layer = l;
      return fail(LF_ERR_STATE, "layer %d: state header does not match the handle (magic 0x%08x, %d pairs, %d items)",
                  l, h->magic, h->n_pairs, h->n_items);
    }
    if (h->fault) {
      report->bad_layer = l;
      return fail(LF_ERR_STATE, "layer %d: a step's wait for another workgroup's published words hit its safety "
                  "bound (fault bits 0x%x: 1 statistics, 2 value sums, 4 candidates); results since are not valid",
                  l, h->fault);
    }
    const lf::PairMeta* meta = reinterpret_cast<const lf::PairMeta*>(img + L.meta);
    const int32_t* ring = reinterpret_cast<const int32_t*>(img + L.ring);
    const uint32_t* count = reinterpret_cast<const uint32_t*>(img + L.count);
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
        report->bad_layer = l;
        return fail(LF_ERR_STATE, "layer %d, pair %d (sequence %d, KV head %d): %s", l, p, p / cfg.n_kv_heads,
                    p % cfg.n_kv_heads, why);
      }
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
  const lf::StateLayout& L = cache->lay;
  const int H = cfg.n_kv_heads, R = cfg.recent, NL = cache->n_layers;
  const size_t stride = cache->layer_stride, mrow = sizeof(lf::PairMeta) * H, rrow = sizeof(int32_t) * H * R;
  std::vector<lf::PairMeta> meta((size_t)NL * H);  // [layer][KV head] of one sequence
  std::vector<int32_t> ring((size_t)NL * H * (R > 0 ? R : 1));
  for (int i = 0; i < n; ++i) {
    const int b = seqs[i];
    // The pairs' epochs tag their exchange cells: read the metadata back (every
    // layer's rows of this sequence, one strided copy) so they carry on (a
    // restarted epoch could match a stale tag).  A sequence's pairs are
    // contiguous in the metadata and in the ring.
    char* m0 = cache->state + L.meta + mrow * b;
    char* r0 = cache->state + L.ring + rrow * b;
    if (lf::copy_rows_and_wait(meta.data(), mrow, m0, stride, mrow, NL, false, stream, g_err, sizeof(g_err)))
      return LF_ERR_HIP;
    for (int l = 0; l < NL; ++l)
      start_sequence(cfg, seq_len[i], cache->budgets[b], meta.data() + (size_t)l * H, ring.data() + (size_t)l * H * R);
    if (lf::copy_rows_and_wait(m0, stride, meta.data(), mrow, mrow, NL, true, stream, g_err, sizeof(g_err)))
      return LF_ERR_HIP;
    if (R > 0 && lf::copy_rows_and_wait(r0, stride, ring.data(), rrow, rrow, NL, true, stream, g_err, sizeof(g_err)))
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
  if (L.total > cache->layer_stride)
    return fail(LF_ERR_ARG, "the new budgets need %zu state bytes per layer, the buffer holds %zu per layer", L.total,
                cache->layer_stride);
  // Header, metadata and rings lie before the work list at offsets that depend
  // only on the numbers of pairs and ring entries, so the old and the new
  // layout place them alike.  Read them back for every layer (after the queued
  // steps), keep every other sequence's position, fill level and ring, restart
  // the listed ones, and write header, metadata, rings, chunk counters and the
  // new work list back.
  const lf::StateLayout& old = cache->lay;
  const int NL = cache->n_layers;
  const size_t stride = cache->layer_stride;
  // The new work list moves the exchange cells.  Instead of clearing them, the
  // pairs of a layer continue from one epoch past the largest of the layer:
  // every word in the cells was written under an epoch below that, so none
  // can look fresh.  Only at the end of the epoch range are the cells zeroed.
  std::vector<char> img((size_t)NL * L.xcell, 0);
  if (lf::copy_rows_and_wait(img.data(), L.xcell, cache->state, stride, old.items, NL, false, stream, g_err,
                             sizeof(g_err)))
    return LF_ERR_HIP;
  bool wrap = false;
  for (int l = 0; l < NL && !wrap; ++l) {
    const lf::PairMeta* cur = reinterpret_cast<const lf::PairMeta*>(img.data() + (size_t)l * L.xcell + L.meta);
    for (int p = 0; p < L.n_pairs; ++p) wrap = wrap || cur[p].epoch == 0xFFFFFFFFu;
  }
  for (int l = 0; l < NL; ++l) {
    char* li = img.data() + (size_t)l * L.xcell;
    const lf::PairMeta* cur = reinterpret_cast<const lf::PairMeta*>(li + L.meta);
    uint32_t top = 0;
    for (int p = 0; p < L.n_pairs; ++p) top = cur[p].epoch > top ? cur[p].epoch : top;
    std::vector<lf::PairMeta> lm = meta;
    for (int p = 0; p < L.n_pairs; ++p) {
      lm[p].t = cur[p].t;
      lm[p].len = cur[p].len;
      lm[p].epoch = wrap ? 1u : top + 1u;
    }
    int32_t* ring = reinterpret_cast<int32_t*>(li + L.ring);
    const int H = cfg.n_kv_heads, R = cfg.recent;
    for (int i = 0; i < n; ++i)
      start_sequence(cfg, seq_len[i], nb[seqs[i]], lm.data() + (size_t)seqs[i] * H, ring + (size_t)seqs[i] * H * R);
    const lf::StateHeader* oldh = reinterpret_cast<const lf::StateHeader*>(li + L.header);
    lf::StateHeader h{lf::kStateMagic, L.n_pairs, L.n_items, L.total_slots, oldh->deferred, oldh->fault, {0, 0}};
    std::memcpy(li + L.header, &h, sizeof(h));
    std::memcpy(li + L.meta, lm.data(), sizeof(lf::PairMeta) * lm.size());
    std::memset(li + L.count, 0, sizeof(uint32_t) * L.n_pairs);
    std::memcpy(li + L.items, items.data(), sizeof(lf::WorkItem) * items.size());
  }
  if (lf::copy_rows_and_wait(cache->state, stride, img.data(), L.xcell, L.xcell, NL, true, stream, g_err,
                             sizeof(g_err)))
    return LF_ERR_HIP;
  if (wrap) {
    // Zeroed exchange cells for the restarted epochs.
    std::vector<char> zero((size_t)NL * (L.logits - L.xcell), 0);
    if (lf::copy_rows_and_wait(cache->state + L.xcell, stride, zero.data(), L.logits - L.xcell, L.logits - L.xcell, NL,
                               true, stream, g_err, sizeof(g_err)))
      return LF_ERR_HIP;
  }
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
           align_up(sizeof(int32_t) * 3 * cfg->batch) + align_up(sizeof(float) * pairs * (size_t)max_prefill * group);
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
