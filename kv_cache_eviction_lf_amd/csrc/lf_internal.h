// Internal layout shared by the host runtime (lf_host.cpp) and the kernels
// (lf_kernel.hip).  Plain C++: no HIP types, so the host part also builds with g++.
#pragma once

#include <cstddef>
#include <cstdint>

namespace lf {

constexpr uint32_t kStateMagic = 0x4C46535Au;  // "LFSZ"
constexpr uint64_t kHandleMagic = 0x4C46434143484531ull;
constexpr int kMaxBudget = 65536;  // LDS bitmap of protected slots: kMaxBudget bits
constexpr int kMaxChunks = 64;     // chunks per (sequence, KV head): one tail lane each
constexpr int kMaxGroup = 8;
constexpr int kThreads = 256;      // threads per workgroup (4 wave64)
constexpr size_t kAlign = 256;
constexpr int kSlotPad = 64;        // per-pair workspace rows are padded to this many slots
constexpr int kTargetItems = 256;   // split pairs into chunks until about this many work items
constexpr int kMaxPrefill = 65536;  // prefill compression: positions fit 16 bits of the selection key
constexpr int kPrefillChunk = 512;  // rows per workgroup of the prefill score passes
constexpr int kPrefillCopyRows = 256;  // kept rows per workgroup of the prefill copy
constexpr int kPrefillArgBatch = 128;  // prefill compression: largest batch whose lengths travel as kernel arguments
// Static device scratch of lf_prefill_compress_noalloc (one copy per GPU).
constexpr size_t kPrefillScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

// Per (sequence, KV head) pair.  Written by lf_init_cache, updated in place by
// the workgroup that finishes the pair at the end of every step.
struct PairMeta {
  int32_t t;        // position of the next incoming token
  int32_t len;      // filled slots, == budget once the cache is full
  int32_t budget;   // slot budget of this sequence
  int32_t nchunk;   // split-KV chunks of this pair
  int32_t item0;    // index of the pair's first work item
  int32_t slot0;    // first slot of the pair in the logit workspace
  uint32_t epoch;   // step counter of a split pair (1 at init, never 0): tags its exchange cells
  int32_t lstride;  // row stride of the pair's logit workspace: budget rounded up to 64
};
static_assert(sizeof(PairMeta) == 32, "PairMeta layout");

// One split-KV work item: rows [start, start + count) of pair `pair`.
struct WorkItem {
  int32_t pair;
  int32_t start;
  int32_t count;
  int32_t chunk;  // index of the chunk within its pair
};
static_assert(sizeof(WorkItem) == 16, "WorkItem layout");

struct StateHeader {
  uint32_t magic;
  int32_t n_pairs;
  int32_t n_items;
  int32_t total_slots;
  uint32_t deferred;  // split chunks that handed their logits over through memory (counted by the kernel)
  uint32_t fault;     // kFault* bits: a wait for another workgroup's words hit its safety bound
  uint32_t pad[2];
};
// Every wait of one workgroup for words another has already issued ends
// within this many s_memrealtime ticks (100 MHz: 0.2 s) even if the protocol
// were broken; the kernel then records a fault bit instead of hanging.
constexpr uint64_t kSafetyTicks = 20000000;
constexpr uint32_t kFaultStats = 1, kFaultValues = 2, kFaultCandidates = 4;

// Byte offsets of the regions of the caller's state buffer.  Everything before
// `items` depends only on the numbers of pairs and ring entries.
struct StateLayout {
  size_t header, meta, ring, count, items, xcell, xcand, xstat, logits, total;
  int32_t n_pairs, n_items, total_slots, chunk, max_nchunk;
};

// Arguments of one fused decode-step launch (passed by value to the kernel).
struct StepArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* out;
  int32_t* evict_idx;
  float* dbg_scores;  // may be null
  float* dbg_lse;     // may be null
  PairMeta* meta;
  int32_t* ring;
  const WorkItem* items;
  // Exchange between the chunks of a split pair, every value a 64-bit word
  // whose high half is the pair's epoch of the step that wrote it:
  uint64_t* xcell;   // [n_items][G][d]: the chunk's weighted value sums
  uint64_t* xcand;   // [n_items][2]: the chunk's (score) and (slot | deferred << 31) candidate
  uint64_t* xstat;   // [n_items][kThreads / 64][G][2]: (max, sum) of every wave of the chunk, per head
  uint32_t* count;   // [n_pairs]: chunks of the pair done with the step (reset by the finisher)
  uint32_t* deferred;  // header counter of deferred chunks
  uint32_t* fault;     // header fault bits (kFault*)
  float* logits;    // per pair [G][lstride], logits of a deferred chunk's rows (VL1: plus log2 |v|_1)
  uint32_t wait_ticks;  // how long (s_memrealtime ticks, 100 MHz) a chunk waits for its pair's statistics; 0: never
  int32_t n_items;
  int32_t n_pairs;  // batch * n_kv_heads
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t max_budget;
  int32_t sink;
  int32_t recent;
  float scale_log2;  // softmax scale * log2(e)
  int32_t vl1;
  int32_t score_none;  // attention only: no logits, importance or eviction
  // Equal budgets: item i is chunk i % u_nchunk of pair i / u_nchunk, rows
  // [c * u_chunk, min((c + 1) * u_chunk, u_budget)); the kernel computes it
  // instead of loading items[i].  u_budget = 0 otherwise.
  int32_t u_budget;
  int32_t u_chunk;
  int32_t u_nchunk;
};

// Tile height (rows per workgroup per pass) of the kernel for a shape; chunk
// lengths are multiples of it.  Defined next to the kernels.
int tile_rows(int dtype, int head_dim, int group);

// Arguments of the one-shot prefill compression (lf_prefill.hip).  Pair p =
// b * n_kv_heads + g; the caller's scratch holds [pairs][max_prefill]
// importances, the per-chunk statistics, the device copies of the prefill
// lengths and budgets, then [pairs][group][max_prefill] logits.
struct PrefillArgs {
  const void* q_last;  // [B][Hq][d]
  const void* k_pre;   // [B][Hkv][max_prefill][d]
  const void* v_pre;
  void* k_cache;       // [B][Hkv][max_budget][d]
  void* v_cache;
  int32_t* kept;       // [B][Hkv][max_budget]: kept positions, increasing
  float* work;         // [pairs][max_prefill]
  float* stats;        // [pairs][n_chunks][8][2]: per-chunk (max, sum) per head
  float* logits;       // [pairs][group][max_prefill]: log2-domain logits of the last query
  const int32_t* prefill;  // device [B] (batches above kPrefillArgBatch)
  const int32_t* budget;   // device [B]
  const int32_t* order;    // device [B]: sequences by decreasing prefill length
  int32_t n_chunks;    // score chunks per pair (max_prefill / 512, rounded up)
  int32_t n_copy;      // copy workgroups per pair (max_budget / 256, rounded up)
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group;
  int32_t max_prefill;
  int32_t max_budget;
  int32_t sink;
  int32_t recent;
  float scale_log2;
  // Batches of up to kPrefillArgBatch sequences carry their prefill lengths,
  // budgets and order in the kernel arguments (no upload, no wait: the call is
  // then fully asynchronous); larger batches use the device arrays above.
  int32_t n_inline;  // B when the lengths are inline, else 0
  int32_t lens[3 * kPrefillArgBatch];
};

// Kernel launch and runtime helpers, implemented in lf_kernel.hip (step) and
// lf_prefill.hip (prefill compression).
int launch_step(int dtype, int head_dim, int group, const StepArgs& a, void* stream, char* err, size_t errlen);
int launch_prefill(int dtype, int head_dim, const PrefillArgs& a, int n_pairs, void* stream, char* err,
                   size_t errlen);
// Device address of the static prefill scratch on the current device (looked
// up once per device); 0 on success.
int prefill_scratch(void** ptr, char* err, size_t errlen);
int upload_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen);
int download_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen);
// `rows` rows of `width` bytes, row r from src + r * spitch to dst + r * dpitch
// (host to device when to_device, else device to host), ordered on `stream`;
// returns once the copy completed.  0 on success.
int copy_rows_and_wait(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t rows,
                       bool to_device, void* stream, char* err, size_t errlen);

}  // namespace lf
