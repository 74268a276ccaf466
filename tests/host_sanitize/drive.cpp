// Drives the C ABI's host runtime (lf_host.cpp) against the host stand-ins of
// stub_device.cpp, under AddressSanitizer / UndefinedBehaviorSanitizer:
// validation, the state layout and work list, the start-up of the recent-slot
// ring, one and several layers, the resets with and without new budgets, the
// state checks and the prefill entry points.  The "device" buffers are host
// memory, so the state the runtime writes is read back directly.  Prints one
// line per failed check; the exit status is the number of failures.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/lf.h"
#include "../../kv_cache_eviction_lf_amd/csrc/lf_internal.h"
#include "stub_device.h"

static int g_fail = 0;
#define CHECK(c)                                                                        \
  do {                                                                                  \
    if (!(c)) {                                                                         \
      std::printf("FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #c, lf_last_error()); \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

namespace {

struct Buf {  // 256-byte aligned host buffer standing in for device memory
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
    std::memset(p, 0, n);
  }
  ~Buf() { std::free(p); }
  char* c() const { return static_cast<char*>(p); }
};

lf_config config(int batch, int hq, int hkv, int d, int max_budget, int sink, int recent, int dtype = LF_BF16) {
  lf_config c{};
  c.batch = batch;
  c.n_q_heads = hq;
  c.n_kv_heads = hkv;
  c.head_dim = d;
  c.max_budget = max_budget;
  c.sink = sink;
  c.recent = recent;
  c.dtype = dtype;
  c.score = LF_SCORE_ATTN;
  return c;
}

// Mirror of the state layout's leading regions (they depend only on the numbers
// of pairs and ring entries): header, meta, ring, count, then the work list.
struct View {
  const lf::StateHeader* h;
  lf::PairMeta* meta;
  int32_t* ring;
  uint32_t* count;
  const lf::WorkItem* items;
};
size_t up(size_t x) { return (x + 255) / 256 * 256; }
View view(char* s, int pairs, int recent) {
  View v;
  size_t off = 0;
  v.h = reinterpret_cast<const lf::StateHeader*>(s);
  off = up(sizeof(lf::StateHeader));
  v.meta = reinterpret_cast<lf::PairMeta*>(s + off);
  off = up(off + sizeof(lf::PairMeta) * pairs);
  v.ring = reinterpret_cast<int32_t*>(s + off);
  off = up(off + sizeof(int32_t) * pairs * recent);
  v.count = reinterpret_cast<uint32_t*>(s + off);
  off = up(off + sizeof(uint32_t) * pairs);
  v.items = reinterpret_cast<const lf::WorkItem*>(s + off);
  return v;
}

// The layout contract of a sequence restarted with t tokens seen and budget
// `budget`: fill level, position, and the ring of the R newest positions.
void check_started(const View& v, int p, int64_t t, int budget, int R) {
  const int64_t len = t < budget ? t : budget;
  CHECK(v.meta[p].t == t);
  CHECK(v.meta[p].len == len);
  CHECK(v.meta[p].budget == budget);
  for (int64_t pos = 0; pos < R; ++pos) {
    const int32_t sl = v.ring[(size_t)p * R + pos];
    // entry pos % R of position pos' in [t - R, t): pos' = t - R + ((pos - t) mod R)
    const int64_t pp = t - R + (((pos - t) % R) + R) % R;
    if (pp < 0) {
      CHECK(sl == -1);
    } else {
      const int64_t want = t <= budget ? pp : budget - (t - pp);
      CHECK(sl == want);
    }
  }
}

// Work items of every pair: its nchunk chunks, contiguous from item0, covering
// [0, budget) in order.
void check_items(const View& v, int pairs) {
  for (int p = 0; p < pairs; ++p) {
    const lf::PairMeta& m = v.meta[p];
    int next = 0;
    for (int c = 0; c < m.nchunk; ++c) {
      const lf::WorkItem& it = v.items[m.item0 + c];
      CHECK(it.pair == p && it.chunk == c && it.start == next && it.count > 0);
      next = it.start + it.count;
    }
    CHECK(next == m.budget);
    CHECK(m.lstride >= m.budget && m.lstride % lf::kSlotPad == 0);
  }
}

void test_validation() {
  size_t n = 0;
  lf_config c = config(2, 8, 2, 128, 512, 4, 16);
  CHECK(lf_state_bytes(&c, nullptr, &n) == LF_OK && n > 0);
  lf_config bad = c;
  bad.batch = 0;
  CHECK(lf_state_bytes(&bad, nullptr, &n) == LF_ERR_ARG);
  bad = c;
  bad.n_q_heads = 18;  // group 9
  CHECK(lf_state_bytes(&bad, nullptr, &n) == LF_ERR_UNSUPPORTED);
  bad = c;
  bad.head_dim = 96;
  CHECK(lf_state_bytes(&bad, nullptr, &n) == LF_ERR_UNSUPPORTED);
  bad = c;
  bad.reserved = 1;
  CHECK(lf_state_bytes(&bad, nullptr, &n) == LF_ERR_ARG);
  const int32_t small[2] = {20, 512};  // <= sink + recent
  CHECK(lf_state_bytes(&c, small, &n) == LF_ERR_ARG);
  CHECK(lf_state_bytes(&c, nullptr, nullptr) == LF_ERR_ARG);
  CHECK(lf_state_bytes(nullptr, nullptr, &n) == LF_ERR_ARG);
  size_t n3 = 0;
  CHECK(lf_state_bytes_layers(&c, nullptr, 3, &n3) == LF_OK && n3 == 3 * n);
  CHECK(lf_state_bytes_layers(&c, nullptr, 0, &n3) == LF_ERR_ARG);
  CHECK(lf_state_bytes_layers(&c, nullptr, 5000, &n3) == LF_ERR_ARG);
}

void test_single_layer() {
  const int B = 3, H = 2, R = 16, S = 512;
  lf_config c = config(B, 8, H, 128, S, 4, R);
  const int32_t bud[B] = {300, 512, 200};
  const int64_t seq[B] = {10, 700, 200};  // short, longer than the budget, exactly full
  size_t n = 0;
  CHECK(lf_state_bytes(&c, bud, &n) == LF_OK);
  Buf st(n), k(64), v(64);
  lf_cache* h = nullptr;
  CHECK(lf_init_cache(&c, bud, seq, k.p, v.p, st.p, n - 1, 0, nullptr, &h) == LF_ERR_ARG && h == nullptr);
  CHECK(lf_init_cache(&c, bud, seq, k.p, v.p, st.c() + 16, n, 0, nullptr, &h) == LF_ERR_ARG);
  CHECK(lf_init_cache(&c, bud, seq, k.c() + 8, v.p, st.p, n, 0, nullptr, &h) == LF_ERR_ARG);
  CHECK(lf_init_cache(&c, bud, seq, k.p, v.p, st.p, n, 0, nullptr, &h) == LF_OK && h);
  View vw = view(st.c(), B * H, R);
  CHECK(vw.h->magic == lf::kStateMagic && vw.h->n_pairs == B * H);
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < H; ++g) {
      check_started(vw, b * H + g, seq[b], bud[b], R);
      CHECK(vw.meta[b * H + g].epoch == 1);
    }
  check_items(vw, B * H);
  // a step: the launch sees the caller's pointers and the state regions
  stub::steps.clear();
  int dummy[4];
  CHECK(lf_decode_step(dummy, dummy, dummy, h, dummy, dummy, nullptr) == LF_OK);
  CHECK(stub::steps.size() == 1 && stub::steps[0].k_cache == k.p && stub::steps[0].meta == vw.meta);
  CHECK(stub::steps[0].n_pairs == B * H && stub::steps[0].u_budget == 0 && stub::steps[0].wait_ticks == 10000);
  CHECK(lf_decode_step(nullptr, dummy, dummy, h, dummy, dummy, nullptr) == LF_ERR_ARG);
  CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, 1, dummy, dummy, nullptr) == LF_ERR_ARG);
  CHECK(lf_set_split_wait(h, 5) == LF_OK);
  CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, 0, dummy, dummy, nullptr) == LF_OK);
  CHECK(stub::steps.back().wait_ticks == 500);
  CHECK(lf_set_split_wait(h, -1) == LF_ERR_ARG && lf_set_split_wait(h, 2000000) == LF_ERR_ARG);
  // state checks: fine, then a broken fill level, a left-over counter, a fault bit
  lf_state_report rep{};
  CHECK(lf_check_state(h, nullptr, &rep) == LF_OK && rep.bad_pair == -1 && rep.bad_layer == -1);
  vw.meta[3].len += 1;
  CHECK(lf_check_state(h, nullptr, &rep) == LF_ERR_STATE && rep.bad_pair == 3 && rep.bad_layer == 0);
  vw.meta[3].len -= 1;
  vw.count[1] = 2;
  CHECK(lf_check_state(h, nullptr, &rep) == LF_ERR_STATE && rep.bad_pair == 1);
  vw.count[1] = 0;
  reinterpret_cast<lf::StateHeader*>(st.p)->fault = lf::kFaultCandidates;
  CHECK(lf_check_state(h, nullptr, &rep) == LF_ERR_STATE && std::strstr(lf_last_error(), "safety bound"));
  reinterpret_cast<lf::StateHeader*>(st.p)->fault = 0;
  // a failing copy is reported, not hidden
  stub::fail_copies = 1;
  CHECK(lf_check_state(h, nullptr, &rep) == LF_ERR_HIP);
  stub::fail_copies = 0;
  lf_free(h);
  lf_free(nullptr);
}

void test_layers_and_resets() {
  const int B = 4, H = 2, R = 8, S = 1024, NL = 3;
  lf_config c = config(B, 8, H, 128, S, 4, R);
  const int32_t bud[B] = {300, 300, 300, 300};
  const int64_t seq[B] = {300, 300, 300, 300};
  size_t one = 0, cap = 0;
  CHECK(lf_state_bytes(&c, bud, &one) == LF_OK);
  const int32_t later[B] = {300, 900, 300, 300};  // room for one larger budget later
  CHECK(lf_state_bytes(&c, later, &cap) == LF_OK && cap > one);
  Buf st(cap * NL);
  std::vector<Buf*> kb, vb;
  void* ks[NL];
  void* vs[NL];
  for (int l = 0; l < NL; ++l) {
    kb.push_back(new Buf(256));
    vb.push_back(new Buf(256));
    ks[l] = kb.back()->p;
    vs[l] = vb.back()->p;
  }
  lf_cache* h = nullptr;
  CHECK(lf_init_layers(&c, NL, bud, seq, ks, vs, st.p, one * NL - 256, 0, nullptr, &h) == LF_ERR_ARG);
  CHECK(lf_init_layers(&c, NL, bud, seq, nullptr, vs, st.p, cap * NL, 0, nullptr, &h) == LF_ERR_ARG);
  void* bad_k[NL] = {ks[0], nullptr, ks[2]};
  CHECK(lf_init_layers(&c, NL, bud, seq, bad_k, vs, st.p, cap * NL, 0, nullptr, &h) == LF_ERR_ARG);
  CHECK(lf_init_layers(&c, 0, bud, seq, ks, vs, st.p, cap * NL, 0, nullptr, &h) == LF_ERR_ARG);
  CHECK(lf_init_layers(&c, NL, bud, seq, ks, vs, st.p, cap * NL, 0, nullptr, &h) == LF_OK && h);
  const size_t stride = cap;  // state_bytes / NL, a multiple of 256
  std::vector<View> vw;
  for (int l = 0; l < NL; ++l) vw.push_back(view(st.c() + l * stride, B * H, R));
  // every layer gets the same image
  for (int l = 1; l < NL; ++l) CHECK(std::memcmp(st.c(), st.c() + l * stride, one) == 0);
  int dummy[4];
  stub::steps.clear();
  CHECK(lf_decode_step(dummy, dummy, dummy, h, dummy, dummy, nullptr) == LF_ERR_ARG);  // several layers
  for (int l = 0; l < NL; ++l) CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, l, dummy, dummy, nullptr) == LF_OK);
  CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, NL, dummy, dummy, nullptr) == LF_ERR_ARG);
  CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, -1, dummy, dummy, nullptr) == LF_ERR_ARG);
  CHECK(stub::steps.size() == (size_t)NL);
  for (int l = 0; l < NL && l < (int)stub::steps.size(); ++l) {
    CHECK(stub::steps[l].k_cache == ks[l] && stub::steps[l].v_cache == vs[l]);
    CHECK(stub::steps[l].meta == vw[l].meta && stub::steps[l].u_budget == 300);
  }
  // what steps would leave: positions advanced, rings moved, epochs counted on
  for (int l = 0; l < NL; ++l)
    for (int p = 0; p < B * H; ++p) {
      vw[l].meta[p].t = 350;
      vw[l].meta[p].epoch = 51 + 7 * l + p;
      for (int j = 0; j < R; ++j) vw[l].ring[p * R + j] = 100 + j;  // distinct filled slots
    }
  lf_state_report rep{};
  CHECK(lf_check_state(h, nullptr, &rep) == LF_OK);
  // restart sequence 2 (same budget) in every layer
  const int32_t s2[1] = {2};
  const int64_t t2[1] = {40};
  CHECK(lf_reset_sequences(h, 1, s2, t2, nullptr) == LF_OK);
  for (int l = 0; l < NL; ++l)
    for (int g = 0; g < H; ++g) {
      const int p = 2 * H + g;
      check_started(vw[l], p, 40, 300, R);
      CHECK(vw[l].meta[p].epoch == (uint32_t)(51 + 7 * l + p));  // carried on
      CHECK(vw[l].meta[0].t == 350 && vw[l].ring[0] == 100);     // sequence 0 untouched
    }
  CHECK(lf_check_state(h, nullptr, &rep) == LF_OK);
  // argument errors change nothing
  const int32_t dup[2] = {1, 1};
  const int64_t tt[2] = {5, 5};
  CHECK(lf_reset_sequences(h, 2, dup, tt, nullptr) == LF_ERR_ARG);
  const int32_t out_of_range[1] = {B};
  CHECK(lf_reset_sequences(h, 1, out_of_range, tt, nullptr) == LF_ERR_ARG);
  CHECK(lf_reset_sequences(h, 0, nullptr, nullptr, nullptr) == LF_OK);
  // new budgets for sequences 1 and 3: one larger, one smaller and not full
  const int32_t s13[2] = {1, 3};
  const int64_t t13[2] = {700, 90};
  const int32_t b13[2] = {900, 120};
  size_t need_big = 0;
  const int32_t all_big[B] = {1024, 1024, 1024, 1024};
  CHECK(lf_state_bytes(&c, all_big, &need_big) == LF_OK);
  CHECK(lf_reset_sequences_budget(h, 2, s13, t13, b13, nullptr) == LF_OK);
  for (int l = 0; l < NL; ++l) {
    uint32_t top = 0;
    for (int p = 0; p < B * H; ++p) top = top > (uint32_t)(51 + 7 * l + p) ? top : (uint32_t)(51 + 7 * l + p);
    for (int g = 0; g < H; ++g) {
      check_started(vw[l], 1 * H + g, 700, 900, R);
      check_started(vw[l], 3 * H + g, 90, 120, R);
      check_started(vw[l], 2 * H + g, 40, 300, R);  // restarted before, kept
      CHECK(vw[l].meta[g].t == 350 && vw[l].meta[g].len == 300 && vw[l].meta[g].budget == 300);
    }
    for (int p = 0; p < B * H; ++p) CHECK(vw[l].meta[p].epoch == top + 1);
    CHECK(vw[l].h->n_items == vw[0].h->n_items);
    check_items(vw[l], B * H);
  }
  CHECK(lf_check_state(h, nullptr, &rep) == LF_OK);
  // budgets the buffer cannot hold: rejected, nothing written
  std::vector<char> snap(st.c(), st.c() + st.n);
  const int32_t s_all[B] = {0, 1, 2, 3};
  const int64_t t_all[B] = {1024, 1024, 1024, 1024};
  CHECK(need_big > stride);
  CHECK(lf_reset_sequences_budget(h, B, s_all, t_all, all_big, nullptr) == LF_ERR_ARG);
  CHECK(std::memcmp(snap.data(), st.c(), st.n) == 0);
  const int32_t tiny[1] = {12};  // <= sink + recent
  CHECK(lf_reset_sequences_budget(h, 1, s2, t2, tiny, nullptr) == LF_ERR_ARG);
  CHECK(std::memcmp(snap.data(), st.c(), st.n) == 0);
  stub::fail_copies = 1;  // a failing read-back leaves the handle as it was
  const int32_t b300[1] = {300};
  CHECK(lf_reset_sequences_budget(h, 1, s2, t2, b300, nullptr) == LF_ERR_HIP);
  CHECK(std::memcmp(snap.data(), st.c(), st.n) == 0);
  stub::fail_copies = 0;
  // steps after the re-layout see the new work list
  stub::steps.clear();
  CHECK(lf_decode_step_layer(dummy, dummy, dummy, h, 2, dummy, dummy, nullptr) == LF_OK);
  CHECK(!stub::steps.empty() && stub::steps.back().u_budget == 0 && stub::steps.back().n_items == vw[2].h->n_items);
  // a layer's broken state names the layer
  vw[1].meta[5].len = vw[1].meta[5].len + 3;
  CHECK(lf_check_state(h, nullptr, &rep) == LF_ERR_STATE && rep.bad_layer == 1 && rep.bad_pair == 5);
  lf_free(h);
  for (auto* p : kb) delete p;
  for (auto* p : vb) delete p;
}

void test_prefill() {
  lf_config c = config(2, 8, 2, 128, 512, 4, 16);
  size_t wb = 0;
  CHECK(lf_prefill_work_bytes(&c, 1024, &wb) == LF_OK && wb > 0);
  CHECK(lf_prefill_work_bytes(&c, 0, &wb) == LF_ERR_ARG);
  Buf work(wb), q(4096), kp(4096), vp(4096), kc(4096), vc(4096), kept(4096);
  const int32_t pre[2] = {1000, 300};
  stub::prefills.clear();
  CHECK(lf_prefill_compress(&c, nullptr, pre, 1024, q.p, kp.p, vp.p, kc.p, vc.p, (int32_t*)kept.p, work.p, wb,
                            nullptr) == LF_OK);
  CHECK(stub::prefills.size() >= 1);
  const int32_t too_long[2] = {1025, 300};
  CHECK(lf_prefill_compress(&c, nullptr, too_long, 1024, q.p, kp.p, vp.p, kc.p, vc.p, (int32_t*)kept.p, work.p, wb,
                            nullptr) == LF_ERR_ARG);
  CHECK(lf_prefill_compress(&c, nullptr, pre, 1024, q.p, kp.p, vp.p, kc.p, vc.p, (int32_t*)kept.p, work.p, wb - 1,
                            nullptr) == LF_ERR_ARG);
  // the static scratch (64 KiB in the stand-in's place is not what the library
  // assumes: only the size check is exercised here)
  lf_config big = config(128, 40, 8, 128, 8192, 4, 64);
  std::vector<int32_t> bb(128, 8192), pp(128, 16384);
  CHECK(lf_prefill_compress_noalloc(&big, bb.data(), pp.data(), 16384, q.p, kp.p, vp.p, kc.p, vc.p,
                                    (int32_t*)kept.p, nullptr) == LF_ERR_ARG);
}

}  // namespace

int main() {
  test_validation();
  test_single_layer();
  test_layers_and_resets();
  test_prefill();
  std::printf("%s: %d failed checks\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail > 255 ? 255 : g_fail;
}
