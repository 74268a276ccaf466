// One-shot compression of prefills longer than the budget (the step before the
// decode path): the last prefill query attends over every prefill token, a
// token's importance is the softmax weight it gets summed over its KV group's
// query heads (the decode step's own importance, LongFlow summary on
// gist.science, section 2.A: from the current query only), and each (sequence,
// KV head) keeps its sink positions, its recent window and the middle
// positions of largest importance (the lower position first on equal
// importance), in position order.  The summary's section 5 leaves long prefill
// to other methods; this selection is the plainest reading that keeps the
// decode step's importance.
//
// Three launches on the caller's stream:
//   prefill_stats_kernel       a workgroup per (pair, 512-row chunk): the
//                              chunk's logits (stored head-major, [G][position])
//                              and their per-head maximum and normaliser.
//   prefill_select_kernel      a workgroup per pair, the pairs of the longest
//                              prefills first: the pair's statistics
//                              combined in chunk order, every position's
//                              importance from its stored logits (no second
//                              pass over K; kept in LDS for prefills up to
//                              kSelLdsMax positions), then radix selection of
//                              the threshold over 48-bit keys (importance, then
//                              the complement of the position, so keys are
//                              unique and the lower position ranks first on
//                              equal importance; passes stop once the bin at
//                              the threshold is wanted whole) and
//                              position-ordered compaction.
//   prefill_copy_kernel        a workgroup per (pair, 256 kept rows): the
//                              kept K/V rows copied in order.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "lf_internal.h"

namespace lf {
namespace {

constexpr int kPT = 256;  // threads per workgroup
constexpr int kPW = kPT / 64;
constexpr int kMaxG = 8;

struct F32E {
  using elem = float;
  static constexpr int kEpl = 4;  // elements per 16-byte load
};
struct BF16E {
  using elem = uint16_t;
  static constexpr int kEpl = 8;
};

__device__ __forceinline__ void unpack16(const uint4& r, float (&x)[4], F32E) {
  x[0] = __uint_as_float(r.x);
  x[1] = __uint_as_float(r.y);
  x[2] = __uint_as_float(r.z);
  x[3] = __uint_as_float(r.w);
}
[[maybe_unused]] __device__ __forceinline__ void unpack16(const uint4& r, float (&x)[8], BF16E) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR consecutive lanes that hold one row, every lane of the row
// getting it: DPP within rows of 16 lanes (quad swaps, half-row and row
// mirrors), a lane swizzle across 16 for 32-lane rows.
template <int LPR>
__device__ __forceinline__ float row_total(float x) {
  if constexpr (LPR >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x);
  if constexpr (LPR >= 32) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  static_assert(LPR <= 32, "rows of at most 32 lanes");
  return x;
}

// 16-byte non-temporal load (data read once).
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// 16-byte non-temporal store (rows written once here; the copy of the kept
// rows measured 2.5 % faster than with plain stores).
__device__ __forceinline__ void store_once(uint4* p, const uint4& v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}

// (max, sum of exp2(x - max)) pairs combined.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (m2 == -INFINITY ? 0.f : l2 * exp2f(m2 - mn));
  m = mn;
}

// Per-sequence prefill length, budget and the sequence of rank r in order of
// decreasing prefill length: from the kernel arguments for small batches,
// else from the device arrays the host uploaded.
__device__ __forceinline__ int prefill_of(const PrefillArgs& a, int b) { return a.n_inline ? a.lens[b] : a.prefill[b]; }
__device__ __forceinline__ int budget_of(const PrefillArgs& a, int b) {
  return a.n_inline ? a.lens[a.n_inline + b] : a.budget[b];
}
__device__ __forceinline__ int seq_of_rank(const PrefillArgs& a, int r) {
  return a.n_inline ? a.lens[2 * a.n_inline + r] : a.order[r];
}

// Rows of one chunk of the score passes: pairs are split so that short
// batches still fill the device.
constexpr int kChunkRows = kPrefillChunk;
constexpr int kSel = 8;  // positions per thread whose loads the selection pass issues together
// Longest prefill whose importances the selection pass keeps in LDS (60 KB
// of the 64 KB a workgroup may hold, beside the histogram, scan and chunk
// statistics arrays); longer prefills are selected from the copy in global
// memory.
constexpr int kSelLdsMax = 15360;

template <class E, int D, int G>
struct ScoreCore {
  using elem = typename E::elem;
  static constexpr int EPL = E::kEpl, LPR = D / EPL, RPW = 64 / LPR;
  static constexpr int kU = 4;  // rows per lane group per iteration (loads first)
  float q[G][EPL];
  const elem* kp;
  int c, rw;

  __device__ ScoreCore(const PrefillArgs& a, int pair) {
    const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
    const int lane = threadIdx.x & 63;
    c = lane % LPR;
    rw = lane / LPR;
    kp = static_cast<const elem*>(a.k_pre) + (size_t)pair * a.max_prefill * D + c * EPL;
    const elem* qb = static_cast<const elem*>(a.q_last) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D + c * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 r = *reinterpret_cast<const uint4*>(qb + (size_t)h * D);
      unpack16(r, q[h], E{});
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[h][e] *= a.scale_log2;
    }
  }
  // Calls f(row, s[G]) with the log2-domain logits of every row of
  // [r0, r1) this lane group owns; rows past r1 are loaded clamped, not used.
  template <class F>
  __device__ void for_rows(int r0, int r1, F f) const {
    const int wave = threadIdx.x >> 6;
    for (int base = r0 + wave * RPW * kU + rw; base < r1; base += kPW * RPW * kU) {
      uint4 kr[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        kr[u] = *reinterpret_cast<const uint4*>(kp + (size_t)min(base + u * RPW, r1 - 1) * D);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float k[EPL];
        unpack16(kr[u], k, E{});
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], k[e], p);
          s[h] = row_total<LPR>(p);
        }
        if (base + u * RPW < r1) f(base + u * RPW, s);
      }
    }
  }
};

// Pass 1: the chunk's logits, stored head-major [G][max_prefill] (lane c of a
// row lineage stores head c), and per head their maximum and normaliser (log2
// domain).
template <class E, int D, int G>
__global__ __launch_bounds__(kPT) void prefill_stats_kernel(PrefillArgs a) {
  const int pair = blockIdx.x / a.n_chunks, chunk = blockIdx.x - pair * a.n_chunks;
  const int b = pair / a.n_kv_heads;
  const int P = prefill_of(a, b);
  if (chunk * kChunkRows >= P) return;  // past this prefill (the grid covers the longest)
  const int r0 = chunk * kChunkRows, r1 = min(P, r0 + kChunkRows);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  const ScoreCore<E, D, G> core(a, pair);
  float* lg = a.logits + (size_t)pair * a.max_prefill * G;
  core.for_rows(r0, r1, [&](int row, const float(&s)[G]) {
    // Running (max, sum) per head: the sum is rescaled only when the max
    // moves (the hardware exp2; all lanes of a row lineage agree).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (s[h] > m[h]) {
        l[h] *= __builtin_amdgcn_exp2f(m[h] - s[h]);
        m[h] = s[h];
      }
      l[h] += __builtin_amdgcn_exp2f(s[h] - m[h]);
    }
    float mine = s[0];
#pragma unroll
    for (int h = 1; h < G; ++h) mine = core.c == h ? s[h] : mine;
    if (core.c < G) lg[(size_t)core.c * a.max_prefill + row] = mine;
  });
  __shared__ float s_m[kPW][kMaxG], s_l[kPW][kMaxG];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mm = core.c == 0 ? m[h] : -INFINITY, ll = core.c == 0 ? l[h] : 0.f;  // one lane per row lineage
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ml_merge(mm, ll, __shfl_xor(mm, o), __shfl_xor(ll, o));
    if (lane == 0) {
      s_m[wave][h] = mm;
      s_l[wave][h] = ll;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float mm = s_m[0][h], ll = s_l[0][h];
#pragma unroll
    for (int w = 1; w < kPW; ++w) ml_merge(mm, ll, s_m[w][h], s_l[w][h]);
    float* st = a.stats + ((size_t)pair * a.n_chunks + chunk) * kMaxG * 2;
    st[2 * h] = mm;
    st[2 * h + 1] = ll;
  }
}

// Pass 1 for bf16 on the matrix cores: each wave takes 128 consecutive rows of
// the chunk in groups of 16; one v_mfma_f32_16x16x32_bf16 per 32 dimensions
// multiplies the group's 16 key rows by the group's query heads (columns,
// heads past G unused), so lane 16 j + n holds the logits of rows 4 j .. 4 j +
// 3 of the group for head n.  Each lane keeps the running (max, sum) of its
// head over its rows; lanes of one head are combined at the end.  Same
// results as the vector-ALU pass up to the order of the dot products' sums.
template <int D, int G>
__global__ __launch_bounds__(kPT) void prefill_stats_mfma_kernel(PrefillArgs a) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int KB = D / 32;
  constexpr int kWaveRows = kChunkRows / kPW;  // 128
  constexpr int NS = 4;                        // 16-row groups in flight per wave (current one included)
  const int pair = blockIdx.x / a.n_chunks, chunk = blockIdx.x - pair * a.n_chunks;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const int P = prefill_of(a, b);
  if (chunk * kChunkRows >= P) return;  // past this prefill (the grid covers the longest)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, j = lane >> 4;
  const int r0 = chunk * kChunkRows + wave * kWaveRows;
  const int r1 = min(P, r0 + kWaveRows);  // this wave's rows [r0, r1)
  uint4 qb[KB];
  {
    const int hq = n < G ? n : 0;  // columns past G load head 0 and are not used
    const uint16_t* qh = static_cast<const uint16_t*>(a.q_last) + ((size_t)b * a.n_q_heads + (size_t)g * G + hq) * D + 8 * j;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qb[kb] = *reinterpret_cast<const uint4*>(qh + 32 * kb);
  }
  const uint16_t* kp = static_cast<const uint16_t*>(a.k_pre) + (size_t)pair * a.max_prefill * D + 8 * j;
  // Logit stores go through a buffer resource over the pair's [G][max_prefill]
  // logits; lanes without a logit to store (heads past G, rows past the wave's
  // range) aim past it and the hardware drops the store, so no store (and no
  // load below) sits under a divergent branch and the loop's waits stay exact.
  // A whole group stores each lane's 4 rows of its head as one 16-byte cell.
  const auto lrs = __builtin_amdgcn_make_buffer_rsrc(a.logits + (size_t)pair * a.max_prefill * G, (short)0,
                                                     G * a.max_prefill * 4, 0x00020000);
  float m = -INFINITY, l = 0.f;
  const int last = max(r1 - 1, 0);
  auto load = [&](int R, uint4(&kk)[KB]) {  // rows clamped to the wave's last valid row
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      kk[kb] = load_once(reinterpret_cast<const uint4*>(kp + (size_t)min(R + n, last) * D + 32 * kb));
  };
  auto process = [&](int R, const uint4(&kk)[KB]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[kb]),
                                                    __builtin_bit_cast(bf16x8_t, qb[kb]), acc, 0, 0, 0);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = R + 4 * j + i;
      sv[i] = row < r1 ? acc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    if (R + 16 <= r1) {
      const u32x4_t x = {__float_as_uint(sv[0]), __float_as_uint(sv[1]), __float_as_uint(sv[2]),
                         __float_as_uint(sv[3])};
      const int off = n < G ? (n * a.max_prefill + R + 4 * j) * 4 : 0x7FFFFFF0;
      __builtin_amdgcn_raw_buffer_store_b128(x, lrs, off, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = R + 4 * j + i;
        const int off = n < G && row < r1 ? (n * a.max_prefill + row) * 4 : 0x7FFFFFF0;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv[i]), lrs, off, 0, 0);
      }
    }
    if (mx > m) {
      l *= __builtin_amdgcn_exp2f(m - mx);
      m = mx;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l += sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m);
  };
  // A ring of NS group buffers: while group t is processed, groups up to
  // t + NS - 1 are in flight.  Loads are unconditional (rows clamped to the
  // wave's last row) and the loop has one exit, so the waits stay exact.
  const int ng = r1 > r0 ? (r1 - r0 + 15) / 16 : 0;
  uint4 buf[NS][KB];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) load(r0 + 16 * s, buf[s]);
  int t = 0;
  while (t + NS <= ng) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      load(r0 + 16 * (t + NS - 1), buf[(s + NS - 1) % NS]);
      process(r0 + 16 * t, buf[s]);
      ++t;
    }
  }
  // Fewer than NS groups left, all of them already loaded.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (t < ng) {
      process(r0 + 16 * t, buf[s]);
      ++t;
    }
  // Combine the 4 lane groups of each head (lanes n, n + 16, n + 32, n + 48),
  // then the waves.
  ml_merge(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16));
  ml_merge(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
  __shared__ float s_m[kPW][16], s_l[kPW][16];
  if (lane < 16) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = l;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float mm = s_m[0][h], ll = s_l[0][h];
#pragma unroll
    for (int w = 1; w < kPW; ++w) ml_merge(mm, ll, s_m[w][h], s_l[w][h]);
    float* st = a.stats + ((size_t)pair * a.n_chunks + chunk) * kMaxG * 2;
    st[2 * h] = mm;
    st[2 * h + 1] = ll;
  }
}

// Key of a middle position: importance bits (non-negative floats order as
// their bit patterns), then the complement of the position (positions are
// below 65536): 48 bits, unique per position.
__device__ __forceinline__ uint64_t rank_key(float x, int pos) {
  return (static_cast<uint64_t>(__float_as_uint(fmaxf(x, 0.f))) << 16) | (0xFFFFu - static_cast<uint32_t>(pos));
}

template <int G, bool kLds>
__global__ __launch_bounds__(kPT) void prefill_select_kernel(PrefillArgs a) {
  extern __shared__ float s_dyn[];  // kLds: the pair's importances, a.max_prefill floats
  // Workgroups take the pairs of the longest prefills first, so the longest
  // selections do not start in a late round of the grid.
  const int rank = blockIdx.x / a.n_kv_heads;
  const int b = seq_of_rank(a, rank);
  const int pair = b * a.n_kv_heads + (blockIdx.x - rank * a.n_kv_heads);
  const int P = prefill_of(a, b), budget = budget_of(a, b);
  const int sink = a.sink, R = a.recent;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* imp_out = a.work + (size_t)pair * a.max_prefill;  // the call's importance output
  const float* imp = kLds ? s_dyn : imp_out;               // what the selection reads
  int32_t* kept = a.kept + (size_t)pair * a.max_budget;
  const int nkeep = min(P, budget);
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_digit, s_want, s_done;
  __shared__ uint32_t s_scan[kPT];

  // The pair's statistics combined in chunk order, then every position's
  // importance from its stored logits (written out as the call's importance
  // output and, with kLds, kept in LDS for the selection below; without it
  // the selection reads the output back).
  {
    // The chunks' (max, sum) of the G heads are loaded together into LDS (one
    // memory round trip instead of one per chunk), merged in chunk order by
    // thread h for head h, and read back by every thread.
    constexpr int kMaxChunksSel = (kLds ? kSelLdsMax : kMaxPrefill) / kChunkRows;
    __shared__ float s_st[kMaxChunksSel * G * 2];
    __shared__ float s_mi[2 * G];
    const int nck = (P + kChunkRows - 1) / kChunkRows;
    const float* st = a.stats + (size_t)pair * a.n_chunks * kMaxG * 2;
    for (int i = tid; i < nck * G * 2; i += kPT) {
      const int k = i / (2 * G), r = i - k * 2 * G;
      s_st[i] = st[k * kMaxG * 2 + r];
    }
    __syncthreads();
    if (tid < G) {
      float mm = -INFINITY, ll = 0.f;
      for (int k = 0; k < nck; ++k) ml_merge(mm, ll, s_st[k * 2 * G + 2 * tid], s_st[k * 2 * G + 2 * tid + 1]);
      s_mi[tid] = mm;
      s_mi[G + tid] = 1.0f / ll;
    }
    __syncthreads();
    float M[G], invL[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      M[h] = s_mi[h];
      invL[h] = s_mi[G + h];
    }
    // kSel positions per thread and pass, their logits loaded before any
    // store (the compiler cannot move a load above a store it cannot tell
    // apart), so a pass costs one memory round trip rather than kSel.
    const float* lg = a.logits + (size_t)pair * a.max_prefill * G;
    constexpr int kImp = kLds ? 2 * kSel : kSel;  // positions per round trip (registers allow more with kLds)
    for (int i0 = tid; i0 < P; i0 += kImp * kPT) {
      float x[kImp][G];
#pragma unroll
      for (int u = 0; u < kImp; ++u) {
        const int i = min(i0 + u * kPT, P - 1);
#pragma unroll
        for (int h = 0; h < G; ++h) x[u][h] = lg[(size_t)h * a.max_prefill + i];
      }
#pragma unroll
      for (int u = 0; u < kImp; ++u) {
        float y = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) y = fmaf(__builtin_amdgcn_exp2f(x[u][h] - M[h]), invL[h], y);
        if (i0 + u * kPT < P) {
          imp_out[i0 + u * kPT] = y;
          if constexpr (kLds) s_dyn[i0 + u * kPT] = y;
        }
      }
    }
    __syncthreads();  // every position's importance written (same workgroup)
  }

  uint64_t thr = 0;  // a middle position is kept when its key is >= thr
  if (P > budget) {
    const int lo = sink, hi = P - R;
    uint64_t prefix = 0, mask = 0;
    if (tid == 0) {
      s_want = budget - sink - R;
      s_done = 0u;
    }
    for (int pass = 0; pass < 6; ++pass) {
      const int shift = 40 - 8 * pass;
      for (int i = tid; i < 256; i += kPT) s_hist[i] = 0u;
      __syncthreads();
      for (int i0 = lo + tid; i0 < hi; i0 += kSel * kPT) {
        float v[kSel];
#pragma unroll
        for (int u = 0; u < kSel; ++u) v[u] = imp[min(i0 + u * kPT, hi - 1)];
#pragma unroll
        for (int u = 0; u < kSel; ++u) {
          const int i = i0 + u * kPT;
          const uint64_t key = rank_key(v[u], i);
          const bool in = i < hi && (key & mask) == prefix;
          const uint32_t bin = static_cast<uint32_t>(key >> shift) & 255u;
          // Importances of one pair often share their leading bits, so most
          // lanes of a wave hit one bin: the bin of the wave's first counted
          // lane is added once for every lane holding it, the others singly.
          const uint64_t act = __builtin_amdgcn_ballot_w64(in);
          if (act) {
            const uint32_t lead = __builtin_amdgcn_readlane(bin, __builtin_ctzll(act));
            const uint64_t same = __builtin_amdgcn_ballot_w64(in && bin == lead);
            if (lane == __builtin_ctzll(act)) atomicAdd(&s_hist[lead], static_cast<uint32_t>(__builtin_popcountll(same)));
            if (in && bin != lead) atomicAdd(&s_hist[bin], 1u);
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 255 - 4l ... 252 - 4l (descending); suffix sums
        // over the lanes find the digit at which the count from the top
        // reaches the number of keys still wanted.
        uint32_t cnt[4], own = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cnt[k] = s_hist[255 - 4 * lane - k];
          own += cnt[k];
        }
        uint32_t incl = own;  // inclusive prefix over lanes 0..lane (higher digits first)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t v = __shfl_up(incl, o);
          if (lane >= o) incl += v;
        }
        const uint32_t want = s_want;
        uint32_t before = incl - own;
        if (before < want && incl >= want) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (before < want && before + cnt[k] >= want) {
              s_digit = 255 - 4 * lane - k;
              s_want = want - before;
              // the whole bin is wanted: every key at or above the bin's
              // smallest key is kept, the lower bits need no further pass
              s_done = before + cnt[k] == want ? 1u : 0u;
              before = want;  // found: no later digit qualifies
            } else {
              before += cnt[k];
            }
          }
        }
      }
      __syncthreads();
      prefix |= static_cast<uint64_t>(s_digit) << shift;
      mask |= 0xFFull << shift;
      const bool done = s_done != 0u;
      __syncthreads();  // s_digit / s_want / s_done are rewritten next pass
      if (done) break;
    }
    thr = prefix;  // keys are unique: exactly budget - sink - R middle keys are >= it
  }

  // Position-ordered compaction: thread t scans positions [t per, (t+1) per).
  const int per = (P + kPT - 1) / kPT;
  const int p0 = min(P, tid * per), p1 = min(P, p0 + per);
  auto keep = [&](int pos, float x) {
    return P <= budget || pos < sink || pos >= P - R || rank_key(x, pos) >= thr;
  };
  // The thread's keep flags, kSel positions per load batch.
  uint32_t n = 0;
  for (int q0 = p0; q0 < p1; q0 += kSel) {
    float v[kSel];
#pragma unroll
    for (int u = 0; u < kSel; ++u) v[u] = imp[min(q0 + u, p1 - 1)];
#pragma unroll
    for (int u = 0; u < kSel; ++u) n += q0 + u < p1 && keep(q0 + u, v[u]) ? 1u : 0u;
  }
  s_scan[tid] = n;
  __syncthreads();
  for (int o = 1; o < kPT; o <<= 1) {  // inclusive scan (Hillis-Steele)
    const uint32_t v = tid >= o ? s_scan[tid - o] : 0u;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  uint32_t j = s_scan[tid] - n;
  for (int q0 = p0; q0 < p1; q0 += kSel) {
    float v[kSel];
#pragma unroll
    for (int u = 0; u < kSel; ++u) v[u] = imp[min(q0 + u, p1 - 1)];
#pragma unroll
    for (int u = 0; u < kSel; ++u)
      if (q0 + u < p1 && keep(q0 + u, v[u]) && j < static_cast<uint32_t>(nkeep)) kept[j++] = q0 + u;  // exactly nkeep are kept
  }
  __syncthreads();  // kept[] of this pair complete (same workgroup)
}

// Row copies of the kept positions: a workgroup per (pair, 256 kept rows),
// one row per 64 / pieces lanes, 16 bytes per lane.
constexpr int kCopyRows = kPrefillCopyRows;

template <class E, int D>
__global__ __launch_bounds__(kPT) void prefill_copy_kernel(PrefillArgs a) {
  using elem = typename E::elem;
  const int pair = blockIdx.x / a.n_copy, part = blockIdx.x - pair * a.n_copy;
  const int b = pair / a.n_kv_heads;
  const int P = prefill_of(a, b), nkeep = min(P, budget_of(a, b));
  const int r0 = part * kCopyRows, r1 = min(nkeep, r0 + kCopyRows);
  const int32_t* kept = a.kept + (size_t)pair * a.max_budget;
  constexpr int kPieces = D * sizeof(elem) / 16;
  constexpr int kRowsPerWave = 64 / kPieces;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / kPieces, piece = lane % kPieces;
  const uint4* ksrc = reinterpret_cast<const uint4*>(static_cast<const elem*>(a.k_pre) + (size_t)pair * a.max_prefill * D);
  const uint4* vsrc = reinterpret_cast<const uint4*>(static_cast<const elem*>(a.v_pre) + (size_t)pair * a.max_prefill * D);
  uint4* kdst = reinterpret_cast<uint4*>(static_cast<elem*>(a.k_cache) + (size_t)pair * a.max_budget * D);
  uint4* vdst = reinterpret_cast<uint4*>(static_cast<elem*>(a.v_cache) + (size_t)pair * a.max_budget * D);
  // Each lane's kept positions first (independent loads, one round trip),
  // then kU rows per lane group per pass with all their loads issued before
  // any store; rows are read once and written once, so loads and stores are
  // non-temporal.
  const int n = r1 - r0;
  if (n <= 0) return;
  constexpr int kU = 16;
  constexpr int kStep = kPW * kRowsPerWave * kU;  // rows per pass of the workgroup
  constexpr int kPasses = (kCopyRows + kStep - 1) / kStep;
  int pos[kPasses][kU];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps)
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(ps * kStep + wave * kRowsPerWave * kU + u * kRowsPerWave + sub, n - 1);
      pos[ps][u] = min(max(kept[r0 + i], 0), P - 1);  // kept[0, nkeep) holds positions below P
    }
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    if (ps * kStep >= n) break;
    uint4 kx[kU], vx[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      kx[u] = load_once(ksrc + (size_t)pos[ps][u] * kPieces + piece);
      vx[u] = load_once(vsrc + (size_t)pos[ps][u] * kPieces + piece);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = ps * kStep + wave * kRowsPerWave * kU + u * kRowsPerWave + sub;
      if (i < n) {
        store_once(kdst + (size_t)(r0 + i) * kPieces + piece, kx[u]);
        store_once(vdst + (size_t)(r0 + i) * kPieces + piece, vx[u]);
      }
    }
  }
}

template <class E, int D, int G>
void launch_scores(const PrefillArgs& a, int n_pairs, hipStream_t s) {
  if constexpr (E::kEpl == 8)
    hipLaunchKernelGGL((prefill_stats_mfma_kernel<D, G>), dim3(n_pairs * a.n_chunks), dim3(kPT), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_stats_kernel<E, D, G>), dim3(n_pairs * a.n_chunks), dim3(kPT), 0, s, a);
  if (a.max_prefill <= kSelLdsMax)
    hipLaunchKernelGGL((prefill_select_kernel<G, true>), dim3(n_pairs), dim3(kPT), sizeof(float) * a.max_prefill, s,
                       a);
  else
    hipLaunchKernelGGL((prefill_select_kernel<G, false>), dim3(n_pairs), dim3(kPT), 0, s, a);
}

template <class E, int D>
void launch_prefill(const PrefillArgs& a, int n_pairs, hipStream_t s) {
  using Fn = void (*)(const PrefillArgs&, int, hipStream_t);
  constexpr Fn kScores[kMaxG] = {launch_scores<E, D, 1>, launch_scores<E, D, 2>, launch_scores<E, D, 3>,
                                 launch_scores<E, D, 4>, launch_scores<E, D, 5>, launch_scores<E, D, 6>,
                                 launch_scores<E, D, 7>, launch_scores<E, D, 8>};
  kScores[a.group - 1](a, n_pairs, s);
  hipLaunchKernelGGL((prefill_copy_kernel<E, D>), dim3(n_pairs * a.n_copy), dim3(kPT), 0, s, a);
}

}  // namespace

// Device scratch of the allocation-free prefill compression
// (lf_prefill_compress_noalloc): every GPU the library runs on holds one copy
// until the process ends.  Host code must not pass `scratch` itself to a
// kernel (in host code the name is a host-side stand-in, not a device
// address): prefill_scratch() looks up each device's address once and the
// kernels receive that pointer.  The prefill kernels write every byte they
// read in a call, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kPrefillScratchBytes];

int prefill_scratch(void** ptr, char* err, size_t errlen) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(err, errlen, "hipGetDevice failed: %s", hipGetErrorString(e));
    return 1;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(err, errlen, "device %d beyond the %d devices the static scratch supports", dev, kMaxDevices);
    return 1;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(err, errlen, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
      return 1;
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_prefill(int dtype, int head_dim, const PrefillArgs& a, int n_pairs, void* stream, char* err,
                   size_t errlen) {
  if (n_pairs <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = dtype == 1;
  if (head_dim == 64)
    bf ? launch_prefill<BF16E, 64>(a, n_pairs, s) : launch_prefill<F32E, 64>(a, n_pairs, s);
  else if (head_dim == 128)
    bf ? launch_prefill<BF16E, 128>(a, n_pairs, s) : launch_prefill<F32E, 128>(a, n_pairs, s);
  else {
    snprintf(err, errlen, "no prefill kernel for head_dim %d", head_dim);
    return 1;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "prefill kernel launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace lf
