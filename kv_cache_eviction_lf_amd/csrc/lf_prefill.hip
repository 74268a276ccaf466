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
// Two launches on the caller's stream:
//   prefill_score_kernel   one workgroup per pair: two passes over the pair's
//                          K rows (maxima and normalisers, then importance).
//   prefill_select_kernel  one workgroup per pair: radix selection of the
//                          threshold over 64-bit keys (importance, then the
//                          complement of the position, so keys are unique and
//                          the lower position ranks first on equal importance),
//                          position-ordered compaction, then the row copies.
#include <hip/hip_runtime.h>
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
__device__ __forceinline__ void unpack16(const uint4& r, float (&x)[8], BF16E) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Sum over the LPR lanes that hold one row (lanes lane ^ 1, 2, ... within the row).
template <int LPR>
__device__ __forceinline__ float row_total(float x) {
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// (max, sum of exp2(x - max)) pairs combined.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (m2 == -INFINITY ? 0.f : l2 * exp2f(m2 - mn));
  m = mn;
}

template <class E, int D>
__global__ __launch_bounds__(kPT) void prefill_score_kernel(PrefillArgs a) {
  using elem = typename E::elem;
  constexpr int EPL = E::kEpl, LPR = D / EPL, RPW = 64 / LPR;
  const int pair = blockIdx.x;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const int G = a.group;
  const int P = a.prefill[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % LPR, rw = lane / LPR;
  const elem* kp = static_cast<const elem*>(a.k_pre) + (size_t)pair * a.max_prefill * D + c * EPL;
  float q[kMaxG][EPL];
  {
    const elem* qb = static_cast<const elem*>(a.q_last) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D + c * EPL;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      const uint4 r = *reinterpret_cast<const uint4*>(qb + (size_t)min(h, G - 1) * D);
      unpack16(r, q[h], E{});
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[h][e] *= a.scale_log2;
    }
  }
  auto logits = [&](int row, float (&s)[kMaxG]) {
    float k[EPL];
    unpack16(*reinterpret_cast<const uint4*>(kp + (size_t)row * D), k, E{});
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], k[e], p);
      s[h] = row_total<LPR>(p);
    }
  };
  // Pass 1: per-head maximum and normaliser (log2 domain), one row lineage per
  // lane group, then across lanes and waves.
  float m[kMaxG], l[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  for (int row = wave * RPW + rw; row < P; row += kPW * RPW) {
    float s[kMaxG];
    logits(row, s);
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) ml_merge(m[h], l[h], s[h], 1.f);
  }
  __shared__ float s_m[kPW][kMaxG], s_l[kPW][kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    float mm = c == 0 ? m[h] : -INFINITY, ll = c == 0 ? l[h] : 0.f;  // one lane per row lineage
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ml_merge(mm, ll, __shfl_xor(mm, o), __shfl_xor(ll, o));
    if (lane == 0) {
      s_m[wave][h] = mm;
      s_l[wave][h] = ll;
    }
  }
  __syncthreads();
  float M[kMaxG], invL[kMaxG];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    float mm = s_m[0][h], ll = s_l[0][h];
#pragma unroll
    for (int w = 1; w < kPW; ++w) ml_merge(mm, ll, s_m[w][h], s_l[w][h]);
    M[h] = mm;
    invL[h] = 1.0f / ll;
  }
  // Pass 2: importance of every prefill position.
  float* imp = a.work + (size_t)pair * a.max_prefill;
  for (int row = wave * RPW + rw; row < P; row += kPW * RPW) {
    float s[kMaxG];
    logits(row, s);
    float x = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h)
      if (h < G) x = fmaf(exp2f(s[h] - M[h]), invL[h], x);
    if (c == 0) imp[row] = x;
  }
}

// Key of a middle position: importance bits (non-negative floats order as
// their bit patterns), then the complement of the position.
__device__ __forceinline__ uint64_t rank_key(float x, int pos) {
  return (static_cast<uint64_t>(__float_as_uint(fmaxf(x, 0.f))) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(pos));
}

template <class E, int D>
__global__ __launch_bounds__(kPT) void prefill_select_kernel(PrefillArgs a) {
  using elem = typename E::elem;
  const int pair = blockIdx.x;
  const int b = pair / a.n_kv_heads;
  const int P = a.prefill[b], budget = a.budget[b];
  const int sink = a.sink, R = a.recent;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* imp = a.work + (size_t)pair * a.max_prefill;
  int32_t* kept = a.kept + (size_t)pair * a.max_budget;
  const int nkeep = min(P, budget);
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_digit, s_want;
  __shared__ uint32_t s_scan[kPT];

  uint64_t thr = 0;  // a middle position is kept when its key is >= thr
  if (P > budget) {
    const int lo = sink, hi = P - R;
    uint64_t prefix = 0, mask = 0;
    if (tid == 0) s_want = budget - sink - R;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += kPT) s_hist[i] = 0u;
      __syncthreads();
      for (int i = lo + tid; i < hi; i += kPT) {
        const uint64_t key = rank_key(imp[i], i);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
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
      __syncthreads();  // s_digit / s_want are rewritten next pass
    }
    thr = prefix;  // keys are unique: exactly budget - sink - R middle keys are >= it
  }

  // Position-ordered compaction: thread t scans positions [t per, (t+1) per).
  const int per = (P + kPT - 1) / kPT;
  const int p0 = min(P, tid * per), p1 = min(P, p0 + per);
  auto keep = [&](int pos) {
    return P <= budget || pos < sink || pos >= P - R || rank_key(imp[pos], pos) >= thr;
  };
  uint32_t n = 0;
  for (int pos = p0; pos < p1; ++pos) n += keep(pos) ? 1u : 0u;
  s_scan[tid] = n;
  __syncthreads();
  for (int o = 1; o < kPT; o <<= 1) {  // inclusive scan (Hillis-Steele)
    const uint32_t v = tid >= o ? s_scan[tid - o] : 0u;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  uint32_t j = s_scan[tid] - n;
  for (int pos = p0; pos < p1; ++pos)
    if (keep(pos) && j < static_cast<uint32_t>(nkeep)) kept[j++] = pos;  // exactly nkeep are kept
  __syncthreads();  // kept[] of this pair complete (same workgroup)

  // Row copies: one row per wave at a time, 16 bytes per lane.
  constexpr int kPieces = D * sizeof(elem) / 16;
  const uint4* ksrc = reinterpret_cast<const uint4*>(static_cast<const elem*>(a.k_pre) + (size_t)pair * a.max_prefill * D);
  const uint4* vsrc = reinterpret_cast<const uint4*>(static_cast<const elem*>(a.v_pre) + (size_t)pair * a.max_prefill * D);
  uint4* kdst = reinterpret_cast<uint4*>(static_cast<elem*>(a.k_cache) + (size_t)pair * a.max_budget * D);
  uint4* vdst = reinterpret_cast<uint4*>(static_cast<elem*>(a.v_cache) + (size_t)pair * a.max_budget * D);
  constexpr int kRowsPerWave = 64 / kPieces;
  const int sub = lane / kPieces, piece = lane % kPieces;
  for (int r = wave * kRowsPerWave + sub; r < nkeep; r += kPW * kRowsPerWave) {
    const int pos = kept[r];
    if (pos < 0 || pos >= P) continue;  // not reached: kept[0, nkeep) holds positions below P
    kdst[(size_t)r * kPieces + piece] = ksrc[(size_t)pos * kPieces + piece];
    vdst[(size_t)r * kPieces + piece] = vsrc[(size_t)pos * kPieces + piece];
  }
}

template <class E, int D>
void launch_prefill(const PrefillArgs& a, int n_pairs, hipStream_t s) {
  hipLaunchKernelGGL((prefill_score_kernel<E, D>), dim3(n_pairs), dim3(kPT), 0, s, a);
  hipLaunchKernelGGL((prefill_select_kernel<E, D>), dim3(n_pairs), dim3(kPT), 0, s, a);
}

}  // namespace

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
