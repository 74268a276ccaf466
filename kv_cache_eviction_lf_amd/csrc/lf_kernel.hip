// Fused LongFlow decode step for gfx950 (MI355X): GQA decode attention over a
// static cache + history-free importance + masked argmin + in-place overwrite,
// in one launch.
//
// What is computed follows the LongFlow summary (gist.science): section 2.A
// (importance from the current query only, as a by-product of attention),
// section 2.B (the LongFlowScore equation: attention weight times the L1 norm
// of the value; removal of the least important token) and section 2.C (one
// fused operator over a statically allocated cache).  The blog post
// (denisavetisyan.com) adds the dataflow of its figure caption: attention
// output O and importance I are produced from S = qK^T and P = softmax(S)
// while KV blocks and a mask stream from HBM, and one token is evicted after
// every attention computation.
//
// Design on gfx950 (wave64, 256 CUs in 8 XCDs, HBM3E):
//  * The step is HBM-bound: every cached K and V byte is read once, so the
//    kernel is a streaming scan, not a contraction.  Each lane issues 16-byte
//    loads of one row segment; a 64-lane load covers 64/LPR consecutive rows
//    (LPR = lanes per row), so every wave load is one contiguous 1 KiB run.
//    Each lane uses exactly the bytes it loads (q for all G heads of the group
//    is held in registers), so K/V go HBM -> VGPR with no LDS round trip.
//  * Split-KV: the (sequence, KV head) pairs are cut into chunks listed in a
//    static work list; one 256-thread workgroup per chunk.  A chunk keeps a
//    running max / sum / weighted value sum per head (online softmax in the
//    log2 domain) and stores its raw logits for the score pass.
//  * The last-arriving workgroup of a pair (device-scope ticket) merges the
//    chunk partials in chunk order, adds the incoming token, writes the output,
//    computes the exact importance of every slot from the stored logits and
//    the global max / normaliser, takes the lexicographic (score, slot) argmin
//    outside the sink slots and the ring of recent slots, and copies k_new /
//    v_new into the victim slot.  No other workgroup touches that pair after
//    its ticket, so the in-place write cannot race with a reader.
//  * Reductions across the lanes of a row use DPP (quad_perm, row mirrors);
//    everything else is fixed-order, so results are bit-reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "lf_internal.h"

namespace lf {
namespace {

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so empty partials merge without NaN
constexpr int kWaves = kThreads / 64;

struct F32T {
  using elem = float;
  static constexpr int kEpl = 4;  // elements per 16-byte load
};
struct BF16T {
  using elem = uint16_t;
  static constexpr int kEpl = 8;
};

template <class T, int D, int G>
struct Shape {
  static constexpr int kEpl = T::kEpl;
  static constexpr int kLpr = D / kEpl;   // lanes per row
  static constexpr int kRpl = 64 / kLpr;  // rows per wave load
  static constexpr int kU = G <= 4 ? 8 : 4;  // row loads per lane per tile (per tensor)
  static constexpr int kTile = kWaves * kRpl * kU;
  // LDS: cross-wave merge [wave][head][D + 2] before the ticket; tail buffers after.
  static constexpr int kMergeFloats = kWaves * G * (D + 2);
  static constexpr int kTailFloats = kMaxChunks * G + 2 * kWaves * G + 3 * G + kMaxBudget / 32 + 2 * kWaves;
  static constexpr int kSmemFloats = kMergeFloats > kTailFloats ? kMergeFloats : kTailFloats;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <class T>
__device__ __forceinline__ void unpack(const uint4& r, float (&x)[T::kEpl]) {
  if constexpr (T::kEpl == 4) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
  } else {
    x[0] = bf16_lo(r.x);
    x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y);
    x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z);
    x[5] = bf16_hi(r.z);
    x[6] = bf16_lo(r.w);
    x[7] = bf16_hi(r.w);
  }
}

// float -> bfloat16 bits, round to nearest, ties to even.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <class T>
__device__ __forceinline__ void store_elem(void* base, size_t i, float v) {
  if constexpr (T::kEpl == 4)
    static_cast<float*>(base)[i] = v;
  else
    static_cast<uint16_t*>(base)[i] = to_bf16(v);
}

template <class T>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (T::kEpl == 4)
    return static_cast<const float*>(base)[i];
  else
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR consecutive lanes that hold one row; every lane of the row
// gets the same bits (each step adds a value and its mirror, a commutative pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (score, slot) lexicographic minimum of two candidates.
__device__ __forceinline__ void argmin_merge(float& s, int& i, float so, int io) {
  if (so < s || (so == s && io < i)) {
    s = so;
    i = io;
  }
}

template <class T, int D, int G>
__global__ __launch_bounds__(kThreads) void lf_step_kernel(StepArgs a) {
  using S = Shape<T, D, G>;
  constexpr int EPL = S::kEpl, LPR = S::kLpr, RPL = S::kRpl, U = S::kU;
  using elem = typename T::elem;
  __shared__ float smem[S::kSmemFloats];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const WorkItem it = a.items[blockIdx.x];
  const int pair = it.pair;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  PairMeta* meta = a.meta + pair;
  const int len = meta->len;
  const int budget = meta->budget;
  const int slot0 = meta->slot0;

  // q of the group's heads, this lane's EPL dimensions, in the log2 domain.
  float q2[G][EPL];
  {
    const elem* qb = static_cast<const elem*>(a.q) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D + c * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x[EPL];
      unpack<T>(*reinterpret_cast<const uint4*>(qb + h * D), x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) q2[h][e] = x[e] * a.scale_log2;
    }
  }

  const size_t pair_off = (size_t)pair * a.max_budget * D;
  const elem* Kp = static_cast<const elem*>(a.k_cache) + pair_off + c * EPL;
  const elem* Vp = static_cast<const elem*>(a.v_cache) + pair_off + c * EPL;
  float* lg = a.logits + (size_t)slot0 * G;  // [G][budget]
  float* vn = a.vnorm + slot0;               // [budget]

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int row_end = min(it.start + it.count, len);
  for (int tb = it.start; tb < row_end; tb += S::kTile) {
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = tb + (wave * U + u) * RPL + r;
      if (row < row_end) {
        kr[u] = *reinterpret_cast<const uint4*>(Kp + (size_t)row * D);
        vr[u] = *reinterpret_cast<const uint4*>(Vp + (size_t)row * D);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    // S = q K^T for the tile (log2 domain); masked rows get -inf.
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = tb + (wave * U + u) * RPL + r;
      float kx[EPL];
      unpack<T>(kr[u], kx);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(q2[h][e], kx[e], p);
        s[u][h] = row_sum<LPR>(p);
      }
      if (row < row_end) {
        if (c < G) {
          float mine = s[u][0];
#pragma unroll
          for (int h = 1; h < G; ++h) mine = c == h ? s[u][h] : mine;
          lg[(size_t)c * budget + row] = mine;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) s[u][h] = -INFINITY;
      }
    }
    if (a.vl1) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = tb + (wave * U + u) * RPL + r;
        float vx[EPL];
        unpack<T>(vr[u], vx);
        float n1 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) n1 += fabsf(vx[e]);
        n1 = row_sum<LPR>(n1);
        if (c == 0 && row < row_end) vn[row] = n1;
      }
    }
    // Online softmax: rescale once per tile, then accumulate P V.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][h]);
      const float mn = fmaxf(m[h], mt);
      const float corr = fast_exp2(m[h] - mn);
      m[h] = mn;
      l[h] *= corr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= corr;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vx[EPL];
      unpack<T>(vr[u], vx);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(s[u][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e]);
      }
    }
  }

  // Merge the RPL row lineages of the wave (lanes c, c + LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float fa = fast_exp2(m[h] - mn), fb = fast_exp2(mo - mn);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * fa + ao * fb;
      }
      m[h] = mn;
    }
  }
  // Merge the waves through LDS and write this chunk's partial.
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = smem + (wave * G + h) * (D + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[c * EPL + e] = acc[h][e];
      if (c == 0) {
        dst[D] = m[h];
        dst[D + 1] = l[h];
      }
    }
  }
  __syncthreads();
  const size_t item = blockIdx.x;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, dim = idx - h * D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, smem[(w * G + h) * (D + 2) + D]);
    float sa = 0.f, sl = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* src = smem + (w * G + h) * (D + 2);
      const float f = fast_exp2(src[D] - mm);
      sa += src[dim] * f;
      sl += src[D + 1] * f;
    }
    a.part_acc[(item * G + h) * D + dim] = sa;
    if (dim == 0) {
      a.part_ml[(item * G + h) * 2] = mm;
      a.part_ml[(item * G + h) * 2 + 1] = sl;
    }
  }

  // Ticket: the last chunk of the pair to finish runs the tail.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&meta->ticket, 1u);
    s_last = prev + 1 == static_cast<unsigned>(meta->nchunk);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---------------------------------------------------------------- tail
  const int t = meta->t;
  const int nchunk = meta->nchunk, item0 = meta->item0;
  float* s_w = smem;                              // [kMaxChunks][G] chunk weights exp2(m_c - M)
  float* s_redm = s_w + kMaxChunks * G;           // [kWaves][G]
  float* s_reds = s_redm + kWaves * G;            // [kWaves][G]
  float* s_ML = s_reds + kWaves * G;              // M[G], 1/L[G], exp2(s_new - M)[G]
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(s_ML + 3 * G);  // protected-slot bitmap
  float* s_arg = reinterpret_cast<float*>(s_bits + kMaxBudget / 32);  // [kWaves] score, [kWaves] slot

  // Logit of the incoming token (every row lineage computes the same value).
  float snew[G];
  {
    const elem* knp = static_cast<const elem*>(a.k_new) + (size_t)pair * D + c * EPL;
    float kx[EPL];
    unpack<T>(*reinterpret_cast<const uint4*>(knp), kx);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(q2[h][e], kx[e], p);
      snew[h] = row_sum<LPR>(p);
    }
  }
  // Global max over chunks and the new token.
  float mc[G], lc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mc[h] = kNegBig;
    lc[h] = 0.f;
  }
  if (tid < nchunk) {
    const float* src = a.part_ml + (size_t)(item0 + tid) * G * 2;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mc[h] = src[2 * h];
      lc[h] = src[2 * h + 1];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = mc[h];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if (lane == 0) s_redm[wave * G + h] = x;
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = snew[h];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x = fmaxf(x, s_redm[w * G + h]);
    M[h] = x;
  }
  // Chunk weights and the normaliser.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float wgt = fast_exp2(mc[h] - M[h]);
    if (tid < nchunk) s_w[tid * G + h] = wgt;
    float x = lc[h] * wgt;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) s_reds[wave * G + h] = x;
  }
  __syncthreads();
  float invL[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float en = fast_exp2(snew[h] - M[h]);
    float L = en;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += s_reds[w * G + h];
    invL[h] = 1.0f / L;
    if (tid == 0) {
      s_ML[h] = M[h];
      s_ML[G + h] = invL[h];
      s_ML[2 * G + h] = en;
      if (a.dbg_lse)
        a.dbg_lse[(size_t)b * a.n_q_heads + g * G + h] = (M[h] + __log2f(L)) * 0.6931471805599453f;
    }
  }
  // Protected-slot bitmap from the ring of recent slots (the sink is an index test).
  const int nwords = (budget + 31) >> 5;
  for (int i = tid; i < nwords; i += kThreads) s_bits[i] = 0u;
  __syncthreads();
  const int R = a.recent;
  const int32_t* ring = a.ring + (size_t)pair * R;
  for (int j = tid; j < R; j += kThreads) {
    const int sl = ring[j];
    if (sl >= 0 && sl < budget) atomicOr(&s_bits[sl >> 5], 1u << (sl & 31));
  }
  // Output: merge chunk partials in chunk order, add the new token, normalise.
  {
    const elem* vnp = static_cast<const elem*>(a.v_new) + (size_t)pair * D;
    const float* pacc = a.part_acc + (size_t)item0 * G * D;
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int h = idx / D, dim = idx - h * D;
      float o = s_ML[2 * G + h] * load_elem<T>(vnp, dim);
      int ci = 0;
      for (; ci + 8 <= nchunk; ci += 8) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = pacc[(size_t)(ci + k) * G * D + idx];
#pragma unroll
        for (int k = 0; k < 8; ++k) o = fmaf(x[k], s_w[(ci + k) * G + h], o);
      }
      for (; ci < nchunk; ++ci) o = fmaf(pacc[(size_t)ci * G * D + idx], s_w[ci * G + h], o);
      store_elem<T>(a.out, ((size_t)b * a.n_q_heads + g * G + h) * D + dim, o * s_ML[G + h]);
    }
  }
  __syncthreads();
  // Importance of every filled slot and the masked argmin.
  float best = INFINITY;
  int besti = 0x7FFFFFFF;
  {
    float* dbg = a.dbg_scores ? a.dbg_scores + (size_t)pair * a.max_budget : nullptr;
    for (int i = tid; i < len; i += kThreads) {
      float sc = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) sc = fmaf(fast_exp2(lg[(size_t)h * budget + i] - M[h]), invL[h], sc);
      if (a.vl1) sc *= vn[i];
      if (dbg) dbg[i] = sc;
      const bool prot = i < a.sink || ((s_bits[i >> 5] >> (i & 31)) & 1u);
      if (!prot && sc < best) {  // i increases per thread: first index kept on ties
        best = sc;
        besti = i;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float so = __shfl_xor(best, off);
    const int io = __shfl_xor(besti, off);
    argmin_merge(best, besti, so, io);
  }
  if (lane == 0) {
    s_arg[wave] = best;
    reinterpret_cast<int*>(s_arg)[kWaves + wave] = besti;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) argmin_merge(best, besti, s_arg[w], reinterpret_cast<int*>(s_arg)[kWaves + w]);

  // Insert the incoming token: append while filling, else overwrite the victim.
  int e, ev;
  if (len < budget) {
    e = len;
    ev = -1;
  } else if (besti < budget) {
    e = besti;
    ev = besti;
  } else {
    e = -1;  // no evictable slot (prevented by init-time validation)
    ev = -2;
  }
  if (e >= 0) {
    constexpr int kVec = D * sizeof(elem) / 16;
    if (tid < 2 * kVec) {
      const int which = tid / kVec, part = tid - which * kVec;
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const elem*>(which ? a.v_new : a.k_new) +
                                                        (size_t)pair * D) + part;
      uint4* dst = reinterpret_cast<uint4*>(static_cast<elem*>(which ? a.v_cache : a.k_cache) + pair_off +
                                            (size_t)e * D) + part;
      *dst = *src;
    }
  }
  if (tid == 0) {
    if (e >= 0) {
      if (R > 0) a.ring[(size_t)pair * R + (t % R)] = e;
      meta->t = t + 1;
      meta->len = len < budget ? len + 1 : budget;
    }
    a.evict_idx[pair] = ev;
    meta->ticket = 0u;
  }
}

template <class T, int D, int G>
void launch_one(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((lf_step_kernel<T, D, G>), dim3(a.n_items), dim3(kThreads), 0, s, a);
}

using LaunchFn = void (*)(const StepArgs&, hipStream_t);

template <class T, int D>
constexpr LaunchFn kTableG[8] = {launch_one<T, D, 1>, launch_one<T, D, 2>, launch_one<T, D, 3>,
                                 launch_one<T, D, 4>, launch_one<T, D, 5>, launch_one<T, D, 6>,
                                 launch_one<T, D, 7>, launch_one<T, D, 8>};

template <class T, int D>
constexpr int kTileG[8] = {Shape<T, D, 1>::kTile, Shape<T, D, 2>::kTile, Shape<T, D, 3>::kTile,
                           Shape<T, D, 4>::kTile, Shape<T, D, 5>::kTile, Shape<T, D, 6>::kTile,
                           Shape<T, D, 7>::kTile, Shape<T, D, 8>::kTile};

}  // namespace

int tile_rows(int dtype, int head_dim, int group) {
  if (group < 1 || group > 8) return 0;
  const bool bf = dtype == 1;
  if (head_dim == 64) return bf ? kTileG<BF16T, 64>[group - 1] : kTileG<F32T, 64>[group - 1];
  if (head_dim == 128) return bf ? kTileG<BF16T, 128>[group - 1] : kTileG<F32T, 128>[group - 1];
  return 0;
}

int launch_step(int dtype, int head_dim, int group, const StepArgs& a, void* stream, char* err, size_t errlen) {
  if (a.n_items <= 0) return 0;
  LaunchFn fn = nullptr;
  const bool bf = dtype == 1;
  if (group >= 1 && group <= 8) {
    if (head_dim == 64) fn = bf ? kTableG<BF16T, 64>[group - 1] : kTableG<F32T, 64>[group - 1];
    if (head_dim == 128) fn = bf ? kTableG<BF16T, 128>[group - 1] : kTableG<F32T, 128>[group - 1];
  }
  if (!fn) {
    snprintf(err, errlen, "no kernel for dtype %d head_dim %d group %d", dtype, head_dim, group);
    return 1;
  }
  fn(a, static_cast<hipStream_t>(stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "kernel launch failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int upload_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    snprintf(err, errlen, "state upload failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace lf
