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
//    kernel is a streaming scan.  K and V rows are read with 16-byte
//    non-temporal loads straight into registers; each wave walks its quarter
//    of a chunk in 16-row groups through a ring of register buffers, every
//    load unconditional so the compiler's waits stay precise.
//  * bf16: q.k and P.V run on the matrix cores (the 16 rows of a group against
//    the group's query heads; V through an LDS tile read back transposed), the
//    online softmax in fp32 on the vector ALUs.  fp32 caches use a vector-ALU
//    path (stream_valu).
//  * Work is a static list of (pair, row range) chunks, pair = (sequence, KV
//    head); pairs are split only when there are too few of them to fill the
//    GPU.  A chunk keeps a running max / sum / weighted value sum per head
//    (log2 domain) and writes its raw logits out for the importance pass, or
//    keeps them in LDS when its own workgroup will run the pair's tail: in
//    fp32 when they fit, else in half precision, from which the tail bounds
//    every slot's importance and scores exactly, from the key rows, only the
//    slots that can still be the minimum.
//  * A pair's tail runs in the workgroup that finishes it: directly when the
//    pair is one chunk, else in the chunk that takes the last ticket
//    (device-scope stores and loads on both sides of a relaxed device-scope
//    fetch-add; the protocol is described at store_wt).  The tail merges the
//    partials in chunk order, adds the incoming token, writes the output,
//    computes the importance of every slot from the stored logits with the
//    global max / normaliser (exactly; or bounded, then exact for the possible
//    minima), takes the lexicographic (score, slot) argmin
//    outside the sink slots and the ring of recent slots, and copies k_new /
//    v_new into the victim slot.  No other workgroup reads the pair after its
//    ticket, so the in-place write cannot race with a reader.
//  * Cross-lane reductions use DPP and lane swaps; every reduction has a fixed
//    order, so results are bit-reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "lf_internal.h"

namespace lf {
namespace {

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so empty partials merge without NaN
constexpr int kWaves = kThreads / 64;
// Where a pair's logits are when its tail runs: written out to the workspace,
// or kept in the streaming waves' LDS buffers (an unsplit pair, bf16), in fp32
// when each wave's range fits kLogitRows rows, else in half precision up to
// twice that (the tail then bounds every slot's importance from the half
// values and recomputes the few slots that could be the minimum exactly from
// their K rows).
constexpr int kLogitsOut = 0, kLogitsFull = 1, kLogitsHalf = 2;
constexpr int kCandCap = 256;  // exactly recomputed candidates per pair before the fallback

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
  static constexpr int kU = 4;            // row loads per lane per tile per tensor (double-buffered)
  static constexpr int kTile = kEpl == 8 ? 16 * kWaves : kWaves * kRpl * kU;
  // LDS: merged chunk partial [G][D + 2] kept for the tail, then a region used
  // first for the cross-wave merge [wave][G][D + 2], V staging and the logit
  // buffers, and later by the tail.
  static constexpr int kPartFloats = G * (D + 2);
  static constexpr int kMergeFloats = kWaves * G * (D + 2);
  // Tail scratch after the merge area: bitmap of protected slots, then the
  // per-wave argmin candidates, the per-wave upper bounds, the candidate count
  // and list of half-precision resident pairs (bf16: inside the V staging area).
  static constexpr int kBitsOffset = kMergeFloats;
  static constexpr int kTailFloats = kBitsOffset + kMaxBudget / 32 + 2 * kWaves + kWaves + 1 + kCandCap;
  // bf16: per-wave tile of 16 value rows, rows padded by 32 bytes against LDS bank conflicts.
  static constexpr int kStageRowBytes = D * 2 + 32;
  static constexpr int kStageFloats = kEpl == 8 ? kWaves * 16 * kStageRowBytes / 4 : 0;
  // bf16: per-wave logit buffer [G][kLogitRows], written out in kLogitRows-row
  // runs.  Logit stores leaving the chip interleave DRAM writes with the K/V
  // read stream and cost far more than their bytes, in proportion to the
  // number of runs rather than their size: against 128-row runs, 512-row runs
  // take the throughput shape (B64, budget 4096) from 212 to 180 us per step,
  // 1024-row runs the ragged shape (budgets up to 8192) from 530 to 448 us, at
  // the price of one workgroup per compute unit for G = 5.  Unsplit pairs write
  // nothing when their logits fit the buffers (fp32) or twice them (half
  // precision), so for G <= 4 512 rows suffice for budgets up to 4096 and leave
  // room for two workgroups per compute unit, one's tail overlapping the
  // other's stream (B64 budget 4096: 165.8 -> 162.4 us; B8 budget 2048 split
  // four ways: 19.0 -> 18.6 us).
  static constexpr int kLogitRows = G <= 4 ? 512 : G <= 5 ? 1024 : 256;
  static constexpr int kLogitFloats = kEpl == 8 ? kWaves * G * kLogitRows : 0;
  static constexpr int kStreamFloats = kMergeFloats + kStageFloats + kLogitFloats;
  // bf16: the tail's inputs that do not depend on the stream (the group's q,
  // k_new and v_new rows, the ring of recent slots) are copied to LDS when the
  // workgroup starts (LDS DMA, no registers held), in 1 KB blocks of 16-byte
  // cells, then up to kPreRing ring entries.
  static constexpr int kPreCells = kEpl == 8 ? (G + 2) * D / 8 : 0;
  static constexpr int kPreBlocks = (kPreCells + 63) / 64;
  static constexpr int kPreRing = kEpl == 8 ? 256 : 0;
  static constexpr int kPreFloats = kPreBlocks * 256 + kPreRing;
  static constexpr int kSmemFloats =
      kPartFloats + (kStreamFloats > kTailFloats ? kStreamFloats : kTailFloats) + kPreFloats;
  // Waves per SIMD the register budget is sized for: bf16 workgroups that fit
  // 3+ per compute unit by LDS get 3 (168 VGPRs), those that fit only fewer
  // get registers to match.
  static constexpr int kBlocksByLds = (160 * 1024) / (kSmemFloats * 4);
  static constexpr int kMinWavesPerSimd = kEpl != 8 ? 1 : kBlocksByLds >= 3 ? 3 : kBlocksByLds < 1 ? 1 : kBlocksByLds;
  // K/V groups in flight per wave in the streaming loop (current one
  // included).  A third where one wave per SIMD leaves the registers for it
  // and it was measured to pay: with G = 4 it does (2 % at 4096-slot pairs),
  // with G = 5 (and 4 stages for G = 4) it cost about 1 %.
  static constexpr int kStages = kMinWavesPerSimd == 1 && G <= 4 ? 3 : 2;
  // The tail's scratch fits in the merge and staging areas, so the logit
  // buffers survive into the tail (see kLogitsFull and kLogitsHalf).
  static_assert(kEpl != 8 || kTailFloats <= kMergeFloats + kStageFloats, "tail scratch overlaps logit buffers");
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

// Reduction within each row of 16 lanes (every lane of the row gets it).
template <class Op>
__device__ __forceinline__ float row_reduce16(float x, Op op) {
  x = op(x, dpp<0xB1>(x));
  x = op(x, dpp<0x4E>(x));
  x = op(x, dpp<0x141>(x));
  return op(x, dpp<0x140>(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Non-temporal (streaming) 16- and 8-byte loads.
// The wave's index in the workgroup, in a scalar register: loop bounds
// derived from it then stay scalar and their loops use scalar branches.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(x[0], x[1]);
}

// Data one workgroup hands to another in the same launch (logits and the
// chunk partials of a split pair) moves only through device-scope stores and
// loads: relaxed agent-scope atomics, or buffer stores and loads with the same
// "sc1" cache policy (on gfx950: written through the non-coherent per-XCD L2
// to memory, and read past it).  Each chunk drains its
// stores (s_waitcnt vmcnt(0): a device-scope store has then reached memory)
// before its thread 0 increments the pair's ticket with a device-scope RMW, and
// the chunk that takes the last ticket reads the others' data with
// device-scope loads issued after that RMW returned.  This is the ordering a
// release/acquire pair would give, without the L2 write-back and invalidate
// that only plain (non-atomic) stores and loads need.
__device__ __forceinline__ void store_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_wt(float2* p, float2 v) {
  const unsigned long long x =
      (unsigned long long)__float_as_uint(v.x) | ((unsigned long long)__float_as_uint(v.y) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-scope store through a buffer resource over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_wt4(__amdgpu_buffer_rsrc_t r, int byte_off, float4 v) {
  typedef unsigned u32x4_t __attribute__((vector_size(16)));
  const u32x4_t x = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, byte_off, 0, 16 /* sc1 */);
}
// Device-scope loads through a buffer resource over [base, base + bytes)
// ("sc1", the policy of a relaxed agent-scope atomic load, as wide as needed).
// A load outside the range returns 0 and touches no memory, so the tail issues
// its loads unconditionally (a load under a branch makes later waits drain
// every load in flight) and gives an empty range where the data is not needed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ float load_c1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 16 /* sc1 */));
}
__device__ __forceinline__ float2 load_c2(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 16 /* sc1 */);
  return make_float2(__uint_as_float(x[0]), __uint_as_float(x[1]));
}
__device__ __forceinline__ float4 load_c4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
  return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The group's q for this lane's dimensions.  bf16: raw packed pairs (logits are
// scaled after the dot); fp32: values pre-multiplied by scale * log2(e).
template <class T, int G>
struct QReg {
  uint32_t w[G][4];
};
template <int G>
struct QReg<F32T, G> {
  float x[G][4];
};

template <class T, int G>
__device__ __forceinline__ void load_q(QReg<T, G>& q, const typename T::elem* qb, int D, float scale_log2) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 r = *reinterpret_cast<const uint4*>(qb + h * D);
    if constexpr (T::kEpl == 8) {
      q.w[h][0] = r.x;
      q.w[h][1] = r.y;
      q.w[h][2] = r.z;
      q.w[h][3] = r.w;
    } else {
      q.x[h][0] = __uint_as_float(r.x) * scale_log2;
      q.x[h][1] = __uint_as_float(r.y) * scale_log2;
      q.x[h][2] = __uint_as_float(r.z) * scale_log2;
      q.x[h][3] = __uint_as_float(r.w) * scale_log2;
    }
  }
}

// This lane's part of q_h . k (before the row reduction and, for bf16, before scaling).
template <class T, int G>
__device__ __forceinline__ float qk_part(const QReg<T, G>& q, int h, const uint4& k) {
  if constexpr (T::kEpl == 8) {
    float p = dot2_bf16(q.w[h][0], k.x, 0.f);
    p = dot2_bf16(q.w[h][1], k.y, p);
    p = dot2_bf16(q.w[h][2], k.z, p);
    return dot2_bf16(q.w[h][3], k.w, p);
  } else {
    float p = q.x[h][0] * __uint_as_float(k.x);
    p = fmaf(q.x[h][1], __uint_as_float(k.y), p);
    p = fmaf(q.x[h][2], __uint_as_float(k.z), p);
    return fmaf(q.x[h][3], __uint_as_float(k.w), p);
  }
}

// (score, slot) lexicographic minimum of two candidates.
__device__ __forceinline__ void argmin_merge(float& s, int& i, float so, int io) {
  const bool lt = so < s || (so == s && io < i);  // selects, no branch
  s = lt ? so : s;
  i = lt ? io : i;
}

// Copies a pair's tail inputs to s_pre with LDS DMA (wave 0 of a bf16
// workgroup, at its start): q of the group [G][D], then the k_new and v_new
// rows, in 16-byte cells; then ring entries (4-byte cells).  Lanes past the
// end load a clamped valid cell into padding that nobody reads.
template <int D, int G>
__device__ void prefetch_tail(const StepArgs& a, int pair, float* s_pre) {
  using S = Shape<BF16T, D, G>;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  constexpr int QC = G * D / 8, KC = D / 8, NC = S::kPreCells;
  const int lane = threadIdx.x & 63;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
  const uint16_t* kr = static_cast<const uint16_t*>(a.k_new) + (size_t)pair * D;
  const uint16_t* vr = static_cast<const uint16_t*>(a.v_new) + (size_t)pair * D;
#pragma unroll
  for (int blk = 0; blk < S::kPreBlocks; ++blk) {
    const int c = min(blk * 64 + lane, NC - 1);
    const uint16_t* src = c < QC ? qg + 8 * c : c < QC + KC ? kr + 8 * (c - QC) : vr + 8 * (c - QC - KC);
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)(s_pre + blk * 256), 16, 0, 0);
  }
  const int R = a.recent;
  if (R > 0) {
    const int32_t* ring = a.ring + (size_t)pair * R;
    float* s_ring = s_pre + S::kPreBlocks * 256;
#pragma unroll
    for (int blk = 0; blk < S::kPreRing / 64; ++blk)
      if (blk * 64 < R)
        __builtin_amdgcn_global_load_lds(ring + min(blk * 64 + lane, R - 1), (lds_ptr)(s_ring + blk * 64),
                                         4, 0, 0);
  }
}

// LDS bitmap of the pair's protected recent slots (the ring's entries) over
// its budget, built before the tail: cleared while the chunk partials merge,
// then set during the ticket's round trip (a barrier between the two).
__device__ __forceinline__ void clear_protect_bits(uint32_t* bits, int budget) {
  for (int i = threadIdx.x; i < (budget + 31) >> 5; i += kThreads) bits[i] = 0u;
}
template <class T, int D, int G>
__device__ void set_protect_bits(const StepArgs& a, int pair, int budget, uint32_t* bits, const float* s_pre) {
  const int R = a.recent, tid = threadIdx.x;
  const int32_t* ring = a.ring + (size_t)pair * R;
  // bf16: the first entries were copied to LDS when the workgroup started.
  const int32_t* first =
      T::kEpl == 8 ? reinterpret_cast<const int32_t*>(s_pre + Shape<T, D, G>::kPreBlocks * 256) : ring;
  if (tid < R) {
    const int sl = first[tid];
    if (sl >= 0 && sl < budget) atomicOr(&bits[sl >> 5], 1u << (sl & 31));
  }
  for (int j = tid + kThreads; j < R; j += kThreads) {
    const int sl = ring[j];
    if (sl >= 0 && sl < budget) atomicOr(&bits[sl >> 5], 1u << (sl & 31));
  }
}

// Wave-wide lexicographic (score, slot) minimum; every lane gets the result.
__device__ __forceinline__ void wave_argmin(float& s, int& i) {
  auto step = [&](float so, int io) { argmin_merge(s, i, so, io); };
#define LF_DPP_STEP(CTRL) step(dpp<CTRL>(s), __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false))
  LF_DPP_STEP(0xB1);
  LF_DPP_STEP(0x4E);
  LF_DPP_STEP(0x141);
  LF_DPP_STEP(0x140);
#undef LF_DPP_STEP
  step(__int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), 0x401F)), __builtin_amdgcn_ds_swizzle(i, 0x401F));
  const auto ss = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  const auto si = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(i), static_cast<unsigned>(i), false, false);
  float s0 = __uint_as_float(ss[0]);
  int i0 = static_cast<int>(si[0]);
  argmin_merge(s0, i0, __uint_as_float(ss[1]), static_cast<int>(si[1]));
  s = s0;
  i = i0;
}

// Tail of one pair: merge chunk partials, output, importance, argmin, insert.
// Every workspace load (chunk statistics and partials, the first logits) is
// issued at once at the start, so the tail costs about one memory round trip
// plus arithmetic; the new token's rows and the ring are already in LDS
// (s_pre) and the bitmap of protected slots was built before the tail.
// s_part: this workgroup's merged partial ([G][D + 2], used when nchunk == 1);
// s_tail: the region after the merge area holds the bitmap and the argmin
// candidates (Shape::kBitsOffset).
template <class T, int D, int G>
__device__ void pair_tail(const StepArgs& a, int pair, const PairMeta& pm, const float* s_part, float* s_tail,
                          const float* s_logit, int lmode, const float* s_pre) {
  using elem = typename T::elem;
  constexpr int kOut = (G * D + kThreads - 1) / kThreads;  // output elements per thread
  constexpr int kCB = G <= 4 ? 8 : 4;                       // chunk partials loaded per batch
  constexpr int kVec = D * sizeof(elem) / 16;               // 16-byte pieces of one K/V row
  // float4 logit cells per head preloaded (more when the register budget is
  // sized for one wave per SIMD).  Every cell past the budget is a wasted
  // load in the tail's first round trip: 2048 slots for G = 3, 4 and 1024
  // for G >= 5 cover the split shapes measured (B8 budget 2048 G 4: 18.43 ->
  // 18.26 us against twice as many; B16 budget 1024 G 7: 14.80 -> 14.62 us).
  constexpr int kPre = Shape<T, D, G>::kMinWavesPerSimd == 1 ? 32 / G : (G <= 2 ? 8 : 8 / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  PairMeta* meta = a.meta + pair;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const int t = pm.t, len = pm.len, budget = pm.budget;
  const int nchunk = pm.nchunk, item0 = pm.item0, lstride = pm.lstride;
  const int R = a.recent;
  const int ring_pos = R > 0 ? t % R : 0;  // ring entry the incoming token takes
  const bool split = nchunk > 1;
  const size_t pair_off = (size_t)pair * a.max_budget * D;

  const uint32_t* s_bits = reinterpret_cast<const uint32_t*>(s_tail + Shape<T, D, G>::kBitsOffset);  // protected slots
  float* s_arg = s_tail + Shape<T, D, G>::kBitsOffset + kMaxBudget / 32;  // [kWaves] score, [kWaves] slot

  // ---- loads that depend on nothing computed here.  Addresses are clamped to
  // valid memory and nothing is branched around, so the loads issue back to
  // back and one wait covers them; out-of-range lanes are masked where used.
  using S = Shape<T, D, G>;
  constexpr int EPL = S::kEpl, LPR = S::kLpr;
  // bf16: q, k_new, v_new and the first ring entries were copied to s_pre when
  // the workgroup started (prefetch_tail).
  constexpr bool kPre16 = T::kEpl == 8;
  const elem* pre = reinterpret_cast<const elem*>(s_pre);
  const elem* qsrc = kPre16 ? pre : static_cast<const elem*>(a.q) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
  const elem* knsrc = kPre16 ? pre + G * D : static_cast<const elem*>(a.k_new) + (size_t)pair * D;
  const elem* vnsrc = kPre16 ? pre + (G + 1) * D : static_cast<const elem*>(a.v_new) + (size_t)pair * D;
  QReg<T, G> q;
  uint4 kn;
  {
    const int c = lane % LPR;
    load_q<T, G>(q, qsrc + c * EPL, D, a.scale_log2);
    kn = *reinterpret_cast<const uint4*>(knsrc + c * EPL);
  }
  // Chunk partials exist only for a split pair; logits are read from memory
  // unless the pair kept them in LDS.
  const auto ml_rs = coh_rsrc(a.part_ml + (size_t)item0 * G * 2, split ? nchunk * G * 8 : 0);
  const auto pa_rs = coh_rsrc(a.part_acc + (size_t)item0 * G * D, split ? nchunk * G * D * 4 : 0);
  const auto lg_rs = coh_rsrc(a.logits + (size_t)pm.slot0 * G, lmode != kLogitsOut || a.score_none ? 0 : G * lstride * 4);
  uint4 ins;
  {
    const int c = min(tid, 2 * kVec - 1), which = c / kVec, part = c - which * kVec;
    ins = reinterpret_cast<const uint4*>(which ? vnsrc : knsrc)[part];
  }
  const elem* vnp = vnsrc;
  float vnv[kOut];
#pragma unroll
  for (int o = 0; o < kOut; ++o) vnv[o] = load_elem<T>(vnp, min(tid + o * kThreads, G * D - 1) % D);
  // bf16 streaming stores raw q.k, fp32 streaming log2-domain logits; with VL1
  // both store the log2-domain logit plus log2 |v|_1 of the slot, so the
  // weight-times-norm product is one exp2.
  const float ls = T::kEpl == 8 && !a.vl1 ? a.scale_log2 : 1.0f;
  auto logit4 = [&](int h, int base) { return load_c4(lg_rs, (h * lstride + base) * 4); };
  // Every workspace value the tail needs first is requested here at once: the
  // chunk partials and the first kPre * 4 * kThreads slots' logits (all of
  // them for budgets up to that).  A pair that kept its logits in LDS needs
  // none of them: it skips the block, which leaves its waits below with
  // nothing to wait for.
  // Chunk statistics, packed: lane 16 r + c holds, for pass k, head 4 k + r of
  // chunks c, c + 16, c + 32, c + 48 (j = 0..3).
  constexpr int KP = (G + 3) / 4;
  const int prow = lane >> 4, pcol = lane & 15;
  float2 ml[KP][4];
  float pa[kOut][kCB];
  float4 lvp[kPre][G];
  if (lmode == kLogitsOut) {
#pragma unroll
    for (int k = 0; k < KP; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) ml[k][j] = load_c2(ml_rs, ((pcol + 16 * j) * G + min(4 * k + prow, G - 1)) * 8);
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
      const int idx = min(tid + o * kThreads, G * D - 1);
#pragma unroll
      for (int k = 0; k < kCB; ++k) pa[o][k] = load_c1(pa_rs, (k * G * D + idx) * 4);
    }
#pragma unroll
    for (int p = 0; p < kPre; ++p) {
      const int base = min(4 * (tid + p * kThreads), lstride - 4);
#pragma unroll
      for (int h = 0; h < G; ++h) lvp[p][h] = logit4(h, base);
    }
  } else {
#pragma unroll
    for (int k = 0; k < KP; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) ml[k][j] = make_float2(0.f, 0.f);
#pragma unroll
    for (int o = 0; o < kOut; ++o)
#pragma unroll
      for (int k = 0; k < kCB; ++k) pa[o][k] = 0.f;
  }
  // ---- global max and normaliser over the chunks and the incoming token.
  // Every wave computes them itself, lane c holding chunk c (the own merged
  // partial in lane 0 for an unsplit pair): no LDS exchange, no barrier.  The
  // reductions give every lane, and every wave, the same bits.
  // Logit of the incoming token (every lane of a row lineage holds it).
  float snew[G];
  {
    const float post_scale = T::kEpl == 8 ? a.scale_log2 : 1.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) snew[h] = row_sum<LPR>(qk_part<T, G>(q, h, kn)) * post_scale;
  }
  // Row reductions (16 lanes) over the packed chunk statistics: one pass
  // serves four heads.  Results are read back per head with readlane, so every
  // wave holds the same values.
  float M[G], invL[G], en[G];
  float wp[KP][4];  // lane (r, c), slot j: weight exp2(m - M) of chunk c + 16 j for head 4 k + r
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int h = 4 * k + prow;
    float sn = snew[0];
#pragma unroll
    for (int hh = 1; hh < G; ++hh) sn = h == hh ? snew[hh] : sn;
    float mcj[4], lcj[4];
    float mx = kNegBig;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = pcol + 16 * j;
      const bool own = h < G && (split ? c < nchunk : c == 0);
      mcj[j] = own ? (split ? ml[k][j].x : s_part[min(h, G - 1) * (D + 2) + D]) : kNegBig;
      lcj[j] = own ? (split ? ml[k][j].y : s_part[min(h, G - 1) * (D + 2) + D + 1]) : 0.f;
      mx = fmaxf(mx, mcj[j]);
    }
    const float Mh = fmaxf(row_reduce16(mx, [](float u, float v) { return fmaxf(u, v); }), sn);
    float ls4 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wp[k][j] = fast_exp2(mcj[j] - Mh);  // 0 without a chunk
      ls4 = fmaf(lcj[j], wp[k][j], ls4);
    }
    const float enh = fast_exp2(sn - Mh);
    const float Lh = row_reduce16(ls4, [](float u, float v) { return u + v; }) + enh;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * k + r < G) {
        M[4 * k + r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Mh), 16 * r));
        en[4 * k + r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(enh), 16 * r));
        const float L = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Lh), 16 * r));
        invL[4 * k + r] = 1.0f / L;
        if (tid == 0 && a.dbg_lse)
          a.dbg_lse[(size_t)b * a.n_q_heads + g * G + 4 * k + r] = (M[4 * k + r] + __log2f(L)) * 0.6931471805599453f;
      }
    }
  }

  // ---- output: chunk partials in chunk order + the new token, normalised
#pragma unroll
  for (int o = 0; o < kOut; ++o) {
    const int idx = tid + o * kThreads;
    if (idx < G * D) {
      const int h = idx / D;
      // h is the same on the whole wave (D is a multiple of 64), so lane c's
      // weight for head h is chunk c's, read with readlane.
      float enh = en[0], il = invL[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh) {
        enh = h == hh ? en[hh] : enh;
        il = h == hh ? invL[hh] : il;
      }
      // Chunk c's weight for head h: lane 16 (h % 4) + c % 16, slot c / 16, pass h / 4.
      float wj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wj[j] = wp[0][j];
#pragma unroll
        for (int k = 1; k < KP; ++k) wj[j] = (h >> 2) == k ? wp[k][j] : wj[j];
      }
      const int wbase = 16 * (h & 3);
      auto wchunk = [&](int c) {
        const float w = (c >> 4) == 0 ? wj[0] : (c >> 4) == 1 ? wj[1] : (c >> 4) == 2 ? wj[2] : wj[3];
        return __builtin_amdgcn_readlane(__float_as_int(w), wbase + (c & 15));
      };
      float acc = enh * vnv[o];
      if (!split) {
        acc = fmaf(s_part[h * (D + 2) + idx - h * D], __int_as_float(wchunk(0)), acc);
      } else {
#pragma unroll
        for (int k = 0; k < kCB; ++k)
          if (k < nchunk) acc = fmaf(pa[o][k], __int_as_float(wchunk(k)), acc);
        for (int ci = kCB; ci < nchunk; ci += kCB) {
          float x[kCB];
#pragma unroll
          for (int k = 0; k < kCB; ++k) x[k] = load_c1(pa_rs, ((ci + k) * G * D + idx) * 4);
#pragma unroll
          for (int k = 0; k < kCB; ++k)
            if (ci + k < nchunk) acc = fmaf(x[k], __int_as_float(wchunk(ci + k)), acc);
        }
      }
      store_elem<T>(a.out, ((size_t)b * a.n_q_heads + g * G + h) * D + idx - h * D, acc * il);
    }
  }

  // ---- importance of every filled slot and the masked first-index argmin
  float best = INFINITY;
  int besti = 0x7FFFFFFF;
  // Without importance (score_none) there is no candidate: besti stays past
  // every slot, so a full cache stores nothing.
  if (!a.score_none) {
    float* dbg = a.dbg_scores ? a.dbg_scores + (size_t)pair * a.max_budget : nullptr;
    auto score4 = [&](int base, const float4(&lv)[G]) {
      const uint32_t bits = s_bits[base >> 5] >> (base & 31);
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sc[0] = fmaf(fast_exp2(fmaf(lv[h].x, ls, -M[h])), invL[h], sc[0]);
        sc[1] = fmaf(fast_exp2(fmaf(lv[h].y, ls, -M[h])), invL[h], sc[1]);
        sc[2] = fmaf(fast_exp2(fmaf(lv[h].z, ls, -M[h])), invL[h], sc[2]);
        sc[3] = fmaf(fast_exp2(fmaf(lv[h].w, ls, -M[h])), invL[h], sc[3]);
      }
      if (dbg) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (base + j < len) dbg[base + j] = sc[j];
      }
      // Branch-free masked minimum; i increases per thread, so the strict
      // comparison keeps the first index on ties.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j;
        const bool ok = i < len && i >= a.sink && !((bits >> j) & 1u);
        const float v = ok ? sc[j] : INFINITY;
        const bool lt = v < best;
        best = lt ? v : best;
        besti = lt ? i : besti;
      }
    };
    // Exact importance of slot i from its key row, on the LPR lanes of one row
    // lineage (every lane of the lineage gets the same value).
    // (key_row issues the loads, exact_score takes them, so that several
    // slots' loads can be in flight together.)
    // With VL1 the value row is loaded too and its |v|_1 taken the stream's way.
    struct KeyRow {
      uint4 k, v;
    };
    auto key_row = [&](int i) {
      const size_t off = pair_off + (size_t)i * D + (lane % LPR) * EPL;
      KeyRow kr;
      kr.k = *reinterpret_cast<const uint4*>(static_cast<const elem*>(a.k_cache) + off);
      kr.v = *reinterpret_cast<const uint4*>(static_cast<const elem*>(a.v_cache) + off);
      return kr;
    };
    auto exact_score = [&](const KeyRow& kr) {
      const float post_scale = T::kEpl == 8 ? a.scale_log2 : 1.0f;
      float sc = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
        sc = fmaf(fast_exp2(row_sum<LPR>(qk_part<T, G>(q, h, kr.k)) * post_scale - M[h]), invL[h], sc);
      if (a.vl1) {
        float vx[EPL];
        unpack<T>(kr.v, vx);
        float n1 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) n1 += fabsf(vx[e]);
        sc *= row_sum<LPR>(n1);
      }
      return sc;
    };
    if (lmode == kLogitsFull) {
      // Every logit of the pair is still in the streaming waves' LDS buffers:
      // slot s of wave w = s / quarter sits at row s - w * quarter of its buffer
      // (the wave ranges of the stream: the item is [0, budget)).
      constexpr int LR = Shape<T, D, G>::kLogitRows;
      const int quarter = ((budget + kWaves - 1) / kWaves + 15) & ~15;
#pragma unroll 4
      for (int base = 4 * tid; base < len; base += 4 * kThreads) {
        int w = 0;  // base / quarter, by comparisons
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) w += base >= ww * quarter;
        const float* src = s_logit + w * G * LR + (base - w * quarter);
        float4 lv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lv[h] = *reinterpret_cast<const float4*>(src + h * LR);
        score4(base, lv);
      }
    } else if (lmode == kLogitsHalf) {
      if constexpr (T::kEpl == 8) {
        // The streaming waves kept half-precision log2-domain logits (same
        // layout as above, 2 LR rows per head).  Pass 1 bounds every eligible
        // slot's importance from them; the slots whose lower bound is not
        // above the smallest upper bound are the only possible minima, and
        // only they are scored exactly from their key rows.
        constexpr int LR = Shape<T, D, G>::kLogitRows;
        constexpr int kCells = 2 * LR * kWaves / (4 * kThreads);  // float4 cells per thread
        static_assert(kCells * 4 <= 32, "eligibility mask");
        const int quarter = ((budget + kWaves - 1) / kWaves + 15) & ~15;
        const _Float16* lb16 = reinterpret_cast<const _Float16*>(s_logit);
        float* s_ub = s_arg + 2 * kWaves;                           // [kWaves]
        int* s_ncand = reinterpret_cast<int*>(s_ub + kWaves);      // [1]
        int* s_cand = s_ncand + 1;                                 // [kCandCap]
        typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
        // A half value x differs from the fp32 logit by at most |x| 2^-11
        // (subnormals: 2^-25), and that logit from the exact recomputation by
        // a few fp32 roundings; every exp2 argument is therefore within
        // E = max_h |x_h| 2^-11 (1 + 2^-8) + 2^-10 of the exact one, and the
        // importance v within the factors 2^-E >= 1 - E and 2^E <= 1 + E (E <= 1).
        // Logits of magnitude 2040 and above (infinite, NaN) give no bound:
        // the slot is always a candidate.  Cells past the filled slots are
        // skipped (the test is the same on the whole workgroup).
        float lo[kCells][4] = {};
        uint32_t okm = 0;
        float ub = INFINITY;
#pragma unroll
        for (int p = 0; p < kCells; ++p) {
          if (4 * p * kThreads >= len) continue;
          const int base = 4 * (tid + p * kThreads);
          int w = 0;
#pragma unroll
          for (int ww = 1; ww < kWaves; ++ww) w += base >= ww * quarter;
          const _Float16* src = lb16 + w * G * 2 * LR + min(base - w * quarter, 2 * LR - 4);
          float sc[4] = {0.f, 0.f, 0.f, 0.f}, ex[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const half4_t x = *reinterpret_cast<const half4_t*>(src + h * 2 * LR);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const float xf = (float)x[jj];
              sc[jj] = fmaf(fast_exp2(xf - M[h]), invL[h], sc[jj]);
              ex[jj] = fmaxf(ex[jj], fabsf(xf));
            }
          }
          const uint32_t bits = s_bits[min(base, kMaxBudget - 32) >> 5] >> (base & 31);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int i = base + jj;
            const bool ok = i < len && i >= a.sink && !((bits >> jj) & 1u);
            const float v = sc[jj];
            const bool wild = !(ex[jj] < 2040.f);
            const float E = fmaf(ex[jj], 0x1.01p-11f, 0x1p-10f);
            const float up = wild ? INFINITY : fmaf(v, E, v);
            lo[p][jj] = wild ? 0.f : fmaf(-v, E, v);
            ub = ok ? fminf(ub, up) : ub;
            okm |= (ok ? 1u : 0u) << (4 * p + jj);
          }
        }
        {
          int dummy = 0;
          wave_argmin(ub, dummy);
        }
        if (lane == 0) s_ub[wave] = ub;
        if (tid == 0) *s_ncand = 0;
        __syncthreads();
        float U = s_ub[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) U = fminf(U, s_ub[w]);
#pragma unroll
        for (int p = 0; p < kCells; ++p)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (((okm >> (4 * p + jj)) & 1u) && lo[p][jj] <= U) {
              const int k = atomicAdd(s_ncand, 1);
              if (k < kCandCap) s_cand[k] = 4 * (tid + p * kThreads) + jj;
            }
        __syncthreads();
        const int ncand = *s_ncand;
        constexpr int RPL = 64 / LPR;  // slots per wave per pass
        const int r = lane / LPR;
        if (ncand == 1 && !dbg) {
          // The minimum is always a candidate (its lower bound is not above
          // its score, which is not above the smallest upper bound), and an
          // exact tie with it would be one too: a single candidate is the
          // argmin, and its score is not needed.
          best = 0.f;
          besti = s_cand[0];
        } else if (ncand <= kCandCap && !dbg) {
          for (int j0 = wave * RPL; j0 < ncand; j0 += kWaves * RPL) {
            const int jc = j0 + r;
            const int i = s_cand[min(jc, ncand - 1)];
            const float v = exact_score(key_row(i));
            argmin_merge(best, besti, jc < ncand ? v : INFINITY, jc < ncand ? i : 0x7FFFFFFF);
          }
        } else {
          // Too many candidates (near-equal importances), or every score is
          // asked for: exact scores of all filled slots.
          // Four rows per lane lineage in flight; per lane the slots
          // increase, but the merge keeps the first index on ties anyway.
          constexpr int kU = 4;
          for (int i0 = wave * RPL * kU; i0 < len; i0 += kWaves * RPL * kU) {
            KeyRow kr[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) kr[u] = key_row(min(i0 + u * RPL + r, len - 1));
#pragma unroll
            for (int u = 0; u < kU; ++u) {
              const int i = i0 + u * RPL + r;
              const float v = exact_score(kr[u]);
              if (dbg && lane % LPR == 0 && i < len) dbg[i] = v;
              const bool ok = i < len && i >= a.sink && !((s_bits[min(i, len - 1) >> 5] >> (i & 31)) & 1u);
              argmin_merge(best, besti, ok ? v : INFINITY, ok ? i : 0x7FFFFFFF);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < kPre; ++p)
        if (4 * (tid + p * kThreads) < len)
          score4(4 * (tid + p * kThreads), lvp[p]);
#pragma unroll 2
      for (int base = 4 * (tid + kPre * kThreads); base < len; base += 4 * kThreads) {
        float4 lv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lv[h] = logit4(h, base);
        score4(base, lv);
      }
    }
    wave_argmin(best, besti);
    if (lane == 0) {
      s_arg[wave] = best;
      reinterpret_cast<int*>(s_arg)[kWaves + wave] = besti;
    }
    __syncthreads();
    {
      float sw[kWaves];
      int iw[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {  // all reads first, one wait
        sw[w] = s_arg[w];
        iw[w] = reinterpret_cast<int*>(s_arg)[kWaves + w];
      }
#pragma unroll
      for (int w = 0; w < kWaves; ++w) argmin_merge(best, besti, sw[w], iw[w]);
    }
  }

  // ---- insert the incoming token: append while filling, else overwrite the victim
  int e, ev;
  if (len < budget) {
    e = len;
    ev = -1;
  } else if (besti < budget) {
    e = besti;
    ev = besti;
  } else {
    e = -1;  // not stored: score_none on a full cache (no evictable slot is prevented by validation)
    ev = -2;
  }
  if (e >= 0 && tid < 2 * kVec) {
    const int which = tid / kVec, part = tid - which * kVec;
    reinterpret_cast<uint4*>(static_cast<elem*>(which ? a.v_cache : a.k_cache) + pair_off + (size_t)e * D)[part] =
        ins;
  }
  if (tid == 0) {
    if (e >= 0) {
      if (R > 0) a.ring[(size_t)pair * R + ring_pos] = e;
      meta->t = t + 1;
      meta->len = len < budget ? len + 1 : budget;
    }
    a.evict_idx[pair] = ev;
    meta->ticket = 0u;
  }
}

// Streaming of one chunk on the vector ALUs (fp32 cache): 16-byte loads of one
// row segment per lane, q.k on the lane's segment + DPP row sum, online softmax
// per row lineage, P.V by FMA.  Leaves the wave's partial (max, sum, weighted
// value sum per head) in s_merge[wave][G][D + 2].
template <class T, int D, int G>
__device__ void stream_valu(const StepArgs& a, int pair, int start, int row_end, float* lg, int lstride,
                            float* s_merge) {
  using S = Shape<T, D, G>;
  constexpr int EPL = S::kEpl, LPR = S::kLpr, RPL = S::kRpl, U = S::kU, TILE = S::kTile;
  using elem = typename T::elem;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int r = lane / LPR, c = lane % LPR;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  QReg<T, G> q;
  load_q<T, G>(q, static_cast<const elem*>(a.q) + ((size_t)b * a.n_q_heads + (size_t)g * G) * D + c * EPL, D,
               a.scale_log2);
  const float post_scale = T::kEpl == 8 ? a.scale_log2 : 1.0f;
  const size_t pair_off = (size_t)pair * a.max_budget * D;
  const elem* Kp = static_cast<const elem*>(a.k_cache) + pair_off + c * EPL;
  const elem* Vp = static_cast<const elem*>(a.v_cache) + pair_off + c * EPL;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int lane_row = wave * U * RPL + r;  // row of load u = 0 within a tile

  auto load_tile = [&](int tb, uint4(&kk)[U], uint4(&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = tb + lane_row + u * RPL;
      if (row < row_end) {
        kk[u] = *reinterpret_cast<const uint4*>(Kp + (size_t)row * D);
        vv[u] = *reinterpret_cast<const uint4*>(Vp + (size_t)row * D);
      } else {
        kk[u] = make_uint4(0, 0, 0, 0);
        vv[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto process_tile = [&](int tb, const uint4(&kk)[U], const uint4(&vv)[U]) {
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = tb + lane_row + u * RPL;
#pragma unroll
      for (int h = 0; h < G; ++h) s[u][h] = row_sum<LPR>(qk_part<T, G>(q, h, kk[u])) * post_scale;
      // With VL1 the stored logit carries log2 |v|_1 of the row (weight times
      // norm = exp2 of the sum), so no norm is stored apart.
      float lnorm = 0.f;
      if (a.vl1) {
        float vx[EPL];
        unpack<T>(vv[u], vx);
        float n1 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) n1 += fabsf(vx[e]);
        lnorm = __log2f(row_sum<LPR>(n1));
      }
      if (row < row_end) {
        if (c < G && !a.score_none) {
          float mine = s[u][0];
#pragma unroll
          for (int h = 1; h < G; ++h) mine = c == h ? s[u][h] : mine;
          store_wt(&lg[(size_t)c * lstride + row], mine + lnorm);
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) s[u][h] = -INFINITY;
      }
    }
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
      unpack<T>(vv[u], vx);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(s[u][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e]);
      }
    }
  };
  {
    uint4 ka[U], va[U], kb[U], vb[U];
    int tb = start;
    if (tb < row_end) load_tile(tb, ka, va);
    while (tb < row_end) {
      const int t1 = tb + TILE;
      if (t1 < row_end) load_tile(t1, kb, vb);
      process_tile(tb, ka, va);
      if (t1 >= row_end) break;
      const int t2 = t1 + TILE;
      if (t2 < row_end) load_tile(t2, ka, va);
      process_tile(t1, kb, vb);
      tb = t2;
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
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = s_merge + (wave * G + h) * (D + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[c * EPL + e] = acc[h][e];
      if (c == 0) {
        dst[D] = m[h];
        dst[D + 1] = l[h];
      }
    }
  }
}

// Streaming of one chunk on the matrix cores (bf16 cache).  A wave handles
// groups of 16 rows:
//  * q.k: v_mfma_f32_16x16x32_bf16 with the K rows as operand A (lane l loads
//    row l % 16, dims [32 kb + 8 (l / 16), +8)) and the group's q as operand B
//    (column n = query head n, zero beyond G).  Lane (j = l / 16, n = l % 16)
//    receives the logits of rows 4 j + i, i < 4, for head n.
//  * P.V: v_mfma_f32_16x16x16_bf16 per block of 16 value dims.  The group's
//    value rows are written row-major to a per-wave LDS tile and read back with
//    ds_read_b64_tr_b16, which transposes 4 x 4 blocks across each 16-lane
//    group: lane (j, n) receives dims 16 blk + n of rows 4 j .. 4 j + 3, the A
//    operand whose contraction index k = 4 j + e is row 4 j + e.  The B operand
//    (row 4 j + e, head n) is then exactly the lane's own probability of logit
//    e, so P never moves between lanes.  P enters as a bf16 hi part plus a bf16
//    residual (two MFMAs), which keeps it to about 2^-17 relative error.
//  * Online softmax with lazy rescaling: the reference max only moves when a
//    group's max exceeds it by more than 2^8, so the accumulators are rescaled
//    rarely; every quantity stays relative to the same reference, so results
//    equal the eager form up to rounding.
// Leaves the wave's partial in s_merge[wave][G][D + 2] like stream_valu.
template <int D, int G>
__device__ void stream_mfma(const StepArgs& a, int pair, int start, int count, PairMeta& pm, int& lmode,
                            float* s_merge, unsigned char* s_stage, float* s_logit) {
  constexpr int KB = D / 32;  // q.k MFMAs per row group
  constexpr int EV = D / 16;  // value dims per lane per row = P.V MFMAs per value row
  constexpr float kLazy = 8.0f;
  using VLoad = typename std::conditional<EV == 8, uint4, uint2>::type;
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int RS = D * 2 + 32;  // staged row stride in bytes
  constexpr int NB = D / 16;      // value-dim blocks
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int n = lane & 15, j = lane >> 4;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const size_t pair_off = (size_t)pair * a.max_budget * D;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.k_cache) + pair_off;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.v_cache) + pair_off;

  // The pair's metadata comes in by vector loads issued first, so that waiting
  // for it (below, after the first K/V rows are requested) covers nothing else;
  // a scalar load would be waited for with every other scalar load, before any
  // K/V row is requested.
  int4 m0, m1;
  {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));  // address looks per-lane: a vector load
    const int4* mp = reinterpret_cast<const int4*>(a.meta + pair) + z;
    m0 = mp[0];
    m1 = mp[1];
  }

  uint4 qb[KB];
  {
    // Lanes past the group's heads load head 0's row (always valid) and never
    // use it: an unconditional load is not waited for at once.
    const int hq = n < G ? n : 0;
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.n_q_heads + (size_t)g * G + hq) * D + 8 * j;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qb[kb] = *reinterpret_cast<const uint4*>(qh + 32 * kb);
  }
  f32x4_t acc[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // This wave's staging tile; lane (j, n) writes value rows 4 j + u at dims
  // [EV n, EV n + EV) and reads, through the transposing load, the address of
  // row 4 j + n / 4, dims 4 (n % 4) (+ 16 blk).
  unsigned char* tile = s_stage + wave * 16 * RS;
  unsigned char* wr = tile + 4 * j * RS + EV * 2 * n;
  const unsigned char* rd = tile + (4 * j + (n >> 2)) * RS + 8 * (n & 3);
  float m = kNegBig, lsum = 0.f;

  // Each wave walks its own contiguous quarter of the chunk in 16-row groups.
  // Full groups run in a two-stage pipeline with pointer bumps and immediate
  // offsets (the next group's loads are in flight while the current one
  // computes); at most one ragged group per wave remains and is loaded with
  // rows clamped to the last valid row (their logits are masked to -inf, so
  // their probabilities are exactly 0).  The raw q.k of every row goes to a
  // per-wave LDS buffer and is written out LR rows at a time as contiguous
  // runs (see Shape::kLogitRows).  An unsplit pair whose wave ranges fit the
  // buffers (kLogitsFull), or fit them in half precision (kLogitsHalf, log2
  // domain), writes nothing: the tail reads the buffers.
  constexpr int LR = Shape<BF16T, D, G>::kLogitRows;  // rows per logit flush
  const float scale = a.scale_log2;
  // Wave ranges split the item's rows [start, start + count), not the filled
  // ones: they do not depend on the fill level, so the first group's loads can
  // be issued before the pair's metadata arrives (rows past the fill level are
  // inside the cache allocation and simply not used).
  const int quarter = ((count + kWaves - 1) / kWaves + 15) & ~15;
  const int R0 = start + wave * quarter;
  const uint16_t* kp = Kp + (size_t)(R0 + n) * D + 8 * j;
  const uint16_t* vp = Vp + (size_t)(R0 + 4 * j) * D + EV * n;
  float* lbuf = s_logit + wave * G * LR;  // [G][LR]
  int flushed = R0;                       // rows below this are already in HBM
  // Known once the metadata has arrived (see below).
  int row_end = 0, Rend = 0, nfull = 0, Rp = 0, lstride = 0;
  float* lg = nullptr;
  __amdgpu_buffer_rsrc_t lrs;

  auto flush = [&](int upto) {  // write buffered logits of rows [flushed, upto)
    // Fixed trip count (no data-dependent loop): the compiler can then count
    // the outstanding stores exactly and never waits for them to complete.
    // Without importance (score_none) nothing is written.
    constexpr int NV = G * LR / 4;  // float4 cells of the buffer
    const int nrows = a.score_none ? 0 : upto - flushed;
#pragma unroll
    for (int it = 0; it < (NV + 63) / 64; ++it) {
      const int idx = lane + 64 * it;
      const int h = idx / (LR / 4), r4 = idx % (LR / 4);
      // A ragged end is only possible at the pair's last filled row (chunk
      // bounds are tile multiples, wave bounds multiples of 16); the slots
      // between it and the next multiple of 4 are unfilled and never read, so
      // whole float4 cells are written (the buffer holds -inf there).
      if ((NV % 64 == 0 || idx < NV) && 4 * r4 < nrows)
        store_wt4(lrs, 4 * (h * lstride + flushed + 4 * r4), *reinterpret_cast<const float4*>(lbuf + h * LR + 4 * r4));
    }
    flushed = upto;
  };
  // K/V are read once per step: non-temporal loads keep them from displacing
  // the workspace (logits, partials) in L2 and the Infinity Cache.
  // A group past the wave's full groups is still "loaded", from one line at
  // the pair's start that every lane shares, and never used: the loads are
  // issued unconditionally, since a load under a branch makes the wait before
  // the next group cover every buffer, which drains the pipeline.
  auto load_grp = [&](uint4(&kk)[KB], VLoad(&vv)[4], bool live) {
    const uint16_t* k = live ? kp : Kp;
    const uint16_t* v = live ? vp : Vp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kk[kb] = load_nt(reinterpret_cast<const uint4*>(k + 32 * kb));
#pragma unroll
    for (int u = 0; u < 4; ++u) vv[u] = load_nt(reinterpret_cast<const VLoad*>(v + u * D));
    kp += 16 * D;
    vp += 16 * D;
  };
  // The first group is loaded before the fill level is known, always (so the
  // number of loads in flight is fixed when the metadata is waited for), with
  // rows clamped into the pair's allocation; it is used only if the filled
  // rows make a full group there.
  auto load_first = [&](uint4(&kk)[KB], VLoad(&vv)[4]) {
    const int mb1 = a.max_budget - 1;
    const uint16_t* k0 = Kp + (size_t)min(R0 + n, mb1) * D + 8 * j;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kk[kb] = load_nt(reinterpret_cast<const uint4*>(k0 + 32 * kb));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vv[u] = load_nt(reinterpret_cast<const VLoad*>(Vp + (size_t)min(R0 + 4 * j + u, mb1) * D + EV * n));
    kp += 16 * D;
    vp += 16 * D;
  };
  auto process = [&](auto full_tag, const uint4(&kk)[KB], const VLoad(&vv)[4], int R) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int r0 = R + 4 * j;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[kb]),
                                                     __builtin_bit_cast(bf16x8_t, qb[kb]), sacc, 0, 0, 0);
    float sv[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};  // raw q.k of rows r0 + i, head n
    if constexpr (!kFull) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = r0 + i < row_end ? sv[i] : -INFINITY;
    }
    // What the tail scores from: the raw q.k, or with VL1 the log2-domain
    // logit plus log2 |v|_1 of the row (weight times norm = exp2 of the sum),
    // so no norm is stored apart.  Every lane of row group j holds the norms
    // of rows r0 .. r0 + 3 after the 16-lane sum.
    float st[4] = {sv[0], sv[1], sv[2], sv[3]};
    if (a.vl1) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float vf[EV];
        if constexpr (EV == 8) {
          unpack<BF16T>(vv[u], vf);
        } else {
          vf[0] = bf16_lo(vv[u].x);
          vf[1] = bf16_hi(vv[u].x);
          vf[2] = bf16_lo(vv[u].y);
          vf[3] = bf16_hi(vv[u].y);
        }
        float n1 = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) n1 += fabsf(vf[e]);
        st[u] = fmaf(sv[u], scale, __log2f(row_sum<16>(n1)));
      }
    }
    if (n < G) {
      if (lmode == kLogitsHalf) {
        // log2-domain values in half precision, 2 LR rows per head (see kLogitsHalf)
        typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
        const float f = a.vl1 ? 1.0f : scale;
        const half4_t x = {(_Float16)(st[0] * f), (_Float16)(st[1] * f), (_Float16)(st[2] * f),
                           (_Float16)(st[3] * f)};
        *reinterpret_cast<half4_t*>(reinterpret_cast<_Float16*>(lbuf) + n * 2 * LR + (r0 - R0)) = x;
      } else {
        *reinterpret_cast<float4*>(lbuf + n * LR + (r0 - flushed)) = make_float4(st[0], st[1], st[2], st[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<VLoad*>(wr + u * RS) = vv[u];
    // Group max per head (log2 domain): in-lane over 4 rows, then across the 4 lane groups.
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = fmaxf(mt, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mt), 0x401F)));  // lane ^ 16
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale;  // lane ^ 32
    }
    if (__builtin_amdgcn_ballot_w64(mt > m + kLazy)) {
      const float mn = fmaxf(m, mt);
      const float corr = fast_exp2(m - mn);
      m = mn;
      lsum *= corr;
#pragma unroll
      for (int e = 0; e < NB; ++e) acc[e] *= corr;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(fmaf(sv[i], scale, -m));
      lsum += p[i];
    }
    const bf16x4_t phi = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    const bf16x4_t plo = {(__bf16)(p[0] - (float)phi[0]), (__bf16)(p[1] - (float)phi[1]),
                          (__bf16)(p[2] - (float)phi[2]), (__bf16)(p[3] - (float)phi[3])};
    const i16x4_t bhi = __builtin_bit_cast(i16x4_t, phi), blo = __builtin_bit_cast(i16x4_t, plo);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const i16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(rd + 32 * blk));
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bhi, acc[blk], 0, 0, 0);
      acc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, blo, acc[blk], 0, 0, 0);
    }
  };
  {
    // Ring of NS group buffers: while group g is processed, groups up to
    // g + NS - 1 are in flight.
    constexpr int NS = Shape<BF16T, D, G>::kStages;
    uint4 kbuf[NS][KB];
    VLoad vbuf[NS][4];
    int g = 0;
    load_first(kbuf[0], vbuf[0]);
    // Keeps the compiler from sinking those loads into the branch that uses
    // them, which would put them behind the wait for the metadata.
    asm volatile("" ::: "memory");
    pm.t = __builtin_amdgcn_readfirstlane(m0.x);
    pm.len = __builtin_amdgcn_readfirstlane(m0.y);
    pm.budget = __builtin_amdgcn_readfirstlane(m0.z);
    pm.nchunk = __builtin_amdgcn_readfirstlane(m0.w);
    pm.item0 = __builtin_amdgcn_readfirstlane(m1.x);
    pm.slot0 = __builtin_amdgcn_readfirstlane(m1.y);
    pm.ticket = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(m1.z));
    pm.lstride = __builtin_amdgcn_readfirstlane(m1.w);
    row_end = min(start + count, pm.len);
    Rend = min(R0 + quarter, row_end);
    nfull = Rend - R0 >= 16 ? (Rend - R0) / 16 : 0;
    Rp = R0 + 16 * nfull;  // first row of the ragged group, if any
    lstride = pm.lstride;
    lg = a.logits + (size_t)pm.slot0 * G;  // [G][lstride]
    lrs = wt_rsrc(lg, a.score_none ? 0 : G * lstride * 4);
    // An unsplit pair whose wave ranges fit the buffers keeps its logits here,
    // in fp32 up to LR rows per wave, in half precision up to 2 LR.
    lmode = pm.nchunk != 1 ? kLogitsOut : quarter <= LR ? kLogitsFull : quarter <= 2 * LR ? kLogitsHalf : kLogitsOut;
#pragma unroll
    for (int s = 1; s < NS - 1; ++s) load_grp(kbuf[s], vbuf[s], s < nfull);
    auto step = [&](const uint4(&kk)[KB], const VLoad(&vv)[4]) {
      process(std::true_type{}, kk, vv, R0 + 16 * g);
      ++g;
      // A full buffer goes out, unless the pair keeps its logits in LDS for
      // the tail.
      if ((g & (LR / 16 - 1)) == 0 && lmode == kLogitsOut) flush(R0 + 16 * g);
    };
    // One exit only (at the top): a second exit is merged with it by the
    // compiler, and the merged path makes the loop's first wait a full drain.
    while (g + NS <= nfull) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // kbuf[s] holds group g; the buffer of group g - 1 takes group g + NS - 1.
        load_grp(kbuf[(s + NS - 1) % NS], vbuf[(s + NS - 1) % NS], g + NS - 1 < nfull);
        step(kbuf[s], vbuf[s]);
      }
    }
    // Fewer than NS full groups are left, all of them already loaded.
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (g < nfull) step(kbuf[s], vbuf[s]);
    if (Rp < Rend) {
      const int last = row_end - 1;
      const uint16_t* kr = Kp + (size_t)min(Rp + n, last) * D + 8 * j;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kbuf[0][kb] = *reinterpret_cast<const uint4*>(kr + 32 * kb);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        vbuf[0][u] = *reinterpret_cast<const VLoad*>(Vp + (size_t)min(Rp + 4 * j + u, last) * D + EV * n);
      process(std::false_type{}, kbuf[0], vbuf[0], Rp);
    }
    if (flushed < Rend && lmode == kLogitsOut) flush(Rend);
  }
  lsum += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lsum), 0x401F));
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (n < G) {
    float* dst = s_merge + (wave * G + n) * (D + 2);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[16 * blk + 4 * j + i] = acc[blk][i];
    if (j == 0) {
      dst[D] = m;
      dst[D + 1] = lsum;
    }
  }
}

template <class T, int D, int G, bool U>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Shape<T, D, G>::kMinWavesPerSimd, 8)))
void lf_step_kernel(StepArgs a) {
  using S = Shape<T, D, G>;
  __shared__ float smem[S::kSmemFloats];
  __shared__ int s_last;
  float* s_part = smem;                   // [G][D + 2]: merged partial of this chunk
  float* s_work = smem + S::kPartFloats;  // cross-wave merge, then tail scratch

  const int tid = threadIdx.x;
  // U (equal budgets): the item follows from the block index, so the first
  // K/V loads wait for no load of the work list.  A separate instantiation:
  // a run-time branch would make every scalar load of the prologue wait.
  WorkItem it;
  if constexpr (U) {
    it.pair = blockIdx.x / a.u_nchunk;
    it.chunk = blockIdx.x - it.pair * a.u_nchunk;
    it.start = it.chunk * a.u_chunk;
    it.count = min(a.u_chunk, a.u_budget - it.start);
  } else {
    it = a.items[blockIdx.x];
  }
  const int pair = it.pair;
  PairMeta* meta = a.meta + pair;  // written only by this pair's tail, after every chunk is done
  float* s_logit = s_work + S::kMergeFloats + S::kStageFloats;
  float* s_pre = smem + S::kSmemFloats - S::kPreFloats;  // prefetched tail inputs
  PairMeta pm;
  int lmode = kLogitsOut;  // where the pair's logits are for its tail
  if constexpr (T::kEpl == 8) {
    if (tid < 64) prefetch_tail<D, G>(a, pair, s_pre);
    stream_mfma<D, G>(a, pair, it.start, it.count, pm, lmode, s_work,
                      reinterpret_cast<unsigned char*>(s_work + S::kMergeFloats), s_logit);
    // The prefetch completed before wave 0's first stream wait (loads return in
    // order); without a row to stream, wave 0 waits for it here.
    if (tid < 64 && min(it.start + it.count, pm.len) <= it.start) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    pm = *meta;
    stream_valu<T, D, G>(a, pair, it.start, min(it.start + it.count, pm.len), a.logits + (size_t)pm.slot0 * G,
                         pm.lstride, s_work);
  }
  const int nchunk = pm.nchunk;
  __syncthreads();
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(s_work + S::kBitsOffset);
  clear_protect_bits(s_bits, pm.budget);

  // Merge the waves' partials into this chunk's partial.
  const size_t item = blockIdx.x;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, dim = idx - h * D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_work[(w * G + h) * (D + 2) + D]);
    float sa = 0.f, sl = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* src = s_work + (w * G + h) * (D + 2);
      const float f = fast_exp2(src[D] - mm);
      sa += src[dim] * f;
      sl += src[D + 1] * f;
    }
    if (nchunk == 1) {
      s_part[h * (D + 2) + dim] = sa;
      if (dim == 0) {
        s_part[h * (D + 2) + D] = mm;
        s_part[h * (D + 2) + D + 1] = sl;
      }
    } else {
      store_wt(&a.part_acc[(item * G + h) * D + dim], sa);
      if (dim == 0) store_wt(&reinterpret_cast<float2*>(a.part_ml)[item * G + h], make_float2(mm, sl));
    }
  }

  if (nchunk == 1) {
    __syncthreads();  // merged partial complete, bitmap cleared
    set_protect_bits<T, D, G>(a, pair, pm.budget, s_bits, s_pre);
    __syncthreads();
  } else {
    // Ticket (the hand-over protocol is described at store_wt): every wave
    // drains its device-scope stores, the barrier orders that before thread
    // 0's device-scope increment, and the last arrival runs the tail.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(&meta->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev + 1 == static_cast<unsigned>(nchunk);
    }
    set_protect_bits<T, D, G>(a, pair, pm.budget, s_bits, s_pre);  // while the ticket is in flight
    __syncthreads();
    if (!s_last) return;
  }
  pair_tail<T, D, G>(a, pair, pm, s_part, s_work, s_logit, lmode, s_pre);
}

template <class T, int D, int G>
void launch_one(const StepArgs& a, hipStream_t s) {
  if (a.u_budget > 0)
    hipLaunchKernelGGL((lf_step_kernel<T, D, G, true>), dim3(a.n_items), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((lf_step_kernel<T, D, G, false>), dim3(a.n_items), dim3(kThreads), 0, s, a);
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

int download_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    snprintf(err, errlen, "state download failed: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

}  // namespace lf
