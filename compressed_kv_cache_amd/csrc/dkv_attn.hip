// libdkv_attn: DKV decode attention over a compressed KV cache, for gfx950.
//
// Method: "DKV: Anchor + Low-Rank Differential KV-Cache Compression for Scalable
// Long-Context Inference" (Zenodo record, abstract) and the Differential-KV README
// ("Core Architecture & Paper Overview", "Decode & Prefill Innovations", "Key
// Environment Knobs").  The C ABI is declared and documented in dkv_attn.h.
//
// Kernels
//   k_route_keys  c = a_k + mean_i(U_i) V_K per (slot, KV head), fp32.
//   k_route_topk  one workgroup per (sequence, KV head): GQA-mean query, scores of
//                 every block, exact top-K by a 4-pass 8-bit radix select with
//                 lowest-index tie breaking, indices emitted in ascending order.
//   k_attend      one workgroup per part (a routed block, or a window chunk).
//                 Each wave takes 16-row tiles; scores and values are MFMA
//                 products (v_mfma_f32_16x16x16_f16) with an online softmax
//                 per query head.  A block's low-rank rows use the augmented
//                 factors Ux = [U | 1] (row 0 = anchor = [0 | 1]),
//                 VKx = [V_K ; a_k] and VVx = [V_V ; a_v], so that
//                   score_i = Ux_i . (VKx q)        (= q.a_k + U_i.(V_K q))
//                   value   = (p^T Ux) VVx          (= (sum p) a_v + (p^T U) V_V)
//                 without reconstructing any key or value row.  Residual
//                 positions are masked out of the low-rank rows; residual rows
//                 and window rows are attended exactly.  fp32 operands of the
//                 MFMA (V_K q, p, p^T U) are split into fp16 hi + lo halves, so
//                 the products keep ~22 bits of the fp32 value.
//   k_merge       log-sum-exp combine of the parts of each query row.
// All reductions run in a fixed order; there are no floating-point atomics.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dkv_attn.h"

typedef _Float16 f16;
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int kD = 128;            // head dim
constexpr int kLowRankRows = 255;  // tokens 1..255 of a block
constexpr int kVStride = 132;      // LDS row stride (halves) of 128-wide tiles: conflict-free column reads
constexpr int kWinChunk = 128;     // window rows per part in dkv_decode

thread_local char g_err[512] = "";

dkv_status fail(dkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// ----------------------------------------------------------------------------
// Kernel arguments (plain structs passed by value)
// ----------------------------------------------------------------------------

struct PoolArgs {
  const f16* ak; int64_t ak_s, ak_h;
  const f16* av; int64_t av_s, av_h;
  const f16* u;  int64_t u_s, u_h;
  const f16* vk; int64_t vk_s, vk_h;
  const f16* vv; int64_t vv_s, vv_h;
  const f16* rk; int64_t rk_s, rk_h;
  const f16* rv; int64_t rv_s, rv_h;
  const uint8_t* rp; int64_t rp_s, rp_h;
  float* key; int64_t key_s, key_h;
  int rank, n_resid, n_kv, n_slots;
};

struct BatchArgs {
  int B, Hq, Hkv, G, W, mb;
  const int32_t* table;
  const int32_t* nblk;
  const int32_t* wlen;
  const f16* q;
  const f16* wk;
  const f16* wv;
};

struct AttnArgs {
  const int32_t* idx;
  int top_k;           // row stride of idx
  int n_block_parts;   // parts per unit that are routed blocks (top_k or 0)
  int block_mode;      // bit 0: low-rank rows of a block, bit 1: its residual rows
  int n_win_parts;
  int win_chunk;
  int items_per_unit;
  int rq;              // augmented rank rounded up to 16 (0 without low-rank rows)
  float scale;
  float* part_o;
  float* part_lse;
  int n_parts;
  int part_offset;
};

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------

__device__ __forceinline__ v4f mfma16(v4h a, v4h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split_hl(float x0, float x1, float x2, float x3, v4h& hi, v4h& lo) {
  const float x[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16 h = (f16)x[e];
    hi[e] = h;
    lo[e] = (f16)(x[e] - (float)h);
  }
}

// LDS hand-off between lanes of one wave: LDS operations of a wave complete in
// order, so waiting for this wave's outstanding LDS operations (lgkmcnt = 0)
// before reading what other lanes wrote is enough; the empty asm and the wave
// barrier keep the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt = 63 (no wait), expcnt = 7, lgkmcnt = 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ v8h ld8(const f16* p) { return *reinterpret_cast<const v8h*>(p); }

// Values handed from one workgroup to another inside a launch are written and
// read with device-scope (agent) relaxed atomics: these go to the device-wide
// coherence point, so no L2 write-back fence is needed on the hot path.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's stores have completed
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }

// Loads are always issued from an in-bounds address and masked afterwards: a
// guarded load would compile to its own branch, and the branch merge to a full
// wait for every outstanding load.
__device__ __forceinline__ v8h ld8_mask(const f16* p, bool keep) {
  uint4 x = *reinterpret_cast<const uint4*>(p);
  const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  x.x &= m;
  x.y &= m;
  x.z &= m;
  x.w &= m;
  return __builtin_bit_cast(v8h, x);
}

__device__ __forceinline__ v4h ld4_mask(const f16* p, bool keep) {
  uint2 x = *reinterpret_cast<const uint2*>(p);
  const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
  x.x &= m;
  x.y &= m;
  return __builtin_bit_cast(v4h, x);
}

__device__ __forceinline__ v4h lo4(v8h x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ v4h hi4(v8h x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

// Online softmax over one 16-row tile for the query head g = lane % 16.  The
// lane holds 4 of the 16 scores; lanes lane ^ 16 and lane ^ 32 hold the rest.
__device__ __forceinline__ void softmax_tile(const float z[4], float& m_run, float& l_run,
                                             float& alpha, float p[4]) {
  float tm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
  tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
  const float mn = fmaxf(m_run, tm);
  const bool none = (mn == -INFINITY);
  alpha = none ? 1.f : __expf(m_run - mn);
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = none ? 0.f : __expf(z[e] - mn);
  float ps = (p[0] + p[1]) + (p[2] + p[3]);
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  l_run = l_run * alpha + ps;
  m_run = mn;
}

// Per-row factor of the accumulator C layout (row g = 4 * (lane / 16) + e) from a
// per-head value held by every lane with lane % 16 == g.
__device__ __forceinline__ void rows_of(float v, int q4, float out[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = __shfl(v, 4 * q4 + e, 64);
}

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Exclusive count of `flag` over the workgroup (NW waves) in thread order, and the total.
template <int NW>
__device__ __forceinline__ void block_count(bool flag, int& excl, int& total, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int in_wave = __popcll(m & lt);
  if (lane == 0) wsum[w] = (uint32_t)__popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = (int)wsum[i];
    off += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  excl = off + in_wave;
  total = tot;
}

// ----------------------------------------------------------------------------
// Routing key precompute
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(128) void k_route_keys(PoolArgs P, const int32_t* slots) {
  const int item = blockIdx.x;
  const int si = item / P.n_kv, h = item % P.n_kv;
  const int slot = slots ? slots[si] : si;
  if (slot < 0 || slot >= P.n_slots) return;
  __shared__ float ubar[DKV_MAX_RANK];
  const int r = P.rank;
  const f16* U = P.u + slot * P.u_s + h * P.u_h;
  const int t = threadIdx.x;
  if (t < r) {
    float s = 0.f;
    for (int i = 0; i < kLowRankRows; ++i) s += (float)U[(int64_t)i * r + t];
    ubar[t] = s / (float)kLowRankRows;
  }
  __syncthreads();
  const f16* VK = P.vk + slot * P.vk_s + h * P.vk_h;
  const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
  float c = 0.f;
  for (int j = 0; j < r; ++j) c += ubar[j] * (float)VK[j * kD + t];
  P.key[slot * P.key_s + h * P.key_h + t] = (float)AK[t] + c;
}

// ----------------------------------------------------------------------------
// Top-K routing: one workgroup of 8 waves per (sequence, KV head)
// ----------------------------------------------------------------------------

constexpr int kRouteThreads = 512;

template <int NW>
struct RouteShared {
  float qbar[kD] __attribute__((aligned(16)));
  uint32_t hist[256];
  uint32_t wsum[NW];
  uint32_t digit, above;
};

// Route one (sequence, KV head) unit u with a workgroup of NT threads.
// lds: scratch of at least 2 * max_blocks words (ordered score keys, slots).
//
// All loads are issued before the first barrier: the G query rows, and for
// the first NT blocks their pool slot and 512-byte routing key.  Up to 1024
// blocks, the top-K selection is done by wave 0 alone with a bit-by-bit radix
// select on wave ballots (no workgroup barriers); beyond that, by a 4-pass
// 8-bit radix select of the whole workgroup.
// Routed-slot words of the fused kernel hold pool slot + kSlotCode (1: no block),
// so that 0, the state of zero-filled memory, means "routing not written yet".
constexpr int32_t kSlotPending = 0;
constexpr int32_t kSlotCode = 2;

template <int NT>
__device__ __forceinline__ void route_unit(const PoolArgs& P, const BatchArgs& Bt, int u, int top_k, int32_t* idx,
                                           float* scores, int32_t* slots_out, uint32_t* lds,
                                           RouteShared<NT / 64>& sh) {
  constexpr int NW = NT / 64;
  float* qbar = sh.qbar;
  uint32_t* hist = sh.hist;
  uint32_t* wsum = sh.wsum;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  int N = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  N = N < 0 ? 0 : (N > Bt.mb ? Bt.mb : N);
  const int keff = top_k < N ? top_k : N;
  uint32_t* keys = lds;
  int32_t* slot_of = reinterpret_cast<int32_t*>(lds + (Bt.mb > 0 ? Bt.mb : 1));

  // ---- issue: query rows, and slot + routing key of block j = tid
  float qv[DKV_MAX_GROUP];
  if (tid < kD) {
#pragma unroll
    for (int g = 0; g < DKV_MAX_GROUP; ++g) {
      const int gc = g < Bt.G ? g : Bt.G - 1;
      qv[g] = (float)Bt.q[((int64_t)b * Bt.Hq + h * Bt.G + gc) * kD + tid];
    }
  }
  float4 kv[kD / 4];
  int slot0 = -1;
  bool ok0 = false;
  if (N > 0) {
    const int jc = tid < N ? tid : N - 1;
    const int sr = Bt.table[(int64_t)b * Bt.mb + jc];
    ok0 = tid < N && sr >= 0 && sr < P.n_slots;
    slot0 = ok0 ? sr : -1;
    const float4* c = reinterpret_cast<const float4*>(P.key + (ok0 ? sr : 0) * P.key_s + h * P.key_h);
#pragma unroll
    for (int i = 0; i < kD / 4; ++i) kv[i] = c[i];
  }
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < DKV_MAX_GROUP; ++g) s += (g < Bt.G) ? qv[g] : 0.f;
    qbar[tid] = s / (float)Bt.G;
  }
  __syncthreads();

  // ---- scores (GQA-mean query against each routing key), as ordered keys
  if (N > 0) {
    const float4* qb = reinterpret_cast<const float4*>(qbar);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kD / 4; ++i) {
      const float4 qq = qb[i];
      acc += kv[i].x * qq.x + kv[i].y * qq.y + kv[i].z * qq.z + kv[i].w * qq.w;
    }
    if (tid < N) {
      keys[tid] = ordered_key(ok0 ? acc : -INFINITY);
      slot_of[tid] = slot0;
    }
    for (int j0 = NT; j0 < N; j0 += NT) {
      const int j = j0 + tid;
      const int jc = j < N ? j : N - 1;
      const int sr = Bt.table[(int64_t)b * Bt.mb + jc];
      const bool ok = j < N && sr >= 0 && sr < P.n_slots;
      const float4* c = reinterpret_cast<const float4*>(P.key + (ok ? sr : 0) * P.key_s + h * P.key_h);
#pragma unroll
      for (int i = 0; i < kD / 4; ++i) kv[i] = c[i];
      float a2 = 0.f;
#pragma unroll
      for (int i = 0; i < kD / 4; ++i) {
        const float4 qq = qb[i];
        a2 += kv[i].x * qq.x + kv[i].y * qq.y + kv[i].z * qq.z + kv[i].w * qq.w;
      }
      if (j < N) {
        keys[j] = ordered_key(ok ? a2 : -INFINITY);
        slot_of[j] = ok ? sr : -1;
      }
    }
  }
  __syncthreads();

  auto emit = [&](int pos, int j, uint32_t k) {
    st_dev(&idx[(int64_t)u * top_k + pos], j);
    if (scores) st_dev(&scores[(int64_t)u * top_k + pos], from_ordered(k));
    if (slots_out) st_dev(&slots_out[(int64_t)u * top_k + pos], (int32_t)slot_of[j] + kSlotCode);
  };

  if (keff > 0 && N <= 1024) {
    // ---- wave 0: bit-by-bit radix select of the keff-th largest key
    if (wave == 0) {
      constexpr int kPer = 16;
      const int per = (N + 63) >> 6;
      uint32_t kk[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int j = lane + 64 * i;
        kk[i] = (i < per && j < N) ? keys[j] : 0u;
      }
      uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)keff;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t bm = 1u << bit;
        uint32_t cnt = 0u;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (i < per) {
            const int j = lane + 64 * i;
            const bool c = (j < N) && ((kk[i] & mask) == prefix) && (kk[i] & bm);
            cnt += (uint32_t)__popcll(__ballot(c));
          }
        }
        if (cnt >= krem) prefix |= bm;
        else krem -= cnt;
        mask |= bm;
      }
      // keys above the threshold T = prefix, then the lowest-index keys equal to it,
      // emitted in ascending block order
      const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
      uint32_t eq_base = 0u, sel_base = 0u;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (i < per) {
          const int j = lane + 64 * i;
          const bool in = j < N;
          const bool eq = in && kk[i] == prefix;
          const unsigned long long em = __ballot(eq);
          const uint32_t er = eq_base + (uint32_t)__popcll(em & lt);
          const bool sel = in && (kk[i] > prefix || (eq && er < krem));
          const unsigned long long smk = __ballot(sel);
          if (sel) emit((int)(sel_base + (uint32_t)__popcll(smk & lt)), j, kk[i]);
          eq_base += (uint32_t)__popcll(em);
          sel_base += (uint32_t)__popcll(smk);
        }
      }
    }
  } else if (keff > 0) {
    // ---- whole workgroup: 4-pass 8-bit radix select
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t krem = (uint32_t)keff;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < N; j += NT) {
        const uint32_t k = keys[j];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t mine = h0 + h1 + h2 + h3;
        uint32_t incl = mine;  // sum over lanes >= this lane
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t v = __shfl_down(incl, off, 64);
          if (lane + off < 64) incl += v;
        }
        const uint32_t above = incl - mine;  // bins 4 * lane + 4 and higher
        const uint32_t s3 = above + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
        if (s3 >= krem && above < krem) { sh.digit = 4 * lane + 3; sh.above = above; }
        if (s2 >= krem && s3 < krem) { sh.digit = 4 * lane + 2; sh.above = s3; }
        if (s1 >= krem && s2 < krem) { sh.digit = 4 * lane + 1; sh.above = s2; }
        if (s0 >= krem && s1 < krem) { sh.digit = 4 * lane; sh.above = s1; }
      }
      __syncthreads();
      prefix |= sh.digit << shift;
      pmask |= 0xFFu << shift;
      krem -= sh.above;
    }
    const uint32_t T = prefix;
    int eq_base = 0, sel_base = 0;
    for (int c0 = 0; c0 < N; c0 += NT) {
      const int j = c0 + tid;
      const bool in = j < N;
      const uint32_t k = in ? keys[j] : 0u;
      const bool eq = in && k == T;
      int eq_rank, eq_tot;
      block_count<NW>(eq, eq_rank, eq_tot, wsum);
      const bool sel = in && (k > T || (eq && (uint32_t)(eq_base + eq_rank) < krem));
      int sel_rank, sel_tot;
      block_count<NW>(sel, sel_rank, sel_tot, wsum);
      if (sel) emit(sel_base + sel_rank, j, k);
      eq_base += eq_tot;
      sel_base += sel_tot;
    }
  }
  for (int pos = keff + tid; pos < top_k; pos += NT) {
    st_dev(&idx[(int64_t)u * top_k + pos], -1);
    if (scores) st_dev(&scores[(int64_t)u * top_k + pos], -INFINITY);
    if (slots_out) st_dev(&slots_out[(int64_t)u * top_k + pos], -1 + kSlotCode);
  }
}

__global__ __launch_bounds__(kRouteThreads) void k_route_topk(PoolArgs P, BatchArgs Bt, int top_k,
                                                              int32_t* idx, float* scores, int32_t* slots_out) {
  extern __shared__ uint32_t route_lds[];  // [2][mb] ordered score keys, pool slots
  __shared__ RouteShared<kRouteThreads / 64> sh;
  route_unit<kRouteThreads>(P, Bt, blockIdx.x, top_k, idx, scores, slots_out, route_lds, sh);
}

// ----------------------------------------------------------------------------
// Attention over one part: a routed block (its low-rank rows and/or its
// residual rows) or a chunk of window rows.  One workgroup of 4 waves per part,
// two workgroups per CU.
//
// Wave w takes low-rank tiles w, w+4, w+8, w+12 (16 block positions each) and
// exact-row tiles w, w+4, ... (16 rows each), with one online-softmax state per
// query head.  Every load a wave needs is issued before its first use, in the
// order of use; exact rows beyond the first two tiles are streamed two tiles
// ahead.  The final phase rescales the four states to the common maximum,
// sums them in a fixed order and applies V_V once: wave w finishes output
// columns 16 w .. 16 w + 15 and 64 + 16 w .. 64 + 16 w + 15.
// ----------------------------------------------------------------------------

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kLRTilesPerWave = 16 / kAttWaves;
constexpr int kRedStride = 132;  // floats per row of the reduction buffer (conflict-free C-layout access)

__host__ __device__ inline int round16(int x) { return (x + 15) & ~15; }

// per-wave scratch: the V tile of an exact tile, or the Ux transpose of a
// low-rank tile, followed by that wave's residual-position bit mask
__host__ __device__ inline int att_scratch_bytes(int rq) {
  const int a = 16 * kVStride * 2;
  const int b = 16 * (rq + 4) * 2;
  return round16((a > b ? a : b) + 32);
}

__host__ __device__ inline int att_region_bytes(int rq) {
  const int scratch = kAttWaves * att_scratch_bytes(rq);
  const int red = kAttWaves * 16 * kRedStride * 4 + kAttWaves * 16 * rq * 4;  // O and W of 4 waves
  return scratch > red ? scratch : red;
}

__host__ __device__ inline int att_lds_bytes(int rq) {
  return 16 * rq * 4 + rq * kVStride * 2 + 2 * kAttWaves * 16 * 4 + att_region_bytes(rq);
}

struct ExState {
  float m, l;
  v4f O[8];
};

template <int NQ>
__device__ __forceinline__ void rescale_state(ExState& st, v4f (&Wacc)[NQ], float alpha, int q4) {
  float ae[4];
  rows_of(alpha, q4, ae);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st.O[n][e] *= ae[e];
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Wacc[n][e] *= ae[e];
  }
}

// One 16-row tile of exact rows t0..t0+15 (rows >= n_ex masked).
template <int NQ>
__device__ __forceinline__ void exact_tile(const v8h (&kx)[4], const v8h (&vx)[4], int t0, int n_ex,
                                           const v4h (&qf)[4][2], float scale, ExState& st, v4f (&Wacc)[NQ],
                                           f16* Vt, int l16, int q4) {
  v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    S = mfma16(lo4(kx[s]), qf[s][0], S);
    S = mfma16(hi4(kx[s]), qf[s][1], S);
  }
  float zz[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) zz[e] = (t0 + 4 * q4 + e < n_ex) ? S[e] * scale : -INFINITY;
  float alpha, pe[4];
  softmax_tile(zz, st.m, st.l, alpha, pe);
  rescale_state<NQ>(st, Wacc, alpha, q4);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    *reinterpret_cast<v4h*>(Vt + l16 * kVStride + 32 * s + 8 * q4) = lo4(vx[s]);
    *reinterpret_cast<v4h*>(Vt + l16 * kVStride + 32 * s + 8 * q4 + 4) = hi4(vx[s]);
  }
  wave_sync_lds();
  v4h ph, pl;
  split_hl(pe[0], pe[1], pe[2], pe[3], ph, pl);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    v4h bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[e] = Vt[(4 * q4 + e) * kVStride + 16 * n + l16];
    st.O[n] = mfma16(ph, bv, st.O[n]);
    st.O[n] = mfma16(pl, bv, st.O[n]);
  }
  wave_sync_lds();
}

__device__ __forceinline__ void load_exact_tile(const f16* kb, const f16* vb, int tile, int ntile, int n_ex,
                                                v8h (&kx)[4], v8h (&vx)[4], int l16, int q4) {
  // rows past n_ex read row n_ex - 1: their scores are masked to -inf and their
  // softmax weights are exactly 0, so the (finite) data never contributes
  const int t = tile * 16 + l16;
  const int tc = (tile < ntile && t < n_ex) ? t : n_ex - 1;  // n_ex >= 1 here
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kx[s] = ld8(kb + (int64_t)tc * kD + 32 * s + 8 * q4);
    vx[s] = ld8(vb + (int64_t)tc * kD + 32 * s + 8 * q4);
  }
}

// NRQ = number of 16-wide column tiles of the augmented rank r + 1 (0 without
// low-rank rows), a template parameter so that every loop over them is static.
constexpr int kSlotLookup = -0x7fffffff;  // attend_part: look the slot up from idx and the block table

template <int NRQ>
__device__ __forceinline__ void attend_part(const PoolArgs& P, const BatchArgs& Bt, const AttnArgs& A, int u, int p,
                                            int slot_in, unsigned char* smem) {
  constexpr int NQ = NRQ > 0 ? NRQ : 1;
  constexpr int RQ = 16 * NRQ;
  constexpr int kVVChunks = (16 * NQ * 16 + kAttThreads - 1) / kAttThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  const int G = Bt.G;
  const int row0 = b * Bt.Hq + h * G;

  // ---- query fragments first (they depend on nothing else): lane holds
  //      q[g = l16][32 s + 8 q4 + 4 hh + e]; lanes of padded heads g >= G load
  //      head 0, whose results they never write
  v4h qf[4][2];
  {
    const f16* qrow = Bt.q + (int64_t)(row0 + (l16 < G ? l16 : 0)) * kD + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v8h x = ld8(qrow + 32 * s);
      qf[s][0] = lo4(x);
      qf[s][1] = hi4(x);
    }
  }

  // ---- what this part covers (uniform over the workgroup)
  bool lr = false;
  int n_ex = 0;
  const f16* exk = nullptr;
  const f16* exv = nullptr;
  int slot = -1;
  if (p < A.n_block_parts) {
    if (slot_in != kSlotLookup) {
      slot = slot_in;  // routed pool slot, or -1
    } else {
      int nb = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
      nb = nb < 0 ? 0 : (nb > Bt.mb ? Bt.mb : nb);
      const int j = A.idx[(int64_t)u * A.top_k + p];
      if (j >= 0 && j < nb) slot = Bt.table[(int64_t)b * Bt.mb + j];
    }
    if (slot >= P.n_slots) slot = -1;
    if (slot >= 0) {
      lr = (A.block_mode & 1) != 0;
      if ((A.block_mode & 2) && P.n_resid > 0) {
        n_ex = P.n_resid;
        exk = P.rk + slot * P.rk_s + h * P.rk_h;
        exv = P.rv + slot * P.rv_s + h * P.rv_h;
      }
    }
  } else {
    const int s = p - A.n_block_parts;
    int wl = Bt.wlen ? Bt.wlen[b] : Bt.W;
    wl = wl < 0 ? 0 : (wl > Bt.W ? Bt.W : wl);
    const int start = s * A.win_chunk;
    const int end = (start + A.win_chunk < wl) ? start + A.win_chunk : wl;
    if (end > start) {
      n_ex = end - start;
      const int64_t base = (((int64_t)b * Bt.Hkv + h) * Bt.W + start) * kD;
      exk = Bt.wk + base;
      exv = Bt.wv + base;
    }
  }

  const int part = A.part_offset + p;
  if (!lr && n_ex == 0) {
    for (int t = tid; t < G * kD; t += kAttThreads) {
      const int g = t / kD, d = t % kD;
      st_dev(&A.part_o[((int64_t)(row0 + g) * A.n_parts + part) * kD + d], 0.f);
    }
    if (tid < G) st_dev(&A.part_lse[(int64_t)(row0 + tid) * A.n_parts + part], -INFINITY);
    return;
  }

  // ---- LDS carve-up
  float* qt = reinterpret_cast<float*>(smem);                     // [16][RQ]  V_K q and q.a_k
  f16* vvx = reinterpret_cast<f16*>(qt + 16 * RQ);                // [RQ][kVStride]  [V_V ; a_v ; *]
  float* wstat = reinterpret_cast<float*>(vvx + RQ * kVStride);   // m [4][16], l [4][16]
  unsigned char* region = reinterpret_cast<unsigned char*>(wstat + 2 * kAttWaves * 16);
  constexpr int TS = RQ + 4;
  unsigned char* my = region + wave * att_scratch_bytes(RQ);
  uint32_t* wmask = reinterpret_cast<uint32_t*>(my + att_scratch_bytes(RQ) - 32);
  const int ntile = (n_ex + 15) >> 4;
  const int r = P.rank;
  const float scale = A.scale;

  ExState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.O[n] = (v4f){0.f, 0.f, 0.f, 0.f};
  v4f Wacc[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) Wacc[n] = (v4f){0.f, 0.f, 0.f, 0.f};

  // ---- issue the loads, in the order of use
  v4h ua[kLRTilesPerWave][NQ];
  int ps[4];
  v8h vvl[kVVChunks];
  v8h vkx[2][4];
  const f16* U = nullptr;
  if (NRQ > 0 && lr) {
    const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
    const f16* AV = P.av + slot * P.av_s + h * P.av_h;
    const f16* VK = P.vk + slot * P.vk_s + h * P.vk_h;
    const f16* VV = P.vv + slot * P.vv_s + h * P.vv_h;
    U = P.u + slot * P.u_s + h * P.u_h;
    {
      const int nres = P.n_resid;
      const uint8_t* pp = nres > 0 ? P.rp + slot * P.rp_s + h * P.rp_h : P.rp;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = lane + 64 * k;
        ps[k] = (nres > 0) ? (int)pp[t < nres ? t : 0] : 0;
      }
    }
    // VVx rows: V_V rows j < r, a_v at j = r.  Padding rows j > r read V_V row 0:
    // their weight in (p^T Ux) is exactly 0 because Ux is zero there.
#pragma unroll
    for (int k = 0; k < kVVChunks; ++k) {
      const int c = tid + kAttThreads * k;
      const int j = (c < RQ * 16) ? (c >> 4) : 0, col = (c & 15) * 8;
      const f16* src = (j < r) ? VV + (int64_t)j * kD : ((j == r) ? AV : VV);
      vvl[k] = ld8(src + col);
    }
    // VKx rows: V_K rows j < r, a_k at j = r; padding rows read V_K row 0
    // (they only meet zero columns of Ux)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = (wave + kAttWaves * k) * 16 + l16;
      const f16* src = (j < r) ? VK + (int64_t)j * kD : ((j == r) ? AK : VK);
      if (wave + kAttWaves * k < NRQ) {
#pragma unroll
        for (int s = 0; s < 4; ++s) vkx[k][s] = ld8(src + 32 * s + 8 * q4);
      }
    }
    if ((r & 3) == 0) {
#pragma unroll
      for (int k = 0; k < kLRTilesPerWave; ++k) {
        const int i = (wave + kAttWaves * k) * 16 + l16;  // position in the block; 0 = anchor
        const f16* row = U + (int64_t)(i > 0 ? i - 1 : 0) * r;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          const int j0 = 16 * s + 4 * q4;
          ua[k][s] = *reinterpret_cast<const v4h*>(row + (j0 < r ? j0 : 0));
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kLRTilesPerWave; ++k) {
        const int i = (wave + kAttWaves * k) * 16 + l16;
        const f16* row = U + (int64_t)(i > 0 ? i - 1 : 0) * r;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * s + 4 * q4 + e;
            ua[k][s][e] = row[j < r ? j : 0];
          }
        }
      }
    }
  }
  v8h ka[4], va[4], kb[4], vb[4];
  int ta = wave, tb = wave + kAttWaves;
  if (n_ex > 0) {
    load_exact_tile(exk, exv, ta, ntile, n_ex, ka, va, l16, q4);
    load_exact_tile(exk, exv, tb, ntile, n_ex, kb, vb, l16, q4);
  }

  // ---- low-rank set-up: residual-position mask (per wave), VVx, VKx q
  if (NRQ > 0 && lr) {
    if (lane < 8) wmask[lane] = 0u;
    wave_sync_lds();
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (ps[k] >= 1 && ps[k] <= kLowRankRows) atomicOr(&wmask[ps[k] >> 5], 1u << (ps[k] & 31));
#pragma unroll
    for (int k = 0; k < kVVChunks; ++k) {
      const int c = tid + kAttThreads * k;
      if (c < RQ * 16) {
        const int j = c >> 4, col = (c & 15) * 8;
        *reinterpret_cast<v4h*>(vvx + j * kVStride + col) = lo4(vvl[k]);
        *reinterpret_cast<v4h*>(vvx + j * kVStride + col + 4) = hi4(vvl[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int jt = wave + kAttWaves * k;
      if (jt < NRQ) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc = mfma16(lo4(vkx[k][s]), qf[s][0], acc);
          acc = mfma16(hi4(vkx[k][s]), qf[s][1], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) qt[l16 * RQ + jt * 16 + 4 * q4 + e] = acc[e];
      }
    }
    __syncthreads();  // V_K q and VVx complete (uniform: lr is uniform)

    // ---- low-rank tiles: 16 positions each (position 0 is the anchor)
    v4h qth[NQ], qtl[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const float4 x = *reinterpret_cast<const float4*>(qt + l16 * RQ + 16 * s + 4 * q4);
      split_hl(x.x, x.y, x.z, x.w, qth[s], qtl[s]);
    }
    f16* T = reinterpret_cast<f16*>(my);
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k) {
      const int i0 = (wave + kAttWaves * k) * 16;
      const int i = i0 + l16;
      // Ux = [U | 1 | 0]; the anchor row has U = 0
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * s + 4 * q4 + e;
          ua[k][s][e] = (j == r) ? (f16)1.0f : ((i > 0 && j < r) ? ua[k][s][e] : (f16)0.0f);
        }
      }
      v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        z = mfma16(ua[k][s], qth[s], z);
        z = mfma16(ua[k][s], qtl[s], z);
      }
      float zz[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = i0 + 4 * q4 + e;
        const bool masked = (ii > 0) & (((wmask[ii >> 5] >> (ii & 31)) & 1u) != 0u);
        zz[e] = masked ? -INFINITY : z[e] * scale;
      }
      float alpha, pe[4];
      softmax_tile(zz, st.m, st.l, alpha, pe);
      rescale_state<NQ>(st, Wacc, alpha, q4);
      v4h ph, pl;
      split_hl(pe[0], pe[1], pe[2], pe[3], ph, pl);
#pragma unroll
      for (int s = 0; s < NQ; ++s) *reinterpret_cast<v4h*>(T + l16 * TS + 16 * s + 4 * q4) = ua[k][s];
      wave_sync_lds();
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        v4h bu;
#pragma unroll
        for (int e = 0; e < 4; ++e) bu[e] = T[(4 * q4 + e) * TS + 16 * n + l16];
        Wacc[n] = mfma16(ph, bu, Wacc[n]);
        Wacc[n] = mfma16(pl, bu, Wacc[n]);
      }
      wave_sync_lds();
    }
  }

  // ---- exact rows: two 16-row tiles in flight
  if (n_ex > 0) {
    f16* Vt = reinterpret_cast<f16*>(my);
    while (ta < ntile) {
      exact_tile<NQ>(ka, va, ta * 16, n_ex, qf, scale, st, Wacc, Vt, l16, q4);
      ta += 2 * kAttWaves;
      if (ta < ntile) load_exact_tile(exk, exv, ta, ntile, n_ex, ka, va, l16, q4);
      if (tb < ntile) {
        exact_tile<NQ>(kb, vb, tb * 16, n_ex, qf, scale, st, Wacc, Vt, l16, q4);
        tb += 2 * kAttWaves;
        if (tb < ntile) load_exact_tile(exk, exv, tb, ntile, n_ex, kb, vb, l16, q4);
      }
    }
  }

  // ---- final phase: common maximum, fixed-order reduction
  if (q4 == 0) {
    wstat[wave * 16 + l16] = st.m;
    wstat[kAttWaves * 16 + wave * 16 + l16] = st.l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, wstat[w * 16 + l16]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kAttWaves; ++w) {
    const float mw = wstat[w * 16 + l16];
    L += (mw == -INFINITY) ? 0.f : wstat[kAttWaves * 16 + w * 16 + l16] * __expf(mw - M);
  }
  float be[4];
  rows_of((st.m == -INFINITY) ? 0.f : __expf(st.m - M), q4, be);
  __syncthreads();  // per-wave scratch becomes the reduction buffer
  float* redO = reinterpret_cast<float*>(region);              // [4][16][kRedStride]
  float* redW = redO + kAttWaves * 16 * kRedStride;            // [4][16][RQ]
  {
    float* dst = redO + wave * 16 * kRedStride;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(4 * q4 + e) * kRedStride + 16 * n + l16] = st.O[n][e] * be[e];
    }
  }
  if (NRQ > 0 && lr) {
    float* dst = redW + wave * 16 * RQ;
#pragma unroll
    for (int n = 0; n < NRQ; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(4 * q4 + e) * RQ + 16 * n + l16] = Wacc[n][e] * be[e];
    }
  }
  __syncthreads();
  v4h wh[NQ], wl[NQ];
  if (NRQ > 0 && lr) {
#pragma unroll
    for (int s = 0; s < NRQ; ++s) {
      float4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int lw = 0; lw < kAttWaves; ++lw) {
        const float4 x = *reinterpret_cast<const float4*>(redW + lw * 16 * RQ + l16 * RQ + 16 * s + 4 * q4);
        w.x += x.x;
        w.y += x.y;
        w.z += x.z;
        w.w += x.w;
      }
      split_hl(w.x, w.y, w.z, w.w, wh[s], wl[s]);
    }
  }
  float Le[4];
  rows_of(L, q4, Le);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int n = wave + kAttWaves * half;  // output columns 16 n .. 16 n + 15
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += redO[w * 16 * kRedStride + (4 * q4 + e) * kRedStride + 16 * n + l16];
    }
    if (NRQ > 0 && lr) {
#pragma unroll
      for (int s = 0; s < NRQ; ++s) {
        v4h bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = vvx[(16 * s + 4 * q4 + e) * kVStride + 16 * n + l16];
        acc = mfma16(wh[s], bv, acc);
        acc = mfma16(wl[s], bv, acc);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int g = 4 * q4 + e;
      if (g < G)
        st_dev(&A.part_o[((int64_t)(row0 + g) * A.n_parts + part) * kD + 16 * n + l16],
               (Le[e] > 0.f) ? acc[e] / Le[e] : 0.f);
    }
  }
  if (wave == 0 && q4 == 0 && l16 < G)
    st_dev(&A.part_lse[(int64_t)(row0 + l16) * A.n_parts + part], (L > 0.f) ? M + __logf(L) : -INFINITY);
}

template <int NRQ>
__global__ __launch_bounds__(kAttThreads, 2) void k_attend(PoolArgs P, BatchArgs Bt, AttnArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int item = blockIdx.x;
  attend_part<NRQ>(P, Bt, A, item / A.items_per_unit, item % A.items_per_unit, kSlotLookup, smem);
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine: one workgroup of 4 waves per query row; wave w takes
// parts w, w + 4, ... (16 at a time, all loads in flight); fixed-order sums.
// ----------------------------------------------------------------------------

constexpr int kMergeThreads = 256;
constexpr int kMergeUnroll = 16;

__global__ __launch_bounds__(kMergeThreads) void k_merge(const float* part_o, const float* part_lse,
                                                        int n_parts, int n_rows, f16* out, float* out_lse) {
  __shared__ float red[4][kD];
  __shared__ float redS[4];
  __shared__ float redM[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const float* L = part_lse + (int64_t)row * n_parts;
  float M = -INFINITY;
  for (int p = tid; p < n_parts; p += kMergeThreads) M = fmaxf(M, L[p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) redM[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(redM[0], redM[1]), fmaxf(redM[2], redM[3]));
  float ax = 0.f, ay = 0.f, S = 0.f;
  if (M != -INFINITY) {
    for (int p0 = wave; p0 < n_parts; p0 += 4 * kMergeUnroll) {
      float lp[kMergeUnroll];
      float2 o[kMergeUnroll];
#pragma unroll
      for (int k = 0; k < kMergeUnroll; ++k) {
        const int p = p0 + 4 * k;
        const bool in = p < n_parts;
        const int pc = in ? p : 0;
        const float l = L[pc];
        const float2 v = *reinterpret_cast<const float2*>(part_o + ((int64_t)row * n_parts + pc) * kD + 2 * lane);
        lp[k] = in ? l : -INFINITY;
        o[k] = in ? v : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kMergeUnroll; ++k) {
        const float w = (lp[k] == -INFINITY) ? 0.f : __expf(lp[k] - M);
        S += w;
        ax += w * o[k].x;
        ay += w * o[k].y;
      }
    }
  }
  red[wave][2 * lane] = ax;
  red[wave][2 * lane + 1] = ay;
  if (lane == 0) redS[wave] = S;
  __syncthreads();
  if (wave == 0) {
    const float St = ((redS[0] + redS[1]) + redS[2]) + redS[3];
    const float x = ((red[0][2 * lane] + red[1][2 * lane]) + red[2][2 * lane]) + red[3][2 * lane];
    const float y = ((red[0][2 * lane + 1] + red[1][2 * lane + 1]) + red[2][2 * lane + 1]) + red[3][2 * lane + 1];
    const bool any = St > 0.f;
    f16* dst = out + (int64_t)row * kD + 2 * lane;
    dst[0] = (f16)(any ? x / St : 0.f);
    dst[1] = (f16)(any ? y / St : 0.f);
    if (lane == 0) out_lse[row] = any ? M + __logf(St) : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine of the G query rows of one (sequence, KV head) unit by
// one workgroup: 8 rows at a time, 32 lanes per row, 4 columns per lane.
// ----------------------------------------------------------------------------

__device__ __forceinline__ void merge_unit(const float* part_o, const float* part_lse, int n_parts, int row0,
                                           int G, f16* out, float* out_lse) {
  constexpr int kChunk = 32;
  const int tid = threadIdx.x;
  const int j = tid & 31;   // lane within the row's 32-lane group: columns 4 j .. 4 j + 3
  const int grp = tid >> 5;
  for (int g0 = 0; g0 < G; g0 += kAttThreads / 32) {
    const int g = g0 + grp;
    const bool valid = g < G;
    const int row = row0 + (valid ? g : 0);
    const float* Lrow = part_lse + (int64_t)row * n_parts;
    const float* Orow = part_o + (int64_t)row * n_parts * kD + 4 * j;
    float m = -INFINITY, S = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int pb = 0; pb < n_parts; pb += kChunk) {
      // every load of the chunk first: its lse values (one per lane) and its partials
      const int pl = pb + j;
      const float lj = Lrow[pl < n_parts ? pl : 0];
      float4 o[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int pk = pb + k < n_parts ? pb + k : 0;
        o[k] = *reinterpret_cast<const float4*>(Orow + (int64_t)pk * kD);
      }
      const float l = (pl < n_parts) ? lj : -INFINITY;
      float cm = l;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 32));
      const float mn = fmaxf(m, cm);
      if (mn == -INFINITY) continue;   // uniform within the row group
      const float alpha = (m == -INFINITY) ? 0.f : __expf(m - mn);
      const float w = (l == -INFINITY) ? 0.f : __expf(l - mn);
      float ws = w;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) ws += __shfl_xor(ws, off, 32);
      S = S * alpha + ws;
      acc.x *= alpha;
      acc.y *= alpha;
      acc.z *= alpha;
      acc.w *= alpha;
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const float wk = (pb + k < n_parts) ? __shfl(w, k, 32) : 0.f;
        acc.x += wk * o[k].x;
        acc.y += wk * o[k].y;
        acc.z += wk * o[k].z;
        acc.w += wk * o[k].w;
      }
      m = mn;
    }
    if (valid) {
      const bool any = S > 0.f;
      v4h h4;
      h4[0] = (f16)(any ? acc.x / S : 0.f);
      h4[1] = (f16)(any ? acc.y / S : 0.f);
      h4[2] = (f16)(any ? acc.z / S : 0.f);
      h4[3] = (f16)(any ? acc.w / S : 0.f);
      *reinterpret_cast<v4h*>(out + (int64_t)row * kD + 4 * j) = h4;
      if (j == 0) out_lse[row] = any ? m + __logf(S) : -INFINITY;
    }
  }
}

// ----------------------------------------------------------------------------
// One decode step of one layer in a single launch.
//
// Work items, handed out in ticket order (an atomic counter, so an item is
// only ever taken by a workgroup that is already running): first the routing
// of every (sequence, KV head) unit, then per unit its routed blocks and its
// window chunks.  A block item waits (bounded) until its unit's routing flag
// is set; routing items precede it in ticket order and are held by running
// workgroups, so the wait always ends.  The workgroup that completes a unit's
// last part merges that unit's partials; the workgroup that finishes last
// leaves the control words zeroed for the next launch.
// ----------------------------------------------------------------------------

struct DecodeArgs {
  AttnArgs att;
  int32_t* idx;          // [units][top_k] routed logical blocks
  int32_t* slots;        // [units][top_k] routed pool slots (-1: none); kSlotPending until routed
  uint32_t* ctrl;        // [0] ticket, [1] finished workgroups, [2] sticky wait-timeout flag
  uint32_t* unit_done;   // [units] parts finished
  f16* out;
  float* out_lse;
  int n_units;
  int n_route;           // units routed in this launch (0 when top_k == 0)
  int n_items;           // n_route + n_units * att.items_per_unit: the grid size
};

constexpr unsigned kRouteWaitLimit = 1u << 24;  // polls before giving up

template <int NRQ>
__global__ __launch_bounds__(kAttThreads, 2) void k_decode(PoolArgs P, BatchArgs Bt, DecodeArgs D) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ RouteShared<kAttWaves> rsh;
  __shared__ uint32_t sh_ticket, sh_flag;
  __shared__ int32_t sh_slot;
  const int tid = threadIdx.x;
  if (tid == 0) sh_ticket = atomicAdd(&D.ctrl[0], 1u);
  __syncthreads();
  const int t = (int)sh_ticket;
  if (t < D.n_route) {
    route_unit<kAttThreads>(P, Bt, t, D.att.top_k, D.idx, nullptr, D.slots, reinterpret_cast<uint32_t*>(smem), rsh);
  } else if (t < D.n_items) {
    const int it = t - D.n_route;
    const int u = it / D.att.items_per_unit, p = it % D.att.items_per_unit;
    int slot = kSlotLookup;
    if (p < D.att.n_block_parts) {
      // wait (bounded) until the unit's routing has written this part's pool slot
      if (tid == 0) {
        const int32_t* sp = &D.slots[(int64_t)u * D.att.top_k + p];
        unsigned n = 0;
        int32_t v = ld_dev(sp);
        while (v == kSlotPending && n < kRouteWaitLimit) {
          __builtin_amdgcn_s_sleep(1);
          v = ld_dev(sp);
          ++n;
        }
        if (v == kSlotPending) {
          atomicOr(&D.ctrl[2], 1u);
          v = -1 + kSlotCode;  // give up: an empty part
        }
        sh_slot = v - kSlotCode;
      }
      __syncthreads();
      slot = sh_slot;
    }
    attend_part<NRQ>(P, Bt, D.att, u, p, slot, smem);
    // count this part once its partial is stored; the unit's last part merges
    stores_done();
    __syncthreads();
    if (tid == 0) sh_flag = (atomicAdd(&D.unit_done[u], 1u) == (uint32_t)(D.att.items_per_unit - 1)) ? 1u : 0u;
    __syncthreads();
    if (sh_flag) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale cached copies of the partials
      const int b = u / Bt.Hkv, h = u % Bt.Hkv;
      merge_unit(D.att.part_o, D.att.part_lse, D.att.n_parts, b * Bt.Hq + h * Bt.G, Bt.G, D.out, D.out_lse);
    }
  }
  // the last workgroup to finish zeroes the control words for the next launch
  __syncthreads();
  if (tid == 0) sh_flag = (atomicAdd(&D.ctrl[1], 1u) == (uint32_t)(D.n_items - 1)) ? 1u : 0u;
  __syncthreads();
  if (sh_flag) {
    for (int i = tid; i < D.n_units; i += kAttThreads) D.unit_done[i] = 0u;
    for (int i = tid; i < D.n_route * D.att.top_k; i += kAttThreads) D.slots[i] = kSlotPending;  // 0
    if (tid == 0) {
      D.ctrl[0] = 0u;
      D.ctrl[1] = 0u;
    }
  }
}

__global__ void k_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// ----------------------------------------------------------------------------
// Host side: validation and launches
// ----------------------------------------------------------------------------

bool al(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

dkv_status check_view(const dkv_view& v, const char* name, int esz, int align) {
  if (!v.ptr) return fail(DKV_ERR_INVALID_ARG, "pool->%s.ptr is NULL", name);
  if (!al(v.ptr, align) || (v.slot_stride * esz) % align != 0 || (v.head_stride * esz) % align != 0)
    return fail(DKV_ERR_UNSUPPORTED, "pool->%s must be %d-byte aligned (pointer and strides)", name, align);
  return DKV_OK;
}

dkv_status check_pool_shape(const dkv_pool* P) {
  if (!P) return fail(DKV_ERR_INVALID_ARG, "pool is NULL");
  if (P->head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", P->head_dim);
  if (P->block_size != DKV_BLOCK_SIZE) return fail(DKV_ERR_UNSUPPORTED, "block_size %d != 256", P->block_size);
  if (P->rank < 1) return fail(DKV_ERR_INVALID_ARG, "rank %d < 1", P->rank);
  if (P->rank > DKV_MAX_RANK) return fail(DKV_ERR_UNSUPPORTED, "rank %d > 64", P->rank);
  if (P->n_resid < 0) return fail(DKV_ERR_INVALID_ARG, "n_resid %d < 0", P->n_resid);
  if (P->n_resid > DKV_MAX_RESID) return fail(DKV_ERR_UNSUPPORTED, "n_resid %d > 255", P->n_resid);
  if (P->n_kv_heads < 1) return fail(DKV_ERR_INVALID_ARG, "n_kv_heads %d < 1", P->n_kv_heads);
  if (P->n_slots < 0) return fail(DKV_ERR_INVALID_ARG, "n_slots %d < 0", P->n_slots);
  return DKV_OK;
}

// which: bit 0 low-rank arrays, bit 1 residual arrays, bit 2 route key
dkv_status check_pool_arrays(const dkv_pool* P, int which) {
  dkv_status s;
  if (which & 1) {
    if ((s = check_view(P->anchor_k, "anchor_k", 2, 16))) return s;
    if ((s = check_view(P->anchor_v, "anchor_v", 2, 16))) return s;
    // U rows are read 4 halves at a time when the rank is a multiple of 4
    if ((s = check_view(P->u, "u", 2, (P->rank % 4 == 0) ? 8 : 2))) return s;
    if ((s = check_view(P->vk, "vk", 2, 16))) return s;
    if ((s = check_view(P->vv, "vv", 2, 16))) return s;
  }
  if ((which & 1) || (which & 2)) {
    if (P->n_resid > 0 && (which & 1))
      if ((s = check_view(P->resid_pos, "resid_pos", 1, 1))) return s;
  }
  if ((which & 2) && P->n_resid > 0) {
    if ((s = check_view(P->resid_k, "resid_k", 2, 16))) return s;
    if ((s = check_view(P->resid_v, "resid_v", 2, 16))) return s;
  }
  if (which & 4)
    if ((s = check_view(P->route_key, "route_key", 4, 16))) return s;
  return DKV_OK;
}

dkv_status check_batch(const dkv_pool* P, const dkv_batch* B, bool need_table, bool need_window) {
  if (!B) return fail(DKV_ERR_INVALID_ARG, "batch is NULL");
  if (B->batch < 0) return fail(DKV_ERR_INVALID_ARG, "batch %d < 0", B->batch);
  if (B->n_q_heads < 1) return fail(DKV_ERR_INVALID_ARG, "n_q_heads %d < 1", B->n_q_heads);
  if (B->n_q_heads % P->n_kv_heads != 0)
    return fail(DKV_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", B->n_q_heads, P->n_kv_heads);
  if (B->n_q_heads / P->n_kv_heads > DKV_MAX_GROUP)
    return fail(DKV_ERR_UNSUPPORTED, "query heads per KV head %d > 16", B->n_q_heads / P->n_kv_heads);
  if (B->window < 0) return fail(DKV_ERR_INVALID_ARG, "window %d < 0", B->window);
  if (B->max_blocks < 0) return fail(DKV_ERR_INVALID_ARG, "max_blocks %d < 0", B->max_blocks);
  if (B->batch == 0) return DKV_OK;
  if (!B->q) return fail(DKV_ERR_INVALID_ARG, "batch->q is NULL");
  if (!al(B->q, 16)) return fail(DKV_ERR_UNSUPPORTED, "batch->q must be 16-byte aligned");
  if (need_table && B->max_blocks > 0) {
    if (!B->block_table) return fail(DKV_ERR_INVALID_ARG, "batch->block_table is NULL");
    if (!B->n_blocks) return fail(DKV_ERR_INVALID_ARG, "batch->n_blocks is NULL");
  }
  if (need_window && B->window > 0) {
    if (!B->win_k || !B->win_v) return fail(DKV_ERR_INVALID_ARG, "batch->win_k / win_v is NULL");
    if (!al(B->win_k, 16) || !al(B->win_v, 16))
      return fail(DKV_ERR_UNSUPPORTED, "batch->win_k / win_v must be 16-byte aligned");
  }
  return DKV_OK;
}

PoolArgs make_pool_args(const dkv_pool* P) {
  PoolArgs a;
  a.ak = (const f16*)P->anchor_k.ptr; a.ak_s = P->anchor_k.slot_stride; a.ak_h = P->anchor_k.head_stride;
  a.av = (const f16*)P->anchor_v.ptr; a.av_s = P->anchor_v.slot_stride; a.av_h = P->anchor_v.head_stride;
  a.u = (const f16*)P->u.ptr; a.u_s = P->u.slot_stride; a.u_h = P->u.head_stride;
  a.vk = (const f16*)P->vk.ptr; a.vk_s = P->vk.slot_stride; a.vk_h = P->vk.head_stride;
  a.vv = (const f16*)P->vv.ptr; a.vv_s = P->vv.slot_stride; a.vv_h = P->vv.head_stride;
  a.rk = (const f16*)P->resid_k.ptr; a.rk_s = P->resid_k.slot_stride; a.rk_h = P->resid_k.head_stride;
  a.rv = (const f16*)P->resid_v.ptr; a.rv_s = P->resid_v.slot_stride; a.rv_h = P->resid_v.head_stride;
  a.rp = (const uint8_t*)P->resid_pos.ptr; a.rp_s = P->resid_pos.slot_stride; a.rp_h = P->resid_pos.head_stride;
  a.key = (float*)P->route_key.ptr; a.key_s = P->route_key.slot_stride; a.key_h = P->route_key.head_stride;
  a.rank = P->rank;
  a.n_resid = P->n_resid;
  a.n_kv = P->n_kv_heads;
  a.n_slots = P->n_slots;
  return a;
}

BatchArgs make_batch_args(const dkv_pool* P, const dkv_batch* B) {
  BatchArgs a;
  a.B = B->batch;
  a.Hq = B->n_q_heads;
  a.Hkv = P->n_kv_heads;
  a.G = B->n_q_heads / P->n_kv_heads;
  a.W = B->window;
  a.mb = B->max_blocks;
  a.table = B->block_table;
  a.nblk = B->n_blocks;
  a.wlen = B->win_len;
  a.q = (const f16*)B->q;
  a.wk = (const f16*)B->win_k;
  a.wv = (const f16*)B->win_v;
  return a;
}

dkv_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DKV_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DKV_OK;
}

int rq_of(int rank) { return ((rank + 1 + 15) / 16) * 16; }

// routing scratch: an ordered score key and a pool slot per logical block
size_t route_lds_bytes(int max_blocks) { return (size_t)2 * (max_blocks > 0 ? max_blocks : 1) * sizeof(uint32_t); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

dkv_status launch_route(const dkv_pool* P, const dkv_batch* B, int top_k, int32_t* idx, float* scores,
                        int32_t* slots, hipStream_t st) {
  const int units = B->batch * P->n_kv_heads;
  if (units == 0) return DKV_OK;
  const size_t shm = route_lds_bytes(B->max_blocks);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_route_topk, hipFuncAttributeMaxDynamicSharedMemorySize, 152 * 1024) !=
        hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_route_topk) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL(k_route_topk, dim3(units), dim3(kRouteThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), top_k, idx, scores, slots);
  return launched("k_route_topk");
}

template <int NRQ>
dkv_status launch_decode_nrq(size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B, const DecodeArgs& D) {
  static bool attr_set = false;
  if (!attr_set) {
    // 160 KB of LDS per workgroup on gfx950, less this kernel's static shared memory
    if (hipFuncSetAttribute((const void*)k_decode<NRQ>, hipFuncAttributeMaxDynamicSharedMemorySize, 158 * 1024) !=
        hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_decode) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL(k_decode<NRQ>, dim3((unsigned)D.n_items), dim3(kAttThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), D);
  return launched("k_decode");
}

template <int NRQ>
dkv_status launch_attend_nrq(int64_t items, size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B,
                             const AttnArgs& a) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_attend<NRQ>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
        hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_attend) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL(k_attend<NRQ>, dim3((unsigned)items), dim3(kAttThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), a);
  return launched("k_attend");
}

dkv_status launch_attend(const dkv_pool* P, const dkv_batch* B, const int32_t* idx, const int32_t* slots,
                         int top_k, int n_block_parts, int block_mode, int n_win_parts, int win_chunk,
                         float scale, float* part_o, float* part_lse, int n_parts, int part_offset,
                         hipStream_t st) {
  const int per_unit = n_block_parts + n_win_parts;
  const int64_t items = (int64_t)B->batch * P->n_kv_heads * per_unit;
  if (items == 0) return DKV_OK;
  if (items > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many attention parts (%lld)", (long long)items);
  AttnArgs a;
  a.idx = idx;
  a.top_k = top_k;
  a.n_block_parts = n_block_parts;
  a.block_mode = block_mode;
  a.n_win_parts = n_win_parts;
  a.win_chunk = win_chunk;
  a.items_per_unit = per_unit;
  a.rq = (n_block_parts > 0 && (block_mode & 1)) ? rq_of(P->rank) : 0;
  a.scale = scale;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.n_parts = n_parts;
  a.part_offset = part_offset;
  const size_t shm = (size_t)att_lds_bytes(a.rq);
  switch (a.rq / 16) {
    case 0: return launch_attend_nrq<0>(items, shm, st, P, B, a);
    case 1: return launch_attend_nrq<1>(items, shm, st, P, B, a);
    case 2: return launch_attend_nrq<2>(items, shm, st, P, B, a);
    case 3: return launch_attend_nrq<3>(items, shm, st, P, B, a);
    case 4: return launch_attend_nrq<4>(items, shm, st, P, B, a);
    case 5: return launch_attend_nrq<5>(items, shm, st, P, B, a);
    default: return fail(DKV_ERR_UNSUPPORTED, "rank %d", P->rank);
  }
}

dkv_status launch_merge(const float* part_o, const float* part_lse, int n_parts, int n_rows, void* out,
                        float* out_lse, hipStream_t st) {
  if (n_rows == 0) return DKV_OK;
  hipLaunchKernelGGL(k_merge, dim3((unsigned)n_rows), dim3(kMergeThreads), 0, st, part_o, part_lse, n_parts, n_rows,
                     (f16*)out, out_lse);
  return launched("k_merge");
}

int win_parts_of(int window) { return (window + kWinChunk - 1) / kWinChunk; }

// dkv_decode gives every unit at least one window part, so that a unit with
// neither routed blocks nor window rows still produces its (empty) output
int decode_win_parts(int window) {
  const int n = win_parts_of(window);
  return n > 0 ? n : 1;
}

// Workspace of dkv_decode: a control area (ticket, counters, per-unit flags;
// zero between calls), then routed indices and slots, then the partials.
struct WsLayout {
  size_t ctrl_bytes, unit_done, slots, idx, part_lse, part_o, total;
};

WsLayout decode_layout(const dkv_pool* pool, const dkv_batch* batch, int top_k) {
  WsLayout w;
  const size_t B = (size_t)batch->batch;
  const size_t units = B * (size_t)pool->n_kv_heads;
  const size_t n_parts = (size_t)top_k + (size_t)decode_win_parts(batch->window);
  const size_t rows = B * (size_t)batch->n_q_heads;
  w.unit_done = 256;
  w.slots = w.unit_done + align256(units * 4);
  w.ctrl_bytes = w.slots + align256(units * (size_t)top_k * 4);
  w.idx = w.ctrl_bytes;
  w.part_lse = w.idx + align256(units * (size_t)top_k * 4);
  w.part_o = w.part_lse + align256(rows * n_parts * 4);
  w.total = w.part_o + align256(rows * n_parts * kD * 4);
  return w;
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

extern "C" {

const char* dkv_status_string(dkv_status s) {
  switch (s) {
    case DKV_OK: return "DKV_OK";
    case DKV_ERR_INVALID_ARG: return "DKV_ERR_INVALID_ARG";
    case DKV_ERR_UNSUPPORTED: return "DKV_ERR_UNSUPPORTED";
    case DKV_ERR_WORKSPACE: return "DKV_ERR_WORKSPACE";
    case DKV_ERR_HIP: return "DKV_ERR_HIP";
    default: return "DKV_ERR_UNKNOWN";
  }
}

const char* dkv_last_error(void) { return g_err; }

int32_t dkv_abi_version(void) { return DKV_ABI_VERSION; }

dkv_status dkv_route_keys(const dkv_pool* pool, const int32_t* slots, int32_t n_list, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if ((s = check_pool_arrays(pool, 1 | 4))) return s;
  if (slots && n_list < 0) return fail(DKV_ERR_INVALID_ARG, "n_list %d < 0", n_list);
  const int64_t n = (int64_t)(slots ? n_list : pool->n_slots) * pool->n_kv_heads;
  if (n == 0) return DKV_OK;
  if (n > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many slots");
  hipLaunchKernelGGL(k_route_keys, dim3((unsigned)n), dim3(128), 0, (hipStream_t)stream,
                     make_pool_args(pool), slots);
  return launched("k_route_keys");
}

dkv_status dkv_route_topk(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, int32_t* idx,
                          float* scores, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 1) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 1", top_k);
  if ((s = check_batch(pool, batch, true, false))) return s;
  if (batch->max_blocks > DKV_MAX_ROUTE_BLOCKS)
    return fail(DKV_ERR_UNSUPPORTED, "max_blocks %d > %d", batch->max_blocks, DKV_MAX_ROUTE_BLOCKS);
  if (batch->batch == 0) return DKV_OK;
  if (!idx) return fail(DKV_ERR_INVALID_ARG, "idx is NULL");
  if (batch->max_blocks > 0 && (s = check_pool_arrays(pool, 4))) return s;
  return launch_route(pool, batch, top_k, idx, scores, nullptr, (hipStream_t)stream);
}

dkv_status dkv_lowrank_attn(const dkv_pool* pool, const dkv_batch* batch, const int32_t* idx, int32_t top_k,
                            float scale, float* part_o, float* part_lse, int32_t n_parts, int32_t part_offset,
                            void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 1) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 1", top_k);
  if ((s = check_batch(pool, batch, true, false))) return s;
  if (part_offset < 0 || n_parts < part_offset + top_k)
    return fail(DKV_ERR_INVALID_ARG, "parts [%d, %d) do not fit n_parts %d", part_offset, part_offset + top_k, n_parts);
  if (batch->batch == 0) return DKV_OK;
  if (!idx || !part_o || !part_lse) return fail(DKV_ERR_INVALID_ARG, "idx / part_o / part_lse is NULL");
  if ((s = check_pool_arrays(pool, 1))) return s;
  return launch_attend(pool, batch, idx, nullptr, top_k, top_k, 1, 0, kWinChunk, scale, part_o, part_lse,
                       n_parts, part_offset, (hipStream_t)stream);
}

dkv_status dkv_exact_attn(const dkv_pool* pool, const dkv_batch* batch, const int32_t* idx, int32_t top_k,
                          int32_t window_splits, float scale, float* part_o, float* part_lse, int32_t n_parts,
                          int32_t part_offset, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 0) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if (!idx && top_k != 0) return fail(DKV_ERR_INVALID_ARG, "idx is NULL but top_k = %d", top_k);
  if (window_splits < 0) return fail(DKV_ERR_INVALID_ARG, "window_splits %d < 0", window_splits);
  if ((s = check_batch(pool, batch, top_k > 0, window_splits > 0))) return s;
  if (part_offset < 0 || n_parts < part_offset + top_k + window_splits)
    return fail(DKV_ERR_INVALID_ARG, "parts [%d, %d) do not fit n_parts %d", part_offset,
                part_offset + top_k + window_splits, n_parts);
  if (batch->batch == 0 || top_k + window_splits == 0) return DKV_OK;
  if (!part_o || !part_lse) return fail(DKV_ERR_INVALID_ARG, "part_o / part_lse is NULL");
  if (top_k > 0 && (s = check_pool_arrays(pool, 2))) return s;
  const int chunk = window_splits > 0 ? (batch->window + window_splits - 1) / window_splits : 1;
  return launch_attend(pool, batch, idx, nullptr, top_k, top_k, 2, window_splits, chunk > 0 ? chunk : 1, scale,
                       part_o, part_lse, n_parts, part_offset, (hipStream_t)stream);
}

dkv_status dkv_lse_merge(const float* part_o, const float* part_lse, int32_t n_parts, int32_t n_rows,
                         int32_t head_dim, void* out, float* out_lse, void* stream) {
  g_err[0] = 0;
  if (head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", head_dim);
  if (n_parts < 0 || n_rows < 0) return fail(DKV_ERR_INVALID_ARG, "negative n_parts / n_rows");
  if (n_rows == 0) return DKV_OK;
  if (!out || !out_lse) return fail(DKV_ERR_INVALID_ARG, "out / out_lse is NULL");
  if (n_parts > 0 && (!part_o || !part_lse)) return fail(DKV_ERR_INVALID_ARG, "part_o / part_lse is NULL");
  if (!al(part_o, 8) || !al(out, 4)) return fail(DKV_ERR_UNSUPPORTED, "part_o / out misaligned");
  return launch_merge(part_o, part_lse, n_parts, n_rows, out, out_lse, (hipStream_t)stream);
}

size_t dkv_decode_workspace_size(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k) {
  if (!pool || !batch || top_k < 0 || batch->batch < 0 || batch->window < 0 || batch->n_q_heads < 1 ||
      pool->n_kv_heads < 1)
    return 0;
  return decode_layout(pool, batch, top_k).total;
}

dkv_status dkv_decode_workspace_init(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 0) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if ((s = check_batch(pool, batch, false, false))) return s;
  const WsLayout w = decode_layout(pool, batch, top_k);
  if (!workspace || workspace_bytes < w.total)
    return fail(DKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                w.total);
  if (!al(workspace, 256)) return fail(DKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int words = (int)(w.ctrl_bytes / 4);
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)workspace, words);
  return launched("k_zero_words");
}

static dkv_status decode_impl(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale,
                              void* workspace, size_t workspace_bytes, void* out, float* out_lse, int32_t* out_idx,
                              void* const* events, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 0) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if ((s = check_batch(pool, batch, top_k > 0, true))) return s;
  if (top_k > 0 && batch->max_blocks > DKV_MAX_ROUTE_BLOCKS)
    return fail(DKV_ERR_UNSUPPORTED, "max_blocks %d > %d", batch->max_blocks, DKV_MAX_ROUTE_BLOCKS);
  if (batch->batch == 0) return DKV_OK;
  if (!out || !out_lse) return fail(DKV_ERR_INVALID_ARG, "out / out_lse is NULL");
  if (!al(out, 4)) return fail(DKV_ERR_UNSUPPORTED, "out must be 4-byte aligned");
  const size_t need = dkv_decode_workspace_size(pool, batch, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(DKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if (!al(workspace, 256)) return fail(DKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (top_k > 0 && (s = check_pool_arrays(pool, 1 | 2 | 4))) return s;

  const hipStream_t st = (hipStream_t)stream;
  const WsLayout w = decode_layout(pool, batch, top_k);
  const int n_win = decode_win_parts(batch->window);
  const int n_parts = top_k + n_win;
  const int units = batch->batch * pool->n_kv_heads;
  unsigned char* ws = (unsigned char*)workspace;

  DecodeArgs D;
  AttnArgs& a = D.att;
  a.idx = nullptr;
  a.top_k = top_k;
  a.n_block_parts = top_k;
  a.block_mode = 3;
  a.n_win_parts = n_win;
  a.win_chunk = kWinChunk;
  a.items_per_unit = n_parts;
  a.rq = top_k > 0 ? rq_of(pool->rank) : 0;
  a.scale = scale;
  a.part_o = (float*)(ws + w.part_o);
  a.part_lse = (float*)(ws + w.part_lse);
  a.n_parts = n_parts;
  a.part_offset = 0;
  D.idx = out_idx ? out_idx : (int32_t*)(ws + w.idx);
  D.slots = (int32_t*)(ws + w.slots);
  D.ctrl = (uint32_t*)ws;
  D.unit_done = (uint32_t*)(ws + w.unit_done);
  D.out = (f16*)out;
  D.out_lse = out_lse;
  D.n_units = units;
  D.n_route = top_k > 0 ? units : 0;
  const int64_t items = (int64_t)D.n_route + (int64_t)units * n_parts;
  if (items > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many work items (%lld)", (long long)items);
  D.n_items = (int)items;
  size_t shm = (size_t)att_lds_bytes(a.rq);
  const size_t route_shm = route_lds_bytes(batch->max_blocks);
  if (top_k > 0 && route_shm > shm) shm = route_shm;

  if (events && hipEventRecord((hipEvent_t)events[0], st) != hipSuccess)
    return fail(DKV_ERR_HIP, "hipEventRecord failed");
  switch (a.rq / 16) {
    case 0: s = launch_decode_nrq<0>(shm, st, pool, batch, D); break;
    case 1: s = launch_decode_nrq<1>(shm, st, pool, batch, D); break;
    case 2: s = launch_decode_nrq<2>(shm, st, pool, batch, D); break;
    case 3: s = launch_decode_nrq<3>(shm, st, pool, batch, D); break;
    case 4: s = launch_decode_nrq<4>(shm, st, pool, batch, D); break;
    case 5: s = launch_decode_nrq<5>(shm, st, pool, batch, D); break;
    default: return fail(DKV_ERR_UNSUPPORTED, "rank %d", pool->rank);
  }
  if (s) return s;
  if (events && hipEventRecord((hipEvent_t)events[1], st) != hipSuccess)
    return fail(DKV_ERR_HIP, "hipEventRecord failed");
  return DKV_OK;
}

dkv_status dkv_decode(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale, void* workspace,
                      size_t workspace_bytes, void* out, float* out_lse, int32_t* out_idx, void* stream) {
  return decode_impl(pool, batch, top_k, scale, workspace, workspace_bytes, out, out_lse, out_idx, nullptr, stream);
}

dkv_status dkv_decode_profiled(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale,
                               void* workspace, size_t workspace_bytes, void* out, float* out_lse, int32_t* out_idx,
                               void* const* events, void* stream) {
  if (!events || !events[0] || !events[1]) {
    g_err[0] = 0;
    return fail(DKV_ERR_INVALID_ARG, "events must hold two hipEvent_t handles");
  }
  return decode_impl(pool, batch, top_k, scale, workspace, workspace_bytes, out, out_lse, out_idx, events, stream);
}

}  // extern "C"
