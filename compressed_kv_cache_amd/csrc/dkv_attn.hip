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
constexpr int kThreads = 256;      // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kLowRankRows = 255;  // tokens 1..255 of a block
constexpr int kVStride = 132;      // LDS row stride (halves) of 128-wide tiles: conflict-free column reads
constexpr int kWinChunk = 128;     // window rows per part in dkv_decode
constexpr int kMaxRQ = 80;         // augmented rank r + 1 rounded up to 16, r <= 64

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

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ v8h ld8(const f16* p) { return *reinterpret_cast<const v8h*>(p); }

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

// Exclusive count of `flag` over the workgroup in thread order, and the total.
__device__ __forceinline__ void block_count(bool flag, int& excl, int& total, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int in_wave = __popcll(m & lt);
  if (lane == 0) wsum[w] = (uint32_t)__popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
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
// Top-K routing
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_route_topk(PoolArgs P, BatchArgs Bt, int top_k,
                                                         int32_t* idx, float* scores) {
  extern __shared__ uint32_t keys[];  // [mb]
  __shared__ float qbar[kD];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t suf[256];
  __shared__ uint32_t wsum[kWaves];
  __shared__ int sh_digit;
  __shared__ uint32_t sh_above;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  int N = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  N = N < 0 ? 0 : (N > Bt.mb ? Bt.mb : N);
  const int keff = top_k < N ? top_k : N;

  if (tid < kD) {
    float s = 0.f;
    for (int g = 0; g < Bt.G; ++g) s += (float)Bt.q[((int64_t)b * Bt.Hq + h * Bt.G + g) * kD + tid];
    qbar[tid] = s / (float)Bt.G;
  }
  __syncthreads();

  const float q0 = qbar[2 * lane], q1 = qbar[2 * lane + 1];
  for (int j = wave; j < N; j += kWaves) {
    const int slot = Bt.table[(int64_t)b * Bt.mb + j];
    const bool ok = slot >= 0 && slot < P.n_slots;
    float part = 0.f;
    if (ok) {
      const float2 c = *reinterpret_cast<const float2*>(P.key + slot * P.key_s + h * P.key_h + 2 * lane);
      part = q0 * c.x + q1 * c.y;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) keys[j] = ordered_key(ok ? part : -INFINITY);
  }
  __syncthreads();

  if (keff > 0) {
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t krem = (uint32_t)keff;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < N; j += kThreads) {
        const uint32_t k = keys[j];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      suf[tid] = hist[tid];
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const uint32_t add = (tid + off < 256) ? suf[tid + off] : 0u;
        __syncthreads();
        suf[tid] += add;
        __syncthreads();
      }
      const uint32_t nxt = (tid < 255) ? suf[tid + 1] : 0u;
      if (suf[tid] >= krem && nxt < krem) {
        sh_digit = tid;
        sh_above = nxt;
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= 0xFFu << shift;
      krem -= sh_above;
      __syncthreads();
    }
    const uint32_t T = prefix;
    int eq_base = 0, sel_base = 0;
    for (int c0 = 0; c0 < N; c0 += kThreads) {
      const int j = c0 + tid;
      const bool in = j < N;
      const uint32_t k = in ? keys[j] : 0u;
      const bool eq = in && k == T;
      int eq_rank, eq_tot;
      block_count(eq, eq_rank, eq_tot, wsum);
      const bool sel = in && (k > T || (eq && (uint32_t)(eq_base + eq_rank) < krem));
      int sel_rank, sel_tot;
      block_count(sel, sel_rank, sel_tot, wsum);
      if (sel) {
        const int pos = sel_base + sel_rank;
        idx[(int64_t)u * top_k + pos] = j;
        if (scores) scores[(int64_t)u * top_k + pos] = from_ordered(k);
      }
      eq_base += eq_tot;
      sel_base += sel_tot;
    }
  }
  for (int pos = keff + tid; pos < top_k; pos += kThreads) {
    idx[(int64_t)u * top_k + pos] = -1;
    if (scores) scores[(int64_t)u * top_k + pos] = -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// Attention over one part: a routed block (low-rank and/or residual rows) or a
// chunk of window rows.  One workgroup of 4 waves per part.
// ----------------------------------------------------------------------------

__host__ __device__ inline int wave_region_bytes(int rq) {
  int a = 16 * kVStride * 2;            // V tile, fp16
  const int b = 16 * (rq + 4) * 2;      // Ux tile, fp16
  const int c = 16 * rq * 4;            // W transpose, fp32
  if (b > a) a = b;
  if (c > a) a = c;
  return (a + 15) & ~15;
}

__host__ __device__ inline int attend_lds_bytes(int rq) {
  return 16 * rq * 4                    // V_K q (fp32) [16][rq]
         + rq * kVStride * 2            // VVx staged [rq][132] fp16
         + 8 * 4                        // residual-position mask
         + 2 * kWaves * 16 * 4          // per-wave softmax statistics
         + kWaves * wave_region_bytes(rq);
}

__global__ __launch_bounds__(kThreads) void k_attend(PoolArgs P, BatchArgs Bt, AttnArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int item = blockIdx.x;
  const int u = item / A.items_per_unit, p = item % A.items_per_unit;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  const int G = Bt.G;
  const int row0 = b * Bt.Hq + h * G;

  // ---- what this part covers (uniform over the workgroup)
  bool lr = false;
  int n_ex = 0;
  const f16* exk = nullptr;
  const f16* exv = nullptr;
  int slot = -1;
  if (p < A.n_block_parts) {
    int nb = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
    nb = nb < 0 ? 0 : (nb > Bt.mb ? Bt.mb : nb);
    const int j = A.idx[(int64_t)u * A.top_k + p];
    if (j >= 0 && j < nb) {
      const int s = Bt.table[(int64_t)b * Bt.mb + j];
      if (s >= 0 && s < P.n_slots) slot = s;
    }
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
    for (int t = tid; t < G * kD; t += kThreads) {
      const int g = t / kD, d = t % kD;
      A.part_o[((int64_t)(row0 + g) * A.n_parts + part) * kD + d] = 0.f;
    }
    if (tid < G) A.part_lse[(int64_t)(row0 + tid) * A.n_parts + part] = -INFINITY;
    return;
  }

  // ---- LDS carve-up
  const int RQ = A.rq;
  float* qt = reinterpret_cast<float*>(smem);                       // [16][RQ]
  f16* vvx = reinterpret_cast<f16*>(qt + 16 * RQ);                  // [RQ][kVStride]
  uint32_t* mask = reinterpret_cast<uint32_t*>(vvx + RQ * kVStride); // [8]
  float* wstat = reinterpret_cast<float*>(mask + 8);                 // m [4][16], l [4][16]
  unsigned char* wreg = reinterpret_cast<unsigned char*>(wstat + 2 * kWaves * 16);
  const int WREG = wave_region_bytes(RQ);
  unsigned char* my = wreg + wave * WREG;

  // ---- query fragments: lane holds q[g = l16][32 s + 8 q4 + 4 hh + e]
  v4h qf[4][2];
  {
    const bool ok = l16 < G;
    const f16* qrow = Bt.q + (int64_t)(row0 + l16) * kD + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v8h x = ok ? ld8(qrow + 32 * s) : (v8h)(f16)0;
      qf[s][0] = lo4(x);
      qf[s][1] = hi4(x);
    }
  }

  const int r = P.rank;
  const int nrq = RQ / 16;
  v4h qth[5], qtl[5];
#pragma unroll
  for (int s = 0; s < 5; ++s) { qth[s] = (v4h)(f16)0; qtl[s] = (v4h)(f16)0; }
  const f16* U = nullptr;
  if (lr) {
    const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
    const f16* AV = P.av + slot * P.av_s + h * P.av_h;
    const f16* VK = P.vk + slot * P.vk_s + h * P.vk_h;
    const f16* VV = P.vv + slot * P.vv_s + h * P.vv_h;
    U = P.u + slot * P.u_s + h * P.u_h;
    if (tid < 8) mask[tid] = 0u;
    // VVx = [V_V ; a_v ; 0] staged in LDS
    for (int c = tid; c < RQ * 16; c += kThreads) {
      const int j = c >> 4, col = (c & 15) * 8;
      v8h x = (v8h)(f16)0;
      if (j < r) x = ld8(VV + (int64_t)j * kD + col);
      else if (j == r) x = ld8(AV + col);
      *reinterpret_cast<v4h*>(vvx + j * kVStride + col) = lo4(x);
      *reinterpret_cast<v4h*>(vvx + j * kVStride + col + 4) = hi4(x);
    }
    // VKx q: rows j of [V_K ; a_k ; 0] against the G queries, C rows j, columns g
    for (int jt = wave; jt < nrq; jt += kWaves) {
      const int j = jt * 16 + l16;
      const f16* src = (j < r) ? VK + (int64_t)j * kD : ((j == r) ? AK : nullptr);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8h x = src ? ld8(src + 32 * s + 8 * q4) : (v8h)(f16)0;
        acc = mfma16(lo4(x), qf[s][0], acc);
        acc = mfma16(hi4(x), qf[s][1], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) qt[l16 * RQ + jt * 16 + 4 * q4 + e] = acc[e];
    }
    __syncthreads();
    const uint8_t* pos = P.rp + slot * P.rp_s + h * P.rp_h;
    for (int t = tid; t < P.n_resid; t += kThreads) {
      const int ps = pos[t];
      if (ps >= 1 && ps <= kLowRankRows) atomicOr(&mask[ps >> 5], 1u << (ps & 31));
    }
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      if (s < nrq) {
        const float4 x = *reinterpret_cast<const float4*>(qt + l16 * RQ + 16 * s + 4 * q4);
        split_hl(x.x, x.y, x.z, x.w, qth[s], qtl[s]);
      }
    }
    __syncthreads();
  }

  float m_run = -INFINITY, l_run = 0.f;
  v4f O[8];
  v4f Wacc[5];
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < 5; ++n) Wacc[n] = (v4f){0.f, 0.f, 0.f, 0.f};
  const float scale = A.scale;

  // ---- low-rank rows: 16 tiles of 16 positions (position 0 is the anchor)
  if (lr) {
    const bool uvec = (r & 3) == 0;
    const int TS = RQ + 4;
    f16* T = reinterpret_cast<f16*>(my);  // [16][RQ + 4] transpose buffer for Ux
    for (int tile = wave; tile < 16; tile += kWaves) {
      const int i0 = tile * 16;
      const int i = i0 + l16;
      v4h ua[5];
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        v4h x = (v4h)(f16)0;
        if (s < nrq) {
          const int j0 = 16 * s + 4 * q4;
          if (i > 0) {
            const f16* row = U + (int64_t)(i - 1) * r;
            if (uvec) {
              if (j0 < r) x = *reinterpret_cast<const v4h*>(row + j0);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (j0 + e < r) x[e] = row[j0 + e];
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e == r) x[e] = (f16)1.0f;
        }
        ua[s] = x;
      }
      v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        if (s < nrq) {
          z = mfma16(ua[s], qth[s], z);
          z = mfma16(ua[s], qtl[s], z);
        }
      }
      float zz[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = i0 + 4 * q4 + e;
        const bool masked = ii > 0 && ((mask[ii >> 5] >> (ii & 31)) & 1u);
        zz[e] = masked ? -INFINITY : z[e] * scale;
      }
      float alpha, pe[4], ae[4];
      softmax_tile(zz, m_run, l_run, alpha, pe);
      rows_of(alpha, q4, ae);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) O[n][e] *= ae[e];
      }
#pragma unroll
      for (int n = 0; n < 5; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Wacc[n][e] *= ae[e];
      }
      v4h ph, pl;
      split_hl(pe[0], pe[1], pe[2], pe[3], ph, pl);
#pragma unroll
      for (int s = 0; s < 5; ++s)
        if (s < nrq) *reinterpret_cast<v4h*>(T + l16 * TS + 16 * s + 4 * q4) = ua[s];
      wave_sync_lds();
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        if (n < nrq) {
          v4h bu;
#pragma unroll
          for (int e = 0; e < 4; ++e) bu[e] = T[(4 * q4 + e) * TS + 16 * n + l16];
          Wacc[n] = mfma16(ph, bu, Wacc[n]);
          Wacc[n] = mfma16(pl, bu, Wacc[n]);
        }
      }
      wave_sync_lds();
    }
  }

  // ---- exact rows (residual rows of a block, or window rows): 16-row tiles
  if (n_ex > 0) {
    const int ntile = (n_ex + 15) / 16;
    f16* Vt = reinterpret_cast<f16*>(my);  // [16][kVStride]
    for (int tile = wave; tile < ntile; tile += kWaves) {
      const int t0 = tile * 16;
      const int t = t0 + l16;
      const bool valid = t < n_ex;
      v8h kx[4], vx[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kx[s] = valid ? ld8(exk + (int64_t)t * kD + 32 * s + 8 * q4) : (v8h)(f16)0;
        vx[s] = valid ? ld8(exv + (int64_t)t * kD + 32 * s + 8 * q4) : (v8h)(f16)0;
      }
      v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        S = mfma16(lo4(kx[s]), qf[s][0], S);
        S = mfma16(hi4(kx[s]), qf[s][1], S);
      }
      float zz[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[e] = (t0 + 4 * q4 + e < n_ex) ? S[e] * scale : -INFINITY;
      float alpha, pe[4], ae[4];
      softmax_tile(zz, m_run, l_run, alpha, pe);
      rows_of(alpha, q4, ae);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) O[n][e] *= ae[e];
      }
#pragma unroll
      for (int n = 0; n < 5; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Wacc[n][e] *= ae[e];
      }
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
        O[n] = mfma16(ph, bv, O[n]);
        O[n] = mfma16(pl, bv, O[n]);
      }
      wave_sync_lds();
    }
  }

  // ---- low-rank values: O += (p^T Ux) VVx, once per wave
  if (lr) {
    float* Wt = reinterpret_cast<float*>(my);  // [16][RQ]
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      if (n < nrq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Wt[(4 * q4 + e) * RQ + 16 * n + l16] = Wacc[n][e];
      }
    }
    wave_sync_lds();
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      if (s < nrq) {
        const float4 w = *reinterpret_cast<const float4*>(Wt + l16 * RQ + 16 * s + 4 * q4);
        v4h wh, wl;
        split_hl(w.x, w.y, w.z, w.w, wh, wl);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          v4h bv;
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[e] = vvx[(16 * s + 4 * q4 + e) * kVStride + 16 * n + l16];
          O[n] = mfma16(wh, bv, O[n]);
          O[n] = mfma16(wl, bv, O[n]);
        }
      }
    }
  }

  // ---- combine the 4 waves: common max, rescale, fixed-order sum
  if (q4 == 0) {
    wstat[wave * 16 + l16] = m_run;
    wstat[kWaves * 16 + wave * 16 + l16] = l_run;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wstat[w * 16 + l16]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = wstat[w * 16 + l16];
    L += (mw == -INFINITY) ? 0.f : wstat[kWaves * 16 + w * 16 + l16] * __expf(mw - M);
  }
  {
    const float beta = (m_run == -INFINITY) ? 0.f : __expf(m_run - M);
    float be[4];
    rows_of(beta, q4, be);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) O[n][e] *= be[e];
    }
  }
  __syncthreads();  // wave regions become the reduction buffer
  float* red = reinterpret_cast<float*>(wreg);  // [2][16][128]
  if (wave >= 2) {
    float* dst = red + (wave - 2) * 16 * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(4 * q4 + e) * kD + 16 * n + l16] = O[n][e];
    }
  }
  __syncthreads();
  if (wave < 2) {
    const float* src = red + wave * 16 * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) O[n][e] += src[(4 * q4 + e) * kD + 16 * n + l16];
    }
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(4 * q4 + e) * kD + 16 * n + l16] = O[n][e];
    }
  }
  __syncthreads();
  if (wave == 0) {
    float Le[4];
    rows_of(L, q4, Le);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int g = 4 * q4 + e;
      if (g < G) {
        float* dst = A.part_o + ((int64_t)(row0 + g) * A.n_parts + part) * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const float v = O[n][e] + red[g * kD + 16 * n + l16];
          dst[16 * n + l16] = (Le[e] > 0.f) ? v / Le[e] : 0.f;
        }
      }
    }
    if (q4 == 0 && l16 < G)
      A.part_lse[(int64_t)(row0 + l16) * A.n_parts + part] = (L > 0.f) ? M + __logf(L) : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine: one wave per query row
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_merge(const float* part_o, const float* part_lse,
                                                   int n_parts, int n_rows, f16* out, float* out_lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const float* L = part_lse + (int64_t)row * n_parts;
  float M = -INFINITY;
  for (int p = lane; p < n_parts; p += 64) M = fmaxf(M, L[p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float ax = 0.f, ay = 0.f, S = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p < n_parts; ++p) {
      const float lp = L[p];
      const float w = (lp == -INFINITY) ? 0.f : __expf(lp - M);
      const float2 o = *reinterpret_cast<const float2*>(part_o + ((int64_t)row * n_parts + p) * kD + 2 * lane);
      S += w;
      ax += w * o.x;
      ay += w * o.y;
    }
  }
  const bool any = S > 0.f;
  f16* dst = out + (int64_t)row * kD + 2 * lane;
  dst[0] = (f16)(any ? ax / S : 0.f);
  dst[1] = (f16)(any ? ay / S : 0.f);
  if (lane == 0) out_lse[row] = any ? M + __logf(S) : -INFINITY;
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

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

dkv_status launch_route(const dkv_pool* P, const dkv_batch* B, int top_k, int32_t* idx, float* scores,
                        hipStream_t st) {
  const int units = B->batch * P->n_kv_heads;
  if (units == 0) return DKV_OK;
  const size_t shm = (size_t)(B->max_blocks > 0 ? B->max_blocks : 1) * sizeof(uint32_t);
  static bool attr_set = false;
  if (shm > 48 * 1024 && !attr_set) {
    hipFuncSetAttribute((const void*)k_route_topk, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL(k_route_topk, dim3(units), dim3(kThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), top_k, idx, scores);
  return launched("k_route_topk");
}

dkv_status launch_attend(const dkv_pool* P, const dkv_batch* B, const int32_t* idx, int top_k,
                         int n_block_parts, int block_mode, int n_win_parts, int win_chunk, float scale,
                         float* part_o, float* part_lse, int n_parts, int part_offset, hipStream_t st) {
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
  const size_t shm = (size_t)attend_lds_bytes(a.rq);
  hipLaunchKernelGGL(k_attend, dim3((unsigned)items), dim3(kThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), a);
  return launched("k_attend");
}

dkv_status launch_merge(const float* part_o, const float* part_lse, int n_parts, int n_rows, void* out,
                        float* out_lse, hipStream_t st) {
  if (n_rows == 0) return DKV_OK;
  const unsigned blocks = (unsigned)((n_rows + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(k_merge, dim3(blocks), dim3(kThreads), 0, st, part_o, part_lse, n_parts, n_rows,
                     (f16*)out, out_lse);
  return launched("k_merge");
}

int win_parts_of(int window) { return (window + kWinChunk - 1) / kWinChunk; }

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
  return launch_route(pool, batch, top_k, idx, scores, (hipStream_t)stream);
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
  return launch_attend(pool, batch, idx, top_k, top_k, 1, 0, kWinChunk, scale, part_o, part_lse, n_parts,
                       part_offset, (hipStream_t)stream);
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
  return launch_attend(pool, batch, idx, top_k, top_k, 2, window_splits, chunk > 0 ? chunk : 1, scale, part_o,
                       part_lse, n_parts, part_offset, (hipStream_t)stream);
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
  const size_t B = (size_t)batch->batch;
  const size_t n_parts = (size_t)top_k + (size_t)win_parts_of(batch->window);
  const size_t rows = B * (size_t)batch->n_q_heads;
  return align256(B * pool->n_kv_heads * (size_t)top_k * sizeof(int32_t)) +
         align256(rows * n_parts * sizeof(float)) + align256(rows * n_parts * kD * sizeof(float));
}

dkv_status dkv_decode(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale, void* workspace,
                      size_t workspace_bytes, void* out, float* out_lse, int32_t* out_idx, void* stream) {
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
  const int n_win = win_parts_of(batch->window);
  const int n_parts = top_k + n_win;
  const size_t B = (size_t)batch->batch;
  const size_t rows = B * (size_t)batch->n_q_heads;
  unsigned char* ws = (unsigned char*)workspace;
  int32_t* idx = (int32_t*)ws;
  float* part_lse = (float*)(ws + align256(B * pool->n_kv_heads * (size_t)top_k * sizeof(int32_t)));
  float* part_o = (float*)((unsigned char*)part_lse + align256(rows * n_parts * sizeof(float)));
  if (out_idx) idx = out_idx;

  if (top_k > 0) {
    if ((s = launch_route(pool, batch, top_k, idx, nullptr, st))) return s;
  }
  if (n_parts > 0) {
    if ((s = launch_attend(pool, batch, idx, top_k, top_k, 3, n_win, kWinChunk, scale, part_o, part_lse, n_parts,
                           0, st)))
      return s;
  }
  return launch_merge(part_o, part_lse, n_parts, (int)rows, out, out_lse, st);
}

}  // extern "C"
