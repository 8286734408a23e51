// dkv_common.h -- device-side pieces shared by the decode translation units of
// libdkv_attn (gfx950): argument structs, MFMA / LDS / coherent-memory helpers,
// wave reductions, top-K routing of one unit, the in-launch log-sum-exp merges
// and the work-queue layout of the fused decode launches.  Everything sits in an
// anonymous namespace: each translation unit holds its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include "dkv_attn.h"

#include <type_traits>

typedef _Float16 f16;
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

namespace {

constexpr int kD = 128;            // head dim
constexpr int kLowRankRows = 255;  // tokens 1..255 of a block
constexpr int kVStride = 132;      // LDS row stride (halves) of 128-wide tiles: conflict-free column reads
constexpr int kWinChunk = 512;     // window rows per window part (when the window has parts of its own)

// ---- codes of the 8- / 4-bit residual formats ------------------------------

// two bytes (low halves of each 16-bit half of w) -> two exact fp16 integers
__device__ __forceinline__ uint32_t bytes2_to_h2(uint32_t w) {
  // 0x6400 | b is the fp16 1024 + b; subtracting 1024 is exact
  const uint32_t m = (w & 0x00FF00FFu) | 0x64006400u;
  const v2h x = __builtin_bit_cast(v2h, m) - (v2h){(f16)1024.0f, (f16)1024.0f};
  return __builtin_bit_cast(uint32_t, x);
}

// 8 codes of a lane -> v8h of exact fp16 integers (dimension order)
template <int BITS>
__device__ __forceinline__ v8h codes_to_h8(typename std::conditional<BITS == 8, uint2, uint32_t>::type c) {
  uint32_t w[4];
  if constexpr (BITS == 8) {
    // bytes b0..b3 of c.x: pairs (b0, b1) and (b2, b3)
    w[0] = bytes2_to_h2(__builtin_amdgcn_perm(0u, c.x, 0x0c010c00u));
    w[1] = bytes2_to_h2(__builtin_amdgcn_perm(0u, c.x, 0x0c030c02u));
    w[2] = bytes2_to_h2(__builtin_amdgcn_perm(0u, c.y, 0x0c010c00u));
    w[3] = bytes2_to_h2(__builtin_amdgcn_perm(0u, c.y, 0x0c030c02u));
  } else {
    // nibbles: dimension 2j = low nibble of byte j, 2j + 1 = high nibble
    const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
    // lo byte j -> low half, hi byte j -> high half
    w[0] = bytes2_to_h2(__builtin_amdgcn_perm(hi, lo, 0x0c040c00u));
    w[1] = bytes2_to_h2(__builtin_amdgcn_perm(hi, lo, 0x0c050c01u));
    w[2] = bytes2_to_h2(__builtin_amdgcn_perm(hi, lo, 0x0c060c02u));
    w[3] = bytes2_to_h2(__builtin_amdgcn_perm(hi, lo, 0x0c070c03u));
  }
  return __builtin_bit_cast(v8h, w);
}

__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(v2h, w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(v2h, w)[1]; }

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
  int rfmt;                                   // residual rows: 0 fp16 (rk, rv), 1 / 2 8- / 4-bit codes
  const uint8_t* rkq; int64_t rkq_s, rkq_h;   // codes [R][128] or [R][64] (bytes)
  const uint8_t* rvq; int64_t rvq_s, rvq_h;
  const f16* rks; int64_t rks_s, rks_h;       // (scale, bias) per 64-dimension group [R][2][2]
  const f16* rvs; int64_t rvs_s, rvs_h;
  // un-rotated pools: theta_j / (2 pi) as hi[64] then lo[64], and each slot's
  // absolute position; rope == nullptr for pools of rotated keys
  const float* rope;
  const int32_t* spos;
  // shared basis (un-rotated pools only): the vk / vv entry of each slot, or nullptr
  const int32_t* basis;
  int n_basis;
};

struct BatchArgs {
  int B, Hq, Hkv, G, W, mb;
  const int32_t* table;
  const int32_t* nblk;
  const int32_t* wlen;
  const f16* q;
  const f16* wk;
  const f16* wv;
  const float* rkeys;  // [B][Hkv][mb][kD] per-sequence routing keys, or NULL
};

struct AttnArgs {
  const int32_t* idx;
  int top_k;           // row stride of idx
  int n_block_parts;   // parts per unit that are routed blocks (top_k or 0)
  int block_mode;      // bit 0: low-rank rows of a block, bit 1: its residual rows
  int n_win_parts;
  int win_chunk;
  int win_tile_stride; // > 0: block part p also attends window tiles p, p + stride, ... (16 rows each)
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

// Four softmax weights in [0, 1] as an fp16 MFMA operand (round to nearest
// even: relative error at most 2^-11 per weight; the row sums stay fp32)
__device__ __forceinline__ v4h to_h4(const float (&x)[4]) {
  v4h h;
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = (f16)x[e];
  return h;
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

// Workgroup barrier for LDS hand-offs: each wave waits for its own LDS (and
// scalar) operations, then all waves meet.  Unlike __syncthreads() it does not
// drain the waves' outstanding global loads, so data requested before it keeps
// streaming in while the workgroup moves on.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt = 0 only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's stores have completed
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }

// Buffer loads at device scope (cache policy sc1): they read the device-coherent
// copy, so they observe data that other workgroups of the same launch wrote with
// device-scope stores and then published through a counter, without an
// invalidation of the whole cache.  Reads outside [base, base + bytes) return 0.
constexpr int kLoadDeviceScope = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float4 ld_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kLoadDeviceScope);  // 4 x 32 raw bits
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}
__device__ __forceinline__ void st_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float4 v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u bits = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(bits, r, (int)byte_off, 0, kLoadDeviceScope);
}
__device__ __forceinline__ float ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kLoadDeviceScope));
}


__device__ __forceinline__ v4h lo4(v8h x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ v4h hi4(v8h x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

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
  lds_barrier();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = (int)wsum[i];
    off += (i < w) ? c : 0;
    tot += c;
  }
  lds_barrier();
  excl = off + in_wave;
  total = tot;
}

// ----------------------------------------------------------------------------
// Wave-wide reductions and scans with DPP lane moves (no LDS round trips)
// ----------------------------------------------------------------------------

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, true);
}

// max (MAX = true) or min over the 64 lanes, returned to every lane
template <bool MAX>
__device__ __forceinline__ float wave_minmax(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  uint32_t u = __float_as_uint(v);
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0xB1>(u, u))));   // quad_perm 1,0,3,2
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0x4E>(u, u))));   // quad_perm 2,3,0,1
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0x141>(u, u))));  // row_half_mirror
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0x140>(u, u))));  // row_mirror
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0x142, 0xa>(u, u))));  // row_bcast:15
  u = __float_as_uint(op(__uint_as_float(u), __uint_as_float(dpp_u32<0x143, 0xc>(u, u))));  // row_bcast:31
  return __uint_as_float(__builtin_amdgcn_readlane(u, 63));
}

// inclusive prefix sum over the 64 lanes in lane order
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  uint32_t s = v + dpp_u32<0x111>(0u, v);  // row_shr:1
  s += dpp_u32<0x112>(0u, v);              // row_shr:2
  s += dpp_u32<0x113>(0u, v);              // row_shr:3
  s += dpp_u32<0x114, 0xf, 0xe>(0u, s);    // row_shr:4 into lanes 4..15 of each row
  s += dpp_u32<0x118, 0xf, 0xc>(0u, s);    // row_shr:8 into lanes 8..15
  s += dpp_u32<0x142, 0xa>(0u, s);         // row_bcast:15 into rows 1 and 3
  s += dpp_u32<0x143, 0xc>(0u, s);         // row_bcast:31 into rows 2 and 3
  return s;
}

// ----------------------------------------------------------------------------
// Top-K routing: one workgroup of 4 waves per (sequence, KV head)
// ----------------------------------------------------------------------------

constexpr int kRouteThreads = 256;
constexpr int kRedRow = 36;          // floats per row of the per-wave transpose area (conflict-free float4 reads)

template <int NW>
struct RouteShared {
  uint32_t hist[256];
  uint32_t wsum[NW];
  float wlo[NW], whi[NW];
  uint32_t digit, above;
  uint32_t ready[2][NW];     // a split routing's block part: per-wave "all words present", by poll parity
  int32_t pick_j, pick_slot; // ... and the routed block it takes, with its pool slot
};

// LDS words route_unit needs for max_blocks blocks and NW waves.
__host__ __device__ constexpr size_t route_lds_words(int max_blocks, int nw) {
  return (size_t)2 * (size_t)(((max_blocks > 0 ? max_blocks : 1) + 3) & ~3) + (size_t)nw * 64 * kRedRow;
}

// The layer-batched streams' schedule (written on the host, read by the
// streams): work items of four words each,
//   w0: layer | kind << 16 | flags << 24 (flag 1: the item opens a run, 2: it
//       closes one; a run is a wave's consecutive items of one unit)
//   w1: window items: the first window row; block items: the routed rank
//       | the first residual row << 16 (residual items)
//   w2: batch row | kv head << 16
//   w3: the run's partial index | rows << 16 (window and residual items)
enum { kItemWin = 0, kItemLowRank = 1, kItemResid = 2 };

// Routed-slot words of the fused kernels hold the launch's tag in the top byte
// and pool slot + kSlotCode in the low 24 bits (1: no block), so that a word
// whose low bits are 0 (zero-filled memory) or whose tag is another launch's
// means "not routed yet in this launch".  The tag is the low byte of the
// workspace's launch counter (control word 3), which the last merge of each
// launch advances: a routing word that arrives after its launch ended can
// never be taken for the next launch's.
constexpr int32_t kSlotPending = 0;
constexpr int32_t kSlotCode = 2;
__device__ __forceinline__ uint32_t slot_tag(uint32_t epoch) { return (epoch & 0xFFu) << 24; }
__device__ __forceinline__ bool slot_ready(int32_t w, uint32_t tag) {
  return ((uint32_t)w & 0xFF000000u) == tag && ((uint32_t)w & 0x00FFFFFFu) != 0u;
}
__device__ __forceinline__ int32_t slot_value(int32_t w) { return (int32_t)((uint32_t)w & 0x00FFFFFFu) - kSlotCode; }

// The GQA-mean query of unit (b, h), columns 4 c4 .. 4 c4 + 3: the group's
// query rows summed in order, then scaled by 1 / G.
__device__ __forceinline__ float4 route_query(const BatchArgs& Bt, int b, int h, int c4) {
  float4 qb = make_float4(0.f, 0.f, 0.f, 0.f);
  const f16* q0 = Bt.q + ((int64_t)b * Bt.Hq + h * Bt.G) * kD + 4 * c4;
  v4h qh[DKV_MAX_GROUP];
#pragma unroll
  for (int g = 0; g < DKV_MAX_GROUP; ++g) qh[g] = *reinterpret_cast<const v4h*>(q0 + (g < Bt.G ? g : Bt.G - 1) * kD);
#pragma unroll
  for (int g = 0; g < DKV_MAX_GROUP; ++g) {
    if (g < Bt.G) {
      qb.x += (float)qh[g][0];
      qb.y += (float)qh[g][1];
      qb.z += (float)qh[g][2];
      qb.w += (float)qh[g][3];
    }
  }
  const float inv = 1.f / (float)Bt.G;
  qb.x *= inv;
  qb.y *= inv;
  qb.z *= inv;
  qb.w *= inv;
  return qb;
}

// A routing score is computed in two steps, the same everywhere a score is
// computed (so every routing path ranks blocks on identical values): each of
// 32 lanes takes the dot product of 4 of the 128 columns (score_share, with
// the multiply-adds written out), then the 32 shares, laid out in one LDS
// row, are added in column order (score_sum).
__device__ __forceinline__ float score_share(const float4& k, const float4& q) {
  return __builtin_fmaf(k.x, q.x, k.y * q.y) + __builtin_fmaf(k.z, q.z, k.w * q.w);
}
__device__ __forceinline__ float score_sum(const float* row) {
  const float4* rr = reinterpret_cast<const float4*>(row);
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float4 v = rr[m];
    acc += (v.x + v.y) + (v.z + v.w);
  }
  return acc;
}

// Blocks one score item covers (a split routing: see score_slice).
constexpr int kScoreChunk = 64;

// Scores of blocks [j0, j1) of unit u, j1 - j0 <= 16 NT / 64 (clipped to the
// unit's block count), each written to words[j] with one device-scope 8-byte
// store: the high word is pool slot + kSlotCode (slot -1 for an invalid
// block-table entry, whose score is -inf), never 0; the low word is the
// ordered score.  Wave w takes blocks j0 + 16 w .. + 15; lanes 0-31 read the even and
// lanes 32-63 the odd ones of each pair, 16 bytes each, and a block's 32
// shares meet in a 16 x kRedRow float area per wave (red).  No workgroup
// barrier: waves without blocks return at once.
template <int NT>
__device__ __forceinline__ void score_slice(const PoolArgs& P, const BatchArgs& Bt, int u, int j0, int j1,
                                            uint64_t* words, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  int N = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  N = N < 0 ? 0 : (N > Bt.mb ? Bt.mb : N);
  const int last = (j1 < N ? j1 : N) - 1;
  const int w0 = j0 + 16 * wave;
  if (w0 > last) return;
  const int c4 = lane & 31, half = lane >> 5;
  // lanes 0..15 look up the slots of blocks w0 .. w0 + 15 (past the end: the last block)
  const int jt = w0 + (lane & 15) <= last ? w0 + (lane & 15) : last;
  const float* seq_keys = Bt.rkeys ? Bt.rkeys + ((int64_t)b * Bt.Hkv + h) * Bt.mb * kD + 4 * c4 : nullptr;
  float4 kv[8];
  if (seq_keys) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = w0 + 2 * i + half <= last ? w0 + 2 * i + half : last;
      kv[i] = *reinterpret_cast<const float4*>(seq_keys + (int64_t)r * kD);
    }
  }
  const int tab = Bt.table[(int64_t)b * Bt.mb + jt];
  const int sl = (tab >= 0 && tab < P.n_slots) ? tab : -1;
  if (!seq_keys) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = __shfl(sl, 2 * i + half);  // the slot of block w0 + 2 i + half (clipped alike)
      kv[i] = *reinterpret_cast<const float4*>(P.key + (int64_t)(s >= 0 ? s : 0) * P.key_s + h * P.key_h + 4 * c4);
    }
  }
  const float4 qb = route_query(Bt, b, h, c4);
  float* rw = red + wave * 16 * kRedRow;
#pragma unroll
  for (int i = 0; i < 8; ++i) rw[(2 * i + half) * kRedRow + c4] = score_share(kv[i], qb);
  wave_sync_lds();
  if (lane < 16 && w0 + lane <= last) {
    const float acc = score_sum(rw + lane * kRedRow);
    const uint32_t key = ordered_key(sl >= 0 ? acc : -INFINITY);
    st_dev(&words[w0 + lane], ((uint64_t)(uint32_t)(sl + kSlotCode) << 32) | (uint64_t)key);
  }
}

// The top keff of N blocks by ordered score key (keys[], in LDS; the
// lowest index first among equal keys), found by the whole workgroup of NT
// threads: emit(pos, j, key) is called once for each routed block j, pos =
// its rank in ascending block order.  lds: route_lds_words(mb, NT / 64) words
// whose first 2 mbp hold keys (and the caller's slots); the rest is scratch.
//
// Finite scores are binned linearly between their minimum and maximum into
// bins 1..255 (-inf and below into bin 0); the bin map is monotone, so every
// block in a bin above the boundary bin b* is routed and none below it.
// Inside b* the blocks are ranked exactly by (score, lower index first)
// against the other members of b*.
template <int NT, class Emit>
__device__ __forceinline__ void route_select(const uint32_t* keys, int N, int keff, uint32_t* lds, int mbp,
                                             RouteShared<NT / 64>& sh, Emit&& emit) {
  constexpr int NW = NT / 64;
  constexpr int kBinWaves = 256 / 64;
  uint32_t* wsum = sh.wsum;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (keff > 0) {
    uint32_t* hist = sh.hist;
    constexpr uint32_t kNegInfKey = 0x007FFFFFu;  // ordered key of -inf
    float lo = INFINITY, hi = -INFINITY;
    for (int jj = tid; jj < N; jj += NT) {
      const float sc = from_ordered(keys[jj]);
      if (isfinite(sc)) {
        lo = fminf(lo, sc);
        hi = fmaxf(hi, sc);
      }
    }
    if (tid < 256) hist[tid] = 0u;
    lo = wave_minmax<false>(lo);
    hi = wave_minmax<true>(hi);
    if (lane == 0) {
      sh.wlo[wave] = lo;
      sh.whi[wave] = hi;
    }
    lds_barrier();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = fminf(lo, sh.wlo[w]);
      hi = fmaxf(hi, sh.whi[w]);
    }
    const float inv = (hi > lo) ? 254.99f / (hi - lo) : 0.f;
    auto bin_of = [&](uint32_t k) -> uint32_t {
      if (k <= kNegInfKey) return 0u;
      const float sc = from_ordered(k);
      if (!(sc <= INFINITY)) return 255u;  // +NaN keys order above +inf
      const float t = (sc - lo) * inv;
      return 1u + (uint32_t)fminf(fmaxf(t, 0.f), 254.f);
    };
    if (tid == 0) {
      sh.digit = 0u;
      sh.above = 0u;
    }
    for (int jj = tid; jj < N; jj += NT) atomicAdd(&hist[bin_of(keys[jj])], 1u);
    lds_barrier();
    // counts of bins >= 255 - tid (a scan of the bins in descending order)
    const uint32_t hb = tid < 256 ? hist[255 - tid] : 0u;
    uint32_t incl = wave_incl_scan(hb);
    if (lane == 63 && wave < kBinWaves) wsum[wave] = incl;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kBinWaves; ++w) incl += (w < wave) ? wsum[w] : 0u;
    const uint32_t excl = incl - hb;
    if (tid < 256 && excl < (uint32_t)keff && incl >= (uint32_t)keff) {
      sh.digit = 255u - (uint32_t)tid;
      sh.above = excl;
    }
    lds_barrier();
    const uint32_t bstar = sh.digit & 255u, need = (uint32_t)keff - sh.above, m = hist[bstar];
    // members of b* that are routed: all of them, or the `need` best by rank
    uint64_t* cand = reinterpret_cast<uint64_t*>(lds + 2 * mbp);  // the score transpose area, now free
    const uint32_t cap = (uint32_t)(NW * 64 * kRedRow / 2 - 2);
    uint32_t* n_cand = reinterpret_cast<uint32_t*>(cand + cap);
    const bool rank_members = m > need;
    const bool listed = m <= cap;
    if (rank_members && listed) {
      if (tid == 0) *n_cand = 0u;
      lds_barrier();
      for (int jj = tid; jj < N; jj += NT) {
        const uint32_t k = keys[jj];
        if (bin_of(k) == bstar) cand[atomicAdd(n_cand, 1u)] = ((uint64_t)k << 32) | (uint64_t)(~(uint32_t)jj);
      }
      lds_barrier();
    }
    int sel_base = 0;
    for (int b0 = 0; b0 < N; b0 += NT) {
      const int jj = b0 + tid;
      bool sel = false;
      uint32_t kj = 0u;
      if (jj < N) {
        kj = keys[jj];
        const uint32_t bj = bin_of(kj);
        sel = bj > bstar;
        if (bj == bstar) {
          if (!rank_members) {
            sel = true;
          } else {
            const uint64_t cj = ((uint64_t)kj << 32) | (uint64_t)(~(uint32_t)jj);
            uint32_t beat = 0u;
            if (listed) {
              for (uint32_t t2 = 0; t2 < m; ++t2) beat += (uint32_t)(cand[t2] > cj);
            } else {
              for (int t2 = 0; t2 < N; ++t2) {
                const uint32_t k2 = keys[t2];
                beat += (uint32_t)(bin_of(k2) == bstar && (((uint64_t)k2 << 32) | (uint64_t)(~(uint32_t)t2)) > cj);
              }
            }
            sel = beat < need;
          }
        }
      }
      int sel_rank, sel_tot;
      block_count<NW>(sel, sel_rank, sel_tot, wsum);
      if (sel) emit(sel_base + sel_rank, jj, kj);
      sel_base += sel_tot;
    }
  }
}

// Route one (sequence, KV head) unit u with a workgroup of NT threads.
// lds: route_lds_words(max_blocks, NT / 64) words: ordered score keys [mb],
// pool slots [mb] (both rounded up to 4), then a 64 x kRedRow float area per wave.
//
// Scores: lane l of a wave holds columns 4 (l % 32) .. +3 of the GQA-mean query;
// a 512-byte routing key is read by 32 lanes, 16 bytes each, two keys per load
// instruction (fully coalesced), and the 32 lane partials of a key are summed
// through LDS.  Selection: block j is routed iff fewer than K blocks beat it
// (a larger score, or an equal score at a smaller index: the lowest-index-first
// tie rule), found with a 256-bin histogram of the scores and an exact ranking
// inside the boundary bin only.  Routed blocks are emitted in ascending block
// order.
template <int NT>
__device__ __forceinline__ void route_unit(const PoolArgs& P, const BatchArgs& Bt, int u, int top_k, int32_t* idx,
                                           float* scores, int32_t* slots_out, uint32_t* lds,
                                           RouteShared<NT / 64>& sh, uint32_t tag = 0u) {
  static_assert(NT == 256 || NT == 512, "route_unit: 256 histogram bins over the first 4 waves");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  int N = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  N = N < 0 ? 0 : (N > Bt.mb ? Bt.mb : N);
  const int keff = top_k < N ? top_k : N;
  const int mbp = ((Bt.mb > 0 ? Bt.mb : 1) + 3) & ~3;
  uint32_t* keys = lds;
  int32_t* slot_of = reinterpret_cast<int32_t*>(lds + mbp);
  float* red = reinterpret_cast<float*>(lds + 2 * mbp) + wave * 64 * kRedRow;

  const int c4 = lane & 31, half = lane >> 5;

  // ---- routing-key rows of a 64-block group: lanes 0-31 read block g0 + 2 i,
  //      lanes 32-63 block g0 + 2 i + 1, 16 bytes each (two whole keys per load)
  const float* seq_keys = Bt.rkeys ? Bt.rkeys + ((int64_t)b * Bt.Hkv + h) * Bt.mb * kD + 4 * c4 : nullptr;
  float4 kv[32];
  auto load_group = [&](int g0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      int r = g0 + 2 * i + half;
      r = r < N ? r : N - 1;
      const float* src;
      if (seq_keys) {
        src = seq_keys + (int64_t)r * kD;
      } else {
        const int sr = slot_of[r];
        src = P.key + (int64_t)(sr >= 0 ? sr : 0) * P.key_s + h * P.key_h + 4 * c4;
      }
      kv[i] = *reinterpret_cast<const float4*>(src);
    }
  };
  // with per-sequence keys the first group does not wait for the block table
  // (nor for the query); the keys, this thread's block-table entry and the
  // query rows are all requested before any of them is used
  if (seq_keys && wave * 64 < N) load_group(wave * 64);
  const int tab0 = tid < N ? Bt.table[(int64_t)b * Bt.mb + tid] : -1;
  // ---- this lane's 4 columns of the GQA-mean query (no barrier needed)
  const float4 qb = route_query(Bt, b, h, c4);

  // ---- pool slots of the unit's blocks (coalesced block-table reads)
  for (int j = tid; j < N; j += NT) {
    const int sr = j == tid ? tab0 : Bt.table[(int64_t)b * Bt.mb + j];
    slot_of[j] = (sr >= 0 && sr < P.n_slots) ? sr : -1;
  }
  lds_barrier();

  // ---- scores of 64-block groups, one group per wave at a time
  for (int g0 = wave * 64; g0 < N; g0 += NT) {
    if (!seq_keys || g0 != wave * 64) load_group(g0);
#pragma unroll
    for (int i = 0; i < 32; ++i) red[(2 * i + half) * kRedRow + c4] = score_share(kv[i], qb);
    wave_sync_lds();
    const float acc = score_sum(red + lane * kRedRow);
    const int j = g0 + lane;
    if (j < N) keys[j] = ordered_key(slot_of[j] >= 0 ? acc : -INFINITY);
    wave_sync_lds();  // the next group reuses the transpose area
  }
  lds_barrier();

  auto emit = [&](int pos, int j, uint32_t k) {
    st_dev(&idx[(int64_t)u * top_k + pos], j);
    if (scores) st_dev(&scores[(int64_t)u * top_k + pos], from_ordered(k));
    if (slots_out) st_dev(&slots_out[(int64_t)u * top_k + pos], (int32_t)(tag | (uint32_t)(slot_of[j] + kSlotCode)));
  };

  route_select<NT>(keys, N, keff, lds, mbp, sh, emit);
  for (int pos = keff + tid; pos < top_k; pos += NT) {
    st_dev(&idx[(int64_t)u * top_k + pos], -1);
    if (scores) st_dev(&scores[(int64_t)u * top_k + pos], -INFINITY);
    if (slots_out) st_dev(&slots_out[(int64_t)u * top_k + pos], (int32_t)(tag | (uint32_t)(-1 + kSlotCode)));
  }
}

__host__ __device__ inline int round16(int x) { return (x + 15) & ~15; }

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;


// ----------------------------------------------------------------------------
// Log-sum-exp merge of the partials of one decode step, inside the launch
// ----------------------------------------------------------------------------


// Log-sum-exp combine of one query row's n_parts partials by one workgroup:
// kMergeSlots slots of 32 lanes (4 columns per lane), slot s taking parts s,
// s + kMergeSlots, ..., every load of a round issued at once; the row maximum
// comes first so the slots' weighted sums add without rescaling, in a fixed
// order.  lds: kMergeSlots * (kD + 1) + kAttWaves floats.
constexpr int kMergeSlots = kAttThreads / 32;
constexpr int kMergeRowChunk = 8;  // parts per slot per round
__device__ __forceinline__ void merge_row(const float* part_o, const float* part_lse, int n_parts, int row,
                                          f16* out, float* out_lse, float* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c4 = tid & 31, sl = tid >> 5;
  float* red = lds;                           // [kMergeSlots][kD]
  float* redS = lds + kMergeSlots * kD;       // [kMergeSlots]
  float* redM = redS + kMergeSlots;           // [kAttWaves]
  const int np = n_parts > 0 ? n_parts : 1;
  const __amdgpu_buffer_rsrc_t Ob = coherent_rsrc(part_o + (int64_t)row * n_parts * kD, (uint32_t)n_parts * kD * 4);
  const __amdgpu_buffer_rsrc_t Lb = coherent_rsrc(part_lse + (int64_t)row * n_parts, (uint32_t)n_parts * 4);
  // first round's partials, then the row maximum over every part
  float4 o[kMergeRowChunk];
  float l[kMergeRowChunk];
#pragma unroll
  for (int k = 0; k < kMergeRowChunk; ++k) {
    const int pp = sl + kMergeSlots * k;
    const int pc = pp < np ? pp : np - 1;
    o[k] = ld_coherent4(Ob, (uint32_t)(pc * kD + 4 * c4) * 4u);
    l[k] = ld_coherent(Lb, (uint32_t)pc * 4u);
  }
  float m = -INFINITY;
  for (int pp = tid; pp < n_parts; pp += kAttThreads) m = fmaxf(m, ld_coherent(Lb, (uint32_t)pp * 4u));
  m = wave_minmax<true>(m);
  if (lane == 0) redM[wave] = m;
  lds_barrier();
#pragma unroll
  for (int w = 0; w < kAttWaves; ++w) m = fmaxf(m, redM[w]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float S = 0.f;
  for (int p0 = 0; p0 < n_parts; p0 += kMergeSlots * kMergeRowChunk) {
    if (p0 > 0) {
#pragma unroll
      for (int k = 0; k < kMergeRowChunk; ++k) {
        const int pp = p0 + sl + kMergeSlots * k;
        const int pc = pp < np ? pp : np - 1;
        o[k] = ld_coherent4(Ob, (uint32_t)(pc * kD + 4 * c4) * 4u);
        l[k] = ld_coherent(Lb, (uint32_t)pc * 4u);
      }
    }
#pragma unroll
    for (int k = 0; k < kMergeRowChunk; ++k) {
      const int pp = p0 + sl + kMergeSlots * k;
      const float w = (pp < n_parts && l[k] != -INFINITY) ? __expf(l[k] - m) : 0.f;
      S += w;
      acc.x += w * o[k].x;
      acc.y += w * o[k].y;
      acc.z += w * o[k].z;
      acc.w += w * o[k].w;
    }
  }
  *reinterpret_cast<float4*>(red + sl * kD + 4 * c4) = acc;
  if (c4 == 0) redS[sl] = S;
  lds_barrier();
  if (tid < 32) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float St = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kMergeSlots; ++s2) {
      const float4 v = *reinterpret_cast<const float4*>(red + s2 * kD + 4 * c4);
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
      St += redS[s2];
    }
    const bool any = St > 0.f;
    v4h h4;
    h4[0] = (f16)(any ? t.x / St : 0.f);
    h4[1] = (f16)(any ? t.y / St : 0.f);
    h4[2] = (f16)(any ? t.z / St : 0.f);
    h4[3] = (f16)(any ? t.w / St : 0.f);
    *reinterpret_cast<v4h*>(out + (int64_t)row * kD + 4 * c4) = h4;
    if (tid == 0) out_lse[row] = any ? m + __logf(St) : -INFINITY;
  }
}

// Log-sum-exp combine of the partials of one unit's G query rows (rows row0 ..
// row0 + G - 1) by one workgroup: each 32-lane slot takes a row (slot s: rows
// s, s + 8, ...), with its lanes on 4 columns each.  The row maximum comes
// first, then the partials are combined in part order, so the result does not
// depend on timing.
__device__ __forceinline__ void merge_unit(const float* part_o, const float* part_lse, int n_parts, int row0, int G,
                                           f16* out, float* out_lse) {
  const int c4 = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int np = n_parts > 0 ? n_parts : 1;
  for (int g = sl; g < G; g += kMergeSlots) {
    const int row = row0 + g;
    const __amdgpu_buffer_rsrc_t Ob = coherent_rsrc(part_o + (int64_t)row * n_parts * kD, (uint32_t)n_parts * kD * 4);
    const __amdgpu_buffer_rsrc_t Lb = coherent_rsrc(part_lse + (int64_t)row * n_parts, (uint32_t)n_parts * 4);
    float m = -INFINITY;
    for (int p0 = 0; p0 < n_parts; p0 += kMergeRowChunk) {
      float l[kMergeRowChunk];
#pragma unroll
      for (int k = 0; k < kMergeRowChunk; ++k) l[k] = ld_coherent(Lb, (uint32_t)(p0 + k < np ? p0 + k : np - 1) * 4u);
#pragma unroll
      for (int k = 0; k < kMergeRowChunk; ++k) m = fmaxf(m, l[k]);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float S = 0.f;
    for (int p0 = 0; p0 < n_parts; p0 += kMergeRowChunk) {
      float4 o[kMergeRowChunk];
      float l[kMergeRowChunk];
#pragma unroll
      for (int k = 0; k < kMergeRowChunk; ++k) {
        const int pc = p0 + k < np ? p0 + k : np - 1;
        o[k] = ld_coherent4(Ob, (uint32_t)(pc * kD + 4 * c4) * 4u);
        l[k] = ld_coherent(Lb, (uint32_t)pc * 4u);
      }
#pragma unroll
      for (int k = 0; k < kMergeRowChunk; ++k) {
        const float w = (p0 + k < n_parts && l[k] != -INFINITY) ? __expf(l[k] - m) : 0.f;
        S += w;
        acc.x += w * o[k].x;
        acc.y += w * o[k].y;
        acc.z += w * o[k].z;
        acc.w += w * o[k].w;
      }
    }
    const bool any = S > 0.f;
    v4h h4;
    h4[0] = (f16)(any ? acc.x / S : 0.f);
    h4[1] = (f16)(any ? acc.y / S : 0.f);
    h4[2] = (f16)(any ? acc.z / S : 0.f);
    h4[3] = (f16)(any ? acc.w / S : 0.f);
    *reinterpret_cast<v4h*>(out + (int64_t)row * kD + 4 * c4) = h4;
    if (c4 == 0) out_lse[row] = any ? m + __logf(S) : -INFINITY;
  }
}


// ----------------------------------------------------------------------------
// One decode step of one layer in a single launch.
//
// Work items, handed out in ticket order (an atomic counter, so an item is
// only ever taken by a workgroup that is already running): first the routing
// of every (sequence, KV head) unit, then per unit its routed blocks and its
// window chunks, then one merge per unit.  A block item waits (bounded) until
// its routed slot is published, a merge until its unit's parts are counted;
// what they wait for precedes them in ticket order and is held by running
// workgroups, so every wait ends.  The last merge leaves the control words
// zeroed for the next launch.
// ----------------------------------------------------------------------------

struct DecodeArgs {
  AttnArgs att;
  int32_t* idx;          // [units][top_k] routed logical blocks
  int32_t* slots;        // [units][top_k] routed-slot words (launch tag | slot + kSlotCode)
  uint32_t* ctrl;        // [1] finished merges, [2] sticky wait-timeout flag, [3] launch counter,
                         // [4] finished score items (split routing), queue counters
  uint32_t* unit_done;   // parts finished: word 0 of each unit's own 256-byte line (u * kDoneStride)
  f16* out;
  float* out_lse;
  uint64_t* rwords;      // split routing: [units][mb] (slot, score) words, zero between launches; else NULL
  int n_units;
  int route_items;       // routing items per unit: 1 (route_unit), or the split routing's score items
  int n_route;           // routing items of this launch: n_units * route_items (0 when top_k == 0)
  int n_part_end;        // n_route + n_units * att.items_per_unit: first merge item
  int merges;            // merge items per unit: G (one per query row) or 1 (one per unit)
  int n_items;           // n_part_end + n_units * merges: the grid size
};

constexpr unsigned kRouteWaitLimit = 1u << 24;  // polls before giving up
constexpr int kCtrlScored = 4;                  // control word: score items finished (split routing)
// Words between per-unit part counters: each unit's counter has a 256-byte
// line of its own.  Counters of several units on one line made the parts'
// atomics and the merges' polls of different units contend for that line at
// the device's coherence point (one launch per layer of the 64k batch-4 stack:
// 27.3 us per layer with one shared line, 22.4 us with a line per unit).
constexpr int kDoneStride = 64;
constexpr int kQueues = 8;                      // one work queue per XCD
constexpr int kQueueStride = 64;                // words between queue counters (separate 256-byte lines)
constexpr int kCtrlQueue = 64;                  // first queue counter
constexpr int kCtrlHeaderBytes = 4096;          // control words: [0..63] misc, then the queue counters



// ----------------------------------------------------------------------------
// Layer-batched decode: the fused steps of several layers in one launch
// ----------------------------------------------------------------------------

struct LayerArgs {
  PoolArgs P;
  BatchArgs Bt;
  DecodeArgs D;  // the layer's workspace region; D.ctrl is the launch-wide control header
  int nrq;
};

struct LayersArgs {
  uint32_t* ctrl;  // [1] merges finished, [2] sticky wait-timeout flag, queue counters
  int n_layers;
  int n_units;     // units per layer (the same in every layer)
  int routes;       // routing items per unit (0 or 1)
  int block_parts;  // routed-block parts per unit
  int win_parts;    // window parts per unit
  int group;        // merges per unit (query heads per KV head)
};

// Position i of XCD queue x (which holds the nx units u = x + 8 j of every
// layer) -> (layer, item index within that layer's launch).  The queue holds
// the routings of every layer, then the window parts of every layer (they wait
// on nothing, and run while the routings finish), then the routed-block parts
// of layer 0, 1, ..., with the merges of layer l placed after the block parts
// of layer l + kMergeLag (as measured, no lag beats placing every merge after
// all block parts: the merges then never wait, and fill the launch's tail).
// Every wait is on an item earlier in the same queue.  Uniform (scalar)
// arithmetic.
constexpr int kMergeLag = 1 << 16;

__device__ __forceinline__ void layers_item(int i, int x, int nx, const LayersArgs& L, int& layer, int& item) {
  const int NL = L.n_layers, NP = L.block_parts, NW = L.win_parts, G = L.group;
  const int per_unit = NP + NW;
  const int n_route = L.routes * L.n_units;
  const int n_part_end = n_route + L.n_units * per_unit;
  const int nR = nx * L.routes, nW = nx * NW, nP = nx * NP, nM = nx * G;
  if (i < NL * nR) {
    layer = i / nR;
    item = x + kQueues * (i % nR);
    return;
  }
  i -= NL * nR;
  if (i < NL * nW) {
    layer = i / nW;
    const int r = i % nW;
    item = n_route + (x + kQueues * (r / NW)) * per_unit + NP + r % NW;
    return;
  }
  i -= NL * nW;
  const int a = NL < kMergeLag ? NL : kMergeLag;
  int kind = 0, r = 0;  // kind 0: block part of `layer`, 1: merge of `layer`
  if (i < a * nP) {
    layer = i / nP;
    r = i % nP;
  } else {
    i -= a * nP;
    const int pair = nP + nM;
    if (i < (NL - a) * pair) {
      const int c = i / pair;
      r = i % pair;
      if (r < nP) {
        layer = a + c;
      } else {
        layer = c;
        r -= nP;
        kind = 1;
      }
    } else {
      i -= (NL - a) * pair;
      layer = NL - a + i / nM;
      r = i % nM;
      kind = 1;
    }
  }
  item = kind == 0 ? n_route + (x + kQueues * (r / NP)) * per_unit + r % NP
                   : n_part_end + (x + kQueues * (r / G)) * G + r % G;
}

// Work items of every layer from the per-XCD queues (see layers_item).
// NMAX: the largest low-rank tile count of any layer (instances hold only the

}  // namespace
