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

#include "dkv_common.h"

#include <mutex>

// The layer-batched streaming step (dkv_stream.hip).
size_t dkv_stream_lds_bytes();
hipError_t dkv_stream_step(const void* table, uint32_t* ctrl, size_t route_lds, const int32_t* sched, int n_waves,
                           int n_sched_items, int top_k, int n_layers, int n_units, void* const* events,
                           hipStream_t st);
hipError_t dkv_stream_read_probe_launch(const void* src, size_t per, int n_waves, uint32_t* sink, hipStream_t st);

#include <algorithm>
#include <queue>
#include <vector>

namespace {

thread_local char g_err[512] = "";

dkv_status fail(dkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
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
  lds_barrier();
  const f16* VK = P.vk + slot * P.vk_s + h * P.vk_h;
  const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
  float c = 0.f;
  for (int j = 0; j < r; ++j) c += ubar[j] * (float)VK[j * kD + t];
  P.key[slot * P.key_s + h * P.key_h + t] = (float)AK[t] + c;
}

// cos and sin of the rotary angle pos * theta_j, with theta_j / (2 pi) given as
// the unevaluated sum fh + fl: the product pos * fh is split exactly into
// a + e (fma), its whole turns dropped from a, and the remaining fraction of a
// turn fed to the hardware sine and cosine, which take their argument in turns.
// pos < 2^24 is exact in fp32.
__device__ __forceinline__ void rope_cs(float pf, float fh, float fl, float& c, float& s) {
  const float a = pf * fh;
  const float e = __builtin_fmaf(pf, fh, -a);
  const float t = __builtin_amdgcn_fractf(a) + __builtin_fmaf(pf, fl, e);
  c = __builtin_amdgcn_cosf(t);
  s = __builtin_amdgcn_sinf(t);
}

// cos and sin of the rotary angle of a row at in-block offset `off` (0..255):
// t0 = the block's own angle in turns, reduced exactly once per block (fract of
// slot_pos * theta / 2 pi), plus off * theta / 2 pi, < 41 turns.  The rounding
// of that sum (< 4e-6 turns) is far below the fp16 rounding of the rotated key.
__device__ __forceinline__ void rope_cs_off(float off, float fh, float t0, float& c, float& s) {
  const float t = __builtin_fmaf(off, fh, t0);
  c = __builtin_amdgcn_cosf(t);
  s = __builtin_amdgcn_sinf(t);
}

// Routing keys of an un-rotated pool: the mean over positions i = 1..255 of
// the reconstructed key a_k + U_i V_K rotated to slot_pos + i.  One workgroup
// per (slot, KV head); thread t takes the dimension pair (j, j + 64) with
// j = t % 64 and the positions of one half of the block, in fp32.
__global__ __launch_bounds__(128) void k_route_keys_rot(PoolArgs P, const int32_t* slots) {
  const int item = blockIdx.x;
  const int si = item / P.n_kv, h = item % P.n_kv;
  const int slot = slots ? slots[si] : si;
  if (slot < 0 || slot >= P.n_slots) return;
  __shared__ float part[2][kD];
  __shared__ float vks[DKV_MAX_RANK * kD];
  const int r = P.rank;
  const int t = threadIdx.x, j = t & 63, half = t >> 6;
  int g = slot;  // the entry holding the block's V_K
  if (P.basis) {
    g = P.basis[slot];
    if (g < 0 || g >= P.n_basis) return;  // uniform over the workgroup
  }
  const f16* U = P.u + slot * P.u_s + h * P.u_h;
  const f16* VK = P.vk + g * P.vk_s + h * P.vk_h;
  const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
  for (int c = 0; c < r; ++c) vks[c * kD + t] = (float)VK[c * kD + t];
  lds_barrier();
  const float a0 = (float)AK[j], a1 = (float)AK[j + 64];
  const float fh = P.rope[j], fl = P.rope[64 + j];
  const int p0 = P.spos[slot];
  float s0 = 0.f, s1 = 0.f;
  const int i_lo = half == 0 ? 1 : 128, i_hi = half == 0 ? 128 : 256;
  for (int i = i_lo; i < i_hi; ++i) {
    const f16* Ui = U + (int64_t)(i - 1) * r;
    float x = a0, y = a1;
    for (int c = 0; c < r; ++c) {
      const float uc = (float)Ui[c];
      x = __builtin_fmaf(uc, vks[c * kD + j], x);
      y = __builtin_fmaf(uc, vks[c * kD + j + 64], y);
    }
    float cs, sn;
    rope_cs((float)(p0 + i), fh, fl, cs, sn);
    s0 += x * cs - y * sn;
    s1 += y * cs + x * sn;
  }
  part[half][j] = s0;
  part[half][j + 64] = s1;
  lds_barrier();
  P.key[slot * P.key_s + h * P.key_h + t] = (part[0][t] + part[1][t]) / (float)kLowRankRows;
}

// Per-sequence routing-key table: one thread per 16 bytes of out.
__global__ void k_gather_route_keys(PoolArgs P, BatchArgs Bt, float* out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)Bt.B * Bt.Hkv * Bt.mb * (kD / 4);
  if (t >= n) return;
  const int c4 = (int)(t % (kD / 4));
  const int64_t row = t / (kD / 4);  // (b, h, j)
  const int j = (int)(row % Bt.mb);
  const int h = (int)((row / Bt.mb) % Bt.Hkv);
  const int b = (int)(row / ((int64_t)Bt.mb * Bt.Hkv));
  int nb = Bt.nblk[b];
  nb = nb < 0 ? 0 : (nb > Bt.mb ? Bt.mb : nb);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j < nb) {
    const int sr = Bt.table[(int64_t)b * Bt.mb + j];
    if (sr >= 0 && sr < P.n_slots) v = *reinterpret_cast<const float4*>(P.key + sr * P.key_s + h * P.key_h + 4 * c4);
  }
  *reinterpret_cast<float4*>(out + row * kD + 4 * c4) = v;
}


__global__ __launch_bounds__(kRouteThreads) void k_route_topk(PoolArgs P, BatchArgs Bt, int top_k,
                                                              int32_t* idx, float* scores, int32_t* slots_out) {
  extern __shared__ __attribute__((aligned(16))) uint32_t route_lds[];  // route_lds_words(mb, 4)
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

constexpr int kLRTilesPerWave = 16 / kAttWaves;
constexpr int kRedStride = 132;  // floats per row of the reduction buffer (conflict-free C-layout access)



// Staged MFMA A operands are stored transposed, so that a lane's four
// elements (four consecutive rows of one column) are one 8-byte LDS read:
//   V^T of a 16-row exact tile: Vt[d][row], d-rows of kVTStride halves;
//   Ux^T of a wave's 64 low-rank positions: T[j][position], j-rows of kTTStride halves.
constexpr int kVTStride = 20;                       // 16 rows + pad (8-byte aligned rows)
constexpr int kTTStride = 4 * 16 + 4;               // 64 positions + pad

// per-wave scratch: the wave's transposed U tiles (low-rank phase) or two
// transposed V tiles (exact phase), then the 256-bit residual-position mask
__host__ __device__ inline int att_scratch_bytes(int rq) {
  const int a = rq * kTTStride * 2;
  const int b = 2 * kD * kVTStride * 2;
  return round16((a > b ? a : b) + 32);
}

// the per-wave scratch areas, later reused for the cross-wave sum of O^T
__host__ __device__ inline int att_region_bytes(int rq) {
  const int scratch = kAttWaves * att_scratch_bytes(rq);
  const int red = kAttWaves * 16 * kRedStride * 4;
  return scratch > red ? scratch : red;
}

__host__ __device__ inline int att_lds_bytes(int rq) {
  return 16 * rq * 4 + rq * kVStride * 2 + 2 * kAttWaves * 16 * 4 + att_region_bytes(rq);
}

// VKx^T of an un-rotated pool's block, staged [d][j] over the V_K q and VVx
// areas: row stride vkt_stride(RQ) halves and the 4-half chunks of a row
// permuted by chunk ^ vkt_swz(RQ, d), so that the 16 lanes of a row group,
// which read one chunk from 16 different rows, hit 32 different banks.  Sizes
// fit the areas (128 * stride * 2 <= 328 * RQ bytes).
__host__ __device__ constexpr int vkt_stride(int rq) { return rq == 64 ? 80 : rq; }
__device__ __forceinline__ constexpr int vkt_swz(int rq, int d) {
  return rq == 32 ? (((d >> 1) ^ (d >> 2)) & 7) : ((d >> 3) & 3);
}
__device__ __forceinline__ constexpr int vkt_at(int rq, int d, int j) {
  return d * vkt_stride(rq) + 4 * ((j >> 2) ^ vkt_swz(rq, d)) + (j & 3);
}
static_assert(128 * vkt_stride(16) * 2 <= 328 * 16 && 128 * vkt_stride(32) * 2 <= 328 * 32 &&
                  128 * vkt_stride(48) * 2 <= 328 * 48 && 128 * vkt_stride(64) * 2 <= 328 * 64 &&
                  128 * vkt_stride(80) * 2 <= 328 * 80,
              "VKx^T must fit the V_K q and VVx areas");


// Reductions over the four lanes l16, l16 + 16, l16 + 32, l16 + 48 (the four
// row groups of an MFMA accumulator), with gfx950 lane-swap moves; every lane
// gets the same bits.
__device__ __forceinline__ float q4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float q4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Attention state of one wave, transposed: head g = lane % 16 is the MFMA
// column, so every per-head factor is the lane's own value.
//   Ot[n]: O^T[d = 16 n + 4 (lane / 16) + e][g]   (sum over rows of p v, unnormalised)
//   m, l:  running maximum and sum of exp for head g
struct ExState {
  float m, l;
  v4f Ot[8];
};

// QK^T of one 16-row exact tile: S[row = 4 q4 + e][head l16]
__device__ __forceinline__ v4f exact_scores(const v8h (&kx)[4], const v4h (&qf)[4][2]) {
  v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    S = mfma16(lo4(kx[s]), qf[s][0], S);
    S = mfma16(hi4(kx[s]), qf[s][1], S);
  }
  return S;
}

// the A operand of O^T += V^T p for output tile n: V rows 4 q4 .. 4 q4 + 3 of
// column d = 16 n + l16, from the transposed staging
__device__ __forceinline__ v4h vt_operand(const f16* Vt, int n, int l16, int q4) {
  return *reinterpret_cast<const v4h*>(Vt + (16 * n + l16) * kVTStride + 4 * q4);
}

// O^T += V^T p for one 16-row tile staged transposed at Vt[d][row]
__device__ __forceinline__ void exact_pv(ExState& st, const f16* Vt, const float (&pe)[4], int l16, int q4) {
  const v4h ph = to_h4(pe);
#pragma unroll
  for (int n = 0; n < 8; ++n) st.Ot[n] = mfma16(vt_operand(Vt, n, l16, q4), ph, st.Ot[n]);
}

// lane (row l16, q4) holds V[l16][32 s + 8 q4 + j]: store it transposed
__device__ __forceinline__ void stage_v_tile(f16* Vt, const v8h (&vx)[4], int l16, int q4) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) Vt[(32 * s + 8 * q4 + j) * kVTStride + l16] = vx[s][j];
  }
}

// One softmax step over two 16-row exact tiles (b optional): scores, a common
// maximum, the rescale of the state and of the low-rank accumulator, and PV.
// rows_a / rows_b: valid rows of each tile (the rest are masked out).
struct NoNext {
  __device__ __forceinline__ void operator()() const {}
};

// scores of the tiles as stored (which: 0 for tile a, 1 for tile b)
struct PlainScore {
  const v4h (&qf)[4][2];
  __device__ __forceinline__ v4f operator()(const v8h (&kx)[4], int) const { return exact_scores(kx, qf); }
};

// next(): issued once the pair's K and V registers are consumed (V staged in
// LDS), to load the following pair into them while this one finishes.
// score(kx, which): the tile's scores, exact_scores of the rows as stored
// unless the rows are rotated first.
template <int NQ, class Next, class Score>
__device__ __forceinline__ void exact_pair_scored(ExState& st, v4f (&Wt)[NQ], const v8h (&ka)[4],
                                                  const v8h (&va)[4], const v8h (&kb)[4], const v8h (&vb)[4],
                                                  int rows_a, int rows_b, bool has_b, float scale, f16* Va, f16* Vb,
                                                  int l16, int q4, Next&& next, Score&& score) {
  const v4f Sa = score(ka, 0);
  const v4f Sb = score(kb, 1);
  float za[4], zb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    za[e] = (4 * q4 + e < rows_a) ? Sa[e] * scale : -INFINITY;
    zb[e] = (has_b && 4 * q4 + e < rows_b) ? Sb[e] * scale : -INFINITY;
  }
  float tm = fmaxf(fmaxf(fmaxf(za[0], za[1]), fmaxf(za[2], za[3])),
                   fmaxf(fmaxf(zb[0], zb[1]), fmaxf(zb[2], zb[3])));
  tm = q4_max(tm);
  const float mn = fmaxf(st.m, tm);
  const bool none = (mn == -INFINITY);
  const float alpha = none ? 1.f : __expf(st.m - mn);
  float pa[4], pb[4];
  float ps_ = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pa[e] = none ? 0.f : __expf(za[e] - mn);
    pb[e] = none ? 0.f : __expf(zb[e] - mn);
    ps_ += pa[e] + pb[e];
  }
  st.l = st.l * alpha + q4_sum(ps_);
  st.m = mn;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st.Ot[n][e] *= alpha;
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Wt[n][e] *= alpha;
  }
  stage_v_tile(Va, va, l16, q4);
  if (has_b) stage_v_tile(Vb, vb, l16, q4);
  next();
  wave_sync_lds();
  exact_pv(st, Va, pa, l16, q4);
  if (has_b) exact_pv(st, Vb, pb, l16, q4);
  wave_sync_lds();
}

template <int NQ, class Next = NoNext>
__device__ __forceinline__ void exact_pair(ExState& st, v4f (&Wt)[NQ], const v8h (&ka)[4], const v8h (&va)[4],
                                           const v8h (&kb)[4], const v8h (&vb)[4], int rows_a, int rows_b,
                                           bool has_b, const v4h (&qf)[4][2], float scale, f16* Va, f16* Vb,
                                           int l16, int q4, Next&& next = Next()) {
  exact_pair_scored<NQ>(st, Wt, ka, va, kb, vb, rows_a, rows_b, has_b, scale, Va, Vb, l16, q4,
                        static_cast<Next&&>(next), PlainScore{qf});
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

// ---- residual rows in the 8- / 4-bit group-quantised formats -------------
// Row x[d] = scale_g code[d] + bias_g, g = d / 64, unsigned codes; 4-bit codes
// two per byte, dimension 2j in the low nibble of byte j.  Codes enter the MFMA
// as exact fp16 integers; the per-row scales and biases are applied in fp32:
//   q.x = s_0 (q.code)_{0..63} + s_1 (q.code)_{64..127} + b_0 sum(q_{0..63}) + b_1 sum(q_{64..127})
//   sum_t p_t x_t[d] = sum_t code_t[d] (s_g p_t) + sum_t b_g p_t
// with s_g p_t rounded to fp16, as the softmax weights of fp16 rows are.

template <int BITS>
struct QTile {
  // per lane: row l16 of the tile, dimensions 32 s + 8 q4 .. + 7 (8 or 4 bytes)
  typename std::conditional<BITS == 8, uint2, uint32_t>::type kc[4], vc[4];
  // per lane: (s0, b0, s1, b1) of rows 4 q4 .. 4 q4 + 3 of the tile
  uint2 ksb[4], vsb[4];
};

// rows past n_ex read row n_ex - 1 (finite, weight 0); n_ex >= 1
template <int BITS>
__device__ __forceinline__ void load_qtile(const uint8_t* kq, const uint8_t* vq, const f16* ks, const f16* vs,
                                           int tile, int ntile, int n_ex, QTile<BITS>& T, int l16, int q4) {
  constexpr int RB = BITS == 8 ? kD : kD / 2;  // code bytes per row
  const int t = tile * 16 + l16;
  const int tc = (tile < ntile && t < n_ex) ? t : n_ex - 1;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t off = (int64_t)tc * RB + (BITS == 8 ? 32 * s + 8 * q4 : 16 * s + 4 * q4);
    if constexpr (BITS == 8) {
      T.kc[s] = *reinterpret_cast<const uint2*>(kq + off);
      T.vc[s] = *reinterpret_cast<const uint2*>(vq + off);
    } else {
      T.kc[s] = *reinterpret_cast<const uint32_t*>(kq + off);
      T.vc[s] = *reinterpret_cast<const uint32_t*>(vq + off);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = tile * 16 + 4 * q4 + e;
    const int rc = (tile < ntile && r < n_ex) ? r : n_ex - 1;
    T.ksb[e] = *reinterpret_cast<const uint2*>(ks + (int64_t)rc * 4);
    T.vsb[e] = *reinterpret_cast<const uint2*>(vs + (int64_t)rc * 4);
  }
}


// One softmax step over two quantised 16-row tiles (b optional).  Q0, Q1: this
// lane's head's query sums over dimensions 0..63 and 64..127.
// ROTK (un-rotated pools): each lane's own key row is dequantised, rotated to
// the block's angle t0 (fq + 64) plus its in-block offset (off_a / off_b) times
// theta_j / 2 pi (fq), rounded once to fp16 and scored; values are as below.
template <int NQ, int BITS, bool ROTK = false, class Next = NoNext>
__device__ __forceinline__ void exact_pair_q(ExState& st, v4f (&Wt)[NQ], const QTile<BITS>& A, const QTile<BITS>& Bq,
                                             int rows_a, int rows_b, bool has_b, const v4h (&qf)[4][2], float Q0,
                                             float Q1, float scale, f16* Va, f16* Vb, int l16, int q4,
                                             Next&& next = Next(), const float* fq = nullptr, float off_a = 0.f,
                                             float off_b = 0.f) {
  // the lane's own row l16: its (scale, bias) pairs are held, as row 4 q4' + e',
  // by the lanes of q4' = l16 / 4
  auto rot_scores = [&](const QTile<BITS>& T, float (&z)[4], int rows, float off) {
    uint32_t sx[4], sy[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sx[e] = (uint32_t)__shfl((int)T.ksb[e].x, 16 * (l16 >> 2));
      sy[e] = (uint32_t)__shfl((int)T.ksb[e].y, 16 * (l16 >> 2));
    }
    const int ee = l16 & 3;
    const uint32_t mx = ee == 0 ? sx[0] : (ee == 1 ? sx[1] : (ee == 2 ? sx[2] : sx[3]));
    const uint32_t my = ee == 0 ? sy[0] : (ee == 1 ? sy[1] : (ee == 2 ? sy[2] : sy[3]));
    const float s0 = h_lo(mx), b0 = h_hi(mx), s1 = h_lo(my), b1 = h_hi(my);
    v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {  // dimension groups s2 (< 64) and s2 + 2 (>= 64), the rotation's pairs
      const v8h ka = codes_to_h8<BITS>(T.kc[s2]);
      const v8h kb = codes_to_h8<BITS>(T.kc[s2 + 2]);
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const int f0 = 32 * s2 + 8 * q4 + 4 * h4;
        const float4 fh = *reinterpret_cast<const float4*>(fq + f0);
        const float4 t0 = *reinterpret_cast<const float4*>(fq + 64 + f0);
        const float fhs[4] = {fh.x, fh.y, fh.z, fh.w}, t0s[4] = {t0.x, t0.y, t0.z, t0.w};
        float xa[4], xb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float cs, sn;
          rope_cs_off(off, fhs[e], t0s[e], cs, sn);
          const float a0 = __builtin_fmaf(s0, (float)ka[4 * h4 + e], b0);
          const float c0 = __builtin_fmaf(s1, (float)kb[4 * h4 + e], b1);
          xa[e] = a0 * cs - c0 * sn;
          xb[e] = c0 * cs + a0 * sn;
        }
        S = mfma16(to_h4(xa), qf[s2][h4], S);
        S = mfma16(to_h4(xb), qf[s2 + 2][h4], S);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = (4 * q4 + e < rows) ? S[e] * scale : -INFINITY;
  };
  // scores per group: rows of the S layout are 4 q4 + e, heads l16
  auto scores = [&](const QTile<BITS>& T, float (&z)[4], int rows) {
    v4f S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v8h k = codes_to_h8<BITS>(T.kc[s]);
      if (s < 2) {
        S0 = mfma16(lo4(k), qf[s][0], S0);
        S0 = mfma16(hi4(k), qf[s][1], S0);
      } else {
        S1 = mfma16(lo4(k), qf[s][0], S1);
        S1 = mfma16(hi4(k), qf[s][1], S1);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s0 = h_lo(T.ksb[e].x), b0 = h_hi(T.ksb[e].x), s1 = h_lo(T.ksb[e].y), b1 = h_hi(T.ksb[e].y);
      const float v = (s0 * S0[e] + s1 * S1[e]) + (b0 * Q0 + b1 * Q1);
      z[e] = (4 * q4 + e < rows) ? v * scale : -INFINITY;
    }
  };
  float za[4], zb[4];
  if constexpr (ROTK) rot_scores(A, za, rows_a, off_a); else scores(A, za, rows_a);
  if (has_b) {
    if constexpr (ROTK) rot_scores(Bq, zb, rows_b, off_b); else scores(Bq, zb, rows_b);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) zb[e] = -INFINITY;
  }
  float tm = fmaxf(fmaxf(fmaxf(za[0], za[1]), fmaxf(za[2], za[3])),
                   fmaxf(fmaxf(zb[0], zb[1]), fmaxf(zb[2], zb[3])));
  tm = q4_max(tm);
  const float mn = fmaxf(st.m, tm);
  const bool none = (mn == -INFINITY);
  const float alpha = none ? 1.f : __expf(st.m - mn);
  float pa[4], pb[4];
  float ps_ = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pa[e] = none ? 0.f : __expf(za[e] - mn);
    pb[e] = none ? 0.f : __expf(zb[e] - mn);
    ps_ += pa[e] + pb[e];
  }
  st.l = st.l * alpha + q4_sum(ps_);
  st.m = mn;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st.Ot[n][e] *= alpha;
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Wt[n][e] *= alpha;
  }
  // the codes of V, staged as exact fp16 integers
  {
    v8h vx[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) vx[s2] = codes_to_h8<BITS>(A.vc[s2]);
    stage_v_tile(Va, vx, l16, q4);
    if (has_b) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) vx[s2] = codes_to_h8<BITS>(Bq.vc[s2]);
      stage_v_tile(Vb, vx, l16, q4);
    }
  }
  wave_sync_lds();
  // per tile: the weights s_g p_t of each group as an fp16 hi + lo pair, the
  // codes of V from LDS, and the bias sums beta_g = sum_t b_g p_t
  float beta0 = 0.f, beta1 = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (tt == 1 && !has_b) break;
    // one tile's LDS reads at a time: keeps the registers they fill few
    __builtin_amdgcn_sched_barrier(0);
    const QTile<BITS>& T = tt == 0 ? A : Bq;
    const float(&pp)[4] = tt == 0 ? pa : pb;
    const f16* Vt = tt == 0 ? Va : Vb;
    const float w0[4] = {h_lo(T.vsb[0].x) * pp[0], h_lo(T.vsb[1].x) * pp[1], h_lo(T.vsb[2].x) * pp[2],
                         h_lo(T.vsb[3].x) * pp[3]};
    const float w1[4] = {h_lo(T.vsb[0].y) * pp[0], h_lo(T.vsb[1].y) * pp[1], h_lo(T.vsb[2].y) * pp[2],
                         h_lo(T.vsb[3].y) * pp[3]};
    const v4h wh[2] = {to_h4(w0), to_h4(w1)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      beta0 += h_hi(T.vsb[e].x) * pp[e];
      beta1 += h_hi(T.vsb[e].y) * pp[e];
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) st.Ot[n] = mfma16(vt_operand(Vt, n, l16, q4), wh[n >> 2], st.Ot[n]);
  }
  beta0 = q4_sum(beta0);
  beta1 = q4_sum(beta1);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const float bb = n < 4 ? beta0 : beta1;
#pragma unroll
    for (int e = 0; e < 4; ++e) st.Ot[n][e] += bb;
  }
  // the tiles' registers are free: load the next pair
  next();
  wave_sync_lds();
}

// NRQ = number of 16-wide column tiles of the augmented rank r + 1 (0 without
// low-rank rows), a template parameter so that every loop over them is static.
// Pool slot of routed block p of unit u from the routed indices and the block
// table (-1: none); the standalone attention kernels use it.
__device__ __forceinline__ int lookup_slot(const BatchArgs& Bt, const AttnArgs& A, int u, int p) {
  const int b = u / Bt.Hkv;
  int nb = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  nb = nb < 0 ? 0 : (nb > Bt.mb ? Bt.mb : nb);
  const int j = A.idx[(int64_t)u * A.top_k + p];
  return (j >= 0 && j < nb) ? Bt.table[(int64_t)b * Bt.mb + j] : -1;
}

// One part of a decode step for unit u = (sequence, KV head), by the whole
// workgroup.  Part p < n_block_parts is routed block p: its low-rank rows and
// residual rows, and, when win_tile_stride > 0, the window's 16-row tiles p,
// p + stride, ..., which are attended first, before get_slot() (which may wait
// for the routing) is called.  Other parts are window chunks of win_chunk rows.
// QK: 0 for pools whose residual rows are fp16, 1 for the quantised formats
// (separate instances, so that the fp16 kernels hold none of that code).
template <int NRQ, int QK, class SlotFn>
__device__ __forceinline__ void attend_part(const PoolArgs& P, const BatchArgs& Bt, const AttnArgs& A, int u, int p,
                                            SlotFn&& get_slot, unsigned char* smem) {
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

  // ---- LDS carve-up
  float* qt = reinterpret_cast<float*>(smem);                     // [16][RQ]  V_K q and q.a_k
  f16* vvx = reinterpret_cast<f16*>(qt + 16 * RQ);                // [RQ][kVStride]  [V_V ; a_v ; *]
  float* wstat = reinterpret_cast<float*>(vvx + RQ * kVStride);   // m [4][16], l [4][16]
  unsigned char* region = reinterpret_cast<unsigned char*>(wstat + 2 * kAttWaves * 16);
  unsigned char* my = region + wave * att_scratch_bytes(RQ);
  uint32_t* wmask = reinterpret_cast<uint32_t*>(my + att_scratch_bytes(RQ) - 32);
  const float scale = A.scale;

  ExState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.Ot[n] = (v4f){0.f, 0.f, 0.f, 0.f};
  v4f Wt[NQ];  // W^T[j = 16 n + 4 q4 + e][head l16] = sum over positions of Ux[pos][j] p[pos][head]
#pragma unroll
  for (int n = 0; n < NQ; ++n) Wt[n] = (v4f){0.f, 0.f, 0.f, 0.f};

  int wl = Bt.wlen ? Bt.wlen[b] : Bt.W;
  wl = wl < 0 ? 0 : (wl > Bt.W ? Bt.W : wl);
  const int64_t win_base = (((int64_t)b * Bt.Hkv + h) * Bt.W) * kD;

  // ---- window tiles owned by a routed-block part: exact rows that do not
  //      depend on the routing, attended while it may still be running
  bool any = false;
  if (QK < 2 && p < A.n_block_parts && A.win_tile_stride > 0) {
    const int n_wt = (wl + 15) >> 4;
    any = p < n_wt;  // uniform
    f16* Va = reinterpret_cast<f16*>(my);
    f16* Vb = Va + kD * kVTStride;
    v8h ka[4], va[4], kb[4], vb[4];
    for (int i = wave; p + A.win_tile_stride * i < n_wt; i += 2 * kAttWaves) {
      const int wa = p + A.win_tile_stride * i, wb = p + A.win_tile_stride * (i + kAttWaves);
      const bool has_b = wb < n_wt;
      const int ra = wl - 16 * wa < 16 ? wl - 16 * wa : 16;
      const int rb = has_b ? (wl - 16 * wb < 16 ? wl - 16 * wb : 16) : 0;
      load_exact_tile(Bt.wk + win_base + (int64_t)16 * wa * kD, Bt.wv + win_base + (int64_t)16 * wa * kD, 0, 1, ra,
                      ka, va, l16, q4);
      load_exact_tile(Bt.wk + win_base + (int64_t)16 * (has_b ? wb : wa) * kD,
                      Bt.wv + win_base + (int64_t)16 * (has_b ? wb : wa) * kD, 0, 1, has_b ? rb : ra, kb, vb, l16, q4);
      exact_pair<NQ>(st, Wt, ka, va, kb, vb, ra, rb, has_b, qf, scale, Va, Vb, l16, q4);
    }
  }

  // ---- what else this part covers (uniform over the workgroup)
  bool lr = false;
  int n_ex = 0;
  const f16* exk = nullptr;
  const f16* exv = nullptr;
  // residual rows in a quantised format: codes and (scale, bias) pairs
  int qbits = 0;
  const uint8_t* exkq = nullptr;
  const uint8_t* exvq = nullptr;
  const f16* exks = nullptr;
  const f16* exvs = nullptr;
  int slot = -1;
  int bpos = 0;  // un-rotated pools: absolute position of the block's token 0
  int bslot = 0; // the vk / vv entry of the block (its slot unless the basis is shared)
  if (p < A.n_block_parts) {
    slot = get_slot();  // routed pool slot, or -1
    if (slot >= P.n_slots) slot = -1;
    bslot = slot;
    if constexpr (QK >= 2) {
      if (slot >= 0 && P.basis) {
        const int g = P.basis[slot];
        if (g < 0 || g >= P.n_basis) slot = -1;  // no basis: no rows
        bslot = g;
      }
    }
    if (slot >= 0) {
      if constexpr (QK >= 2) bpos = P.spos[slot];
      lr = (A.block_mode & 1) != 0;
      if ((A.block_mode & 2) && P.n_resid > 0) {
        n_ex = P.n_resid;
        if (P.rfmt == 0) {
          exk = P.rk + slot * P.rk_s + h * P.rk_h;
          exv = P.rv + slot * P.rv_s + h * P.rv_h;
        } else {
          qbits = P.rfmt == 1 ? 8 : 4;
          exkq = P.rkq + slot * P.rkq_s + h * P.rkq_h;
          exvq = P.rvq + slot * P.rvq_s + h * P.rvq_h;
          exks = P.rks + slot * P.rks_s + h * P.rks_h;
          exvs = P.rvs + slot * P.rvs_s + h * P.rvs_h;
        }
      }
    }
  } else {
    const int s = p - A.n_block_parts;
    const int start = s * A.win_chunk;
    const int end = (start + A.win_chunk < wl) ? start + A.win_chunk : wl;
    if (end > start) {
      n_ex = end - start;
      exk = Bt.wk + win_base + (int64_t)start * kD;
      exv = Bt.wv + win_base + (int64_t)start * kD;
    }
  }

  const int part = A.part_offset + p;
  if (!lr && n_ex == 0 && !any) {
    for (int t = tid; t < G * kD; t += kAttThreads) {
      const int g = t / kD, d = t % kD;
      st_dev(&A.part_o[((int64_t)(row0 + g) * A.n_parts + part) * kD + d], 0.f);
    }
    if (tid < G) st_dev(&A.part_lse[(int64_t)(row0 + tid) * A.n_parts + part], -INFINITY);
    return;
  }
  // Everything from here on is straight-line from the issue of the loads to
  // their uses (with or without the low-rank rows, chosen once), so that the
  // compiler's wait counts let the first data be used while the rest is still
  // in flight.
  auto body = [&](auto lr_tag, auto bits_tag) {
  constexpr bool LR = decltype(lr_tag)::value && NRQ > 0;
  constexpr int QB = decltype(bits_tag)::value;  // 0: fp16 exact rows; 8 / 4: quantised residual rows
  // QK == 2 / 3: an un-rotated pool (fp16 / quantised residual rows), whose block keys are rotated to their
  // absolute positions here; the frequency table sits in the statistics area
  // until the final phase
  constexpr bool ROT = QK == 2 || QK == 3;
  const int ntile = (n_ex + 15) >> 4;
  const int r = P.rank;
  float* fq = wstat;  // ROT: theta_j / (2 pi) [64], then the block's angles in turns [64]
  if constexpr (ROT) {
    if (tid < 64) {
      fq[tid] = P.rope[tid];
    } else if (tid < 128) {
      const int j = tid - 64;
      const float fh = P.rope[j], fl = P.rope[64 + j], pf = (float)bpos;
      const float a = pf * fh;
      const float e = __builtin_fmaf(pf, fh, -a);
      fq[tid] = __builtin_amdgcn_fractf(__builtin_amdgcn_fractf(a) + __builtin_fmaf(pf, fl, e));
    }
    if constexpr (!LR) lds_barrier();
  }

  // ---- issue the loads, in the order of use
  v4h ua[kLRTilesPerWave][NQ];
  int ps[4];
  v8h vvl[kVVChunks];
  v8h vkx[2][4];
  const f16* U = nullptr;
  if constexpr (LR) {
    const f16* AK = P.ak + slot * P.ak_s + h * P.ak_h;
    const f16* AV = P.av + slot * P.av_s + h * P.av_h;
    const f16* VK = P.vk + bslot * P.vk_s + h * P.vk_h;
    const f16* VV = P.vv + bslot * P.vv_s + h * P.vv_h;
    U = P.u + slot * P.u_s + h * P.u_h;
    {
      // positions 0 (none) for lanes past n_resid; a pool without residual rows
      // reads (and ignores) the first byte of the block's U
      const int nres = P.n_resid;
      const uint8_t* pp = nres > 0 ? P.rp + slot * P.rp_s + h * P.rp_h : reinterpret_cast<const uint8_t*>(U);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = lane + 64 * k;
        const int v = (int)pp[t < nres ? t : 0];
        ps[k] = t < nres ? v : 0;
      }
    }
    // VVx rows: V_V rows j < r, a_v at j = r.  Padding rows j > r read V_V row 0:
    // their weight in (p^T Ux) is exactly 0 because Ux is zero there.  (An
    // un-rotated pool loads them half-way through its scores.)
    if constexpr (!ROT) {
#pragma unroll
      for (int k = 0; k < kVVChunks; ++k) {
        const int c = tid + kAttThreads * k;
        const int j = (c < RQ * 16) ? (c >> 4) : 0, col = (c & 15) * 8;
        const f16* src = (j < r) ? VV + (int64_t)j * kD : ((j == r) ? AV : VV);
        vvl[k] = ld8(src + col);
      }
    }
    // VKx rows: V_K rows j < r, a_k at j = r; padding rows read V_K row 0
    // (they only meet zero columns of Ux)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (kAttWaves * k < NRQ) {  // compile time; every wave loads (tiles past NRQ read V_K row 0, unused)
        const int j = (wave + kAttWaves * k) * 16 + l16;
        const f16* src = (j < r) ? VK + (int64_t)j * kD : ((j == r) ? AK : VK);
#pragma unroll
        for (int s = 0; s < 4; ++s) vkx[k][s] = ld8(src + 32 * s + 8 * q4);
      }
    }
    // U: four columns j0 .. j0 + 3 of row i - 1 per lane, as one 8-byte load
    // (2-byte aligned when r % 4 != 0).  Padding columns read columns 0 .. 3.
    // A load that would run past the block's last U element starts 1 .. 3
    // elements earlier and is shifted back into place before use.
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k) {
      const int i = (wave + kAttWaves * k) * 16 + l16;  // position in the block; 0 = anchor
      const int row = i > 0 ? i - 1 : 0;
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const int j0 = 16 * s + 4 * q4;
        const int e0 = row * r + (j0 < r ? j0 : 0);
        const int lim = kLowRankRows * r - 4;
        __builtin_memcpy(&ua[k][s], U + (e0 < lim ? e0 : (lim > 0 ? lim : 0)), 8);
      }
    }
  }
  // The wave's first two exact tiles.  Issued in every case (a part without
  // exact rows reads its first query row, unused), so that no branch separates
  // these loads from the waits for earlier ones.  With low-rank rows they are
  // issued once the low-rank scores are formed: the U registers are free by
  // then, and the loads overlap the rest of the low-rank step while this
  // workgroup's first burst has already been consumed.
  v8h ka[4], va[4], kb[4], vb[4];
  QTile<QB == 4 ? 4 : 8> qta, qtb;  // quantised residual tiles (QB != 0; n_ex > 0 there)
  int ta = wave, tb = wave + kAttWaves;
  auto issue_exact = [&]() {
    if constexpr (QB == 0) {
      const bool none = n_ex == 0;
      const f16* qrow0 = Bt.q + (int64_t)row0 * kD;
      load_exact_tile(none ? qrow0 : exk, none ? qrow0 : exv, ta, none ? 1 : ntile, none ? 1 : n_ex, ka, va, l16,
                      q4);
      load_exact_tile(none ? qrow0 : exk, none ? qrow0 : exv, tb, none ? 1 : ntile, none ? 1 : n_ex, kb, vb, l16,
                      q4);
    } else {
      load_qtile<QB>(exkq, exvq, exks, exvs, ta, ntile, n_ex, qta, l16, q4);
      load_qtile<QB>(exkq, exvq, exks, exvs, tb, ntile, n_ex, qtb, l16, q4);
    }
  };
  if constexpr (!LR) issue_exact();

  // ---- low-rank set-up: residual-position mask (per wave), VVx, VKx q
  if constexpr (LR) {
    if (lane < 8) wmask[lane] = 0u;
    wave_sync_lds();
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (ps[k] >= 1 && ps[k] <= kLowRankRows) atomicOr(&wmask[ps[k] >> 5], 1u << (ps[k] & 31));
    if constexpr (!ROT) {
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
    } else {
      // VKx^T [d][j] over the V_K q and VVx areas (VVx is staged after the scores)
      f16* vkt = reinterpret_cast<f16*>(qt);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int jt = wave + kAttWaves * k;
        if (jt < NRQ) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) vkt[vkt_at(RQ, 32 * s + 8 * q4 + jj, jt * 16 + l16)] = vkx[k][s][jj];
          }
        }
      }
    }
    lds_barrier();  // V_K q (or VKx^T) and VVx complete (uniform: lr is uniform)

    // ---- the wave's four 16-position tiles as one softmax step (position 0 is the anchor)
    v4h qth[NQ], qtl[NQ];
    if constexpr (!ROT) {
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const float4 x = *reinterpret_cast<const float4*>(qt + l16 * RQ + 16 * s + 4 * q4);
        split_hl(x.x, x.y, x.z, x.w, qth[s], qtl[s]);
      }
    }
    f16* T = reinterpret_cast<f16*>(my);  // Ux^T [RQ][kTTStride]: column j of the wave's 64 positions
    float zz[kLRTilesPerWave][4];
    // Ux = [U | 1 | 0]; the anchor row has U = 0.  Per lane and 16-column
    // tile: a 64-bit mask keeping the columns below r and the fp16 1.0 at
    // column r (if it is among the lane's four).
    uint64_t keep[NQ], one[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int j0 = 16 * s + 4 * q4;
      const int nk = r - j0;  // columns of the four below r
      keep[s] = nk >= 4 ? ~0ull : (nk <= 0 ? 0ull : ((1ull << (16 * nk)) - 1ull));
      one[s] = (nk >= 0 && nk < 4) ? (0x3C00ull << (16 * nk)) : 0ull;
    }
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k) {
      const int i0 = (wave + kAttWaves * k) * 16;
      const int i = i0 + l16;
      const int row = i > 0 ? i - 1 : 0;
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        const int j0 = 16 * s + 4 * q4;
        const int e0 = row * r + (j0 < r ? j0 : 0);
        const int lim = kLowRankRows * r - 4;
        const int back = e0 - (e0 < lim ? e0 : (lim > 0 ? lim : 0));  // 0 .. 3 elements
        uint64_t w = __builtin_bit_cast(uint64_t, ua[k][s]) >> (16 * back);
        w = (w & (i > 0 ? keep[s] : 0ull)) | one[s];
        ua[k][s] = __builtin_bit_cast(v4h, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) T[(16 * s + 4 * q4 + e) * kTTStride + k * 16 + l16] = ua[k][s][e];
      }
      v4f z = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!ROT) {
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          z = mfma16(ua[k][s], qth[s], z);
          z = mfma16(ua[k][s], qtl[s], z);
        }
      } else {
        // the 16 keys themselves, K^T = VKx^T Ux^T in fp32: kt holds
        // dimensions 32 s + 8 q4 + 4 hh + e of position i0 + l16 (the order of
        // the query fragments), rotated in fp32 and rounded once to fp16, the
        // precision of the rotated keys a rotated pool stores
        // Two halves: dimension groups s = hf and s = hf + 2 (the rotation's
        // pairs), m = 2 (s >> 1) + hh.
        const f16* vkt = reinterpret_cast<const f16*>(qt);
        const float off = (float)i;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          v4f kt[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) kt[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < NQ; ++t) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int dim = 32 * (hf + 2 * (m >> 1)) + 8 * (l16 >> 2) + 4 * (m & 1) + (l16 & 3);
              const v4h a = *reinterpret_cast<const v4h*>(vkt + vkt_at(RQ, dim, 16 * t + 4 * q4));
              kt[m] = mfma16(a, ua[k][t], kt[m]);
            }
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int f0 = 32 * hf + 8 * q4 + 4 * hh;
            const float4 fh = *reinterpret_cast<const float4*>(fq + f0);
            const float4 t0 = *reinterpret_cast<const float4*>(fq + 64 + f0);
            const float fhs[4] = {fh.x, fh.y, fh.z, fh.w}, t0s[4] = {t0.x, t0.y, t0.z, t0.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float cs, sn;
              rope_cs_off(off, fhs[e], t0s[e], cs, sn);
              const float x = kt[hh][e], y = kt[2 + hh][e];
              kt[hh][e] = x * cs - y * sn;
              kt[2 + hh][e] = y * cs + x * sn;
            }
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float km[4] = {kt[m][0], kt[m][1], kt[m][2], kt[m][3]};
            z = mfma16(to_h4(km), qf[hf + 2 * (m >> 1)][m & 1], z);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = i0 + 4 * q4 + e;
        const bool masked = (ii > 0) & (((wmask[ii >> 5] >> (ii & 31)) & 1u) != 0u);
        zz[k][e] = masked ? -INFINITY : z[e] * scale;
      }
      if constexpr (ROT) {
        // V_V and a_v, into the registers of the U tiles already used: after
        // the second tile, or (the largest ranks, short of registers) the last
        if (k == (NRQ >= 5 ? kLRTilesPerWave - 1 : 1)) {
          const f16* AV = P.av + slot * P.av_s + h * P.av_h;
          const f16* VV = P.vv + bslot * P.vv_s + h * P.vv_h;
#pragma unroll
          for (int c2 = 0; c2 < kVVChunks; ++c2) {
            const int c = tid + kAttThreads * c2;
            const int j = (c < RQ * 16) ? (c >> 4) : 0, col = (c & 15) * 8;
            const f16* src = (j < r) ? VV + (int64_t)j * kD : ((j == r) ? AV : VV);
            vvl[c2] = ld8(src + col);
          }
        }
      }
    }
    issue_exact();
    float tm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k)
      tm = fmaxf(tm, fmaxf(fmaxf(zz[k][0], zz[k][1]), fmaxf(zz[k][2], zz[k][3])));
    tm = q4_max(tm);
    const float mn = fmaxf(st.m, tm);
    const bool none = (mn == -INFINITY);
    const float alpha = none ? 1.f : __expf(st.m - mn);
    float pe[kLRTilesPerWave][4];
    float ps_ = 0.f;
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[k][e] = none ? 0.f : __expf(zz[k][e] - mn);
        ps_ += pe[k][e];
      }
    }
    st.l = st.l * alpha + q4_sum(ps_);
    st.m = mn;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int e = 0; e < 4; ++e) st.Ot[n][e] *= alpha;  // (W^T is still zero here)
    }
    wave_sync_lds();
#pragma unroll
    for (int k = 0; k < kLRTilesPerWave; ++k) {
      const v4h ph = to_h4(pe[k]);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const v4h au = *reinterpret_cast<const v4h*>(T + (16 * n + l16) * kTTStride + k * 16 + 4 * q4);
        Wt[n] = mfma16(au, ph, Wt[n]);
      }
    }
    wave_sync_lds();
  }

  // ---- exact rows: two 16-row tiles per softmax step
  if (QB != 0 && n_ex > 0) {
    f16* Va = reinterpret_cast<f16*>(my);
    f16* Vb = Va + kD * kVTStride;
    // this lane's head's query sums over dimensions 0..63 and 64..127
    float Q0 = 0.f, Q1 = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = (float)qf[s2][0][e] + (float)qf[s2][1][e];
        if (s2 < 2) Q0 += x; else Q1 += x;
      }
    }
    Q0 = q4_sum(Q0);
    Q1 = q4_sum(Q1);
    // un-rotated pools: the in-block position of the lane's residual row
    auto row_off = [&](int tile) -> float {
      if constexpr (ROT) {
        const int row = 16 * tile + l16;
        int rpos;
        if constexpr (LR) {
          const int k4 = tile >> 2;
          const int src = k4 == 0 ? ps[0] : (k4 == 1 ? ps[1] : (k4 == 2 ? ps[2] : ps[3]));
          rpos = __shfl(src, 16 * (tile & 3) + l16);
        } else {
          rpos = row < n_ex ? (int)P.rp[slot * P.rp_s + h * P.rp_h + row] : 0;
        }
        return (float)(row < n_ex ? rpos : 0);
      } else {
        return 0.f;
      }
    };
    while (ta < ntile) {
      const bool has_b = tb < ntile;  // uniform over the wave
      const int ta_n = ta + 2 * kAttWaves, tb_n = tb + 2 * kAttWaves;
      exact_pair_q<NQ, (QB == 4 ? 4 : 8), ROT>(st, Wt, qta, qtb, n_ex - 16 * ta, n_ex - 16 * tb, has_b, qf, Q0, Q1,
                                               scale, Va, Vb, l16, q4, [&]() {
        if (ta_n < ntile) load_qtile<(QB == 4 ? 4 : 8)>(exkq, exvq, exks, exvs, ta_n, ntile, n_ex, qta, l16, q4);
        if (tb_n < ntile) load_qtile<(QB == 4 ? 4 : 8)>(exkq, exvq, exks, exvs, tb_n, ntile, n_ex, qtb, l16, q4);
      }, fq, row_off(ta), row_off(tb));
      ta = ta_n;
      tb = tb_n;
    }
  }
  if (QB == 0 && n_ex > 0 && !(ROT && p < A.n_block_parts)) {
    f16* Va = reinterpret_cast<f16*>(my);
    f16* Vb = Va + kD * kVTStride;
    while (ta < ntile) {
      const bool has_b = tb < ntile;  // uniform over the wave
      const int ta_n = ta + 2 * kAttWaves, tb_n = tb + 2 * kAttWaves;
      exact_pair<NQ>(st, Wt, ka, va, kb, vb, n_ex - 16 * ta, n_ex - 16 * tb, has_b, qf, scale, Va, Vb, l16, q4,
                     [&]() {
                       if (ta_n < ntile) load_exact_tile(exk, exv, ta_n, ntile, n_ex, ka, va, l16, q4);
                       if (tb_n < ntile) load_exact_tile(exk, exv, tb_n, ntile, n_ex, kb, vb, l16, q4);
                     });
      ta = ta_n;
      tb = tb_n;
    }
  }
  if constexpr (ROT && QB == 0) {
    // residual rows of an un-rotated block: row t of the pool is rotated to
    // the block's position + resid_pos[t] (in fp32, rounded once to fp16)
    if (n_ex > 0 && p < A.n_block_parts) {
      f16* Va = reinterpret_cast<f16*>(my);
      f16* Vb = Va + kD * kVTStride;
      const uint8_t* rpb = P.rp + slot * P.rp_s + h * P.rp_h;
      auto rot_score = [&](const v8h (&kx)[4], int which) -> v4f {
        const int tile = which == 0 ? ta : tb;
        const int row = 16 * tile + l16;
        int rpos;
        if constexpr (LR) {
          // the low-rank pass holds every residual position in registers
          // (position t in lane t % 64 of ps[t / 64]): a cross-lane read
          const int k4 = tile >> 2;
          const int src = k4 == 0 ? ps[0] : (k4 == 1 ? ps[1] : (k4 == 2 ? ps[2] : ps[3]));
          rpos = __shfl(src, 16 * (tile & 3) + l16);
        } else {
          rpos = row < n_ex ? (int)rpb[row] : 0;
        }
        const float off = (float)(row < n_ex ? rpos : 0);
        v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {  // dimension groups s2 and s2 + 2 (the rotation's pairs)
#pragma unroll
          for (int h4 = 0; h4 < 2; ++h4) {
            const int f0 = 32 * s2 + 8 * q4 + 4 * h4;
            const float4 fh = *reinterpret_cast<const float4*>(fq + f0);
            const float4 t0 = *reinterpret_cast<const float4*>(fq + 64 + f0);
            const float fhs[4] = {fh.x, fh.y, fh.z, fh.w}, t0s[4] = {t0.x, t0.y, t0.z, t0.w};
            float xa[4], xb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float cs, sn;
              rope_cs_off(off, fhs[e], t0s[e], cs, sn);
              const float a0 = (float)kx[s2][4 * h4 + e], b0 = (float)kx[s2 + 2][4 * h4 + e];
              xa[e] = a0 * cs - b0 * sn;
              xb[e] = b0 * cs + a0 * sn;
            }
            S = mfma16(to_h4(xa), qf[s2][h4], S);
            S = mfma16(to_h4(xb), qf[s2 + 2][h4], S);
          }
        }
        return S;
      };
      while (ta < ntile) {
        const bool has_b = tb < ntile;  // uniform over the wave
        const int ta_n = ta + 2 * kAttWaves, tb_n = tb + 2 * kAttWaves;
        exact_pair_scored<NQ>(st, Wt, ka, va, kb, vb, n_ex - 16 * ta, n_ex - 16 * tb, has_b, scale, Va, Vb, l16,
                              q4, [&]() {
                                if (ta_n < ntile) load_exact_tile(exk, exv, ta_n, ntile, n_ex, ka, va, l16, q4);
                                if (tb_n < ntile) load_exact_tile(exk, exv, tb_n, ntile, n_ex, kb, vb, l16, q4);
                              }, rot_score);
        ta = ta_n;
        tb = tb_n;
      }
    }
  }
  if constexpr (ROT) {
    lds_barrier();  // every wave is done with the frequency table (and VKx^T)
    if constexpr (LR) {
#pragma unroll
      for (int k = 0; k < kVVChunks; ++k) {
        const int c = tid + kAttThreads * k;
        if (c < RQ * 16) {
          const int j = c >> 4, col = (c & 15) * 8;
          *reinterpret_cast<v4h*>(vvx + j * kVStride + col) = lo4(vvl[k]);
          *reinterpret_cast<v4h*>(vvx + j * kVStride + col + 4) = hi4(vvl[k]);
        }
      }
    }
  }

  // ---- final phase: common maximum over the waves; the low-rank values
  //      (VVx^T W^T, linear in W) folded once from the waves' summed W^T;
  //      fixed-order sum over the waves; stores
  if (q4 == 0) {
    wstat[wave * 16 + l16] = st.m;
    wstat[kAttWaves * 16 + wave * 16 + l16] = st.l;
  }
  lds_barrier();  // statistics visible; every wave is done with its scratch
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, wstat[w * 16 + l16]);
  const float be = (st.m == -INFINITY) ? 0.f : __expf(st.m - M);
  float* red = reinterpret_cast<float*>(region);  // [kAttWaves][16 heads][kRedStride]
  v4f F[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};  // VVx^T W^T for d tiles 2 wave, 2 wave + 1
  if constexpr (LR) {
    constexpr int WS = RQ + 4;  // floats per head row of wred
    float* wred = red;          // [kAttWaves][16 heads][WS]: each wave's W, at the common maximum
#pragma unroll
    for (int s = 0; s < NQ; ++s)
      *reinterpret_cast<float4*>(wred + (wave * 16 + l16) * WS + 16 * s + 4 * q4) =
          make_float4(Wt[s][0] * be, Wt[s][1] * be, Wt[s][2] * be, Wt[s][3] * be);
    lds_barrier();
    v4h wh[NQ], wl[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kAttWaves; ++w) {
        const float4 y = *reinterpret_cast<const float4*>(wred + (w * 16 + l16) * WS + 16 * s + 4 * q4);
        x.x += y.x;
        x.y += y.y;
        x.z += y.z;
        x.w += y.w;
      }
      split_hl(x.x, x.y, x.z, x.w, wh[s], wl[s]);
    }
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int n = 2 * wave + nn;
#pragma unroll
      for (int s = 0; s < NRQ; ++s) {
        v4h av;
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = vvx[(16 * s + 4 * q4 + e) * kVStride + 16 * n + l16];
        F[nn] = mfma16(av, wh[s], F[nn]);
        F[nn] = mfma16(av, wl[s], F[nn]);
      }
    }
    lds_barrier();  // every wave has read wred before red overwrites it
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    float4 v = make_float4(st.Ot[n][0] * be, st.Ot[n][1] * be, st.Ot[n][2] * be, st.Ot[n][3] * be);
    if ((n >> 1) == wave) {  // uniform
      const v4f f = F[n & 1];
      v.x += f[0];
      v.y += f[1];
      v.z += f[2];
      v.w += f[3];
    }
    *reinterpret_cast<float4*>(red + (wave * 16 + l16) * kRedStride + 16 * n + 4 * q4) = v;
  }
  lds_barrier();
  const __amdgpu_buffer_rsrc_t Po = coherent_rsrc(A.part_o + ((int64_t)row0 * A.n_parts + part) * kD, 0xFFFFFFFFu);
  for (int t = tid; t < G * (kD / 4); t += kAttThreads) {
    const int g = t / (kD / 4), c4 = t % (kD / 4);
    float Mg = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) Mg = fmaxf(Mg, wstat[w * 16 + g]);
    float Lg = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
      const float mw = wstat[w * 16 + g];
      Lg += (mw == -INFINITY) ? 0.f : wstat[kAttWaves * 16 + w * 16 + g] * __expf(mw - Mg);
      const float4 x = *reinterpret_cast<const float4*>(red + (w * 16 + g) * kRedStride + 4 * c4);
      o.x += x.x;
      o.y += x.y;
      o.z += x.z;
      o.w += x.w;
    }
    const float inv = (Lg > 0.f) ? 1.f / Lg : 0.f;
    st_coherent4(Po, (uint32_t)((g * A.n_parts * kD + 4 * c4) * 4),
                 make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
    if (c4 == 0) st_dev(&A.part_lse[(int64_t)(row0 + g) * A.n_parts + part], (Lg > 0.f) ? Mg + __logf(Lg) : -INFINITY);
  }
  };
  using I0 = std::integral_constant<int, 0>;
  using I8 = std::integral_constant<int, 8>;
  using I4 = std::integral_constant<int, 4>;
  if constexpr (QK == 0 || QK == 2) {
    if (NRQ > 0 && lr)
      body(std::true_type{}, I0{});
    else
      body(std::false_type{}, I0{});
  } else {
    if (NRQ > 0 && lr) {
      if (qbits == 8)
        body(std::true_type{}, I8{});
      else if (qbits == 4)
        body(std::true_type{}, I4{});
      else
        body(std::true_type{}, I0{});
    } else {
      if (qbits == 8)
        body(std::false_type{}, I8{});
      else if (qbits == 4)
        body(std::false_type{}, I4{});
      else
        body(std::false_type{}, I0{});
    }
  }
}

template <int NRQ, int QK>
__global__ __launch_bounds__(kAttThreads, 2) void k_attend(PoolArgs P, BatchArgs Bt, AttnArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int item = blockIdx.x;
  const int u = item / A.items_per_unit, p = item % A.items_per_unit;
  attend_part<NRQ, QK>(P, Bt, A, u, p, [&]() { return lookup_slot(Bt, A, u, p); }, smem);
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine: one workgroup of 4 waves per query row; wave w takes
// parts w, w + 4, ... (16 at a time, all loads in flight); fixed-order sums.
// ----------------------------------------------------------------------------

constexpr int kMergeThreads = 256;
constexpr int kMergeUnroll = 16;

__global__ __launch_bounds__(kMergeThreads) void k_merge(const float* part_o, const float* part_lse,
                                                        int n_parts, f16* out, float* out_lse) {
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
  lds_barrier();
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
  lds_barrier();
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
// The routed block of part p of unit u under a split routing: wait (bounded)
// until the unit's score items have written all of its (slot, score) words,
// then rank the blocks exactly as route_unit does (the same selection on the
// same scores) and take the one at position p in ascending block order.  The
// part also writes that position of the routed indices (-1 past the routed
// count).  Returns the pool slot, or -1 (no block).
__device__ __forceinline__ int split_route_slot(const BatchArgs& Bt, const DecodeArgs& D, int u, int p,
                                                unsigned char* smem, RouteShared<kAttWaves>& rsh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = u / Bt.Hkv;
  int N = (Bt.nblk && Bt.mb > 0) ? Bt.nblk[b] : 0;
  N = N < 0 ? 0 : (N > Bt.mb ? Bt.mb : N);
  const int keff = D.att.top_k < N ? D.att.top_k : N;
  const int mbp = ((Bt.mb > 0 ? Bt.mb : 1) + 3) & ~3;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  int32_t* slot_of = reinterpret_cast<int32_t*>(keys + mbp);
  const uint64_t* src = D.rwords + (int64_t)u * Bt.mb;
  lds_barrier();  // every wave is past its window tiles, whose LDS scratch is reused here
  if (tid == 0) {
    rsh.pick_j = -1;
    rsh.pick_slot = -1;
  }
  bool ready = false;
  for (unsigned n = 0;; ++n) {
    bool ok = true;
    for (int j = tid; j < N; j += kAttThreads) {
      const uint64_t v = ld_dev(src + j);
      const uint32_t hi = (uint32_t)(v >> 32);
      ok = ok && hi != 0u;
      keys[j] = (uint32_t)v;
      slot_of[j] = (int32_t)hi - kSlotCode;
    }
    const bool wok = __all(ok);
    if (lane == 0) rsh.ready[n & 1][wave] = wok ? 1u : 0u;
    lds_barrier();
    uint32_t all = 1u;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) all &= rsh.ready[n & 1][w];
    if (all) {
      ready = true;
      break;
    }
    if (n >= kRouteWaitLimit) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ready) {
    if (tid == 0) {
      atomicOr(&D.ctrl[2], 1u);  // give up: an empty part
      st_dev(&D.idx[(int64_t)u * D.att.top_k + p], -1);
    }
    return -1;
  }
  route_select<kAttThreads>(keys, N, keff, keys, mbp, rsh, [&](int pos, int j, uint32_t) {
    if (pos == p) {
      rsh.pick_j = j;
      rsh.pick_slot = slot_of[j];
    }
  });
  lds_barrier();
  const int j = rsh.pick_j, slot = rsh.pick_slot;
  if (tid == 0) st_dev(&D.idx[(int64_t)u * D.att.top_k + p], j);
  return slot;
}

// One work item of a fused decode step: t < n_route routes, unit t /
// route_items; then the parts (u, p) = ((t - n_route) / P, (t - n_route) % P);
// then the merges, per query row (u, g) or per unit u.  sh_slot: a shared word
// of the calling workgroup.  SPLIT: the routing items are score items
// (score_slice, one per kScoreChunk blocks of a unit) and each block part
// selects its own block (split_route_slot); otherwise one route_unit per unit.
template <int NRQ, int QK, bool SPLIT = false>
__device__ __forceinline__ void decode_item(const PoolArgs& P, const BatchArgs& Bt, const DecodeArgs& D, int t,
                                            unsigned char* smem, RouteShared<kAttWaves>& rsh, int32_t& sh_slot) {
  const int tid = threadIdx.x;
  if (t < 0) {
    // no item
  } else if (t < D.n_route) {
    __builtin_amdgcn_s_setprio(2);  // every other item of the launch waits on routing
    if constexpr (SPLIT) {
      const int u = t / D.route_items, s = t % D.route_items;
      score_slice<kAttThreads>(P, Bt, u, s * kScoreChunk, (s + 1) * kScoreChunk, D.rwords + (int64_t)u * Bt.mb,
                               reinterpret_cast<float*>(smem));
      // counted once its words are written: the launch's last merge clears
      // the words only after every score item is counted
      stores_done();
      __syncthreads();
      if (tid == 0) atomicAdd(&D.ctrl[kCtrlScored], 1u);
    } else {
      route_unit<kAttThreads>(P, Bt, t, D.att.top_k, D.idx, nullptr, D.slots, reinterpret_cast<uint32_t*>(smem), rsh,
                              slot_tag(ld_dev(&D.ctrl[3])));
    }
  } else if (t < D.n_part_end) {
    const int it = t - D.n_route;
    const int u = it / D.att.items_per_unit, p = it % D.att.items_per_unit;
    // the routed slot of a block part: wait (bounded) until the unit's routing
    // has written it; called after the part's window tiles are done
    auto get_slot = [&]() {
      if constexpr (SPLIT) {
        return split_route_slot(Bt, D, u, p, smem, rsh);
      } else {
        if (tid == 0) {
          const int32_t* sp = &D.slots[(int64_t)u * D.att.top_k + p];
          const uint32_t tag = slot_tag(ld_dev(&D.ctrl[3]));
          unsigned n = 0;
          int32_t v = ld_dev(sp);
          while (!slot_ready(v, tag) && n < kRouteWaitLimit) {
            __builtin_amdgcn_s_sleep(1);
            v = ld_dev(sp);
            ++n;
          }
          if (!slot_ready(v, tag)) {
            atomicOr(&D.ctrl[2], 1u);
            v = (int32_t)(tag | (uint32_t)(-1 + kSlotCode));  // give up: an empty part
          }
          sh_slot = slot_value(v);
        }
        lds_barrier();
        return (int)sh_slot;
      }
    };
    attend_part<NRQ, QK>(P, Bt, D.att, u, p, get_slot, smem);
    // count this part once its partial is stored
    stores_done();
    __syncthreads();
    if (tid == 0) atomicAdd(&D.unit_done[u * kDoneStride], 1u);
  } else if (t < D.n_items) {
    // merge item: one query row of a unit, or all G of them, once all of the
    // unit's parts are stored
    const int it = t - D.n_part_end;
    const int u = it / D.merges, g = it % D.merges;
    if (tid == 0) {
      const uint32_t want = (uint32_t)D.att.items_per_unit;
      unsigned n = 0;
      uint32_t v = ld_dev(&D.unit_done[u * kDoneStride]);
      while (v < want && n < kRouteWaitLimit) {
        __builtin_amdgcn_s_sleep(2);
        v = ld_dev(&D.unit_done[u * kDoneStride]);
        ++n;
      }
      if (v < want) atomicOr(&D.ctrl[2], 1u);
    }
    lds_barrier();
    const int b = u / Bt.Hkv, h = u % Bt.Hkv;
    if (D.merges == 1)
      merge_unit(D.att.part_o, D.att.part_lse, D.att.n_parts, b * Bt.Hq + h * Bt.G, Bt.G, D.out, D.out_lse);
    else
      merge_row(D.att.part_o, D.att.part_lse, D.att.n_parts, b * Bt.Hq + h * Bt.G + g, D.out, D.out_lse,
                reinterpret_cast<float*>(smem));
  }
}

// Work items of a launch, in one list per XCD: the units u with u % 8 == x
// form list x, holding their routing items, then their parts, then their
// merges.  Workgroup x + 8 i takes item i of list x (workgroups are handed to
// the XCDs in turn, so list x runs on XCD x and a unit's hand-offs stay in one
// XCD's L2).  Every wait is on an item earlier in the same list, which has a
// smaller workgroup index and so was dispatched first.  Returns the item, or
// -1 for a workgroup past the end of its list.
__host__ __device__ inline int decode_item_of(int wg, int n_units, int routes_per_unit, int parts_per_unit,
                                              int merges_per_unit, int n_route, int n_part_end) {
  const int x = wg % kQueues, i = wg / kQueues;
  const int nx = n_units > x ? (n_units - x + kQueues - 1) / kQueues : 0;
  const int R = routes_per_unit, Pp = parts_per_unit, G = merges_per_unit;
  if (i >= nx * (R + Pp + G)) return -1;
  if (i < R * nx) return (x + kQueues * (i / R)) * R + i % R;
  if (i < (R + Pp) * nx) {
    const int j = i - R * nx;
    return n_route + (x + kQueues * (j / Pp)) * Pp + j % Pp;
  }
  const int j = i - (R + Pp) * nx;
  return n_part_end + (x + kQueues * (j / G)) * G + j % G;
}

// Workgroups of a dkv_decode launch: 8 lists as long as the longest (list 0).
inline int64_t decode_grid(const DecodeArgs& D) {
  const int64_t n0 = (D.n_units + kQueues - 1) / kQueues;
  const int R = D.n_route > 0 ? D.route_items : 0;
  return (int64_t)kQueues * n0 * (R + D.att.items_per_unit + D.merges);
}

template <int NRQ, int QK>
__global__ __launch_bounds__(kAttThreads, 2) void k_decode(PoolArgs P, BatchArgs Bt, DecodeArgs D) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ RouteShared<kAttWaves> rsh;
  __shared__ uint32_t sh_flag;
  __shared__ int32_t sh_slot;
  const int tid = threadIdx.x;
  const int t = decode_item_of((int)blockIdx.x, D.n_units, D.n_route > 0 ? D.route_items : 0, D.att.items_per_unit,
                               D.merges, D.n_route, D.n_part_end);
  decode_item<NRQ, QK, true>(P, Bt, D, t, smem, rsh, sh_slot);
  // The last merge to finish resets the control area for the next launch:
  // merges start only after all of their unit's parts are stored, and every
  // part only after its unit's score words are all written; it waits (bounded)
  // for the count of finished score items, so that none writes a word after
  // the words are cleared.
  if (t >= D.n_part_end) {
    __syncthreads();
    if (tid == 0) sh_flag = (atomicAdd(&D.ctrl[1], 1u) == (uint32_t)(D.n_items - D.n_part_end - 1)) ? 1u : 0u;
    lds_barrier();
    if (sh_flag) {
      if (tid == 0) {
        unsigned n = 0;
        while (ld_dev(&D.ctrl[kCtrlScored]) < (uint32_t)D.n_route && n < kRouteWaitLimit) {
          __builtin_amdgcn_s_sleep(2);
          ++n;
        }
        if (ld_dev(&D.ctrl[kCtrlScored]) < (uint32_t)D.n_route) atomicOr(&D.ctrl[2], 1u);
      }
      __syncthreads();
      if (D.rwords) {
        uint4* w = reinterpret_cast<uint4*>(D.rwords);
        const int64_t n16 = (int64_t)D.n_units * Bt.mb / 2;
        for (int64_t i = tid; i < n16; i += kAttThreads) w[i] = make_uint4(0u, 0u, 0u, 0u);
        if (tid == 0 && ((int64_t)D.n_units * Bt.mb) & 1) D.rwords[(int64_t)D.n_units * Bt.mb - 1] = 0ull;
      }
      for (int i = tid; i < D.n_units; i += kAttThreads) D.unit_done[i * kDoneStride] = 0u;
      if (tid == 0) {
        D.ctrl[1] = 0u;
        D.ctrl[kCtrlScored] = 0u;
        D.ctrl[3] = D.ctrl[3] + 1u;  // the next launch's routed-slot tag
      }
    }
  }
}
// attention variants up to it, which keeps register use down).
template <int NMAX, int QK>
__global__ __launch_bounds__(kAttThreads, 2) void k_decode_layers(const LayerArgs* __restrict__ table, LayersArgs L) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ RouteShared<kAttWaves> rsh;
  __shared__ int32_t sh_item, sh_layer, sh_slot;
  __shared__ uint32_t sh_flag;
  const int tid = threadIdx.x;
  // wave 0 takes the ticket: lane 0 does the atomic, the mapping runs on the
  // scalar unit
  if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
    const int x0 = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (kQueues - 1));  // XCC_ID
    const int per_unit = L.routes + L.block_parts + L.win_parts + L.group;
    int item = -1, layer = 0;
    for (int k = 0; k < kQueues && item < 0; ++k) {
      const int x = (x0 + k) & (kQueues - 1);
      const int nx = L.n_units > x ? (L.n_units - x + kQueues - 1) / kQueues : 0;
      const uint32_t size = (uint32_t)(L.n_layers * nx * per_unit);
      if (size == 0u) continue;
      uint32_t i = 0u;
      if (tid == 0) i = atomicAdd(&L.ctrl[kCtrlQueue + x * kQueueStride], 1u);
      i = __builtin_amdgcn_readfirstlane(i);
      if (i >= size) continue;
      layers_item((int)i, x, nx, L, layer, item);
    }
    if (tid == 0) {
      sh_item = item;
      sh_layer = layer;
    }
  }
  lds_barrier();
  // the item and its layer are the same in every lane: keep them, and the
  // layer's arguments, in scalar registers
  const int t = __builtin_amdgcn_readfirstlane(sh_item);
  // read through the constant address space (scalar loads, scalar registers)
  static_assert(sizeof(LayerArgs) % 4 == 0, "LayerArgs is copied as 32-bit words");
  constexpr int kArgWords = (int)(sizeof(LayerArgs) / 4);
  typedef const __attribute__((address_space(4))) uint32_t ConstWord;
  uint32_t words[kArgWords];
  {
    ConstWord* src = (ConstWord*)table + (int64_t)__builtin_amdgcn_readfirstlane(sh_layer) * kArgWords;
#pragma unroll
    for (int k = 0; k < kArgWords; ++k) words[k] = src[k];
  }
  const LayerArgs la = __builtin_bit_cast(LayerArgs, words);
  if (t >= 0) {
    if (la.nrq <= 0 || NMAX == 0)
      decode_item<0, QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
    else if (la.nrq == 1 || NMAX == 1)
      decode_item<(NMAX < 1 ? NMAX : 1), QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
    else if (la.nrq == 2 || NMAX == 2)
      decode_item<(NMAX < 2 ? NMAX : 2), QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
    else if (la.nrq == 3 || NMAX == 3)
      decode_item<(NMAX < 3 ? NMAX : 3), QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
    else if (la.nrq == 4 || NMAX == 4)
      decode_item<(NMAX < 4 ? NMAX : 4), QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
    else
      decode_item<NMAX, QK>(la.P, la.Bt, la.D, t, smem, rsh, sh_slot);
  }
  // The last merge of the launch zeroes every layer's control words and the
  // queue counters: it finishes after every part, and every part after its
  // routing, so no other item still uses them.
  if (t >= la.D.n_part_end) {
    __syncthreads();
    if (tid == 0)
      sh_flag = (atomicAdd(&L.ctrl[1], 1u) == (uint32_t)(L.n_layers * L.n_units * L.group - 1)) ? 1u : 0u;
    lds_barrier();
    if (sh_flag) {
      for (int l = 0; l < L.n_layers; ++l) {
        const DecodeArgs& D = table[l].D;
        for (int i = tid; i < D.n_units; i += kAttThreads) D.unit_done[i * kDoneStride] = 0u;
      }
      if (tid < kQueues) L.ctrl[kCtrlQueue + tid * kQueueStride] = 0u;
      if (tid == 0) {
        L.ctrl[1] = 0u;
        L.ctrl[3] = L.ctrl[3] + 1u;  // the next launch's routed-slot tag
      }
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
  if (P->n_slots > DKV_MAX_SLOTS) return fail(DKV_ERR_UNSUPPORTED, "n_slots %d > %d", P->n_slots, DKV_MAX_SLOTS);
  if (P->resid_format != DKV_RESID_FP16 && P->resid_format != DKV_RESID_INT8 && P->resid_format != DKV_RESID_INT4)
    return fail(DKV_ERR_INVALID_ARG, "resid_format %d unknown", P->resid_format);
  if (P->rope_freq) {
    if (!P->slot_pos) return fail(DKV_ERR_INVALID_ARG, "un-rotated pool (rope_freq set) without slot_pos");
    if (!al(P->rope_freq, 16) || !al(P->slot_pos, 4))
      return fail(DKV_ERR_UNSUPPORTED, "rope_freq must be 16-byte and slot_pos 4-byte aligned");
  }
  if (P->basis_of) {
    if (!P->rope_freq) return fail(DKV_ERR_UNSUPPORTED, "a shared basis needs an un-rotated pool (rope_freq)");
    if (P->n_basis < 1) return fail(DKV_ERR_INVALID_ARG, "n_basis %d < 1 with basis_of set", P->n_basis);
    if (!al(P->basis_of, 4)) return fail(DKV_ERR_UNSUPPORTED, "basis_of must be 4-byte aligned");
  }
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
    // exact residual rows of an un-rotated pool are rotated by their position
    if (P->n_resid > 0 && ((which & 1) || P->rope_freq))
      if ((s = check_view(P->resid_pos, "resid_pos", 1, 1))) return s;
  }
  if ((which & 2) && P->n_resid > 0) {
    if (P->resid_format == DKV_RESID_FP16) {
      if ((s = check_view(P->resid_k, "resid_k", 2, 16))) return s;
      if ((s = check_view(P->resid_v, "resid_v", 2, 16))) return s;
    } else {
      if ((s = check_view(P->resid_k, "resid_k", 1, 16))) return s;
      if ((s = check_view(P->resid_v, "resid_v", 1, 16))) return s;
      if ((s = check_view(P->resid_k_sb, "resid_k_sb", 2, 16))) return s;
      if ((s = check_view(P->resid_v_sb, "resid_v_sb", 2, 16))) return s;
    }
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
  if (B->route_keys && !al(B->route_keys, 16))
    return fail(DKV_ERR_UNSUPPORTED, "batch->route_keys must be 16-byte aligned");
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
  a.rfmt = P->resid_format;
  a.rkq = a.rvq = nullptr;
  a.rks = a.rvs = nullptr;
  a.rkq_s = a.rkq_h = a.rvq_s = a.rvq_h = a.rks_s = a.rks_h = a.rvs_s = a.rvs_h = 0;
  if (P->resid_format != DKV_RESID_FP16) {
    a.rk = a.rv = nullptr;
    a.rkq = (const uint8_t*)P->resid_k.ptr; a.rkq_s = P->resid_k.slot_stride; a.rkq_h = P->resid_k.head_stride;
    a.rvq = (const uint8_t*)P->resid_v.ptr; a.rvq_s = P->resid_v.slot_stride; a.rvq_h = P->resid_v.head_stride;
    a.rks = (const f16*)P->resid_k_sb.ptr; a.rks_s = P->resid_k_sb.slot_stride; a.rks_h = P->resid_k_sb.head_stride;
    a.rvs = (const f16*)P->resid_v_sb.ptr; a.rvs_s = P->resid_v_sb.slot_stride; a.rvs_h = P->resid_v_sb.head_stride;
  }
  a.rope = P->rope_freq;
  a.spos = P->rope_freq ? P->slot_pos : nullptr;
  a.basis = P->rope_freq ? P->basis_of : nullptr;
  a.n_basis = P->n_basis;
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
  a.rkeys = B->route_keys;
  return a;
}

dkv_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DKV_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DKV_OK;
}

int rq_of(int rank) { return ((rank + 1 + 15) / 16) * 16; }

// routing scratch: an ordered score key and a pool slot per logical block
size_t route_lds_bytes(int max_blocks, int nw) { return route_lds_words(max_blocks, nw) * sizeof(uint32_t); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

dkv_status launch_route(const dkv_pool* P, const dkv_batch* B, int top_k, int32_t* idx, float* scores,
                        int32_t* slots, hipStream_t st) {
  const int units = B->batch * P->n_kv_heads;
  if (units == 0) return DKV_OK;
  const size_t shm = route_lds_bytes(B->max_blocks, kRouteThreads / 64);
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

template <int NRQ, int QK>
dkv_status launch_decode_nrq_q(size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B,
                               const DecodeArgs& D) {
  static bool attr_set = false;
  if (!attr_set) {
    // 160 KB of LDS per workgroup on gfx950, less this kernel's static shared memory
    if (hipFuncSetAttribute((const void*)k_decode<NRQ, QK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            158 * 1024) != hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_decode) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL((k_decode<NRQ, QK>), dim3((unsigned)decode_grid(D)), dim3(kAttThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), D);
  return launched("k_decode");
}

template <int NRQ>
dkv_status launch_decode_nrq(size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B, const DecodeArgs& D) {
  if (P->rope_freq)
    return P->resid_format == DKV_RESID_FP16 ? launch_decode_nrq_q<NRQ, 2>(shm, st, P, B, D)
                                             : launch_decode_nrq_q<NRQ, 3>(shm, st, P, B, D);
  return P->resid_format == DKV_RESID_FP16 ? launch_decode_nrq_q<NRQ, 0>(shm, st, P, B, D)
                                           : launch_decode_nrq_q<NRQ, 1>(shm, st, P, B, D);
}

template <int NRQ, int QK>
dkv_status launch_attend_nrq_q(int64_t items, size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B,
                               const AttnArgs& a) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_attend<NRQ, QK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024) != hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_attend) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL((k_attend<NRQ, QK>), dim3((unsigned)items), dim3(kAttThreads), shm, st, make_pool_args(P),
                     make_batch_args(P, B), a);
  return launched("k_attend");
}

template <int NRQ>
dkv_status launch_attend_nrq(int64_t items, size_t shm, hipStream_t st, const dkv_pool* P, const dkv_batch* B,
                             const AttnArgs& a) {
  if (P->rope_freq)
    return P->resid_format == DKV_RESID_FP16 ? launch_attend_nrq_q<NRQ, 2>(items, shm, st, P, B, a)
                                             : launch_attend_nrq_q<NRQ, 3>(items, shm, st, P, B, a);
  return P->resid_format == DKV_RESID_FP16 ? launch_attend_nrq_q<NRQ, 0>(items, shm, st, P, B, a)
                                           : launch_attend_nrq_q<NRQ, 1>(items, shm, st, P, B, a);
}

dkv_status launch_attend(const dkv_pool* P, const dkv_batch* B, const int32_t* idx,
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
  a.win_tile_stride = 0;
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
  hipLaunchKernelGGL(k_merge, dim3((unsigned)n_rows), dim3(kMergeThreads), 0, st, part_o, part_lse, n_parts,
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
  size_t ctrl_bytes, unit_done, slots, rwords, idx, part_lse, part_o, total;
};

// fold: the window's tiles are shared out over the routed-block parts (else
// the window has parts of its own, of kWinChunk rows).  Un-rotated pools never
// fold: their block parts then start with empty output accumulators, which
// keeps the registers the rotation needs free.
//
// Parts per unit reserved in a decode workspace: enough for the fused launch
// with the window folded or not.
size_t reserved_parts(const dkv_pool* pool, const dkv_batch* batch, int top_k, bool fold) {
  fold = fold && !pool->rope_freq;
  return (top_k > 0 && fold) ? (size_t)top_k : (size_t)top_k + (size_t)decode_win_parts(batch->window);
}

bool al_view(const dkv_view& v, int esz, int a) {
  return al(v.ptr, a) && (v.slot_stride * esz) % a == 0 && (v.head_stride * esz) % a == 0;
}

// The streaming launch (dkv_stream.hip) takes pools of rotated keys with
// residual rows in any format, ranks that are multiples of 8 up to 56,
// residual counts that are multiples of 4, 16-byte aligned row, code and
// (scale, bias) arrays and 4-byte aligned positions.  DKV_STREAM=0 in the
// environment selects the classic launch.
bool stream_eligible(const dkv_pool* P, const dkv_batch* B) {
  static const int enabled = [] {
    const char* e = getenv("DKV_STREAM");
    return (e && e[0] == '0') ? 0 : 1;
  }();
  if (!enabled || P->rope_freq || P->basis_of) return false;
  if (P->rank % 8 != 0 || P->rank > 56 || P->n_resid % 4 != 0) return false;
  if (!al_view(P->anchor_k, 2, 16) || !al_view(P->anchor_v, 2, 16) || !al_view(P->u, 2, 16) ||
      !al_view(P->vk, 2, 16) || !al_view(P->vv, 2, 16))
    return false;
  if (P->n_resid > 0) {
    if (!al_view(P->resid_pos, 1, 4)) return false;
    if (P->resid_format == DKV_RESID_FP16) {
      if (!al_view(P->resid_k, 2, 16) || !al_view(P->resid_v, 2, 16)) return false;
    } else if (P->resid_format == DKV_RESID_INT8 || P->resid_format == DKV_RESID_INT4) {
      if (!al_view(P->resid_k, 1, 16) || !al_view(P->resid_v, 1, 16) || !al_view(P->resid_k_sb, 2, 16) ||
          !al_view(P->resid_v_sb, 2, 16))
        return false;
    } else {
      return false;
    }
  }
  return al(B->q, 16) && al(B->win_k, 16) && al(B->win_v, 16);
}

// min_parts: at least this many parts per unit (the layer-batched streams' schedule)
WsLayout decode_layout(const dkv_pool* pool, const dkv_batch* batch, int top_k, bool fold = true,
                       size_t min_parts = 0) {
  WsLayout w;
  const size_t B = (size_t)batch->batch;
  const size_t units = B * (size_t)pool->n_kv_heads;
  size_t n_parts = reserved_parts(pool, batch, top_k, fold);
  if (min_parts > n_parts) n_parts = min_parts;
  const size_t rows = B * (size_t)batch->n_q_heads;
  w.unit_done = kCtrlHeaderBytes;
  w.slots = w.unit_done + align256(units * 4 * kDoneStride);
  w.rwords = w.slots + align256(units * (size_t)top_k * 4);
  const size_t mb = top_k > 0 && batch->max_blocks > 0 ? (size_t)batch->max_blocks : 0;
  w.ctrl_bytes = w.rwords + align256(units * mb * 8);
  w.idx = w.ctrl_bytes;
  w.part_lse = w.idx + align256(units * (size_t)top_k * 4);
  w.part_o = w.part_lse + align256(rows * n_parts * 4);
  w.total = w.part_o + align256(rows * n_parts * kD * 4);
  return w;
}

// Arguments of one layer's fused decode over the workspace region ws (laid out
// by decode_layout); ctrl: the control header the launch uses.
dkv_status build_decode_args(const dkv_pool* pool, const dkv_batch* batch, int top_k, float scale, unsigned char* ws,
                             uint32_t* ctrl, void* out, float* out_lse, int32_t* out_idx, DecodeArgs& D, size_t& shm,
                             bool fold = true, bool row_merges = true, size_t min_parts = 0,
                             bool split_routing = false) {
  const WsLayout w = decode_layout(pool, batch, top_k, fold, min_parts);
  // folded, each routed-block part also takes its share of the window;
  // otherwise the window comes in chunks of kWinChunk rows
  fold = fold && top_k > 0 && !pool->rope_freq;
  const int n_block = top_k;
  const int n_win = fold ? 0 : decode_win_parts(batch->window);
  const int n_parts = n_block + n_win;
  const int units = batch->batch * pool->n_kv_heads;
  AttnArgs& a = D.att;
  a.idx = nullptr;
  a.top_k = top_k;
  a.n_block_parts = n_block;
  a.block_mode = 3;
  a.n_win_parts = n_win;
  a.win_chunk = kWinChunk;
  a.win_tile_stride = fold ? top_k : 0;
  a.items_per_unit = n_parts;
  a.rq = top_k > 0 ? rq_of(pool->rank) : 0;
  a.scale = scale;
  a.part_o = (float*)(ws + w.part_o);
  a.part_lse = (float*)(ws + w.part_lse);
  a.n_parts = n_parts;
  a.part_offset = 0;
  D.idx = out_idx ? out_idx : (int32_t*)(ws + w.idx);
  D.slots = (int32_t*)(ws + w.slots);
  D.ctrl = ctrl;
  D.unit_done = (uint32_t*)(ws + w.unit_done);
  D.out = (f16*)out;
  D.out_lse = out_lse;
  D.n_units = units;
  // split routing (dkv_decode): ceil(max_blocks / kScoreChunk) score items per
  // unit, each scoring kScoreChunk blocks; else one routing item per unit
  D.rwords = (split_routing && top_k > 0) ? (uint64_t*)(ws + w.rwords) : nullptr;
  D.route_items = D.rwords ? (batch->max_blocks > kScoreChunk ? (batch->max_blocks + kScoreChunk - 1) / kScoreChunk : 1)
                           : 1;
  D.n_route = top_k > 0 ? units * D.route_items : 0;
  const int64_t part_end = (int64_t)D.n_route + (int64_t)units * n_parts;
  // row_merges (one launch per layer, whose merges end the launch): a merge
  // workgroup per query row; otherwise (several layers in one launch, where
  // merges overlap other layers' parts) one per unit
  D.merges = row_merges ? batch->n_q_heads / pool->n_kv_heads : 1;
  const int64_t items = part_end + (int64_t)units * D.merges;
  if (items > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many work items (%lld)", (long long)items);
  D.n_part_end = (int)part_end;
  D.n_items = (int)items;
  shm = (size_t)att_lds_bytes(a.rq);
  const size_t route_shm = route_lds_bytes(batch->max_blocks, kAttWaves);
  if (top_k > 0 && route_shm > shm) shm = route_shm;
  return DKV_OK;
}

}  // namespace

// Error reporting for the library's other translation unit (the block sealer):
// the same thread-local message that dkv_last_error() returns.
__attribute__((visibility("hidden"))) dkv_status dkv_fail_message(dkv_status s, const char* msg) {
  return fail(s, "%s", msg);
}
__attribute__((visibility("hidden"))) void dkv_clear_error_message() { g_err[0] = 0; }

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

// Scratch of dkv_decode_noalloc: the decode workspace of callers that cannot
// allocate, in a fixed device array (each GPU holds its own copy for the life
// of the process).  Host code must not use the array's name as a device
// address: its address on a device comes from hipGetSymbolAddress, taken once
// per device with that device current and kept here.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

static dkv_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DKV_ERR_HIP, "hipGetDevice failed or device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DKV_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DKV_OK;
}

template <int NMAX, int QK>
static dkv_status launch_layers_q(const dkv_layers_plan* plan, const LayersArgs& L, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_decode_layers<NMAX, QK>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            158 * 1024) != hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_decode_layers) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL((k_decode_layers<NMAX, QK>), dim3((unsigned)plan->n_items), dim3(kAttThreads),
                     (size_t)plan->lds_bytes, st, (const LayerArgs*)plan->table, L);
  return launched("k_decode_layers");
}

template <int NMAX>
static dkv_status launch_layers(const dkv_layers_plan* plan, const LayersArgs& L, hipStream_t st) {
  if (plan->unrotated) return plan->quantised ? launch_layers_q<NMAX, 3>(plan, L, st) : launch_layers_q<NMAX, 2>(plan, L, st);
  return plan->quantised ? launch_layers_q<NMAX, 1>(plan, L, st) : launch_layers_q<NMAX, 0>(plan, L, st);
}

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
  if (pool->rope_freq) {
    hipLaunchKernelGGL(k_route_keys_rot, dim3((unsigned)n), dim3(128), 0, (hipStream_t)stream,
                       make_pool_args(pool), slots);
    return launched("k_route_keys_rot");
  }
  hipLaunchKernelGGL(k_route_keys, dim3((unsigned)n), dim3(128), 0, (hipStream_t)stream,
                     make_pool_args(pool), slots);
  return launched("k_route_keys");
}

dkv_status dkv_rope_freqs(double base, int32_t head_dim, float* out) {
  g_err[0] = 0;
  if (!out) return fail(DKV_ERR_INVALID_ARG, "out is NULL");
  if (head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", head_dim);
  if (!(base > 1.0) || !isfinite(base)) return fail(DKV_ERR_INVALID_ARG, "rope base must be finite and > 1");
  const int half = head_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int j = 0; j < half; ++j) {
    const double f = pow(base, -2.0 * j / head_dim) / two_pi;
    const float hi = (float)f;
    out[j] = hi;
    out[half + j] = (float)(f - (double)hi);
  }
  return DKV_OK;
}

dkv_status dkv_gather_route_keys(const dkv_pool* pool, const dkv_batch* batch, float* out, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if ((s = check_batch(pool, batch, true, false))) return s;
  const int64_t n = (int64_t)batch->batch * pool->n_kv_heads * batch->max_blocks * (DKV_HEAD_DIM / 4);
  if (n == 0) return DKV_OK;
  if (!out) return fail(DKV_ERR_INVALID_ARG, "out is NULL");
  if (!al(out, 16)) return fail(DKV_ERR_UNSUPPORTED, "out must be 16-byte aligned");
  if ((s = check_pool_arrays(pool, 4))) return s;
  if ((n + 255) / 256 > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "routing-key table too large");
  hipLaunchKernelGGL(k_gather_route_keys, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     make_pool_args(pool), make_batch_args(pool, batch), out);
  return launched("k_gather_route_keys");
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
  if (batch->max_blocks > 0 && !batch->route_keys && (s = check_pool_arrays(pool, 4))) return s;
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
  return launch_attend(pool, batch, idx, top_k, top_k, 1, 0, kWinChunk, scale, part_o, part_lse,
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
  return launch_attend(pool, batch, idx, top_k, top_k, 2, window_splits, chunk > 0 ? chunk : 1, scale,
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
  if (top_k > 0 && (s = check_pool_arrays(pool, 1 | 2 | (batch->route_keys ? 0 : 4)))) return s;

  const hipStream_t st = (hipStream_t)stream;
  DecodeArgs D;
  size_t shm = 0;
  if ((s = build_decode_args(pool, batch, top_k, scale, (unsigned char*)workspace, (uint32_t*)workspace, out, out_lse,
                             out_idx, D, shm, true, true, 0, true)))
    return s;
  const AttnArgs& a = D.att;

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

dkv_status dkv_decode_noalloc(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale, void* out,
                              float* out_lse, int32_t* out_idx, void* stream) {
  g_err[0] = 0;
  dkv_status s;
  if ((s = check_pool_shape(pool))) return s;
  if (top_k < 0) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if ((s = check_batch(pool, batch, top_k > 0, true))) return s;
  const size_t need = dkv_decode_workspace_size(pool, batch, top_k);
  if (need > kScratchBytes)
    return fail(DKV_ERR_WORKSPACE, "this decode needs %zu bytes of scratch; dkv_decode_noalloc holds %zu (use dkv_decode "
                "with a workspace)", need, kScratchBytes);
  if (batch->batch == 0) return DKV_OK;
  void* ws = nullptr;
  if ((s = scratch_address(&ws))) return s;
  // the control area starts at zero for this call, whatever an earlier call left
  const WsLayout w = decode_layout(pool, batch, top_k);
  const int words = (int)(w.ctrl_bytes / 4);
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)ws, words);
  if ((s = launched("k_zero_words"))) return s;
  return decode_impl(pool, batch, top_k, scale, ws, kScratchBytes, out, out_lse, out_idx, nullptr, stream);
}

size_t dkv_decode_noalloc_max_bytes(void) { return kScratchBytes; }

// ---- layer-batched decode -------------------------------------------------

size_t dkv_decode_layers_table_size(int32_t n_layers) {
  return n_layers > 0 ? (size_t)n_layers * sizeof(LayerArgs) : 0;
}

// the layer-batched launch gives the window parts of their own: with many
// layers in flight no part waits long for its routing, and a part then has
// one load phase rather than two
constexpr bool kLayersFoldWindow = false;

// Streams of the layer-batched streaming launches: at most this many one-wave
// workgroups (eight per CU of the MI355X's 256).
constexpr int kStreamMaxWaves = 2048;
// Work items of the streams: a unit's window rows in items of at most
// kStreamWinRows rows, each routed block's low-rank part, and its residual rows
// (one item); the schedule splits window and residual items where a wave's
// share ends (at most once per wave boundary).
constexpr int kStreamWinRows = 1024;

static bool layers_stream(const dkv_pool* pools, const dkv_batch* batches, int n_layers, int top_k) {
  if (top_k < 1) return false;
  for (int l = 0; l < n_layers; ++l)
    if (!stream_eligible(&pools[l], &batches[l])) return false;
  return true;
}

// The streams' schedule: every unit's work items in order (layer, batch row,
// kv head; its window items, then per routed rank the block's low-rank item
// and its residual item), cut into n_waves contiguous segments of about equal
// cost.  A window or residual item that a segment's end falls inside is split
// there, at a page boundary (16 fp16 rows, 32 rows of codes); a low-rank item
// is not split: when one would straddle the end, the block's residual item
// goes first and is split instead, else the low-rank item stays with the
// segment if it holds the item's middle.  Each segment's end is recomputed as
// the walk goes (the remaining cost over the remaining waves), so that the
// last segment gets its share.  A wave's consecutive items of one unit form a
// run: one attention state, one partial.
struct StreamSchedule {
  std::vector<int32_t> words;        // [n_waves + 1] item offsets, four words per item, parts per (layer, unit)
  int n_waves = 0;
  int64_t n_items = 0;
  std::vector<int32_t> layer_parts;  // per layer: the most partials a unit of it has
};

// fewest cost units per wave (about four K/V page pairs), so that small steps
// run on fewer, fuller waves
constexpr int64_t kStreamMinShare = 15000;

// false when the shapes exceed the schedule's word formats (or the layers'
// unit counts differ)
static bool build_stream_schedule(const dkv_pool* pools, const dkv_batch* batches, int n_layers, int top_k,
                                  StreamSchedule& S) {
  const dkv_pool& p0 = pools[0];
  const dkv_batch& b0 = batches[0];
  const int64_t units = (int64_t)b0.batch * p0.n_kv_heads;
  if (n_layers > 0xFFFF || top_k > 0xFFFF || b0.batch > 0xFFFF || p0.n_kv_heads > 0xFFFF || units < 0)
    return false;
  int64_t n_base = 0;
  for (int l = 0; l < n_layers; ++l) {
    if ((int64_t)batches[l].batch * pools[l].n_kv_heads != units || batches[l].window < 0 ||
        batches[l].window > 0x7FFFFFFF - kStreamWinRows)
      return false;
    const int64_t nwin = (batches[l].window + kStreamWinRows - 1) / kStreamWinRows;
    n_base += units * (nwin + (int64_t)top_k * (1 + (pools[l].n_resid > 0 ? 1 : 0)));
  }
  if (n_base > 0x3FFFFFFF - kStreamMaxWaves) return false;
  struct Item {
    uint32_t w[4];
    int64_t cost;   // the whole item's, its entry (and run start) included
    int32_t unit;   // layer * units + unit
    int32_t pairs;  // splittable items: their K/V page pairs (0: not splittable)
    int32_t rpp;    // rows per pair
    int64_t pair;   // cost per pair
  };
  // An item's cost, in stream clock cycles (fitted to the streams' measured
  // wave durations per page kind): a fixed cost per page (kPage: a memory
  // latency over the ring depth and an issue slot) plus its own arithmetic --
  // a K page's scores and softmax, a V page's products, a V_K or V_V page's
  // tile (the first V_K page also builds the position mask and q . a_k), a U
  // page by how many 32-position groups it holds (4, 2, 1 for ranks up to 16,
  // 32, 64) and its 16-wide rank tiles, a quantised K or V page's 32 rows --
  // plus the entry into each item and the start of each unit's run.
  const int64_t kPage = 1500, kK = 500, kV = 110, kVK = 650, kVK0 = 700, kVV = 700;
  const int64_t kU[5] = {0, 1311, 1070, 0, 4630}, kUTile = 250;
  const int64_t kQK8 = 700, kQV8 = 564, kQK4 = 1100, kQV4 = 818;
  const int64_t kItemEntry = 3790, kRunStart = 1100;
  std::vector<Item> items;
  items.reserve((size_t)n_base);
  for (int l = 0; l < n_layers; ++l) {
    const int r = pools[l].rank, R = pools[l].n_resid, W = batches[l].window, fmt = pools[l].resid_format;
    const int nq = (r + 15) / 16, mu = r <= 16 ? 4 : (r <= 32 ? 2 : 1), nu = 8 / mu;
    const int nq_min = mu == 4 ? 1 : (mu == 2 ? 2 : 3);
    const int64_t u_page = kPage + kU[mu] + (nq > nq_min ? nq - nq_min : 0) * kUTile;
    const int64_t lowrank = kItemEntry + nq * (2 * kPage + kVK + kVV) + kVK0 + nu * u_page;
    const int64_t kv_pair = 2 * kPage + kK + kV;
    // (a 4-bit tile is one page: both sides' codes and pairs)
    const int64_t res_pair = fmt == DKV_RESID_INT8 ? 2 * kPage + kQK8 + kQV8
                           : fmt == DKV_RESID_INT4 ? kPage + kQK4 + kQV4 : kv_pair;
    const int res_rpp = fmt == DKV_RESID_FP16 ? 16 : 32;
    for (int64_t u = 0; u < units; ++u) {
      const uint32_t bh = (uint32_t)(u / p0.n_kv_heads) | ((uint32_t)(u % p0.n_kv_heads) << 16);
      const int32_t ug = (int32_t)(l * units + u);
      const size_t first = items.size();
      for (int r0 = 0; r0 < W; r0 += kStreamWinRows) {
        const int rows = W - r0 < kStreamWinRows ? W - r0 : kStreamWinRows;
        const int pairs = (rows + 15) / 16;
        items.push_back({{(uint32_t)l | (kItemWin << 16), (uint32_t)r0, bh, (uint32_t)rows << 16},
                         kItemEntry + pairs * kv_pair, ug, pairs, 16, kv_pair});
      }
      for (int k = 0; k < top_k; ++k) {
        items.push_back({{(uint32_t)l | (kItemLowRank << 16), (uint32_t)k, bh, 0u}, lowrank, ug, 0, 0, 0});
        if (R > 0) {
          const int pairs = (R + res_rpp - 1) / res_rpp;
          items.push_back({{(uint32_t)l | (kItemResid << 16), (uint32_t)k, bh, (uint32_t)R << 16},
                           kItemEntry + pairs * res_pair, ug, pairs, res_rpp, res_pair});
        }
      }
      if (items.size() > first) items[first].cost += kRunStart;
    }
  }
  double base = 0.0;
  for (const Item& it : items) base += (double)it.cost;
  const int64_t want = (int64_t)std::ceil(base / (double)kStreamMinShare);
  const int n_waves = (int)std::max<int64_t>(1, std::min<int64_t>(kStreamMaxWaves, want));
  // the walk: cum is the cost emitted so far, w the wave being filled, end its
  // end (the remaining cost, the expected splits' entries included, over the
  // remaining waves)
  std::vector<Item> cut;
  std::vector<int32_t> wave_of;
  cut.reserve(items.size() + (size_t)n_waves);
  wave_of.reserve(items.size() + (size_t)n_waves);
  double cum = 0.0;
  int w = 0;
  int64_t splits = 0;
  auto end_of = [&](int wave, double c) {
    if (wave + 1 >= n_waves) return (double)INFINITY;
    const int rem = n_waves - wave;
    const double rate = wave > 0 ? std::min(1.0, (double)splits / wave) : 0.5;
    const double est = base + (double)splits * kItemEntry + rate * (rem - 1) * kItemEntry;
    return c + (est - c) / rem;
  };
  double end = end_of(0, 0.0);
  bool empty = true;  // nothing in wave w's segment yet: it takes at least one item (or page pair)
  auto advance = [&]() {
    if (w + 1 < n_waves) ++w;
    end = end_of(w, cum);
    empty = true;
  };
  auto emit = [&](const Item& it) {
    cut.push_back(it);
    wave_of.push_back(w);
    cum += (double)it.cost;
    empty = false;
  };
  for (size_t i = 0; i < items.size(); ++i) {
    for (;;) {
      Item& it = items[i];
      if (cum + (double)it.cost <= end) {
        emit(it);
        break;
      }
      if (it.pairs <= 1) {
        if (i + 1 < items.size() && items[i + 1].pairs > 1 && items[i + 1].unit == it.unit &&
            cum + (double)items[i + 1].cost > end) {
          // the block's residual item fills the segment; the low-rank item follows
          std::swap(items[i], items[i + 1]);
          continue;
        }
        if (empty || cum + 0.5 * (double)it.cost <= end) {
          emit(it);
          advance();
          break;
        }
        advance();
        continue;
      }
      // the pairs that fit before the segment's end stay in wave w
      const int64_t fixed = it.cost - (int64_t)it.pairs * it.pair;  // the entry (and run start)
      int m = (int)std::lround((end - cum - (double)fixed) / (double)it.pair);
      if (empty && m < 1) m = 1;
      if (m >= it.pairs) {
        emit(it);
        break;
      }
      if (m <= 0) {
        advance();
        continue;
      }
      Item a = it;
      const int rows_a = m * it.rpp;
      const int rows_all = (int)(it.w[3] >> 16);
      a.w[3] = (uint32_t)rows_a << 16;
      a.pairs = m;
      a.cost = fixed + (int64_t)m * it.pair;
      emit(a);
      ++splits;
      // the rest, from the row after the first part's, in the next wave
      if ((it.w[0] >> 16) == (uint32_t)kItemWin)
        it.w[1] += (uint32_t)rows_a;
      else
        it.w[1] += (uint32_t)rows_a << 16;
      it.w[3] = (uint32_t)(rows_all - rows_a) << 16;
      it.pairs -= m;
      it.cost = kItemEntry + (int64_t)it.pairs * it.pair;
      advance();
    }
  }
  // runs: the flags, each run's partial index within its unit, the units' counts
  std::vector<int32_t> unit_parts((size_t)(n_layers * units), 0);
  for (size_t i = 0; i < cut.size(); ++i) {
    const bool first = i == 0 || wave_of[i - 1] != wave_of[i] || cut[i - 1].unit != cut[i].unit;
    const bool last = i + 1 == cut.size() || wave_of[i + 1] != wave_of[i] || cut[i + 1].unit != cut[i].unit;
    if (first) ++unit_parts[(size_t)cut[i].unit];
    const int part = unit_parts[(size_t)cut[i].unit] - 1;
    cut[i].w[0] |= (first ? 1u << 24 : 0u) | (last ? 2u << 24 : 0u);
    cut[i].w[3] |= (uint32_t)part;
  }
  S.n_waves = n_waves;
  S.n_items = (int64_t)cut.size();
  S.layer_parts.assign((size_t)n_layers, 1);
  for (int l = 0; l < n_layers; ++l)
    for (int64_t u = 0; u < units; ++u)
      S.layer_parts[(size_t)l] = std::max(S.layer_parts[(size_t)l], unit_parts[(size_t)(l * units + u)]);
  S.words.clear();
  S.words.reserve((size_t)n_waves + 1 + 4 * cut.size() + unit_parts.size());
  size_t i = 0;
  for (int wv = 0; wv < n_waves; ++wv) {
    S.words.push_back((int32_t)i);
    while (i < cut.size() && wave_of[i] == wv) ++i;
  }
  S.words.push_back((int32_t)i);
  for (const Item& it : cut)
    for (int k = 0; k < 4; ++k) S.words.push_back((int32_t)it.w[k]);
  S.words.insert(S.words.end(), unit_parts.begin(), unit_parts.end());
  return true;
}

static size_t layer_region_bytes(const dkv_pool* pool, const dkv_batch* batch, int top_k, size_t min_parts) {
  return align256(decode_layout(pool, batch, top_k, kLayersFoldWindow, min_parts).total);
}

size_t dkv_decode_layers_workspace_size(const dkv_pool* pools, const dkv_batch* batches, int32_t n_layers,
                                        int32_t top_k) {
  if (!pools || !batches || n_layers < 1 || top_k < 0) return 0;
  StreamSchedule S;
  const bool streams = layers_stream(pools, batches, n_layers, top_k) &&
                       build_stream_schedule(pools, batches, n_layers, top_k, S);
  size_t total = kCtrlHeaderBytes;
  for (int l = 0; l < n_layers; ++l)
    total += layer_region_bytes(&pools[l], &batches[l], top_k, streams ? (size_t)S.layer_parts[(size_t)l] : 0);
  if (streams) total += align256(S.words.size() * 4);
  return total;
}

dkv_status dkv_decode_layers_prepare(const dkv_pool* pools, const dkv_batch* batches, int32_t n_layers,
                                     int32_t top_k, float scale, void* const* outs, float* const* out_lses,
                                     int32_t* const* out_idxs, void* table, size_t table_bytes,
                                     void* workspace, size_t workspace_bytes, dkv_layers_plan* plan) {
  g_err[0] = 0;
  if (!pools || !batches || !plan) return fail(DKV_ERR_INVALID_ARG, "pools / batches / plan is NULL");
  if (n_layers < 1) return fail(DKV_ERR_INVALID_ARG, "n_layers %d < 1", n_layers);
  if (top_k < 0) return fail(DKV_ERR_INVALID_ARG, "top_k %d < 0", top_k);
  if (!outs || !out_lses) return fail(DKV_ERR_INVALID_ARG, "outs / out_lses is NULL");
  if (!table || table_bytes < dkv_decode_layers_table_size(n_layers))
    return fail(DKV_ERR_WORKSPACE, "table of %zu bytes given, %zu needed", table ? table_bytes : 0,
                dkv_decode_layers_table_size(n_layers));
  if (!al(table, 16)) return fail(DKV_ERR_WORKSPACE, "table must be 16-byte aligned");
  const size_t need = dkv_decode_layers_workspace_size(pools, batches, n_layers, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(DKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if (!al(workspace, 256)) return fail(DKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const dkv_pool& p0 = pools[0];
  const dkv_batch& b0 = batches[0];
  LayerArgs* host = (LayerArgs*)calloc((size_t)n_layers, sizeof(LayerArgs));
  if (!host) return fail(DKV_ERR_HIP, "out of host memory");
  dkv_status s = DKV_OK;
  size_t shm = 0, off = kCtrlHeaderBytes;
  unsigned char* ws = (unsigned char*)workspace;
  const bool streams = layers_stream(pools, batches, n_layers, top_k);
  StreamSchedule S;
  if (streams && !build_stream_schedule(pools, batches, n_layers, top_k, S)) {
    free(host);
    return fail(DKV_ERR_INVALID_ARG, "the layers' shapes exceed the streams' schedule");
  }
  for (int l = 0; l < n_layers && s == DKV_OK; ++l) {
    const dkv_pool* pool = &pools[l];
    const dkv_batch* batch = &batches[l];
    if ((s = check_pool_shape(pool))) break;
    if ((s = check_batch(pool, batch, top_k > 0, true))) break;
    if (pool->n_kv_heads != p0.n_kv_heads || batch->batch != b0.batch || batch->n_q_heads != b0.n_q_heads ||
        batch->window != b0.window || batch->max_blocks != b0.max_blocks) {
      s = fail(DKV_ERR_INVALID_ARG, "layer %d: batch shape or KV heads differ from layer 0", l);
      break;
    }
    if (top_k > 0 && batch->max_blocks > DKV_MAX_ROUTE_BLOCKS) {
      s = fail(DKV_ERR_UNSUPPORTED, "max_blocks %d > %d", batch->max_blocks, DKV_MAX_ROUTE_BLOCKS);
      break;
    }
    if (b0.batch > 0 && (!outs[l] || !out_lses[l])) {
      s = fail(DKV_ERR_INVALID_ARG, "layer %d: out / out_lse is NULL", l);
      break;
    }
    if (outs[l] && !al(outs[l], 4)) {
      s = fail(DKV_ERR_UNSUPPORTED, "layer %d: out must be 4-byte aligned", l);
      break;
    }
    if (top_k > 0 && b0.batch > 0 && (s = check_pool_arrays(pool, 1 | 2 | (batch->route_keys ? 0 : 4)))) break;
    if ((pool->rope_freq != nullptr) != (p0.rope_freq != nullptr)) {
      s = fail(DKV_ERR_UNSUPPORTED, "layer %d: pools must be all rotated or all un-rotated", l);
      break;
    }
    size_t shm_l = 0;
    const size_t min_parts = streams ? (size_t)S.layer_parts[(size_t)l] : 0;
    if ((s = build_decode_args(pool, batch, top_k, scale, ws + off, (uint32_t*)workspace, outs[l], out_lses[l],
                               out_idxs ? out_idxs[l] : nullptr, host[l].D, shm_l, kLayersFoldWindow,
                               /*row_merges=*/false, min_parts)))
      break;
    host[l].P = make_pool_args(pool);
    host[l].Bt = make_batch_args(pool, batch);
    host[l].nrq = host[l].D.att.rq / 16;
    if (streams) {
      // the routings launch needs only routing LDS; the partials are the
      // streams' runs' (at most one per item of the unit)
      shm_l = route_lds_bytes(batch->max_blocks, kAttWaves);
      DecodeArgs& D = host[l].D;
      D.att.n_block_parts = 0;
      D.att.n_win_parts = 0;
      D.att.items_per_unit = 0;
      D.att.n_parts = (int)min_parts;
      D.merges = 0;
      D.n_part_end = D.n_route;
      D.n_items = D.n_route;
    }
    if (shm_l > shm) shm = shm_l;
    off += layer_region_bytes(pool, batch, top_k, min_parts);
  }
  const std::vector<int32_t>& sched = S.words;
  const int n_waves = S.n_waves;
  const int64_t n_sched = S.n_items;
  const size_t sched_off = align256(off);
  if (s == DKV_OK) {
    if (hipMemcpy(table, host, (size_t)n_layers * sizeof(LayerArgs), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(workspace, 0, need) != hipSuccess ||
        (!sched.empty() && hipMemcpy(ws + sched_off, sched.data(), sched.size() * 4, hipMemcpyHostToDevice) !=
                               hipSuccess) ||
        hipDeviceSynchronize() != hipSuccess)
      s = fail(DKV_ERR_HIP, "table upload or workspace clear failed");
  }
  if (s == DKV_OK) {
    const int units = b0.batch * p0.n_kv_heads;
    plan->n_layers = n_layers;
    plan->n_units = units;
    plan->routes = top_k > 0 ? 1 : 0;
    plan->parts = streams ? 0 : host[0].D.att.n_block_parts;
    plan->win_parts = host[0].D.att.n_win_parts;
    plan->group = streams ? 0 : 1;  // merges per unit (the streams: a launch of their own)
    // the launch's work items (with the streams: the first launch's, the routings)
    const int64_t items = (int64_t)n_layers * units * (plan->routes + plan->parts + plan->win_parts + plan->group);
    if (items > 0x7FFFFFFF) s = fail(DKV_ERR_INVALID_ARG, "too many work items (%lld)", (long long)items);
    plan->n_items = (int32_t)items;
    plan->lds_bytes = (int32_t)shm;
    int nmax = 0;
    for (int l = 0; l < n_layers; ++l) nmax = host[l].nrq > nmax ? host[l].nrq : nmax;
    plan->max_tiles = nmax;
    int quant = 0;
    for (int l = 0; l < n_layers; ++l) quant |= pools[l].resid_format != DKV_RESID_FP16 ? 1 : 0;
    plan->quantised = quant;
    plan->unrotated = p0.rope_freq ? 1 : 0;
    plan->stream = streams ? 1 : 0;
    plan->stream_top_k = streams ? top_k : 0;
    plan->stream_items = (int32_t)n_sched;
    plan->stream_waves = n_waves;
    plan->stream_sched = (int32_t)(sched_off / 4);
    plan->table = table;
    plan->workspace = workspace;
  }
  free(host);
  return s;
}

static dkv_status layers_step(const dkv_layers_plan* plan, void* const* events, void* stream);

dkv_status dkv_decode_layers(const dkv_layers_plan* plan, void* stream) { return layers_step(plan, nullptr, stream); }

dkv_status dkv_decode_layers_profiled(const dkv_layers_plan* plan, void* const* events, void* stream) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3]) {
    g_err[0] = 0;
    return fail(DKV_ERR_INVALID_ARG, "events must hold four hipEvent_t handles");
  }
  return layers_step(plan, events, stream);
}

dkv_status dkv_stream_read_probe(const void* src, size_t bytes, int32_t n_waves, uint32_t* sink, void* stream) {
  g_err[0] = 0;
  if (!src || !sink) return fail(DKV_ERR_INVALID_ARG, "src / sink is NULL");
  if (n_waves < 1 || n_waves > 65536) return fail(DKV_ERR_INVALID_ARG, "n_waves %d out of [1, 65536]", n_waves);
  if (!al(src, 16) || bytes % ((size_t)4096 * n_waves) != 0 || bytes / n_waves > 0xFFFFF000u)
    return fail(DKV_ERR_INVALID_ARG, "bytes %zu must be a multiple of 4096 * n_waves (< 4 GiB per wave), src 16-byte aligned",
                bytes);
  if (bytes == 0) return DKV_OK;
  const hipError_t e = dkv_stream_read_probe_launch(src, bytes / n_waves, n_waves, sink, (hipStream_t)stream);
  return e == hipSuccess ? DKV_OK : fail(DKV_ERR_HIP, "read probe launch failed: %s", hipGetErrorString(e));
}

static dkv_status layers_step(const dkv_layers_plan* plan, void* const* events, void* stream) {
  g_err[0] = 0;
  if (!plan || !plan->table || !plan->workspace) return fail(DKV_ERR_INVALID_ARG, "plan is NULL or not prepared");
  if (plan->n_items == 0 && !plan->stream) {
    for (int k = 0; events && k < 4; ++k)
      if (hipEventRecord((hipEvent_t)events[k], (hipStream_t)stream) != hipSuccess)
        return fail(DKV_ERR_HIP, "hipEventRecord failed");
    return DKV_OK;
  }
  LayersArgs L;
  L.ctrl = (uint32_t*)plan->workspace;
  L.n_layers = plan->n_layers;
  L.n_units = plan->n_units;
  L.routes = plan->routes;
  L.block_parts = plan->parts;
  L.win_parts = plan->win_parts;
  L.group = plan->group;
  const hipStream_t st = (hipStream_t)stream;
  if (events && hipEventRecord((hipEvent_t)events[0], st) != hipSuccess)
    return fail(DKV_ERR_HIP, "hipEventRecord failed");
  dkv_status s = DKV_OK;
  if (plan->stream) {
    const hipError_t e = dkv_stream_step(plan->table, L.ctrl, (size_t)plan->lds_bytes,
                                         (const int32_t*)plan->workspace + plan->stream_sched, plan->stream_waves,
                                         plan->stream_items, plan->stream_top_k, plan->n_layers, plan->n_units,
                                         events, st);
    if (e != hipSuccess) return fail(DKV_ERR_HIP, "streaming launches failed: %s", hipGetErrorString(e));
  } else {
    switch (plan->max_tiles) {  // the largest low-rank tile count of the layers
      case 0: s = launch_layers<0>(plan, L, st); break;
      case 1: s = launch_layers<1>(plan, L, st); break;
      case 2: s = launch_layers<2>(plan, L, st); break;
      case 3: s = launch_layers<3>(plan, L, st); break;
      case 4: s = launch_layers<4>(plan, L, st); break;
      case 5: s = launch_layers<5>(plan, L, st); break;
      default: return fail(DKV_ERR_INVALID_ARG, "plan is corrupt (tile count %d)", plan->max_tiles);
    }
    if (s) return s;
    if (events && (hipEventRecord((hipEvent_t)events[1], st) != hipSuccess ||
                   hipEventRecord((hipEvent_t)events[2], st) != hipSuccess))
      return fail(DKV_ERR_HIP, "hipEventRecord failed");
  }
  if (events && hipEventRecord((hipEvent_t)events[3], st) != hipSuccess)
    return fail(DKV_ERR_HIP, "hipEventRecord failed");
  return DKV_OK;
}

}  // extern "C"
