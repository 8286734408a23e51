// Block sealer of the DKV compressed KV cache on gfx950: the write side.
//
// A 256-token block of one KV head is reduced to its anchor (the first token,
// exact), a rank-r joint K|V delta U (255 x r, singular values folded in),
// V_K, V_V (r x 128), and the R tokens the delta reconstructs worst, kept
// exact (pages: "DKV: Anchor + Low-Rank Differential KV-Cache Compression for
// Scalable Long-Context Inference", Zenodo abstract; Differential-KV README,
// "Core Architecture & Paper Overview" items 1-3, "Content-Aware /
// Rarity-Aware Residual Selection" for the plain L2 selection, "Key
// Environment Knobs" for the seeded randomised SVD).
//
// One workgroup (256 threads) per (block, KV head).  With A = [K[1:] - K[0] |
// V[1:] - V[0]] (255 x 256), the steps of a randomised subspace iteration:
//   Y = A omega, Q = orth(Y); power_iters times Z = orth(A^T Q), Q = orth(A Z);
//   B^T = A^T Q; C = B B^T (width x width) = Z_B^T Z_B; C = E diag(l) E^T by
//   cyclic Jacobi; U S = Q E_r S_r, W_r = B^T E_r S_r^-1, [V_K | V_V] = W_r^T.
// Thread mapping: a row product (Y = A F) gives thread t row t of the result,
// a column product (Z = A^T F) thread c row c; the factor F sits in LDS and
// every thread reads the same row of it at a time (LDS broadcast).  orth() is
// Cholesky QR, twice: the Gram matrix in LDS (4 x 4 register blocks), its
// Cholesky factor by one wave, the triangular solve on each thread's row in
// registers; pivots below 1e-5 of the largest diagonal drop their column (a
// rank-deficient Y spans fewer directions).  All arithmetic is fp32; the
// factors are stored as fp16 (round to nearest even), and the residual errors
// are measured against the reconstruction from those stored factors.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "dkv_attn.h"

#include <vector>

__attribute__((visibility("hidden"))) dkv_status dkv_fail_message(dkv_status s, const char* msg);
__attribute__((visibility("hidden"))) void dkv_clear_error_message();

typedef _Float16 f16;
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

namespace {

constexpr int kD = 128;
constexpr int kRows = 255;          // delta rows: tokens 1..255
constexpr int kThreads = 256;
constexpr int kMaxWidth = 80;       // columns of the test matrix
constexpr int kMaxPowerIters = 8;
constexpr int kMaxSweeps = 24;      // Jacobi sweeps (they stop once no rotation is needed)
constexpr int kOrthPasses = 2;      // Cholesky QR passes per orthonormalisation
constexpr float kDropPivot = 1e-5f; // relative pivot below which a column is dropped
constexpr float kJacobiSkip = 1e-7f;

struct SealArgs {
  const f16* sk; int64_t sk_s, sk_h;
  const f16* sv; int64_t sv_s, sv_h;
  const int32_t* slots;
  int n_heads, n_slots;
  const float* omega; int width;
  int rank, n_resid, power_iters;
  f16* ak; int64_t ak_s, ak_h;
  f16* av; int64_t av_s, av_h;
  f16* u; int64_t u_s, u_h;
  f16* vk; int64_t vk_s, vk_h;
  f16* vv; int64_t vv_s, vv_h;
  f16* rk; int64_t rk_s, rk_h;
  f16* rv; int64_t rv_s, rv_h;
  uint8_t* rp; int64_t rp_s, rp_h;
  int resid_bits;                  // 16 (fp16 rows), or 8 / 4 (codes in rk / rv as bytes, strides in bytes)
  f16* rks; int64_t rks_s, rks_h;  // quantised: (scale, bias) pairs [R][2][2] of the K rows
  f16* rvs; int64_t rvs_s, rvs_h;  // the same for the V rows
};

// One fp16 row (128 dims) into the group-quantised format: per group of 64,
// bias = the smallest value, scale = (largest - smallest) / L in fp32 rounded
// up to fp16 (the grid reaches the largest value), code = round((x - bias) /
// scale) in fp32 with ties to even, clamped to [0, L] (0 for a zero scale).
// codes: 128 bytes (8 bits) or 64 bytes (4 bits, dimension 2j in the low
// nibble of byte j); sb: (scale, bias) of dims 0..63, then 64..127.
__device__ void quantize_row(const f16* x, int bits, uint8_t* codes, f16* sb) {
  const float L = (float)((1 << bits) - 1);
  for (int g = 0; g < 2; ++g) {
    float lo = (float)x[64 * g], hi = lo;
    for (int d = 1; d < 64; ++d) {
      const float v = (float)x[64 * g + d];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    const float s32 = __fdiv_rn(hi - lo, L);
    f16 s16 = (f16)s32;
    if ((float)s16 < s32) s16 = __builtin_bit_cast(f16, (uint16_t)(__builtin_bit_cast(uint16_t, s16) + 1u));
    const f16 b16 = (f16)lo;
    const float sf = (float)s16, bf = (float)b16;
    sb[2 * g] = s16;
    sb[2 * g + 1] = b16;
    for (int d = 0; d < 64; d += 2) {
      uint32_t c[2];
      for (int e = 0; e < 2; ++e) {
        const float q = sf > 0.f ? rintf(__fdiv_rn((float)x[64 * g + d + e] - bf, sf)) : 0.f;
        c[e] = (uint32_t)fminf(fmaxf(q, 0.f), L);
      }
      if (bits == 8) {
        codes[64 * g + d] = (uint8_t)c[0];
        codes[64 * g + d + 1] = (uint8_t)c[1];
      } else {
        codes[32 * g + d / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  }
}

// LDS layout (in 4-byte words) for a padded width LP (a multiple of 8).  E
// shares S's area: E is written from the Jacobi step on, when S's rows are no
// longer read, and it sits at the end of S, past the rounded V_K that the
// right-factor step writes at S's start while it still reads E.
template <int LP>
struct Lay {
  static constexpr int SS = LP + 4;  // row stride of S, G, E: 16-byte aligned rows
  static constexpr int S = 0;                    // [256][SS] the factor of a product / rows for a Gram
  static constexpr int E = S + (256 - LP) * SS;  // [LP][SS] Jacobi eigenvectors (the end of S's area)
  static constexpr int G = S + 256 * SS;         // [LP][SS] Gram, Cholesky factor, Jacobi matrix
  static constexpr int ANC = G + LP * SS;        // [256] anchor row (fp32)
  static constexpr int ERR = ANC + 256;          // [256] squared key errors
  static constexpr int SEL = ERR + 256;          // [256] selected flags
  static constexpr int INV = SEL + 256;          // [LP] inverse Cholesky pivots
  static constexpr int SIG = INV + LP;           // [LP] singular values, descending
  static constexpr int PERM = SIG + LP;          // [LP] eigenvalue order
  static constexpr int RC = PERM + LP;           // [LP / 2] rotation cosines
  static constexpr int RS = RC + LP / 2;         // [LP / 2] rotation sines
  static constexpr int RP = RS + LP / 2;         // [LP / 2] rotation pairs (p)
  static constexpr int RQ = RP + LP / 2;         // [LP / 2] rotation pairs (q)
  static constexpr int FLAG = RQ + LP / 2;       // [4] rotation counters of the sweeps
  static constexpr int WORDS = FLAG + 4;
  static constexpr size_t bytes = (size_t)WORDS * 4;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS operations are done
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// v = A[t] F for row t of A (thread t; row 255 does not exist and gives 0)
template <int LP>
__device__ __forceinline__ void row_product(const f16* xk, const f16* xv, const float* anc, const float* F, int t,
                                            float (&v)[LP]) {
  constexpr int SS = Lay<LP>::SS;
#pragma unroll
  for (int j = 0; j < LP; ++j) v[j] = 0.f;
  if (t >= kRows) return;
  const f16* kr = xk + (int64_t)(t + 1) * kD;
  const f16* vr = xv + (int64_t)(t + 1) * kD;
  constexpr int kAhead = 4;  // 16-byte chunks of the row loaded together
  for (int c0 = 0; c0 < 2 * kD / 8; c0 += kAhead) {
    v8h x[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) {
      const int c8 = c0 + q;
      x[q] = *reinterpret_cast<const v8h*>(c8 < kD / 8 ? kr + 8 * c8 : vr + 8 * (c8 - kD / 8));
    }
#pragma unroll
    for (int q = 0; q < kAhead; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * (c0 + q) + e;
        const float a = (float)x[q][e] - anc[c];
        const float4* fr = reinterpret_cast<const float4*>(F + c * SS);
#pragma unroll
        for (int j4 = 0; j4 < LP / 4; ++j4) {
          const float4 f = fr[j4];
          v[4 * j4 + 0] = fmaf(a, f.x, v[4 * j4 + 0]);
          v[4 * j4 + 1] = fmaf(a, f.y, v[4 * j4 + 1]);
          v[4 * j4 + 2] = fmaf(a, f.z, v[4 * j4 + 2]);
          v[4 * j4 + 3] = fmaf(a, f.w, v[4 * j4 + 3]);
        }
      }
    }
  }
}

// v = (A^T F)[c] = sum_t A[t][c] F[t] for column c of A (thread c)
template <int LP>
__device__ __forceinline__ void col_product(const f16* xk, const f16* xv, const float* anc, const float* F, int c,
                                            float (&v)[LP]) {
  constexpr int SS = Lay<LP>::SS;
#pragma unroll
  for (int j = 0; j < LP; ++j) v[j] = 0.f;
  const f16* col = (c < kD ? xk + c : xv + (c - kD)) + kD;  // row 1 of column c
  const float ac = anc[c];
  constexpr int kAhead = 8;  // rows of the column loaded together
  for (int t0 = 0; t0 < 256; t0 += kAhead) {
    float a[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) {
      const int t = t0 + q < kRows ? t0 + q : kRows - 1;  // row 256 does not exist: read row 255, weight 0
      a[q] = t0 + q < kRows ? (float)col[(int64_t)t * kD] - ac : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kAhead; ++q) {
      const float4* fr = reinterpret_cast<const float4*>(F + (t0 + q) * SS);  // F has 256 rows
#pragma unroll
      for (int j4 = 0; j4 < LP / 4; ++j4) {
        const float4 f = fr[j4];
        v[4 * j4 + 0] = fmaf(a[q], f.x, v[4 * j4 + 0]);
        v[4 * j4 + 1] = fmaf(a[q], f.y, v[4 * j4 + 1]);
        v[4 * j4 + 2] = fmaf(a[q], f.z, v[4 * j4 + 2]);
        v[4 * j4 + 3] = fmaf(a[q], f.w, v[4 * j4 + 3]);
      }
    }
  }
}

template <int LP>
__device__ __forceinline__ void store_row(float* S, int t, const float (&v)[LP]) {
  float4* d = reinterpret_cast<float4*>(S + t * Lay<LP>::SS);
#pragma unroll
  for (int j4 = 0; j4 < LP / 4; ++j4) d[j4] = make_float4(v[4 * j4], v[4 * j4 + 1], v[4 * j4 + 2], v[4 * j4 + 3]);
}

// G = S^T S over the 256 rows of S (both triangles), in 4 x 4 blocks
template <int LP>
__device__ __forceinline__ void gram(const float* S, float* G, int tid) {
  constexpr int SS = Lay<LP>::SS, NB = LP / 4, NP = NB * (NB + 1) / 2;
  if constexpr (NP <= kThreads / 2) {
    // two halves of the rows: threads 128.. sum rows 128..255 and leave their
    // 4 x 4 sum in the block's mirror position; threads 0.. sum rows 0..127,
    // add it and write both triangles
    const int half = tid >= kThreads / 2 ? 1 : 0, e = tid - half * (kThreads / 2);
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
    int bi = 0, bj = 0;
    if (e < NP) {
      while ((bi + 1) * (bi + 2) / 2 <= e) ++bi;
      bj = e - bi * (bi + 1) / 2;
      for (int t = half * 128; t < half * 128 + 128; ++t) {
        const float4 x = *reinterpret_cast<const float4*>(S + t * SS + 4 * bi);
        const float4 y = *reinterpret_cast<const float4*>(S + t * SS + 4 * bj);
        const float xa[4] = {x.x, x.y, x.z, x.w}, yb[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(xa[a], yb[b], acc[a][b]);
      }
      if (half) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) G[(4 * bj + b) * SS + 4 * bi + a] = acc[a][b];
      }
    }
    __syncthreads();
    if (e < NP && !half) {
      float part[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) part[a][b] = G[(4 * bj + b) * SS + 4 * bi + a];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float g = acc[a][b] + part[a][b];
          G[(4 * bi + a) * SS + 4 * bj + b] = g;
          G[(4 * bj + b) * SS + 4 * bi + a] = g;
        }
    }
    return;
  }
  for (int e = tid; e < NP; e += kThreads) {
    int bi = 0;
    while ((bi + 1) * (bi + 2) / 2 <= e) ++bi;
    const int bj = e - bi * (bi + 1) / 2;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
    for (int t = 0; t < 256; ++t) {
      const float4 x = *reinterpret_cast<const float4*>(S + t * SS + 4 * bi);
      const float4 y = *reinterpret_cast<const float4*>(S + t * SS + 4 * bj);
      const float xa[4] = {x.x, x.y, x.z, x.w}, yb[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(xa[a], yb[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        G[(4 * bi + a) * SS + 4 * bj + b] = acc[a][b];
        G[(4 * bj + b) * SS + 4 * bi + a] = acc[a][b];
      }
  }
}

// Cholesky factor of G (one wave): L in G's lower triangle, inv[k] = 1 / L[k][k],
// or 0 for a pivot below kDropPivot of the largest diagonal (its column dropped)
template <int LP>
__device__ __forceinline__ void cholesky(float* G, float* inv, int lane) {
  constexpr int SS = Lay<LP>::SS, R2 = (LP + 63) / 64;
  float mx = 0.f;
  for (int i = lane; i < LP; i += 64) mx = fmaxf(mx, G[i * SS + i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float tol = kDropPivot * mx;
  for (int k = 0; k < LP; ++k) {
    float s[R2];
#pragma unroll
    for (int r2 = 0; r2 < R2; ++r2) {
      const int i = lane + 64 * r2;
      s[r2] = 0.f;
      if (i >= k && i < LP) {
        // sum over m < k of L[i][m] L[k][m]: 16-byte reads, four partial sums
        const float* li = G + i * SS;
        const float* lk = G + k * SS;
        float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
        int m = 0;
        for (; m + 4 <= k; m += 4) {
          const float4 a = *reinterpret_cast<const float4*>(li + m);
          const float4 b = *reinterpret_cast<const float4*>(lk + m);
          acc4.x = fmaf(a.x, b.x, acc4.x);
          acc4.y = fmaf(a.y, b.y, acc4.y);
          acc4.z = fmaf(a.z, b.z, acc4.z);
          acc4.w = fmaf(a.w, b.w, acc4.w);
        }
        float acc = (acc4.x + acc4.y) + (acc4.z + acc4.w);
        for (; m < k; ++m) acc = fmaf(li[m], lk[m], acc);
        s[r2] = G[i * SS + k] - acc;
      }
    }
    const float d = __shfl(k < 64 ? s[0] : s[R2 - 1], k & 63);
    const float lkk = d > tol ? sqrtf(d) : 0.f;
    const float ik = lkk > 0.f ? 1.f / lkk : 0.f;
#pragma unroll
    for (int r2 = 0; r2 < R2; ++r2) {
      const int i = lane + 64 * r2;
      if (i > k && i < LP) G[i * SS + k] = s[r2] * ik;
    }
    if (lane == (k & 63)) {
      G[k * SS + k] = lkk;
      inv[k] = ik;
    }
    wave_sync();
  }
}

// v <- v L^-T (row v of Y becomes row of Q = Y L^-T); dropped columns give 0
template <int LP>
__device__ __forceinline__ void solve_row(const float* G, const float* inv, float (&v)[LP]) {
  constexpr int SS = Lay<LP>::SS;
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    float acc = v[j];
#pragma unroll
    for (int m = 0; m < j; ++m) acc = fmaf(-v[m], G[j * SS + m], acc);
    v[j] = acc * inv[j];
  }
}

// player in a slot of round k of the circle method (n players, n even)
__device__ __forceinline__ int player(int slot, int k, int n) { return slot == 0 ? 0 : 1 + (slot - 1 + k) % (n - 1); }

// C (in G, symmetric LP x LP) = E diag(C) E^T by cyclic Jacobi with the
// rotations of each round (LP / 2 disjoint pairs) applied together
template <int LP>
__device__ __forceinline__ void jacobi(float* G, float* E, float* rc, float* rs, int* rp, int* rq, int* flag,
                                       int tid) {
  constexpr int SS = Lay<LP>::SS, NP = LP / 2;
  for (int e = tid; e < LP * LP; e += kThreads) E[(e / LP) * SS + e % LP] = (e / LP == e % LP) ? 1.f : 0.f;
  if (tid < 4) flag[tid] = 0;
  __syncthreads();
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) flag[(sweep + 1) % 3] = 0;  // the counter of the next sweep (last read two sweeps ago)
    for (int round = 0; round < LP - 1; ++round) {
      if (tid < NP) {
        const int a = player(tid, round, LP), b = player(LP - 1 - tid, round, LP);
        const int p = a < b ? a : b, q = a < b ? b : a;
        const float app = G[p * SS + p], aqq = G[q * SS + q], apq = G[p * SS + q];
        float c = 1.f, s = 0.f;
        if (fabsf(apq) > kJacobiSkip * sqrtf(fabsf(app * aqq)) + 1e-30f) {
          const float tau = (aqq - app) / (2.f * apq);
          const float t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
          atomicAdd(&flag[sweep % 3], 1);
        }
        rc[tid] = c;
        rs[tid] = s;
        rp[tid] = p;
        rq[tid] = q;
      }
      __syncthreads();
      // C[P][Q] <- J_P^T C[P][Q] J_Q, with J = [[c, s], [-s, c]] on (p, q), and
      // E <- E J.  The blocks of a round are disjoint, so every read of this
      // thread's blocks is issued before any of its writes.
      constexpr int NGB = (NP * NP + kThreads - 1) / kThreads, NEB = (LP * NP + kThreads - 1) / kThreads;
      float m[NGB][4];
      int gi[NGB][4];
#pragma unroll
      for (int k = 0; k < NGB; ++k) {
        const int e = tid + k * kThreads;
        const int P = e < NP * NP ? e / NP : 0, Q = e < NP * NP ? e % NP : 0;
        const int p1 = rp[P], p2 = rq[P], q1 = rp[Q], q2 = rq[Q];
        gi[k][0] = p1 * SS + q1;
        gi[k][1] = p1 * SS + q2;
        gi[k][2] = p2 * SS + q1;
        gi[k][3] = p2 * SS + q2;
#pragma unroll
        for (int x = 0; x < 4; ++x) m[k][x] = G[gi[k][x]];
      }
      float ev[NEB][2];
      int ei[NEB][2];
#pragma unroll
      for (int k = 0; k < NEB; ++k) {
        const int e = tid + k * kThreads;
        const int i = e < LP * NP ? e / NP : 0, P = e < LP * NP ? e % NP : 0;
        ei[k][0] = i * SS + rp[P];
        ei[k][1] = i * SS + rq[P];
        ev[k][0] = E[ei[k][0]];
        ev[k][1] = E[ei[k][1]];
      }
#pragma unroll
      for (int k = 0; k < NGB; ++k) {
        const int e = tid + k * kThreads;
        if (e < NP * NP) {
          const int P = e / NP, Q = e % NP;
          const float cp = rc[P], sp = rs[P], cq = rc[Q], sq = rs[Q];
          const float m11 = m[k][0], m12 = m[k][1], m21 = m[k][2], m22 = m[k][3];
          const float t11 = cp * m11 - sp * m21, t12 = cp * m12 - sp * m22;
          const float t21 = sp * m11 + cp * m21, t22 = sp * m12 + cp * m22;
          G[gi[k][0]] = cq * t11 - sq * t12;
          G[gi[k][1]] = sq * t11 + cq * t12;
          G[gi[k][2]] = cq * t21 - sq * t22;
          G[gi[k][3]] = sq * t21 + cq * t22;
        }
      }
#pragma unroll
      for (int k = 0; k < NEB; ++k) {
        const int e = tid + k * kThreads;
        if (e < LP * NP) {
          const int P = e % NP;
          const float c = rc[P], s = rs[P];
          const float ep = ev[k][0], eq = ev[k][1];
          E[ei[k][0]] = c * ep - s * eq;
          E[ei[k][1]] = s * ep + c * eq;
        }
      }
      __syncthreads();
    }
    if (flag[sweep % 3] == 0) break;  // uniform: read after the sweep's last barrier
  }
}

// Workgroups per CU: four for widths up to 24, three up to 32, two up to 56
// (LDS and registers), one above.  The work is latency-bound: more workgroups
// per CU win even where the register limit spills 50-90 VGPRs (rank 16:
// 2.38 -> 1.77 ms, rank 24: 3.55 -> 2.83 ms for one layer's 2,016 blocks).
template <int LP>
__global__ __launch_bounds__(kThreads, LP <= 24 ? 4 : (LP <= 32 ? 3 : (LP <= 56 ? 2 : 1))) void k_seal(SealArgs A) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  typedef Lay<LP> L;
  constexpr int SS = L::SS;
  float* S = lds + L::S;
  float* G = lds + L::G;
  float* E = lds + L::E;
  float* anc = lds + L::ANC;
  float* errv = lds + L::ERR;
  int* sel = reinterpret_cast<int*>(lds + L::SEL);
  float* inv = lds + L::INV;
  float* sig = lds + L::SIG;
  int* perm = reinterpret_cast<int*>(lds + L::PERM);
  float* rc = lds + L::RC;
  float* rs = lds + L::RS;
  int* rp = reinterpret_cast<int*>(lds + L::RP);
  int* rq = reinterpret_cast<int*>(lds + L::RQ);
  int* flag = reinterpret_cast<int*>(lds + L::FLAG);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / A.n_heads, h = blockIdx.x % A.n_heads;
  const int slot = A.slots[b];
  if (slot < 0 || slot >= A.n_slots) return;  // the same in every thread
  const f16* xk = A.sk + b * A.sk_s + h * A.sk_h;  // [256][128]
  const f16* xv = A.sv + b * A.sv_s + h * A.sv_h;

  // anchor row, and the test matrix (zero-padded to LP columns)
  anc[tid] = (float)(tid < kD ? xk[tid] : xv[tid - kD]);
  for (int i = tid; i < 256 * LP; i += kThreads) {
    const int c = i / LP, j = i % LP;
    S[c * SS + j] = j < A.width ? A.omega[(int64_t)c * A.width + j] : 0.f;
  }
  __syncthreads();

  // ---- range finder: v holds this thread's row of Y, Z or Q.  Step 0 is
  //      Y = A omega; then odd steps Z = A^T Q, even steps Y = A Z; each
  //      result is orthonormalised.
  float v[LP];
  const int n_steps = 1 + 2 * A.power_iters;
  for (int step = 0; step < n_steps; ++step) {
    if (step > 0) {
      store_row<LP>(S, tid, v);  // the factor of this step's product
      __syncthreads();
    }
    if (step & 1)
      col_product<LP>(xk, xv, anc, S, tid, v);
    else
      row_product<LP>(xk, xv, anc, S, tid, v);
    __syncthreads();  // every thread is done reading S
    for (int pass = 0; pass < kOrthPasses; ++pass) {
      store_row<LP>(S, tid, v);
      __syncthreads();
      gram<LP>(S, G, tid);
      __syncthreads();
      if (wave == 0) cholesky<LP>(G, inv, lane);
      __syncthreads();
      solve_row<LP>(G, inv, v);
      __syncthreads();  // G and S are rewritten next
    }
  }
  // ---- B^T = A^T Q (thread c: row c), C = B B^T
  float z[LP];
  store_row<LP>(S, tid, v);
  __syncthreads();
  col_product<LP>(xk, xv, anc, S, tid, z);
  __syncthreads();
  store_row<LP>(S, tid, z);
  __syncthreads();
  gram<LP>(S, G, tid);
  __syncthreads();
  if (tid < LP) perm[tid] = tid;  // (every entry is rewritten below; never left unset)
  jacobi<LP>(G, E, rc, rs, rp, rq, flag, tid);
  // ---- singular values in descending order (equal ones by index)
  if (tid < LP) {
    const float lt = G[tid * SS + tid];
    int r = 0;
    for (int i = 0; i < LP; ++i) {
      const float li = G[i * SS + i];
      r += (li > lt || (li == lt && i < tid)) ? 1 : 0;
    }
    r = r < LP ? r : LP - 1;
    perm[r] = tid;
    sig[r] = sqrtf(fmaxf(lt, 0.f));
  }
  __syncthreads();
  // ---- right factors: W_k = B^T E_k / sigma_k (thread c: entry c), stored
  //      as fp16 and kept (rounded) in S for the residual errors
  const int rank = A.rank;
  {
    const int c = tid;
    f16* dst = c < kD ? A.vk + slot * A.vk_s + h * A.vk_h + c : A.vv + slot * A.vv_s + h * A.vv_h + (c - kD);
    for (int k = 0; k < rank; ++k) {
      const int pk = min(max(perm[k], 0), LP - 1);
      float w = 0.f;
#pragma unroll
      for (int j = 0; j < LP; ++j) w = fmaf(z[j], E[j * SS + pk], w);
      const float sk = sig[k];
      const f16 w16 = (f16)(sk > 0.f ? w / sk : 0.f);
      dst[(int64_t)k * kD] = w16;
      if (c < kD) S[k * kD + c] = (float)w16;  // V_K [rank][128]: rank * 128 <= LP * 128 < 256 * SS
    }
  }
  __syncthreads();
  // ---- left factors U S = Q E_k sigma_k (thread t: row t), the reconstruction
  //      of its key from the stored factors, and its squared error
  const int t = tid;
  if (t < kRows) {
    // the key's 128 columns in two halves of 64 (fewer live registers); each
    // column and the squared error are summed in the same order either way
    constexpr int kHalf = kD / 2;
    f16* urow = A.u + slot * A.u_s + h * A.u_h + (int64_t)t * rank;
    const f16* kr = xk + (int64_t)(t + 1) * kD;
    float e2 = 0.f;
    for (int half = 0; half < 2; ++half) {
      const int c0 = half * kHalf;
      float rec[kHalf];
#pragma unroll
      for (int c = 0; c < kHalf; ++c) rec[c] = anc[c0 + c];
      for (int k = 0; k < rank; ++k) {
        const int pk = min(max(perm[k], 0), LP - 1);
        float uk = 0.f;
#pragma unroll
        for (int j = 0; j < LP; ++j) uk = fmaf(v[j], E[j * SS + pk], uk);
        const f16 u16 = (f16)(uk * sig[k]);
        if (half == 0) urow[k] = u16;
        const float uf = (float)u16;
        const float4* vkr = reinterpret_cast<const float4*>(S + k * kD + c0);
#pragma unroll
        for (int c4 = 0; c4 < kHalf / 4; ++c4) {
          const float4 w = vkr[c4];
          rec[4 * c4 + 0] = fmaf(uf, w.x, rec[4 * c4 + 0]);
          rec[4 * c4 + 1] = fmaf(uf, w.y, rec[4 * c4 + 1]);
          rec[4 * c4 + 2] = fmaf(uf, w.z, rec[4 * c4 + 2]);
          rec[4 * c4 + 3] = fmaf(uf, w.w, rec[4 * c4 + 3]);
        }
      }
#pragma unroll
      for (int c8 = 0; c8 < kHalf / 8; ++c8) {
        const v8h x = *reinterpret_cast<const v8h*>(kr + c0 + 8 * c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = (float)x[e] - rec[8 * c8 + e];
          e2 = fmaf(d, d, e2);
        }
      }
    }
    errv[t] = e2;
  }
  // ---- anchors (exact copies)
  {
    const int c = tid;
    if (c < kD)
      A.ak[slot * A.ak_s + h * A.ak_h + c] = xk[c];
    else
      A.av[slot * A.av_s + h * A.av_h + (c - kD)] = xv[c - kD];
  }
  __syncthreads();
  // ---- residual rows: the n_resid largest errors (equal errors: lower
  //      position first), stored in ascending position order
  if (A.n_resid > 0) {
    if (t < kRows) {
      const float et = errv[t];
      int r = 0;
      for (int i = 0; i < kRows; ++i) {
        const float ei = errv[i];
        r += (ei > et || (ei == et && i < t)) ? 1 : 0;
      }
      sel[t] = r < A.n_resid ? 1 : 0;
    }
    __syncthreads();
    if (t < kRows && sel[t]) {
      int o = 0;
      for (int i = 0; i < t; ++i) o += sel[i];
      if (o >= A.n_resid) return;  // only with non-finite errors (ranks then tie): never write past R rows
      A.rp[slot * A.rp_s + h * A.rp_h + o] = (uint8_t)(t + 1);
      if (A.resid_bits != 16) {
        const int rb = A.resid_bits == 8 ? kD : kD / 2;  // code bytes per row
        quantize_row(xk + (int64_t)(t + 1) * kD, A.resid_bits,
                     reinterpret_cast<uint8_t*>(A.rk) + slot * A.rk_s + h * A.rk_h + (int64_t)o * rb,
                     A.rks + slot * A.rks_s + h * A.rks_h + (int64_t)o * 4);
        quantize_row(xv + (int64_t)(t + 1) * kD, A.resid_bits,
                     reinterpret_cast<uint8_t*>(A.rv) + slot * A.rv_s + h * A.rv_h + (int64_t)o * rb,
                     A.rvs + slot * A.rvs_s + h * A.rvs_h + (int64_t)o * 4);
        return;
      }
      const v8h* ks = reinterpret_cast<const v8h*>(xk + (int64_t)(t + 1) * kD);
      const v8h* vs = reinterpret_cast<const v8h*>(xv + (int64_t)(t + 1) * kD);
      v8h* kd = reinterpret_cast<v8h*>(A.rk + slot * A.rk_s + h * A.rk_h + (int64_t)o * kD);
      v8h* vd = reinterpret_cast<v8h*>(A.rv + slot * A.rv_s + h * A.rv_h + (int64_t)o * kD);
#pragma unroll
      for (int c8 = 0; c8 < kD / 8; ++c8) {
        kd[c8] = ks[c8];
        vd[c8] = vs[c8];
      }
    }
  }
}

dkv_status fail(dkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dkv_status fail(dkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return dkv_fail_message(s, buf);
}

bool al(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

dkv_status check_out(const dkv_view& v, const char* name, int esz, int align) {
  if (!v.ptr) return fail(DKV_ERR_INVALID_ARG, "pool->%s.ptr is NULL", name);
  if (!al(v.ptr, align) || (v.slot_stride * esz) % align != 0 || (v.head_stride * esz) % align != 0)
    return fail(DKV_ERR_UNSUPPORTED, "pool->%s must be %d-byte aligned (pointer and strides)", name, align);
  return DKV_OK;
}

template <int LP>
dkv_status launch_seal(const SealArgs& a, unsigned grid, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_seal<LP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)Lay<LP>::bytes) != hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_seal) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL((k_seal<LP>), dim3(grid), dim3(kThreads), Lay<LP>::bytes, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DKV_ERR_HIP, "k_seal launch failed: %s", hipGetErrorString(e));
  return DKV_OK;
}

// ---------------------------------------------------------------------------
// Joining blocks to a shared basis: for block slot s (current basis entry
// cur) and target entry g, with V = [V_K | V_V] rows of the entries,
//   M = V_cur V_g^T (r x r),  U' = U M,
//   retained energy = |U' V_g|^2 / |U V_cur|^2 = tr(C M G_g M^T) / tr(C G_cur),
// C = U^T U, G = V V^T.  One workgroup per (item, KV head); all products fp32
// from the fp16 arrays staged in LDS; U' is written back to slot s as fp16.
// ---------------------------------------------------------------------------

struct JoinArgs {
  f16* u; int64_t u_s, u_h;
  const f16* vk; int64_t vk_s, vk_h;
  const f16* vv; int64_t vv_s, vv_h;
  const int32_t* slots;
  const int32_t* entries;
  const int32_t* basis_of;
  int n_heads, n_slots, n_entries, rank, write;
  float* energy;
};

constexpr int kJoinThreads = 256;
constexpr int kJoinR = DKV_MAX_RANK;
// Vc, Vg [64][256] f16; Us [255][64] f16 (later T [64][64] fp32); M, C, Gg [64][64] fp32; 8 partial sums
constexpr int kJoinLds = 2 * kJoinR * 256 * 2 + 255 * kJoinR * 2 + 3 * kJoinR * kJoinR * 4 + 64;
static_assert(255 * kJoinR * 2 >= kJoinR * kJoinR * 4, "T must fit the U area");

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int k = 0; k < kJoinThreads / 64; ++k) t += red[k];
  return t;
}

__global__ __launch_bounds__(kJoinThreads) void k_join(JoinArgs a) {
  extern __shared__ __align__(16) unsigned char jsm[];
  f16* Vc = reinterpret_cast<f16*>(jsm);
  f16* Vg = Vc + kJoinR * 256;
  f16* Us = Vg + kJoinR * 256;
  float* M = reinterpret_cast<float*>(Us + 255 * kJoinR);
  float* C = M + kJoinR * kJoinR;
  float* Gg = C + kJoinR * kJoinR;
  float* red = Gg + kJoinR * kJoinR;
  const int item = blockIdx.x / a.n_heads, h = blockIdx.x % a.n_heads;
  const int t = threadIdx.x, r = a.rank;
  const int s = a.slots[item], g = a.entries[item];
  const int cur = (s >= 0 && s < a.n_slots) ? (a.basis_of ? a.basis_of[s] : s) : -1;
  if (s < 0 || s >= a.n_slots || g < 0 || g >= a.n_entries || cur < 0 || cur >= a.n_entries) {
    if (t == 0) a.energy[blockIdx.x] = -1.f;  // uniform: nothing joined
    return;
  }
  for (int e = t; e < r * 256; e += kJoinThreads) {
    const int j = e >> 8, c = e & 255;
    Vc[j * 256 + c] = c < 128 ? a.vk[cur * a.vk_s + h * a.vk_h + j * 128 + c]
                              : a.vv[cur * a.vv_s + h * a.vv_h + j * 128 + (c - 128)];
    Vg[j * 256 + c] = c < 128 ? a.vk[g * a.vk_s + h * a.vk_h + j * 128 + c]
                              : a.vv[g * a.vv_s + h * a.vv_h + j * 128 + (c - 128)];
  }
  f16* U = a.u + s * a.u_s + h * a.u_h;
  for (int e = t; e < 255 * r; e += kJoinThreads) Us[e] = U[e];
  __syncthreads();
  float eo = 0.f;
  for (int e = t; e < r * r; e += kJoinThreads) {
    const int i = e / r, j = e % r;
    float c = 0.f, m = 0.f, gc = 0.f, gg = 0.f;
    for (int k = 0; k < 255; ++k) c = __builtin_fmaf((float)Us[k * r + i], (float)Us[k * r + j], c);
    for (int k = 0; k < 256; ++k) {
      const float vi = (float)Vc[i * 256 + k], gi = (float)Vg[i * 256 + k];
      m = __builtin_fmaf(vi, (float)Vg[j * 256 + k], m);
      gc = __builtin_fmaf(vi, (float)Vc[j * 256 + k], gc);
      gg = __builtin_fmaf(gi, (float)Vg[j * 256 + k], gg);
    }
    C[e] = c;
    M[e] = m;
    Gg[e] = gg;
    eo = __builtin_fmaf(c, gc, eo);
  }
  __syncthreads();
  // X = M Gg^-1 (least squares: U' = U X solves U' V_g = U V_cur best), by a
  // Cholesky factor Gg = L L^T computed in place; a pivot below 1e-6 of the
  // largest diagonal drops its direction (rows of V_g are meant to be
  // independent).  X takes the place of the two bases, now free.
  float* X = reinterpret_cast<float*>(Vc);
  __shared__ float piv_floor;
  if (t == 0) {
    float mx = 0.f;
    for (int k = 0; k < r; ++k) mx = fmaxf(mx, Gg[k * r + k]);
    piv_floor = 1e-6f * mx;
  }
  __syncthreads();
  for (int k = 0; k < r; ++k) {
    if (t == 0) {
      const float d = Gg[k * r + k];
      Gg[k * r + k] = d > piv_floor ? sqrtf(d) : 0.f;
    }
    __syncthreads();
    const float lkk = Gg[k * r + k];
    for (int i = k + 1 + t; i < r; i += kJoinThreads) Gg[i * r + k] = lkk > 0.f ? Gg[i * r + k] / lkk : 0.f;
    __syncthreads();
    const int m = r - k - 1;
    for (int e = t; e < m * m; e += kJoinThreads) {
      const int i = k + 1 + e / m, j = k + 1 + e % m;
      if (j <= i) Gg[i * r + j] -= Gg[i * r + k] * Gg[j * r + k];
    }
    __syncthreads();
  }
  if (t < r) {
    // row t of X: x L L^T = m_t; forward L y = m_t^T, then backward L^T x^T = y
    float* x = X + t * r;
    for (int i = 0; i < r; ++i) {
      float acc = M[t * r + i];
      for (int j = 0; j < i; ++j) acc -= Gg[i * r + j] * x[j];
      const float lii = Gg[i * r + i];
      x[i] = lii > 0.f ? acc / lii : 0.f;
    }
    for (int i = r - 1; i >= 0; --i) {
      float acc = x[i];
      for (int j = i + 1; j < r; ++j) acc -= Gg[j * r + i] * x[j];
      const float lii = Gg[i * r + i];
      x[i] = lii > 0.f ? acc / lii : 0.f;
    }
  }
  __syncthreads();
  if (t < 255) {
    for (int j = 0; j < r; ++j) {
      float acc = 0.f;
      for (int i = 0; i < r; ++i) acc = __builtin_fmaf((float)Us[t * r + i], X[i * r + j], acc);
      if (a.write) U[t * r + j] = (f16)acc;
    }
  }
  // retained energy |U X V_g|^2 = tr(C X Gg X^T) = tr(C M X^T), over tr(C G_cur)
  float en = 0.f;
  for (int e = t; e < r * r; e += kJoinThreads) {
    const int i = e / r, j = e % r;
    float q = 0.f;
    for (int k = 0; k < r; ++k) q = __builtin_fmaf(M[i * r + k], X[j * r + k], q);
    en = __builtin_fmaf(C[e], q, en);
  }
  const float so = block_sum(eo, red);
  const float sn = block_sum(en, red + 4);
  if (t == 0) a.energy[blockIdx.x] = so > 0.f ? sn / so : 1.f;
}

static_assert(Lay<kMaxWidth>::bytes <= 160 * 1024, "sealer LDS exceeds 160 KB");
static_assert(kJoinLds <= 160 * 1024, "join LDS exceeds 160 KB");
static_assert(Lay<16>::SS >= 1, "padded width");
// the rounded V_K ([rank <= LP][128] at S's start) stays clear of E
static_assert(80 * kD <= Lay<80>::E && 64 * kD <= Lay<64>::E && 56 * kD <= Lay<56>::E && 48 * kD <= Lay<48>::E &&
                  32 * kD <= Lay<32>::E && 24 * kD <= Lay<24>::E && 16 * kD <= Lay<16>::E,
              "V_K overlaps the eigenvectors");

}  // namespace

extern "C" {

dkv_status dkv_seal_blocks(const dkv_pool* pool, dkv_view src_k, dkv_view src_v, const int32_t* slots,
                           int32_t n_blocks, const float* omega, int32_t width, int32_t power_iters, void* stream) {
  dkv_clear_error_message();
  const dkv_pool* P = pool;
  if (!P) return fail(DKV_ERR_INVALID_ARG, "pool is NULL");
  if (P->head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", P->head_dim);
  if (P->block_size != DKV_BLOCK_SIZE) return fail(DKV_ERR_UNSUPPORTED, "block_size %d != 256", P->block_size);
  if (P->rank < 1) return fail(DKV_ERR_INVALID_ARG, "rank %d < 1", P->rank);
  if (P->rank > DKV_MAX_RANK) return fail(DKV_ERR_UNSUPPORTED, "rank %d > 64", P->rank);
  if (P->n_resid < 0) return fail(DKV_ERR_INVALID_ARG, "n_resid %d < 0", P->n_resid);
  if (P->n_resid > DKV_MAX_RESID) return fail(DKV_ERR_UNSUPPORTED, "n_resid %d > 255", P->n_resid);
  if (P->n_kv_heads < 1) return fail(DKV_ERR_INVALID_ARG, "n_kv_heads %d < 1", P->n_kv_heads);
  if (P->n_slots < 0) return fail(DKV_ERR_INVALID_ARG, "n_slots %d < 0", P->n_slots);
  if (P->resid_format != DKV_RESID_FP16 && P->resid_format != DKV_RESID_INT8 && P->resid_format != DKV_RESID_INT4)
    return fail(DKV_ERR_INVALID_ARG, "resid_format %d", P->resid_format);
  const bool quant = P->resid_format != DKV_RESID_FP16;
  if (width < P->rank) return fail(DKV_ERR_INVALID_ARG, "width %d < rank %d", width, P->rank);
  if (width > kMaxWidth) return fail(DKV_ERR_UNSUPPORTED, "width %d > %d", width, kMaxWidth);
  if (power_iters < 0 || power_iters > kMaxPowerIters)
    return fail(DKV_ERR_INVALID_ARG, "power_iters %d not in 0..%d", power_iters, kMaxPowerIters);
  if (n_blocks < 0) return fail(DKV_ERR_INVALID_ARG, "n_blocks %d < 0", n_blocks);
  if (n_blocks == 0) return DKV_OK;
  if (!slots || !omega) return fail(DKV_ERR_INVALID_ARG, "slots / omega is NULL");
  if (!al(omega, 4)) return fail(DKV_ERR_UNSUPPORTED, "omega must be 4-byte aligned");
  if (!src_k.ptr || !src_v.ptr) return fail(DKV_ERR_INVALID_ARG, "src_k / src_v is NULL");
  if (!al(src_k.ptr, 16) || !al(src_v.ptr, 16) || (src_k.slot_stride * 2) % 16 || (src_k.head_stride * 2) % 16 ||
      (src_v.slot_stride * 2) % 16 || (src_v.head_stride * 2) % 16)
    return fail(DKV_ERR_UNSUPPORTED, "src_k / src_v must be 16-byte aligned (pointers and strides)");
  dkv_status s;
  if ((s = check_out(P->anchor_k, "anchor_k", 2, 2)) || (s = check_out(P->anchor_v, "anchor_v", 2, 2)) ||
      (s = check_out(P->u, "u", 2, 2)) || (s = check_out(P->vk, "vk", 2, 2)) || (s = check_out(P->vv, "vv", 2, 2)))
    return s;
  if (P->n_resid > 0 && !quant &&
      ((s = check_out(P->resid_k, "resid_k", 2, 16)) || (s = check_out(P->resid_v, "resid_v", 2, 16)) ||
       (s = check_out(P->resid_pos, "resid_pos", 1, 1))))
    return s;
  if (P->n_resid > 0 && quant &&
      ((s = check_out(P->resid_k, "resid_k", 1, 1)) || (s = check_out(P->resid_v, "resid_v", 1, 1)) ||
       (s = check_out(P->resid_k_sb, "resid_k_sb", 2, 2)) || (s = check_out(P->resid_v_sb, "resid_v_sb", 2, 2)) ||
       (s = check_out(P->resid_pos, "resid_pos", 1, 1))))
    return s;
  const int64_t grid = (int64_t)n_blocks * P->n_kv_heads;
  if (grid > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many blocks");
  SealArgs a;
  a.sk = (const f16*)src_k.ptr; a.sk_s = src_k.slot_stride; a.sk_h = src_k.head_stride;
  a.sv = (const f16*)src_v.ptr; a.sv_s = src_v.slot_stride; a.sv_h = src_v.head_stride;
  a.slots = slots;
  a.n_heads = P->n_kv_heads;
  a.n_slots = P->n_slots;
  a.omega = omega;
  a.width = width;
  a.rank = P->rank;
  a.n_resid = P->n_resid;
  a.power_iters = power_iters;
  a.ak = (f16*)P->anchor_k.ptr; a.ak_s = P->anchor_k.slot_stride; a.ak_h = P->anchor_k.head_stride;
  a.av = (f16*)P->anchor_v.ptr; a.av_s = P->anchor_v.slot_stride; a.av_h = P->anchor_v.head_stride;
  a.u = (f16*)P->u.ptr; a.u_s = P->u.slot_stride; a.u_h = P->u.head_stride;
  a.vk = (f16*)P->vk.ptr; a.vk_s = P->vk.slot_stride; a.vk_h = P->vk.head_stride;
  a.vv = (f16*)P->vv.ptr; a.vv_s = P->vv.slot_stride; a.vv_h = P->vv.head_stride;
  a.rk = (f16*)P->resid_k.ptr; a.rk_s = P->resid_k.slot_stride; a.rk_h = P->resid_k.head_stride;
  a.rv = (f16*)P->resid_v.ptr; a.rv_s = P->resid_v.slot_stride; a.rv_h = P->resid_v.head_stride;
  a.rp = (uint8_t*)P->resid_pos.ptr; a.rp_s = P->resid_pos.slot_stride; a.rp_h = P->resid_pos.head_stride;
  a.resid_bits = P->resid_format == DKV_RESID_INT8 ? 8 : (P->resid_format == DKV_RESID_INT4 ? 4 : 16);
  a.rks = (f16*)P->resid_k_sb.ptr; a.rks_s = P->resid_k_sb.slot_stride; a.rks_h = P->resid_k_sb.head_stride;
  a.rvs = (f16*)P->resid_v_sb.ptr; a.rvs_s = P->resid_v_sb.slot_stride; a.rvs_h = P->resid_v_sb.head_stride;
  hipStream_t st = (hipStream_t)stream;
  const unsigned g = (unsigned)grid;
  if (width <= 16)
    s = launch_seal<16>(a, g, st);
  else if (width <= 24)
    s = launch_seal<24>(a, g, st);
  else if (width <= 32)
    s = launch_seal<32>(a, g, st);
  else if (width <= 48)
    s = launch_seal<48>(a, g, st);
  else if (width <= 56)
    s = launch_seal<56>(a, g, st);  // 79 KB of LDS: two workgroups per CU
  else if (width <= 64)
    s = launch_seal<64>(a, g, st);
  else
    s = launch_seal<80>(a, g, st);
  if (s != DKV_OK) return s;
  if (P->route_key.ptr) return dkv_route_keys(P, slots, n_blocks, stream);
  return DKV_OK;
}

static dkv_status launch_join(const JoinArgs& a, int64_t grid, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_join, hipFuncAttributeMaxDynamicSharedMemorySize, kJoinLds) != hipSuccess)
      return fail(DKV_ERR_HIP, "hipFuncSetAttribute(k_join) failed");
    attr_set = true;
  }
  hipLaunchKernelGGL(k_join, dim3((unsigned)grid), dim3(kJoinThreads), kJoinLds, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DKV_ERR_HIP, "k_join launch failed: %s", hipGetErrorString(e));
  return DKV_OK;
}

dkv_status dkv_join_basis(const dkv_pool* pool, const int32_t* slots, const int32_t* entries, int32_t n,
                          int32_t write, float* energy, void* stream) {
  dkv_clear_error_message();
  const dkv_pool* P = pool;
  if (!P) return fail(DKV_ERR_INVALID_ARG, "pool is NULL");
  if (P->head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", P->head_dim);
  if (P->rank < 1) return fail(DKV_ERR_INVALID_ARG, "rank %d < 1", P->rank);
  if (P->rank > DKV_MAX_RANK) return fail(DKV_ERR_UNSUPPORTED, "rank %d > 64", P->rank);
  if (P->n_kv_heads < 1) return fail(DKV_ERR_INVALID_ARG, "n_kv_heads %d < 1", P->n_kv_heads);
  if (P->n_slots < 0) return fail(DKV_ERR_INVALID_ARG, "n_slots %d < 0", P->n_slots);
  if (P->basis_of && P->n_basis < 1) return fail(DKV_ERR_INVALID_ARG, "n_basis %d < 1 with basis_of set", P->n_basis);
  if (n < 0) return fail(DKV_ERR_INVALID_ARG, "n %d < 0", n);
  if (n == 0) return DKV_OK;
  if (!slots || !entries || !energy) return fail(DKV_ERR_INVALID_ARG, "slots / entries / energy is NULL");
  if (!al(slots, 4) || !al(entries, 4) || !al(energy, 4) || (P->basis_of && !al(P->basis_of, 4)))
    return fail(DKV_ERR_UNSUPPORTED, "slots, entries, energy and basis_of must be 4-byte aligned");
  dkv_status s;
  if ((s = check_out(P->u, "u", 2, 2)) || (s = check_out(P->vk, "vk", 2, 2)) || (s = check_out(P->vv, "vv", 2, 2)))
    return s;
  const int64_t grid = (int64_t)n * P->n_kv_heads;
  if (grid > 0x7FFFFFFF) return fail(DKV_ERR_INVALID_ARG, "too many blocks");
  JoinArgs a;
  a.u = (f16*)P->u.ptr; a.u_s = P->u.slot_stride; a.u_h = P->u.head_stride;
  a.vk = (const f16*)P->vk.ptr; a.vk_s = P->vk.slot_stride; a.vk_h = P->vk.head_stride;
  a.vv = (const f16*)P->vv.ptr; a.vv_s = P->vv.slot_stride; a.vv_h = P->vv.head_stride;
  a.slots = slots;
  a.entries = entries;
  a.basis_of = P->basis_of;
  a.n_heads = P->n_kv_heads;
  a.n_slots = P->n_slots;
  a.n_entries = P->basis_of ? P->n_basis : P->n_slots;
  a.rank = P->rank;
  a.write = write ? 1 : 0;
  a.energy = energy;
  return launch_join(a, grid, (hipStream_t)stream);
}

/* Shared bases under a budget: see dkv_attn.h.  Host-driven: block i is
 * scored against every entry open so far with k_join (write = 0), the energies
 * come back to the host, the rule picks, and a join writes U' with k_join
 * (write = 1); at the end the openers' bases are copied into the store. */
dkv_status dkv_share_bases(const dkv_pool* pool, const int32_t* slots, int32_t n, int32_t capacity, float threshold,
                           dkv_view store_vk, dkv_view store_vv, int32_t* entry, int32_t* opener, float* energy,
                           int32_t* kind, int32_t* n_entries, void* stream) {
  dkv_clear_error_message();
  const dkv_pool* P = pool;
  if (!P) return fail(DKV_ERR_INVALID_ARG, "pool is NULL");
  if (P->head_dim != DKV_HEAD_DIM) return fail(DKV_ERR_UNSUPPORTED, "head_dim %d != 128", P->head_dim);
  if (P->rank < 1) return fail(DKV_ERR_INVALID_ARG, "rank %d < 1", P->rank);
  if (P->rank > DKV_MAX_RANK) return fail(DKV_ERR_UNSUPPORTED, "rank %d > 64", P->rank);
  if (P->n_kv_heads < 1) return fail(DKV_ERR_INVALID_ARG, "n_kv_heads %d < 1", P->n_kv_heads);
  if (P->basis_of) return fail(DKV_ERR_INVALID_ARG, "the pool must hold each block's own basis (basis_of NULL)");
  if (n < 0 || capacity < 1) return fail(DKV_ERR_INVALID_ARG, "n %d < 0 or capacity %d < 1", n, capacity);
  if (!slots || !entry || !opener || !energy || !kind || !n_entries)
    return fail(DKV_ERR_INVALID_ARG, "slots / entry / opener / energy / kind / n_entries is NULL");
  if (!store_vk.ptr || !store_vv.ptr) return fail(DKV_ERR_INVALID_ARG, "store arrays are NULL");
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= P->n_slots) return fail(DKV_ERR_INVALID_ARG, "slot %d out of range", slots[i]);
    for (int k = 0; k < i; ++k)
      if (slots[k] == slots[i]) return fail(DKV_ERR_INVALID_ARG, "slot %d given twice", slots[i]);
  }
  dkv_status s;
  if ((s = check_out(P->u, "u", 2, 2)) || (s = check_out(P->vk, "vk", 2, 2)) || (s = check_out(P->vv, "vv", 2, 2)) ||
      (s = check_out(store_vk, "store_vk", 2, 2)) || (s = check_out(store_vv, "store_vv", 2, 2)))
    return s;
  *n_entries = 0;
  if (n == 0) return DKV_OK;
  const int H = P->n_kv_heads, cap = capacity < n ? capacity : n;
  const hipStream_t st = (hipStream_t)stream;
  // device scratch of this call: candidate slots and entries, their energies
  int32_t* d = nullptr;
  float* d_e = nullptr;
  if (hipMalloc((void**)&d, sizeof(int32_t) * 2 * (size_t)cap) != hipSuccess ||
      hipMalloc((void**)&d_e, sizeof(float) * (size_t)cap * H) != hipSuccess) {
    (void)hipFree(d);
    return fail(DKV_ERR_HIP, "hipMalloc failed");
  }
  std::vector<int32_t> cand_s((size_t)cap), open_slot;
  std::vector<float> es((size_t)cap * H);
  JoinArgs a;
  a.u = (f16*)P->u.ptr; a.u_s = P->u.slot_stride; a.u_h = P->u.head_stride;
  a.vk = (const f16*)P->vk.ptr; a.vk_s = P->vk.slot_stride; a.vk_h = P->vk.head_stride;
  a.vv = (const f16*)P->vv.ptr; a.vv_s = P->vv.slot_stride; a.vv_h = P->vv.head_stride;
  a.basis_of = nullptr;
  a.n_heads = H;
  a.n_slots = P->n_slots;
  a.n_entries = P->n_slots;
  a.rank = P->rank;
  a.slots = d;
  a.entries = d + cap;
  a.energy = d_e;
  for (int i = 0; i < n && s == DKV_OK; ++i) {
    const int m = (int)open_slot.size();
    int best = -1;
    float best_e = -INFINITY;
    if (m > 0) {
      for (int j = 0; j < m; ++j) cand_s[(size_t)j] = slots[i];
      a.write = 0;
      if (hipMemcpyAsync(d, cand_s.data(), sizeof(int32_t) * m, hipMemcpyHostToDevice, st) != hipSuccess ||
          hipMemcpyAsync(d + cap, open_slot.data(), sizeof(int32_t) * m, hipMemcpyHostToDevice, st) != hipSuccess) {
        s = fail(DKV_ERR_HIP, "hipMemcpyAsync failed");
        break;
      }
      if ((s = launch_join(a, (int64_t)m * H, st))) break;
      if (hipMemcpyAsync(es.data(), d_e, sizeof(float) * m * H, hipMemcpyDeviceToHost, st) != hipSuccess ||
          hipStreamSynchronize(st) != hipSuccess) {
        s = fail(DKV_ERR_HIP, "reading the join energies failed");
        break;
      }
      for (int j = 0; j < m; ++j) {
        float e = 0.f;
        for (int h = 0; h < H; ++h) e += es[(size_t)j * H + h];
        e /= (float)H;
        if (e > best_e) {
          best_e = e;
          best = j;
        }
      }
    }
    if (best >= 0 && best_e >= threshold) {
      entry[i] = best;
      energy[i] = best_e;
      kind[i] = 1;
    } else if (m < capacity) {
      entry[i] = m;
      energy[i] = 1.f;
      kind[i] = 0;
      open_slot.push_back(slots[i]);
      continue;
    } else {
      entry[i] = best;
      energy[i] = best_e;
      kind[i] = 2;
    }
    // the join: U' into the block's U
    a.write = 1;
    const int32_t pair[2] = {slots[i], open_slot[(size_t)entry[i]]};
    if (hipMemcpyAsync(d, &pair[0], sizeof(int32_t), hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(d + cap, &pair[1], sizeof(int32_t), hipMemcpyHostToDevice, st) != hipSuccess) {
      s = fail(DKV_ERR_HIP, "hipMemcpyAsync failed");
      break;
    }
    if ((s = launch_join(a, H, st))) break;
    if (hipStreamSynchronize(st) != hipSuccess) s = fail(DKV_ERR_HIP, "join failed");
  }
  // the store: entry j holds the basis of the block that opened it
  const size_t rowb = (size_t)P->rank * DKV_HEAD_DIM * 2;
  for (size_t j = 0; j < open_slot.size() && s == DKV_OK; ++j) {
    opener[j] = open_slot[j];
    for (int h = 0; h < H && s == DKV_OK; ++h) {
      const int64_t src = (int64_t)open_slot[j] * P->vk.slot_stride + (int64_t)h * P->vk.head_stride;
      const int64_t srv = (int64_t)open_slot[j] * P->vv.slot_stride + (int64_t)h * P->vv.head_stride;
      const int64_t dk = (int64_t)j * store_vk.slot_stride + (int64_t)h * store_vk.head_stride;
      const int64_t dv = (int64_t)j * store_vv.slot_stride + (int64_t)h * store_vv.head_stride;
      if (hipMemcpyAsync((f16*)store_vk.ptr + dk, (const f16*)P->vk.ptr + src, rowb, hipMemcpyDeviceToDevice, st) !=
              hipSuccess ||
          hipMemcpyAsync((f16*)store_vv.ptr + dv, (const f16*)P->vv.ptr + srv, rowb, hipMemcpyDeviceToDevice, st) !=
              hipSuccess)
        s = fail(DKV_ERR_HIP, "copying a basis into the store failed");
    }
  }
  if (hipStreamSynchronize(st) != hipSuccess && s == DKV_OK) s = fail(DKV_ERR_HIP, "stream failed");
  (void)hipFree(d);
  (void)hipFree(d_e);
  if (s == DKV_OK) *n_entries = (int32_t)open_slot.size();
  return s;
}

}  // extern "C"
