// dkv_stream.hip -- the streaming decode launch of libdkv_attn (gfx950).
//
// The fused decode step of one or several layers (routing, attention of the
// routed blocks and of the window, log-sum-exp merge; the Zenodo abstract's
// decode path and the README's "Decode & Prefill Innovations": low-rank space
// scoring, values gathered through the factors, flash-style LSE combine), for
// pools of rotated keys with fp16 residual rows.  Work items come from the
// same per-XCD queues as the other fused launches (routings, window parts,
// block parts, merges), but an attention part streams its data through LDS:
//
//   * the part's bytes are cut into pages of at most 16 KB (a block: V_K with
//     a_k; U positions 0..127; U positions 128..255; then K and V rows 64 at a
//     time; last V_V with a_v.  A window chunk: K and V rows 64 at a time);
//   * pages are copied straight from HBM into a ring of four 17 KB LDS slots
//     with 16-byte direct-to-LDS loads (global_load_lds_dwordx4), three pages
//     ahead of the one being used, so no register holds data in flight and the
//     next pages stream in while a page is being used;
//   * each 16-byte chunk may come from any address, which gives three things
//     for free: 128-wide rows are stored 272 bytes apart (a 16-byte pad, so
//     MFMA operand reads of 16 rows hit 16 different bank groups), rows beyond
//     the data are filled from a zero chunk (no stale LDS is ever read), and U
//     positions 0..127 start with a zero row for the anchor;
//   * the MFMA operands that need rows of a page as columns (V^T for p.V, U^T
//     for p^T U, V_V^T for the fold) are read with ds_read_b64_tr_b16.
//
// A block part may hold several routed blocks of one unit, streamed back to
// back (the softmax state runs across them), so that a part's fixed costs are
// shared and its loads stay in flight across block boundaries.

#include "dkv_common.h"

namespace {

constexpr int kSRowB = 272;                      // bytes per 128-wide fp16 row in LDS: 256 + one 16-byte pad
constexpr int kSPage = 64 * kSRowB;              // bytes per ring slot: 64 such rows
constexpr int kSSlots = 4;                       // ring depth
constexpr int kSRing = kSPage * kSSlots;
constexpr int kSQOff = kSRing;                   // the unit's query rows [16][128] fp16 (4 KB)
constexpr int kSQtOff = kSQOff + 16 * kD * 2;    // V_K q exchange [64][16] fp32 (4 KB)
constexpr int kSMaskOff = kSQtOff + 64 * 16 * 4; // residual-position masks [2][8] u32
constexpr int kSMaxBlocks = 32;                  // routed blocks per part at most
constexpr int kSSlotOff = kSMaskOff + 64;        // the part's routed pool slots [kSMaxBlocks]
constexpr int kSNvOff = kSSlotOff + 4 * kSMaxBlocks;
constexpr int kSLds = kSNvOff + 16;
constexpr int kSRows = 64;                       // K / V rows per page

static_assert(kSLds % 16 == 0, "LDS areas are 16-byte aligned");

typedef __attribute__((address_space(3))) void lds_void;

// 16 zero bytes in global memory: the source of every chunk of a page that
// holds no data (a page is always filled completely)
__device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

// wait until at most n of this wave's vector-memory operations are outstanding
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

// max / sum over the four lanes that share a query head (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float hq_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float hq_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __fp16 v4fp16 __attribute__((__vector_size__(4 * sizeof(__fp16))));

// Transposed LDS read: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte reads of lanes 4 j + i / 4 (j = 0..3).  A lane that
// addresses row k0 + (s >> 2), columns c0 + 4 (s & 3) .. + 3 of a row-major
// fp16 matrix (s = its index in the group) so receives rows k0 .. k0 + 3 of
// column c0 + i: the MFMA operand layout of a matrix stored with the
// contraction index as its rows.
__device__ __forceinline__ v4h ld_tr(const unsigned char* p) {
  const v4fp16 t = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) v4fp16*)p);
  return __builtin_bit_cast(v4h, t);
}

__device__ __forceinline__ v4f mfma32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// byte offset of (row, 8-half chunk c) of a 128-wide fp16 page: rows of 17
// chunks (the last one padding), so that the 16 rows of an MFMA tile start in
// 16 different bank groups
__device__ __forceinline__ int swz(int row, int c) { return row * kSRowB + (c << 4); }

// Page layout of a part.  A block has 4 + 2 nt pages: 0 V_K rows and a_k (row
// r) plus the residual positions (dwords at kPosOff); 1 U positions 0..127 (a
// zero row, then U rows 0..126); 2 U positions 128..255 (U rows 127..254);
// then K and V pages of 64 residual rows each; last V_V rows and a_v (row r).
// A window part has 2 nt pages, K and V of 64 rows each.
enum PageKind { kPageVK = 0, kPageU0 = 1, kPageU1 = 2, kPageK = 3, kPageV = 4, kPageVV = 5 };

struct StreamGeom {
  int r, nq;       // rank and round16(r) / 16
  int R, nt;       // residual rows, and their 64-row tiles
  int ppb;         // pages per block
  bool window;     // a window part
  int nrows;       // window part: its rows
  int total;       // pages of the part
};

// A page cursor: block `blk` of the part and page `k` of that block (for a
// window part, blk = 0 and k counts its pages), advanced one page at a time.
struct PageCursor {
  int blk, k;
  __device__ __forceinline__ void next(const StreamGeom& g) {
    if (++k == g.ppb && !g.window) {
      k = 0;
      ++blk;
    }
  }
  // kind of the page and its K / V tile
  __device__ __forceinline__ void kind(const StreamGeom& g, int& kd, int& t) const {
    if (g.window) {
      kd = kPageK + (k & 1);
      t = k >> 1;
    } else if (k < 3) {
      kd = k;
      t = 0;
    } else if (k == g.ppb - 1) {
      kd = kPageVV;
      t = 0;
    } else {
      kd = kPageK + ((k - 3) & 1);
      t = (k - 3) >> 1;
    }
  }
};

__device__ __forceinline__ int rows_of_tile(const StreamGeom& g, int t) {
  const int n = g.window ? g.nrows : g.R;
  const int rem = n - kSRows * t;
  return rem < kSRows ? rem : kSRows;
}

constexpr int kPosOff = 57 * kSRowB;  // residual positions (bytes) in a V_K page: after at most 57 rows

// Per-block source addresses, gathered once per part into LDS (bytes):
// a_k, a_v, U, V_K, V_V, K rows, V rows, positions.
enum { kBaseAK = 0, kBaseAV, kBaseU, kBaseVK, kBaseVV, kBaseRK, kBaseRV, kBaseRP, kBases };
constexpr int kSBaseOff = kSLds;                        // [kSMaxBlocks][kBases] u64
constexpr int kSLdsTotal = kSBaseOff + kSMaxBlocks * kBases * 8;

__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4b(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, off, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutside = 0xFFFFFFF0u;  // a buffer offset past every resource: the load returns zeros

// Issue this wave's loads of the page at cursor `cur` into ring slot `dst`;
// returns how many vector-memory instructions this wave issued for it.  The
// loads are buffer loads straight into LDS: each source array is a buffer
// resource sized to its data, and every 16-byte chunk of the page whose
// offset falls outside it (row pads, rows past the data, U's leading zero row)
// is written as zeros by the range check.  A 128-wide row page maps chunk p to
// row p / 17, chunk p % 17 (chunk 16 is the row's pad); a U page maps p
// linearly.  The extra row r of a V_K / V_V page (a_k / a_v) comes from a load
// of its own.
__device__ __forceinline__ int issue_page(const StreamGeom& g, const PageCursor& cur, unsigned char* dst,
                                          const uint64_t* bases, const char* wk_rows, const char* wv_rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int kind, t;
  cur.kind(g, kind, t);
  const int r = g.r;
  const uint64_t* bb = bases + cur.blk * kBases;
  int ops = 0;
  if (kind == kPageU0 || kind == kPageU1) {
    // U positions 0..127: a zero row (offsets below the data), U rows 0..126;
    // positions 128..255: U rows 127..254; then a zero chunk past the data
    const bool first = kind == kPageU0;
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_of((const char*)bb[kBaseU] + (first ? 0 : 254 * r), (uint32_t)(first ? 254 * r : 256 * r));
    const int ni = (16 * r + 1 + 63) >> 6;
    const int p_off = first ? (r >> 3) : 0;
    for (int i = wave; i < ni; i += kAttWaves) {
      dma16b(rs, (uint32_t)(16 * (64 * i + lane - p_off)), dst + 1024 * i);
      ++ops;
    }
    return ops;
  }
  const char* base0;
  int nvalid, special = -1, rows;
  if (kind == kPageVK || kind == kPageVV) {
    base0 = (const char*)bb[kind == kPageVK ? kBaseVK : kBaseVV];
    nvalid = r;
    special = r;
    rows = kind == kPageVK ? r + 1 : round16(r + 1);  // the fold reads round16(r + 1) rows
  } else {
    nvalid = rows_of_tile(g, t);
    if (g.window)
      base0 = (kind == kPageK ? wk_rows : wv_rows) + (int64_t)kSRows * t * 256;
    else
      base0 = (const char*)bb[kind == kPageK ? kBaseRK : kBaseRV] + (int64_t)kSRows * t * 256;
    rows = round16(nvalid);
  }
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base0, (uint32_t)nvalid * 256u);
  const int nch = 17 * rows;
  const int ni = (nch + 63) >> 6;
  for (int i = wave; i < ni; i += kAttWaves) {
    const int p = 64 * i + lane;
    const int row = (p * 3856) >> 16;  // p / 17 for p < 4097
    const int c = p - 17 * row;
    const uint32_t off = c < 16 ? (uint32_t)(row * 256 + 16 * c) : kOutside;
    if (p < nch && row != special) dma16b(rs, off, dst + 1024 * i);
    ++ops;
  }
  if (special >= 0 && wave == kAttWaves - 1) {
    // row r: a_k or a_v (16 chunks) and its pad
    const __amdgpu_buffer_rsrc_t rs1 = rsrc_of((const char*)bb[kind == kPageVK ? kBaseAK : kBaseAV], 256u);
    if (lane < 17) dma16b(rs1, lane < 16 ? (uint32_t)(16 * lane) : kOutside, dst + kSRowB * special);
    ++ops;
  }
  if (kind == kPageVK && wave == 0 && g.R > 0) {
    // residual positions: R bytes as R / 4 dwords (R % 4 == 0)
    const __amdgpu_buffer_rsrc_t rp = rsrc_of((const char*)bb[kBaseRP], (uint32_t)g.R);
    if (4 * lane < g.R) dma4b(rp, (uint32_t)(4 * lane), dst + kPosOff);
    ++ops;
  }
  return ops;
}

// Attention state of one wave (transposed accumulators: the query head is the
// MFMA column, lane % 16, so every per-head factor is the lane's own value).
struct SState {
  v4f Ot[8];   // O^T[d = 16 n + 4 (lane / 16) + e][head]
  v4f Wt[4];   // W^T[j = 16 k + 4 (lane / 16) + e][head] = sum_pos Ux[pos][j] p[pos][head] of the current block
  float m;     // running maximum of the head's scaled scores
  float l;     // this lane's share of sum p (all rows)
  float llr;   // this lane's share of sum p over the current block's low-rank rows (anchor included)
};

// Reference maximum slack: the weights exp(z - m) stay below 2 (m is raised,
// and the state rescaled, only when a score exceeds m by more than ln 2), so
// that they, and sums of up to 256 of them times U, stay well inside fp16.
constexpr float kLn2 = 0.69314718f;

// New scores of the wave's rows (NS values per lane, already scaled, -inf for
// masked rows): raise the reference maximum m (per query head, the same in the
// head's four lanes) if some score exceeds it by more than ln 2, rescaling the
// state, and return the weights exp(z - m).  The common case needs no
// cross-lane step.
template <int NS>
__device__ __forceinline__ void softmax_step(SState& st, float (&z)[NS], bool lowrank) {
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) tm = fmaxf(tm, z[i]);
  if (__ballot(tm > st.m + kLn2) != 0ull) {
    tm = hq_max(tm);
    if (tm > st.m) {
      const float mn = tm;
      const float alpha = (st.m == -INFINITY) ? 0.f : __expf(st.m - mn);
#pragma unroll
      for (int n = 0; n < 8; ++n) st.Ot[n] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) st.Wt[k] *= alpha;
      st.l *= alpha;
      st.llr *= alpha;
      st.m = mn;
    }
  }
  const bool none = st.m == -INFINITY;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    z[i] = none ? 0.f : __expf(z[i] - st.m);
    s += z[i];
  }
  st.l += s;
  if (lowrank) st.llr += s;
}

__device__ __forceinline__ v4h to_h4v(float a, float b, float c, float d) {
  v4h h;
  h[0] = (f16)a;
  h[1] = (f16)b;
  h[2] = (f16)c;
  h[3] = (f16)d;
  return h;
}

__device__ __forceinline__ void split4(v4f x, v4h& hi, v4h& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16 hh = (f16)x[e];
    hi[e] = hh;
    lo[e] = (f16)(x[e] - (float)hh);
  }
}

// Store a part's partial (o normalised, lse) for the unit's G query rows.
__device__ __forceinline__ void store_empty(const AttnArgs& A, int row0, int G, int part) {
  const int tid = threadIdx.x;
  for (int t = tid; t < G * kD; t += kAttThreads) {
    const int g = t / kD, d = t % kD;
    st_dev(&A.part_o[((int64_t)(row0 + g) * A.n_parts + part) * kD + d], 0.f);
  }
  if (tid < G) st_dev(&A.part_lse[(int64_t)(row0 + tid) * A.n_parts + part], -INFINITY);
}

// One attention part of unit u: part p < n_block_parts holds routed ranks
// [p * bpi, min((p + 1) * bpi, top_k)); the others are window chunks of
// win_chunk rows.
__device__ __forceinline__ void stream_part(const PoolArgs& P, const BatchArgs& Bt, const AttnArgs& A,
                                         const int32_t* slots, uint32_t* ctrl, int u, int p, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  const int G = Bt.G;
  const int row0 = b * Bt.Hq + h * G;
  const int part = A.part_offset + p;
  int32_t* slist = reinterpret_cast<int32_t*>(smem + kSSlotOff);
  int32_t* shn = reinterpret_cast<int32_t*>(smem + kSNvOff);
  uint32_t* masks = reinterpret_cast<uint32_t*>(smem + kSMaskOff);

  StreamGeom g;
  g.r = P.rank;
  g.nq = round16(P.rank) >> 4;
  g.R = P.n_resid;
  g.nt = (P.n_resid + kSRows - 1) / kSRows;
  g.ppb = 4 + 2 * g.nt;
  g.window = p >= A.n_block_parts;
  g.nrows = 0;
  int wrow0 = 0;
  int nv = 0;
  if (!g.window) {
    // the part's routed slots, waited for (bounded) until the routing wrote them
    const int k0 = p * A.blocks_per_item;
    const int kn = (A.top_k - k0 < A.blocks_per_item ? A.top_k - k0 : A.blocks_per_item);
    if (wave == 0) {
      int32_t slot = -1;
      if (lane < kn) {
        const int32_t* sp = &slots[(int64_t)u * A.top_k + k0 + lane];
        unsigned n = 0;
        int32_t v = ld_dev(sp);
        while (v == kSlotPending && n < kRouteWaitLimit) {
          __builtin_amdgcn_s_sleep(1);
          v = ld_dev(sp);
          ++n;
        }
        if (v == kSlotPending) {
          atomicOr(&ctrl[2], 1u);
          v = -1 + kSlotCode;
        }
        slot = v - kSlotCode;
        if (slot >= P.n_slots) slot = -1;
      }
      const bool ok = slot >= 0;
      const uint64_t m = __ballot(ok);
      const int pos = __popcll(m & ((1ull << lane) - 1ull));
      if (ok) slist[pos] = slot;
      if (lane == 0) shn[0] = __popcll(m);
    }
    lds_barrier();
    nv = shn[0];
    g.total = nv * g.ppb;
  } else {
    const int s = p - A.n_block_parts;
    int wl = Bt.wlen ? Bt.wlen[b] : Bt.W;
    wl = wl < 0 ? 0 : (wl > Bt.W ? Bt.W : wl);
    const int start = s * A.win_chunk;
    const int end = (start + A.win_chunk < wl) ? start + A.win_chunk : wl;
    g.nrows = end > start ? end - start : 0;
    wrow0 = start;
    g.total = 2 * ((g.nrows + kSRows - 1) / kSRows);
  }
  if (g.total == 0) {
    store_empty(A, row0, G, part);
    return;
  }
  const int64_t win_base = (((int64_t)b * Bt.Hkv + h) * Bt.W) * kD;
  const char* wk_rows = (const char*)(Bt.wk + win_base + (int64_t)wrow0 * kD);
  const char* wv_rows = (const char*)(Bt.wv + win_base + (int64_t)wrow0 * kD);

  // ---- the source addresses of the part's blocks, once
  uint64_t* bases = reinterpret_cast<uint64_t*>(smem + kSBaseOff);
  if (!g.window && tid < nv * kBases) {
    const int blk = tid / kBases, which = tid % kBases;
    const int64_t slot = slist[blk];
    const void* a;
    switch (which) {
      case kBaseAK: a = P.ak + slot * P.ak_s + h * P.ak_h; break;
      case kBaseAV: a = P.av + slot * P.av_s + h * P.av_h; break;
      case kBaseU: a = P.u + slot * P.u_s + h * P.u_h; break;
      case kBaseVK: a = P.vk + slot * P.vk_s + h * P.vk_h; break;
      case kBaseVV: a = P.vv + slot * P.vv_s + h * P.vv_h; break;
      case kBaseRK: a = P.rk + slot * P.rk_s + h * P.rk_h; break;
      case kBaseRV: a = P.rv + slot * P.rv_s + h * P.rv_h; break;
      default: a = P.rp + slot * P.rp_s + h * P.rp_h; break;
    }
    bases[tid] = (uint64_t)a;
  }
  if (tid < 16) masks[tid] = 0u;
  lds_barrier();

  // ---- prologue: the query rows (heads past G read the zero chunk), the first pages.
  // in_flight: this wave's load-instruction counts of the pages issued and not
  // yet waited for, one byte each, the oldest in the low byte.
  unsigned char* qrows = smem + kSQOff;
  {
    const int hh = tid >> 4, c = tid & 15;
    const void* src = hh < G ? (const void*)(Bt.q + (int64_t)(row0 + hh) * kD + 8 * c) : (const void*)kZeroChunk;
    dma16(src, qrows + 1024 * wave);
  }
  PageCursor ic = {0, 0};   // next page to issue
  int n_issued = 0;
  uint32_t in_flight = 0u;
  for (; n_issued < kSSlots - 1 && n_issued < g.total; ++n_issued) {
    const int ops = issue_page(g, ic, smem + kSPage * n_issued, bases, wk_rows, wv_rows) + (n_issued == 0 ? 1 : 0);
    in_flight |= (uint32_t)ops << (8 * n_issued);
    ic.next(g);
  }

  SState st;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.Ot[n] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  st.llr = 0.f;
  const float scale = A.scale;
  v8h qf[4];          // q[head = l16][32 s + 8 q4 + 0..7], the B operand of the d-contractions
  v4h qth[4], qtl[4];  // V_K q of the current block (hi + lo fp16), rows 16 k + 4 q4 + e, head l16
  float qa = 0.f;     // scale * q . a_k of the current block
  uint32_t mbits = 0u; // residual-position bits of the lane's positions in the current block
  v4h pv;             // weights of the wave's rows of the current K page (fp16), for its V page
  PageCursor cc = {0, 0};   // page being used

  for (int n = 0; n < g.total; ++n, cc.next(g)) {
    // this wave's loads of the pages issued after page n may stay in flight
    const uint32_t after = in_flight >> 8;
    wait_vm((int)((after & 0xFFu) + ((after >> 8) & 0xFFu) + (after >> 16)));
    lds_barrier();
    in_flight = after;
    if (n_issued < g.total) {
      const int ops = issue_page(g, ic, smem + kSPage * (n_issued % kSSlots), bases, wk_rows, wv_rows);
      in_flight |= (uint32_t)ops << (8 * (n_issued - n - 1));
      ic.next(g);
      ++n_issued;
    }
    if (n == 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qf[s] = *reinterpret_cast<const v8h*>(qrows + l16 * 256 + 64 * s + 16 * q4);
    }
    const unsigned char* pg = smem + kSPage * (n % kSSlots);
    int kind, t;
    cc.kind(g, kind, t);
    const int blk = cc.blk;
    const int r = g.r;
    if (kind == kPageVK) {
      // V_K q (rows j < r) and q . a_k (row r): wave w takes rows 16 w .. 16 w + 15
      if (16 * wave < r + 1) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const int j = 16 * wave + l16;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma32(*reinterpret_cast<const v8h*>(pg + swz(j, 4 * s + q4)), qf[s], acc);
        float* qt = reinterpret_cast<float*>(smem + kSQtOff);
#pragma unroll
        for (int e = 0; e < 4; ++e) qt[(16 * wave + 4 * q4 + e) * 16 + l16] = acc[e];
      }
      // residual-position mask of this block; the other buffer is cleared for the next block
      uint32_t* mk = masks + 8 * (blk & 1);
      if (wave == 1 && lane < 8) masks[8 * ((blk + 1) & 1) + lane] = 0u;
      if (tid < g.R) {
        const int ps = pg[kPosOff + tid];
        if (ps >= 1 && ps <= kLowRankRows) atomicOr(&mk[ps >> 5], 1u << (ps & 31));
      }
    } else if (kind == kPageU0 || kind == kPageU1) {
      if (kind == kPageU0) {
        // this block's scaled V_K q rows (zero beyond r) and q . a_k, and the
        // residual-position bits of the lane's 16 positions (4 q4 + e of its
        // two tiles, in both U pages)
        const float* qt = reinterpret_cast<const float*>(smem + kSQtOff);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k < g.nq) {
            v4f x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = 16 * k + 4 * q4 + e;
              x[e] = j < r ? qt[j * 16 + l16] * scale : 0.f;
            }
            split4(x, qth[k], qtl[k]);
          }
        }
        qa = qt[r * 16 + l16] * scale;
        const uint32_t* mk = masks + 8 * (blk & 1);
        const uint32_t w0 = mk[wave], w1 = mk[wave + 4];
        mbits = ((w0 >> (4 * q4)) & 0xFu) | (((w0 >> (16 + 4 * q4)) & 0xFu) << 4) |
                (((w1 >> (4 * q4)) & 0xFu) << 8) | (((w1 >> (16 + 4 * q4)) & 0xFu) << 12);
      }
      const uint32_t pbits = kind == kPageU0 ? (mbits & 0xFFu) : (mbits >> 8);
      float z[8];
      v4f zt[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int lrow = 32 * wave + 16 * tt + l16;  // row of the page = position - posbase
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k < g.nq) {
            const v4h a = *reinterpret_cast<const v4h*>(pg + 2 * (lrow * r + 16 * k + 4 * q4));
            acc = mfma16(a, qth[k], acc);
            acc = mfma16(a, qtl[k], acc);
          }
        }
        zt[tt] = acc;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool masked = ((pbits >> (4 * tt + e)) & 1u) != 0u;
          z[4 * tt + e] = masked ? -INFINITY : zt[tt][e] + qa;
        }
      }
      softmax_step<8>(st, z, true);
      v8h pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (f16)z[e];
      // W^T += Ux^T p over the wave's 32 positions (positions 4 q4 + t of both tiles)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < g.nq) {
          const int c0 = 16 * k + 4 * (l16 & 3);
          const int ra = 32 * wave + 4 * q4 + (l16 >> 2);
          const v4h a0 = ld_tr(pg + 2 * (ra * r + c0));
          const v4h a1 = ld_tr(pg + 2 * ((ra + 16) * r + c0));
          const v8h a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
          st.Wt[k] = mfma32(a, pf, st.Wt[k]);
        }
      }
    } else if (kind == kPageK) {
      const int nr = rows_of_tile(g, t);
      if (16 * wave < nr) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const int row = 16 * wave + l16;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma32(*reinterpret_cast<const v8h*>(pg + swz(row, 4 * s + q4)), qf[s], acc);
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = (16 * wave + 4 * q4 + e < nr) ? acc[e] * scale : -INFINITY;
        softmax_step<4>(st, z, false);
        pv = to_h4v(z[0], z[1], z[2], z[3]);
      }
    } else if (kind == kPageV) {
      const int nr = rows_of_tile(g, t);
      if (16 * wave < nr) {
        const int s4 = l16 & 3;
        const int row = 16 * wave + 4 * q4 + (l16 >> 2);
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
          const v4h a = ld_tr(pg + swz(row, 2 * nn + (s4 >> 1)) + 8 * (s4 & 1));
          st.Ot[nn] = mfma16(a, pv, st.Ot[nn]);
        }
      }
    } else {
      // kPageVV: fold this block's low-rank values, (p^T U) V_V + (sum p) a_v,
      // as one product: row r of W^T is the block's low-rank weight sum, row r
      // of the page a_v
      const int nqv = round16(r + 1) >> 4;
      const float llr = hq_sum(st.llr);
      st.llr = 0.f;
      v4h wh[4], wlo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < nqv) {
          v4f x = st.Wt[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * k + 4 * q4 + e;
            x[e] = j < r ? x[e] : (j == r ? llr : 0.f);
          }
          split4(x, wh[k], wlo[k]);
          st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
        }
      }
      const int s4 = l16 & 3;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        v4f acc = st.Ot[nn];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k < nqv) {
            const int row = 16 * k + 4 * q4 + (l16 >> 2);
            const v4h a = ld_tr(pg + swz(row, 2 * nn + (s4 >> 1)) + 8 * (s4 & 1));
            acc = mfma16(a, wh[k], acc);
            acc = mfma16(a, wlo[k], acc);
          }
        }
        st.Ot[nn] = acc;
      }
    }
  }

  // ---- the four waves' states at their common maximum, summed in wave order
  lds_barrier();  // every wave is done with the ring
  float* red = reinterpret_cast<float*>(smem);            // [4 waves][16 heads][132]
  float* wst = reinterpret_cast<float*>(smem + 4 * 16 * 132 * 4);  // m [4][16], l [4][16]
  const float lt = hq_sum(st.l);
  if (q4 == 0) {
    wst[wave * 16 + l16] = st.m;
    wst[64 + wave * 16 + l16] = lt;
  }
#pragma unroll
  for (int nn = 0; nn < 8; ++nn)
    *reinterpret_cast<v4f*>(red + (wave * 16 + l16) * 132 + 16 * nn + 4 * q4) = st.Ot[nn];
  lds_barrier();
  const __amdgpu_buffer_rsrc_t Po = coherent_rsrc(A.part_o + ((int64_t)row0 * A.n_parts + part) * kD, 0xFFFFFFFFu);
  for (int t2 = tid; t2 < G * (kD / 4); t2 += kAttThreads) {
    const int gg = t2 / (kD / 4), c4 = t2 % (kD / 4);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, wst[w * 16 + gg]);
    float Lg = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
      const float mw = wst[w * 16 + gg];
      const float f = (mw == -INFINITY) ? 0.f : __expf(mw - M);
      Lg += wst[64 + w * 16 + gg] * f;
      const float4 x = *reinterpret_cast<const float4*>(red + (w * 16 + gg) * 132 + 4 * c4);
      o.x += x.x * f;
      o.y += x.y * f;
      o.z += x.z * f;
      o.w += x.w * f;
    }
    const float inv = (Lg > 0.f) ? 1.f / Lg : 0.f;
    st_coherent4(Po, (uint32_t)((gg * A.n_parts * kD + 4 * c4) * 4),
                 make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
    if (c4 == 0) st_dev(&A.part_lse[(int64_t)(row0 + gg) * A.n_parts + part], (Lg > 0.f) ? M + __logf(Lg) : -INFINITY);
  }
}

// One work item of a streaming decode launch (see decode_item in the other
// fused launches: routings, then attention parts, then merges).
__device__ __forceinline__ void stream_item(const PoolArgs& P, const BatchArgs& Bt, const DecodeArgs& D, int t,
                                            unsigned char* smem, RouteShared<kAttWaves>& rsh) {
  const int tid = threadIdx.x;
  if (t < 0) {
    // no item
  } else if (t < D.n_route) {
    __builtin_amdgcn_s_setprio(2);  // every other item of the launch waits on routing
    route_unit<kAttThreads>(P, Bt, t, D.att.top_k, D.idx, nullptr, D.slots, reinterpret_cast<uint32_t*>(smem), rsh);
  } else if (t < D.n_part_end) {
    const int it = t - D.n_route;
    const int u = it / D.att.items_per_unit, p = it % D.att.items_per_unit;
    stream_part(P, Bt, D.att, D.slots, D.ctrl, u, p, smem);
    stores_done();
    __syncthreads();
    if (tid == 0) atomicAdd(&D.unit_done[u], 1u);
  } else if (t < D.n_items) {
    const int it = t - D.n_part_end;
    const int u = it / D.merges, g = it % D.merges;
    if (tid == 0) {
      const uint32_t want = (uint32_t)D.att.items_per_unit;
      unsigned n = 0;
      uint32_t v = ld_dev(&D.unit_done[u]);
      while (v < want && n < kRouteWaitLimit) {
        __builtin_amdgcn_s_sleep(2);
        v = ld_dev(&D.unit_done[u]);
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

// byte offset of the single-layer record in the kernel arguments (after the table pointer)
constexpr int kOneArgOffset = (int)((sizeof(void*) + alignof(LayerArgs) - 1) / alignof(LayerArgs) * alignof(LayerArgs));

// The streaming launch: the work items of n_layers layers from the per-XCD
// queues (layers_item), with the layers' arguments from `table` (device
// memory) or, for a single layer, from `one`.
__global__ __launch_bounds__(kAttThreads, 2) void k_stream(const LayerArgs* __restrict__ table, LayerArgs one,
                                                           LayersArgs L) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ RouteShared<kAttWaves> rsh;
  __shared__ int32_t sh_item, sh_layer;
  __shared__ uint32_t sh_flag;
  const int tid = threadIdx.x;
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
  const int t = __builtin_amdgcn_readfirstlane(sh_item);
  // The layer's arguments stay in memory (the table, or the kernel-argument
  // segment, where `one` follows the 8-byte table pointer) and are read through
  // the constant address space: scalar loads when a field is used, rather than
  // a copy of the whole record in registers.
  typedef const __attribute__((address_space(4))) LayerArgs CLayer;
  typedef const __attribute__((address_space(4))) unsigned char CByte;
  CLayer* cla = table ? (CLayer*)table + __builtin_amdgcn_readfirstlane(sh_layer)
                      : (CLayer*)((CByte*)__builtin_amdgcn_kernarg_segment_ptr() + kOneArgOffset);
  const LayerArgs& la = *(const LayerArgs*)cla;
  if (t >= 0) stream_item(la.P, la.Bt, la.D, t, smem, rsh);
  // the last merge of the launch leaves every layer's control words zero
  if (t >= la.D.n_part_end) {
    __syncthreads();
    if (tid == 0)
      sh_flag = (atomicAdd(&L.ctrl[1], 1u) == (uint32_t)(L.n_layers * L.n_units * L.group - 1)) ? 1u : 0u;
    lds_barrier();
    if (sh_flag) {
      for (int l = 0; l < L.n_layers; ++l) {
        const DecodeArgs& D = table ? table[l].D : la.D;
        for (int i = tid; i < D.n_units; i += kAttThreads) D.unit_done[i] = 0u;
        for (int i = tid; i < D.n_route * D.att.top_k; i += kAttThreads) D.slots[i] = kSlotPending;  // 0
      }
      if (tid < kQueues) L.ctrl[kCtrlQueue + tid * kQueueStride] = 0u;
      if (tid == 0) L.ctrl[1] = 0u;
    }
  }
}

}  // namespace

// LDS bytes of the streaming attention parts (the routing and merge items of
// the launch may need more: the caller takes the maximum).
__attribute__((visibility("hidden"))) size_t dkv_stream_lds_bytes() { return (size_t)kSLdsTotal; }

// Launch the streaming decode (see k_stream); table == nullptr: one layer, `one`.
// The argument structs come as bytes: their types are private to each
// translation unit (both see the same definitions).
__attribute__((visibility("hidden"))) hipError_t dkv_stream_launch(const void* table, const void* one_bytes,
                                                                   const void* layers_bytes, int n_items, size_t lds,
                                                                   hipStream_t st) {
  LayerArgs one;
  LayersArgs L;
  memcpy(&one, one_bytes, sizeof(one));
  memcpy(&L, layers_bytes, sizeof(L));
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)k_stream, hipFuncAttributeMaxDynamicSharedMemorySize, 158 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_stream, dim3((unsigned)n_items), dim3(kAttThreads), lds, st, (const LayerArgs*)table, one, L);
  return hipGetLastError();
}
