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

constexpr int kSRowB = 272;                 // bytes per 128-wide fp16 row in LDS: 256 + one 16-byte pad
constexpr int kWRows = 16;                  // rows per page
constexpr int kWPage = kWRows * kSRowB;     // bytes per ring slot (a U page of 32 positions also fits)
constexpr int kWSlots = 4;                  // ring depth per wave
constexpr int kWRing = kWPage * kWSlots;    // one wave's ring
constexpr int kSMaxBlocks = 32;             // routed blocks per part at most
constexpr int kWQOff = kAttWaves * kWRing;  // the unit's query rows [16][128] fp16 (4 KB)
constexpr int kWPosOff = kWQOff + 16 * kD * 2;        // residual positions, per wave [4][128] bytes
constexpr int kWMaskOff = kWPosOff + kAttWaves * 128;  // residual-position masks, per wave [4][8] u32
constexpr int kWSlotOff = kWMaskOff + kAttWaves * 32; // the part's routed pool slots [kSMaxBlocks]
constexpr int kWNvOff = kWSlotOff + 4 * kSMaxBlocks;
constexpr int kWBaseOff = kWNvOff + 16;                 // per-block source addresses [kSMaxBlocks][kBases] u64
enum { kBaseAK = 0, kBaseAV, kBaseU, kBaseVK, kBaseVV, kBaseRK, kBaseRV, kBaseRP, kBases };
constexpr int kWLds = kWBaseOff + kSMaxBlocks * kBases * 8;
static_assert(kWLds % 16 == 0, "LDS areas are 16-byte aligned");
static_assert(32 * 2 * 56 + 16 <= kWPage, "a U page of 32 positions fits a slot");

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
  // n is the same on every lane: branch on a scalar.  The count's low four
  // bits sit in bits 0..3 of the immediate, its high two in bits 14..15;
  // expcnt and lgkmcnt are left at their maximum (no wait).
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: __builtin_amdgcn_s_waitcnt(0xf70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xf71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xf72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xf73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xf74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xf75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xf76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0xf77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0xf78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0xf79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0xf7a); break;
    case 11: __builtin_amdgcn_s_waitcnt(0xf7b); break;
    case 12: __builtin_amdgcn_s_waitcnt(0xf7c); break;
    case 13: __builtin_amdgcn_s_waitcnt(0xf7d); break;
    case 14: __builtin_amdgcn_s_waitcnt(0xf7e); break;
    case 15: __builtin_amdgcn_s_waitcnt(0xf7f); break;
    case 16: __builtin_amdgcn_s_waitcnt(0x4f70); break;
    case 17: __builtin_amdgcn_s_waitcnt(0x4f71); break;
    case 18: __builtin_amdgcn_s_waitcnt(0x4f72); break;
    case 19: __builtin_amdgcn_s_waitcnt(0x4f73); break;
    case 20: __builtin_amdgcn_s_waitcnt(0x4f74); break;
    case 21: __builtin_amdgcn_s_waitcnt(0x4f75); break;
    case 22: __builtin_amdgcn_s_waitcnt(0x4f76); break;
    case 23: __builtin_amdgcn_s_waitcnt(0x4f77); break;
    case 24: __builtin_amdgcn_s_waitcnt(0x4f78); break;
    case 25: __builtin_amdgcn_s_waitcnt(0x4f79); break;
    case 26: __builtin_amdgcn_s_waitcnt(0x4f7a); break;
    case 27: __builtin_amdgcn_s_waitcnt(0x4f7b); break;
    case 28: __builtin_amdgcn_s_waitcnt(0x4f7c); break;
    case 29: __builtin_amdgcn_s_waitcnt(0x4f7d); break;
    case 30: __builtin_amdgcn_s_waitcnt(0x4f7e); break;
    case 31: __builtin_amdgcn_s_waitcnt(0x4f7f); break;
    case 32: __builtin_amdgcn_s_waitcnt(0x8f70); break;
    case 33: __builtin_amdgcn_s_waitcnt(0x8f71); break;
    case 34: __builtin_amdgcn_s_waitcnt(0x8f72); break;
    case 35: __builtin_amdgcn_s_waitcnt(0x8f73); break;
    case 36: __builtin_amdgcn_s_waitcnt(0x8f74); break;
    case 37: __builtin_amdgcn_s_waitcnt(0x8f75); break;
    case 38: __builtin_amdgcn_s_waitcnt(0x8f76); break;
    case 39: __builtin_amdgcn_s_waitcnt(0x8f77); break;
    case 40: __builtin_amdgcn_s_waitcnt(0x8f78); break;
    case 41: __builtin_amdgcn_s_waitcnt(0x8f79); break;
    case 42: __builtin_amdgcn_s_waitcnt(0x8f7a); break;
    case 43: __builtin_amdgcn_s_waitcnt(0x8f7b); break;
    case 44: __builtin_amdgcn_s_waitcnt(0x8f7c); break;
    case 45: __builtin_amdgcn_s_waitcnt(0x8f7d); break;
    case 46: __builtin_amdgcn_s_waitcnt(0x8f7e); break;
    case 47: __builtin_amdgcn_s_waitcnt(0x8f7f); break;
    case 48: __builtin_amdgcn_s_waitcnt(0xcf70); break;
    case 49: __builtin_amdgcn_s_waitcnt(0xcf71); break;
    case 50: __builtin_amdgcn_s_waitcnt(0xcf72); break;
    case 51: __builtin_amdgcn_s_waitcnt(0xcf73); break;
    case 52: __builtin_amdgcn_s_waitcnt(0xcf74); break;
    case 53: __builtin_amdgcn_s_waitcnt(0xcf75); break;
    case 54: __builtin_amdgcn_s_waitcnt(0xcf76); break;
    case 55: __builtin_amdgcn_s_waitcnt(0xcf77); break;
    case 56: __builtin_amdgcn_s_waitcnt(0xcf78); break;
    case 57: __builtin_amdgcn_s_waitcnt(0xcf79); break;
    case 58: __builtin_amdgcn_s_waitcnt(0xcf7a); break;
    case 59: __builtin_amdgcn_s_waitcnt(0xcf7b); break;
    case 60: __builtin_amdgcn_s_waitcnt(0xcf7c); break;
    case 61: __builtin_amdgcn_s_waitcnt(0xcf7d); break;
    case 62: __builtin_amdgcn_s_waitcnt(0xcf7e); break;
    default: __builtin_amdgcn_s_waitcnt(0xcf7f); break;
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

// LDS reads of ring pages, written as inline asm that waits for its own
// reads before it ends (outputs early-clobber: a read that lands must not
// overwrite the address of the next): the compiler would otherwise wait for every load in
// flight to LDS (it cannot tell which slot they fill) before each LDS read,
// and the ring would drain at every page.  Addresses are LDS byte offsets.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// four 16-byte reads at a, a + 64, a + 128, a + 192
__device__ __forceinline__ void lds_b128x4(uint32_t a, v8h (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:64\n\t"
      "ds_read_b128 %2, %4 offset:128\n\t"
      "ds_read_b128 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a)
      : "memory");
}
// eight transposed 8-byte reads at a + 32 k (k = 0..7)
__device__ __forceinline__ void lds_tr8(uint32_t a, v4h (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:160\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a)
      : "memory");
}
// transposed 8-byte reads at a + 32 k and b + 32 k (k = 0..3)
__device__ __forceinline__ void lds_tr44(uint32_t a, uint32_t b, v4h (&o)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
      "ds_read_b64_tr_b16 %4, %9\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:32\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:64\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a), "v"(b)
      : "memory");
}
// plain 8-byte reads at a + 32 k and b + 32 k (k = 0..3)
__device__ __forceinline__ void lds_b64x44(uint32_t a, uint32_t b, v4h (&o)[8]) {
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %8 offset:32\n\t"
      "ds_read_b64 %2, %8 offset:64\n\t"
      "ds_read_b64 %3, %8 offset:96\n\t"
      "ds_read_b64 %4, %9\n\t"
      "ds_read_b64 %5, %9 offset:32\n\t"
      "ds_read_b64 %6, %9 offset:64\n\t"
      "ds_read_b64 %7, %9 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a), "v"(b)
      : "memory");
}
// two bytes at a and a + 64
__device__ __forceinline__ void lds_u8x2(uint32_t a, uint32_t& x, uint32_t& y) {
  asm volatile(
      "ds_read_u8 %0, %2\n\t"
      "ds_read_u8 %1, %2 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(a)
      : "memory");
}

// OR over the 64 lanes, returned to every lane
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp_u32<0xB1>(0u, v);        // quad_perm 1,0,3,2
  v |= dpp_u32<0x4E>(0u, v);        // quad_perm 2,3,0,1
  v |= dpp_u32<0x141>(0u, v);       // row_half_mirror
  v |= dpp_u32<0x140>(0u, v);       // row_mirror
  v |= dpp_u32<0x142, 0xa>(0u, v);  // row_bcast:15
  v |= dpp_u32<0x143, 0xc>(0u, v);  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ v4f mfma32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// byte offset of (row, 8-half chunk c) of a 128-wide fp16 page: rows of 17
// chunks (the last one padding), so that the 16 rows of an MFMA tile start in
// 16 different bank groups
__device__ __forceinline__ int swz(int row, int c) { return row * kSRowB + (c << 4); }

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

// The pages one wave streams.  A block: V_K tiles (16 rows of [V_K ; a_k] each,
// a_k at row r), 8 U pages of 32 positions, K and V tiles of 16 residual rows,
// V_V tiles (16 rows of [V_V ; a_v]).  A window share: K and V tiles of 16 rows.
enum PageKind { kPageVK = 0, kPageU = 1, kPageK = 2, kPageV = 3, kPageVV = 4 };

struct WaveGeom {
  int r, nq, nqv;  // rank, round16(r) / 16, round16(r + 1) / 16 (V_K / V_V tiles)
  int R, nt;       // residual rows (or the wave's window rows) and their 16-row tiles
  int ppb;         // pages of the wave's block (or window share)
  bool window;
};

__device__ __forceinline__ void page_kind(const WaveGeom& g, int k, int& kind, int& i) {
  if (g.window) {
    kind = kPageK + (k & 1);
    i = k >> 1;
    return;
  }
  if (k < g.nqv) {
    kind = kPageVK;
    i = k;
  } else if ((k -= g.nqv) < 8) {
    kind = kPageU;
    i = k;
  } else if ((k -= 8) < 2 * g.nt) {
    kind = kPageK + (k & 1);
    i = k >> 1;
  } else {
    kind = kPageVV;
    i = k - 2 * g.nt;
  }
}

// Issue the loads of page k of this wave's stream into its ring slot `dst`;
// returns the number of vector-memory instructions issued.  The loads are
// buffer loads straight into LDS: each source array is a buffer resource
// sized to its data, and every 16-byte chunk of the page whose offset falls
// outside it (row pads, rows past the data, U's leading zero row, the end of
// U) is written as zeros by the range check.  A 128-wide row page maps chunk p
// to row p / 17, chunk p % 17 (chunk 16 is the row's pad); a U page maps p
// linearly.  Row r of [V_K ; a_k] and [V_V ; a_v] comes from a load of its own.
// Per lane: the source offset of chunk 64 q + lane (q = 0..4) of a 128-wide
// row page (row p / 17, chunk p % 17 of the row; chunk 16, the row's pad, is
// kOutside), the same for every row page.
struct RowOffs {
  uint32_t off[5];
};

__device__ __forceinline__ RowOffs row_offs() {
  const int lane = threadIdx.x & 63;
  RowOffs o;
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int p = 64 * q + lane;
    const int row = (p * 3856) >> 16;  // p / 17 for p < 17 * 16 * 2
    const int c = p - 17 * row;
    o.off[q] = c < 16 ? (uint32_t)(row * 256 + 16 * c) : kOutside;
  }
  return o;
}

__device__ __forceinline__ int issue_page(const WaveGeom& g, int k, unsigned char* dst, const uint64_t* bb,
                                          const char* wk_rows, const char* wv_rows, unsigned char* posdst,
                                          const RowOffs& ro) {
  const int lane = threadIdx.x & 63;
  int kind, i;
  page_kind(g, k, kind, i);
  const int r = g.r;
  int ops = 0;
  if (kind == kPageU) {
    // positions 32 i .. 32 i + 31: U rows 32 i - 1 .. 32 i + 30 (row -1 reads
    // as zeros: the anchor), and 16 bytes more for the last row's column overrun
    const __amdgpu_buffer_rsrc_t rs = rsrc_of((const char*)bb[kBaseU], (uint32_t)(510 * r));
    const int nch = 4 * r + 1;
    const int start = (32 * i - 1) * 2 * r;
    for (int q = 0; q < nch; q += 64) {
      dma16b(rs, (uint32_t)(start + 16 * (q + lane)), dst + 16 * q);
      ++ops;
    }
    return ops;
  }
  const char* base;
  int nvalid, special = -1;
  if (kind == kPageVK || kind == kPageVV) {
    base = (const char*)bb[kind == kPageVK ? kBaseVK : kBaseVV] + 16 * i * 256;
    nvalid = r - 16 * i;
    nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
    special = r - 16 * i;
    if (special > 15) special = -1;
  } else {
    const int rem = g.R - 16 * i;
    nvalid = rem < 16 ? rem : 16;
    if (g.window)
      base = (kind == kPageK ? wk_rows : wv_rows) + 16 * i * 256;
    else
      base = (const char*)bb[kind == kPageK ? kBaseRK : kBaseRV] + 16 * i * 256;
  }
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base, (uint32_t)nvalid * 256u);
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    // chunks past the page's 17 * 16 (lanes 16.. of the last load) are not loaded;
    // a pad chunk's offset (kOutside) has no row that equals `special`
    const uint32_t off = ro.off[q];
    if ((q < 4 || lane < 16) && (int)(off >> 8) != special) dma16b(rs, off, dst + 1024 * q);
    ++ops;
  }
  if (special >= 0) {
    const __amdgpu_buffer_rsrc_t rs1 = rsrc_of((const char*)bb[kind == kPageVK ? kBaseAK : kBaseAV], 256u);
    if (lane < 17) dma16b(rs1, lane < 16 ? (uint32_t)(16 * lane) : kOutside, dst + kSRowB * special);
    ++ops;
  }
  if (kind == kPageVK && i == 0 && g.R > 0) {
    // the block's residual positions: R bytes as R / 4 dwords (R % 4 == 0)
    const __amdgpu_buffer_rsrc_t rp = rsrc_of((const char*)bb[kBaseRP], (uint32_t)g.R);
    if (4 * lane < g.R) dma4b(rp, (uint32_t)(4 * lane), posdst);
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

// q~ (or W^T) tile number i of a four-tile register array, i uniform
template <class T>
__device__ __forceinline__ T pick4(const T (&a)[4], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : (i == 2 ? a[2] : a[3]));
}

// One page of a wave's stream: the work of page kind `kind`, number i, held in
// LDS at pg (the wave's own ring slot).  st and the per-block values (q~ as hi +
// lo, q . a_k, the block's low-rank weight sum, the current K tile's weights)
// carry over from page to page.
struct BlockRegs {
  v4h qth[4], qtl[4];  // scaled V_K q of the block (hi + lo fp16): rows 16 k + 4 q4 + e, head l16
  float qa;            // scale * q . a_k
  float llr_tot;       // the block's low-rank weight sum per head (at its first V_V tile)
  v4h pv;              // weights of the current K tile (fp16), for its V tile
  uint32_t mw[8];      // the block's residual-position mask (bit p of word p / 32: position p)
};

// The page kinds' work.  P0: the page's LDS byte address (the wave's own ring
// slot); i: the page's number within its kind.  st and br carry over from page
// to page.  With i a compile-time constant every register array index folds.

// V_K q rows 16 i .. 16 i + 15 (q . a_k at row r); page 0 also turns the
// block's residual positions (bytes at LDS address posb) into the mask words.
__device__ __forceinline__ void page_vk(const WaveGeom& g, int i, uint32_t P0, const v8h (&qf)[4], BlockRegs& br,
                                        float scale, uint32_t posb) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4;
  const int r = g.r;
  v8h a[4];
  lds_b128x4(P0 + l16 * kSRowB + 16 * q4, a);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) acc = mfma32(a[s2], qf[s2], acc);
  v4f x;
  float qr = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 16 * i + 4 * q4 + e;
    x[e] = j < r ? acc[e] * scale : 0.f;
    qr += j == r ? acc[e] * scale : 0.f;
  }
  v4h hi, lo;
  split4(x, hi, lo);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    br.qth[k] = k == i ? hi : br.qth[k];
    br.qtl[k] = k == i ? lo : br.qtl[k];
  }
  if (16 * i <= r && r < 16 * i + 16) br.qa = hq_sum(qr);
  if (i == 0) {
    uint32_t p1 = 0u, p2 = 0u;
    lds_u8x2(posb + lane, p1, p2);
    p1 = lane < g.R ? p1 : 0u;
    p2 = lane + 64 < g.R ? p2 : 0u;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t v = ((p1 >> 5) == (uint32_t)w && p1 >= 1u ? 1u << (p1 & 31) : 0u) |
                         ((p2 >> 5) == (uint32_t)w && p2 >= 1u ? 1u << (p2 & 31) : 0u);
      br.mw[w] = wave_or(v);
    }
  }
}

// U page i: positions 32 i + 16 tt + row (row 0 of page 0 is the anchor):
// low-rank scores, then W^T += Ux^T p over the page's 32 positions.
__device__ __forceinline__ void page_u(const WaveGeom& g, int i, uint32_t P0, SState& st, BlockRegs& br) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4, s4 = l16 & 3;
  const int r = g.r;
  const uint32_t mw = i == 0 ? br.mw[0] : i == 1 ? br.mw[1] : i == 2 ? br.mw[2] : i == 3 ? br.mw[3]
                    : i == 4 ? br.mw[4] : i == 5 ? br.mw[5] : i == 6 ? br.mw[6] : br.mw[7];
  v4h ua[8];  // [tt * 4 + k]: U rows 16 tt + l16, columns 16 k + 4 q4 .. + 3
  const uint32_t a0 = P0 + 2 * (l16 * r + 4 * q4);
  lds_b64x44(a0, a0 + 32 * r, ua);
  float z[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < g.nq) {
        acc = mfma16(ua[4 * tt + k], br.qth[k], acc);
        acc = mfma16(ua[4 * tt + k], br.qtl[k], acc);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool masked = ((mw >> (16 * tt + 4 * q4 + e)) & 1u) != 0u;
      z[4 * tt + e] = masked ? -INFINITY : acc[e] + br.qa;
    }
  }
  softmax_step<8>(st, z, true);
  v8h pf;
#pragma unroll
  for (int e = 0; e < 8; ++e) pf[e] = (f16)z[e];
  v4h ut[8];  // [k], [4 + k]: transposed U of rows 4 q4 .., 16 + 4 q4 .., columns 16 k + l16
  const uint32_t b0 = P0 + 2 * ((4 * q4 + (l16 >> 2)) * r + 4 * s4);
  lds_tr44(b0, b0 + 32 * r, ut);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < g.nq) {
      const v8h a = __builtin_shufflevector(ut[k], ut[4 + k], 0, 1, 2, 3, 4, 5, 6, 7);
      st.Wt[k] = mfma32(a, pf, st.Wt[k]);
    }
  }
}

// K page i: scores of residual (or window) rows 16 i .. 16 i + 15.
__device__ __forceinline__ void page_k(const WaveGeom& g, int i, uint32_t P0, SState& st, const v8h (&qf)[4],
                                       BlockRegs& br, float scale) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4;
  const int nr = g.R - 16 * i;
  v8h a[4];
  lds_b128x4(P0 + l16 * kSRowB + 16 * q4, a);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) acc = mfma32(a[s2], qf[s2], acc);
  float z[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = (4 * q4 + e < nr) ? acc[e] * scale : -INFINITY;
  softmax_step<4>(st, z, false);
  br.pv = to_h4v(z[0], z[1], z[2], z[3]);
}

// V page: O^T += V^T p of the K page before it.
__device__ __forceinline__ void page_v(uint32_t P0, SState& st, const BlockRegs& br) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4, s4 = l16 & 3;
  v4h a[8];
  lds_tr8(P0 + (4 * q4 + (l16 >> 2)) * kSRowB + 16 * (s4 >> 1) + 8 * (s4 & 1), a);
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = mfma16(a[nn], br.pv, st.Ot[nn]);
}

// V_V page i: O^T += [V_V ; a_v]^T rows 16 i .. 16 i + 15 times W^T rows (row
// r of W^T: the block's low-rank weight sum, for a_v).
__device__ __forceinline__ void page_vv(const WaveGeom& g, int i, uint32_t P0, SState& st, BlockRegs& br) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4, s4 = l16 & 3;
  const int r = g.r;
  if (i == 0) {
    br.llr_tot = hq_sum(st.llr);
    st.llr = 0.f;
  }
  v4f x = pick4(st.Wt, i);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 16 * i + 4 * q4 + e;
    x[e] = j < r ? x[e] : (j == r ? br.llr_tot : 0.f);
  }
  v4h wh, wlo;
  split4(x, wh, wlo);
  v4h a[8];
  lds_tr8(P0 + (4 * q4 + (l16 >> 2)) * kSRowB + 16 * (s4 >> 1) + 8 * (s4 & 1), a);
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = mfma16(a[nn], wlo, mfma16(a[nn], wh, st.Ot[nn]));
  if (i == g.nqv - 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
  }
}

// One page of a wave's stream, of any kind (kind and i at run time).
__device__ __forceinline__ void compute_page(const WaveGeom& g, int kind, int i, const unsigned char* pg, SState& st,
                                             const v8h (&qf)[4], BlockRegs& br, float scale,
                                             const unsigned char* posb) {
  const uint32_t P0 = lds_off(pg);
  if (kind == kPageVK)
    page_vk(g, i, P0, qf, br, scale, lds_off(posb));
  else if (kind == kPageU)
    page_u(g, i, P0, st, br);
  else if (kind == kPageK)
    page_k(g, i, P0, st, qf, br, scale);
  else if (kind == kPageV)
    page_v(P0, st, br);
  else
    page_vv(g, i, P0, st, br);
}


// One attention part of unit u: part p < n_block_parts holds routed ranks
// [p * bpi, min((p + 1) * bpi, top_k)), at most four: wave w streams block w.
// The other parts are window chunks of win_chunk rows: wave w streams rows
// [w c / 4, (w + 1) c / 4) of the chunk.  Each wave keeps its own softmax state
// over its rows; the four states are combined at the end into the part's
// partial.
__device__ __forceinline__ void stream_part(const PoolArgs& P, const BatchArgs& Bt, const AttnArgs& A,
                                            const int32_t* slots, uint32_t* ctrl, int u, int p, unsigned char* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int b = u / Bt.Hkv, h = u % Bt.Hkv;
  const int G = Bt.G;
  const int row0 = b * Bt.Hq + h * G;
  const int part = A.part_offset + p;
  int32_t* slist = reinterpret_cast<int32_t*>(smem + kWSlotOff);
  int32_t* shn = reinterpret_cast<int32_t*>(smem + kWNvOff);
  uint64_t* bases = reinterpret_cast<uint64_t*>(smem + kWBaseOff);

  WaveGeom g;
  g.r = P.rank;
  g.nq = round16(P.rank) >> 4;
  g.nqv = round16(P.rank + 1) >> 4;
  g.window = p >= A.n_block_parts;
  int nv = 0, wrow0 = 0, wrows = 0;
  if (!g.window) {
    // the part's routed slots, waited for (bounded) until the routing wrote them
    const int k0 = p * A.blocks_per_item;
    const int kn = (A.top_k - k0 < A.blocks_per_item ? A.top_k - k0 : A.blocks_per_item);
    if (wave == 0) {
      int32_t slot = -1;
      if (lane < kn) {
        const int32_t* sp = &slots[(int64_t)u * A.top_k + k0 + lane];
        const uint32_t tag = slot_tag(ld_dev(&ctrl[3]));
        unsigned n = 0;
        int32_t v = ld_dev(sp);
        while (!slot_ready(v, tag) && n < kRouteWaitLimit) {
          __builtin_amdgcn_s_sleep(1);
          v = ld_dev(sp);
          ++n;
        }
        if (!slot_ready(v, tag)) {
          atomicOr(&ctrl[2], 1u);
          v = (int32_t)(tag | (uint32_t)(-1 + kSlotCode));
        }
        slot = slot_value(v);
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
    g.R = P.n_resid;
  } else {
    const int s = p - A.n_block_parts;
    int wl = Bt.wlen ? Bt.wlen[b] : Bt.W;
    wl = wl < 0 ? 0 : (wl > Bt.W ? Bt.W : wl);
    const int start = s * A.win_chunk;
    const int end = (start + A.win_chunk < wl) ? start + A.win_chunk : wl;
    const int rows = end > start ? end - start : 0;
    // wave w: a quarter of the chunk, in whole 16-row tiles
    const int per = (((A.win_chunk + kAttWaves - 1) / kAttWaves) + 15) & ~15;
    wrow0 = start + per * wave;
    const int lim = rows - per * wave;
    wrows = lim < 0 ? 0 : (lim > per ? per : lim);
    g.R = wrows;
    nv = rows > 0 ? 1 : 0;
  }
  g.nt = (g.R + 15) >> 4;
  if (nv == 0) {
    store_empty(A, row0, G, part);
    return;
  }
  g.ppb = g.window ? 2 * g.nt : 2 * g.nqv + 8 + 2 * g.nt;
  const bool mine = g.window ? wrows > 0 : wave < nv;   // uniform over the wave
  const int total = mine ? g.ppb : 0;
  const int64_t win_base = (((int64_t)b * Bt.Hkv + h) * Bt.W) * kD;
  const char* wk_rows = (const char*)(Bt.wk + win_base + (int64_t)wrow0 * kD);
  const char* wv_rows = (const char*)(Bt.wv + win_base + (int64_t)wrow0 * kD);

  // ---- the blocks' source addresses and the query rows, once per part
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
  unsigned char* qrows = smem + kWQOff;
  {
    const int hh = tid >> 4, c = tid & 15;
    const void* src = hh < G ? (const void*)(Bt.q + (int64_t)(row0 + hh) * kD + 8 * c) : (const void*)kZeroChunk;
    dma16(src, qrows + 1024 * wave);
  }
  lds_barrier();  // the source addresses are in place (the query rows are still in flight)

  // ---- this wave's stream: pages through its own ring, kWSlots - 1 ahead
  unsigned char* ring = smem + wave * kWRing;
  unsigned char* posb = smem + kWPosOff + 128 * wave;
  const uint64_t* bb = bases + (g.window ? 0 : wave) * kBases;
  SState st;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.Ot[n] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  st.llr = 0.f;
  const float scale = A.scale;
  // the first pages, then the query rows (loaded before them) once every wave has its share
  int n_issued = 0;
  const RowOffs ro = row_offs();
  uint32_t in_flight = 0u;  // this wave's load counts of the pages issued and not yet waited for (bytes, oldest low)
  for (; n_issued < kWSlots - 1 && n_issued < total; ++n_issued)
    in_flight |= (uint32_t)issue_page(g, n_issued, ring + kWPage * n_issued, bb, wk_rows, wv_rows, posb, ro)
                 << (8 * n_issued);
  wait_vm((int)((in_flight & 0xFFu) + ((in_flight >> 8) & 0xFFu) + (in_flight >> 16)));
  lds_barrier();
  v8h qf[4];  // q[head = l16][32 s + 8 q4 + 0..7], the B operand of the d-contractions
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const v8h*>(qrows + l16 * 256 + 64 * s + 16 * q4);

  if (total > 0) {
    const int r = g.r;
    BlockRegs br;
    br.qa = 0.f;
    br.llr_tot = 0.f;
    for (int n = 0; n < total; ++n) {
      const uint32_t after = in_flight >> 8;
      wait_vm((int)((after & 0xFFu) + ((after >> 8) & 0xFFu) + (after >> 16)));
      in_flight = after;
      if (n_issued < total) {
        in_flight |= (uint32_t)issue_page(g, n_issued, ring + kWPage * (n_issued % kWSlots), bb, wk_rows, wv_rows,
                                          posb, ro)
                     << (8 * (n_issued - n - 1));
        ++n_issued;
      }
      const unsigned char* pg = ring + kWPage * (n % kWSlots);
      int kind, i;
      page_kind(g, n, kind, i);
      compute_page(g, kind, i, pg, st, qf, br, scale, posb);
    }
  }

  // ---- the four waves' states at their common maximum, summed in wave order
  lds_barrier();  // every wave is done with its ring
  float* red = reinterpret_cast<float*>(smem);                    // [4 waves][16 heads][132]
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
    route_unit<kAttThreads>(P, Bt, t, D.att.top_k, D.idx, nullptr, D.slots, reinterpret_cast<uint32_t*>(smem), rsh,
                            slot_tag(ld_dev(&D.ctrl[3])));
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
  // The last merge of the launch leaves every layer's control words zero; a
  // launch without merges (routings and window parts only, ahead of the block
  // streams) counts every item instead.
  const bool counted = L.group > 0 ? t >= la.D.n_part_end : t >= 0;
  const uint32_t n_counted = (uint32_t)(L.n_layers * L.n_units *
                                        (L.group > 0 ? L.group : L.routes + L.block_parts + L.win_parts));
  if (counted) {
    __syncthreads();
    if (tid == 0) sh_flag = (atomicAdd(&L.ctrl[1], 1u) == n_counted - 1u) ? 1u : 0u;
    lds_barrier();
    if (sh_flag) {
      for (int l = 0; l < L.n_layers; ++l) {
        const DecodeArgs& D = table ? table[l].D : la.D;
        for (int i = tid; i < D.n_units; i += kAttThreads) D.unit_done[i] = 0u;
      }
      if (tid < kQueues) L.ctrl[kCtrlQueue + tid * kQueueStride] = 0u;
      if (tid == 0) {
        L.ctrl[1] = 0u;
        // the next launch's routed-slot tag (with block streams, the merge launch
        // that ends the step advances it)
        if (L.group > 0) L.ctrl[3] = L.ctrl[3] + 1u;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streams: after the routing of a step has run, each one-wave workgroup
// streams a contiguous segment of the step's work (every unit's window rows
// and routed blocks, cut on the host into segments of equal bytes) through its
// LDS ring.  No item waits on another: the routing finished in an earlier
// launch.
// ---------------------------------------------------------------------------

struct BlocksArgs {
  const LayerArgs* table;
  const int32_t* sched;  // the step's schedule (see k_blocks)
  const uint32_t* ctrl;  // the step's control header (word 3: the routed-slot tag of this step)
  int n_waves;
  int top_k;
};

constexpr int kBPosOff = kWRing;                 // residual positions [128] bytes
constexpr int kBBaseOff = kBPosOff + 128;        // the issuing item's source addresses [kBases] u64
constexpr int kBLds = kBBaseOff + kBases * 8;

typedef const __attribute__((address_space(4))) int32_t CInt;
typedef const __attribute__((address_space(4))) uint32_t CUint;
typedef const __attribute__((address_space(4))) LayerArgs CLayerArgs;

// What one side of a stream needs to know about a work item.
struct SItem {
  WaveGeom g;
  int npages;        // pages of the item's stream: the unit's query rows first if it opens a run
  int kind, first, last;
  int G, row0, part; // the unit's query rows row0 .. row0 + G - 1; the run's partial index
  int layer, h;
  int64_t slot;      // block items: the routed pool slot, or -1 (nothing to stream)
  const char* rows_k;  // window and residual items: their first key and value rows
  const char* rows_v;
};

__device__ __forceinline__ SItem sched_item(const BlocksArgs& A, CInt* item, uint32_t tag) {
  const uint32_t w0 = ((CUint*)item)[0], w1 = ((CUint*)item)[1], w2 = ((CUint*)item)[2], w3 = ((CUint*)item)[3];
  SItem it;
  it.layer = (int)(w0 & 0xFFFFu);
  it.kind = (int)((w0 >> 16) & 0xFFu);
  it.first = (int)((w0 >> 24) & 1u);
  it.last = (int)((w0 >> 25) & 1u);
  const int b = (int)(w2 & 0xFFFFu), h = (int)(w2 >> 16);
  it.part = (int)(w3 & 0xFFFFu);
  const int nrows = (int)(w3 >> 16);
  const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)A.table + it.layer);
  const PoolArgs& P = la.P;
  const int Hkv = la.Bt.Hkv, G = la.Bt.G;
  it.h = h;
  it.G = G;
  it.row0 = b * la.Bt.Hq + h * G;
  it.g.r = P.rank;
  it.g.nq = round16(P.rank) >> 4;
  it.g.nqv = round16(P.rank + 1) >> 4;
  it.slot = -1;
  it.rows_k = nullptr;
  it.rows_v = nullptr;
  int pages;
  if (it.kind == kItemWin) {
    // window rows row0 .. row0 + nrows - 1, as far as the row's window reaches
    const int r0 = (int)w1;
    int wl = la.Bt.wlen ? ((CInt*)la.Bt.wlen)[b] : la.Bt.W;
    wl = wl < 0 ? 0 : (wl > la.Bt.W ? la.Bt.W : wl);
    int rows = wl - r0;
    rows = rows < 0 ? 0 : (rows > nrows ? nrows : rows);
    const int64_t base = (((int64_t)b * Hkv + h) * la.Bt.W + r0) * kD;
    it.rows_k = (const char*)(la.Bt.wk + base);
    it.rows_v = (const char*)(la.Bt.wv + base);
    it.g.window = true;
    it.g.R = rows;
    it.g.nt = (rows + 15) >> 4;
    pages = 2 * it.g.nt;
  } else {
    const int rank = (int)(w1 & 0xFFFFu);
    const int unit = b * Hkv + h;
    const int32_t w = ((CInt*)la.D.slots)[(int64_t)unit * A.top_k + rank];  // a scalar load
    int64_t slot = slot_ready(w, tag) ? slot_value(w) : -1;
    if (slot >= P.n_slots) slot = -1;
    it.slot = slot;
    if (it.kind == kItemLowRank) {
      it.g.window = false;
      it.g.R = P.n_resid;
      it.g.nt = 0;
      pages = slot >= 0 ? 2 * it.g.nqv + 8 : 0;
    } else {
      const int r0 = (int)(w1 >> 16);
      it.g.window = true;
      it.g.R = slot >= 0 ? nrows : 0;
      it.g.nt = (it.g.R + 15) >> 4;
      if (slot >= 0) {
        it.rows_k = (const char*)(P.rk + slot * P.rk_s + h * P.rk_h + (int64_t)r0 * kD);
        it.rows_v = (const char*)(P.rv + slot * P.rv_s + h * P.rv_h + (int64_t)r0 * kD);
      }
      pages = 2 * it.g.nt;
    }
  }
  it.g.ppb = pages;
  it.npages = it.first + pages;
  return it;
}

// the source addresses of the low-rank item an issuing stream enters, into its LDS
__device__ __forceinline__ void item_bases(const BlocksArgs& A, const SItem& it, uint64_t* bases) {
  const int lane = threadIdx.x & 63;
  const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)A.table + it.layer);
  const PoolArgs& P = la.P;
  const int h = it.h;
  const int64_t slot = it.slot;
  if (lane < kBases) {
    const void* a;
    switch (lane) {
      case kBaseAK: a = P.ak + slot * P.ak_s + h * P.ak_h; break;
      case kBaseAV: a = P.av + slot * P.av_s + h * P.av_h; break;
      case kBaseU: a = P.u + slot * P.u_s + h * P.u_h; break;
      case kBaseVK: a = P.vk + slot * P.vk_s + h * P.vk_h; break;
      case kBaseVV: a = P.vv + slot * P.vv_s + h * P.vv_h; break;
      case kBaseRK: a = P.rk + slot * P.rk_s + h * P.rk_h; break;
      case kBaseRV: a = P.rv + slot * P.rv_s + h * P.rv_h; break;
      default: a = P.rp + slot * P.rp_s + h * P.rp_h; break;
    }
    bases[lane] = (uint64_t)a;
  }
  wave_sync_lds();
}

// Issue page k of item `it` (page 0 of an item that opens a run: the unit's
// query rows, 16 rows of 256 bytes, rows past G zero).
__device__ __forceinline__ int issue_item_page(const BlocksArgs& A, const SItem& it, int k, unsigned char* dst,
                                               const uint64_t* bases, unsigned char* posb, const RowOffs& ro) {
  if (it.first && k == 0) {
    const int lane = threadIdx.x & 63;
    const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)A.table + it.layer);
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(la.Bt.q + (int64_t)it.row0 * kD, (uint32_t)(it.G * 256));
#pragma unroll
    for (int q = 0; q < 256; q += 64) dma16b(rs, (uint32_t)(16 * (q + lane)), dst + 16 * q);
    return 4;
  }
  return issue_page(it.g, k - it.first, dst, bases, it.rows_k, it.rows_v, posb, ro);
}

// The issuing side of a wave's stream: its pages, in order, into the ring's
// kWSlots slots; in_flight holds the vector-memory operation counts of the
// pages in flight, one byte each, byte 0 the oldest (the next to be used).
struct Issuer {
  SItem it;        // the item being issued
  int ii, ik;      // its index in the wave's list, its next page
  int i1;          // the end of the list
  int n_issued, total;
  uint32_t in_flight;
};

// enter item ii of the list (items without pages are passed over)
__device__ __forceinline__ void issuer_enter(const BlocksArgs& A, CInt* items, uint32_t tag, Issuer& S,
                                             uint64_t* bases) {
  for (; S.ii < S.i1; ++S.ii) {
    S.it = sched_item(A, items + 4 * S.ii, tag);
    if (S.it.npages > 0) break;
  }
  S.ik = 0;
  if (S.ii < S.i1 && S.it.kind == kItemLowRank && S.it.slot >= 0) item_bases(A, S.it, bases);
}

// issue the stream's next page, if any; n_next: the oldest page not yet used
__device__ __forceinline__ void issue_next(const BlocksArgs& A, CInt* items, uint32_t tag, Issuer& S, int n_next,
                                           unsigned char* ring, uint64_t* bases, unsigned char* posb,
                                           const RowOffs& ro) {
  if (S.n_issued >= S.total) return;
  const int ops = issue_item_page(A, S.it, S.ik, ring + kWPage * (S.n_issued & (kWSlots - 1)), bases, posb, ro);
  S.in_flight |= (uint32_t)ops << (8 * (S.n_issued - n_next));
  ++S.n_issued;
  if (++S.ik == S.it.npages) {
    ++S.ii;
    issuer_enter(A, items, tag, S, bases);
  }
}

// wait until the oldest page in flight has landed (in-order completion of the
// counted operations: the newer ones may still be in flight)
__device__ __forceinline__ void wait_oldest(uint32_t in_flight) {
  const uint32_t a = in_flight >> 8;
  wait_vm((int)((a & 0xFFu) + ((a >> 8) & 0xFFu) + (a >> 16)));
}

// Vector-memory operations of a run's partial store (eight 16-byte stores of
// o and one of the lse per lane, in inline asm so that the count is exact).
constexpr int kPartialStoreOps = 9;

// The streams of a decode step: wave w runs the schedule's items sched[w] ..
// sched[w + 1] - 1 (window rows of a unit, the low-rank part of a routed block,
// or residual rows of one) as one stream of pages through its ring: the next
// item's first pages load while the current item's last ones are used.  The
// wave's consecutive items of one unit (a run) share one attention state and
// leave one partial; its store joins the count of operations in flight
// instead of draining it.  An item's pages come in a fixed order, so the work
// of each page kind runs in a loop of its own.
//
// Schedule layout (int32 words): [n_waves + 1] item offsets per wave, then
// the items (four words each, see kItemWin), then the partial count of each
// (layer, unit).
__global__ __launch_bounds__(64, 2) void k_blocks(BlocksArgs A) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x, l16 = lane & 15, q4 = lane >> 4;
  CInt* sched = (CInt*)A.sched;  // scalar loads: the schedule is the same for the whole wave
  const int i0 = sched[blockIdx.x], i1 = sched[blockIdx.x + 1];
  if (i0 >= i1) return;
  CInt* items = sched + A.n_waves + 1;
  const uint32_t tag = slot_tag(((CUint*)A.ctrl)[3]);
  unsigned char* ring = smem;
  unsigned char* posb = smem + kBPosOff;
  uint64_t* bases = reinterpret_cast<uint64_t*>(smem + kBBaseOff);
  const uint32_t ring0 = lds_off(ring), posb0 = lds_off(posb);
  const RowOffs ro = row_offs();

  Issuer S;
  S.total = 0;
  for (int j = i0; j < i1; ++j) S.total += sched_item(A, items + 4 * j, tag).npages;
  S.ii = i0;
  S.i1 = i1;
  S.n_issued = 0;
  S.in_flight = 0u;
  issuer_enter(A, items, tag, S, bases);
#pragma unroll 1
  for (int k = 0; k < kWSlots; ++k) issue_next(A, items, tag, S, 0, ring, bases, posb, ro);

  SState st;
  BlockRegs br;
  v8h qf[4];
  int n = 0;  // the next page to use
  for (int ci = i0; ci < i1; ++ci) {
    const SItem cur = sched_item(A, items + 4 * ci, tag);
    const WaveGeom& g = cur.g;
    const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)A.table + cur.layer);
    const float scale = la.D.att.scale;
    if (cur.first) {
      // a new run: the unit's query rows, a fresh state
      wait_oldest(S.in_flight);
      lds_b128x4(ring0 + kWPage * (n & (kWSlots - 1)) + l16 * 256 + 16 * q4, qf);
      S.in_flight >>= 8;
      issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      st.l = 0.f;
      st.llr = 0.f;
    }
    if (cur.kind == kItemLowRank) {
      if (cur.slot >= 0) {
        br.qa = 0.f;
        br.llr_tot = 0.f;
        for (int i = 0; i < g.nqv; ++i) {
          wait_oldest(S.in_flight);
          page_vk(g, i, ring0 + kWPage * (n & (kWSlots - 1)), qf, br, scale, posb0);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
        }
        for (int i = 0; i < 8; ++i) {
          wait_oldest(S.in_flight);
          page_u(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, br);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
        }
        for (int i = 0; i < g.nqv; ++i) {
          wait_oldest(S.in_flight);
          page_vv(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, br);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
        }
      }
    } else {
      for (int i = 0; i < g.nt; ++i) {
        wait_oldest(S.in_flight);
        page_k(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, qf, br, scale);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
        wait_oldest(S.in_flight);
        page_v(ring0 + kWPage * (n & (kWSlots - 1)), st, br);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, ring, bases, posb, ro);
      }
    }
    if (cur.last) {
      // the run's partial: o normalised, lse (every lane of a head writes the
      // same lse).  G >= 1, so lane 0 always stores and every store issues.
      const int np = la.D.att.n_parts;
      const float lt = hq_sum(st.l);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? st.m + __logf(lt) : -INFINITY;
      if (l16 < cur.G) {
        float* po = la.D.att.part_o + ((int64_t)(cur.row0 + l16) * np + cur.part) * kD + 4 * q4;
        float* pl = la.D.att.part_lse + (int64_t)(cur.row0 + l16) * np + cur.part;
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
          const v4f v = st.Ot[nn] * inv;
          // (one wait state before the store data registers may be rewritten)
          asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" : : "v"(po + 16 * nn), "v"(v) : "memory");
        }
        asm volatile("global_store_dword %0, %1, off\n\ts_nop 1" : : "v"(pl), "v"(lse) : "memory");
      }
      // the stores count as part of the newest page in flight: waiting for an
      // older page then also allows for them, waiting for that page waits for them
      if (S.n_issued > n) S.in_flight += (uint32_t)kPartialStoreOps << (8 * (S.n_issued - 1 - n));
    }
  }
}

// The log-sum-exp merges of a step: one workgroup per (layer, unit), a wave
// per query row (rows w, w + 4, ...), two columns per lane.  The unit's
// partials are its runs', in run order; n_parts[layer * n_units + unit] of
// them.  The sum runs in part order, so the result does not depend on timing.
__global__ __launch_bounds__(kAttThreads) void k_merges(const LayerArgs* __restrict__ table, int n_units,
                                                        const int32_t* __restrict__ unit_parts, uint32_t* ctrl) {
  const int layer = blockIdx.x / n_units, u = blockIdx.x - layer * n_units;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)table + layer);
  const int b = u / la.Bt.Hkv, h = u - b * la.Bt.Hkv;
  const int G = la.Bt.G, row0 = b * la.Bt.Hq + h * G;
  const int stride = la.D.att.n_parts;
  const int np = ((CInt*)unit_parts)[blockIdx.x];
  for (int g = wave; g < G; g += kAttWaves) {
    const int row = row0 + g;
    const float* lse = la.D.att.part_lse + (int64_t)row * stride;
    const float* po = la.D.att.part_o + (int64_t)row * stride * kD + 2 * lane;
    float m = -INFINITY;
    for (int p = lane; p < np; p += 64) m = fmaxf(m, lse[p]);
    m = wave_minmax<true>(m);
    float2 acc = make_float2(0.f, 0.f);
    float S = 0.f;
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int p = p0 + lane;
      const float lp = p < np ? lse[p] : -INFINITY;
      const float wl = lp != -INFINITY ? __expf(lp - m) : 0.f;
      const int cnt = np - p0 < 64 ? np - p0 : 64;
      for (int k0 = 0; k0 < cnt; k0 += 8) {
        float2 o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int kk = k0 + k < cnt ? k0 + k : cnt - 1;
          o[k] = *reinterpret_cast<const float2*>(po + (int64_t)(p0 + kk) * kD);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float w = k0 + k < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k0 + k)) : 0.f;
          S += w;
          acc.x += w * o[k].x;
          acc.y += w * o[k].y;
        }
      }
    }
    const bool any = S > 0.f;
    const float inv = any ? 1.f / S : 0.f;
    typedef f16 v2h __attribute__((ext_vector_type(2)));
    v2h r2;
    r2[0] = (f16)(acc.x * inv);
    r2[1] = (f16)(acc.y * inv);
    *reinterpret_cast<v2h*>(la.D.out + (int64_t)row * kD + 2 * lane) = r2;
    if (lane == 0) la.D.out_lse[row] = any ? m + __logf(S) : -INFINITY;
  }
  // the last workgroup advances the step's routed-slot tag (the launch order
  // makes every earlier reader done with it)
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) ctrl[3] = ctrl[3] + 1u;
}

}  // namespace

// LDS bytes of the streaming attention parts (the routing and merge items of
// the launch may need more: the caller takes the maximum).
__attribute__((visibility("hidden"))) size_t dkv_stream_lds_bytes() { return (size_t)kWLds; }

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

// One decode step of several layers as three launches on `st`: the routings
// (k_stream), the streams (k_blocks), the merges (k_merges).  layers_a: the
// LayersArgs of the first launch; sched: the step's schedule in device memory
// (see k_blocks), with n_waves streams, over n_layers * n_units units.
__attribute__((visibility("hidden"))) hipError_t dkv_stream_step(const void* table, const void* layers_a_bytes,
                                                                 int n_items_a, size_t lds_a, const int32_t* sched,
                                                                 int n_waves, int n_sched_items, int top_k,
                                                                 int n_layers, int n_units, hipStream_t st) {
  LayerArgs none;
  memset(&none, 0, sizeof(none));
  hipError_t e = dkv_stream_launch(table, &none, layers_a_bytes, n_items_a, lds_a, st);
  if (e != hipSuccess) return e;
  LayersArgs L;
  memcpy(&L, layers_a_bytes, sizeof(L));
  BlocksArgs B;
  B.table = (const LayerArgs*)table;
  B.sched = sched;
  B.ctrl = L.ctrl;
  B.n_waves = n_waves;
  B.top_k = top_k;
  if (n_waves > 0) {
    hipLaunchKernelGGL(k_blocks, dim3((unsigned)n_waves), dim3(64), (size_t)kBLds, st, B);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int32_t* unit_parts = sched + (n_waves + 1) + 4 * (int64_t)n_sched_items;
  hipLaunchKernelGGL(k_merges, dim3((unsigned)(n_layers * n_units)), dim3(kAttThreads), 0, st,
                     (const LayerArgs*)table, n_units, unit_parts, L.ctrl);
  return hipGetLastError();
}
