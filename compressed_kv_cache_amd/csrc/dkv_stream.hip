// dkv_stream.hip -- the layer-batched streaming decode step of libdkv_attn
// (gfx950).
//
// One decode step of several layers (the Zenodo abstract's decode path and
// the README's "Decode & Prefill Innovations": routing by the blocks' routing
// keys, low-rank space scoring, values gathered through the factors, exact
// residual and window rows, flash-style log-sum-exp combine), for pools of
// rotated keys with fp16 residual rows, as three launches:
//
//   k_routes   every (layer, unit)'s top-k routing (one workgroup each);
//   k_blocks   the streams: one-wave workgroups, each running a contiguous
//              segment of the step's work (cut on the host into segments of
//              about equal cost) as one stream of pages through its own LDS
//              ring.  A work item is 128 window rows of a unit, the low-rank
//              part of a routed block (V_K, U, V_V and the anchor rows), or
//              64 residual rows of one.  A wave's consecutive items of one
//              unit share one attention state and leave one partial;
//   k_merges   the log-sum-exp combine of each unit's partials.
//
// The streams:
//   * pages are copied straight from HBM into a ring of four 4352-byte LDS
//     slots with 16-byte direct-to-LDS buffer loads, up to four pages ahead of
//     the one being used; a wave waits for a page by counting its own
//     vector-memory operations (they complete in order), so the next pages
//     stay in flight while a page is used, also across item boundaries;
//   * each 16-byte chunk may come from any offset: 128-wide rows are stored
//     272 bytes apart (a 16-byte pad, so that MFMA operand reads of 16 rows hit
//     16 different bank groups), and chunks outside the source (pads, rows past
//     the data, the anchor's zero U row) read as zeros through the buffer's
//     range check;
//   * the MFMA operands that need a page's rows as columns (V^T for p.V, U^T
//     for p^T U, V_V^T for the fold) are read with ds_read_b64_tr_b16;
//   * LDS reads are inline asm that waits for its own reads: compiled reads
//     would wait for every load in flight to LDS first.

#include "dkv_common.h"

namespace {

constexpr int kSRowB = 272;                 // bytes per 128-wide fp16 row in LDS: 256 + one 16-byte pad
constexpr int kWRows = 16;                  // rows per row page
constexpr int kWPage = kWRows * kSRowB + 256;  // bytes per ring slot: a row page (16 rows), or the
                                               // 4608 bytes of a 4-bit residual page
constexpr int kWChunks = kWPage / 16;       // 16-byte chunks per ring slot
constexpr int kWSlots = 4;                  // ring depth per wave
constexpr int kWRing = kWPage * kWSlots;    // one wave's ring
enum { kBaseAK = 0, kBaseAV, kBaseU, kBaseVK, kBaseVV, kBaseRP, kBases };
constexpr int kBPosOff = kWRing;            // the residual positions of a low-rank item [256] bytes
constexpr int kBBaseOff = kBPosOff + 256;   // the issuing low-rank item's source addresses [kBases] u64
constexpr int kBAncOff = kBBaseOff + 64;    // anchor rows a_k, a_v of low-rank items, two buffers [2][512] bytes
constexpr int kBLds = kBAncOff + 2 * 512;

static_assert(kBases * 8 <= 64, "source address table");
static_assert(kBLds % 16 == 0, "LDS areas are 16-byte aligned");
static_assert(32 * 64 * 2 + 16 <= kWPage, "a U page (32 mu positions of rank r, mu r <= 64) fits a slot");

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

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
// four bytes at a, a + 64, a + 128, a + 192
__device__ __forceinline__ void lds_u8x4(uint32_t a, uint32_t (&x)[4]) {
  asm volatile(
      "ds_read_u8 %0, %4\n\t"
      "ds_read_u8 %1, %4 offset:64\n\t"
      "ds_read_u8 %2, %4 offset:128\n\t"
      "ds_read_u8 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(a)
      : "memory");
}

// Eight reads at eight addresses (8-byte, 4-byte, or the transposing reads of
// 8-bit and 4-bit elements: in each 16-lane group, ds_read_b64_tr_b8 gives
// lane i byte column i of the eight rows the group's lanes 2 k, 2 k + 1 name,
// and ds_read_b64_tr_b4 nibble column i of the sixteen rows its lanes name),
// and four 16-byte reads at b, b + 16, b + 32, b + 48, in one round trip.
#define DKV_LDS_X8S(NAME, INSN, T)                                                                     \
  __device__ __forceinline__ void NAME(const uint32_t(&a)[8], uint32_t b, T(&o)[8], v4u(&sb)[4]) {    \
    asm volatile(INSN " %0, %12\n\t" INSN " %1, %13\n\t" INSN " %2, %14\n\t" INSN " %3, %15\n\t"    \
                 INSN " %4, %16\n\t" INSN " %5, %17\n\t" INSN " %6, %18\n\t" INSN " %7, %19\n\t"    \
                 "ds_read_b128 %8, %20\n\t"                                                          \
                 "ds_read_b128 %9, %20 offset:16\n\t"                                                \
                 "ds_read_b128 %10, %20 offset:32\n\t"                                               \
                 "ds_read_b128 %11, %20 offset:48\n\t"                                               \
                 "s_waitcnt lgkmcnt(0)"                                                               \
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),      \
                   "=&v"(o[6]), "=&v"(o[7]), "=&v"(sb[0]), "=&v"(sb[1]), "=&v"(sb[2]), "=&v"(sb[3])   \
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),       \
                   "v"(a[7]), "v"(b)                                                                  \
                 : "memory");                                                                         \
  }
DKV_LDS_X8S(lds_b64x8s, "ds_read_b64", v2u)
DKV_LDS_X8S(lds_b32x8s, "ds_read_b32", uint32_t)
DKV_LDS_X8S(lds_trb8x8s, "ds_read_b64_tr_b8", v2u)
DKV_LDS_X8S(lds_trb4x8s, "ds_read_b64_tr_b4", v2u)
#undef DKV_LDS_X8S

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

// eight plain 8-byte reads at a + 32 k (k = 0..7)
__device__ __forceinline__ void lds_b64x8(uint32_t a, v4h (&o)[8]) {
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %8 offset:32\n\t"
      "ds_read_b64 %2, %8 offset:64\n\t"
      "ds_read_b64 %3, %8 offset:96\n\t"
      "ds_read_b64 %4, %8 offset:128\n\t"
      "ds_read_b64 %5, %8 offset:160\n\t"
      "ds_read_b64 %6, %8 offset:192\n\t"
      "ds_read_b64 %7, %8 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a)
      : "memory");
}

__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4b(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, off, 0, 0, 0);
}
// a 64-bit value that is the same on every lane, as a scalar (so that a buffer
// resource made from it needs no per-lane loop)
__device__ __forceinline__ const char* uniform_ptr(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutside = 0xFFFFFFF0u;  // a buffer offset past every resource: the load returns zeros


// ---------------------------------------------------------------------------
// Pages
//
// A low-rank item streams nq V_K pages (rows 16 i .. of V_K), nu = 8 / mu U
// pages (positions 32 mu i .. 32 mu (i + 1) - 1, position 0 the anchor, whose
// U row is zero) and nq V_V pages; its anchor rows a_k and a_v load with its
// first V_K page into one of two anchor buffers (items alternate), its
// residual positions into the position buffer.  A K/V item (window rows, or
// residual rows of a block) streams K and V pages, alternating: 16 fp16 rows
// (272-byte LDS rows), or 32 rows of 8- or 4-bit codes.
// ---------------------------------------------------------------------------

enum PageKind { kPageVK = 0, kPageU = 1, kPageK = 2, kPageV = 3, kPageVV = 4 };

struct WaveGeom {
  int r, nq;   // rank; its 16-row tiles (V_K and V_V pages)
  int mu, nu;  // 32-position groups per U page (4, 2 or 1: mu r <= 64); U pages (8 / mu)
  int R, nt;   // low-rank item: residual rows (the mask); K/V item: its rows and their 16- or 32-row tiles
  bool kv;     // a K/V item
  int qb;      // K/V item: 0 fp16 rows, 8 or 4: residual rows of 8- or 4-bit codes
};

// A page of an 8-bit residual item holds 32 rows of one side (K or V): the
// rows' codes (128 bytes each), 16-byte chunk c of row j at chunk position
// c ^ swz(j) of the row, a swizzle that spreads the page's row and column reads
// over the LDS banks; then, at kQSbOff, the rows' (scale, bias) pairs, 8 bytes
// per row.  A page of a 4-bit residual item holds both sides of 32 rows: the K
// codes (64 bytes a row), the V codes at kQ4VOff, the K pairs at kQSbOff and
// the V pairs at kQ4VSbOff.
constexpr int kQRows = 32;
constexpr int kQSbOff = 4096;
constexpr int kQ4VOff = 2048;
constexpr int kQ4VSbOff = kQSbOff + kQRows * 8;
static_assert(kQSbOff + kQRows * 8 <= kWPage && kQRows * kD <= kQSbOff, "an 8-bit page fits a slot");
static_assert(kQ4VSbOff + kQRows * 8 <= kWPage && kQ4VOff + kQRows * kD / 2 <= kQSbOff, "a 4-bit page fits a slot");
__device__ __forceinline__ int q8_swz(int j) { return (j ^ ((j >> 3) << 1)) & 7; }
__device__ __forceinline__ int q4_swz(int j) { return (j >> 2) & 3; }

__device__ __forceinline__ int u_groups(int r) { return r <= 16 ? 4 : (r <= 32 ? 2 : 1); }

__device__ __forceinline__ void page_kind(const WaveGeom& g, int k, int& kind, int& i) {
  if (g.kv && g.qb == 4) {
    kind = kPageK;  // K and V of the tile's rows
    i = k;
  } else if (g.kv) {
    kind = kPageK + (k & 1);
    i = k >> 1;
  } else if (k < g.nq) {
    kind = kPageVK;
    i = k;
  } else if ((k -= g.nq) < g.nu) {
    kind = kPageU;
    i = k;
  } else {
    kind = kPageVV;
    i = k - g.nu;
  }
}

// The lane's index.  (Address arithmetic built on it is hoisted out of the
// streams' loops and held in registers: k_blocks then uses all 256 VGPRs of its
// two-waves-per-SIMD budget, without spills, and runs its quantised pages ~5%
// faster than with that arithmetic recomputed per page.)
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Per lane: the source offset of chunk 64 q + lane (q = 0..4) of a 128-wide
// row page (row p / 17, chunk p % 17 of the row; chunk 16, the row's pad, is
// kOutside), the same for every row page.
__device__ __forceinline__ uint32_t row_off(int q) {
  const int p = 64 * q + lane_id();
  const int row = (p * 3856) >> 16;  // p / 17 for p < 17 * 16 * 2
  const int c = p - 17 * row;
  return c < 16 ? (uint32_t)(row * 256 + 16 * c) : kOutside;
}

// Issue the loads of page k of an item's stream into the ring slot `dst`;
// returns the number of vector-memory instructions issued.  The loads are
// buffer loads straight into LDS: each source is a buffer resource sized to
// its data, and every 16-byte chunk whose offset falls outside it reads as
// zeros.  bb: the low-rank item's source addresses; rows_k / rows_v: the K/V
// item's first rows (codes, for quantised rows, and rows_ks / rows_vs their
// scale and bias pairs); posdst / ancdst: the position and anchor buffers.
__device__ __forceinline__ int issue_page(const WaveGeom& g, int k, unsigned char* dst, const uint64_t* bb,
                                          const char* rows_k, const char* rows_v, const char* rows_ks,
                                          const char* rows_vs, unsigned char* posdst, unsigned char* ancdst) {
  const int lane = threadIdx.x & 63;
  int kind, i;
  page_kind(g, k, kind, i);
  const int r = g.r;
  int ops = 0;
  if (g.qb) {
    // 32 rows of codes (swizzled chunks), then their scale and bias pairs; a
    // 4-bit page takes the V side's as well
    int nvalid = g.R - kQRows * i;
    nvalid = nvalid > kQRows ? kQRows : nvalid;
    if (g.qb == 8) {
      const __amdgpu_buffer_rsrc_t rs =
          rsrc_of((kind == kPageK ? rows_k : rows_v) + kQRows * i * kD, (uint32_t)(nvalid * kD));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = 64 * q + lane;
        dma16b(rs, (uint32_t)(128 * (p >> 3) + 16 * ((p & 7) ^ q8_swz(p >> 3))), dst + 1024 * q);
        ++ops;
      }
      const __amdgpu_buffer_rsrc_t rsb =
          rsrc_of((kind == kPageK ? rows_ks : rows_vs) + kQRows * i * 8, (uint32_t)(nvalid * 8));
      if (lane < kQRows / 2) dma16b(rsb, (uint32_t)(16 * lane), dst + kQSbOff);
      ++ops;
    } else {
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const __amdgpu_buffer_rsrc_t rs =
            rsrc_of((side == 0 ? rows_k : rows_v) + kQRows * i * (kD / 2), (uint32_t)(nvalid * (kD / 2)));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int p = 64 * q + lane;
          dma16b(rs, (uint32_t)(64 * (p >> 2) + 16 * ((p & 3) ^ q4_swz(p >> 2))), dst + kQ4VOff * side + 1024 * q);
          ++ops;
        }
        const __amdgpu_buffer_rsrc_t rsb =
            rsrc_of((side == 0 ? rows_ks : rows_vs) + kQRows * i * 8, (uint32_t)(nvalid * 8));
        if (lane < kQRows / 2) dma16b(rsb, (uint32_t)(16 * lane), dst + (side == 0 ? kQSbOff : kQ4VSbOff));
        ++ops;
      }
    }
    return ops;
  }
  if (kind == kPageU) {
    // U rows 32 mu i - 1 .. (row -1 reads as zeros: the anchor), dense, and 16
    // bytes more: the last row's reads run one chunk past its end
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(uniform_ptr(bb[kBaseU]), (uint32_t)(510 * r));
    const int nch = 4 * g.mu * r + 1;
    const int start = (32 * g.mu * i - 1) * 2 * r;
    for (int q = 0; q < nch; q += 64) {
      if (q + lane < kWChunks) dma16b(rs, (uint32_t)(start + 16 * (q + lane)), dst + 16 * q);
      ++ops;
    }
    return ops;
  }
  const char* base;
  int nvalid;
  if (g.kv) {
    base = (kind == kPageK ? rows_k : rows_v) + 16 * i * 256;
    nvalid = g.R - 16 * i;
  } else {
    base = uniform_ptr(bb[kind == kPageVK ? kBaseVK : kBaseVV]) + 16 * i * 256;
    nvalid = r - 16 * i;
  }
  nvalid = nvalid > 16 ? 16 : nvalid;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base, (uint32_t)nvalid * 256u);
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    // chunks past the page's 17 * 16 (lanes 16.. of the last load) are not loaded
    if (q < 4 || lane < 16) dma16b(rs, row_off(q), dst + 1024 * q);
    ++ops;
  }
  if (kind == kPageVK && i == 0) {
    // the anchor rows: a_k to bytes 0..255, a_v to 256..511 of the anchor buffer
    const char* a = lane < 16 ? uniform_ptr(bb[kBaseAK]) + 16 * lane : uniform_ptr(bb[kBaseAV]) + 16 * (lane - 16);
    if (lane < 32) dma16(a, ancdst);
    ++ops;
    if (g.R > 0) {
      // the residual positions: R <= 255 bytes as R / 4 dwords (R % 4 == 0)
      const __amdgpu_buffer_rsrc_t rp = rsrc_of(uniform_ptr(bb[kBaseRP]), (uint32_t)g.R);
      if (4 * lane < g.R) dma4b(rp, (uint32_t)(4 * lane), posdst);
      ++ops;
    }
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
  float bq0, bq1;  // this lane's share of the quantised rows' bias terms of columns 0..63 and 64..127
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
template <int NS, bool LOWRANK>
__device__ __forceinline__ void softmax_step(SState& st, float (&z)[NS]) {
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
      if (LOWRANK) {
        // (outside a low-rank item W and its weight sum are zero and dead)
#pragma unroll
        for (int k = 0; k < 4; ++k) st.Wt[k] *= alpha;
        st.llr *= alpha;
      }
      st.l *= alpha;
      st.bq0 *= alpha;
      st.bq1 *= alpha;
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
  if (LOWRANK) st.llr += s;
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

// q~ (or W^T) tile number i of a four-tile register array, i uniform
template <class T>
__device__ __forceinline__ T pick4(const T (&a)[4], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : (i == 2 ? a[2] : a[3]));
}

struct BlockRegs {
  v4h qth[4], qtl[4];  // scaled V_K q of the block (hi + lo fp16): rows 16 k + 4 q4 + e, head l16
  float qa;            // scale * q . a_k
  v4h pv;              // weights of the current K tile (fp16), for its V tile
  uint32_t mw[8];      // the block's residual-position mask (bit p of word p / 32: position p)
};

// The page kinds' work.  P0: the page's LDS byte address (the wave's own ring
// slot); i: the page's number within its kind.  st and br carry over from page
// to page.

// V_K page i: q~ rows 16 i .. 16 i + 15.  Page 0 also takes q . a_k from the
// anchor buffer (a one-row MFMA tile) and turns the block's residual
// positions into the mask words.
__device__ __forceinline__ void page_vk(const WaveGeom& g, int i, uint32_t P0, const v8h (&qf)[4], BlockRegs& br,
                                        float scale, uint32_t posb, uint32_t anc) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4;
  const int r = g.r;
  v8h a[4];
  lds_b128x4(P0 + l16 * kSRowB + 16 * q4, a);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) acc = mfma32(a[s2], qf[s2], acc);
  v4f x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = 16 * i + 4 * q4 + e < r ? acc[e] * scale : 0.f;
  v4h hi, lo;
  split4(x, hi, lo);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    br.qth[k] = k == i ? hi : br.qth[k];
    br.qtl[k] = k == i ? lo : br.qtl[k];
  }
  if (i == 0) {
    v8h ak[4];
    lds_b128x4(anc + 16 * q4, ak);
    const v8h zero = {};
    v4f aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) aq = mfma32(l16 == 0 ? ak[s2] : zero, qf[s2], aq);
    br.qa = hq_sum(q4 == 0 ? aq[0] * scale : 0.f);
    // positions lane + 64 j of the block's R (distinct, in 1..255, any order)
    uint32_t p[4];
    lds_u8x4(posb + lane, p);
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = lane + 64 * j < g.R ? p[j] : 0u;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t v = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) v |= (p[j] >> 5) == (uint32_t)w && p[j] >= 1u ? 1u << (p[j] & 31) : 0u;
      br.mw[w] = wave_or(v);
    }
  }
}

// 32 U positions starting at position 32 w of the block (U rows at LDS
// address P0, r halves each): low-rank scores, then W^T += Ux^T p.
__device__ __forceinline__ void u_group(const WaveGeom& g, int w, uint32_t P0, SState& st, BlockRegs& br) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4, s4 = l16 & 3;
  const int r = g.r;
  const uint32_t mw = w == 0 ? br.mw[0] : w == 1 ? br.mw[1] : w == 2 ? br.mw[2] : w == 3 ? br.mw[3]
                    : w == 4 ? br.mw[4] : w == 5 ? br.mw[5] : w == 6 ? br.mw[6] : br.mw[7];
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
  softmax_step<8, true>(st, z);
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

// U page i: its mu groups of 32 positions
__device__ __forceinline__ void page_u(const WaveGeom& g, int i, uint32_t P0, SState& st, BlockRegs& br) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < g.mu) u_group(g, g.mu * i + j, P0 + 64 * j * g.r, st, br);
}

// K page i: scores of rows 16 i .. 16 i + 15 of a K/V item.
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
  softmax_step<4, false>(st, z);
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

// V_V page i: O^T += V_V^T rows 16 i .. 16 i + 15 times W^T rows.  Page 0 also
// adds a_v times the block's low-rank weight sum (the anchor's value and the
// U-row-independent part of every low-rank row's value).
__device__ __forceinline__ void page_vv(const WaveGeom& g, int i, uint32_t P0, SState& st, uint32_t anc) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, q4 = lane >> 4, s4 = l16 & 3;
  const int r = g.r;
  if (i == 0) {
    const float lt = hq_sum(st.llr);
    st.llr = 0.f;
    v4h av[8];  // a_v[16 nn + 4 q4 .. + 3]
    lds_b64x8(anc + 256 + 8 * q4, av);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn)
#pragma unroll
      for (int e = 0; e < 4; ++e) st.Ot[nn][e] += (float)av[nn][e] * lt;
  }
  v4f x = pick4(st.Wt, i);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = 16 * i + 4 * q4 + e < r ? x[e] : 0.f;
  v4h wh, wlo;
  split4(x, wh, wlo);
  v4h a[8];
  lds_tr8(P0 + (4 * q4 + (l16 >> 2)) * kSRowB + 16 * (s4 >> 1) + 8 * (s4 & 1), a);
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = mfma16(a[nn], wlo, mfma16(a[nn], wh, st.Ot[nn]));
}

// Quantised residual rows (x[d] = scale_g code[d] + bias_g, g = d / 64): the
// codes enter the MFMAs as the exact fp16 values 1024 + code (0x64 above the
// code's byte, one byte permute per pair of codes), the scales and biases apply
// in fp32 and take the offset back out:
//   q . x_t = s_0 (q . (1024 + code_t))_{0..63} + s_1 (q . (1024 + code_t))_{64..127}
//             + (b_0 - 1024 s_0) Q_0 + (b_1 - 1024 s_1) Q_1,
// Q_g the sum of q over group g; for V the scales fold into the weights
// (rounded to fp16, as the weights of fp16 rows are), and the bias terms
// sum_t p_t b_g,t - 1024 sum_t w_g,t (w the rounded weights) accumulate in the
// state (bq0, bq1) and join O at the run's end.  The offset costs a few bits of
// the fp32 sums' 24 (sums about nine times larger than the codes' own).

// 8 bytes -> v8h of 1024 + byte, in order
__device__ __forceinline__ v8h bytes8_b1024(v2u c) {
  uint32_t w[4];
  w[0] = __builtin_amdgcn_perm(0x64646464u, c[0], 0x04010400u);
  w[1] = __builtin_amdgcn_perm(0x64646464u, c[0], 0x04030402u);
  w[2] = __builtin_amdgcn_perm(0x64646464u, c[1], 0x04010400u);
  w[3] = __builtin_amdgcn_perm(0x64646464u, c[1], 0x04030402u);
  return __builtin_bit_cast(v8h, w);
}
// 8 nibbles (nibble k: bits 4 k .. 4 k + 3) -> v8h of 1024 + nibble in the
// order 0 4 1 5 2 6 3 7 (the k order of the 4-bit pages: the V pages' weights
// and the K pages' query follow it).  The even and odd nibbles are masked into
// bytes, and each output word takes two of their bytes beside 0x64 high bytes.
__device__ __forceinline__ v8h nibbles8_b1024_il(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;  // nibbles 0 2 4 6, 1 3 5 7
  uint32_t w[4];
  w[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04020400u);  // nibbles 0, 4
  w[1] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04020400u);  // 1, 5
  w[2] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030401u);  // 2, 6
  w[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030401u);  // 3, 7
  return __builtin_bit_cast(v8h, w);
}

// The (scale, bias) pairs of rows 8 q4 .. 8 q4 + 7 of a quantised page come
// with the codes' reads: row 8 q4 + k in dwords 2 (k & 1), 2 (k & 1) + 1 of
// sb[k / 2] (s0 | b0 << 16, s1 | b1 << 16).

// K page i of a quantised residual item: the scores of its rows 8 q4 + k
// (k = 0..7), head l16, through the softmax step, into the weights z[k].
// Score tile tt takes row 8 (l16 / 4) + 4 tt + l16 % 4 as its MFMA row l16, so
// that output row 4 q4 + e is row 8 q4 + 4 tt + e: the lane's eight weights are
// then those of the rows the V page's MFMA takes as its k = 8 q4 + k.
__device__ __forceinline__ void page_qk(const WaveGeom& g, int i, uint32_t P0, SState& st, const v8h (&qf)[4],
                                        float Q0, float Q1, float scale, float (&z)[8]) {
  const int lane = lane_id(), l16 = lane & 15, q4 = lane >> 4;
  uint32_t a[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int j = 8 * (l16 >> 2) + 4 * tt + (l16 & 3);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)  // dimensions 32 s2 + 8 q4 .. + 7
      a[4 * tt + s2] = g.qb == 8 ? P0 + 128 * j + 16 * ((2 * s2 + (q4 >> 1)) ^ q8_swz(j)) + 8 * (q4 & 1)
                                 : P0 + 64 * j + 16 * (s2 ^ q4_swz(j)) + 4 * q4;
  }
  const uint32_t b = P0 + kQSbOff + 64 * q4;
  v8h kc[8];
  v4u sb[4];
  if (g.qb == 8) {
    v2u c[8];
    lds_b64x8s(a, b, c, sb);
#pragma unroll
    for (int t = 0; t < 8; ++t) kc[t] = bytes8_b1024(c[t]);
  } else {
    uint32_t c[8];
    lds_b32x8s(a, b, c, sb);
#pragma unroll
    for (int t = 0; t < 8; ++t) kc[t] = nibbles8_b1024_il(c[t]);
  }
  // 4-bit codes come in the k order 0 4 1 5 2 6 3 7: the query takes the same
  v8h qk[4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2)
    qk[s2] = g.qb == 8 ? qf[s2] : __builtin_shufflevector(qf[s2], qf[s2], 0, 4, 1, 5, 2, 6, 3, 7);
  const int nr = g.R - kQRows * i;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const v4f S0 = mfma32(kc[4 * tt + 1], qk[1], mfma32(kc[4 * tt], qk[0], zero));
    const v4f S1 = mfma32(kc[4 * tt + 3], qk[3], mfma32(kc[4 * tt + 2], qk[2], zero));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * tt + e;
      const uint32_t x = sb[k >> 1][2 * (k & 1)], y = sb[k >> 1][2 * (k & 1) + 1];
      const float s0 = h_lo(x), s1 = h_lo(y);
      const float v = (s0 * S0[e] + s1 * S1[e]) + ((h_hi(x) - 1024.f * s0) * Q0 + (h_hi(y) - 1024.f * s1) * Q1);
      z[k] = 8 * q4 + k < nr ? v * scale : -INFINITY;
    }
  }
  softmax_step<8, false>(st, z);
}

// V side of a quantised residual tile (codes at P0, scale and bias pairs at
// Psb): O^T += V^T p, the codes of rows
// 8 q4 + k read transposed (column d = 16 nn + l16 of them, as the MFMA's
// k = 8 q4 + k; for 4-bit codes in the k order 0 4 1 5 2 6 3 7, which the
// weights follow), one MFMA per 16 columns.
__device__ __forceinline__ void page_qv(const WaveGeom& g, uint32_t P0, uint32_t Psb, SState& st, const float (&z)[8]) {
  const int lane = lane_id(), l16 = lane & 15, q4 = lane >> 4;
  // Q8: the group's lanes 2 k, 2 k + 1 name row 8 q4 + k, bytes 16 nn .. + 7 and
  // + 8 .. + 15.  Q4: the group's lane k names row 16 (q4 / 2) + (k + 8 q4) % 16,
  // bytes 8 nn .. + 7 (columns 16 nn .. + 15): its first eight rows, the low
  // word of the result, are then the rows 8 q4 .. + 7 the lane keeps.
  const int j = g.qb == 8 ? 8 * q4 + (l16 >> 1) : 16 * (q4 >> 1) + ((l16 + 8 * q4) & 15);
  uint32_t a[8];
#pragma unroll
  for (int nn = 0; nn < 8; ++nn)
    a[nn] = g.qb == 8 ? P0 + 128 * j + 16 * (nn ^ q8_swz(j)) + 8 * (l16 & 1)
                      : P0 + 64 * j + 16 * ((nn >> 1) ^ q4_swz(j)) + 8 * (nn & 1);
  const uint32_t b = Psb + 64 * q4;
  v2u c[8];
  v4u sb[4];
  if (g.qb == 8)
    lds_trb8x8s(a, b, c, sb);
  else
    lds_trb4x8s(a, b, c, sb);
  v8h w0, w1;
  float be0 = 0.f, be1 = 0.f, ws0 = 0.f, ws1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t x = sb[k >> 1][2 * (k & 1)], y = sb[k >> 1][2 * (k & 1) + 1];
    w0[k] = (f16)(z[k] * h_lo(x));
    w1[k] = (f16)(z[k] * h_lo(y));
    be0 += z[k] * h_hi(x);
    be1 += z[k] * h_hi(y);
    ws0 += (float)w0[k];
    ws1 += (float)w1[k];
  }
  st.bq0 += be0 - 1024.f * ws0;
  st.bq1 += be1 - 1024.f * ws1;
  if (g.qb == 8) {
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = mfma32(bytes8_b1024(c[nn]), nn < 4 ? w0 : w1, st.Ot[nn]);
  } else {
    w0 = __builtin_shufflevector(w0, w0, 0, 4, 1, 5, 2, 6, 3, 7);
    w1 = __builtin_shufflevector(w1, w1, 0, 4, 1, 5, 2, 6, 3, 7);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn)
      st.Ot[nn] = mfma32(nibbles8_b1024_il(c[nn][0]), nn < 4 ? w0 : w1, st.Ot[nn]);
  }
}

// ---------------------------------------------------------------------------
// The launches
// ---------------------------------------------------------------------------

typedef const __attribute__((address_space(4))) int32_t CInt;
typedef const __attribute__((address_space(4))) uint32_t CUint;
typedef const __attribute__((address_space(4))) LayerArgs CLayerArgs;

// The routings of a step: workgroup (layer, unit) routes the unit's query
// (route_unit), writing the routed slots tagged with the step's tag.
__global__ __launch_bounds__(kAttThreads) void k_routes(const LayerArgs* __restrict__ table, int n_units,
                                                        int top_k) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ RouteShared<kAttWaves> rsh;
  const int layer = blockIdx.x / n_units, u = blockIdx.x - layer * n_units;
  const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)table + layer);
  const uint32_t tag = slot_tag(((CUint*)la.D.ctrl)[3]);
  route_unit<kAttThreads>(la.P, la.Bt, u, top_k, la.D.idx, nullptr, la.D.slots, reinterpret_cast<uint32_t*>(smem),
                          rsh, tag);
}

struct BlocksArgs {
  const LayerArgs* table;
  const int32_t* sched;  // the step's schedule (see k_blocks)
  const uint32_t* ctrl;  // the step's control header (word 3: the routed-slot tag of this step)
  int n_waves;
  int top_k;
};

// What one side of a stream needs to know about a work item.
struct SItem {
  WaveGeom g;
  int npages;          // pages of the item's stream: the unit's query rows first if it opens a run
  int kind, first, last;
  int G, row0, part;   // the unit's query rows row0 .. row0 + G - 1; the run's partial index
  int layer, h;
  int64_t slot;        // block items: the routed pool slot, or -1 (nothing to stream)
  const char* rows_k;  // K/V items: their first key and value rows (quantised: codes)
  const char* rows_v;
  const char* rows_ks; // quantised residual items: the first rows' scale and bias pairs
  const char* rows_vs;
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
  it.g.mu = u_groups(P.rank);
  it.g.nu = 8 / it.g.mu;
  it.g.qb = 0;
  it.slot = -1;
  it.rows_k = nullptr;
  it.rows_v = nullptr;
  it.rows_ks = nullptr;
  it.rows_vs = nullptr;
  int pages;
  if (it.kind == kItemWin) {
    // window rows r0 .. r0 + nrows - 1, as far as the batch row's window reaches
    const int r0 = (int)w1;
    int wl = la.Bt.wlen ? ((CInt*)la.Bt.wlen)[b] : la.Bt.W;
    wl = wl < 0 ? 0 : (wl > la.Bt.W ? la.Bt.W : wl);
    int rows = wl - r0;
    rows = rows < 0 ? 0 : (rows > nrows ? nrows : rows);
    const int64_t base = (((int64_t)b * Hkv + h) * la.Bt.W + r0) * kD;
    it.rows_k = (const char*)(la.Bt.wk + base);
    it.rows_v = (const char*)(la.Bt.wv + base);
    it.g.kv = true;
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
      it.g.kv = false;
      it.g.R = P.n_resid;
      it.g.nt = 0;
      pages = slot >= 0 ? 2 * it.g.nq + it.g.nu : 0;
    } else {
      // residual rows r0 .. r0 + nrows - 1 of the routed block
      const int r0 = (int)(w1 >> 16);
      it.g.kv = true;
      it.g.R = slot >= 0 ? nrows : 0;
      if (P.rfmt == 0) {
        it.g.nt = (it.g.R + 15) >> 4;
        if (slot >= 0) {
          it.rows_k = (const char*)(P.rk + slot * P.rk_s + h * P.rk_h + (int64_t)r0 * kD);
          it.rows_v = (const char*)(P.rv + slot * P.rv_s + h * P.rv_h + (int64_t)r0 * kD);
        }
      } else {
        it.g.qb = P.rfmt == 1 ? 8 : 4;
        it.g.nt = (it.g.R + kQRows - 1) / kQRows;  // 4-bit: one page a tile, 8-bit: two
        const int cb = P.rfmt == 1 ? kD : kD / 2;
        if (slot >= 0) {
          it.rows_k = (const char*)(P.rkq + slot * P.rkq_s + h * P.rkq_h + (int64_t)r0 * cb);
          it.rows_v = (const char*)(P.rvq + slot * P.rvq_s + h * P.rvq_h + (int64_t)r0 * cb);
          it.rows_ks = (const char*)(P.rks + slot * P.rks_s + h * P.rks_h + (int64_t)r0 * 4);
          it.rows_vs = (const char*)(P.rvs + slot * P.rvs_s + h * P.rvs_h + (int64_t)r0 * 4);
        }
      }
      pages = it.g.qb == 4 ? it.g.nt : 2 * it.g.nt;
    }
  }
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
      default: a = P.rp + slot * P.rp_s + h * P.rp_h; break;
    }
    bases[lane] = (uint64_t)a;
  }
  wave_sync_lds();
}

// The issuing side of a wave's stream: its pages, in order, into the ring's
// kWSlots slots; in_flight holds the vector-memory operation counts of the
// pages in flight, one byte each, byte 0 the oldest (the next to be used).
struct Issuer {
  SItem it;        // the item being issued
  int ii, ik;      // its index in the wave's list, its next page
  int i1;          // the end of the list
  int n_issued;        // pages issued
  int n_lowrank;   // low-rank items entered (their anchor buffer alternates)
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
  if (S.ii < S.i1 && S.it.kind == kItemLowRank && S.it.slot >= 0) {
    item_bases(A, S.it, bases);
    ++S.n_lowrank;
  }
}

// issue the stream's next page, if any; n_next: the oldest page not yet used
__device__ __forceinline__ void issue_next(const BlocksArgs& A, CInt* items, uint32_t tag, Issuer& S, int n_next,
                                           unsigned char* smem, uint64_t* bases) {
  if (S.ii >= S.i1) return;  // every item issued
  unsigned char* dst = smem + kWPage * (S.n_issued & (kWSlots - 1));
  int ops;
  if (S.it.first && S.ik == 0) {
    // the unit's query rows: 16 rows of 256 bytes, rows past G zero
    const int lane = threadIdx.x & 63;
    const LayerArgs& la = *(const LayerArgs*)((CLayerArgs*)A.table + S.it.layer);
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(la.Bt.q + (int64_t)S.it.row0 * kD, (uint32_t)(S.it.G * 256));
#pragma unroll
    for (int q = 0; q < 256; q += 64) dma16b(rs, (uint32_t)(16 * (q + lane)), dst + 16 * q);
    ops = 4;
  } else {
    ops = issue_page(S.it.g, S.ik - S.it.first, dst, bases, S.it.rows_k, S.it.rows_v, S.it.rows_ks,
                     S.it.rows_vs, smem + kBPosOff, smem + kBAncOff + 512 * (S.n_lowrank & 1));
  }
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
// sched[w + 1] - 1 as one stream of pages through its ring: the next item's
// first pages load while the current item's last ones are used.  The wave's
// consecutive items of one unit (a run) share one attention state and leave
// one partial; its store joins the count of operations in flight instead of
// draining it.  An item's pages come in a fixed order, so the work of each
// page kind runs in a loop of its own.
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
  uint64_t* bases = reinterpret_cast<uint64_t*>(smem + kBBaseOff);
  const uint32_t ring0 = lds_off(smem), posb0 = lds_off(smem + kBPosOff), anc0 = lds_off(smem + kBAncOff);

  Issuer S;
  S.ii = i0;
  S.i1 = i1;
  S.n_issued = 0;
  S.n_lowrank = 0;
  S.in_flight = 0u;
  issuer_enter(A, items, tag, S, bases);
#pragma unroll 1
  for (int k = 0; k < kWSlots; ++k) issue_next(A, items, tag, S, 0, smem, bases);

  SState st;
  BlockRegs br;
  v8h qf[4];
  float Q0 = 0.f, Q1 = 0.f;  // the sums of the query over dimensions 0..63 and 64..127 (head l16)
  int n = 0;         // the next page to use
  int n_lowrank = 0; // low-rank items used
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
      issue_next(A, items, tag, S, ++n, smem, bases);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s0 += (float)qf[0][e] + (float)qf[1][e];
        s1 += (float)qf[2][e] + (float)qf[3][e];
      }
      Q0 = hq_sum(s0);
      Q1 = hq_sum(s1);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.Ot[nn] = (v4f){0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      st.l = 0.f;
      st.llr = 0.f;
      st.bq0 = 0.f;
      st.bq1 = 0.f;
    }
    if (cur.kind == kItemLowRank) {
      if (cur.slot >= 0) {
        const uint32_t anc = anc0 + 512 * (++n_lowrank & 1);
        // the block's W and q~ start from zero (so that neither is live outside
        // the low-rank items)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          st.Wt[k] = (v4f){0.f, 0.f, 0.f, 0.f};
          br.qth[k] = (v4h){};
          br.qtl[k] = (v4h){};
        }
        for (int i = 0; i < g.nq; ++i) {
          wait_oldest(S.in_flight);
          page_vk(g, i, ring0 + kWPage * (n & (kWSlots - 1)), qf, br, scale, posb0, anc);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, smem, bases);
        }
        for (int i = 0; i < g.nu; ++i) {
          wait_oldest(S.in_flight);
          page_u(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, br);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, smem, bases);
        }
        for (int i = 0; i < g.nq; ++i) {
          wait_oldest(S.in_flight);
          page_vv(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, anc);
          S.in_flight >>= 8;
          issue_next(A, items, tag, S, ++n, smem, bases);
        }
      }
    } else if (g.qb == 8) {
      for (int i = 0; i < g.nt; ++i) {
        float z[8];
        wait_oldest(S.in_flight);
        page_qk(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, qf, Q0, Q1, scale, z);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, smem, bases);
        wait_oldest(S.in_flight);
        const uint32_t P0 = ring0 + kWPage * (n & (kWSlots - 1));
        page_qv(g, P0, P0 + kQSbOff, st, z);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, smem, bases);
      }
    } else if (g.qb == 4) {
      for (int i = 0; i < g.nt; ++i) {
        float z[8];
        wait_oldest(S.in_flight);
        const uint32_t P0 = ring0 + kWPage * (n & (kWSlots - 1));
        page_qk(g, i, P0, st, qf, Q0, Q1, scale, z);
        page_qv(g, P0 + kQ4VOff, P0 + kQ4VSbOff, st, z);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, smem, bases);
      }
    } else {
      for (int i = 0; i < g.nt; ++i) {
        wait_oldest(S.in_flight);
        page_k(g, i, ring0 + kWPage * (n & (kWSlots - 1)), st, qf, br, scale);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, smem, bases);
        wait_oldest(S.in_flight);
        page_v(ring0 + kWPage * (n & (kWSlots - 1)), st, br);
        S.in_flight >>= 8;
        issue_next(A, items, tag, S, ++n, smem, bases);
      }
    }
    if (cur.last) {
      // the run's partial: o normalised, lse (every lane of a head writes the
      // same lse).  G >= 1, so lane 0 always stores and every store issues.
      const int np = la.D.att.n_parts;
      const float bq0 = hq_sum(st.bq0), bq1 = hq_sum(st.bq1);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) st.Ot[nn] += nn < 4 ? bq0 : bq1;
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

// The streams' read ceiling: workgroup w reads bytes [w per, (w + 1) per) of
// src through its four-page ring with the same 16-byte buffer loads into LDS
// (four per 4096-byte page, up to four pages ahead), reads each page back
// once and writes the wrapping sum of its 32-bit words to sink[w].
__global__ __launch_bounds__(64) void k_read_probe(const unsigned char* __restrict__ src, uint32_t per,
                                                   uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(src + (size_t)blockIdx.x * per, per);
  const int npages = (int)(per / 4096u);
  const uint32_t ring0 = lds_off(smem);
  uint32_t acc = 0u;
  for (int n = 0; n < 4 && n < npages; ++n)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dma16b(rs, (uint32_t)n * 4096u + 1024u * k + 16u * lane, smem + 4096 * n + 1024 * k);
  for (int n = 0; n < npages; ++n) {
    const int newer = npages - n - 1 < 3 ? npages - n - 1 : 3;
    wait_vm(4 * newer);
    v4u w[4];  // bytes 16 lane + 1024 k of the page
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
        : "v"(ring0 + 4096u * (uint32_t)(n & 3) + 16u * (uint32_t)lane)
        : "memory");
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += w[k][0] + w[k][1] + w[k][2] + w[k][3];
    if (n + 4 < npages)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dma16b(rs, (uint32_t)(n + 4) * 4096u + 1024u * k + 16u * lane, smem + 4096 * (n & 3) + 1024 * k);
  }
  for (int o = 32; o > 0; o >>= 1) acc += (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

// LDS bytes of a stream (one-wave workgroup).
__attribute__((visibility("hidden"))) size_t dkv_stream_lds_bytes() { return (size_t)kBLds; }

// One decode step of several layers as three launches on `st`: the routings
// (k_routes, route_lds bytes of dynamic LDS), the streams (k_blocks), the
// merges (k_merges).  sched: the step's schedule in device memory (see
// k_blocks), with n_waves streams and n_sched_items items, over n_layers *
// n_units units; ctrl: the step's control header.
// events: NULL, or hipEvent_t handles [1] (recorded after the routings) and
// [2] (after the streams).
__attribute__((visibility("hidden"))) hipError_t dkv_stream_step(const void* table, uint32_t* ctrl,
                                                                 size_t route_lds, const int32_t* sched,
                                                                 int n_waves, int n_sched_items, int top_k,
                                                                 int n_layers, int n_units, void* const* events,
                                                                 hipStream_t st) {
  const LayerArgs* T = (const LayerArgs*)table;
  if (top_k > 0) {
    hipLaunchKernelGGL(k_routes, dim3((unsigned)(n_layers * n_units)), dim3(kAttThreads), route_lds, st, T,
                       n_units, top_k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (events) {
    hipError_t e = hipEventRecord((hipEvent_t)events[1], st);
    if (e != hipSuccess) return e;
  }
  BlocksArgs B;
  B.table = T;
  B.sched = sched;
  B.ctrl = ctrl;
  B.n_waves = n_waves;
  B.top_k = top_k;
  if (n_waves > 0) {
    hipLaunchKernelGGL(k_blocks, dim3((unsigned)n_waves), dim3(64), (size_t)kBLds, st, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (events) {
    hipError_t e = hipEventRecord((hipEvent_t)events[2], st);
    if (e != hipSuccess) return e;
  }
  const int32_t* unit_parts = sched + (n_waves + 1) + 4 * (int64_t)n_sched_items;
  hipLaunchKernelGGL(k_merges, dim3((unsigned)(n_layers * n_units)), dim3(kAttThreads), 0, st, T, n_units,
                     unit_parts, ctrl);
  return hipGetLastError();
}

// The streams' read ceiling (see k_read_probe): n_waves workgroups of `per`
// bytes each (a multiple of 4096).
__attribute__((visibility("hidden"))) hipError_t dkv_stream_read_probe_launch(const void* src, size_t per,
                                                                              int n_waves, uint32_t* sink,
                                                                              hipStream_t st) {
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)n_waves), dim3(64), (size_t)(4 * 4096), st,
                     (const unsigned char*)src, (uint32_t)per, sink);
  return hipGetLastError();
}
