// Device-side types and helpers shared by the gfx950 forward and backward
// kernels: vector types for MFMA operands, lane-layout permutations, and the
// view of the layout blob.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;  // head dimension handled by these kernels

// ---------------------------------------------------------------------------
// 32x32 MFMA lane layout (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2f32).
// A operand: lane L holds row L%32; B operand: lane L holds column L%32; the
// K slots of lane L belong to half g = L/32.  The result holds column L%32 in
// lane L and row 8*(r/4) + 4*g + r%4 in register r (16 registers).
//
// Loading the A-operand rows through sigma (swap bits 2 and 3 of the row
// index) makes register r of half g hold logical row kappa(r, g) =
// 16*(r/8) + 8*g + r%8: registers 0..7 of a half are 8 consecutive rows and
// registers 8..15 the next group of 16.  That is exactly the K-slot order of
// a following 32x32x16 MFMA, so a result can feed the next product as a B
// operand without any data movement.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sigma32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
__device__ __forceinline__ int kappa32(int r, int g) { return 16 * (r >> 3) + 8 * g + (r & 7); }

__device__ __forceinline__ floatx16 mfma_bf16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma_f32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Transposed A operand from a row-major LDS tile (gfx950 transposing LDS read).
//
// ds_read_b64_tr_b16 works on groups of 16 lanes: with lane j of a group
// addressing four consecutive 16-bit values D[j][0..3], lane i of the group
// receives D[4*s + i/4][i%4] for s = 0..3.  If lane j addresses row
// k0 + 8*g + j/4 of a row-major matrix M at column c0 + 16*q + 4*swap2(j%4)
// (g = lane/32, q = (lane/16)&1, swap2 exchanges the two bits of j%4), lane i
// receives M[k0 + 8*g + s][c0 + sigma32(16*q + i)]: one column over four
// consecutive rows.  Two such reads (rows +0..3 and +4..7) give the A operand
// of a 32x32x16 MFMA for A[row][k] = M[k0 + k][c0 + sigma32(row)], i.e. the
// transposed tile, with the same sigma row order as the row-major loads.
// stride is the row stride of M in elements (a multiple of 4).
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ v4i16 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) bf16*)(p)));
}

__device__ __forceinline__ bf16x8 load_a_transposed(const bf16* m, int stride, int k0, int c0,
                                                    int lane) {
  const int g = lane >> 5, q = (lane >> 4) & 1, j = lane & 15;
  const int t = j & 3;
  const int tsw = ((t & 1) << 1) | (t >> 1);
  const bf16* p0 = m + (k0 + 8 * g + (j >> 2)) * stride + c0 + 16 * q + 4 * tsw;
  const v4i16 a = lds_read_tr16(p0);
  const v4i16 b = lds_read_tr16(p0 + 4 * stride);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles filled by direct global->LDS loads.
//
// A tile is row-major [rows][64] bf16 (128 bytes per row, no padding); the
// eight 16-byte chunks of row r are stored XOR-swizzled, logical chunk c at
// physical chunk c ^ key(r) with key(r) = 2 (r mod 4) + bit 3 of r.  The key
// serves both read patterns of the kernels without bank conflicts:
//   16-byte operand reads: each group of 8 lanes reads one chunk column of
//     rows {0,1,2,3,8,9,10,11} (+4) (the sigma row order): the keys of those
//     rows are all different;
//   transposing 8-byte reads: each group of 16 lanes reads chunks c and c^1
//     of 4 consecutive rows 4a..4a+3: their keys are 2m + const, m = 0..3,
//     so the 8 (row, chunk) pairs land on 8 different chunk slots.
//
// The gfx950 16-byte global->LDS load writes lane L's 16 bytes to
// lds_base + 16 L (lds_base wave-uniform): one instruction fills a 1 KB block
// = 8 rows.  Lane L therefore fetches row (L / 8) of its block, logical chunk
// (L % 8) ^ key(row).  The loads count on vmcnt; wait_vmem() before the
// barrier that publishes the tile.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_key(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kD + ((chunk ^ swz_key(row)) << 3);
}

__device__ __forceinline__ void dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_dst, 16, 0, 0);
}

// The same direct load through a buffer resource over one (b, h) slice of a
// [B, H, n, 64] bf16 tensor: the lane's source is a 32-bit byte offset into
// the slice (one VALU operation) instead of a 64-bit address.  Offsets stay
// below n * 128 bytes, which the host keeps under 2^32.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ BufRsrc slice_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), kBufWord3);
}
__device__ __forceinline__ void dma16_buf(BufRsrc r, uint32_t voff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16,
                                           int(voff), 0, 0, 0);
}
// 32-bit loads through a buffer resource over an int32 / float array (the
// blob's index arrays, a (b, h) slice of LSE or D): the lane's element is a
// 32-bit byte offset.  No range is enforced (the callers index in bounds).
__device__ __forceinline__ BufRsrc array_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), 0x7fffffff, kBufWord3);
}
__device__ __forceinline__ int buf_i32(BufRsrc r, int index) {
  return int(__builtin_amdgcn_raw_buffer_load_b32(r, index * 4, 0, 0));
}
__device__ __forceinline__ float buf_f32(BufRsrc r, int index) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, index * 4, 0, 0));
}

// Byte offset of 16-byte chunk `chunk` of row `token` in a slice (clamped to
// row 0 for padding entries, -1).
__device__ __forceinline__ uint32_t row_chunk_offset(int token, int chunk) {
  return uint32_t(token < 0 ? 0 : token) * uint32_t(kD * 2) + uint32_t(chunk) * 16u;
}

// s_waitcnt vmcnt(0): every global load of this wave (direct-to-LDS included)
// has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposed A operand (see load_a_transposed) from a swizzled tile.
__device__ __forceinline__ bf16x8 load_a_transposed_swz(const bf16* m, int k0, int c0, int lane) {
  const int g = lane >> 5, q = (lane >> 4) & 1, j = lane & 15;
  const int t = j & 3;
  const int tsw = ((t & 1) << 1) | (t >> 1);
  const int col = c0 + 16 * q + 4 * tsw;  // multiple of 4: half of a 16-byte chunk
  const int r0 = k0 + 8 * g + (j >> 2), r1 = r0 + 4;
  const v4i16 a = lds_read_tr16(m + swz(r0, col >> 3) + (col & 7));
  const v4i16 b = lds_read_tr16(m + swz(r1, col >> 3) + (col & 7));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// Combining a value with the one in lane L ^ 32 (the other half of the
// wave) through v_permlane32_swap (gfx950): swapping lanes 32..63 of one copy
// with lanes 0..31 of another leaves every lane holding (x[L % 32],
// x[L % 32 + 32]); one VALU exchange instead of an LDS permute.
__device__ __forceinline__ void halves(float x, float* lo, float* hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  *lo = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
  *hi = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}
// max / sum of x over lanes L and L ^ 32 (the same value in both lanes).
__device__ __forceinline__ float pair_max(float x) {
  float lo, hi;
  halves(x, &lo, &hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float pair_sum(float x) {
  float lo, hi;
  halves(x, &lo, &hi);
  return lo + hi;
}

// Two floats -> two bf16 packed in 32 bits, round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  floatx2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  u32x4 u = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
             pack_bf16x2(p[6], p[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_to_float(bf16 x) { return float(x); }

// ---------------------------------------------------------------------------
// Layout blob (device copy): header + per-pattern records, see sparse_attn.h.
// ---------------------------------------------------------------------------
// Patterns whose query (bit 0) or key (bit 1) map is the identity on [0, n):
// a position is then its own token, -1 past n, with no load.
__host__ __device__ inline int identity_maps(int kind) {
  switch (kind) {
    case SA_LOCAL: case SA_SAMEBLOCK: case SA_LOCAL_GLOBAL: return 3;
    case SA_SUMMARY: case SA_FIXED_MERGED: return 1;
    default: return 0;
  }
}
__device__ __forceinline__ int identity_token(int pos, int n) { return pos < n ? pos : -1; }

struct PatView {
  const int32_t* qmap;
  const int32_t* kmap;
  const int32_t* lo;
  const int32_t* hi;
  const int32_t* pre;  // key prefix [0, pre[p]) of each row; nullptr = all empty
  int32_t ident;       // bit 0: query map is the identity, bit 1: key map is
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* fflag;
  const int32_t* col_ptr;
  const int32_t* row;
  const uint8_t* bflag;
};

__device__ __forceinline__ PatView pattern_of_index(const uint8_t* blob, int pi) {
  const sa_blob_header* hdr = reinterpret_cast<const sa_blob_header*>(blob);
  const sa_pattern_rec* rec =
      reinterpret_cast<const sa_pattern_rec*>(blob + hdr->pattern_off) + pi;
  PatView v;
  v.qmap = reinterpret_cast<const int32_t*>(blob + rec->qmap_off);
  v.kmap = reinterpret_cast<const int32_t*>(blob + rec->kmap_off);
  v.lo = reinterpret_cast<const int32_t*>(blob + rec->lo_off);
  v.hi = reinterpret_cast<const int32_t*>(blob + rec->hi_off);
  v.pre = rec->pre_off ? reinterpret_cast<const int32_t*>(blob + rec->pre_off) : nullptr;
  v.ident = identity_maps(rec->kind);
  v.row_ptr = reinterpret_cast<const int32_t*>(blob + rec->row_ptr_off);
  v.col = reinterpret_cast<const int32_t*>(blob + rec->col_off);
  v.fflag = blob + rec->fflag_off;
  v.col_ptr = reinterpret_cast<const int32_t*>(blob + rec->col_ptr_off);
  v.row = reinterpret_cast<const int32_t*>(blob + rec->row_off);
  v.bflag = blob + rec->bflag_off;
  return v;
}

__device__ __forceinline__ PatView pattern_of_head(const uint8_t* blob, int head) {
  const sa_blob_header* hdr = reinterpret_cast<const sa_blob_header*>(blob);
  const int32_t* head_pat = reinterpret_cast<const int32_t*>(blob + hdr->head_pattern_off);
  return pattern_of_index(blob, head_pat[head]);
}

// The first kArgPatterns patterns travel in the kernel arguments (resolved on
// the host), so a workgroup reaches its pattern's arrays without a chain of
// dependent loads through the blob; later patterns are read from the blob.
constexpr int kArgPatterns = 8;
struct PatTable {
  PatView pv[kArgPatterns];
};

__device__ __forceinline__ PatView pattern_view(const PatTable& t, const uint8_t* blob, int pi) {
  return pi < kArgPatterns ? t.pv[pi] : pattern_of_index(blob, pi);
}

// Pattern field of a schedule entry: pattern index, (index among two-part
// heads + 1) << 16, and kPartInit on the first chunk of such a head's tile
// (it starts from the state the head's second part left in the workspace).
constexpr int kPartInit = 1 << 30;
__device__ __forceinline__ int field_pattern(int f) { return f & 0xffff; }
__device__ __forceinline__ int field_merged(int f) { return ((f >> 16) & 0x3fff) - 1; }

// A wave's register window over a tile list (CSR or CSC entries [e0, e1)):
// lane l holds entry base + l packed as (tile << 1) | FULL, so the loop reads
// an entry with one readlane instead of a global load whose latency would
// stall the prefetch issued before it (the vector-memory counter drains in
// order).  A loop may read up to two entries ahead of the one it works on:
// entries are requested in non-decreasing order apart from that look-ahead,
// and a window that has to advance starts two entries before the requested
// one, so the entries still in use stay inside it.
struct TileWindow {
  const int32_t* tile;
  const uint8_t* flag;
  int e1, base, packed;
  __device__ __forceinline__ void load(int b) {
    const int e = b + int(__lane_id());
    base = b;
    packed = e < e1 ? (tile[e] << 1) | (flag[e] == SA_TILE_FULL ? 1 : 0) : 0;
  }
  // Entry e (uniform, e >= base); moves the window forward when e is past it.
  __device__ __forceinline__ int get(int e) {
    if (e >= base + 64) load(e - 2);
    return __builtin_amdgcn_readlane(packed, e - base);
  }
};

__device__ __forceinline__ TileWindow tile_window(const int32_t* tile, const uint8_t* flag,
                                                  int e0, int e1) {
  TileWindow w;
  w.tile = tile;
  w.flag = flag;
  w.e1 = e1;
  w.load(e0);
  return w;
}

// Workgroup -> (batch element, schedule entry) through the per-XCD lists of
// the layout (workgroup w runs on XCD w % SA_XCDS), whose entries are stored
// in list order.  Launch grids are SA_XCDS * len * B workgroups; nullptr =
// padding, nothing to do.
__device__ __forceinline__ const int32_t* xcd_work_entry(const int32_t* xitems, int len, int B,
                                                         int* b) {
  const int w = int(blockIdx.x);
  const int x = w % SA_XCDS, j = w / SA_XCDS;
  *b = j / len;
  const int32_t* e = xitems + size_t(x * len + j % len) * SA_SCHED_FIELDS;
  return (*b < B && e[0] >= 0) ? e : nullptr;
}

}  // namespace sa
