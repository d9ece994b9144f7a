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

// Value of lane L ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

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
struct PatView {
  const int32_t* qmap;
  const int32_t* kmap;
  const int32_t* lo;
  const int32_t* hi;
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* fflag;
  const int32_t* col_ptr;
  const int32_t* row;
  const uint8_t* bflag;
};

__device__ __forceinline__ PatView pattern_of_head(const uint8_t* blob, int head) {
  const sa_blob_header* hdr = reinterpret_cast<const sa_blob_header*>(blob);
  const int32_t* head_pat = reinterpret_cast<const int32_t*>(blob + hdr->head_pattern_off);
  const int pi = head_pat[head];
  const sa_pattern_rec* rec =
      reinterpret_cast<const sa_pattern_rec*>(blob + hdr->pattern_off) + pi;
  PatView v;
  v.qmap = reinterpret_cast<const int32_t*>(blob + rec->qmap_off);
  v.kmap = reinterpret_cast<const int32_t*>(blob + rec->kmap_off);
  v.lo = reinterpret_cast<const int32_t*>(blob + rec->lo_off);
  v.hi = reinterpret_cast<const int32_t*>(blob + rec->hi_off);
  v.row_ptr = reinterpret_cast<const int32_t*>(blob + rec->row_ptr_off);
  v.col = reinterpret_cast<const int32_t*>(blob + rec->col_off);
  v.fflag = blob + rec->fflag_off;
  v.col_ptr = reinterpret_cast<const int32_t*>(blob + rec->col_ptr_off);
  v.row = reinterpret_cast<const int32_t*>(blob + rec->row_off);
  v.bflag = blob + rec->bflag_off;
  return v;
}

// Workgroup -> (batch element, schedule entry) through the per-XCD lists of
// the layout (workgroup w runs on XCD w % SA_XCDS).  Launch grids are
// SA_XCDS * len * B workgroups; false = padding, nothing to do.
__device__ __forceinline__ bool xcd_work_item(const int32_t* xl, int len, int B, int* b,
                                              int* item) {
  const int w = int(blockIdx.x);
  const int x = w % SA_XCDS, j = w / SA_XCDS;
  *b = j / len;
  *item = xl[x * len + j % len];
  return *item >= 0 && *b < B;
}

}  // namespace sa
