// Forward kernels: fused block-sparse attention with an online softmax.
//
// One workgroup handles one query tile (block_q rows of one (batch, head)) of
// the layout and walks that tile's CSR list of active key tiles
// ("Sparse Transformers 深度解读报告", section 3.5: blocked sub-blocks of
// Q/K/V, the softmax fused into a single kernel with its intermediates in
// registers, masked-out tiles never computed).  Per key tile:
//   1. K and V rows (through the pattern's key map) are copied straight from
//      global memory into LDS (direct loads, no registers), row-major with
//      XOR-swizzled 16-byte chunks, double-buffered, one barrier per tile;
//      V^T reaches the MFMA through transposing LDS reads;
//   2. each wave owns 32 query rows and computes S^T = K Q^T on the MFMA
//      units (fp32 accumulation; Q stays in registers for the whole walk);
//   3. on PARTIAL tiles the fine mask is a few integer compares against the
//      row's key prefix and interval; FULL tiles apply no mask;
//   4. running max update in base 2 with the softmax scale folded into one
//      FMA per score; the running max (and the rescale of the accumulators)
//      only moves when a tile's max exceeds it by more than 2^kRescaleLog2,
//      so P <= 2^kRescaleLog2 and most tiles skip the rescale; the row max
//      pairs the two half-waves through a lane swap;
//   5. O^T += V^T P^T on the MFMA units, P rounded to the input type; the
//      row sums accumulate the unrounded P in float32.
// The epilogue writes O rows (through the query map) and the per-row
// log-sum-exp that the backward pass rebuilds probabilities from (report
// section 3.4).  A wave skips the arithmetic of a tile none of its rows can
// see (it still takes part in the staging).
//
// Query tiles with long CSR lists run as several chunks (one workgroup each).
// A chunk stores its unnormalised O, running max and running sum in float32;
// a further launch merges the chunks of each split tile exactly (rescaling
// each to the common max) in chunk order.
//
// Merged strided heads run in two parts with disjoint key sets (see the
// layout builder): a launch of the same kernel over the second parts stores
// each token's softmax state (unnormalised O, running max, running sum) in
// the workspace, and the first chunk of each main tile of such a head starts
// its online softmax from that state.

#include <math.h>

#include <type_traits>

#include "device_common.hpp"

namespace sa {

constexpr float kNegInit = -3.0e38f;  // running-max start: exp2(kNegInit - x) == 0
constexpr float kMasked = -1.0e30f;   // masked logit in the base-2 domain (float32 path)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (P <= 256)

struct FwdParams {
  const uint8_t* blob;
  const int32_t* xitems;  // per-XCD lists of query-tile entries (SA_SCHED_FIELDS ints each)
  int32_t xl_len;
  int32_t B, H, n, num_qslots;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;  // [B, num_qslots, BQ, 64]: unnormalised O of a chunk
  float* part_m;  // [B, num_qslots, BQ]: running max (base 2)
  float* part_l;  // [B, num_qslots, BQ]: running sum
  const int32_t* csched;  // (head, q-tile, first slot, chunks) of each split query tile
  // Two-part heads: float32 softmax state of every token after the second
  // part, [B, num_merged, n] rows (unnormalised O of 64 floats, running max
  // base 2, running sum).  `part` != 0 in the launch of the second parts,
  // which write it; the main launch's first chunks read it.
  float* st_o;
  float* st_m;
  float* st_l;
  int32_t num_merged, part;
  float scale_log2;  // softmax scale * log2(e)
  PatTable pats;     // arrays of the first patterns (device addresses)
};


// Merge of a split query tile (all chunks have stored their partials): per
// row, m = max of the chunk maxima, O = sum_c 2^(m_c - m) acc_c / l with
// l = sum_c 2^(m_c - m) l_c, LSE = (m + log2 l) ln 2.  Chunks are taken in
// order.  One thread per (row, 8 features).
template <typename T, int BQ>
__device__ __forceinline__ void fwd_merge_row(const FwdParams& p, const PatView& pv, size_t base,
                                              int b, int qt, int slot0, int chunks, int row,
                                              int part) {
  {
    const int tok = pv.qmap[qt * BQ + row];
    if (tok < 0) return;
    const size_t r0 = (size_t(b) * p.num_qslots + slot0) * BQ + row;
    float m = -INFINITY;
    for (int c = 0; c < chunks; ++c) m = fmaxf(m, p.part_m[r0 + size_t(c) * BQ]);
    float l = 0.f;
    floatx4 a = floatx4{}, a2 = floatx4{};
    for (int c = 0; c < chunks; ++c) {
      const size_t rc = r0 + size_t(c) * BQ;
      const float wgt = fast_exp2(p.part_m[rc] - m);
      l += wgt * p.part_l[rc];
      const floatx4* src = reinterpret_cast<const floatx4*>(p.part_o + rc * kD + 8 * part);
      a += wgt * src[0];
      a2 += wgt * src[1];
    }
    const float inv = 1.0f / l;
    float tmp[8] = {a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv,
                    a2[0] * inv, a2[1] * inv, a2[2] * inv, a2[3] * inv};
    T* dst = static_cast<T*>(p.o) + (base + size_t(tok)) * kD + 8 * part;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x8*>(dst) = pack_bf16x8(tmp);
    } else {
      *reinterpret_cast<floatx4*>(dst) = floatx4{tmp[0], tmp[1], tmp[2], tmp[3]};
      *reinterpret_cast<floatx4*>(dst + 4) = floatx4{tmp[4], tmp[5], tmp[6], tmp[7]};
    }
    if (part == 0) p.lse[base + tok] = (m + log2f(l)) * kLn2;
  }
}

// Epilogue shared by both element types.  Register r of half g of oacc[fb]
// holds feature 32*fb + kappa(r, g) of the lane's query row; l_tot is the
// row's full sum of probabilities.  Unsplit tiles
// write O = acc / l and LSE; chunks of split tiles store (acc, m, l).
template <typename T, int BQ>
__device__ __forceinline__ void fwd_epilogue(const FwdParams& p, const floatx16 (&oacc)[2],
                                             float m_run, float l_tot, int tok, size_t base,
                                             int b, int slot, int row, int g) {
  if (slot < 0) {
    if (tok < 0) return;
    const float inv = 1.0f / l_tot;
    T* orow = static_cast<T*>(p.o) + (base + size_t(tok)) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = oacc[fb][8 * h8 + j] * inv;
        T* dst = orow + 32 * fb + 16 * h8 + 8 * g;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x8*>(dst) = pack_bf16x8(tmp);
        } else {
          *reinterpret_cast<floatx4*>(dst) = floatx4{tmp[0], tmp[1], tmp[2], tmp[3]};
          *reinterpret_cast<floatx4*>(dst + 4) = floatx4{tmp[4], tmp[5], tmp[6], tmp[7]};
        }
      }
    if (g == 0) p.lse[base + tok] = (m_run + log2f(l_tot)) * kLn2;
    return;
  }
  const size_t prow = (size_t(b) * p.num_qslots + slot) * BQ + row;
  float* po = p.part_o + prow * kD;
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const int f0 = 32 * fb + 16 * h8 + 8 * g;
      *reinterpret_cast<floatx4*>(po + f0) =
          floatx4{oacc[fb][8 * h8], oacc[fb][8 * h8 + 1], oacc[fb][8 * h8 + 2], oacc[fb][8 * h8 + 3]};
      *reinterpret_cast<floatx4*>(po + f0 + 4) = floatx4{oacc[fb][8 * h8 + 4], oacc[fb][8 * h8 + 5],
                                                         oacc[fb][8 * h8 + 6], oacc[fb][8 * h8 + 7]};
    }
  if (g == 0) {
    p.part_m[prow] = m_run;
    p.part_l[prow] = l_tot;
  }
}

// --------------------------------------------------------------------------
// bfloat16 inputs, 32x32x16 bf16 MFMA
// --------------------------------------------------------------------------
// Occupancy: 2 waves per SIMD for query tiles of 64 and more rows (measured
// faster than 3: with two 128-row workgroups per CU, fewer long query tiles
// run at once and the longest-first list order evens out the CUs' work), and
// up to 3 for 32-row tiles (one-wave workgroups, 10 per CU by LDS).
template <int BQ, int BK, bool PRE>
__global__ __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(2, BQ >= 64 ? 2 : 3)))
void fwd_bf16_kernel(FwdParams p) {
  constexpr int NW = BQ / 32;
  constexpr int NKB = BK / 32;
  constexpr int IPW = BK / 8 / NW;  // 1 KB direct loads per wave, tensor and tile
  static_assert(IPW >= 1 && (BK / 8) % NW == 0, "tile/wave mismatch");
  // Two buffers per tensor as separate arrays, selected by a compile-time
  // parity (the loop is unrolled by two): the compiler can then tell that the
  // reads of one buffer never touch the direct loads in flight into the other,
  // and does not drain those loads before the reads.
  __shared__ __attribute__((aligned(16))) bf16 k0s[BK * kD], k1s[BK * kD];
  __shared__ __attribute__((aligned(16))) bf16 v0s[BK * kD], v1s[BK * kD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b;
  const int32_t* it8 = xcd_work_entry(p.xitems, p.xl_len, p.B, &b);
  if (!it8) return;
  const int head = it8[0], qt = it8[1], e0 = it8[2], e1 = it8[3], pf = it8[5];
  const PatView pv = pattern_view(p.pats, p.blob, field_pattern(pf));
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const bf16* qg = static_cast<const bf16*>(p.q) + base * kD;
  const bf16* kg = static_cast<const bf16*>(p.k) + base * kD;
  const bf16* vg = static_cast<const bf16*>(p.v) + base * kD;

  const int prow = qt * BQ + w * 32 + l32;
  const int tok = (pv.ident & 1) ? identity_token(prow, p.n) : pv.qmap[prow];
  const int lo = pv.lo[prow], hi = pv.hi[prow];
  // PRE: some pattern of the layout has key prefixes; this head's pattern may
  // still have none (no array).
  const int pre = (PRE && pv.pre) ? pv.pre[prow] : 0;

  bf16x8 qf[4];
  if (tok >= 0) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(qg + size_t(tok) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = src[2 * c + g];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = bf16x8{};
  }

  // Staging of K and V tiles: wave w fills rows [8 (w IPW + i), +8) of each
  // tile with its i-th direct load.  Padding keys (map entry -1) fetch token
  // 0 instead: they are never visible, so their probabilities are exactly 0.
  const int drow = lane >> 3;
  const BufRsrc krs = slice_rsrc(kg, uint32_t(p.n) * uint32_t(kD * 2));
  const BufRsrc vrs = slice_rsrc(vg, uint32_t(p.n) * uint32_t(kD * 2));
  const BufRsrc kmap_rs = array_rsrc(pv.kmap);
  int kidx[IPW];  // key-map entries of the next tile to load (fetched a tile early)
  auto iload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int pos = kt * BK + 8 * (w * IPW + i) + drow;
      kidx[i] = (pv.ident & 2) ? identity_token(pos, p.n) : buf_i32(kmap_rs, pos);
    }
  };
  auto dload = [&](auto par) {
    constexpr int P = decltype(par)::value;
    bf16* kd = P ? k1s : k0s;
    bf16* vd = P ? v1s : v0s;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t off = row_chunk_offset(kidx[i], (lane & 7) ^ swz_key(8 * (w * IPW + i) + drow));
      dma16_buf(krs, off, kd + 8 * (w * IPW + i) * kD);
      dma16_buf(vrs, off, vd + 8 * (w * IPW + i) * kD);
    }
  };

  floatx16 oacc[2];
  oacc[0] = floatx16{};
  oacc[1] = floatx16{};
  float m_run = kNegInit, l_run = 0.f;  // l_run: this half-wave's share of the row sum
  // Main part of a two-part head: start from the second part's state.
  const size_t srow = (size_t(b) * p.num_merged + field_merged(pf)) * size_t(p.n) + size_t(tok);
  if ((pf & kPartInit) && tok >= 0) {
    m_run = p.st_m[srow];
    l_run = g == 0 ? p.st_l[srow] : 0.f;
    const float* so = p.st_o + srow * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(so + 32 * fb + 16 * h8 + 8 * g);
        const floatx4 c = *reinterpret_cast<const floatx4*>(so + 32 * fb + 16 * h8 + 8 * g + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          oacc[fb][8 * h8 + j] = a[j];
          oacc[fb][8 * h8 + 4 + j] = c[j];
        }
      }
  }
  const float c2 = p.scale_log2;

  TileWindow win = tile_window(pv.col, pv.fflag, e0, e1);
  if (e0 < e1) {
    iload(it8[8] >> 1);  // the first entry travels in the schedule entry
    dload(std::integral_constant<int, 0>{});
    if (e0 + 1 < e1) iload(win.get(e0 + 1) >> 1);
  }
  wait_vmem();
  __syncthreads();
  // One tile; P = parity of (it - e0) selects the buffers.
  auto tile_step = [&](auto par, int it) {
    constexpr int P = decltype(par)::value;
    const bf16* kcur = P ? k1s : k0s;
    const bf16* vcur = P ? v1s : v0s;
    const int ent = win.get(it);
    const int kt = ent >> 1;
    const bool full = (ent & 1) != 0;
    if (it + 1 < e1) {
      dload(std::integral_constant<int, 1 - P>{});       // tile it+1, indices already here
      if (it + 2 < e1) iload(win.get(it + 2) >> 1);    // indices of tile it+2
    }
    const int k0 = kt * BK;
    const bool mine = ((lo <= hi) && (lo <= k0 + BK - 1) && (hi >= k0)) || (PRE && pre > k0);
    if (__any(mine)) {
      floatx16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = floatx16{};
        const int kr = 32 * kb + sigma32(l32);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          s[kb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(&kcur[swz(kr, g + 2 * c)]), qf[c],
                            s[kb]);
      }
      if (!full) {
        // Key k0 + c is visible iff k0 + c < pre or lo <= k0 + c <= hi;
        // c = 32*kb + kappa(r, g) = 8*g + (a constant per register).
        if (__all(lo > hi || lo <= k0)) {
          // Every row's visible keys in this tile end at one bound (the usual
          // causal diagonal): hi when its interval starts at or before the
          // tile (a prefix ends before the interval), pre - 1 when the
          // interval is empty.  One compare per score.
          const int up_rel = (lo <= hi ? hi : pre - 1) - k0 - 8 * g;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int cr = 32 * kb + 16 * (r >> 3) + (r & 7);
              s[kb][r] = cr <= up_rel ? s[kb][r] : -INFINITY;
            }
        } else {
          const int lo_rel = lo - k0 - 8 * g, hi_rel = hi - k0 - 8 * g, pre_rel = pre - k0 - 8 * g;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int cr = 32 * kb + 16 * (r >> 3) + (r & 7);
              s[kb][r] = ((PRE && cr < pre_rel) || (cr >= lo_rel && cr <= hi_rel)) ? s[kb][r] : -INFINITY;
            }
        }
      }
      float mx = -INFINITY;  // max of the raw scores (scale > 0)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair_max(mx) * c2;
      if (__any(mx > m_run + kRescaleLog2)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          oacc[0][r] *= alpha;
          oacc[1][r] *= alpha;
        }
        m_run = m_new;
      }
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = fast_exp2(fmaf(s[kb][r], c2, -m_run));
          lsum += s[kb][r];
        }
      l_run += lsum;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          float tmp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) tmp[j] = s[kb][8 * h8 + j];
          const bf16x8 pb = pack_bf16x8(tmp);
#pragma unroll
          for (int fb = 0; fb < 2; ++fb)
            oacc[fb] = mfma_bf16(load_a_transposed_swz(vcur, 32 * kb + 16 * h8, 32 * fb, lane),
                                 pb, oacc[fb]);
        }
      }
    }
    wait_vmem();  // tile it+1 is in LDS (this wave's part)
    __syncthreads();
  };
  for (int it = e0; it < e1; it += 2) {
    tile_step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < e1) tile_step(std::integral_constant<int, 1>{}, it + 1);
  }

  const float l_tot = pair_sum(l_run);
  if (p.part) {
    // Second part of a two-part head: keep the state for the main part.
    if (tok >= 0) {
      float* so = p.st_o + srow * kD;
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const int f0 = 32 * fb + 16 * h8 + 8 * g;
          *reinterpret_cast<floatx4*>(so + f0) = floatx4{oacc[fb][8 * h8], oacc[fb][8 * h8 + 1],
                                                         oacc[fb][8 * h8 + 2], oacc[fb][8 * h8 + 3]};
          *reinterpret_cast<floatx4*>(so + f0 + 4) =
              floatx4{oacc[fb][8 * h8 + 4], oacc[fb][8 * h8 + 5], oacc[fb][8 * h8 + 6], oacc[fb][8 * h8 + 7]};
        }
      if (g == 0) {
        p.st_m[srow] = m_run;
        p.st_l[srow] = l_tot;
      }
    }
    return;
  }
  fwd_epilogue<bf16, BQ>(p, oacc, m_run, l_tot, tok, base, b, it8[4], w * 32 + l32, g);
}

// --------------------------------------------------------------------------
// float32 inputs, 32x32x2 f32 MFMA (same structure; K slot = one feature)
// --------------------------------------------------------------------------
template <int BQ, int BK, bool PRE>
__global__ __launch_bounds__(BQ * 2) void fwd_f32_kernel(FwdParams p) {
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  constexpr int NKB = BK / 32;
  constexpr int KS = kD + 4;
  constexpr int VS = BK + 4;
  constexpr int CPT = BK * 16 / NT;
  static_assert(CPT >= 1 && (BK * 16) % NT == 0, "tile/wave mismatch");
  __shared__ __attribute__((aligned(16))) float ks[2][BK * KS];
  __shared__ __attribute__((aligned(16))) float vt[2][kD * VS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b;
  const int32_t* it8 = xcd_work_entry(p.xitems, p.xl_len, p.B, &b);
  if (!it8) return;
  const int head = it8[0], qt = it8[1], e0 = it8[2], e1 = it8[3];
  const PatView pv = pattern_view(p.pats, p.blob, field_pattern(it8[5]));
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const float* qg = static_cast<const float*>(p.q) + base * kD;
  const float* kg = static_cast<const float*>(p.k) + base * kD;
  const float* vg = static_cast<const float*>(p.v) + base * kD;

  const int prow = qt * BQ + w * 32 + l32;
  const int tok = pv.qmap[prow];
  const int lo = pv.lo[prow], hi = pv.hi[prow];
  // PRE: some pattern of the layout has key prefixes; this head's pattern may
  // still have none (no array).
  const int pre = (PRE && pv.pre) ? pv.pre[prow] : 0;

  float qf[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) qf[c] = tok >= 0 ? qg[size_t(tok) * kD + 2 * c + g] : 0.f;

  floatx4 kreg[CPT], vreg[CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, j = c >> 4, cc = c & 15;
      const int tk = pv.kmap[kt * BK + j];
      if (tk >= 0) {
        kreg[i] = reinterpret_cast<const floatx4*>(kg + size_t(tk) * kD)[cc];
        vreg[i] = reinterpret_cast<const floatx4*>(vg + size_t(tk) * kD)[cc];
      } else {
        kreg[i] = floatx4{};
        vreg[i] = floatx4{};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, j = c >> 4, cc = c & 15;
      *reinterpret_cast<floatx4*>(&ks[buf][j * KS + cc * 4]) = kreg[i];
#pragma unroll
      for (int t = 0; t < 4; ++t) vt[buf][(cc * 4 + t) * VS + j] = vreg[i][t];
    }
  };

  floatx16 oacc[2];
  oacc[0] = floatx16{};
  oacc[1] = floatx16{};
  float m_run = kNegInit, l_run = 0.f;
  const float c2 = p.scale_log2;

  if (e0 < e1) {
    gload(pv.col[e0]);
    lstore(0);
  }
  __syncthreads();
  for (int it = e0; it < e1; ++it) {
    const int buf = (it - e0) & 1;
    const int kt = pv.col[it];
    const bool full = pv.fflag[it] == SA_TILE_FULL;
    if (it + 1 < e1) gload(pv.col[it + 1]);
    const int k0 = kt * BK;
    const bool mine = ((lo <= hi) && (lo <= k0 + BK - 1) && (hi >= k0)) || (PRE && pre > k0);
    if (__any(mine)) {
      floatx16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = floatx16{};
        const float* krow = &ks[buf][(32 * kb + sigma32(l32)) * KS + g];
#pragma unroll
        for (int c = 0; c < 32; ++c) s[kb] = mfma_f32(krow[2 * c], qf[c], s[kb]);
      }
      float mx = kNegInit;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kp = k0 + 32 * kb + kappa32(r, g);
          const float x = (full || (PRE && kp < pre) || (kp >= lo && kp <= hi)) ? s[kb][r] * c2 : kMasked;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(s[kb][r] - m_new);
          s[kb][r] = pr;
          lsum += pr;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        oacc[0][r] *= alpha;
        oacc[1][r] *= alpha;
      }
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const float* vrow = &vt[buf][(32 * fb + sigma32(l32)) * VS];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[fb] = mfma_f32(vrow[32 * kb + kappa32(r, g)], s[kb][r], oacc[fb]);
      }
    }
    if (it + 1 < e1) lstore(buf ^ 1);
    __syncthreads();
  }

  fwd_epilogue<float, BQ>(p, oacc, m_run, pair_sum(l_run), tok, base, b, it8[4], w * 32 + l32, g);
}

// --------------------------------------------------------------------------
// Merge the chunks of split query tiles: with chunk c holding (O_c, m_c, l_c)
// (unnormalised O, base-2 running max, running sum), m = max_c m_c,
// l = sum_c 2^(m_c - m) l_c, O = sum_c 2^(m_c - m) O_c / l, LSE = (m + log2 l) ln 2.
// Chunks are summed in chunk order.  8 threads per row (8 features each).
// --------------------------------------------------------------------------
// Merge launch: one workgroup of 256 threads per (batch element, split query
// tile, 32-row block of the tile); thread = (row, 8 features).
template <typename T, int BQ>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  constexpr int RB = BQ / 32;  // row blocks per tile
  const int b = blockIdx.x % p.B;
  const int gi = blockIdx.x / p.B;
  const int32_t* c4 = p.csched + 4 * (gi / RB);
  const PatView pv = pattern_of_head(p.blob, c4[0]);
  const size_t base = (size_t(b) * p.H + c4[0]) * size_t(p.n);
  const int row = (gi % RB) * 32 + (threadIdx.x >> 3);
  fwd_merge_row<T, BQ>(p, pv, base, b, c4[1], c4[2], c4[3], row, threadIdx.x & 7);
}

}  // namespace sa

// --------------------------------------------------------------------------
// C ABI entry point
// --------------------------------------------------------------------------
#include "abi_common.hpp"

namespace {

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [partial O float32[B, slots, BQ, 64]] [partial max float32[B,
// slots, BQ]] [partial sum, same]; each part starts on a 256-byte boundary.
// Empty when no query tile is split.
struct FwdWorkspace {
  size_t part_o, part_m, part_l, st_o, st_m, st_l, total;
};

// Chunk partials of split query tiles, then the token state of two-part heads.
FwdWorkspace fwd_workspace_layout(int B, const sa_blob_header& h) {
  FwdWorkspace w{};
  if (B == 0) return w;
  const size_t rows = size_t(B) * size_t(h.num_qslots) * size_t(h.block_q);
  const size_t srows = size_t(B) * size_t(h.num_merged) * size_t(h.n);
  w.part_o = 0;
  w.part_m = w.part_o + round256(rows * sa::kD * sizeof(float));
  w.part_l = w.part_m + round256(rows * sizeof(float));
  w.st_o = w.part_l + round256(rows * sizeof(float));
  w.st_m = w.st_o + round256(srows * sa::kD * sizeof(float));
  w.st_l = w.st_m + round256(srows * sizeof(float));
  w.total = w.st_l + round256(srows * sizeof(float));
  return w;
}

}  // namespace

extern "C" int sparse_attn_fwd_workspace(const void* blob_host, int B, int H, int d, int dtype,
                                         size_t* bytes) {
  using namespace sa;
  if (!bytes || !blob_host) return SA_EINVAL;
  sa_blob_header h;
  memcpy(&h, blob_host, sizeof(h));
  if (h.magic != SA_BLOB_MAGIC || h.version != SA_BLOB_VERSION) return SA_EINVAL;
  if (B < 0 || H < 1 || H != h.num_heads) return SA_EINVAL;
  if (dtype != SA_BF16 && dtype != SA_FP32) return SA_EINVAL;
  if (d != 64) return SA_EUNSUPPORTED;
  *bytes = fwd_workspace_layout(B, h).total;
  return SA_OK;
}

extern "C" int sparse_attn_fwd_phases(const void* blob_host, const void* blob_dev, int B, int H,
                                      int d, int dtype, const void* q, const void* k,
                                      const void* v, void* o, float* lse, void* workspace,
                                      size_t ws_bytes, float scale, unsigned phases,
                                      void* stream) {
  using namespace sa;
  if (phases == 0 || (phases & ~unsigned(SA_FWD_ALL)) != 0) return SA_EINVAL;
  LaunchInfo li;
  int rc = validate_common(blob_host, blob_dev, B, H, d, dtype, &li);
  if (rc != SA_OK) return rc;
  float sc;
  rc = resolve_scale(scale, d, &sc);
  if (rc != SA_OK) return rc;
  sa_blob_header h;
  memcpy(&h, blob_host, sizeof(h));
  const int bq = li.block_q, bk = li.block_k;
  const bool shape_ok =
      dtype == SA_BF16 ? (bk == 32 || bk == 64 || (bq == 128 && bk == 128)) : (bk == 32);
  if (!shape_ok) return SA_EUNSUPPORTED;
  if (dtype != SA_BF16 && li.num_merged > 0) return SA_EUNSUPPORTED;  // two-part heads: bf16 only
  if (B == 0 || li.fwd_xl_len == 0) return SA_OK;  // empty batch: pointers may be NULL
  const FwdWorkspace wl = fwd_workspace_layout(B, h);
  if (ws_bytes < wl.total) return SA_ESIZE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (wl.total > 0 && !aligned16(workspace)))
    return SA_EINVAL;
  const int64_t grid = int64_t(SA_XCDS) * li.fwd_xl_len * B;
  const int64_t mgrid = int64_t(h.comb_sched_len) * (bq / 32) * B;
  const int64_t pgrid = int64_t(SA_XCDS) * li.fwdp_xl_len * B;
  if (grid > INT32_MAX || mgrid > INT32_MAX || pgrid > INT32_MAX) return SA_EUNSUPPORTED;

  FwdParams prm;
  prm.blob = static_cast<const uint8_t*>(blob_dev);
  prm.xitems = reinterpret_cast<const int32_t*>(prm.blob + li.fwd_xitem_off);
  fill_pattern_table(blob_host, blob_dev, &prm.pats);
  prm.xl_len = li.fwd_xl_len;
  prm.B = B;
  prm.H = H;
  prm.n = int32_t(li.n);
  prm.num_qslots = h.num_qslots;
  prm.csched = reinterpret_cast<const int32_t*>(prm.blob + h.comb_sched_off);
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool split = wl.total > 0;
  prm.part_o = split ? reinterpret_cast<float*>(ws + wl.part_o) : nullptr;
  prm.part_m = split ? reinterpret_cast<float*>(ws + wl.part_m) : nullptr;
  prm.part_l = split ? reinterpret_cast<float*>(ws + wl.part_l) : nullptr;
  prm.st_o = split ? reinterpret_cast<float*>(ws + wl.st_o) : nullptr;
  prm.st_m = split ? reinterpret_cast<float*>(ws + wl.st_m) : nullptr;
  prm.st_l = split ? reinterpret_cast<float*>(ws + wl.st_l) : nullptr;
  prm.num_merged = li.num_merged;
  prm.part = 0;
  prm.scale_log2 = float(double(sc) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
#define SA_LAUNCH(kern, g, threads) \
  hipLaunchKernelGGL(kern, dim3(unsigned(g)), dim3(threads), 0, st, prm)
// Kernels for layouts with key prefixes are separate instantiations, so the
// other layouts run code without the prefix compares.
#define SA_LAUNCH_P(KN, A, C, g, threads)               \
  do {                                                  \
    if (li.has_pre) SA_LAUNCH((KN<A, C, true>), g, threads); \
    else SA_LAUNCH((KN<A, C, false>), g, threads);      \
  } while (0)
  if ((phases & SA_FWD_MAIN) && pgrid > 0) {
    // Second parts of two-part heads first: they leave the softmax state of
    // every token for the main launch.
    FwdParams pp = prm;
    pp.part = 1;
    pp.xitems = reinterpret_cast<const int32_t*>(pp.blob + li.fwdp_xitem_off);
    pp.xl_len = li.fwdp_xl_len;
#define SA_LAUNCH_PART(BQv, BKv, threads)                                                        \
  hipLaunchKernelGGL((fwd_bf16_kernel<BQv, BKv, false>), dim3(unsigned(pgrid)), dim3(threads), 0, \
                     st, pp)
    if (bq == 32 && bk == 32) SA_LAUNCH_PART(32, 32, 64);
    else if (bq == 32 && bk == 64) SA_LAUNCH_PART(32, 64, 64);
    else if (bq == 64 && bk == 32) SA_LAUNCH_PART(64, 32, 128);
    else if (bq == 64 && bk == 64) SA_LAUNCH_PART(64, 64, 128);
    else if (bq == 128 && bk == 32) SA_LAUNCH_PART(128, 32, 256);
    else if (bq == 128 && bk == 64) SA_LAUNCH_PART(128, 64, 256);
    else SA_LAUNCH_PART(128, 128, 256);
#undef SA_LAUNCH_PART
  }
  if (phases & SA_FWD_MAIN) {
    if (dtype == SA_BF16) {
      if (bq == 32 && bk == 32) SA_LAUNCH_P(fwd_bf16_kernel, 32, 32, grid, 64);
      else if (bq == 32 && bk == 64) SA_LAUNCH_P(fwd_bf16_kernel, 32, 64, grid, 64);
      else if (bq == 64 && bk == 32) SA_LAUNCH_P(fwd_bf16_kernel, 64, 32, grid, 128);
      else if (bq == 64 && bk == 64) SA_LAUNCH_P(fwd_bf16_kernel, 64, 64, grid, 128);
      else if (bq == 128 && bk == 32) SA_LAUNCH_P(fwd_bf16_kernel, 128, 32, grid, 256);
      else if (bq == 128 && bk == 64) SA_LAUNCH_P(fwd_bf16_kernel, 128, 64, grid, 256);
      else SA_LAUNCH_P(fwd_bf16_kernel, 128, 128, grid, 256);
    } else {
      if (bq == 32) SA_LAUNCH_P(fwd_f32_kernel, 32, 32, grid, 64);
      else if (bq == 64) SA_LAUNCH_P(fwd_f32_kernel, 64, 32, grid, 128);
      else SA_LAUNCH_P(fwd_f32_kernel, 128, 32, grid, 256);
    }
  }
  if ((phases & SA_FWD_MERGE) && mgrid > 0) {
    if (dtype == SA_BF16) {
      if (bq == 32) SA_LAUNCH((fwd_merge_kernel<bf16, 32>), mgrid, 256);
      else if (bq == 64) SA_LAUNCH((fwd_merge_kernel<bf16, 64>), mgrid, 256);
      else SA_LAUNCH((fwd_merge_kernel<bf16, 128>), mgrid, 256);
    } else {
      if (bq == 32) SA_LAUNCH((fwd_merge_kernel<float, 32>), mgrid, 256);
      else if (bq == 64) SA_LAUNCH((fwd_merge_kernel<float, 64>), mgrid, 256);
      else SA_LAUNCH((fwd_merge_kernel<float, 128>), mgrid, 256);
    }
  }
#undef SA_LAUNCH_P
#undef SA_LAUNCH
  return hipGetLastError() == hipSuccess ? SA_OK : SA_EHIP;
}

extern "C" int sparse_attn_fwd(const void* blob_host, const void* blob_dev, int B, int H, int d,
                               int dtype, const void* q, const void* k, const void* v, void* o,
                               float* lse, void* workspace, size_t ws_bytes, float scale,
                               void* stream) {
  return sparse_attn_fwd_phases(blob_host, blob_dev, B, H, d, dtype, q, k, v, o, lse, workspace,
                                ws_bytes, scale, SA_FWD_ALL, stream);
}
