// Backward kernels: gradients by recomputation from the per-row log-sum-exp.
//
// "Sparse Transformers 深度解读报告", section 3.4: attention weights are not
// kept from the forward pass; the backward pass rebuilds them.  With
// P_ij = exp(S_ij - LSE_i) on the visible pairs:
//     dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
//     dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,
//     dK_j = scale sum_i dS_ij q_i.
//
// Launches on the caller's stream:
//   bwd_dq    one workgroup per query tile (the forward's tiling, long tiles
//             in chunks): D_i for its rows (kept in the workspace for the
//             next pass), then a walk of the tile's CSR key tiles: S^T = K Q^T
//             and dP^T = V dO^T on the MFMA units, P and dS in registers,
//             dQ^T += K^T dS^T on the MFMA units; dQ written once;
//   bwd_dkdv  one workgroup per key tile (or per chunk of a long key tile's
//             CSC list): each wave owns 32 keys with K, V held as MFMA
//             operands and dK, dV accumulated in registers; per query tile,
//             Q, dO (row-major), LSE and D are staged in LDS; S = Q K^T and
//             dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T
//             through transposing LDS reads, issued before the softmax so
//             their latency overlaps it).  Unsplit tiles write dK, dV (exact
//             zeros for keys no query reads).
// Chunks of split tiles store float32 partial sums in the workspace; a third
// launch (bwd_merge) sums the chunks of every split key tile (dK, dV) and
// split query tile (dQ) in chunk order and writes their gradients.  No
// atomics: every result is deterministic.
//
// Merged strided heads run in two parts with disjoint key sets: before each
// of the two passes, a launch of the same kernel over the second parts stores
// each token's dQ (or dK, dV) sums in the workspace, and the first chunk of
// each main tile of such a head starts from them.

#include <limits.h>
#include <math.h>

#include <type_traits>

#include "device_common.hpp"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const uint8_t* blob;
  const int32_t* qitems;    // per-XCD lists of query-tile entries (the forward's)
  const int32_t* kitems;    // per-XCD lists of key-tile entries
  const int32_t* sitems;    // per-XCD lists of segments (segment pass)
  int32_t qxl_len, kxl_len, sxl_len;
  int32_t B, H, n, num_slots, num_qslots;
  const int32_t* rsched;    // (head, k-tile, first slot, chunks) of each split key tile
  const int32_t* csched;    // (head, q-tile, first slot, chunks) of each split query tile
  int32_t kgroups;          // split key tiles (rsched entries)
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dsum;     // D, [B, H, n]
  float* partial;  // [B, num_slots, 2, BK, 64]: dK, dV chunks of split key tiles
  float* part_dq;  // [B, num_qslots, BQ, 64]: dQ chunks of split query tiles
  // Two-part heads: float32 sums of every token after the second part,
  // [B, num_merged, n, 64] each (dQ, dK, dV before the scale).  `part` != 0
  // in the launches of the second parts, which write them; the main
  // launches' first chunks read them.
  float* st_dq;
  float* st_dk;
  float* st_dv;
  int32_t num_merged, part;
  float scale;
  float scale_log2;
  PatTable pats;  // arrays of the first patterns (device addresses)
};

// Store the 64 features of a lane's row from two 32x32 accumulators (register
// r of half g: feature 32*fb + kappa(r, g)) as float32, times `scale`.
__device__ __forceinline__ void store_rows16(float* dst, const floatx16 (&acc)[2], int g, float scale) {
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const int f0 = 32 * fb + 16 * h8 + 8 * g;
      floatx4 x0, x1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x0[j] = acc[fb][8 * h8 + j] * scale;
        x1[j] = acc[fb][8 * h8 + 4 + j] * scale;
      }
      *reinterpret_cast<floatx4*>(dst + f0) = x0;
      *reinterpret_cast<floatx4*>(dst + f0 + 4) = x1;
    }
}

// Load what store_rows16 stored (scale 1) into two accumulators.
__device__ __forceinline__ void load_rows16(const float* src, floatx16 (&acc)[2], int g) {
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(src + 32 * fb + 16 * h8 + 8 * g);
      const floatx4 c = *reinterpret_cast<const floatx4*>(src + 32 * fb + 16 * h8 + 8 * g + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[fb][8 * h8 + j] = a[j];
        acc[fb][8 * h8 + 4 + j] = c[j];
      }
    }
}

// --------------------------------------------------------------------------
// dQ pass: one workgroup per query tile, BQ = 32 * NW rows, key tiles of BK.
// --------------------------------------------------------------------------
template <int BQ, int BK, bool PRE>
__global__ __launch_bounds__(BQ * 2, (BQ == 32 && BK == 64) ? 1 : 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int NW = BQ / 32;
  constexpr int NKB = BK / 32;
  constexpr int IPW = BK / 8 / NW;  // 1 KB direct loads per wave, tensor and tile
  static_assert(IPW >= 1 && (BK / 8) % NW == 0, "tile/wave mismatch");
  // Swizzled tiles, two buffers per tensor as separate arrays selected by a
  // compile-time parity (loop unrolled by two), so that reads of one buffer
  // are not made to wait for the direct loads in flight into the other.
  __shared__ __attribute__((aligned(16))) bf16 k0s[BK * kD], k1s[BK * kD];
  __shared__ __attribute__((aligned(16))) bf16 v0s[BK * kD], v1s[BK * kD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b;
  const int32_t* it8 = xcd_work_entry(p.qitems, p.qxl_len, p.B, &b);
  if (!it8) return;
  const int head = it8[0], qt = it8[1], e0 = it8[2], e1 = it8[3], slot = it8[4], pf = it8[5];
  const PatView pv = pattern_view(p.pats, p.blob, field_pattern(pf));
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);

  const int prow = qt * BQ + w * 32 + l32;
  const int tok = (pv.ident & 1) ? identity_token(prow, p.n) : pv.qmap[prow];
  const int lo = pv.lo[prow], hi = pv.hi[prow];
  // PRE: some pattern of the layout has key prefixes; this head's pattern may
  // still have none (no array).
  const int pre = (PRE && pv.pre) ? pv.pre[prow] : 0;

  bf16x8 qf[4], dof[4];
  float dsum = 0.f, lse2 = 0.f;
  if (tok >= 0) {
    const bf16x8* qsrc = reinterpret_cast<const bf16x8*>(p.q + (base + tok) * kD);
    const bf16x8* dsrc = reinterpret_cast<const bf16x8*>(p.dout + (base + tok) * kD);
    const bf16x8* osrc = reinterpret_cast<const bf16x8*>(p.o + (base + tok) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = qsrc[2 * c + g];
      dof[c] = dsrc[2 * c + g];
      const bf16x8 oo = osrc[2 * c + g];
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += float(oo[j]) * float(dof[c][j]);
    }
    lse2 = p.lse[base + tok] * kLog2e;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = bf16x8{};
      dof[c] = bf16x8{};
    }
  }
  dsum = pair_sum(dsum);
  if (tok >= 0 && g == 0) p.dsum[base + tok] = dsum;
  floatx16 ndv;  // -D of the lane's row in every register: seeds the dP accumulator
#pragma unroll
  for (int r = 0; r < 16; ++r) ndv[r] = -dsum;

  // K, V tiles by direct loads, as in the forward; padding keys fetch token 0
  // (never visible: their probabilities, hence dS, are exactly 0).
  const BufRsrc krs = slice_rsrc(p.k + base * kD, uint32_t(p.n) * uint32_t(kD * 2));
  const BufRsrc vrs = slice_rsrc(p.v + base * kD, uint32_t(p.n) * uint32_t(kD * 2));
  const int drow = lane >> 3;
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

  floatx16 dqa[2];
  dqa[0] = dqa[1] = floatx16{};
  // Register r of half g: feature 32*fb + kappa(r, g); lane = query row.
  const size_t srow = (size_t(b) * p.num_merged + field_merged(pf)) * size_t(p.n) + size_t(tok);
  if ((pf & kPartInit) && tok >= 0) load_rows16(p.st_dq + srow * kD, dqa, g);  // main part of a two-part head
  const float c2 = p.scale_log2;
  TileWindow win = tile_window(pv.col, pv.fflag, e0, e1);
  if (e0 < e1) {
    iload(it8[8] >> 1);  // the first entry travels in the schedule entry
    dload(std::integral_constant<int, 0>{});
    if (e0 + 1 < e1) iload(win.get(e0 + 1) >> 1);
  }
  wait_vmem();
  __syncthreads();
  // One key tile; P = parity of (it - e0) selects the buffers.
  auto key_step = [&](auto par, int it) {
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
    // One tile; MASK is a compile-time copy of the tile's mask kind so the
    // element loops carry no branch: 0 FULL (no mask), 1 every row's visible
    // keys in the tile end at one bound (up_rel), 2 prefix and interval.
    const int up = lo <= hi ? hi : pre - 1;
    auto tile = [&](auto mask_tag) {
      constexpr int MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        floatx16 s = floatx16{}, dp = ndv;  // dp accumulates dP - D
        const int kr = 32 * kb + sigma32(l32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int off = swz(kr, g + 2 * c);
          s = mfma_bf16(*reinterpret_cast<const bf16x8*>(&kcur[off]), qf[c], s);
          dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(&vcur[off]), dof[c], dp);
        }
        // Register r of half g: key k0 + 32*kb + kappa(r, g); lane = query.
        const int lo_rel = lo - k0 - 32 * kb - 8 * g, hi_rel = hi - k0 - 32 * kb - 8 * g;
        const int pre_rel = pre - k0 - 32 * kb - 8 * g, up_rel = up - k0 - 32 * kb - 8 * g;
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(fmaf(s[r], c2, -lse2));
          const int cr = 16 * (r >> 3) + (r & 7);  // key offset beyond 32*kb + 8*g
          if (MASK == 1) pr = cr <= up_rel ? pr : 0.f;
          if (MASK == 2) pr = ((PRE && cr < pre_rel) || (cr >= lo_rel && cr <= hi_rel)) ? pr : 0.f;
          ds[r] = pr * dp[r];
        }
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const bf16x8 db = pack_bf16x8(&ds[8 * h8]);
#pragma unroll
          for (int fb = 0; fb < 2; ++fb)
            dqa[fb] = mfma_bf16(load_a_transposed_swz(kcur, 32 * kb + 16 * h8, 32 * fb, lane),
                                db, dqa[fb]);
        }
      }
    };
    if (__any(mine)) {
      if (full)
        tile(std::integral_constant<int, 0>{});
      else if (__all(lo > hi || lo <= k0))  // see the forward: one bound per row
        tile(std::integral_constant<int, 1>{});
      else
        tile(std::integral_constant<int, 2>{});
    }
    wait_vmem();  // tile it+1 is in LDS (this wave's part)
    __syncthreads();
  };
  for (int it = e0; it < e1; it += 2) {
    key_step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < e1) key_step(std::integral_constant<int, 1>{}, it + 1);
  }

  if (p.part) {  // second part of a two-part head: keep the sums
    if (tok >= 0) store_rows16(p.st_dq + srow * kD, dqa, g, 1.f);
    return;
  }
  if (slot < 0) {
    if (tok >= 0) {
      bf16* row = p.dq + (base + tok) * kD;
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          float tmp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) tmp[j] = dqa[fb][8 * h8 + j] * p.scale;
          *reinterpret_cast<bf16x8*>(row + 32 * fb + 16 * h8 + 8 * g) = pack_bf16x8(tmp);
        }
    }
  } else {
    float* prow = p.part_dq + ((size_t(b) * p.num_qslots + slot) * BQ + w * 32 + l32) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int f0 = 32 * fb + 16 * h8 + 8 * g;
        floatx4 x0, x1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x0[j] = dqa[fb][8 * h8 + j] * p.scale;
          x1[j] = dqa[fb][8 * h8 + 4 + j] * p.scale;
        }
        *reinterpret_cast<floatx4*>(prow + f0) = x0;
        *reinterpret_cast<floatx4*>(prow + f0 + 4) = x1;
      }
  }
}

// --------------------------------------------------------------------------
// dK/dV pass: one workgroup per (key tile, chunk of its CSC list).
// BK = 32 * NW keys; query tiles of BQ rows are processed in steps of
// QS = min(BQ, 64) rows, or of all 128 rows with 128-key tiles (four waves
// share each staged Q / dO tile: half the barriers and staging per key).
// --------------------------------------------------------------------------
// Workgroups of two or more waves: held to two waves per SIMD (256 registers;
// the prefix compares would otherwise take one more and halve the occupancy).
template <int BQ, int BK, bool PRE>
__global__ __launch_bounds__(BK * 2) __attribute__((amdgpu_waves_per_eu(BK >= 64 ? 2 : 1, 2)))
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = BK / 32;
  constexpr int QS = BK == 128 ? 128 : (BQ < 64 ? BQ : 64);
  constexpr int NSTEP = BQ / QS;
  constexpr int NQB = QS / 32;
  constexpr int IPW = QS / 8 / NW;  // 1 KB direct loads per wave, tensor and step
  static_assert(IPW >= 1 && (QS / 8) % NW == 0, "tile/wave mismatch");

  // Swizzled tiles, two buffers per tensor as separate arrays selected by a
  // compile-time parity (loop unrolled by two), so that reads of one buffer
  // are not made to wait for the direct loads in flight into the other.
  __shared__ __attribute__((aligned(16))) bf16 q0s[QS * kD], q1s[QS * kD];
  __shared__ __attribute__((aligned(16))) bf16 o0s[QS * kD], o1s[QS * kD];
  // LSE * log2(e) and -D of each staged query row.  -D seeds the dP
  // accumulator (the MFMA then yields dP - D directly).
  __shared__ __attribute__((aligned(16))) float slse[2][QS];
  __shared__ __attribute__((aligned(16))) float snd[2][QS];
  __shared__ __attribute__((aligned(16))) int32_t slo[2][QS];
  __shared__ __attribute__((aligned(16))) int32_t shi[2][QS];
  __shared__ __attribute__((aligned(16))) int32_t spre[2][QS];  // only for patterns with prefixes

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b;
  const int32_t* it8 = xcd_work_entry(p.kitems, p.kxl_len, p.B, &b);
  if (!it8) return;
  const int head = it8[0], kt = it8[1], c0 = it8[2], c1 = it8[3], slot = it8[4], pf = it8[5];
  const PatView pv = pattern_view(p.pats, p.blob, field_pattern(pf));
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);

  const int kpos = kt * BK + 32 * w + l32;
  const int ktok = (pv.ident & 2) ? identity_token(kpos, p.n) : pv.kmap[kpos];
  bf16x8 kq[4], vq[4];
  if (ktok >= 0) {
    const bf16x8* ksrc = reinterpret_cast<const bf16x8*>(p.k + (base + ktok) * kD);
    const bf16x8* vsrc = reinterpret_cast<const bf16x8*>(p.v + (base + ktok) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kq[c] = ksrc[2 * c + g];
      vq[c] = vsrc[2 * c + g];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kq[c] = bf16x8{};
      vq[c] = bf16x8{};
    }
  }

  floatx16 dva[2], dka[2];
  dva[0] = dva[1] = dka[0] = dka[1] = floatx16{};
  // Register r of half g: feature 32*fb + kappa(r, g); lane = key.
  const size_t srow = (size_t(b) * p.num_merged + field_merged(pf)) * size_t(p.n) + size_t(ktok);
  if ((pf & kPartInit) && ktok >= 0) {  // main part of a two-part head
    load_rows16(p.st_dk + srow * kD, dka, g);
    load_rows16(p.st_dv + srow * kD, dva, g);
  }
  const int nsteps = (c1 - c0) * NSTEP;
  const float c2 = p.scale_log2;

  // Q, dO rows by direct loads (swizzled tiles); per-row LSE, D and key
  // intervals through registers.  Padding query rows fetch token 0 and get
  // LSE = +inf, so their probabilities (hence dS) are exactly 0.
  const BufRsrc qrs = slice_rsrc(p.q + base * kD, uint32_t(p.n) * uint32_t(kD * 2));
  const BufRsrc drs = slice_rsrc(p.dout + base * kD, uint32_t(p.n) * uint32_t(kD * 2));
  const int drow = lane >> 3;
  float lse_r = 0.f, dd_r = 0.f;
  int lo_r = 1, hi_r = 0, pre_r = 0;
  const bool has_pre = PRE && pv.pre != nullptr;
  int qidx[IPW], rtok = -1;  // query-map entries of the next step to load (fetched a step early)
  // Per-row metadata: each wave loads and stores that of QS / NW rows.
  constexpr int MPW = QS / NW;
  const bool mthr = lane < MPW;
  const int mrow = w * MPW + lane;
  TileWindow win = tile_window(pv.row, pv.bflag, c0, c1);
  const BufRsrc qmap_rs = array_rsrc(pv.qmap), lo_rs = array_rsrc(pv.lo), hi_rs = array_rsrc(pv.hi);
  const BufRsrc lse_rs = array_rsrc(p.lse + base), dsum_rs = array_rsrc(p.dsum + base);
  // CSC entry e; the first one travels in the schedule entry.
  auto entry = [&](int e) { return e == c0 ? it8[8] : win.get(e); };
  const bool qid = (pv.ident & 1) != 0;
  auto iload = [&](int step) {
    const int r0 = (entry(c0 + step / NSTEP) >> 1) * BQ + (step % NSTEP) * QS;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int pos = r0 + 8 * (w * IPW + i) + drow;
      qidx[i] = qid ? identity_token(pos, p.n) : buf_i32(qmap_rs, pos);
    }
    if (mthr) rtok = qid ? identity_token(r0 + mrow, p.n) : buf_i32(qmap_rs, r0 + mrow);
  };
  auto gload = [&](int step, auto par) {
    constexpr int P = decltype(par)::value;
    bf16* qd = P ? q1s : q0s;
    bf16* od = P ? o1s : o0s;
    const int ent = entry(c0 + step / NSTEP);
    const int r0 = (ent >> 1) * BQ + (step % NSTEP) * QS;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t off = row_chunk_offset(qidx[i], (lane & 7) ^ swz_key(8 * (w * IPW + i) + drow));
      dma16_buf(qrs, off, qd + 8 * (w * IPW + i) * kD);
      dma16_buf(drs, off, od + 8 * (w * IPW + i) * kD);
    }
    if (mthr) {
      const int r = r0 + mrow;
      const int tk = rtok;
      // Row intervals are read only by the masked body (PARTIAL tiles).
      if ((ent & 1) == 0) {
        lo_r = buf_i32(lo_rs, r);
        hi_r = buf_i32(hi_rs, r);
        if (has_pre) pre_r = pv.pre[r];
      }
      lse_r = tk >= 0 ? buf_f32(lse_rs, tk) * kLog2e : INFINITY;
      dd_r = tk >= 0 ? buf_f32(dsum_rs, tk) : 0.f;
    }
  };
  auto mstore = [&](int buf) {
    if (mthr) {
      slse[buf][mrow] = lse_r;
      snd[buf][mrow] = -dd_r;
      slo[buf][mrow] = lo_r;
      shi[buf][mrow] = hi_r;
      if (has_pre) spre[buf][mrow] = pre_r;
    }
  };

  if (nsteps > 0) {
    iload(0);
    gload(0, std::integral_constant<int, 0>{});
    if (nsteps > 1) iload(1);
  }
  wait_vmem();
  mstore(0);
  __syncthreads();
  // One query step; P = parity of the step selects the buffers.
  auto q_step = [&](auto par, int step) {
    constexpr int P = decltype(par)::value;
    constexpr int buf = P;
    const bf16* qcur = P ? q1s : q0s;
    const bf16* ocur = P ? o1s : o0s;
    // PARTIAL tiles set hidden scores to -inf (probability 0) under one
    // uniform branch; FULL tiles (every pair visible) skip it.
    const bool full = (win.get(c0 + step / NSTEP) & 1) != 0;
    if (step + 1 < nsteps) {
      gload(step + 1, std::integral_constant<int, 1 - P>{});  // indices already here
      if (step + 2 < nsteps) iload(step + 2);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // Register r of half g: query 32*qb + kappa(r, g); lane = key.  Registers
      // 0..7 are rows 32*qb + 8*g + 0..7, registers 8..15 the same + 16.
      const int qa = 32 * qb + 8 * g;
      const floatx4* nd0 = reinterpret_cast<const floatx4*>(&snd[buf][qa]);
      const floatx4* nd1 = reinterpret_cast<const floatx4*>(&snd[buf][qa + 16]);
      const floatx4 n0 = nd0[0], n1 = nd0[1], n2 = nd1[0], n3 = nd1[1];
      floatx16 s = floatx16{};
      floatx16 dp = {n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                     n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
      const int qr = 32 * qb + sigma32(l32);
      // All operands of the S and dP products first, then the products.
      bf16x8 qop[4], oop[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = swz(qr, g + 2 * c);
        qop[c] = *reinterpret_cast<const bf16x8*>(&qcur[off]);
        oop[c] = *reinterpret_cast<const bf16x8*>(&ocur[off]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = mfma_bf16(qop[c], kq[c], s);
        dp = mfma_bf16(oop[c], vq[c], dp);
      }
      // Transposed operands of the dV and dK products, read before the
      // softmax so that their latency overlaps it.
      bf16x8 ot[2][2], qtr[2][2];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
          ot[h8][fb] = load_a_transposed_swz(ocur, 32 * qb + 16 * h8, 32 * fb, lane);
          qtr[h8][fb] = load_a_transposed_swz(qcur, 32 * qb + 16 * h8, 32 * fb, lane);
        }
      if (!full) {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const int qloc = 32 * qb + 16 * h8 + 8 * g;
          const int4 loa = *reinterpret_cast<const int4*>(&slo[buf][qloc]);
          const int4 lob = *reinterpret_cast<const int4*>(&slo[buf][qloc + 4]);
          const int4 hia = *reinterpret_cast<const int4*>(&shi[buf][qloc]);
          const int4 hib = *reinterpret_cast<const int4*>(&shi[buf][qloc + 4]);
          int4 pra = int4{0, 0, 0, 0}, prb = int4{0, 0, 0, 0};
          if (has_pre) {
            pra = *reinterpret_cast<const int4*>(&spre[buf][qloc]);
            prb = *reinterpret_cast<const int4*>(&spre[buf][qloc + 4]);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int qlo = j < 4 ? loa[j] : lob[j - 4];
            const int qhi = j < 4 ? hia[j] : hib[j - 4];
            const int qpre = j < 4 ? pra[j] : prb[j - 4];
            const int r = 8 * h8 + j;
            s[r] = ((PRE && kpos < qpre) || (kpos >= qlo && kpos <= qhi)) ? s[r] : -INFINITY;
          }
        }
      }
      float pr[16], ds[16];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int qloc = 32 * qb + 16 * h8 + 8 * g;
        const floatx4 la = *reinterpret_cast<const floatx4*>(&slse[buf][qloc]);
        const floatx4 lb = *reinterpret_cast<const floatx4*>(&slse[buf][qloc + 4]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * h8 + j;
          const float l2 = j < 4 ? la[j] : lb[j - 4];
          const float pp = fast_exp2(fmaf(s[r], c2, -l2));
          pr[r] = pp;
          ds[r] = pp * dp[r];  // dp holds dP - D
        }
      }
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const bf16x8 pb = pack_bf16x8(&pr[8 * h8]);
        const bf16x8 sb = pack_bf16x8(&ds[8 * h8]);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
          dva[fb] = mfma_bf16(ot[h8][fb], pb, dva[fb]);
          dka[fb] = mfma_bf16(qtr[h8][fb], sb, dka[fb]);
        }
      }
    }
    wait_vmem();  // step+1 staged (this wave's part)
    if (step + 1 < nsteps) mstore(buf ^ 1);
    __syncthreads();
  };
  for (int step = 0; step < nsteps; step += 2) {
    q_step(std::integral_constant<int, 0>{}, step);
    if (step + 1 < nsteps) q_step(std::integral_constant<int, 1>{}, step + 1);
  }

  if (p.part) {  // second part of a two-part head: keep the sums
    if (ktok >= 0) {
      store_rows16(p.st_dk + srow * kD, dka, g, 1.f);
      store_rows16(p.st_dv + srow * kD, dva, g, 1.f);
    }
    return;
  }
  if (slot < 0) {
    if (ktok >= 0) {
      bf16* dkrow = p.dk + (base + ktok) * kD;
      bf16* dvrow = p.dv + (base + ktok) * kD;
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          float tk[8], tv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            tk[j] = dka[fb][8 * h8 + j] * p.scale;
            tv[j] = dva[fb][8 * h8 + j];
          }
          const int f0 = 32 * fb + 16 * h8 + 8 * g;
          *reinterpret_cast<bf16x8*>(dkrow + f0) = pack_bf16x8(tk);
          *reinterpret_cast<bf16x8*>(dvrow + f0) = pack_bf16x8(tv);
        }
    }
  } else {
    float* part = p.partial + (size_t(b) * p.num_slots + slot) * 2 * BK * kD;
    float* pk = part + (32 * w + l32) * kD;
    float* pvv = part + BK * kD + (32 * w + l32) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int f0 = 32 * fb + 16 * h8 + 8 * g;
        floatx4 k0, k1, v0, v1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          k0[j] = dka[fb][8 * h8 + j] * p.scale;
          k1[j] = dka[fb][8 * h8 + 4 + j] * p.scale;
          v0[j] = dva[fb][8 * h8 + j];
          v1[j] = dva[fb][8 * h8 + 4 + j];
        }
        *reinterpret_cast<floatx4*>(pk + f0) = k0;
        *reinterpret_cast<floatx4*>(pk + f0 + 4) = k1;
        *reinterpret_cast<floatx4*>(pvv + f0) = v0;
        *reinterpret_cast<floatx4*>(pvv + f0 + 4) = v1;
      }
  }
}

// --------------------------------------------------------------------------
// Segment pass: one workgroup per (batch element, segment) of a head whose
// rows read only keys of their own segment -- a stride head's residue class:
// tokens r + l t, t < rows, token t reading the tokens t' <= t of its class
// ("Sparse Transformers 深度解读报告", section 2.2).  The entry gives r, l and
// rows, so tokens and masks need no map loads.  NT = 32-row sub-tiles of the
// longest segment; wave w owns sub-tile w, as queries (dQ) and as keys (dK,
// dV).  The segment's Q, K, V and dO rows are staged once, in LDS:
//   phase 1, wave a, key sub-tiles b <= a: S^T = K_b Q_a^T, dP^T - D and the
//            dQ products as in the dQ pass; the bf16 P and dS of each pair
//            (the values the products use) stay in registers and go to LDS,
//            into the space of K and V, once every wave is done with those;
//   phase 2, wave b, query sub-tiles a >= b: dV_b^T += dO_a^T P_ab and
//            dK_b^T += Q_a^T dS_ab, every operand through transposing reads.
// Each visible pair's S and dP are formed once, every row is read from HBM
// once and every gradient row written once.  Work per wave: a + 1 pairs in
// phase 1, NT - b in phase 2.
// --------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(64 * NT) __attribute__((amdgpu_waves_per_eu(NT <= 3 ? 3 : 2)))
void bwd_seg_kernel(BwdParams p) {
  constexpr int NP = NT * (NT + 1) / 2;  // sub-tile pairs b <= a
  constexpr int KVX = (2 * NT > NP ? 2 * NT : NP) * 32 * kD;
  // Swizzled [32 * NT][64] tiles; per pair a [32 query rows][64] tile holding
  // P (columns 0..31, keys of sub-tile b) and dS (columns 32..63).  Phase 2
  // needs no K or V: the pair tiles take their place once every wave is done
  // with them (three workgroups per CU for 96-row segments).
  __shared__ __attribute__((aligned(16))) bf16 qs[NT * 32 * kD], dos[NT * 32 * kD];
  __shared__ __attribute__((aligned(16))) bf16 kvx[KVX];
  bf16* const ks = kvx;
  bf16* const vs = kvx + NT * 32 * kD;
  bf16* const xs = kvx;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b;
  const int32_t* it8 = xcd_work_entry(p.sitems, p.sxl_len, p.B, &b);
  if (!it8) return;
  const int head = it8[0], res = it8[2], rows = it8[3], l = it8[4];
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const int nst = (rows + 31) >> 5;  // sub-tiles of this segment
  const bool active = w < nst;

  // Staging: wave w fetches rows 32w .. 32w + 31 of the segment (1 KB = 8
  // rows per direct load); rows past the segment fetch token 0 and are masked.
  const uint32_t slice_bytes = uint32_t(p.n) * uint32_t(kD * 2);
  if (active) {
    const BufRsrc qrs = slice_rsrc(p.q + base * kD, slice_bytes);
    const BufRsrc krs = slice_rsrc(p.k + base * kD, slice_bytes);
    const BufRsrc vrs = slice_rsrc(p.v + base * kD, slice_bytes);
    const BufRsrc drs = slice_rsrc(p.dout + base * kD, slice_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 32 * w + 8 * i + (lane >> 3);
      const uint32_t off = row_chunk_offset(t < rows ? res + l * t : -1, (lane & 7) ^ swz_key(t));
      const int dst = (32 * w + 8 * i) * kD;
      dma16_buf(qrs, off, qs + dst);
      dma16_buf(drs, off, dos + dst);
      dma16_buf(krs, off, ks + dst);
      dma16_buf(vrs, off, vs + dst);
    }
  }
  // The lane's query row t = 32 w + l32 of the class (both halves of the
  // wave hold it); it reads the class's tokens t' <= t.
  const int r = 32 * w + l32;
  const bool valid = r < rows;
  const int tq = valid ? res + l * r : -1;
  const int hi = valid ? r : -1;
  // D = dO . O of the lane's row, from its own global reads (the O row is
  // needed nowhere else), before the staged tiles are waited for.
  bf16x8 dof[4];
  float lse2 = 0.f, dsum = 0.f;
  if (tq >= 0) {
    const bf16x8* osrc = reinterpret_cast<const bf16x8*>(p.o + (base + tq) * kD);
    const bf16x8* dsrc = reinterpret_cast<const bf16x8*>(p.dout + (base + tq) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 oo = osrc[2 * c + g];
      dof[c] = dsrc[2 * c + g];
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += float(oo[j]) * float(dof[c][j]);
    }
    lse2 = p.lse[base + tq] * kLog2e;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) dof[c] = bf16x8{};
  }
  dsum = pair_sum(dsum);
  wait_vmem();
  __syncthreads();

  const float c2 = p.scale_log2;
  floatx16 dqa[2];
  dqa[0] = dqa[1] = floatx16{};
  bf16x8 px[NT][4];  // per key sub-tile: P (keys 0..15, 16..31), dS (likewise), bf16
  if (active) {
    bf16x8 qf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(&qs[swz(r, 2 * c + g)]);
#pragma unroll
    for (int kb = 0; kb < NT; ++kb) {
      if (kb > w) break;
      const bf16* kt = ks + 32 * kb * kD;
      const bf16* vt = vs + 32 * kb * kD;
      floatx16 sa = floatx16{}, dp = floatx16{};
      const int kr = sigma32(l32);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = swz(kr, g + 2 * c);
        sa = mfma_bf16(*reinterpret_cast<const bf16x8*>(&kt[off]), qf[c], sa);
        dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(&vt[off]), dof[c], dp);
      }
      // Register i of half g: class row 32 kb + kappa(i, g).
      const int hi_rel = hi - (32 * kb + 8 * g);
      float pr[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cr = 16 * (i >> 3) + (i & 7);
        const float e = fast_exp2(fmaf(sa[i], c2, -lse2));
        pr[i] = cr <= hi_rel ? e : 0.f;
        dsv[i] = pr[i] * (dp[i] - dsum);
      }
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const bf16x8 db = pack_bf16x8(&dsv[8 * h8]);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
          dqa[fb] = mfma_bf16(load_a_transposed_swz(kt, 16 * h8, 32 * fb, lane), db, dqa[fb]);
        px[kb][h8] = pack_bf16x8(&pr[8 * h8]);
        px[kb][2 + h8] = db;
      }
    }
  }
  __syncthreads();  // every wave is done with K and V
  if (active) {
#pragma unroll
    for (int kb = 0; kb < NT; ++kb) {
      if (kb > w) break;
      bf16* x = xs + (w * (w + 1) / 2 + kb) * 32 * kD;
      // Keys 16 h8 + 8 g .. + 7 of the lane's query row: chunk 2 h8 + g.
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        *reinterpret_cast<bf16x8*>(&x[swz(l32, 2 * h8 + g)]) = px[kb][h8];
        *reinterpret_cast<bf16x8*>(&x[swz(l32, 4 + 2 * h8 + g)]) = px[kb][2 + h8];
      }
    }
  }
  __syncthreads();
  if (!active) return;
  if (tq >= 0) {
    bf16* row = p.dq + (base + tq) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = dqa[fb][8 * h8 + j] * p.scale;
        *reinterpret_cast<bf16x8*>(row + 32 * fb + 16 * h8 + 8 * g) = pack_bf16x8(tmp);
      }
  }
  // Phase 2: key sub-tile w.  Lane l32 holds key 32 w + sigma32(l32) (the
  // column order of the transposing reads); register i of half g feature
  // 32 fb + kappa(i, g).
  floatx16 dka[2], dva[2];
  dka[0] = dka[1] = dva[0] = dva[1] = floatx16{};
#pragma unroll
  for (int a = 0; a < NT; ++a) {
    if (a < w || a >= nst) continue;
    const bf16* x = xs + (a * (a + 1) / 2 + w) * 32 * kD;
    const bf16* qt = qs + 32 * a * kD;
    const bf16* dt = dos + 32 * a * kD;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 pb = load_a_transposed_swz(x, 16 * h, 0, lane);
      const bf16x8 sb = load_a_transposed_swz(x, 16 * h, 32, lane);
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        dva[fb] = mfma_bf16(load_a_transposed_swz(dt, 16 * h, 32 * fb, lane), pb, dva[fb]);
        dka[fb] = mfma_bf16(load_a_transposed_swz(qt, 16 * h, 32 * fb, lane), sb, dka[fb]);
      }
    }
  }
  const int kr = 32 * w + sigma32(l32);
  if (kr < rows) {
    const int tk = res + l * kr;
    bf16* krow = p.dk + (base + tk) * kD;
    bf16* vrow = p.dv + (base + tk) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        float tk8[8], tv8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          tk8[j] = dka[fb][8 * h8 + j] * p.scale;
          tv8[j] = dva[fb][8 * h8 + j];
        }
        const int f0 = 32 * fb + 16 * h8 + 8 * g;
        *reinterpret_cast<bf16x8*>(krow + f0) = pack_bf16x8(tk8);
        *reinterpret_cast<bf16x8*>(vrow + f0) = pack_bf16x8(tv8);
      }
  }
}

// --------------------------------------------------------------------------
// Sum the chunk partials of each split key tile (chunk order) -> dK, dV.
// --------------------------------------------------------------------------
// Merge launch: the chunks of each split key tile (dK, dV: 2 * BK * 64
// floats per slot) and of each split query tile (dQ: BQ * 64 floats per slot)
// are summed in chunk order.  One workgroup of 256 threads per (batch
// element, group, 2048-float block); thread = 8 consecutive floats.
template <int BQ, int BK>
__global__ __launch_bounds__(256) void bwd_merge_kernel(BwdParams p) {
  constexpr int KPER = 2 * BK * kD, QPER = BQ * kD;  // floats per slot
  constexpr int KBLK = KPER / 2048, QBLK = QPER / 2048;
  const int b = blockIdx.x % p.B;
  int gi = blockIdx.x / p.B;
  const bool key_tile = gi < p.kgroups * KBLK;
  if (!key_tile) gi -= p.kgroups * KBLK;
  const int blk = key_tile ? gi % KBLK : gi % QBLK;
  const int32_t* g4 = key_tile ? p.rsched + 4 * (gi / KBLK) : p.csched + 4 * (gi / QBLK);
  const int head = g4[0], tile = g4[1], slot0 = g4[2], chunks = g4[3];
  const PatView pv = pattern_of_head(p.blob, head);
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const int idx = blk * 2048 + threadIdx.x * 8;
  const int per = key_tile ? KPER : QPER;
  const float* part0 = key_tile ? p.partial + (size_t(b) * p.num_slots + slot0) * KPER
                                : p.part_dq + (size_t(b) * p.num_qslots + slot0) * QPER;
  bf16* dst;
  if (key_tile) {
    const int t = idx / (BK * kD);  // 0: dK, 1: dV
    const int tok = pv.kmap[tile * BK + (idx / kD) % BK];
    if (tok < 0) return;
    dst = (t == 0 ? p.dk : p.dv) + (base + tok) * kD + idx % kD;
  } else {
    const int tok = pv.qmap[tile * BQ + idx / kD];
    if (tok < 0) return;
    dst = p.dq + (base + tok) * kD + idx % kD;
  }
  floatx4 a = floatx4{}, c = floatx4{};
  for (int ch = 0; ch < chunks; ++ch) {
    const floatx4* src = reinterpret_cast<const floatx4*>(part0 + size_t(ch) * per + idx);
    a += src[0];
    c += src[1];
  }
  float tmp[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  *reinterpret_cast<bf16x8*>(dst) = pack_bf16x8(tmp);
}

}  // namespace sa

// --------------------------------------------------------------------------
// C ABI entry points
// --------------------------------------------------------------------------
#include "abi_common.hpp"

namespace {

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [D float32[B, H, n]] [dK, dV partials float32[B, slots, 2, BK,
// 64]] [dQ partials float32[B, query slots, BQ, 64]]; each part starts on a
// 256-byte boundary.
struct BwdWorkspace {
  size_t dsum, partial, part_dq, st_dq, st_dk, st_dv, total;
};

// D, chunk partials of split key and query tiles, then the token sums of
// two-part heads.
BwdWorkspace bwd_workspace_layout(int B, int H, const sa_blob_header& h) {
  BwdWorkspace w{};
  const size_t st = round256(size_t(B) * size_t(h.num_merged) * size_t(h.n) * sa::kD * sizeof(float));
  w.dsum = 0;
  w.partial = w.dsum + round256(size_t(B) * size_t(H) * size_t(h.n) * sizeof(float));
  w.part_dq = w.partial + round256(size_t(B) * size_t(h.num_slots) * 2 * size_t(h.block_k) *
                                   sa::kD * sizeof(float));
  w.st_dq = w.part_dq + round256(size_t(B) * size_t(h.num_qslots) * size_t(h.block_q) * sa::kD *
                                 sizeof(float));
  w.st_dk = w.st_dq + st;
  w.st_dv = w.st_dk + st;
  w.total = w.st_dv + st;
  return w;
}

}  // namespace

extern "C" int sparse_attn_bwd_workspace(const void* blob_host, int B, int H, int d, int dtype,
                                         size_t* bytes) {
  using namespace sa;
  if (!bytes || !blob_host) return SA_EINVAL;
  sa_blob_header h;
  memcpy(&h, blob_host, sizeof(h));
  if (h.magic != SA_BLOB_MAGIC || h.version != SA_BLOB_VERSION) return SA_EINVAL;
  if (B < 0 || H < 1 || H != h.num_heads) return SA_EINVAL;
  if (dtype != SA_BF16 && dtype != SA_FP32) return SA_EINVAL;
  if (d != 64 || dtype != SA_BF16) return SA_EUNSUPPORTED;
  *bytes = bwd_workspace_layout(B, H, h).total;
  return SA_OK;
}

extern "C" int sparse_attn_bwd_phases(const void* blob_host, const void* blob_dev, int B, int H,
                                      int d, int dtype, const void* q, const void* k,
                                      const void* v, const void* o, const float* lse,
                                      const void* dO, void* dq, void* dk, void* dv,
                                      void* workspace, size_t ws_bytes, float scale,
                                      unsigned phases, void* stream) {
  using namespace sa;
  if (phases == 0 || (phases & ~unsigned(SA_BWD_ALL)) != 0) return SA_EINVAL;
  LaunchInfo li;
  int rc = validate_common(blob_host, blob_dev, B, H, d, dtype, &li);
  if (rc != SA_OK) return rc;
  if (dtype != SA_BF16) return SA_EUNSUPPORTED;
  const int bq = li.block_q, bk = li.block_k;
  if (!(bq == 32 || bq == 64 || bq == 128) || !(bk == 32 || bk == 64 || (bq == 128 && bk == 128)))
    return SA_EUNSUPPORTED;
  float sc;
  rc = resolve_scale(scale, d, &sc);
  if (rc != SA_OK) return rc;
  sa_blob_header h;
  memcpy(&h, blob_host, sizeof(h));
  if (B == 0) return SA_OK;  // empty batch: pointers may be NULL
  const BwdWorkspace wl = bwd_workspace_layout(B, H, h);
  if (ws_bytes < wl.total) return SA_ESIZE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return SA_EINVAL;
  const int64_t gq = int64_t(SA_XCDS) * li.dq_xl_len * B;
  const int64_t gs = int64_t(SA_XCDS) * li.seg_xl_len * B;
  const int64_t gk = int64_t(SA_XCDS) * li.bwd_xl_len * B;
  const int64_t gm = (int64_t(h.red_sched_len) * (2 * bk * kD / 2048) +
                      int64_t(h.comb_sched_len) * (bq * kD / 2048)) * B;
  const int64_t gqp = int64_t(SA_XCDS) * li.fwdp_xl_len * B;
  const int64_t gkp = int64_t(SA_XCDS) * li.bwdp_xl_len * B;
  if (gq > INT32_MAX || gk > INT32_MAX || gm > INT32_MAX || gqp > INT32_MAX || gkp > INT32_MAX ||
      gs > INT32_MAX)
    return SA_EUNSUPPORTED;
  if (gs > 0 && (li.seg_tiles < 1 || li.seg_tiles > 4)) return SA_EINVAL;

  BwdParams prm;
  prm.blob = static_cast<const uint8_t*>(blob_dev);
  prm.qitems = reinterpret_cast<const int32_t*>(prm.blob + li.dq_xitem_off);
  prm.kitems = reinterpret_cast<const int32_t*>(prm.blob + li.bwd_xitem_off);
  prm.sitems = reinterpret_cast<const int32_t*>(prm.blob + li.seg_xitem_off);
  prm.sxl_len = li.seg_xl_len;
  fill_pattern_table(blob_host, blob_dev, &prm.pats);
  prm.num_qslots = h.num_qslots;
  prm.kgroups = h.red_sched_len;
  prm.rsched = reinterpret_cast<const int32_t*>(prm.blob + h.red_sched_off);
  prm.csched = reinterpret_cast<const int32_t*>(prm.blob + h.comb_sched_off);
  prm.qxl_len = li.dq_xl_len;
  prm.kxl_len = li.bwd_xl_len;
  prm.B = B;
  prm.H = H;
  prm.n = int32_t(li.n);
  prm.num_slots = h.num_slots;
  prm.q = static_cast<const bf16*>(q);
  prm.k = static_cast<const bf16*>(k);
  prm.v = static_cast<const bf16*>(v);
  prm.o = static_cast<const bf16*>(o);
  prm.lse = lse;
  prm.dout = static_cast<const bf16*>(dO);
  prm.dq = static_cast<bf16*>(dq);
  prm.dk = static_cast<bf16*>(dk);
  prm.dv = static_cast<bf16*>(dv);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  prm.dsum = reinterpret_cast<float*>(ws + wl.dsum);
  prm.partial = reinterpret_cast<float*>(ws + wl.partial);
  prm.part_dq = reinterpret_cast<float*>(ws + wl.part_dq);
  prm.st_dq = reinterpret_cast<float*>(ws + wl.st_dq);
  prm.st_dk = reinterpret_cast<float*>(ws + wl.st_dk);
  prm.st_dv = reinterpret_cast<float*>(ws + wl.st_dv);
  prm.num_merged = li.num_merged;
  prm.part = 0;
  prm.scale = sc;
  prm.scale_log2 = float(double(sc) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();

#define SA_LAUNCH(kern, grid, threads) \
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(threads), 0, st, prm)
// Kernels for layouts with key prefixes are separate instantiations, so the
// other layouts run code without the prefix compares.
#define SA_LAUNCH_P(KN, A, C, g, threads)               \
  do {                                                  \
    if (li.has_pre) SA_LAUNCH((KN<A, C, true>), g, threads); \
    else SA_LAUNCH((KN<A, C, false>), g, threads);      \
  } while (0)
  if ((phases & SA_BWD_SEG) && gs > 0) {
    if (li.seg_tiles == 1) SA_LAUNCH((bwd_seg_kernel<1>), gs, 64);
    else if (li.seg_tiles == 2) SA_LAUNCH((bwd_seg_kernel<2>), gs, 128);
    else if (li.seg_tiles == 3) SA_LAUNCH((bwd_seg_kernel<3>), gs, 192);
    else SA_LAUNCH((bwd_seg_kernel<4>), gs, 256);
  }
  // Second parts of two-part heads run first in each pass: they leave their
  // sums of every token for the main launch.
  BwdParams pp = prm;
  pp.part = 1;
  pp.qitems = reinterpret_cast<const int32_t*>(pp.blob + li.fwdp_xitem_off);
  pp.kitems = reinterpret_cast<const int32_t*>(pp.blob + li.bwdp_xitem_off);
  pp.qxl_len = li.fwdp_xl_len;
  pp.kxl_len = li.bwdp_xl_len;
#define SA_LAUNCH_PART(kern, grid, threads) \
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(threads), 0, st, pp)
  if ((phases & SA_BWD_DQ) && gqp > 0) {
    if (bq == 32 && bk == 32) SA_LAUNCH_PART((bwd_dq_kernel<32, 32, false>), gqp, 64);
    else if (bq == 32 && bk == 64) SA_LAUNCH_PART((bwd_dq_kernel<32, 64, false>), gqp, 64);
    else if (bq == 64 && bk == 32) SA_LAUNCH_PART((bwd_dq_kernel<64, 32, false>), gqp, 128);
    else if (bq == 64 && bk == 64) SA_LAUNCH_PART((bwd_dq_kernel<64, 64, false>), gqp, 128);
    else if (bq == 128 && bk == 32) SA_LAUNCH_PART((bwd_dq_kernel<128, 32, false>), gqp, 256);
    else if (bq == 128 && bk == 64) SA_LAUNCH_PART((bwd_dq_kernel<128, 64, false>), gqp, 256);
    else SA_LAUNCH_PART((bwd_dq_kernel<128, 128, false>), gqp, 256);
  }
  if ((phases & SA_BWD_DQ) && gq > 0) {
    if (bq == 32 && bk == 32) SA_LAUNCH_P(bwd_dq_kernel, 32, 32, gq, 64);
    else if (bq == 32 && bk == 64) SA_LAUNCH_P(bwd_dq_kernel, 32, 64, gq, 64);
    else if (bq == 64 && bk == 32) SA_LAUNCH_P(bwd_dq_kernel, 64, 32, gq, 128);
    else if (bq == 64 && bk == 64) SA_LAUNCH_P(bwd_dq_kernel, 64, 64, gq, 128);
    else if (bq == 128 && bk == 32) SA_LAUNCH_P(bwd_dq_kernel, 128, 32, gq, 256);
    else if (bq == 128 && bk == 64) SA_LAUNCH_P(bwd_dq_kernel, 128, 64, gq, 256);
    else SA_LAUNCH_P(bwd_dq_kernel, 128, 128, gq, 256);
  }
  if ((phases & SA_BWD_DKDV) && gkp > 0) {
    if (bq == 32 && bk == 32) SA_LAUNCH_PART((bwd_dkdv_kernel<32, 32, false>), gkp, 64);
    else if (bq == 64 && bk == 32) SA_LAUNCH_PART((bwd_dkdv_kernel<64, 32, false>), gkp, 64);
    else if (bq == 128 && bk == 32) SA_LAUNCH_PART((bwd_dkdv_kernel<128, 32, false>), gkp, 64);
    else if (bq == 32 && bk == 64) SA_LAUNCH_PART((bwd_dkdv_kernel<32, 64, false>), gkp, 128);
    else if (bq == 64 && bk == 64) SA_LAUNCH_PART((bwd_dkdv_kernel<64, 64, false>), gkp, 128);
    else if (bq == 128 && bk == 64) SA_LAUNCH_PART((bwd_dkdv_kernel<128, 64, false>), gkp, 128);
    else SA_LAUNCH_PART((bwd_dkdv_kernel<128, 128, false>), gkp, 256);
  }
#undef SA_LAUNCH_PART
  if ((phases & SA_BWD_DKDV) && gk > 0) {
    if (bq == 32 && bk == 32) SA_LAUNCH_P(bwd_dkdv_kernel, 32, 32, gk, 64);
    else if (bq == 64 && bk == 32) SA_LAUNCH_P(bwd_dkdv_kernel, 64, 32, gk, 64);
    else if (bq == 128 && bk == 32) SA_LAUNCH_P(bwd_dkdv_kernel, 128, 32, gk, 64);
    else if (bq == 32 && bk == 64) SA_LAUNCH_P(bwd_dkdv_kernel, 32, 64, gk, 128);
    else if (bq == 64 && bk == 64) SA_LAUNCH_P(bwd_dkdv_kernel, 64, 64, gk, 128);
    else if (bq == 128 && bk == 64) SA_LAUNCH_P(bwd_dkdv_kernel, 128, 64, gk, 128);
    else SA_LAUNCH_P(bwd_dkdv_kernel, 128, 128, gk, 256);
  }
  if ((phases & SA_BWD_MERGE) && gm > 0) {
    if (bq == 32 && bk == 32) SA_LAUNCH((bwd_merge_kernel<32, 32>), gm, 256);
    else if (bq == 32 && bk == 64) SA_LAUNCH((bwd_merge_kernel<32, 64>), gm, 256);
    else if (bq == 64 && bk == 32) SA_LAUNCH((bwd_merge_kernel<64, 32>), gm, 256);
    else if (bq == 64 && bk == 64) SA_LAUNCH((bwd_merge_kernel<64, 64>), gm, 256);
    else if (bq == 128 && bk == 32) SA_LAUNCH((bwd_merge_kernel<128, 32>), gm, 256);
    else if (bq == 128 && bk == 64) SA_LAUNCH((bwd_merge_kernel<128, 64>), gm, 256);
    else SA_LAUNCH((bwd_merge_kernel<128, 128>), gm, 256);
  }
#undef SA_LAUNCH_P
#undef SA_LAUNCH
  return hipGetLastError() == hipSuccess ? SA_OK : SA_EHIP;
}

extern "C" int sparse_attn_bwd(const void* blob_host, const void* blob_dev, int B, int H, int d,
                               int dtype, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dO, void* dq,
                               void* dk, void* dv, void* workspace, size_t ws_bytes, float scale,
                               void* stream) {
  return sparse_attn_bwd_phases(blob_host, blob_dev, B, H, d, dtype, q, k, v, o, lse, dO, dq, dk,
                                dv, workspace, ws_bytes, scale, SA_BWD_ALL, stream);
}

// --------------------------------------------------------------------------
// Allocation-free backward: the workspace is a file-scope device array of
// SA_STATIC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
// --------------------------------------------------------------------------
#include <mutex>

namespace {

static __device__ __align__(256) uint8_t scratch[SA_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on each GPU, resolved once per device with that
// device current (the host-side name `scratch` is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int static_scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SA_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return SA_EHIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return SA_OK;
}

}  // namespace

extern "C" int sparse_attn_bwd_static(const void* blob_host, const void* blob_dev, int B, int H,
                                      int d, int dtype, const void* q, const void* k,
                                      const void* v, const void* o, const float* lse,
                                      const void* dO, void* dq, void* dk, void* dv, float scale,
                                      void* stream) {
  size_t need = 0;
  int rc = sparse_attn_bwd_workspace(blob_host, B, H, d, dtype, &need);
  if (rc != SA_OK) return rc;
  if (need > size_t(SA_STATIC_SCRATCH_BYTES)) return SA_ESIZE;
  void* ws = nullptr;
  if (B > 0) {
    rc = static_scratch_address(&ws);
    if (rc != SA_OK) return rc;
  }
  return sparse_attn_bwd_phases(blob_host, blob_dev, B, H, d, dtype, q, k, v, o, lse, dO, dq, dk,
                                dv, ws, size_t(SA_STATIC_SCRATCH_BYTES), scale, SA_BWD_ALL, stream);
}
