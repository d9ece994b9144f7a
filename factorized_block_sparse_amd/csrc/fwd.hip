// Forward kernels: fused block-sparse attention with an online softmax.
//
// One workgroup handles one query tile (block_q rows of one (batch, head)) of
// the layout and walks that tile's CSR list of active key tiles
// ("Sparse Transformers 深度解读报告", section 3.5: blocked sub-blocks of
// Q/K/V, the softmax fused into a single kernel with its intermediates in
// registers, masked-out tiles never computed).  Per key tile:
//   1. K and V rows (through the pattern's key map) are staged into LDS
//      row-major, double-buffered, one barrier per tile; V^T reaches the MFMA
//      through transposing LDS reads;
//   2. each wave owns 32 query rows and computes S^T = K Q^T on the MFMA
//      units (fp32 accumulation; Q stays in registers for the whole walk);
//   3. on PARTIAL tiles the fine mask is two integer compares against the
//      row's key interval; FULL tiles apply no mask;
//   4. running max / sum update in base 2 with the softmax scale folded into
//      one FMA per score; the running max (and the rescale of the output
//      accumulator) only moves when a tile's max exceeds it by more than
//      2^kRescaleLog2, so P <= 2^kRescaleLog2 and most tiles skip the rescale;
//   5. O^T += V^T P^T on the MFMA units, P rounded to the input type.
// The epilogue writes O rows (through the query map) and the per-row
// log-sum-exp that the backward pass rebuilds probabilities from (report
// section 3.4).  A wave skips the arithmetic of a tile none of its rows can
// see (it still takes part in the staging).

#include <math.h>

#include "device_common.hpp"

namespace sa {

struct FwdParams {
  const uint8_t* blob;
  const int32_t* sched;  // (head, q-tile) pairs
  const int32_t* xl;     // per-XCD lists of schedule entries
  int32_t xl_len;
  int32_t B, H, n;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float scale_log2;  // softmax scale * log2(e)
};

constexpr float kNegInit = -3.0e38f;  // running-max start: exp2(kNegInit - x) == 0
constexpr float kMasked = -1.0e30f;   // masked logit in the base-2 domain (float32 path)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (P <= 256)

// --------------------------------------------------------------------------
// bfloat16 inputs, 32x32x16 bf16 MFMA
// --------------------------------------------------------------------------
template <int BQ, int BK>
__global__ __launch_bounds__(BQ * 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  constexpr int NKB = BK / 32;
  constexpr int KS = kD + 8;  // LDS row stride of K and V (elements)
  constexpr int CPT = BK * 8 / NT;  // 16-byte chunks per thread and tensor
  static_assert(CPT >= 1 && (BK * 8) % NT == 0, "tile/wave mismatch");
  __shared__ __attribute__((aligned(16))) bf16 ks[2][BK * KS];
  __shared__ __attribute__((aligned(16))) bf16 vs[2][BK * KS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  int b, item;
  if (!xcd_work_item(p.xl, p.xl_len, p.B, &b, &item)) return;
  const int head = p.sched[2 * item], qt = p.sched[2 * item + 1];
  const PatView pv = pattern_of_head(p.blob, head);
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const bf16* qg = static_cast<const bf16*>(p.q) + base * kD;
  const bf16* kg = static_cast<const bf16*>(p.k) + base * kD;
  const bf16* vg = static_cast<const bf16*>(p.v) + base * kD;

  const int prow = qt * BQ + w * 32 + l32;
  const int tok = pv.qmap[prow];
  const int lo = pv.lo[prow], hi = pv.hi[prow];

  bf16x8 qf[4];
  if (tok >= 0) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(qg + size_t(tok) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = src[2 * c + g];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = bf16x8{};
  }

  const int e0 = pv.row_ptr[qt], e1 = pv.row_ptr[qt + 1];
  u32x4 kreg[CPT], vreg[CPT];
  int kidx[CPT];  // key-map entries of the next tile to load (fetched a tile early)
  auto iload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) kidx[i] = pv.kmap[kt * BK + ((tid + i * NT) >> 3)];
  };
  auto gload = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = (tid + i * NT) & 7;
      const int tk = kidx[i];
      if (tk >= 0) {
        kreg[i] = reinterpret_cast<const u32x4*>(kg + size_t(tk) * kD)[cc];
        vreg[i] = reinterpret_cast<const u32x4*>(vg + size_t(tk) * kD)[cc];
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, j = c >> 3, cc = c & 7;
      *reinterpret_cast<u32x4*>(&ks[buf][j * KS + cc * 8]) = kreg[i];
      *reinterpret_cast<u32x4*>(&vs[buf][j * KS + cc * 8]) = vreg[i];
    }
  };

  floatx16 oacc[2];
  oacc[0] = floatx16{};
  oacc[1] = floatx16{};
  float m_run = kNegInit, l_run = 0.f;
  const float c2 = p.scale_log2;

  if (e0 < e1) {
    iload(pv.col[e0]);
    gload();
    lstore(0);
    if (e0 + 1 < e1) iload(pv.col[e0 + 1]);
  }
  __syncthreads();
  for (int it = e0; it < e1; ++it) {
    const int buf = (it - e0) & 1;
    const int kt = pv.col[it];
    const bool full = pv.fflag[it] == SA_TILE_FULL;
    if (it + 1 < e1) {
      gload();                                   // tile it+1, indices already here
      if (it + 2 < e1) iload(pv.col[it + 2]);    // indices of tile it+2
    }
    const int k0 = kt * BK;
    const bool mine = (lo <= hi) && (lo <= k0 + BK - 1) && (hi >= k0);
    if (__any(mine)) {
      floatx16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = floatx16{};
        const bf16* krow = &ks[buf][(32 * kb + sigma32(l32)) * KS + 8 * g];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          s[kb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(krow + 16 * c), qf[c], s[kb]);
      }
      if (!full) {
        // Key k0 + c is visible iff lo <= k0 + c <= hi; c = 32*kb + kappa(r, g)
        // = 8*g + (a constant per register).
        const int lo_rel = lo - k0 - 8 * g, hi_rel = hi - k0 - 8 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int cr = 32 * kb + 16 * (r >> 3) + (r & 7);
            s[kb][r] = (cr >= lo_rel && cr <= hi_rel) ? s[kb][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;  // max of the raw scores (scale > 0)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, other_half(mx)) * c2;
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
          const float pr = fast_exp2(fmaf(s[kb][r], c2, -m_run));
          s[kb][r] = pr;
          lsum += pr;
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
            oacc[fb] = mfma_bf16(load_a_transposed(vs[buf], KS, 32 * kb + 16 * h8, 32 * fb, lane),
                                 pb, oacc[fb]);
        }
      }
    }
    if (it + 1 < e1) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + other_half(l_run);
  if (tok >= 0) {
    const float inv = 1.0f / l_tot;
    bf16* orow = static_cast<bf16*>(p.o) + (base + size_t(tok)) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        float tmp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tmp[j] = oacc[fb][8 * h8 + j] * inv;
        *reinterpret_cast<bf16x8*>(orow + 32 * fb + 16 * h8 + 8 * g) = pack_bf16x8(tmp);
      }
    if (g == 0) p.lse[base + tok] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// --------------------------------------------------------------------------
// float32 inputs, 32x32x2 f32 MFMA (same structure; K slot = one feature)
// --------------------------------------------------------------------------
template <int BQ, int BK>
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
  int b, item;
  if (!xcd_work_item(p.xl, p.xl_len, p.B, &b, &item)) return;
  const int head = p.sched[2 * item], qt = p.sched[2 * item + 1];
  const PatView pv = pattern_of_head(p.blob, head);
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);
  const float* qg = static_cast<const float*>(p.q) + base * kD;
  const float* kg = static_cast<const float*>(p.k) + base * kD;
  const float* vg = static_cast<const float*>(p.v) + base * kD;

  const int prow = qt * BQ + w * 32 + l32;
  const int tok = pv.qmap[prow];
  const int lo = pv.lo[prow], hi = pv.hi[prow];

  float qf[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) qf[c] = tok >= 0 ? qg[size_t(tok) * kD + 2 * c + g] : 0.f;

  const int e0 = pv.row_ptr[qt], e1 = pv.row_ptr[qt + 1];
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
    const bool mine = (lo <= hi) && (lo <= k0 + BK - 1) && (hi >= k0);
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
          const float x = (full || (kp >= lo && kp <= hi)) ? s[kb][r] * c2 : kMasked;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, other_half(mx));
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

  const float l_tot = l_run + other_half(l_run);
  if (tok >= 0) {
    const float inv = 1.0f / l_tot;
    float* orow = static_cast<float*>(p.o) + (base + size_t(tok)) * kD;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        floatx4 a, c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = oacc[fb][8 * h8 + j] * inv;
          c[j] = oacc[fb][8 * h8 + 4 + j] * inv;
        }
        float* dst = orow + 32 * fb + 16 * h8 + 8 * g;
        *reinterpret_cast<floatx4*>(dst) = a;
        *reinterpret_cast<floatx4*>(dst + 4) = c;
      }
    if (g == 0) p.lse[base + tok] = (m_run + log2f(l_tot)) * kLn2;
  }
}

}  // namespace sa

// --------------------------------------------------------------------------
// C ABI entry point
// --------------------------------------------------------------------------
#include "abi_common.hpp"

extern "C" int sparse_attn_fwd(const void* blob_host, const void* blob_dev, int B, int H, int d,
                               int dtype, const void* q, const void* k, const void* v, void* o,
                               float* lse, float scale, void* stream) {
  using namespace sa;
  LaunchInfo li;
  int rc = validate_common(blob_host, blob_dev, B, H, d, dtype, &li);
  if (rc != SA_OK) return rc;
  float sc;
  rc = resolve_scale(scale, d, &sc);
  if (rc != SA_OK) return rc;
  if (B == 0 || li.fwd_xl_len == 0) return SA_OK;  // empty batch: pointers may be NULL
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return SA_EINVAL;
  const int64_t grid = int64_t(SA_XCDS) * li.fwd_xl_len * B;
  if (grid > INT32_MAX) return SA_EUNSUPPORTED;

  FwdParams prm;
  prm.blob = static_cast<const uint8_t*>(blob_dev);
  prm.sched = reinterpret_cast<const int32_t*>(prm.blob + li.fwd_sched_off);
  prm.xl = reinterpret_cast<const int32_t*>(prm.blob + li.fwd_xl_off);
  prm.xl_len = li.fwd_xl_len;
  prm.B = B;
  prm.H = H;
  prm.n = int32_t(li.n);
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.scale_log2 = float(double(sc) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int bq = li.block_q, bk = li.block_k;
  const dim3 grd{unsigned(grid), 1u, 1u};
  if (dtype == SA_BF16) {
    if (bq == 32 && bk == 32) hipLaunchKernelGGL((fwd_bf16_kernel<32, 32>), grd, dim3(64), 0, st, prm);
    else if (bq == 32 && bk == 64) hipLaunchKernelGGL((fwd_bf16_kernel<32, 64>), grd, dim3(64), 0, st, prm);
    else if (bq == 64 && bk == 32) hipLaunchKernelGGL((fwd_bf16_kernel<64, 32>), grd, dim3(128), 0, st, prm);
    else if (bq == 64 && bk == 64) hipLaunchKernelGGL((fwd_bf16_kernel<64, 64>), grd, dim3(128), 0, st, prm);
    else if (bq == 128 && bk == 32) hipLaunchKernelGGL((fwd_bf16_kernel<128, 32>), grd, dim3(256), 0, st, prm);
    else if (bq == 128 && bk == 64) hipLaunchKernelGGL((fwd_bf16_kernel<128, 64>), grd, dim3(256), 0, st, prm);
    else return SA_EUNSUPPORTED;
  } else {
    if (bq == 32 && bk == 32) hipLaunchKernelGGL((fwd_f32_kernel<32, 32>), grd, dim3(64), 0, st, prm);
    else if (bq == 64 && bk == 32) hipLaunchKernelGGL((fwd_f32_kernel<64, 32>), grd, dim3(128), 0, st, prm);
    else if (bq == 128 && bk == 32) hipLaunchKernelGGL((fwd_f32_kernel<128, 32>), grd, dim3(256), 0, st, prm);
    else return SA_EUNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? SA_OK : SA_EHIP;
}
