// Backward kernels: gradients by recomputation from the per-row log-sum-exp.
//
// "Sparse Transformers 深度解读报告", section 3.4: attention weights are not
// kept from the forward pass; the backward pass rebuilds them.  With
// P_ij = exp(S_ij - LSE_i) on the visible pairs:
//     dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
//     dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,
//     dK_j = scale sum_i dS_ij q_i.
//
// Three launches on the caller's stream:
//   bwd_pre   D_i = rowsum(dO_i * O_i) (float32) and a zeroed float32 dQ
//             accumulator, one pass over the query rows;
//   bwd_main  one workgroup per key tile (block_k keys of one (batch, head)),
//             walking that tile's CSC list of query tiles.  Each wave owns
//             32 keys and keeps K, V (as MFMA operands) and its dK, dV
//             accumulators in registers.  Per query tile: Q, Q^T, dO, dO^T,
//             LSE and D are staged in LDS; S = Q K^T and dP = dO V^T on the
//             MFMA units; P and dS in registers; dV^T += dO^T P and
//             dK^T += Q^T dS on the MFMA units; dS goes through LDS so that
//             dQ = dS K (all keys of the tile) is formed per query block and
//             added to the float32 accumulator with atomics.  The tile's dK,
//             dV rows are written once at the end (exact zeros for keys no
//             query reads);
//   bwd_post  dQ = scale * accumulator, cast to the output type.

#include <math.h>

#include "device_common.hpp"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const uint8_t* blob;
  const int32_t* sched;  // (head, k-tile) pairs
  int32_t B, H, n;
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dsum;    // D, [B, H, n]
  float* dq_acc;  // [B, H, n, 64]
  float scale;
  float scale_log2;
  int64_t rows;  // B * H * n
};

// --------------------------------------------------------------------------
// D = rowsum(dO * O); zero the dQ accumulator.  8 threads per row.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t >> 3;
  const int part = int(t & 7);
  float acc = 0.f;
  if (row < p.rows) {
    const bf16x8 a = reinterpret_cast<const bf16x8*>(p.o + row * kD)[part];
    const bf16x8 b = reinterpret_cast<const bf16x8*>(p.dout + row * kD)[part];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += float(a[j]) * float(b[j]);
    floatx4* z = reinterpret_cast<floatx4*>(p.dq_acc + row * kD) + 2 * part;
    z[0] = floatx4{};
    z[1] = floatx4{};
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (row < p.rows && part == 0) p.dsum[row] = acc;
}

// --------------------------------------------------------------------------
// dQ = scale * accumulator -> bf16.  One thread per 8 features.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdParams p) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= p.rows * 8) return;
  const floatx4* src = reinterpret_cast<const floatx4*>(p.dq_acc) + 2 * t;
  const floatx4 a = src[0], b = src[1];
  float tmp[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int j = 0; j < 8; ++j) tmp[j] *= p.scale;
  reinterpret_cast<bf16x8*>(p.dq)[t] = pack_bf16x8(tmp);
}

// --------------------------------------------------------------------------
// Main kernel.  BK = 32 * NW keys per workgroup; query tiles of BQ rows are
// processed in steps of QS = min(BQ, 64) rows.
// --------------------------------------------------------------------------
template <int BQ, int BK>
__global__ __launch_bounds__(BK * 2) void bwd_main_kernel(BwdParams p) {
  constexpr int NW = BK / 32;
  constexpr int NT = NW * 64;
  constexpr int QS = BQ < 64 ? BQ : 64;  // query rows per step
  constexpr int NSTEP = BQ / QS;
  constexpr int NQB = QS / 32;          // 32-row query blocks per step
  constexpr int RS = kD + 8;            // row stride of Q / dO in LDS
  constexpr int TS = QS + 8;            // row stride of Q^T / dO^T in LDS
  constexpr int DSS = BK + 8;           // row stride of dS in LDS
  constexpr int KTS = BK + 8;           // row stride of K^T in LDS
  constexpr int CPT = QS * 8 / NT;      // 16-byte chunks per thread and tensor per step
  static_assert(CPT >= 1 && (QS * 8) % NT == 0, "tile/wave mismatch");
  constexpr int NUNITS = NQB * 2;       // dQ work units: (query block, feature block)

  __shared__ __attribute__((aligned(16))) bf16 sq[QS * RS];
  __shared__ __attribute__((aligned(16))) bf16 sqt[kD * TS];
  __shared__ __attribute__((aligned(16))) bf16 sdo[QS * RS];
  __shared__ __attribute__((aligned(16))) bf16 sdot[kD * TS];
  __shared__ __attribute__((aligned(16))) bf16 sds[QS * DSS];
  __shared__ __attribute__((aligned(16))) bf16 skt[kD * KTS];
  __shared__ __attribute__((aligned(16))) float slse[QS];
  __shared__ __attribute__((aligned(16))) float sdd[QS];
  __shared__ __attribute__((aligned(16))) int32_t slo[QS];
  __shared__ __attribute__((aligned(16))) int32_t shi[QS];
  __shared__ __attribute__((aligned(16))) int32_t stok[2][QS];  // by step parity: read after restaging

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.x % p.B;
  const int item = blockIdx.x / p.B;
  const int head = p.sched[2 * item], kt = p.sched[2 * item + 1];
  const PatView pv = pattern_of_head(p.blob, head);
  const size_t base = (size_t(b) * p.H + head) * size_t(p.n);

  // This lane's key (column of S): position kt*BK + 32w + l32.
  const int kpos = kt * BK + 32 * w + l32;
  const int ktok = pv.kmap[kpos];
  bf16x8 kq[4], vq[4];
  if (ktok >= 0) {
    const bf16x8* ks = reinterpret_cast<const bf16x8*>(p.k + (base + ktok) * kD);
    const bf16x8* vs = reinterpret_cast<const bf16x8*>(p.v + (base + ktok) * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kq[c] = ks[2 * c + g];
      vq[c] = vs[2 * c + g];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kq[c] = bf16x8{};
      vq[c] = bf16x8{};
    }
  }
  // K^T for the dQ product: skt[feature][key].
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) skt[(16 * c + 8 * g + j) * KTS + 32 * w + l32] = kq[c][j];

  floatx16 dva[2], dka[2];
  dva[0] = dva[1] = dka[0] = dka[1] = floatx16{};

  const int c0 = pv.col_ptr[kt], c1 = pv.col_ptr[kt + 1];
  const int nsteps = (c1 - c0) * NSTEP;
  const float c2 = p.scale_log2;

  u32x4 qreg[CPT], doreg[CPT];
  float lse_r = 0.f, dd_r = 0.f;
  int lo_r = 1, hi_r = 0, tok_r = -1;
  auto gload = [&](int step) {
    const int e = c0 + step / NSTEP;
    const int r0 = pv.row[e] * BQ + (step % NSTEP) * QS;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, j = c >> 3, cc = c & 7;
      const int tk = pv.qmap[r0 + j];
      if (tk >= 0) {
        qreg[i] = reinterpret_cast<const u32x4*>(p.q + (base + tk) * kD)[cc];
        doreg[i] = reinterpret_cast<const u32x4*>(p.dout + (base + tk) * kD)[cc];
      } else {
        qreg[i] = u32x4{0u, 0u, 0u, 0u};
        doreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < QS) {
      const int r = r0 + tid;
      tok_r = pv.qmap[r];
      lo_r = pv.lo[r];
      hi_r = pv.hi[r];
      if (tok_r >= 0) {
        lse_r = p.lse[base + tok_r] * kLog2e;
        dd_r = p.dsum[base + tok_r];
      } else {
        lse_r = 0.f;
        dd_r = 0.f;
      }
    }
  };
  auto lstore = [&](int parity) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT, j = c >> 3, cc = c & 7;
      *reinterpret_cast<u32x4*>(&sq[j * RS + cc * 8]) = qreg[i];
      *reinterpret_cast<u32x4*>(&sdo[j * RS + cc * 8]) = doreg[i];
      const bf16x8 a = __builtin_bit_cast(bf16x8, qreg[i]);
      const bf16x8 d = __builtin_bit_cast(bf16x8, doreg[i]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        sqt[(cc * 8 + t) * TS + j] = a[t];
        sdot[(cc * 8 + t) * TS + j] = d[t];
      }
    }
    if (tid < QS) {
      slse[tid] = lse_r;
      sdd[tid] = dd_r;
      slo[tid] = lo_r;
      shi[tid] = hi_r;
      stok[parity][tid] = tok_r;
    }
  };

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int e = c0 + step / NSTEP;
    const bool full = pv.bflag[e] == SA_TILE_FULL;
    if (step + 1 < nsteps) gload(step + 1);

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      floatx16 s = floatx16{}, dp = floatx16{};
      const bf16* qrow = &sq[(32 * qb + sigma32(l32)) * RS + 8 * g];
      const bf16* dorow = &sdo[(32 * qb + sigma32(l32)) * RS + 8 * g];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = mfma_bf16(*reinterpret_cast<const bf16x8*>(qrow + 16 * c), kq[c], s);
        dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(dorow + 16 * c), vq[c], dp);
      }
      // Register r of half g holds query 32*qb + kappa(r, g), key = lane.
      float pr[16], ds[16];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int qloc = 32 * qb + 16 * h8 + 8 * g;
        const floatx4 la = *reinterpret_cast<const floatx4*>(&slse[qloc]);
        const floatx4 lb = *reinterpret_cast<const floatx4*>(&slse[qloc + 4]);
        const floatx4 da = *reinterpret_cast<const floatx4*>(&sdd[qloc]);
        const floatx4 db = *reinterpret_cast<const floatx4*>(&sdd[qloc + 4]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * h8 + j;
          const float lse2 = j < 4 ? la[j] : lb[j - 4];
          const float dd = j < 4 ? da[j] : db[j - 4];
          float pv_ = fast_exp2(s[r] * c2 - lse2);
          if (!full) {
            const int qi = qloc + j;
            const bool vis = kpos >= slo[qi] && kpos <= shi[qi];
            pv_ = vis ? pv_ : 0.f;
          }
          pr[r] = pv_;
          ds[r] = pv_ * (dp[r] - dd);
        }
      }
      // dV^T += dO^T P ;  dK^T += Q^T dS   (K slots = 16 queries per MFMA).
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const bf16x8 pb = pack_bf16x8(&pr[8 * h8]);
        const bf16x8 sb = pack_bf16x8(&ds[8 * h8]);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
          const int trow = (32 * fb + sigma32(l32)) * TS + 32 * qb + 16 * h8 + 8 * g;
          dva[fb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(&sdot[trow]), pb, dva[fb]);
          dka[fb] = mfma_bf16(*reinterpret_cast<const bf16x8*>(&sqt[trow]), sb, dka[fb]);
        }
      }
      // dS -> LDS as [query][key] (bf16) for the dQ product.
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sds[(32 * qb + kappa32(r, g)) * DSS + 32 * w + l32] = bf16(ds[r]);
    }
    __syncthreads();
    if (step + 1 < nsteps) lstore((step + 1) & 1);  // staging buffers are free; dS, K^T untouched

    // dQ[query block][feature block] = dS K over all BK keys of the tile.
    for (int u = w; u < NUNITS; u += NW) {
      const int qb = u >> 1, fb = u & 1;
      floatx16 acc = floatx16{};
      const bf16* arow = &sds[(32 * qb + sigma32(l32)) * DSS + 8 * g];
      const bf16* brow = &skt[(32 * fb + l32) * KTS + 8 * g];
#pragma unroll
      for (int c = 0; c < BK / 16; ++c)
        acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(arow + 16 * c),
                        *reinterpret_cast<const bf16x8*>(brow + 16 * c), acc);
      // Register r of half g: query 32*qb + kappa(r, g), feature 32*fb + lane.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tq = stok[step & 1][32 * qb + kappa32(r, g)];
        if (tq >= 0) unsafeAtomicAdd(p.dq_acc + (base + tq) * kD + 32 * fb + l32, acc[r]);
      }
    }
    __syncthreads();
  }

  // dK, dV rows of this wave's 32 keys; register r of half g = feature
  // 32*fb + kappa(r, g), lane = key.
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
}

}  // namespace sa

// --------------------------------------------------------------------------
// C ABI entry points
// --------------------------------------------------------------------------
#include "abi_common.hpp"

namespace {

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

size_t workspace_bytes(int64_t rows) {
  return round256(size_t(rows) * sizeof(float)) + size_t(rows) * sa::kD * sizeof(float);
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
  *bytes = workspace_bytes(int64_t(B) * H * h.n);
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
  const bool bq_ok = li.block_q == 32 || li.block_q == 64 || li.block_q == 128;
  const bool bk_ok = li.block_k == 32 || li.block_k == 64;
  if (!bq_ok || !bk_ok) return SA_EUNSUPPORTED;
  float sc;
  rc = resolve_scale(scale, d, &sc);
  if (rc != SA_OK) return rc;
  const int64_t rows = int64_t(B) * H * li.n;
  if (B == 0) return SA_OK;  // empty batch: pointers may be NULL
  if (ws_bytes < workspace_bytes(rows)) return SA_ESIZE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return SA_EINVAL;
  const int64_t grid = int64_t(li.bwd_sched_len) * B;
  if (grid > INT32_MAX || rows * 8 / 256 + 1 > INT32_MAX) return SA_EUNSUPPORTED;

  BwdParams prm;
  prm.blob = static_cast<const uint8_t*>(blob_dev);
  prm.sched = reinterpret_cast<const int32_t*>(prm.blob + li.bwd_sched_off);
  prm.B = B;
  prm.H = H;
  prm.n = int32_t(li.n);
  prm.q = static_cast<const bf16*>(q);
  prm.k = static_cast<const bf16*>(k);
  prm.v = static_cast<const bf16*>(v);
  prm.o = static_cast<const bf16*>(o);
  prm.lse = lse;
  prm.dout = static_cast<const bf16*>(dO);
  prm.dq = static_cast<bf16*>(dq);
  prm.dk = static_cast<bf16*>(dk);
  prm.dv = static_cast<bf16*>(dv);
  prm.dsum = static_cast<float*>(workspace);
  prm.dq_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                        ((size_t(rows) * sizeof(float) + 255) & ~size_t(255)));
  prm.scale = sc;
  prm.scale_log2 = float(double(sc) * 1.4426950408889634);
  prm.rows = rows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 pre_grid{unsigned((rows * 8 + 255) / 256), 1u, 1u};
  if (phases & SA_BWD_PREPARE) hipLaunchKernelGGL(bwd_pre_kernel, pre_grid, dim3(256), 0, st, prm);
  const dim3 grd{unsigned(grid), 1u, 1u};
  const int bq = li.block_q, bk = li.block_k;
  if (!(phases & SA_BWD_MAIN) || grid == 0) {
    // nothing to launch for the main phase
  } else if (bq == 32 && bk == 32) hipLaunchKernelGGL((bwd_main_kernel<32, 32>), grd, dim3(64), 0, st, prm);
  else if (bq == 64 && bk == 32) hipLaunchKernelGGL((bwd_main_kernel<64, 32>), grd, dim3(64), 0, st, prm);
  else if (bq == 128 && bk == 32) hipLaunchKernelGGL((bwd_main_kernel<128, 32>), grd, dim3(64), 0, st, prm);
  else if (bq == 32 && bk == 64) hipLaunchKernelGGL((bwd_main_kernel<32, 64>), grd, dim3(128), 0, st, prm);
  else if (bq == 64 && bk == 64) hipLaunchKernelGGL((bwd_main_kernel<64, 64>), grd, dim3(128), 0, st, prm);
  else if (bq == 128 && bk == 64) hipLaunchKernelGGL((bwd_main_kernel<128, 64>), grd, dim3(128), 0, st, prm);
  if (phases & SA_BWD_FINISH) hipLaunchKernelGGL(bwd_post_kernel, pre_grid, dim3(256), 0, st, prm);
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
