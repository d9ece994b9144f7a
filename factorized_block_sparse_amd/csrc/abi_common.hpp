// Argument validation shared by the C ABI entry points (host code).
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "sparse_attn.h"

namespace sa {

struct LaunchInfo {
  int64_t n;
  int32_t block_q, block_k, num_heads, n_pad, nqt, nkt;
  int32_t fwd_sched_len, bwd_sched_len;
  int64_t fwd_sched_off, bwd_sched_off, total_bytes;
  int64_t fwd_xl_off, bwd_xl_off, fwd_xitem_off, bwd_xitem_off;
  int32_t fwd_xl_len, bwd_xl_len;
  bool has_pre;  // some pattern's rows read a key prefix
  int32_t num_merged, fwdp_xl_len, bwdp_xl_len;  // two-part heads and their part lists
  int64_t fwdp_xitem_off, bwdp_xitem_off;
  int32_t dq_xl_len, seg_xl_len, seg_tiles;  // the dQ pass's list; the segment pass
  int64_t dq_xitem_off, seg_xitem_off;
};

inline bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the blob and the shapes common to forward and backward; fills `li`.
inline int validate_common(const void* blob_host, const void* blob_dev, int B, int H, int d,
                           int dtype, LaunchInfo* li) {
  if (!blob_host) return SA_EINVAL;
  sa_blob_header h;
  memcpy(&h, blob_host, sizeof(h));
  if (h.magic != SA_BLOB_MAGIC || h.version != SA_BLOB_VERSION) return SA_EINVAL;
  const int rc = sparse_attn_layout_check(blob_host, size_t(h.total_bytes));
  if (rc != SA_OK) return rc;
  if (!blob_dev || (reinterpret_cast<uintptr_t>(blob_dev) & 63u) != 0) return SA_EINVAL;
  if (B < 0 || H < 1 || H != h.num_heads) return SA_EINVAL;
  if (dtype != SA_BF16 && dtype != SA_FP32) return SA_EINVAL;
  if (d != 64) return SA_EUNSUPPORTED;
  // Element offsets of [B, H, n, d] must fit the kernels' 64-bit arithmetic and
  // per-(b, h) 32-bit row indices.
  if (int64_t(B) * H * h.n > (int64_t(1) << 40)) return SA_EUNSUPPORTED;
  // bf16 kernels address a (b, h) slice with 32-bit byte offsets (128 B rows).
  if (dtype == SA_BF16 && h.n >= (int64_t(1) << 25)) return SA_EUNSUPPORTED;
  li->n = h.n;
  li->block_q = h.block_q;
  li->block_k = h.block_k;
  li->num_heads = h.num_heads;
  li->n_pad = h.n_pad;
  li->nqt = h.nqt;
  li->nkt = h.nkt;
  li->fwd_sched_len = h.fwd_sched_len;
  li->bwd_sched_len = h.bwd_sched_len;
  li->fwd_sched_off = h.fwd_sched_off;
  li->bwd_sched_off = h.bwd_sched_off;
  li->total_bytes = h.total_bytes;
  li->fwd_xl_off = h.fwd_xl_off;
  li->bwd_xl_off = h.bwd_xl_off;
  li->fwd_xl_len = h.fwd_xl_len;
  li->bwd_xl_len = h.bwd_xl_len;
  li->fwd_xitem_off = h.fwd_xitem_off;
  li->bwd_xitem_off = h.bwd_xitem_off;
  li->num_merged = h.num_merged;
  li->fwdp_xl_len = h.fwdp_xl_len;
  li->bwdp_xl_len = h.bwdp_xl_len;
  li->fwdp_xitem_off = h.fwdp_xitem_off;
  li->bwdp_xitem_off = h.bwdp_xitem_off;
  li->dq_xl_len = h.dq_xl_len;
  li->seg_xl_len = h.seg_xl_len;
  li->seg_tiles = h.seg_tiles;
  li->dq_xitem_off = h.dq_xitem_off;
  li->seg_xitem_off = h.seg_xitem_off;
  li->has_pre = false;
  for (int32_t i = 0; i < h.num_patterns; ++i) {
    sa_pattern_rec r;
    memcpy(&r, static_cast<const uint8_t*>(blob_host) + h.pattern_off + i * sizeof(r), sizeof(r));
    li->has_pre |= r.pre_off != 0;
  }
  return SA_OK;
}

// Device addresses of the first kArgPatterns patterns' arrays (host side of
// PatTable: offsets from the host blob, added to the device copy's address).
template <typename Table>
inline void fill_pattern_table(const void* blob_host, const void* blob_dev, Table* t) {
  const uint8_t* hb = static_cast<const uint8_t*>(blob_host);
  const uint8_t* db = static_cast<const uint8_t*>(blob_dev);
  sa_blob_header h;
  memcpy(&h, hb, sizeof(h));
  const int np = h.num_patterns < kArgPatterns ? h.num_patterns : kArgPatterns;
  memset(t, 0, sizeof(*t));
  for (int i = 0; i < np; ++i) {
    sa_pattern_rec r;
    memcpy(&r, hb + h.pattern_off + i * sizeof(sa_pattern_rec), sizeof(r));
    auto& v = t->pv[i];
    v.qmap = reinterpret_cast<const int32_t*>(db + r.qmap_off);
    v.kmap = reinterpret_cast<const int32_t*>(db + r.kmap_off);
    v.lo = reinterpret_cast<const int32_t*>(db + r.lo_off);
    v.hi = reinterpret_cast<const int32_t*>(db + r.hi_off);
    v.pre = r.pre_off ? reinterpret_cast<const int32_t*>(db + r.pre_off) : nullptr;
    v.ident = identity_maps(r.kind);
    v.row_ptr = reinterpret_cast<const int32_t*>(db + r.row_ptr_off);
    v.col = reinterpret_cast<const int32_t*>(db + r.col_off);
    v.fflag = db + r.fflag_off;
    v.col_ptr = reinterpret_cast<const int32_t*>(db + r.col_ptr_off);
    v.row = reinterpret_cast<const int32_t*>(db + r.row_off);
    v.bflag = db + r.bflag_off;
  }
}

// scale <= 0 selects 1/sqrt(d) (blog post on sliding windows, section 01).
inline int resolve_scale(float scale, int d, float* out) {
  if (scale != scale || isinf(scale)) return SA_EINVAL;
  *out = scale > 0.f ? scale : float(1.0 / sqrt(double(d)));
  return SA_OK;
}

}  // namespace sa
