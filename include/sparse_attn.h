/*
 * sparse_attn.h -- C ABI of the causal factorized block-sparse attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Masked softmax attention (blog post "长序列为何不必让每个
 * token 看见全部历史？滑动窗口、块稀疏与全局 token", section 02): with
 * S_ij = scale * q_i . k_j over the keys j that query i may read,
 *     O_i = sum_j softmax_j(S_ij) v_j,    LSE_i = log sum_j exp(S_ij),
 * and its gradients.  The sets of keys come from the factorized heads of
 * "Sparse Transformers 深度解读报告", section 2.2 (all causal, j <= i):
 *     SA_LOCAL      strided head 1:  {max(0, i - l) .. i}
 *     SA_STRIDE     strided head 2:  {j <= i : (i - j) mod l == 0}
 *     SA_SAMEBLOCK  fixed head 1:    {j <= i : floor(j / l) == floor(i / l)}
 *     SA_SUMMARY    fixed head 2:    {j <= i : s <= j mod l <= s + c - 1},
 *                   s = l - (k + 1) c for sub-block k = sub mod (l / c)
 *     SA_FIXED_MERGED  one head reading the union of the two fixed sets (the
 *                   merged integration of report section 3.1, Eq. 7)
 *     SA_LOCAL_GLOBAL  {j <= i : i - j <= l or j < c}: the causal window plus
 *                   the first c positions as global tokens (blog post sections
 *                   03 and 04)
 *     SA_STRIDED_MERGED  one head reading the union of the two strided sets
 *                   (report section 3.1, Eq. 7), run in two parts with
 *                   disjoint key sets: the stride members at distance >= 2l
 *                   first, then the local band, which starts from the first
 *                   part's softmax state (forward) or sums (backward)
 * Rows left empty by a summary head (i < s) read only themselves when
 * SA_SELF_IF_EMPTY is set (the default reading; without it such a layout is
 * rejected, since an empty row has no softmax).  Execution is at tile
 * granularity: only (query-tile, key-tile) pairs holding at least one
 * visible pair are computed (report section 3.5; blog post section 05).
 *
 * Conventions.
 *   - Tensors are contiguous [B, H, n, d] (batch, head, position, feature),
 *     d innermost; LSE is [B, H, n] float32.  Head h uses the layout's
 *     pattern of head h; H must equal the layout's num_heads.
 *   - d must be 64.  dtype SA_BF16 (bfloat16 data, float32 accumulation)
 *     for forward and backward, with n < 2^25 (SA_EUNSUPPORTED otherwise);
 *     SA_FP32 (float32 throughout) for forward, on layouts without two-part
 *     heads (SA_STRIDED_MERGED; SA_EUNSUPPORTED otherwise).
 *   - Tile shapes run by the kernels: bf16, any block_q of 32, 64, 128 with
 *     block_k of 32 or 64, and block_q = block_k = 128; fp32, block_k = 32.
 *     Other layouts build, and their calls return SA_EUNSUPPORTED.
 *   - Pointers q, k, v, o, lse, dO, dq, dk, dv and workspace are device
 *     pointers (hipMalloc'd or equivalent) aligned to 16 bytes; blob_host is
 *     a host pointer; blob_dev is a device copy of the same bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work and return without synchronising.
 *
 * Ownership.  The caller owns every buffer.  The library allocates and frees
 * no device memory and keeps no global mutable state, with one exception:
 * sparse_attn_bwd_static works in a file-scope device array of its own (one
 * per GPU, see there).  The layout blob is an immutable, position-independent
 * byte array that may be shared across streams and calls.
 *
 * Errors.  Every function returns SA_OK (0) or a negative status and never
 * aborts.  Arguments are validated before anything is enqueued, so an error
 * leaves every output untouched.  A failed kernel launch returns SA_EHIP;
 * faults during execution surface at the caller's next synchronisation.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sa_status {
  SA_OK = 0,
  SA_EINVAL = -1,        /* malformed argument: NULL/misaligned pointer, bad size or pattern */
  SA_EUNSUPPORTED = -2,  /* well-formed but not implemented: d != 64, dtype, tile shape */
  SA_ESIZE = -3,         /* a caller buffer is too small (blob or workspace) */
  SA_EHIP = -4,          /* the HIP runtime reported an error at launch */
  SA_ENOMEM = -5         /* the layout build ran out of host memory */
};

enum sa_head_kind {
  SA_LOCAL = 0,
  SA_STRIDE = 1,
  SA_SAMEBLOCK = 2,
  SA_SUMMARY = 3,
  SA_FIXED_MERGED = 4,
  SA_LOCAL_GLOBAL = 5,
  SA_STRIDED_MERGED = 6,
  /* blob-only pattern kind (never a head's kind): {j <= i : i - j >= 2l,
   * (i - j) mod l == 0}, the second part of an SA_STRIDED_MERGED head */
  SA_STRIDE_FAR = 7
};

enum sa_dtype { SA_BF16 = 0, SA_FP32 = 1 };

/* Layout flag: a row whose set is empty reads itself (report section 2.2 gives
 * no rule; the blog post's section 02 forbids empty rows). */
#define SA_SELF_IF_EMPTY 1u
/* Layout flag: no segment pass (see sa_blob_header); every head's backward
 * then runs through the dQ and dK/dV passes, for comparisons. */
#define SA_NO_SEGMENT_PASS 2u

/* One head's pattern.  c is the summary width (SA_SUMMARY, SA_FIXED_MERGED)
 * or the number of leading global tokens (SA_LOCAL_GLOBAL); sub is used by
 * SA_SUMMARY and SA_FIXED_MERGED only. */
typedef struct {
  int32_t kind;  /* enum sa_head_kind */
  int32_t l;     /* band width / stride / block length, >= 1 */
  int32_t c;     /* summary width, 1 <= c <= l; or global tokens, >= 0 */
  int32_t sub;   /* summary sub-block index, >= 0 (taken mod l / c) */
} sa_head_pattern;

typedef struct {
  int64_t n;                     /* sequence length, 1 <= n <= 2^26 */
  int32_t block_q;               /* query-tile rows: 32, 64 or 128 */
  int32_t block_k;               /* key-tile columns: 32, 64 or 128 */
  int32_t num_heads;             /* 1 .. 4096 */
  const sa_head_pattern* heads;  /* num_heads entries, host memory */
  uint32_t flags;                /* SA_SELF_IF_EMPTY, SA_NO_SEGMENT_PASS, or 0 */
  int32_t split_keys;            /* query-tile chunk cap in keys; 0 = SA_SPLIT_KEYS */
  int32_t split_rows;            /* key-tile chunk cap in query rows; 0 = SA_SPLIT_ROWS */
} sa_layout_desc;

/* ---------------------------------------------------------------------------
 * Layout blob.  Built once per (n, tiles, head patterns) and reused by every
 * forward and backward call (blog post section 09: build the block mask once
 * for a fixed length and pattern).  All offsets are bytes from the start of
 * the blob and 64-byte aligned.
 *
 * Each distinct head pattern is described in its own "layout space": query
 * position p in [0, n_pad) holds token qmap[p], key position q holds token
 * kmap[q] (-1 = padding past n).  The maps are permutations of [0, n):
 *   SA_LOCAL, SA_SAMEBLOCK: identity.
 *   SA_STRIDE: residue-class order (the column view of the (n/l) x l grid,
 *     comparison article "稀疏与局部注意力", section 2): token t*l + r sits at
 *     position (number of tokens of residues < r) + t, for queries and keys.
 *   SA_SUMMARY: queries identity; keys are the summary cells in increasing
 *     order, then the tokens of rows that read only themselves, then every
 *     other token (keys nobody reads: their dK/dV are zero).
 *   SA_FIXED_MERGED: queries identity; keys are the summary cells in
 *     increasing order, then every other token in increasing order.
 *   SA_LOCAL_GLOBAL: identity.
 *   SA_STRIDE_FAR: residue-class order as SA_STRIDE; a row reads its own class
 *     up to two positions before itself.
 * In layout space every query row reads a prefix and one interval of key
 * positions, [0, pre[p]) and [lo[p], hi[p]], with pre[p] <= lo[p] when the
 * interval is not empty (lo > hi: empty).  The prefix is empty except for
 * SA_FIXED_MERGED (a row's summary cells up to itself; the interval holds
 * the other tokens of its block up to itself) and SA_LOCAL_GLOBAL (global
 * tokens before the window).  This is what makes the per-tile fine mask a
 * few comparisons.  Tiles: q-tile i covers positions
 * [i*block_q, (i+1)*block_q), k-tile j covers [j*block_k, (j+1)*block_k).  A
 * tile pair is active iff it holds a visible pair, FULL iff every pair in it
 * is visible.  CSR lists each q-tile's active k-tiles (ascending), CSC each
 * k-tile's active q-tiles (ascending).
 * ------------------------------------------------------------------------- */

#define SA_BLOB_MAGIC 0x31415053u /* "SPA1" */
#define SA_BLOB_VERSION 11u
#define SA_SCHED_FIELDS 9
/* Default chunk caps (sa_layout_desc.split_rows / split_keys).  Key tiles read
 * by more than split_rows query rows are split into chunks of at most that
 * many rows (rounded down to whole query tiles, at least one) for the dK/dV
 * pass, each chunk a workgroup; their partial sums are reduced in a fixed
 * order.  Query tiles that read more than split_keys keys are split the same
 * way for the forward and dQ passes; chunk results are merged in a fixed
 * order.  A cap of at least n disables splitting. */
#define SA_SPLIT_ROWS 1536
#define SA_SPLIT_KEYS 3072
/* Longest segment of the segment pass, in rows. */
#define SA_SEGMENT_ROWS 128
/* Number of accelerator complex dies (XCDs, each with its own L2) that
 * workgroups are dealt to round-robin on MI355X. */
#define SA_XCDS 8
#define SA_TILE_PARTIAL 0u
#define SA_TILE_FULL 1u

typedef struct {
  int32_t kind, l, c, sub;
  int32_t s;           /* summary: first residue of the sub-block; 0 otherwise */
  int32_t nnz;         /* active tiles */
  int64_t pairs;       /* visible (query, key) pairs */
  int64_t qmap_off;    /* int32[n_pad] */
  int64_t kmap_off;    /* int32[n_pad] */
  int64_t lo_off;      /* int32[n_pad] */
  int64_t hi_off;      /* int32[n_pad] */
  int64_t pre_off;     /* int32[n_pad]; 0 when every prefix is empty */
  int64_t count_off;   /* int32[n]: visible keys of token i (token order) */
  int64_t row_ptr_off; /* int32[nqt + 1] */
  int64_t col_off;     /* int32[nnz]: k-tile of each CSR entry */
  int64_t fflag_off;   /* uint8[nnz]: SA_TILE_FULL / SA_TILE_PARTIAL (CSR order) */
  int64_t col_ptr_off; /* int32[nkt + 1] */
  int64_t row_off;     /* int32[nnz]: q-tile of each CSC entry */
  int64_t bflag_off;   /* uint8[nnz]: flags in CSC order */
} sa_pattern_rec;

typedef struct {
  uint32_t magic, version;
  int64_t n;
  int32_t block_q, block_k;
  int32_t num_heads, num_patterns;
  int32_t n_pad;            /* n rounded up to a multiple of max(block_q, block_k) */
  int32_t nqt, nkt;         /* n_pad / block_q, n_pad / block_k */
  uint32_t flags;
  int64_t total_bytes;
  int64_t head_pattern_off; /* int32[num_heads]: pattern index of each head */
  int64_t pattern_off;      /* sa_pattern_rec[num_patterns] */
  int64_t fwd_sched_off;    /* int32[SA_SCHED_FIELDS * fwd_sched_len]: (head, q-tile,
                               first CSR entry, end CSR entry, partial slot, pattern index
                               of the head, first slot of the tile, chunks of the tile,
                               the first CSR entry's k-tile packed as (tile << 1) | FULL or
                               -1 for an empty list), heaviest first; unsplit tiles have
                               slot = slot0 = -1 and chunks = 1 */
  int64_t bwd_sched_off;    /* int32[SA_SCHED_FIELDS * bwd_sched_len]: the same fields over
                               k-tiles and CSC entries */
  int32_t fwd_sched_len, bwd_sched_len;
  int64_t red_sched_off;    /* int32[4 * red_sched_len]: (head, k-tile, first slot, chunks) */
  int32_t red_sched_len;
  int32_t num_slots;        /* partial slots per batch element */
  /* Per-XCD launch order.  Workgroup w of a launch runs on XCD w % SA_XCDS
   * (round-robin dispatch); its batch element and schedule entry are
   * b = (w / SA_XCDS) / len and xl[(w % SA_XCDS) * len + (w / SA_XCDS) % len]
   * (-1 = nothing to do).  Each XCD's list is a contiguous run of the
   * (head, tile) work in natural order -- so an XCD's L2 holds few heads --
   * sorted heaviest first and padded to the common length. */
  int64_t fwd_xl_off;       /* int32[SA_XCDS * fwd_xl_len], indices into fwd_sched */
  int64_t bwd_xl_off;       /* int32[SA_XCDS * bwd_xl_len], indices into bwd_sched */
  int32_t fwd_xl_len, bwd_xl_len;
  int64_t fwd_xitem_off;    /* int32[SA_XCDS * fwd_xl_len * SA_SCHED_FIELDS]: the entries
                               the lists name, in list order (all -1 for padding), so a
                               workgroup finds its work with a single read */
  int64_t bwd_xitem_off;    /* the same for bwd_sched */
  int64_t comb_sched_off;   /* int32[4 * comb_sched_len]: (head, q-tile, first slot, chunks) */
  int32_t comb_sched_len;
  int32_t num_qslots;       /* query-tile partial slots per batch element */
  int32_t split_keys, split_rows; /* chunk caps the schedules were built with */
  int64_t pairs_all_heads;  /* sum of pairs over the heads (one batch element) */
  int64_t tiles_all_heads;  /* sum of active tiles over the heads */
  /* Two-part heads (SA_STRIDED_MERGED).  The head's first pattern (head
   * pattern table) is its local band; its second part is listed here and runs
   * in separate launches before the main ones, writing float32 state per
   * token (forward: unnormalised O, running max, row sum; backward: dQ, dK,
   * dV sums) into the workspace; the main launches' first chunk of each of
   * the head's tiles starts from it.  Schedule entries of two-part heads
   * carry (index among them + 1) << 16 in the pattern field, and main
   * entries that start from the state also 1 << 30; the pattern index is
   * the low 16 bits. */
  int64_t head_part_off;    /* int32[num_heads]: second-part pattern, -1 if none */
  int64_t head_merged_off;  /* int32[num_heads]: index among two-part heads, -1 */
  int32_t num_merged;       /* two-part heads */
  int32_t fwdp_sched_len, bwdp_sched_len;
  int32_t fwdp_xl_len, bwdp_xl_len;
  int32_t pad0;
  int64_t fwdp_sched_off;   /* int32[SA_SCHED_FIELDS * fwdp_sched_len]: second-part q-tiles
                               (every one, none split) */
  int64_t bwdp_sched_off;   /* the same over second-part k-tiles */
  int64_t fwdp_xitem_off;   /* int32[SA_XCDS * fwdp_xl_len * SA_SCHED_FIELDS], as fwd_xitem */
  int64_t bwdp_xitem_off;   /* int32[SA_XCDS * bwdp_xl_len * SA_SCHED_FIELDS] */
  /* Segment pass of the backward.  A head whose rows read keys of their own
   * segment only -- a contiguous run of layout positions closed under the
   * pattern: an SA_STRIDE head's residue classes ("Sparse Transformers
   * 深度解读报告", section 2.2) -- takes dQ, dK and dV from one workgroup
   * per segment instead of the dQ and dK/dV passes, when its segments hold
   * at most SA_SEGMENT_ROWS rows, none of its tiles is split and the layout
   * was built without SA_NO_SEGMENT_PASS.  Its tiles then leave the dQ list
   * and the backward schedule; the forward is unchanged. */
  int32_t dq_xl_len, seg_xl_len;
  int32_t seg_len;          /* segments of one batch element */
  int32_t seg_tiles;        /* 32-row sub-tiles of the longest segment (1..4); 0 if none */
  int64_t dq_xitem_off;     /* int32[SA_XCDS * dq_xl_len * SA_SCHED_FIELDS]: the forward's
                               query-tile entries of the heads without segments, per-XCD
                               lists as fwd_xitem (the dQ pass's work) */
  int64_t seg_xitem_off;    /* int32[SA_XCDS * seg_xl_len * SA_SCHED_FIELDS]: (head, first
                               position, residue r, rows, stride l, pattern field, -1, 1,
                               -1) of each segment -- the class of tokens r + l t,
                               t < rows, in which token t reads t' <= t -- per-XCD lists
                               as fwd_xitem */
} sa_blob_header;

/* Build the layout.  With blob == NULL, only *blob_bytes is set (size query).
 * Otherwise *blob_bytes must hold the blob's capacity (SA_ESIZE if too small)
 * and is set to the bytes written.  Host-only; needs no GPU.  A pattern whose
 * active tiles could exceed INT32_MAX (the CSR / CSC index range) is refused
 * with SA_EUNSUPPORTED; SA_ENOMEM when host memory for the build runs out. */
int sparse_attn_layout(const sa_layout_desc* desc, void* blob, size_t* blob_bytes);

/* Check a blob's header and internal offsets (host). */
int sparse_attn_layout_check(const void* blob_host, size_t blob_bytes);

/* Split tiles and the workspace.  A query tile that reads more than
 * split_keys keys (a key tile read by more than split_rows query rows) runs as
 * several workgroups, each over one chunk of its CSR (CSC) list.  Each chunk
 * writes float32 partial results to the workspace; a merge launch combines
 * the chunks of every split tile in chunk order and writes the tile's
 * outputs.  No atomics: repeated calls are bitwise identical.
 *
 * Workspace (both passes): at least the size the *_workspace call returns,
 * 16-byte aligned, in device memory; its contents on entry do not matter.
 * Calls that share a workspace must not overlap in time (issue them on one
 * stream). */

/* Bytes of device workspace sparse_attn_fwd needs for these sizes (0 when
 * the layout splits no query tile and has no two-part head; the workspace
 * may then be NULL).  Two-part heads add float32 state of every token:
 * B * (two-part heads) * n * (64 + 2) floats. */
int sparse_attn_fwd_workspace(const void* blob_host, int B, int H, int d, int dtype,
                              size_t* bytes);

/* Forward (report sections 3.5 and 3.4): o [B,H,n,d] in dtype, lse [B,H,n]
 * float32.  scale <= 0 selects 1/sqrt(d).  B == 0 is a valid no-op (the
 * tensor pointers may then be NULL). */
int sparse_attn_fwd(const void* blob_host, const void* blob_dev, int B, int H, int d, int dtype,
                    const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t ws_bytes, float scale, void* stream);

/* The forward's two launches, separately (same arguments, one stream, in
 * order): SA_FWD_MAIN runs the block-sparse kernel (second parts of two-part
 * heads first, in a launch of their own; then unsplit query tiles write O
 * and LSE, chunks of split tiles write partial results to the workspace);
 * SA_FWD_MERGE merges the chunks of split tiles (the running
 * maxima rescaled to their common maximum) and writes their O and LSE.
 * sparse_attn_fwd runs SA_FWD_ALL. */
enum { SA_FWD_MAIN = 1, SA_FWD_MERGE = 2, SA_FWD_ALL = 3 };
int sparse_attn_fwd_phases(const void* blob_host, const void* blob_dev, int B, int H, int d,
                           int dtype, const void* q, const void* k, const void* v, void* o,
                           float* lse, void* workspace, size_t ws_bytes, float scale,
                           unsigned phases, void* stream);

/* Bytes of device workspace sparse_attn_bwd needs for these sizes. */
int sparse_attn_bwd_workspace(const void* blob_host, int B, int H, int d, int dtype,
                              size_t* bytes);

/* Backward by recomputation from LSE (report section 3.4): gradients of
 * sum(O * dO) with respect to q, k, v, written in dtype.  `o` and `lse` must
 * be the forward's outputs for the same inputs and scale.  Keys no query
 * reads in a head get exact zeros.  Only SA_BF16.  Two-part heads add three
 * float32 [B, two-part heads, n, 64] sums to the workspace. */
int sparse_attn_bwd(const void* blob_host, const void* blob_dev, int B, int H, int d, int dtype,
                    const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    void* workspace, size_t ws_bytes, float scale, void* stream);

/* The backward's launches, separately, for callers that interleave other
 * work between them or time them one by one:
 *   SA_BWD_SEG    per segment of the heads the segment pass runs (see
 *                 sa_blob_header): their dQ, dK and dV, independent of the
 *                 other phases;
 *   SA_BWD_DQ     per query tile of the other heads (long tiles in chunks):
 *                 D_i = dO_i . O_i (kept in the workspace) and dQ, or
 *                 float32 partial dQ of split tiles (workspace); second parts
 *                 of two-part heads first, in a launch of their own;
 *   SA_BWD_DKDV   per key tile of the other heads (long tiles in chunks): dK
 *                 and dV, or float32 partial sums of split tiles (workspace);
 *                 second parts first, likewise;
 *   SA_BWD_MERGE  sums the partials of split query and key tiles in a fixed
 *                 order and writes their dQ, dK, dV.
 * Phases must run in this order on one stream with the same arguments and
 * workspace; sparse_attn_bwd is sparse_attn_bwd_phases(..., SA_BWD_ALL). */
enum { SA_BWD_DQ = 1, SA_BWD_DKDV = 2, SA_BWD_MERGE = 4, SA_BWD_SEG = 8, SA_BWD_ALL = 15 };
int sparse_attn_bwd_phases(const void* blob_host, const void* blob_dev, int B, int H, int d,
                           int dtype, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dO, void* dq, void* dk, void* dv,
                           void* workspace, size_t ws_bytes, float scale, unsigned phases,
                           void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * (code under stream capture, serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as sparse_attn_bwd, without the
 * workspace: the library uses a file-scope device array of
 * SA_STATIC_SCRATCH_BYTES instead, one per GPU, held from the library's first
 * use on that GPU until the process ends.  Its device address is looked up
 * once per GPU (the current device of the first call).  Returns SA_ESIZE,
 * before any work is enqueued, when these sizes need more workspace than
 * that (sparse_attn_bwd_workspace tells how much).  Calls allocate and free
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller; the array keeps the previous call's contents,
 * which the backward never reads before writing. */
#define SA_STATIC_SCRATCH_BYTES (64u << 20)
int sparse_attn_bwd_static(const void* blob_host, const void* blob_dev, int B, int H, int d,
                           int dtype, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dO, void* dq, void* dk, void* dv,
                           float scale, void* stream);

/* Static description of a status code. */
const char* sparse_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
