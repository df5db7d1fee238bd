/*
 * blockdiag.h -- C ABI of the block-diagonal (per-document causal) packed
 * attention library for AMD Instinct MI355X (gfx950).
 *
 * What it computes (Automodel page "feat(distributed): block-diagonal varlen
 * CP for packed sequences"):
 *   - Summary / Motivation: a packed row holds several documents back to back;
 *     a query attends a key only inside its own document and only at or before
 *     its own position (block-causal), exactly as a dense masked SDPA would.
 *   - Design overview, batch.py and packed.py; key property 1: one GPU holds a
 *     contiguous chunk of query rows [row_offset, row_offset + q_len) of every
 *     batch row and the K/V of the whole row; row_offset = 0 with q_len = S is
 *     the single-GPU packed case.
 *   - Summary and Design overview, kernels.py: the varlen kernel is driven by
 *     cu_seqlens metadata that is computed and validated on the host once per
 *     step, so no layer needs a host sync and no bad offset reaches a kernel.
 *   - key property 2: a document that starts left of the chunk gives its first
 *     segment more keys than queries, aligned bottom-right.
 *
 * Conventions shared by every call:
 *   - Every function returns a bd_status; nothing throws across the ABI.  On a
 *     non-OK status blockdiag_last_error() returns a message (thread-local,
 *     valid until the next call on the same thread).
 *   - Argument checks run on the host before anything is enqueued: a call that
 *     returns an error has launched nothing.
 *   - "device" pointers are HIP device memory; "host" pointers are ordinary
 *     host memory.  The caller allocates and owns every buffer; the library
 *     never allocates or frees memory, keeps no pointer after returning, and
 *     creates no stream.  Work is enqueued on the caller's stream (a
 *     hipStream_t passed as void*; NULL = the default stream) with no host
 *     synchronisation.  A fault during execution surfaces at the caller's next
 *     synchronisation.
 *   - Tensors are dense, row-major, contiguous:
 *       q, o, dO, dq : [batch][q_len][h_q][head_dim]
 *       k, v, dk, dv : [batch][kv_len][h_kv][head_dim]: keys
 *                      [kv_begin, kv_begin + kv_len) of every row -- the
 *                      whole packed row (kv_begin = 0, kv_len = seq_len) or
 *                      a window holding every key the chunk attends (Summary
 *                      and Design overview, exchange.py: needed-only K/V)
 *       lse          : [batch][h_q][q_len] float32, natural log of the softmax
 *                      denominator in units of scaled logits; -inf on rows
 *                      that attend no key (padding)
 *     Element type: float32 (BD_F32) or bfloat16 (BD_BF16) for every tensor
 *     except lse (always float32).  Grouped-query attention: query head h reads
 *     K/V head h / (h_q / h_kv).
 *   - Padding: positions past the sum of a row's document lengths belong to no
 *     document.  A padding query row gets O = 0, LSE = -inf, dQ = 0; a key no
 *     local row attends gets dK = dV = 0.
 */
#ifndef BLOCKDIAG_H
#define BLOCKDIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BD_OK = 0,
  BD_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size    */
  BD_ERR_BAD_METADATA = 2,  /* document lengths or segment table malformed    */
  BD_ERR_CAPACITY = 3,      /* output arrays too small; *n_seg holds the need */
  BD_ERR_WORKSPACE = 4,     /* workspace smaller than blockdiag_workspace_bytes */
  BD_ERR_UNSUPPORTED = 5,   /* valid but not implemented (dtype, head_dim)    */
  BD_ERR_HIP = 6            /* the HIP runtime refused a launch               */
} bd_status;

typedef enum { BD_F32 = 0, BD_BF16 = 1 } bd_dtype;

/*
 * blockdiag_segment -- varlen segment table of one chunk (host only, integer
 * only, deterministic).  Summary: per-step precomputed cu_seqlens; Design
 * overview, kernels.py: varlen segmentation plus host-side validation.  Call
 * once per step; every layer reuses the result.
 *
 * Inputs (host):
 *   doc_lens[sum(docs_per_row)]  document lengths of all batch rows, row after
 *                                row; each >= 0 (a zero-length document holds
 *                                no token); per row the sum is <= seq_len and
 *                                the rest of the row is padding.
 *   docs_per_row[batch]          number of documents in each row (>= 0).
 *   batch >= 0, seq_len >= 0, 0 <= row_offset, 0 <= q_len,
 *   row_offset + q_len <= seq_len.
 *   capacity                     entries available in the output arrays
 *                                (cu arrays must hold capacity + 1).
 * Outputs (host), one segment per (row, document meeting the chunk), in row
 * then position order, plus one padding segment per row whose padding tail
 * reaches into the chunk:
 *   cu_seqlens_q[n+1]  local query rows of segment s are
 *                      [cu_seqlens_q[s], cu_seqlens_q[s+1]) of the flattened
 *                      [batch * q_len] rows; 0 .. batch*q_len, increasing.
 *   cu_seqlens_k[n+1]  prefix sums of segment key counts (non-decreasing; a
 *                      padding segment adds 0).
 *   seg_k_begin[n]     flattened key index (b * seq_len + position) of the
 *                      segment's first key; for a padding segment, the
 *                      position of its first row.
 *   *n_seg, *max_seqlen_q, *max_seqlen_k.
 * Row t of segment s (0-based) attends keys seg_k_begin[s] + 0 ..
 * seg_k_begin[s] + t + (k_len - q_len) inclusive (bottom-right alignment).
 * Errors: BD_ERR_INVALID_ARG (null pointer, bad sizes), BD_ERR_BAD_METADATA
 * (negative length, row sum > seq_len), BD_ERR_CAPACITY (*n_seg is set to the
 * number of segments needed; nothing else is written).  The table is checked
 * with blockdiag_validate before returning.
 */
bd_status blockdiag_segment(const int32_t *doc_lens, const int32_t *docs_per_row,
                            int32_t batch, int32_t seq_len, int32_t row_offset,
                            int32_t q_len, int32_t capacity, int32_t *cu_seqlens_q,
                            int32_t *cu_seqlens_k, int32_t *seg_k_begin, int32_t *n_seg,
                            int32_t *max_seqlen_q, int32_t *max_seqlen_k);

/*
 * blockdiag_validate -- host check of a segment table built anywhere (Design
 * overview, kernels.py, and key property 4: every offset a kernel consumes is
 * validated on the host, since a bad terminal offset would otherwise be an
 * asynchronous illegal memory access).  Host pointers.  Checks: cu_q[0] = 0,
 * strictly increasing, cu_q[n] = batch * q_len; cu_k[0] = 0, non-decreasing;
 * each segment's rows lie in one batch row; a non-padding segment's keys lie
 * in the same batch row, number at least its rows, and end exactly one past
 * the global position of its last row; padding segments have no keys and
 * only follow the row's last document; segments of a row are contiguous and
 * in order.  Returns BD_OK or BD_ERR_BAD_METADATA with a message.
 */
bd_status blockdiag_validate(const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                             const int32_t *seg_k_begin, int32_t n_seg, int32_t batch,
                             int32_t seq_len, int32_t row_offset, int32_t q_len);

/*
 * blockdiag_kv_plan -- needed-only K/V exchange plan of one context-parallel
 * rank (host only, integer only).  Summary: instead of all-gathering the
 * whole row's K/V, a rank can receive only the keys its rows attend -- from
 * its left neighbour (halo p2p), or with an all-to-all-v when a document
 * spans more than two ranks -- which cuts its K/V from the whole row to its
 * own chunk plus the straddling prefix; Design overview, batch.py (rows
 * padded to a multiple of cp, contiguous slice per rank) and exchange.py;
 * Proof: the plan geometry is checked on the CPU.
 *
 * Rank r of cp holds rows [r * S/cp, (r + 1) * S/cp) of every batch row
 * (seq_len must be a multiple of cp).  Its rows of batch row b attend the
 * keys [doc_start(r0), min(r1, end of the row's documents)) -- empty when
 * r0 is padding -- and the part left of r0 is the halo, owned by lower
 * ranks.
 * Inputs (host): doc_lens / docs_per_row / batch / seq_len as for
 *   blockdiag_segment; cp >= 1; 0 <= rank < cp; align >= 1.
 * Outputs (host):
 *   *kv_begin, *kv_end  the rank's K/V window [kv_begin, kv_end) for
 *       blockdiag_attn_fwd / _bwd: kv_end = r1, kv_begin = the smallest key
 *       any of its rows attends (at most r0), rounded down to a multiple of
 *       align (64 for the attention calls).  Keys of the window that are not
 *       in a row's receive ranges or own chunk are never attended by that
 *       row; the caller zero-fills them.
 *   recv[*n_recv]  ranges (row, peer, begin, end): keys [begin, end) of batch
 *       row `row` that this rank receives from rank `peer` (exactly the halo,
 *       split by owning rank, rows in order, lower ranks first).
 *   send[*n_send]  ranges this rank sends: keys [begin, end) of its own chunk
 *       that rank `peer` > rank attends (rows in order, peers ascending).
 *   *rank_mode  0: no halo; 1: every received key comes from rank - 1 (halo
 *       p2p); 2: some come from a rank further left (all-to-all-v).
 *   *step_mode  the largest rank_mode over all ranks: the exchange every
 *       rank of the step runs (0 none, 1 halo, 2 all-to-all-v), so no rank
 *       takes a different collective.
 * Errors: BD_ERR_INVALID_ARG, BD_ERR_BAD_METADATA (negative length, row sum
 * > seq_len), BD_ERR_CAPACITY (*n_recv / *n_send hold the counts needed;
 * the range arrays may then be partly written).
 */
typedef struct bd_kv_range {
  int32_t row;    /* batch row                     */
  int32_t peer;   /* the other rank                */
  int32_t begin;  /* first key position (in row)   */
  int32_t end;    /* one past the last             */
} bd_kv_range;
bd_status blockdiag_kv_plan(const int32_t *doc_lens, const int32_t *docs_per_row, int32_t batch,
                            int32_t seq_len, int32_t cp, int32_t rank, int32_t align,
                            int32_t *kv_begin, int32_t *kv_end, int32_t capacity,
                            bd_kv_range *recv, int32_t *n_recv, bd_kv_range *send,
                            int32_t *n_send, int32_t *rank_mode, int32_t *step_mode);

/*
 * bd_meta -- host descriptor of a device metadata buffer.  It records the
 * sizes the buffer was built for, so the attention calls can check in O(1)
 * on the host that the metadata matches their own sizes before anything is
 * launched (key property 4: no offset a kernel consumes goes unchecked; the
 * kernels index the metadata with the call's batch, seq_len and q_len).
 * Filled only by blockdiag_meta_build / blockdiag_meta_build_host; a caller
 * treats it as opaque.  It stays valid while the buffer holds what that
 * build wrote (a later build into the same buffer needs its own
 * descriptor).  The descriptor holds the device pointer but owns nothing.
 */
#define BD_META_MAGIC 0x54454d42u /* "BMET" */
typedef struct bd_meta {
  uint32_t magic;       /* BD_META_MAGIC after a successful build, else 0  */
  int32_t batch;        /* sizes of the chunk the buffer describes         */
  int32_t seq_len;
  int32_t row_offset;
  int32_t q_len;
  int32_t n_seg;        /* segments of the table it was built from         */
  int32_t kv_lo;        /* keys the chunk attends, over all batch rows:    */
  int32_t kv_hi;        /*   [kv_lo, kv_hi) (kv_lo = 0 when unknown)       */
  int32_t max_seg_k;    /* most keys of one segment (-1 when unknown)      */
  uint64_t n_ints;      /* int32 entries written: blockdiag_meta_ints(...) */
  const int32_t *data;  /* the device buffer (caller-owned)                */
} bd_meta;

/*
 * blockdiag_meta_ints -- number of int32 in the device metadata buffer that
 * blockdiag_meta_build fills: 2 * batch * q_len + 2 * batch * seq_len,
 * plus nq + 2 with nq = batch * ceil(q_len / 32) when 1 <= nq <= 8192,
 * plus 1 + 3 * nb with nb = batch * (2 * ceil((q_len + 127) / 128) + 1)
 * when batch * q_len > 0.
 *
 * blockdiag_meta_build -- expands a validated segment table (device copy)
 * into per-row and per-key mask bounds on the device, once per step, so the
 * attention kernels find each tile's live key range, each key tile's live
 * query range and every element's mask with plain loads (skipping fully
 * masked tiles, Summary: per-step precompute, zero per-layer host syncs).
 *   d_table   device int32 [3 * n_seg + 2] = cu_seqlens_q[n_seg+1] ++
 *             cu_seqlens_k[n_seg+1] ++ seg_k_begin[n_seg], as produced by
 *             blockdiag_segment and accepted by blockdiag_validate.
 *   d_meta    device int32 [meta_capacity] with meta_capacity >=
 *             blockdiag_meta_ints(...), written as
 *             row_lo[batch][q_len], row_hi[batch][q_len]: local row t of
 *               batch row b attends key positions row_lo <= j < row_hi
 *               (row_lo = row_hi = 0 on padding rows);
 *             key_qlo[batch][seq_len], key_qhi[batch][seq_len]: key position
 *               j of row b is attended by local rows key_qlo <= t < key_qhi
 *               (both 0 when no local row attends it);
 *             q_order[batch * ceil(q_len / 32)]: a launch order of the
 *               32-row query tiles, a permutation of the codes b * n_qt + qt
 *               sorted by the number of 32-key tiles each visits, most first
 *               (ties in ascending code order); then q_stats[2]: the largest
 *               and the total visit count (saturated at 2^31 - 1).  Present
 *               for at most 8192 query tiles over the batch; the order is
 *               written for tables of at most 2047 segments (larger ones get
 *               statistics {0, 2^31 - 1}, which no kernel follows).  The
 *               forward and dQ kernels launch their tiles in this order when
 *               the largest visit count is at least half of one workgroup
 *               slot's share of the total (then the launch order sets the
 *               tail), otherwise last tiles first; results do not depend on
 *               the order.  Absent (no entries) for more than 8192 tiles.
 *             bins[1 + 3 * nb]: the short-document bins.  bins[0] is their
 *               count, then per bin the first and one-past-last local row
 *               (flattened [batch * q_len] index) and the flattened key
 *               index (b * seq_len + position) of its first key; its keys
 *               end one past its last row's position.  Consecutive
 *               documents of one batch row are grouped greedily in table
 *               order while the group's keys span at most 128 positions; a
 *               padding segment or a new batch row starts a new bin.  Built
 *               only when no segment has more than 128 keys (else the count
 *               is 0); every row of a document and every key it attends then
 *               lies in exactly one bin.
 *   desc      (host, required) receives the buffer's descriptor for the
 *             attention calls; on any error its magic is set to 0.
 *   h_table   (host, optional) the same table in host memory: the
 *             descriptor then records the key window the chunk attends
 *             (kv_lo, kv_hi), which a window-only K/V call is checked
 *             against, and the most keys of one segment (max_seg_k), by
 *             which the backward picks its short-document kernel.  NULL
 *             records kv_lo = 0, kv_hi = row_offset + q_len (so only K/V
 *             windows starting at key 0 are accepted) and max_seg_k = -1.
 * The table is not re-validated here (that needs a sync); the kernel clamps
 * every bound to its row so a corrupt table cannot make later kernels read
 * out of bounds.  Errors: BD_ERR_INVALID_ARG, BD_ERR_CAPACITY (meta_capacity
 * too small; nothing is launched), BD_ERR_HIP.
 */
size_t blockdiag_meta_ints(int32_t batch, int32_t seq_len, int32_t q_len);
bd_status blockdiag_meta_build(const int32_t *d_table, const int32_t *h_table, int32_t n_seg,
                               int32_t batch, int32_t seq_len, int32_t row_offset, int32_t q_len,
                               int32_t *d_meta, size_t meta_capacity, bd_meta *desc,
                               void *stream);

/*
 * blockdiag_meta_build_host -- blockdiag_meta_build for a table in host
 * memory (h_table, same layout as d_table) of at most
 * blockdiag_meta_inline_max_seg() segments: the table is read on the host
 * during the call and travels to the kernel in its launch arguments, so the
 * step needs no host-to-device copy of it (Summary: per-step precompute,
 * zero per-layer host syncs).  h_table is not retained after the call
 * returns.  d_meta, meta_capacity, desc (with the key window recorded), the
 * output and the stream ordering are as for blockdiag_meta_build.  Errors: BD_ERR_CAPACITY when n_seg
 * exceeds the limit (use blockdiag_meta_build) or meta_capacity is too
 * small (nothing is launched), BD_ERR_INVALID_ARG, BD_ERR_BAD_METADATA,
 * BD_ERR_HIP.
 */
int32_t blockdiag_meta_inline_max_seg(void);
bd_status blockdiag_meta_build_host(const int32_t *h_table, int32_t n_seg, int32_t batch,
                                    int32_t seq_len, int32_t row_offset, int32_t q_len,
                                    int32_t *d_meta, size_t meta_capacity, bd_meta *desc,
                                    void *stream);

/*
 * bd_dropout -- attention dropout of the attention calls (Proof section: the
 * varlen path forwards a dropout probability and the native kernel applies
 * it).  The pages fix no random-number contract; this one is stated so a
 * caller (or a reference) can reproduce every mask: the weights that
 * multiply V are P_ij * Z_ij * c, with Z from Philox4x32-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).  The pair (query
 * position i, key position j) -- positions in the packed row, so masks do
 * not depend on chunking or on the K/V window -- of batch row b and query
 * head h draws counter (j / 4, i / 4, b * h_q + h, offset) under key
 * (seed mod 2^32, seed / 2^32); byte j % 4 (least significant first) of
 * output word i % 4 is kept iff it is >= thr = min(255, round(256 p)), and
 * kept weights are scaled by c = 256 / (256 - thr) (so the drop rate is
 * thr / 256).  LSE is that of the undropped softmax.  The backward must get
 * the forward's p, seed and offset.  A NULL pointer or p = 0 is no dropout.
 */
typedef struct bd_dropout {
  float p;          /* drop probability, 0 <= p < 1                  */
  uint32_t offset;  /* counter word 3: e.g. layer and step           */
  uint64_t seed;    /* generator key                                 */
} bd_dropout;

/*
 * blockdiag_workspace_bytes -- device scratch the forward (is_bwd = 0) or
 * backward (is_bwd = 1) needs for these sizes (0 is a valid answer).
 */
size_t blockdiag_workspace_bytes(int is_bwd, bd_dtype dtype, int32_t batch, int32_t seq_len,
                                 int32_t q_len, int32_t h_q, int32_t h_kv, int32_t head_dim);

/*
 * blockdiag_attn_fwd -- O and LSE of the chunk (Summary: the varlen kernel;
 * Design overview, runtime.py: drop-in SDPA; packed.py: row_offset = 0).
 *   kv_begin, kv_len: the K/V window held by k and v (whole row: 0 and
 *   seq_len).  kv_begin must be a multiple of 64, at most the first key the
 *   chunk attends (the descriptor's kv_lo) and at most row_offset; the
 *   window must reach the chunk's end: row_offset + q_len <= kv_begin +
 *   kv_len <= seq_len.  Keys of the window that a row does not attend are
 *   read but weighted by exactly zero; they must hold finite values (the
 *   exchange plan's callers zero-fill them).  Results do not depend on the
 *   window: O, LSE and dQ are bitwise those of the whole-row call, dK / dV
 *   bitwise its rows of the window.
 *   q, k, v (device, dtype) as in the conventions above; meta (host) the
 *   descriptor blockdiag_meta_build wrote for the same batch, seq_len,
 *   row_offset and q_len (a descriptor built for other sizes, or not built,
 *   is rejected with BD_ERR_INVALID_ARG before any launch); o (device,
 *   dtype) and lse (device, float32) are written in full.
 *   scale multiplies q.k (1/sqrt(head_dim) is the usual choice); dropout
 *   (host, may be NULL) as described at bd_dropout.
 *   Supported: any head_dim up to 256 that is a multiple of 8, float32 or
 *   bf16, h_q % h_kv = 0.  bf16 with h_q / h_kv a multiple of 4 runs on the
 *   matrix-core kernels for head_dim 64, 128 and 256 when
 *   one batch row of K (or V), in bytes, stays below 2^31 with one tile of
 *   slack: (kv_len + 32) * h_kv * head_dim * 2 for the forward; the
 *   backward needs (kv_len + 64) * h_kv * head_dim * 2 and
 *   (q_len + 32) * h_q * head_dim * 2 below 2^31.  Everything else runs on
 *   the generic kernels (64-bit indexing, float32 arithmetic).
 *   bf16 inputs are multiplied on matrix cores with float32 accumulation; the
 *   outputs are rounded to nearest even.  The forward is bitwise
 *   deterministic (no atomics), so a replayed forward equals the original.
 * q_len = 0 or batch = 0 is a no-op returning BD_OK.
 * Errors: BD_ERR_INVALID_ARG, BD_ERR_UNSUPPORTED, BD_ERR_WORKSPACE, BD_ERR_HIP.
 */
bd_status blockdiag_attn_fwd(bd_dtype dtype, int32_t batch, int32_t seq_len, int32_t row_offset,
                             int32_t q_len, int32_t kv_begin, int32_t kv_len, int32_t h_q,
                             int32_t h_kv, int32_t head_dim,
                             float scale, const bd_dropout *dropout, const void *q, const void *k,
                             const void *v,
                             const bd_meta *meta, void *o, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * blockdiag_attn_bwd -- dQ, dK, dV of the loss sum(dO * O) for the chunk
 * (Proof section: forward/backward parity and input gradients).  LSE has no
 * incoming gradient.  o and lse are the forward's outputs; d_o like o;
 * meta as for blockdiag_attn_fwd (not read, and may be NULL, when q_len or
 * batch is 0).
 *   dq (device, like q) is written in full; dk, dv (device, like k: the
 *   window [kv_begin, kv_begin + kv_len) of every row) are written for every
 *   key of the window -- the chunk's partial gradients, zero at keys no local
 *   row attends, so summing them over the chunks of a row gives the full
 *   gradient (Design overview, exchange.py: the K/V gradient is
 *   reduce-scattered with SUM, or index-added back for needed-only K/V).
 *   workspace: at least blockdiag_workspace_bytes(1, ...) bytes of device
 *   memory (float32 row statistics: lse * log2(e) and delta = rowsum(dO * O)
 *   per row and query head, 8 bytes each).
 * The backward is bitwise deterministic (no atomics): each of dQ, dK, dV is
 * written once by the workgroup that owns its rows or keys.
 * Errors: as blockdiag_attn_fwd.
 */
bd_status blockdiag_attn_bwd(bd_dtype dtype, int32_t batch, int32_t seq_len, int32_t row_offset,
                             int32_t q_len, int32_t kv_begin, int32_t kv_len, int32_t h_q,
                             int32_t h_kv, int32_t head_dim,
                             float scale, const bd_dropout *dropout, const void *q, const void *k,
                             const void *v,
                             const void *o, const float *lse, const void *d_o,
                             const bd_meta *meta, void *dq, void *dk, void *dv,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * blockdiag_attn_bwd_noalloc -- blockdiag_attn_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, which is replaced by a static device array of
 * blockdiag_noalloc_scratch_bytes() bytes (16 MiB) that the library holds on
 * every GPU it runs on until the process ends.  The array holds the float32
 * row statistics (8 bytes per local row and query head), so
 * batch * q_len * h_q may be at most 2^21; larger calls return
 * BD_ERR_WORKSPACE before anything is launched.  The call allocates
 * nothing; its first call on a device looks up that device's copy of the
 * array (the caller's current device).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, threads)
 * race and give wrong results; calls ordered on one stream are safe.
 * Results are those of blockdiag_attn_bwd, bit for bit.
 */
size_t blockdiag_noalloc_scratch_bytes(void);
bd_status blockdiag_attn_bwd_noalloc(bd_dtype dtype, int32_t batch, int32_t seq_len,
                                     int32_t row_offset, int32_t q_len, int32_t kv_begin,
                                     int32_t kv_len, int32_t h_q, int32_t h_kv,
                                     int32_t head_dim, float scale, const bd_dropout *dropout,
                                     const void *q, const void *k,
                                     const void *v, const void *o, const float *lse,
                                     const void *d_o, const bd_meta *meta, void *dq, void *dk,
                                     void *dv, void *stream);

/*
 * blockdiag_mark_main_kernel -- profiling hook.  The next blockdiag_attn_fwd
 * or blockdiag_attn_bwd call made on this thread records start_event on its
 * stream right before launching its main attention kernel and stop_event
 * right after it (the backward's main kernel is its dK/dV kernel; the dQ
 * and row-statistics kernels before it fall outside the pair), then forgets
 * both.  The events are hipEvent_t
 * handles passed as void*, created and owned by the caller; NULL, NULL
 * clears a pending request.  Lets a caller time the dominant kernel with
 * events on the stream it runs on.  Returns BD_OK, or BD_ERR_INVALID_ARG
 * if exactly one handle is NULL.
 */
bd_status blockdiag_mark_main_kernel(void *start_event, void *stop_event);

/*
 * blockdiag_clock_probe -- measurement aid (not an attention operation):
 * the engine clock the GPU runs at, for pricing a measured rate against
 * peaks quoted at 2.4 GHz.  Launches n_workgroups single-wave workgroups on
 * stream; each spins for `ticks` counts of the constant 100 MHz real-time
 * counter and writes two uint64 to d_out[2 * w], d_out[2 * w + 1]: the
 * shader-clock cycles (one per engine clock) and the real-time ticks that
 * elapsed.  cycles / ticks * 100 is the clock in MHz of the CU that ran
 * workgroup w.  d_out is device memory of 2 * n_workgroups uint64, owned
 * by the caller and written asynchronously.  Errors: BD_ERR_INVALID_ARG
 * (n_workgroups outside 1..65536, ticks outside 1..10^7, NULL d_out),
 * BD_ERR_HIP.
 */
bd_status blockdiag_clock_probe(int32_t n_workgroups, uint32_t ticks, uint64_t *d_out, void *stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char *blockdiag_last_error(void);

/* Library version string. */
const char *blockdiag_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKDIAG_H */
