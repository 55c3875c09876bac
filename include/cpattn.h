/*
 * cpattn -- one device's share of context-parallel Pass-KV ring attention on
 * AMD MI355X (gfx950).  C ABI of libcpattn.so.
 *
 * The method (sources are the two pages named below; the LSE/merge formulas
 * and the backward are the plain definition of softmax attention and its
 * exact gradient, which the pages leave implicit):
 *   - "Context Parallelism for Scalable Million-Token Inference" (MLSys 2025
 *     talk summary): sections "Load Balancing in CP" (2R-chunk sharding),
 *     "Ring Attention Algorithms" (Pass KV, merge of partial outputs) and
 *     "Attention Compute Patterns in Multi-Turn Chat" (causal full prefill).
 *   - "Announcing Long-Context Training on TPUs with MaxText Context
 *     Parallelism": section "Context Parallelism in MaxText" (P2P ring,
 *     Figure 3) and "Built on a fast attention kernel" (one kernel call per
 *     ring step, forward and backward; fully masked blocks skipped; packed
 *     sequences without padding).
 *
 * Conventions shared by every call:
 *   - Tensors are caller-owned.  "device" pointers are HIP device memory,
 *     "host" pointers are ordinary CPU memory.  The library keeps no pointer
 *     after a call returns and allocates no device memory.
 *   - Layouts (row = token of the local tensor, contiguous, no padding):
 *       Q, dO, O, dQ      [rows, Hq,  D]   (bf16 inputs, fp32 outputs)
 *       K, V, dK, dV      [rows, Hkv, D]
 *       LSE, Delta        [Hq, rows]       fp32, natural log
 *     Query head h reads key/value head h / (Hq / Hkv).
 *   - bf16 is IEEE bfloat16 (uint16 bit pattern in memory).
 *   - Device calls are asynchronous on the given stream (NULL = the default
 *     stream) and never synchronise.  They validate every argument first and
 *     launch nothing when they return an error.
 *   - Supported: D in {64, 128}; Hq % Hkv == 0; positions and rows < 2^31.
 *   - Thread-safe; no global state beyond the last-error string, which is
 *     thread-local.  (The diagnostics call in cpattn_diag.h is the one
 *     exception: a process-wide recording switch, off unless set.)
 *   - Calls marked "Helper" are not steps of the method: the pages define no
 *     such operation; they expose the library's own tiling and work split so
 *     that callers and tests can size buffers and check the kernels' choices.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_ABI_VERSION 5

typedef enum cp_status {
    CP_OK = 0,
    CP_ERR_INVALID_ARG = -1, /* bad pointer, size, layout or enum value */
    CP_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 96) */
    CP_ERR_HIP = -3          /* a HIP runtime call failed (launch error) */
} cp_status;

/* Class of one (query chunk, key chunk) pair of a ring step. */
typedef enum cp_mask {
    CP_MASK_FULL = 0,        /* every key visible to every query: no element mask */
    CP_MASK_DIAG_CAUSAL = 1, /* key visible iff key position <= query position
                                (and inside the sliding window, if any) */
    CP_MASK_DOC = 2,         /* DIAG_CAUSAL and inside the same packed document */
    CP_MASK_SKIP = 3         /* nothing visible: the pair is not computed */
} cp_mask;

/* Block-map tile classes (cp_block_map, tile_map_out). */
#define CP_TILE_SKIP 0
#define CP_TILE_PARTIAL 1
#define CP_TILE_FULL 2

/* A contiguous run of rows of a local tensor that holds consecutive global
 * sequence positions (one zigzag chunk, or part of one). */
typedef struct cp_segment {
    int64_t row0; /* first row of the run in the local tensor */
    int64_t pos0; /* global sequence position of that row */
    int64_t len;  /* number of rows (0 allowed) */
} cp_segment;

/* One ring step's problem: the local queries against the KV block held now.
 * At most two query segments (the rank's two zigzag chunks) and two KV
 * segments (the source rank's two chunks).  Query segments must not share
 * rows.  mask[i][j] is the class of (query segment i, KV segment j); the
 * kernels trust FULL and SKIP and apply element masks only on partially
 * visible tiles of DIAG_CAUSAL and DOC pairs.  Positions are read only for
 * DIAG_CAUSAL and DOC pairs: a segment whose pairs are all FULL or SKIP may
 * hold rows from several position ranges (its pos0 is then not used).
 *
 * Sliding window ("Announcing Long-Context Training ...", closing section:
 * models such as Gemma mix sliding-window layers with global ones): with
 * window = W > 0, a DIAG_CAUSAL or DOC pair sees key k from query q only if
 * q - W < k <= q (the W most recent positions, q itself included).  A pair
 * the window cuts must not be marked FULL: cp_step_masks_window classifies
 * ring steps accordingly.  window = 0: no window. */
typedef struct cp_attn_problem {
    int32_t hq, hkv, head_dim;/* hq <= 8192, a multiple of hkv; head_dim 64 or 128 */
    float scale;              /* softmax scale, normally 1/sqrt(head_dim) */
    int64_t q_rows;           /* rows of the local query tensor */
    int64_t kv_rows;          /* rows of the KV block tensor */
    int32_t n_q_seg, n_kv_seg;/* 1 or 2 each */
    cp_segment q_seg[2];
    cp_segment kv_seg[2];
    int32_t mask[2][2];       /* cp_mask values */
    /* Packed documents (any mask == CP_MASK_DOC): document start offsets,
     * int32 [n_docs + 1], non-decreasing, cu_seqlens[0] == 0, last entry
     * >= every position used.  A DEVICE pointer for the step calls, a HOST
     * pointer for cp_block_map and cp_count_pairs. */
    const int32_t* cu_seqlens;
    int32_t n_docs;
    int32_t window;           /* sliding window in tokens, 0 = none (>= 0) */
    /* Backward only: the number of workgroups (1..8) over which the dK/dV
     * kernel spreads each 128-key block's query tiles; 0 = chosen by the
     * library from the positions (1 when a mask is DOC, whose ranges need the
     * documents on the host: see cp_bwd_kv_split).  Above 1, the first part
     * of a block writes dK/dV and each later part with tiles writes its
     * partial sums to the caller's workspace (cp_bwd_workspace_size); a second
     * pass adds them to dK/dV in part order.  No atomics: results are the same
     * bits on every run.  The forward calls ignore it. */
    int32_t kv_split;
} cp_attn_problem;

/* ---------------------------------------------------------------- host ---- */

int32_t cp_abi_version(void);
const char* cp_status_string(cp_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* cp_last_error(void);

/* Load-balanced partition ("Context Parallelism for Scalable Million-Token
 * Inference", section "Load Balancing in CP"): the sequence is cut into
 * 2*cp_size chunks of c = seq_len / (2*cp_size) tokens; rank r holds chunks
 * r and 2*cp_size-1-r.  Writes the global positions of rank r's local tokens,
 * in local order [chunk r ; chunk 2R-1-r], to pos_out (host, int64
 * [seq_len / cp_size]).  INVALID_ARG if seq_len is not a positive multiple of
 * 2*cp_size, rank is out of range or pos_out is NULL. */
cp_status cp_partition_zigzag(int64_t seq_len, int32_t cp_size, int32_t rank, int64_t* pos_out);

/* Ring order of Pass KV ("... Million-Token Inference", section "Ring
 * Attention Algorithms"): KV blocks move from rank r to rank r+1 each step,
 * so at step t rank r holds the block of rank (r - t) mod cp_size. */
cp_status cp_ring_source(int32_t cp_size, int32_t rank, int32_t step, int32_t* src_out);

/* Chunk-pair classes of step t for rank r: mask_out[2*i + j] is the class of
 * (query chunk i of rank r, key chunk j of the source rank), chunks in local
 * order.  Causal: chunk index of the key below / equal to / above that of the
 * query gives FULL / DIAG_CAUSAL / SKIP.  packed != 0: every non-SKIP pair is
 * DOC (document boundaries may fall anywhere). */
cp_status cp_step_masks(int32_t cp_size, int32_t rank, int32_t step, int32_t packed, int32_t mask_out[4]);

/* Chunk-pair classes of step t for rank r in a layer with a sliding window of
 * `window` tokens (0 = none, which gives cp_step_masks), for a sequence of
 * seq_len tokens (chunks of c = seq_len / (2*cp_size)).  A pair (query chunk
 * I, key chunk J) is SKIP when J > I or when its closest pair is at least
 * `window` positions apart ((I-J-1)*c + 1 >= window), FULL when J < I and
 * its farthest pair is inside the window ((I-J+1)*c - 1 < window, or no
 * window), DIAG_CAUSAL otherwise; packed != 0 turns every non-SKIP class into
 * DOC.  With window <= c only the rank's own block and its ring neighbours'
 * (steps 0, 1 and cp_size-1) have any visible pair: the short exchange between
 * neighbouring chips the pages describe for window layers.
 * INVALID_ARG as cp_step_masks, or for seq_len not a positive multiple of
 * 2*cp_size or window < 0. */
cp_status cp_step_masks_window(int64_t seq_len, int32_t cp_size, int32_t rank, int32_t step, int32_t packed,
                               int64_t window, int32_t mask_out[4]);

/* Helper.  Tile shape of the forward kernel for this head configuration: bm
 * query rows x bn keys (bm depends on the head counts, which decide how many
 * heads of a GQA group share a workgroup).  The block map and tile_map_out use
 * this shape.  UNSUPPORTED for head_dim not in {64, 128}. */
cp_status cp_tile_shape(int32_t hq, int32_t hkv, int32_t head_dim, int32_t* bm_out, int32_t* bn_out);

/* Helper.  Size of a step's block map: query tiles (over both query segments,
 * each segment tiled from its first row, last tile possibly short) and key
 * tiles. */
cp_status cp_block_map_size(const cp_attn_problem* p, int64_t* n_q_tiles, int64_t* n_k_tiles);

/* Host computation of the block map the forward kernel follows: map_out (host,
 * uint8 [n_q_tiles, n_k_tiles]) gets SKIP for tiles with no visible pair,
 * FULL for tiles with every pair visible and PARTIAL otherwise ("Announcing
 * Long-Context Training ...", section "Built on a fast attention kernel":
 * fully masked blocks are skipped).  cu_seqlens is a host pointer here. */
cp_status cp_block_map(const cp_attn_problem* p, uint8_t* map_out);

/* Helper.  Number of visible (query, key) pairs of the step, per query head
 * (host; cu_seqlens is a host pointer here): the step's causal-counted work,
 * and zero for a block that none of the local queries can see (a ring need not
 * receive or compute it). */
cp_status cp_count_pairs(const cp_attn_problem* p, int64_t* pairs_out);

/* -------------------------------------------------------------- device ---- */

/* Device calls: every tensor pointer is a device address, 16-byte aligned (the
 * kernels move 16-byte vectors; a torch allocation, or a view of it starting
 * at a row, qualifies).  A misaligned or NULL tensor gives INVALID_ARG before
 * anything is launched.  Launches are asynchronous on `stream`. */

/* Forward of one ring step: blockwise flash attention of the local queries
 * against the KV block held at this step ("Announcing Long-Context Training
 * ...", section "Built on a fast attention kernel": the kernel runs once per
 * ring step on the local queries and the block just received).
 *   q       device bf16 [q_rows, Hq, D]
 *   k, v    device bf16 [kv_rows, Hkv, D]
 *   o_step  device fp32 [q_rows, Hq, D]   out: softmax-normalised partial output
 *   lse_step device fp32 [Hq, q_rows]     out: ln sum_j exp(scale q.k_j)
 * Rows inside a query segment with no visible key get O = 0, LSE = -inf (the
 * identity of cp_merge_partials).  Rows outside every query segment are not
 * written.  tile_map_out (optional device uint8 [n_q_tiles, n_k_tiles], see
 * cp_block_map_size) receives the tile classes the kernel itself used.
 * Softmax scores use bf16 MFMA products with fp32 accumulation; P is rounded
 * to bf16 before the PV product. */
cp_status cp_attn_fwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                           float* o_step, float* lse_step, uint8_t* tile_map_out, hipStream_t stream);

/* Merge of partial outputs over disjoint key sets ("... Million-Token
 * Inference", section "Ring Attention Algorithms": the partial attention
 * outputs of all steps are merged into the full output).  In place on the
 * accumulator: L = ln(e^La + e^Lb); O_acc = e^(La-L) O_acc + e^(Lb-L) O_step;
 * LSE_acc = L.  Both -inf gives (0, -inf).  Start from (0, -inf).
 *   o_acc, o_step     device fp32 [rows, heads, head_dim]
 *   lse_acc, lse_step device fp32 [heads, rows] */
cp_status cp_merge_partials(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                            int64_t rows, int32_t heads, int32_t head_dim, hipStream_t stream);

/* Merge of n_parts (1..64) partial outputs of the same rows over disjoint key
 * sets, each read once: what an owner does with the partials Pass Q's
 * all-to-all delivers to it ("... Million-Token Inference", section "Ring
 * Attention Algorithms": with Pass Q the partial outputs are sent to the
 * ranks that own the queries, which merge them).  L = ln sum_i e^(L_i);
 * O = sum_i e^(L_i - L) O_i; all -inf gives (0, -inf).  o_parts / lse_parts
 * are HOST arrays of n_parts device pointers, each part laid out as in
 * cp_merge_partials.  o_out / lse_out may be the first part's buffers (in
 * place), but no other part's.
 *   o_out    device fp32 [rows, heads, head_dim]   out
 *   lse_out  device fp32 [heads, rows]             out
 * INVALID_ARG on n_parts outside [1, 64] or a NULL or misaligned pointer. */
cp_status cp_merge_partials_n(float* o_out, float* lse_out, const float* const* o_parts,
                              const float* const* lse_parts, int32_t n_parts, int64_t rows, int32_t heads,
                              int32_t head_dim, hipStream_t stream);

/* Forward of one ring step fused with the merge of its partial output into the
 * running accumulator ("... Million-Token Inference", section "Ring Attention
 * Algorithms": the partial outputs are merged as the KV blocks circulate).
 * Same problem, inputs, tiles and masks as cp_attn_fwd_step; the result equals
 * cp_attn_fwd_step into temporaries followed by cp_merge_partials, up to the
 * order of rounding.
 *   o_acc   device fp32 [q_rows, Hq, D]   in/out: merged output so far
 *   lse_acc device fp32 [Hq, q_rows]      in/out: merged LSE so far
 * The accumulator must hold a valid state: (0, -inf), the output of an earlier
 * cp_attn_fwd_step, or an earlier merge.  Rows with no visible key in this step
 * are neither read nor written; nor are rows outside every query segment.
 * tile_map_out as for cp_attn_fwd_step. */
cp_status cp_attn_fwd_step_merge(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                 float* o_acc, float* lse_acc, uint8_t* tile_map_out, hipStream_t stream);

/* Backward preprocessing: delta[h, i] = sum_d dO[i, h, d] * O[i, h, d] with
 * the final merged O.  The pages give no backward formulas: this is the row
 * term of the exact softmax gradient (dS = P (dP - delta)) that the per-step
 * backward below needs, computed once per row from the merged output.
 * d_o device bf16 [rows, heads, D]; o device fp32 [rows, heads, D]; delta
 * device fp32 [heads, rows] (overwritten).  INVALID_ARG on a NULL or
 * misaligned pointer or a bad size. */
cp_status cp_attn_bwd_prep(const void* d_o, const float* o, float* delta, int64_t rows, int32_t heads,
                           int32_t head_dim, hipStream_t stream);

/* Helper.  Split of the dK/dV work that cp_attn_bwd_step would choose for
 * kv_split = 0, computed here with HOST cu_seqlens, so DOC problems can be
 * balanced too: a key block that many more query tiles see than an even share
 * of the GPU's dK/dV slots (2 per CU, n_cu CUs) is spread over up to 8
 * workgroups.  Such blocks occur where visibility is a band or a triangle
 * (sliding windows, the edge of a document).  Writes 1..8 to split_out.
 * INVALID_ARG on a bad problem, n_cu < 1 or a NULL split_out. */
cp_status cp_bwd_kv_split(const cp_attn_problem* p, int32_t n_cu, int32_t* split_out);

/* Helper.  Workspace bytes cp_attn_bwd_step needs for the dK/dV split kv_split
 * (1..8) of problem p: (kv_split - 1) slots of 2 x 128 x head_dim floats per
 * 128-key block of every KV head; 0 for kv_split = 1.  INVALID_ARG on a bad
 * problem, a kv_split outside [1, 8] or a NULL bytes_out. */
cp_status cp_bwd_workspace_size(const cp_attn_problem* p, int32_t kv_split, int64_t* bytes_out);

/* Backward of one ring step ("Announcing Long-Context Training ...", section
 * "Built on a fast attention kernel": the ring runs the kernel per step in the
 * backward pass too), from the final LSE and delta of every local row:
 *   P = exp(scale q.k - LSE) on visible pairs; dV_j = sum_i P_ij dO_i;
 *   dS = P (dO.v - delta); dQ_i += scale sum_j dS_ij k_j;
 *   dK_j = scale sum_i dS_ij q_i; dK/dV summed over the heads of a group.
 *   q, d_o   device bf16 [q_rows, Hq, D];  k, v device bf16 [kv_rows, Hkv, D]
 *   lse, delta device fp32 [Hq, q_rows]
 *   dq_acc   device fp32 [q_rows, Hq, D]   ACCUMULATED (+=) across steps
 *   dk_out, dv_out device fp32 [kv_rows, Hkv, D]  OVERWRITTEN: this step's
 *            contribution of the local queries to the visiting block; rows
 *            outside every KV segment are not written.
 *   workspace  device memory of workspace_bytes bytes (16-byte aligned; may be
 *            NULL with 0 bytes), caller-owned, used only by the dK/dV split:
 *            p->kv_split > 1 needs cp_bwd_workspace_size bytes (INVALID_ARG
 *            otherwise); with p->kv_split = 0 the library's choice falls back
 *            to 1 when the workspace is too small.  Its contents need no
 *            initial value and are not meaningful afterwards; calls that share
 *            one workspace must be ordered (e.g. on one stream).
 * dQ, dK and dV are the same bits on every run: nothing is summed in an order
 * that depends on timing. */
cp_status cp_attn_bwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                           const void* d_o, const float* lse, const float* delta, float* dq_acc,
                           float* dk_out, float* dv_out, void* workspace, int64_t workspace_bytes,
                           hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * backward step as cp_attn_bwd_step, with the dK/dV split's workspace taken
 * from a fixed 64 MiB array that the library holds on each device it runs on
 * (for the life of the process) instead of from the caller.  It calls no
 * allocator.  A p->kv_split > 1 whose workspace (cp_bwd_workspace_size)
 * exceeds 64 MiB gives INVALID_ARG; with p->kv_split = 0 the library's choice
 * falls back to 1 when its workspace would not fit.  The array needs no
 * initial value and keeps whatever the last call left; calls that overlap on
 * one GPU (other streams, other threads) share it and race, so order them.
 * Same arguments, layouts, results and errors as cp_attn_bwd_step otherwise
 * (CP_ERR_HIP if the array's device address cannot be looked up). */
cp_status cp_attn_bwd_step_noalloc(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                   const void* d_o, const float* lse, const float* delta, float* dq_acc,
                                   float* dk_out, float* dv_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H */
