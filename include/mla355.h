/*
 * mla355.h -- C ABI of the shared-latent MLA attention forward library for
 * AMD Instinct MI355X (gfx950).  libmla355.so exports exactly the functions
 * declared here.
 *
 * The operation (TT-NN ttnn.transformer.ring_mla, description, "Parameters"
 * and "Returns"; TensorRT-LLM mla.py, MLA.__init__ building the absorbed
 * backend with head_dim = kv_lora_rank + qk_rope_head_dim, num_kv_heads = 1,
 * v_head_dim = kv_lora_rank):
 *
 *   causal flash-style attention of many query heads over one shared KV head.
 *   The score of query row i and key row j is scale * <q_i, kv_j> over the
 *   full KV width (512 latent + 64 RoPE columns); the value is the first
 *   head_dim_v columns of the same KV row.  Every call returns the output and
 *   the per-row natural log-sum-exp of the scaled visible scores (LSE).
 *
 * Around it: a fold of a previous (out, LSE) pair into a new one (Ascend
 * RingMLAOperation, members prevOut / prevLse and calcType), which makes
 * successive KV chunks on one device a ring, and a top-k sparse variant that
 * gathers the selected latent-cache rows (NKI mla_sparse_attention_cte_kernel,
 * "Parameters").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: every data pointer is a DEVICE pointer on the current HIP device.
 *   The library never allocates, frees or synchronises; it only enqueues work
 *   on `stream` (0 = the null stream).  The caller keeps every buffer alive
 *   until that work completes.
 * - Element types: activations and outputs are bfloat16 (passed as uint16_t
 *   bit patterns), LSE values are float32, indices and lengths int32.
 * - Layout: a tensor argument is an mla_rows view: element (b, h, t, d) lives
 *   at data[b*stride_b + h*stride_h + t*stride_t + d], strides in elements,
 *   the innermost (feature) dimension contiguous.  Both the [B, H, N, D]
 *   layout of the TT-NN page and the [tokens, heads, D] layout of the Ascend
 *   page are such views.  Data pointers and the b/h/t strides of bf16 views
 *   must be multiples of 8 elements (16 bytes).  LSE views use the same
 *   struct with d absent (D = 1, any strides).
 * - Empty views: a view that holds no rows (a zero size: B, the query or
 *   token count, or the key/cache row count) may have a NULL data pointer;
 *   nothing is read or written through it.  A call whose output has no rows
 *   enqueues nothing.  With query rows but no key rows (Nkv = 0) every row
 *   sees no key: out = 0 and lse = -inf, or the previous pair unchanged
 *   when one is folded in.
 * - Errors: every function validates all arguments before enqueuing anything.
 *   On failure it enqueues nothing, returns a non-zero mla_status and
 *   mla_last_error() describes the first problem found.  A HIP launch error
 *   is returned as MLA_ERR_HIP.  Nothing aborts or throws across the ABI.
 * - Shapes without a kernel return MLA_ERR_UNSUPPORTED; there is no slow or
 *   host fallback.
 * - Workspace (mla_fwd, mla_sparse_fwd): optional.  When `workspace` is not
 *   NULL it must point to at least mla_workspace_size() bytes of device
 *   memory, 16-byte aligned, given as `workspace_bytes`; its contents need no
 *   initialisation and are left unspecified.  With it, the workgroups of
 *   the shared-latent kernel and of the sparse kernel (K <= 2048) take their
 *   row blocks, longest first, from a counter in the workspace (which the
 *   call resets on `stream` before its launch) rather than by their launch
 *   index, so that the parts of the chip that run faster take more of the
 *   work (TT-NN ring_mla, is_balanced; the queue is this library's reading
 *   of "balanced").  Launches with few row blocks ignore it.  Results are
 *   bit-identical with and without it.  Calls that may run at the same time
 *   need distinct workspaces.
 */
#ifndef MLA355_H
#define MLA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,   /* a shape, stride, alignment or option is invalid */
  MLA_ERR_UNSUPPORTED = 2,   /* valid, but no kernel is built for it */
  MLA_ERR_HIP = 3            /* the HIP runtime reported an error */
} mla_status;

/* A view of bf16 (or fp32 for LSE) rows; see "Layout" above. */
typedef struct {
  void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
} mla_rows;

/* flags for mla_fwd */
#define MLA_CAUSAL 1u        /* key j visible to query i iff kv_offset + j <= q_offset + i */
#define MLA_OUT_F32 2u       /* out holds float32 instead of bf16 */
#define MLA_PREV_OUT_F32 4u  /* prev_out holds float32 instead of bf16 */
#define MLA_VALID_LENS 8u    /* seq_lens holds the valid rows of each batch of padded tensors */
#define MLA_SEQ_LENS_QK 16u  /* seq_lens holds 2 * n_seqs lengths: queries, then keys */

/*
 * mla_fwd -- one attention call (one ring step).
 *
 * Query rows: q [B, Hq, Nq, dq] plus, optionally, q_rope [B, Hq, Nq, dr]; the
 * query vector is their concatenation (dq + dr columns).  Key rows: kv
 * [B, Hkv, Nkv, dq] plus, optionally, k_rope [B, Hkv, Nkv, dr]; same split.
 * Query head h reads KV head h / (Hq / Hkv).  Value rows: v [B, Hkv, Nkv, dv]
 * or, when v is NULL, the first dv columns of the kv rows (the shared-latent
 * form: TT-NN ring_mla, head_dim_v read from the KV prefix).  The split form
 * (q, q_rope, kv, k_rope, v all given) is the Ascend RingMLAOperation step:
 * querySplit1/2, keySplit1/2 and value.
 *
 * Masking: with MLA_CAUSAL, query row i sits at global position q_offset + i
 * and key row j at kv_offset + j, and j is visible iff its position is not
 * after i's (TT-NN logical_n: positions are global; Ascend maskType 1 = TRIU).
 * Without it every key is visible.  Key rows that no query row of the call
 * can see are never read into the result, so they may hold any bits (NaN
 * included).
 *
 * Varlen (Ascend seqLen of shape [batch]): when seq_lens (device int32
 * [n_seqs]) is given, B must be 1 and Nq == Nkv == the token count T; the
 * sequences are packed along t, sequence s owning tokens [cu_s, cu_s + len_s)
 * for queries and keys alike, and a query sees only keys of its own sequence
 * (positions restart at 0 in each sequence; q_offset and kv_offset must be 0).
 * Lengths must be >= 0 and sum to T; the device reads them, so this is not
 * checked before launch (a negative length counts as 0, the sum is clipped to
 * T, and tokens past the sum are left unwritten).
 *
 * Separate query and key lengths (MLA_SEQ_LENS_QK; Ascend seqLen of shape
 * [2, batch], as a non-first card of the ring meets another chunk's keys):
 * seq_lens is a device int32 [2, n_seqs] array, row 0 the query lengths and
 * row 1 the key lengths.  The queries are packed along t of q (Nq rows) and
 * the keys along t of kv, k_rope and v (Nkv rows), each sequence's keys in
 * the same order as its queries.  With MLA_CAUSAL the last query and the
 * last key of a sequence share a position: query i of a sequence with Lq
 * queries and Lk keys sees key j iff j <= i + Lk - Lq, so its first
 * Lq - Lk queries see no key when Lk < Lq (a query chunk meeting its cached
 * prefix and itself, as in chunked prefill; equal lengths give the plain
 * TRIU).  A length is clipped to the rows left in its tensor, as above.
 *
 * Padded batches (MLA_VALID_LENS; shared-latent form): seq_lens is a device
 * int32 [B] array (n_seqs == B) of valid lengths: batch b's query rows
 * [0, min(len_b, Nq)) attend its key rows [0, min(len_b, Nkv)) (with the
 * usual offsets and mask); later query rows are not written and later key
 * rows are not attended (TT-NN ring_mla: padded chunks with a valid length,
 * kv_actual_isl).  A negative length counts as 0.
 *
 * Ring fold (Ascend calcType): prev_out [B, Hq, Nq, dv] and prev_lse
 * [B, Hq, Nq] are both NULL (first ring step) or both given; when given the
 * result is folded into them:  L = logaddexp(prev_lse, lse_new),
 * out = exp(prev_lse - L) * prev_out + exp(lse_new - L) * out_new, where a
 * side whose LSE is -inf has weight 0.  out may alias prev_out and lse may
 * alias prev_lse (same views); any other overlap is undefined.
 *
 * Outputs: out [B, Hq, Nq, dv] bf16 (round to nearest even); lse [B, Hq, Nq]
 * float32 natural-log LSE, or NULL when no LSE is wanted.  A row with no
 * visible key (and no prev) gets out = 0 and lse = -inf.
 *
 * Element types of the fold: MLA_OUT_F32 makes out a float32 view and
 * MLA_PREV_OUT_F32 makes prev_out one (16-byte aligned, strides multiples of
 * 4 elements).  The pages' prevOut is bf16; a float32 running output lets a
 * caller fold many ring steps without rounding the carry to bf16 each time,
 * rounding once in the last step.
 *
 * scale multiplies q.k (Ascend qkScale; TensorRT-LLM softmax_scale =
 * 1/sqrt(qk_head_dim) for q_scaling = 1); it has no default here.
 *
 * Kernels exist for:
 *   - shared latent:  Hkv == 1, v == NULL, dq + dr == 576, dv == 512
 *     (dr == 0 or 64), no packed seq_lens (MLA_VALID_LENS is supported);
 *   - split:          v != NULL, q_rope and k_rope given, dq == 128, dr == 64,
 *     dv == 128, Hq % Hkv == 0, with or without seq_lens (of one or two rows).
 * Other shapes return MLA_ERR_UNSUPPORTED.
 */
mla_status mla_fwd(const mla_rows* q, const mla_rows* q_rope,
                   const mla_rows* kv, const mla_rows* k_rope, const mla_rows* v,
                   int32_t B, int32_t Hq, int32_t Hkv, int64_t Nq, int64_t Nkv,
                   int32_t dq, int32_t dr, int32_t dv,
                   const int32_t* seq_lens, int32_t n_seqs,
                   float scale, uint32_t flags, int64_t q_offset, int64_t kv_offset,
                   const mla_rows* prev_out, const mla_rows* prev_lse,
                   const mla_rows* out, const mla_rows* lse,
                   void* workspace, size_t workspace_bytes,
                   void* stream /* hipStream_t */);

/*
 * mla_fwd_fp8 -- the shared-latent attention over FP8 inputs (TensorRT-LLM
 * mla.py, forward_absorption_context: the fused FP8 query and the FP8 latent
 * cache in float8_e4m3fn with the BMM1 and BMM2 scales; the output stays
 * bf16).
 *
 * q8 [B, Hq, Nq, 576] and kv8 [B, 1, Nkv, 576]: OCP FP8 E4M3 codes (one byte
 * per element; mla_rows views with strides in bytes, data and strides
 * multiples of 16, the kv8 view's stride_h ignored), dequantised as
 * code * q_scale and code * kv_scale (positive, finite; 1 for the page's
 * unit-scale fused query).  The score is scale * q . kv over all 576 columns,
 * the value the first 512 dequantised columns of the kv row; masking and
 * offsets as mla_fwd (flags: 0 or MLA_CAUSAL).
 *
 * Arithmetic: both products run on 8-bit MFMA with fp32 accumulation; the
 * softmax weights are rounded to e4m3 for the P.V product, each taken
 * against its row's reference max (so a weight is at most 2^8); O is divided
 * by the sum of the rounded weights, and lse (natural log, fp32) uses the
 * exact sum.  An e4m3 weight carries 3 mantissa bits, so O differs from the
 * exact attention of the dequantised inputs by up to a few percent of the
 * spread of the values on rows dominated by few keys (less on long rows);
 * the LSE is as exact as in the bf16 form.
 *
 * out [B, Hq, Nq, 512] bf16 (round to nearest even); lse [B, Hq, Nq] or NULL.
 * workspace: as mla_fwd (the item queue's counter).  Kernels exist for
 * dk == 576, dv == 512; other shapes return MLA_ERR_UNSUPPORTED.
 */
mla_status mla_fwd_fp8(const mla_rows* q8, const mla_rows* kv8, int32_t B, int32_t Hq, int64_t Nq, int64_t Nkv,
                       int32_t dk, int32_t dv, float scale, float q_scale, float kv_scale, uint32_t flags,
                       int64_t q_offset, int64_t kv_offset, const mla_rows* out, const mla_rows* lse,
                       void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * mla_fwd_group -- up to MLA_MAX_GROUP shared-latent mla_fwd calls in one
 * launch: one ring step for every query chunk at once (TT-NN ring_mla, the
 * ring's steps; Ascend RingMLAOperation, one call per ring step).  Each call
 * computes exactly what mla_fwd computes with the same arguments (the
 * shared-latent form: v == NULL, Hkv == 1, no seq_lens; no workspace); the
 * calls must not write memory another call of the group reads or writes.
 * Calls are validated in order before anything is launched; the first
 * failure returns its status, and mla_last_error() names the call.  A call
 * with no rows is skipped; n == 0 launches nothing.
 */
#define MLA_MAX_GROUP 4

typedef struct {
  const mla_rows* q;            /* as mla_fwd */
  const mla_rows* q_rope;
  const mla_rows* kv;
  const mla_rows* k_rope;
  int32_t B, Hq;
  int64_t Nq, Nkv;
  int32_t dq, dr, dv;
  float scale;
  uint32_t flags;
  int64_t q_offset, kv_offset;
  const mla_rows* prev_out;
  const mla_rows* prev_lse;
  const mla_rows* out;
  const mla_rows* lse;
} mla_fwd_call;

mla_status mla_fwd_group(int32_t n, const mla_fwd_call* calls, void* stream /* hipStream_t */);

/*
 * mla_ring_fwd -- causal shared-latent attention of q over kv computed as a
 * ring of n_chunks contiguous chunks on one device (TT-NN ring_mla: the
 * sequence split into chunks, each query chunk meeting the KV chunks in
 * turn, the output carried with its statistics; TensorRT-LLM mla.py,
 * forward_context_with_chunked_prefill: earlier chunks with a full mask,
 * the current one causal, partial outputs merged through their softmax
 * stats; Ascend RingMLAOperation calcType: the first ring step has no prev).
 *
 * q [B, H, N, dq] and kv [B, 1, N, dq] (mla_rows views, the kv view's
 * stride_h ignored), dq = 576 (512 latent + 64 RoPE columns in one row),
 * value = the first dv = 512 columns of each kv row.  n_chunks: 1 .. 64;
 * C = ceil(N / n_chunks), chunk r holds rows [r*C, min((r+1)*C, N)) (the last
 * chunks may be shorter, or empty, when N is not a multiple: TT-NN ring_mla's
 * logical length).  Query chunk r attends each KV chunk k <= r through one
 * call equivalent to mla_fwd with q_offset = r*C and kv_offset = k*C (so the diagonal chunk is causal, earlier ones full,
 * later ones are never visited: their keys lie in the causal future), and
 * every call after a chunk's first folds into the running result.  The
 * running result between folds is float32, kept in the workspace; only each
 * query chunk's last call writes out (bf16) and its final lse.
 *
 * Execution: one kernel launch (for n_chunks > 1).  A work item is one block
 * of 32 query rows of up to 4 heads of one chunk; its workgroup runs all of
 * that chunk's calls for those rows in turn, in the chunk's fold order,
 * taking items from a queue (the last chunk, with the longest chains,
 * first).  Each call computes exactly what the corresponding mla_fwd call
 * would (bit for bit), so the result equals the ring of separate calls; the
 * float32 running result stays in the workspace in the kernel's own layout.
 *
 * order: the order each query chunk's calls fold in (mla_ring_schedule:
 * a chunk's calls fold in increasing step index).  Results agree up to
 * rounding between orders: the fold is commutative and associative.
 *
 * out [B, H, N, 512] bf16 and lse [B, H, N] fp32, both required.
 * workspace: device memory of at least
 * mla_ring_workspace_size(B, H, N, n_chunks) bytes, 256-byte aligned (may be
 * NULL when that size is 0: one chunk, or an empty problem); contents
 * unspecified on return.  It also holds the launch's item counter, so two
 * ring calls in flight at once need two workspaces.  Every argument and
 * every call is validated before anything is enqueued.
 */
#define MLA_RING_ORDER 0     /* step s is ring step s: chunk r meets KV chunk (r - s) mod P */
#define MLA_RING_BALANCED 1  /* the same calls in equally full steps, the diagonals last */
mla_status mla_ring_fwd(const mla_rows* q, const mla_rows* kv, int32_t B, int32_t H, int64_t N,
                        int32_t dq, int32_t dv, float scale, int32_t n_chunks, int32_t order,
                        const mla_rows* out, const mla_rows* lse,
                        void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/* Bytes of the workspace mla_ring_fwd needs: the float32 running results,
 * B * ceil(H/4)*4 * n_chunks * ceil(C/32)*32 * 512 * 4 with C = ceil(N / n_chunks),
 * plus 256 for the item counter, for n_chunks > 1 and N > 0; 0 for one chunk,
 * no rows or invalid sizes; SIZE_MAX when the product overflows (mla_ring_fwd
 * then fails with MLA_ERR_UNSUPPORTED). */
size_t mla_ring_workspace_size(int32_t B, int32_t H, int64_t N, int32_t n_chunks);

/*
 * mla_ring_schedule -- the steps of the ring for P = n_chunks, which fix
 * the order mla_ring_fwd folds each query chunk's calls in (host only;
 * nothing is enqueued).  launch_of: host int32 array of P (P + 1) / 2
 * entries; entry r (r + 1) / 2 + k receives the step index of the call of
 * query chunk r on KV chunk k (k <= r).  *n_launches receives the number of
 * steps (P).  A query chunk has at most one call per step, and its calls
 * fold in step order.  (The steps are what a ring of P devices would run
 * together; on one device mla_ring_fwd runs them all in one launch.)
 *
 * MLA_RING_ORDER: step s is ring step s, as each device of a P-device
 * ring runs it (P diagonal calls, then P - 1, ..., 1 full calls).
 * MLA_RING_BALANCED: each query chunk's full calls (k < r), longest chains
 * first, go to the r least-filled of the first P - 1 steps, and the P
 * diagonal calls (half the work of a full call each) come last; the steps
 * are then equally full.
 */
mla_status mla_ring_schedule(int32_t n_chunks, int32_t order, int32_t* launch_of, int32_t* n_launches);

/*
 * mla_merge_lse -- fold two partial results over disjoint key sets
 * (TensorRT-LLM mla.py, forward_context_with_chunked_prefill: partial outputs
 * merged with their softmax stats; Ascend RingMLAOperation prevOut/prevLse).
 *
 *   L = logaddexp(lse_a, lse_b)
 *   out = exp(lse_a - L) * out_a + exp(lse_b - L) * out_b
 * with weight exactly 0 (and no multiply) for a side whose LSE is -inf; both
 * -inf gives out = 0, lse = -inf.
 *
 * out_a, out_b, out: bf16 [B, H, N, dv]; lse_a, lse_b, lse: fp32 [B, H, N].
 * dv must be a multiple of 8.  out may alias out_a or out_b and lse may alias
 * lse_a or lse_b (each element is read before it is written by the same
 * thread); other overlaps are undefined.
 */
mla_status mla_merge_lse(const mla_rows* out_a, const mla_rows* lse_a,
                         const mla_rows* out_b, const mla_rows* lse_b,
                         int32_t B, int32_t H, int64_t N, int32_t dv,
                         const mla_rows* out, const mla_rows* lse,
                         void* stream /* hipStream_t */);

/*
 * mla_sparse_fwd -- top-k sparse latent attention (NKI
 * mla_sparse_attention_cte_kernel, "Parameters" and "Returns").
 *
 * q_lift [B, S, H, L] and q_pe [B, S, H, R] (views with t = query, h = head);
 * c_kv [B, S_kv, L] and k_pe [B, S_kv, R] (views with t = cache row, stride_h
 * unused); topk_idx: device int32 [B, S, K] contiguous.  Query i attends
 * exactly the K listed cache rows (a multiset: repeats count; order is
 * irrelevant; no extra mask) with score scale * (q_lift . c_kv + q_pe . k_pe)
 * and value c_kv.  All H heads of a query share its index list.  An index
 * outside [0, S_kv) is not attended (the pages leave it undefined; it is
 * treated like a padding sentinel); a query with no valid index gets out = 0.
 * The list's order changes the result only by rounding; lists sorted
 * ascending gather with better cache locality, since neighbouring queries
 * then fetch nearby rows at the same step (measured at S = 4096, K = 2048,
 * H = 128: 2.18 ms unsorted, 2.07 ms sorted, 2.04 ms for one contiguous
 * range).
 *
 * out [B, S, H*L] bf16 as a view with t = query, h = head (stride_h = L for
 * the page's row-major h*L + l order); lse [B, S, H] fp32 (view with t =
 * query, h = head) or NULL.  L == 512, R == 64, H <= 128, 1 <= K <= 4096
 * (larger K returns MLA_ERR_UNSUPPORTED).
 *
 * flags: 0, MLA_OUT_MX4 or MLA_OUT_F32.  With MLA_OUT_MX4 each head's L
 * latent columns are written in MX 4-pack order (NKI
 * mla_sparse_attention_cte_kernel, "Returns" and "Notes": the layout its
 * o_proj load expects): natural column l = 4 * group + sub is stored at
 * sub * (L / 4) + group.  With MLA_OUT_F32 (the value mla_fwd uses) out is a
 * float32 view (16-byte aligned, strides multiples of 4 elements) holding
 * the result before its rounding to bf16; it is not combined with
 * MLA_OUT_MX4 (MLA_ERR_UNSUPPORTED).  Other bits return MLA_ERR_INVALID_ARG.
 */
#define MLA_OUT_MX4 1u
mla_status mla_sparse_fwd(const mla_rows* q_lift, const mla_rows* q_pe,
                          const mla_rows* c_kv, const mla_rows* k_pe,
                          const int32_t* topk_idx,
                          int32_t B, int64_t S, int64_t S_kv, int32_t H,
                          int32_t L, int32_t R, int32_t K, float scale, uint32_t flags,
                          const mla_rows* out, const mla_rows* lse,
                          void* workspace, size_t workspace_bytes,
                          void* stream /* hipStream_t */);

/*
 * mla_decode_fwd -- token generation: one new query per sequence over its
 * valid cache rows, with the rows split into ranges processed in parallel
 * and a separate reduction (Mojo mha_single_batch_pipelined, token-generation
 * description: seq_len = 1, num_keys valid entries per sequence, and a key
 * split whose partial results are reduced by a kernel of their own).
 *
 * q [B, H, dq] plus, optionally, q_rope [B, H, dr]: the newest token of each
 * sequence (views with b = sequence, h = head; stride_t is ignored).
 * kv [n_slots, Nkv, dq] plus, optionally, k_rope [n_slots, Nkv, dr]: the
 * latent cache (views with b = cache slot, t = cache row; stride_h is
 * ignored).  kv_slots: device int32 [B], the cache slot each sequence reads
 * (TT-NN ring_mla kv_cache_batch_idx: one batch slot of an indexed cache),
 * with n_slots > 0 slots; a slot outside [0, n_slots) leaves the sequence
 * without valid rows.  NULL: sequence b reads slot b (n_slots 0 or >= B).
 * kv_lens: device int32 [B], the valid rows of each sequence (clamped to
 * [0, Nkv]), or NULL for Nkv everywhere.  Sequence b's query sees the first
 * kv_lens[b] rows of its slot, all of them; the score is scale * q.row over
 * dq + dr columns, the value the first dv columns of the row.
 *
 * out [B, H, dv] bf16 and lse [B, H] fp32 natural-log LSE (or NULL), views
 * with stride_t ignored.  A sequence with no valid row gets out = 0 and
 * lse = -inf.
 *
 * n_splits: key ranges per sequence, or 0 for the library's choice; a range
 * holds at most 2048 rows and there are at most 64 (Nkv <= 131072).  With
 * more than one range, each writes an fp32 partial result (output and LSE)
 * and a reduction kernel folds them through their LSE; with one, the
 * attention kernel writes out and lse itself.  Results do not depend on
 * the split beyond rounding.
 *
 * workspace: device memory of at least
 * mla_decode_workspace_size(B, H, Nkv, n_splits) bytes, 256-byte aligned,
 * given as workspace_bytes (required): the partial results and the item
 * queue's counter.  It needs no initialisation; calls that may run at the
 * same time need distinct workspaces.
 *
 * Kernels exist for dq + dr == 576 (dr == 0 or 64), dv == 512, H <= 128;
 * other shapes return MLA_ERR_UNSUPPORTED.
 */
mla_status mla_decode_fwd(const mla_rows* q, const mla_rows* q_rope,
                          const mla_rows* kv, const mla_rows* k_rope,
                          const int32_t* kv_lens,
                          const int32_t* kv_slots, int32_t n_slots,
                          int32_t B, int32_t H, int64_t Nkv,
                          int32_t dq, int32_t dr, int32_t dv, float scale,
                          int32_t n_splits,
                          const mla_rows* out, const mla_rows* lse,
                          void* workspace, size_t workspace_bytes,
                          void* stream /* hipStream_t */);

/* Bytes of the workspace mla_decode_fwd needs for these sizes (0 if no split
 * fits: n_splits too small for Nkv, or Nkv > 131072). */
size_t mla_decode_workspace_size(int32_t B, int32_t H, int64_t Nkv, int32_t n_splits);

/*
 * mla_decode_fwd_noalloc -- mla_decode_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, the same kernels and the same
 * results bit for bit, but no workspace argument.  The partial results and
 * the item queue's counter live in a static device array of the library,
 * MLA_DECODE_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends; the call itself allocates and frees nothing.  Sizes whose workspace
 * (mla_decode_workspace_size) exceeds MLA_DECODE_SCRATCH_BYTES return
 * MLA_ERR_UNSUPPORTED and enqueue nothing.  The workspace is 256 bytes plus,
 * with more than one key range, (dv + 1) * 4 bytes per (sequence, range,
 * head), rounded up: at H = 128 up to 319 (sequence, range) pairs fit, e.g.
 * 64 sequences of 8192 rows in 4 ranges each; a call with one range per
 * sequence always fits.  Every call on one GPU shares that
 * GPU's array and leaves its contents behind (each call resets what must
 * start at zero): calls that may overlap on one GPU (different streams
 * without ordering between them) race and must not be issued.  The first
 * call on each device looks the array's address up (hipGetSymbolAddress);
 * a failure there returns MLA_ERR_HIP.
 */
#define MLA_DECODE_SCRATCH_BYTES (80u << 20)
mla_status mla_decode_fwd_noalloc(const mla_rows* q, const mla_rows* q_rope,
                                  const mla_rows* kv, const mla_rows* k_rope,
                                  const int32_t* kv_lens,
                                  const int32_t* kv_slots, int32_t n_slots,
                                  int32_t B, int32_t H, int64_t Nkv,
                                  int32_t dq, int32_t dr, int32_t dv, float scale,
                                  int32_t n_splits,
                                  const mla_rows* out, const mla_rows* lse,
                                  void* stream /* hipStream_t */);

/*
 * mla_vup -- V-up projection of the latent attention output (TensorRT-LLM
 * mla.py, forward_absorption_context and forward_absorption_generation: the
 * per-head product [heads, tokens, kv_lora_rank] x [heads, kv_lora_rank,
 * v_head_dim] after latent attention, which yields o_proj's input):
 *
 *   out[b, h, t, c] = sum_l o[b, h, t, l] * w_uv[h, c, l],  l < L, c < dvh
 *
 * o: bf16 rows view [B, H, T, L] (mla_fwd's out as it is; mla_sparse_fwd's
 * out [B, S, H*L] as stride_b, stride_h = L, stride_t = H*L; mla_decode_fwd's
 * out [B, H, dv] with T = 1).  w_uv: device bf16 [H, dvh, L] contiguous, 16-byte
 * aligned (the page's v_b_proj layout [heads, v_head_dim, kv_lora_rank]).
 * out: bf16 rows view [B, H, T, dvh] (for o_proj's [tokens, H*dvh] input:
 * stride_h = dvh, stride_t = H*dvh).  fp32 accumulation, out rounded to bf16
 * (round to nearest even).  L == 512 and dvh == 128 (else
 * MLA_ERR_UNSUPPORTED); out must not overlap o or w_uv.
 *
 * flags: 0 or MLA_OUT_MX4 -- o's columns of each head are in MX 4-pack order
 * (as mla_sparse_fwd writes them with that flag); the result is the same
 * projection of the natural-order values.  Other bits: MLA_ERR_INVALID_ARG.
 */
mla_status mla_vup(const mla_rows* o, const void* w_uv, int32_t B, int32_t H, int64_t T,
                   int32_t L, int32_t dvh, uint32_t flags, const mla_rows* out,
                   void* stream /* hipStream_t */);

/*
 * mla_debug_gather -- test export.  Gathers the top-k rows of one query's
 * index list through the same device tile loader mla_sparse_fwd uses (with
 * its LDS swizzle undone on the way out): rows_out [K, L + R] bf16 contiguous,
 * row k = c_kv[b, idx[k]] concatenated with k_pe[b, idx[k]] (an out-of-range
 * index yields a row of zeros).  Backs the bit-exact gather check.
 */
mla_status mla_debug_gather(const mla_rows* c_kv, const mla_rows* k_pe,
                            const int32_t* idx, int32_t b, int64_t S_kv,
                            int32_t L, int32_t R, int32_t K,
                            uint16_t* rows_out, void* stream /* hipStream_t */);

/* Bytes of the optional workspace of mla_fwd and mla_sparse_fwd (see
 * "Workspace" above); the same for every shape. */
size_t mla_workspace_size(void);

/* Thread-local description of the last non-OK status on this thread. */
const char* mla_last_error(void);

/* Library version string. */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA355_H */
