// Internal interface between the C-ABI layer and the HIP kernels of
// libmla355.so.  Not installed; the public contract is include/mla355.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Longest top-k index list of the sparse kernel (it stages a query's list in
// LDS).
constexpr int kSparseMaxTopk = 4096;

// Bytes of the optional workspace (word 0: the item queue's counter; the
// rest is reserved).
constexpr size_t kWorkspaceBytes = 256;

// A row view: element (b, h, t, d) at p[b*sb + h*sh + t*st + d] (strides in
// elements; bf16 unless a flag says float32, in which case the pointer is
// reinterpreted).
struct RowsC {
  const uint16_t* p;
  int64_t sb, sh, st;
};
struct RowsM {
  uint16_t* p;
  int64_t sb, sh, st;
};
// A float32 per-row view (LSE): element (b, h, t) at p[b*sb + h*sh + t*st].
struct LseC {
  const float* p;
  int64_t sb, sh, st;
};
struct LseM {
  float* p;
  int64_t sb, sh, st;
};

// Parameters of one attention launch.  The key (and query) vector of a row is
// the concatenation of part A (da columns) and part B (the rest).
struct AttnParams {
  RowsC qa, qb;             // query parts
  RowsC ka, kb;             // key parts (sparse: c_kv, k_pe)
  RowsC v;                  // explicit value rows (split form only)
  RowsM out;
  RowsC prev_out;           // p == nullptr: no fold
  LseM lse;                 // p == nullptr: not written
  LseC prev_lse;
  const int32_t* idx;       // sparse: [B, S, K] contiguous
  const int32_t* seq_lens;  // split varlen: [n_seqs] or nullptr
  const int32_t* kv_seq_lens;  // split varlen: the key lengths [n_seqs], or nullptr (the same as seq_lens)
  const int32_t* valid_lens;  // latent: valid rows of each batch [B] (padded tensors), or nullptr
  int32_t n_seqs;
  int32_t da;               // columns in part A
  int32_t B, Hq, group;     // group = Hq / Hkv
  int64_t Nq, Nkv;          // sparse: Nq = S, Nkv = S_kv
  int32_t topk;
  int64_t q_offset, kv_offset;
  float scale_log2;         // scale * log2(e)
  int32_t causal;
  int32_t out_f32;          // out holds float32 (else bf16)
  int32_t prev_f32;         // prev_out holds float32 (else bf16)
  int32_t mx4;              // sparse: each head's latent columns in MX 4-pack order
  int32_t n_qblk, n_hgrp;   // grid factors (see each launcher)
  unsigned* queue;          // item queue's counter, or nullptr
  // token generation (sparse kernel): each item's list is the range
  // [q0 * topk, (q0 + 1) * topk) of its sequence's valid cache rows
  int32_t decode;
  const int32_t* kv_lens;   // decode: valid rows per sequence [B], or nullptr (Nkv)
  const int32_t* kv_slots;  // decode: cache slot of each sequence [B], or nullptr (slot b)
  int32_t n_slots;          // decode: slots of the cache
  float v_scale;            // FP8 form: dequantisation scale of the value rows (applied to O)
};

// Several shared-latent calls in one launch (a ring step for all query
// chunks): call k serves workgroups [first[k], first[k+1]), or every n-th
// workgroup when the calls have equal item counts (interleave).
constexpr int kMaxGroup = 4;
struct GroupParams {
  int32_t n;
  int32_t interleave;       // all calls have the same item count: item i of call k is workgroup i*n + k
  int32_t first[kMaxGroup + 1];
  AttnParams sub[kMaxGroup];
};
static_assert(sizeof(GroupParams) <= 4096, "kernel arguments are limited to 4 KB");

// The one-device ring in one launch (mla_ring_fwd).  A work item is one
// latent item (32 query rows of up to 4 heads) of query chunk r together with
// every call of that chunk: its workgroup runs them one after another in the
// chunk's fold order, each call folding into the float32 carry the one
// before it wrote.  Items are taken from a queue, the last chunk (the longest
// chains) first.
constexpr int kMaxRing = 64;
// The running result of an item is kept between its calls in the output
// accumulators' own layout (kRingCarryFloats floats per item: wave w's
// float4 k of lane l at ((w * 64 + k) * 64 + l) * 4), so that each lane
// writes and reads back its own accumulators in whole 1 KB wave accesses.
constexpr int64_t kRingCarryFloats = 4 * 64 * 64 * 4;
struct RingParams {
  AttnParams base;           // the call of query chunk 0 on KV chunk 0 (views at row 0)
  float* carry;              // [P][chunk_items][kRingCarryFloats] float32 running results
  unsigned* queue;           // the item counter (zeroed before the launch)
  int64_t chunk_items;       // items of a full chunk (the carry's chunk stride)
  int64_t C, N;              // chunk length (the last chunks may be shorter or empty), rows
  int32_t P, n_items;        // chunks; items of all chunks
  int32_t chunk_first[kMaxRing + 1];  // items of chunk P-1-j: [chunk_first[j], chunk_first[j+1])
  uint8_t fold_k[kMaxRing * (kMaxRing + 1) / 2];  // chunk r's s-th call meets KV chunk fold_k[r(r+1)/2 + s]
};
static_assert(sizeof(RingParams) <= 4096, "kernel arguments are limited to 4 KB");

// Decode split-K reduction: partial results of S key ranges per (b, h),
// element (b, s, h, d) of po at ((b * S + s) * H + h) * dv + d and its LSE
// at pl[(b * S + s) * H + h].
struct CombineParams {
  const float* po;
  const float* pl;
  int32_t B, H, S, dv;
  RowsM out;                // [B, H, dv] bf16 (t unused)
  LseM lse;                 // [B, H] or nullptr
};

struct MergeParams {
  RowsC oa, ob;
  LseC la, lb;
  RowsM out;
  LseM lse;
  int32_t B, H;
  int64_t N;
  int32_t dv;
};

// V-up projection: out[b, h, t, c] = sum_l o[b, h, t, l] * w[h, c, l]
// (l < 512, c < 128; w contiguous [H, 128, 512]).
struct VupParams {
  RowsC o;
  const uint16_t* w;
  RowsM out;
  int32_t B, H;
  int64_t T;
  int32_t mx4;              // o's columns in MX 4-pack order
  int64_t blocks_per_part;  // set by the launcher
};

struct GatherParams {
  RowsC ka, kb;
  const int32_t* idx;
  int32_t b;
  int64_t Nkv;
  int32_t K;
  uint16_t* rows_out;
};

hipError_t launch_latent_dense(const AttnParams& p, hipStream_t s);
hipError_t launch_latent_group(const GroupParams& g, hipStream_t s);
hipError_t launch_latent_ring(const RingParams& g, hipStream_t s);
hipError_t launch_latent_sparse(const AttnParams& p, hipStream_t s);
hipError_t launch_split(const AttnParams& p, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_decode(const AttnParams& p, int64_t items, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_debug_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_vup(const VupParams& p, hipStream_t s);
hipError_t launch_latent_fp8(const AttnParams& p, hipStream_t s);

// Compute units of the current device, cached per device (0 if unknown).
int cu_count();

// The decode workspace that mla_decode_fwd_noalloc uses in place of a
// caller-provided one: a static device array of kDecodeScratchBytes per GPU
// (mla_scratch.hip).  decode_scratch() returns the current device's copy,
// looked up on the first call on that device.
constexpr size_t kDecodeScratchBytes = (size_t)80 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace mla
