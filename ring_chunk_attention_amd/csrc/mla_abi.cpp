// C ABI of libmla355.so: argument validation, kernel selection and launch.
// The contract is documented in include/mla355.h.
#include "mla355.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <tuple>
#include <vector>

#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

// The optional workspace: the item queue's counter.
mla_status check_workspace(void* ws, size_t bytes) {
  if (!ws) return MLA_OK;
  if (reinterpret_cast<uintptr_t>(ws) & 15u) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (bytes < mla::kWorkspaceBytes)
    return fail(MLA_ERR_INVALID_ARG, "workspace_bytes (%zu) is below mla_workspace_size() (%zu)", bytes,
                (size_t)mla::kWorkspaceBytes);
  return MLA_OK;
}

// Token generation: keys per split (`chunk`, a multiple of the 32-row tile,
// at most the sparse kernel's 2048-entry list) and splits per sequence.  The
// library's choice (req == 0) takes the fewest splits that give 256 work
// items (one per compute unit of an MI355X), with at least 256 rows per
// split: every extra split adds a 256 KB fp32 partial to write and reduce
// (measured on 64 sequences of 8192 rows: 4 splits 0.19 ms, 8 splits
// 0.25 ms).  Returns false if no choice fits (more than 64 splits).
bool decode_split(int32_t B, int64_t Nkv, int32_t req, int32_t* S, int32_t* chunk) {
  constexpr int64_t kMaxChunk = 2048, kMinChunk = 256, kMaxSplits = 64, kTargetItems = 256;
  const int64_t n = Nkv > 0 ? Nkv : 1;
  int64_t s;
  if (req > 0) {
    s = req;
  } else {
    const int64_t s_min = (n + kMaxChunk - 1) / kMaxChunk;
    const int64_t s_fill = B > 0 ? (kTargetItems + B - 1) / B : 1;
    const int64_t s_cap = std::max<int64_t>(1, (n + kMinChunk - 1) / kMinChunk);
    // (never past the most ranges there may be: few long sequences ask for more)
    s = std::max(s_min, std::min({s_fill, s_cap, kMaxSplits}));
  }
  int64_t c = (n + s - 1) / s;
  c = (c + 31) / 32 * 32;
  if (c > kMaxChunk) return false;
  s = (n + c - 1) / c;
  if (s > kMaxSplits) return false;
  *S = (int32_t)s;
  *chunk = (int32_t)c;
  return true;
}

// Decode workspace: the queue counter, then (S > 1) the partial LSEs and
// the fp32 partial outputs, each 256-byte aligned.
size_t decode_ws_bytes(int32_t B, int32_t H, int32_t S, int32_t dv, size_t* off_l, size_t* off_o) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  *off_l = 256;
  if (S <= 1) {
    *off_o = 256;
    return 256;
  }
  *off_o = *off_l + up((size_t)B * S * H * sizeof(float));
  return *off_o + up((size_t)B * S * H * dv * sizeof(float));
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A bf16 row view used by a kernel: data 16-byte aligned, b/h/t strides
// multiples of 8 elements, non-negative.  `empty`: the view holds no rows
// (a zero size), so its data pointer may be NULL (nothing is read or
// written through it).
mla_status check_rows(const mla_rows* r, const char* name, bool need_h = true, bool empty = false) {
  if (!r) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (!r->data && !empty) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (!aligned16(r->data)) return fail(MLA_ERR_INVALID_ARG, "%s: data pointer must be 16-byte aligned", name);
  if (r->stride_b < 0 || r->stride_h < 0 || r->stride_t < 0)
    return fail(MLA_ERR_INVALID_ARG, "%s: negative stride", name);
  if (r->stride_b % 8 || (need_h && r->stride_h % 8) || r->stride_t % 8)
    return fail(MLA_ERR_INVALID_ARG, "%s: strides must be multiples of 8 elements", name);
  return MLA_OK;
}

// A float32 row view: data 16-byte aligned, b/h/t strides multiples of 4.
mla_status check_rows_f32(const mla_rows* r, const char* name, bool empty = false) {
  if (!r) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (!r->data && !empty) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (!aligned16(r->data)) return fail(MLA_ERR_INVALID_ARG, "%s: data pointer must be 16-byte aligned", name);
  if (r->stride_b < 0 || r->stride_h < 0 || r->stride_t < 0)
    return fail(MLA_ERR_INVALID_ARG, "%s: negative stride", name);
  if (r->stride_b % 4 || r->stride_h % 4 || r->stride_t % 4)
    return fail(MLA_ERR_INVALID_ARG, "%s: float32 strides must be multiples of 4 elements", name);
  return MLA_OK;
}

mla_status check_lse(const mla_rows* r, const char* name, bool empty = false) {
  if (!r) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (!r->data && !empty) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
  if (reinterpret_cast<uintptr_t>(r->data) & 3u) return fail(MLA_ERR_INVALID_ARG, "%s: data pointer must be 4-byte aligned", name);
  if (r->stride_b < 0 || r->stride_h < 0 || r->stride_t < 0)
    return fail(MLA_ERR_INVALID_ARG, "%s: negative stride", name);
  return MLA_OK;
}

mla::RowsC rc(const mla_rows* r) {
  return mla::RowsC{static_cast<const uint16_t*>(r->data), r->stride_b, r->stride_h, r->stride_t};
}
mla::RowsM rm(const mla_rows* r) {
  return mla::RowsM{static_cast<uint16_t*>(r->data), r->stride_b, r->stride_h, r->stride_t};
}
mla::LseC lc(const mla_rows* r) {
  if (!r) return mla::LseC{nullptr, 0, 0, 0};
  return mla::LseC{static_cast<const float*>(r->data), r->stride_b, r->stride_h, r->stride_t};
}
mla::LseM lm(const mla_rows* r) {
  if (!r) return mla::LseM{nullptr, 0, 0, 0};
  return mla::LseM{static_cast<float*>(r->data), r->stride_b, r->stride_h, r->stride_t};
}

bool same_view(const mla_rows* a, const mla_rows* b) {
  return a->data == b->data && a->stride_b == b->stride_b && a->stride_h == b->stride_h &&
         a->stride_t == b->stride_t;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kMaxGrid = 0x7fffffff;

// The product of non-negative sizes is at most kMaxGrid, with no overflow on
// the way (sizes come from the caller and may be anything).
bool fits_grid(std::initializer_list<int64_t> factors) {
  int64_t prod = 1;
  for (int64_t f : factors)
    if (__builtin_mul_overflow(prod, f, &prod)) return false;
  return prod <= kMaxGrid;
}

}  // namespace

namespace {

enum { FORM_EMPTY = 0, FORM_LATENT = 1, FORM_SPLIT = 2 };

// Validates one mla_fwd call and fills its kernel parameters; *form says
// which kernel serves it (FORM_EMPTY: nothing to launch).
mla_status prepare_fwd(const mla_rows* q, const mla_rows* q_rope, const mla_rows* kv,
                       const mla_rows* k_rope, const mla_rows* v, int32_t B, int32_t Hq,
                       int32_t Hkv, int64_t Nq, int64_t Nkv, int32_t dq, int32_t dr, int32_t dv,
                       const int32_t* seq_lens, int32_t n_seqs, float scale, uint32_t flags,
                       int64_t q_offset, int64_t kv_offset, const mla_rows* prev_out,
                       const mla_rows* prev_lse, const mla_rows* out, const mla_rows* lse,
                       void* workspace, size_t workspace_bytes, mla::AttnParams* pp, int* form) {
  mla_status st;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Nq < 0 || Nkv < 0)
    return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, Hq > 0, Hkv > 0, Nq >= 0, Nkv >= 0");
  if (Hq % Hkv) return fail(MLA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (dq <= 0 || dr < 0 || dv <= 0 || dq % 8 || dr % 8 || dv % 8)
    return fail(MLA_ERR_INVALID_ARG, "head dims must be positive multiples of 8 (dq=%d dr=%d dv=%d)", dq, dr, dv);
  if (flags & ~(MLA_CAUSAL | MLA_OUT_F32 | MLA_PREV_OUT_F32 | MLA_VALID_LENS | MLA_SEQ_LENS_QK))
    return fail(MLA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARG, "scale must be finite");
  if ((st = check_workspace(workspace, workspace_bytes))) return st;
  const bool out_f32 = flags & MLA_OUT_F32, prev_f32 = flags & MLA_PREV_OUT_F32;
  // query-side views are empty without query rows, key-side ones without key rows
  const bool no_q = B == 0 || Nq == 0, no_kv = B == 0 || Nkv == 0;
  if ((st = check_rows(q, "q", true, no_q)) || (st = check_rows(kv, "kv", true, no_kv))) return st;
  if ((st = out_f32 ? check_rows_f32(out, "out", no_q) : check_rows(out, "out", true, no_q))) return st;
  if ((q_rope == nullptr) != (k_rope == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "q_rope and k_rope must both be given or both be NULL");
  if ((q_rope == nullptr) != (dr == 0))
    return fail(MLA_ERR_INVALID_ARG, "dr must be 0 exactly when q_rope/k_rope are NULL");
  if (q_rope && ((st = check_rows(q_rope, "q_rope", true, no_q)) || (st = check_rows(k_rope, "k_rope", true, no_kv))))
    return st;
  if (v && (st = check_rows(v, "v", true, no_kv))) return st;
  if (!v && dv > dq)
    return fail(MLA_ERR_INVALID_ARG, "head_dim_v (%d) must not exceed the kv width (%d) when V is the KV prefix", dv, dq);
  if ((prev_out == nullptr) != (prev_lse == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "prev_out and prev_lse must both be given or both be NULL");
  if (prev_f32 && !prev_out) return fail(MLA_ERR_INVALID_ARG, "MLA_PREV_OUT_F32 given without prev_out");
  if (prev_out && ((st = prev_f32 ? check_rows_f32(prev_out, "prev_out", no_q)
                                  : check_rows(prev_out, "prev_out", true, no_q)) ||
                   (st = check_lse(prev_lse, "prev_lse", no_q))))
    return st;
  // (aliasing is judged on real buffers: empty views may all be NULL)
  if (prev_out && out->data && out->data == prev_out->data && out_f32 != prev_f32)
    return fail(MLA_ERR_INVALID_ARG, "out may alias prev_out only with the same element type");
  if (lse && (st = check_lse(lse, "lse", no_q))) return st;
  if (prev_out && out->data && out->data == prev_out->data && !same_view(out, prev_out))
    return fail(MLA_ERR_INVALID_ARG, "out may alias prev_out only as the identical view");
  if (prev_lse && lse && lse->data && lse->data == prev_lse->data && !same_view(lse, prev_lse))
    return fail(MLA_ERR_INVALID_ARG, "lse may alias prev_lse only as the identical view");
  const bool valid_lens = flags & MLA_VALID_LENS, lens_qk = flags & MLA_SEQ_LENS_QK;
  if (lens_qk && (valid_lens || !seq_lens))
    return fail(MLA_ERR_INVALID_ARG, "MLA_SEQ_LENS_QK needs packed seq_lens (and no MLA_VALID_LENS)");
  if (valid_lens) {
    if (!seq_lens) return fail(MLA_ERR_INVALID_ARG, "MLA_VALID_LENS needs seq_lens (valid rows per batch)");
    if (n_seqs != B) return fail(MLA_ERR_INVALID_ARG, "MLA_VALID_LENS needs n_seqs == B (one length per batch)");
    if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_INVALID_ARG, "seq_lens must be 4-byte aligned");
  } else if (seq_lens) {
    if (B != 1) return fail(MLA_ERR_INVALID_ARG, "seq_lens requires B == 1 (tokens packed along t)");
    if (n_seqs <= 0) return fail(MLA_ERR_INVALID_ARG, "seq_lens given with n_seqs <= 0");
    if (!lens_qk && Nq != Nkv)
      return fail(MLA_ERR_INVALID_ARG, "seq_lens of one row requires Nq == Nkv (same lengths for query and key)");
    if (q_offset || kv_offset) return fail(MLA_ERR_INVALID_ARG, "seq_lens requires q_offset == kv_offset == 0");
    if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_INVALID_ARG, "seq_lens must be 4-byte aligned");
  }

  mla::AttnParams& p = *pp;
  p = mla::AttnParams{};
  p.qa = rc(q);
  p.qb = q_rope ? rc(q_rope) : rc(q);
  p.ka = rc(kv);
  p.kb = k_rope ? rc(k_rope) : rc(kv);
  p.v = v ? rc(v) : mla::RowsC{nullptr, 0, 0, 0};
  p.out = rm(out);
  p.prev_out = prev_out ? rc(prev_out) : mla::RowsC{nullptr, 0, 0, 0};
  p.lse = lm(lse);
  p.prev_lse = lc(prev_lse);
  p.seq_lens = valid_lens ? nullptr : seq_lens;
  p.kv_seq_lens = lens_qk ? seq_lens + n_seqs : nullptr;
  p.n_seqs = seq_lens && !valid_lens ? n_seqs : 0;
  p.valid_lens = valid_lens ? seq_lens : nullptr;
  p.da = dq;
  p.B = B;
  p.Hq = Hq;
  p.group = Hq / Hkv;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.q_offset = q_offset;
  p.kv_offset = kv_offset;
  p.scale_log2 = scale * kLog2e;
  p.causal = (flags & MLA_CAUSAL) ? 1 : 0;
  p.out_f32 = out_f32 ? 1 : 0;
  p.prev_f32 = prev_f32 ? 1 : 0;
  p.queue = static_cast<unsigned*>(workspace);

  const bool latent = !v && Hkv == 1 && dq + dr == 576 && dv == 512 && (dr == 0 || dr == 64) &&
                      (!seq_lens || valid_lens);
  const bool split = v && q_rope && dq == 128 && dr == 64 && dv == 128 && !valid_lens;
  if (latent) {
    if (dr == 0) {
      // one 576-column tensor: the kernel reads its last 64 columns as the RoPE part
      // (kv may be NULL when it has no rows: the kernel then loads no key tile)
      p.qb.p = p.qa.p + (dq - 64);
      p.kb.p = p.ka.p ? p.ka.p + (dq - 64) : nullptr;
      p.da = dq - 64;
    }
    const int64_t n_qblk = Nq / 32 + (Nq % 32 != 0), n_hgrp = (Hq + 3) / 4;
    if (!fits_grid({n_qblk, n_hgrp, B})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
    p.n_qblk = (int32_t)n_qblk;
    p.n_hgrp = (int32_t)n_hgrp;
    *form = Nq == 0 || B == 0 ? FORM_EMPTY : FORM_LATENT;
    return MLA_OK;
  }
  if (split) {
    const int64_t nb = Nq / 128 + (Nq % 128 != 0);
    if (!fits_grid({nb, B})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
    const int64_t qb = seq_lens ? nb + n_seqs : nb * B;
    if (!fits_grid({qb, Hq})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
    *form = Nq == 0 || B == 0 ? FORM_EMPTY : FORM_SPLIT;
    return MLA_OK;
  }
  return fail(MLA_ERR_UNSUPPORTED,
              "no kernel for Hq=%d Hkv=%d dq=%d dr=%d dv=%d v=%s seq_lens=%s (built: shared latent "
              "(packed seq_lens: no; MLA_VALID_LENS: yes) "
              "Hkv=1 dq+dr=576 dv=512 v=NULL; split dq=128 dr=64 dv=128 with v)",
              Hq, Hkv, dq, dr, dv, v ? "given" : "NULL", seq_lens ? "given" : "NULL");
}

// The calls of one mla_fwd_group launch, validated and prepared (nothing is
// launched).  g->n == 0: nothing to launch.
mla_status prepare_group(int32_t n, const mla_fwd_call* calls, mla::GroupParams* gp) {
  mla::GroupParams& g = *gp;
  g = mla::GroupParams{};
  if (n < 0 || n > MLA_MAX_GROUP) return fail(MLA_ERR_INVALID_ARG, "n (%d) must lie in [0, %d]", n, MLA_MAX_GROUP);
  if (n > 0 && !calls) return fail(MLA_ERR_INVALID_ARG, "calls: missing");
  int64_t items = 0;
  g.first[0] = 0;
  for (int32_t i = 0; i < n; ++i) {
    const mla_fwd_call& c = calls[i];
    mla::AttnParams p;
    int form = FORM_EMPTY;
    if (mla_status st = prepare_fwd(c.q, c.q_rope, c.kv, c.k_rope, nullptr, c.B, c.Hq, 1, c.Nq, c.Nkv, c.dq, c.dr,
                                    c.dv, nullptr, 0, c.scale, c.flags, c.q_offset, c.kv_offset, c.prev_out,
                                    c.prev_lse, c.out, c.lse, nullptr, 0, &p, &form)) {
      char buf[600];
      snprintf(buf, sizeof(buf), "call %d: %s", i, g_last_error.c_str());
      g_last_error = buf;
      return st;
    }
    if (form == FORM_EMPTY) continue;
    if (form != FORM_LATENT)
      return fail(MLA_ERR_UNSUPPORTED, "call %d: a group holds shared-latent calls only", i);
    items += (int64_t)p.n_qblk * p.n_hgrp * p.B;
    if (items > kMaxGrid) return fail(MLA_ERR_UNSUPPORTED, "group too large for one launch");
    g.sub[g.n] = p;
    g.first[++g.n] = (int32_t)items;
  }
  g.interleave = 1;
  for (int k = 1; k < g.n; ++k)
    if (g.first[k + 1] - g.first[k] != g.first[1]) g.interleave = 0;
  return MLA_OK;
}

// One-device ring (the value width of the shared-latent form; the most
// chunks; the bytes after the carry that hold the item queue's counter).
constexpr int kRingDv = 512;
constexpr int kMaxRingChunks = mla::kMaxRing;
constexpr size_t kRingQueueBytes = 256;

// Launch index of each call (r, k), k <= r, at launch_of[r (r + 1) / 2 + k];
// returns the number of launches.  MLA_RING_ORDER: launch s is ring step s,
// in which query chunk r meets KV chunk (r - s) mod P (for s <= r that is
// r - s; later steps bring chunks after r, which are skipped).
// MLA_RING_BALANCED: each query chunk's full calls (k < r), longest chains
// first, go to the r least-filled of the first P - 1 launches (ties: the
// earlier launch), and every diagonal call (k = r) runs in the last launch.
int ring_schedule(int P, int order, int32_t* launch_of) {
  auto id = [](int r, int k) { return r * (r + 1) / 2 + k; };
  if (order == MLA_RING_ORDER) {
    for (int r = 0; r < P; ++r)
      for (int s = 0; s <= r; ++s) launch_of[id(r, r - s)] = s;
    return P;
  }
  int fill[kMaxRingChunks] = {0};
  int order_of[kMaxRingChunks];
  for (int r = P - 1; r >= 1; --r) {
    for (int j = 0; j < P - 1; ++j) order_of[j] = j;
    std::stable_sort(order_of, order_of + P - 1, [&](int a, int b) { return fill[a] < fill[b]; });
    std::sort(order_of, order_of + r);  // the chosen launches, in launch order
    for (int k = 0; k < r; ++k) {
      launch_of[id(r, k)] = order_of[k];
      ++fill[order_of[k]];
    }
  }
  for (int r = 0; r < P; ++r) launch_of[id(r, r)] = P - 1;
  return P;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_version(void) { return "mla355 0.1 gfx950"; }

size_t mla_workspace_size(void) { return mla::kWorkspaceBytes; }

mla_status mla_fwd(const mla_rows* q, const mla_rows* q_rope, const mla_rows* kv,
                   const mla_rows* k_rope, const mla_rows* v, int32_t B, int32_t Hq,
                   int32_t Hkv, int64_t Nq, int64_t Nkv, int32_t dq, int32_t dr, int32_t dv,
                   const int32_t* seq_lens, int32_t n_seqs, float scale, uint32_t flags,
                   int64_t q_offset, int64_t kv_offset, const mla_rows* prev_out,
                   const mla_rows* prev_lse, const mla_rows* out, const mla_rows* lse,
                   void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla::AttnParams p;
  int form = FORM_EMPTY;
  if (mla_status st = prepare_fwd(q, q_rope, kv, k_rope, v, B, Hq, Hkv, Nq, Nkv, dq, dr, dv, seq_lens, n_seqs,
                                  scale, flags, q_offset, kv_offset, prev_out, prev_lse, out, lse, workspace,
                                  workspace_bytes, &p, &form))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (form == FORM_LATENT) return hip_status(mla::launch_latent_dense(p, s), "latent attention launch");
  if (form == FORM_SPLIT) return hip_status(mla::launch_split(p, s), "split attention launch");
  return MLA_OK;
}

mla_status mla_fwd_fp8(const mla_rows* q8, const mla_rows* kv8, int32_t B, int32_t Hq, int64_t Nq, int64_t Nkv,
                       int32_t dk, int32_t dv, float scale, float q_scale, float kv_scale, uint32_t flags,
                       int64_t q_offset, int64_t kv_offset, const mla_rows* out, const mla_rows* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st;
  if (B < 0 || Hq <= 0 || Nq < 0 || Nkv < 0)
    return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, Hq > 0, Nq >= 0, Nkv >= 0");
  if (dk != 576 || dv != 512)
    return fail(MLA_ERR_UNSUPPORTED, "the FP8 form is built for dk = 576 (512 latent + 64 RoPE), dv = 512 (got %d, %d)",
                dk, dv);
  if (flags & ~MLA_CAUSAL) return fail(MLA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~MLA_CAUSAL);
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARG, "scale must be finite");
  if (!(std::isfinite(q_scale) && q_scale > 0.f) || !(std::isfinite(kv_scale) && kv_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "q_scale and kv_scale must be finite and positive");
  if (!std::isfinite(scale * q_scale * kv_scale * kLog2e))
    return fail(MLA_ERR_INVALID_ARG, "scale * q_scale * kv_scale overflows float");
  if ((st = check_workspace(workspace, workspace_bytes))) return st;
  const bool no_q = B == 0 || Nq == 0, no_kv = B == 0 || Nkv == 0;
  // e4m3 rows: one byte per element, rows 16-byte aligned
  for (auto [r, name, empty] : {std::tuple{q8, "q8", no_q}, std::tuple{kv8, "kv8", no_kv}}) {
    if (!r) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
    if (!r->data && !empty) return fail(MLA_ERR_INVALID_ARG, "%s: missing", name);
    if (!aligned16(r->data)) return fail(MLA_ERR_INVALID_ARG, "%s: data pointer must be 16-byte aligned", name);
    if (r->stride_b < 0 || r->stride_h < 0 || r->stride_t < 0)
      return fail(MLA_ERR_INVALID_ARG, "%s: negative stride", name);
    if (r->stride_b % 16 || r->stride_h % 16 || r->stride_t % 16)
      return fail(MLA_ERR_INVALID_ARG, "%s: strides must be multiples of 16 bytes", name);
  }
  if ((st = check_rows(out, "out", true, no_q))) return st;
  if (lse && (st = check_lse(lse, "lse", no_q))) return st;
  if (kv8->stride_t > (1 << 24)) return fail(MLA_ERR_UNSUPPORTED, "kv8 rows must lie less than 16 MiB apart");
  const int64_t n_qblk = Nq / 32 + (Nq % 32 != 0), n_hgrp = (Hq + 3) / 4;
  if (!fits_grid({n_qblk, n_hgrp, B})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
  if (no_q) return MLA_OK;
  mla::AttnParams p{};
  p.qa = mla::RowsC{static_cast<const uint16_t*>(q8->data), q8->stride_b, q8->stride_h, q8->stride_t};
  p.ka = mla::RowsC{static_cast<const uint16_t*>(kv8->data), kv8->stride_b, kv8->stride_h, kv8->stride_t};
  p.out = rm(out);
  p.lse = lm(lse);
  p.B = B;
  p.Hq = Hq;
  p.group = Hq;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.q_offset = q_offset;
  p.kv_offset = kv_offset;
  p.scale_log2 = scale * q_scale * kv_scale * kLog2e;
  p.v_scale = kv_scale;
  p.causal = (flags & MLA_CAUSAL) ? 1 : 0;
  p.n_qblk = (int32_t)n_qblk;
  p.n_hgrp = (int32_t)n_hgrp;
  p.queue = static_cast<unsigned*>(workspace);
  return hip_status(mla::launch_latent_fp8(p, static_cast<hipStream_t>(stream)), "FP8 attention launch");
}

mla_status mla_fwd_group(int32_t n, const mla_fwd_call* calls, void* stream) {
  g_last_error.clear();
  mla::GroupParams g;
  if (mla_status st = prepare_group(n, calls, &g)) return st;
  if (g.n == 0) return MLA_OK;
  return hip_status(mla::launch_latent_group(g, static_cast<hipStream_t>(stream)), "group attention launch");
}

mla_status mla_ring_schedule(int32_t n_chunks, int32_t order, int32_t* launch_of, int32_t* n_launches) {
  g_last_error.clear();
  if (n_chunks < 1 || n_chunks > kMaxRingChunks)
    return fail(MLA_ERR_INVALID_ARG, "n_chunks (%d) must lie in [1, %d]", n_chunks, kMaxRingChunks);
  if (order != MLA_RING_ORDER && order != MLA_RING_BALANCED)
    return fail(MLA_ERR_INVALID_ARG, "order (%d) must be MLA_RING_ORDER or MLA_RING_BALANCED", order);
  if (!launch_of || !n_launches) return fail(MLA_ERR_INVALID_ARG, "launch_of and n_launches must be given");
  *n_launches = ring_schedule(n_chunks, order, launch_of);
  return MLA_OK;
}

size_t mla_ring_workspace_size(int32_t B, int32_t H, int64_t N, int32_t n_chunks) {
  if (B < 0 || H <= 0 || N < 0 || n_chunks < 1 || n_chunks > kMaxRingChunks) return 0;
  if (n_chunks == 1) return 0;
  const uint64_t C = (uint64_t)N / n_chunks + ((uint64_t)N % n_chunks != 0);  // chunk length (the last may be shorter)
  // the carry: per chunk, one block of 4 heads x 32 rows x 512 float32 per
  // work item (items of ceil(C / 32) row blocks x ceil(H / 4) head groups x B)
  uint64_t bytes = (uint64_t)B;
  for (uint64_t f : {((uint64_t)H + 3) / 4 * 4, (uint64_t)n_chunks, (C + 31) / 32 * 32, (uint64_t)kRingDv,
                     (uint64_t)sizeof(float)})
    if (__builtin_mul_overflow(bytes, f, &bytes)) return SIZE_MAX;  // no buffer can be that large
  if (bytes == 0) return 0;  // no rows: nothing is launched
  // the carry, then the item queue's counter (the carry is a multiple of 2 KB)
  if (__builtin_add_overflow(bytes, (uint64_t)kRingQueueBytes, &bytes) || bytes > (uint64_t)SIZE_MAX - 1)
    return SIZE_MAX;
  return (size_t)bytes;
}

mla_status mla_ring_fwd(const mla_rows* q, const mla_rows* kv, int32_t B, int32_t H, int64_t N, int32_t dq,
                        int32_t dv, float scale, int32_t n_chunks, int32_t order, const mla_rows* out,
                        const mla_rows* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B < 0 || H <= 0 || N < 0) return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, H > 0, N >= 0");
  if (n_chunks < 1 || n_chunks > kMaxRingChunks)
    return fail(MLA_ERR_INVALID_ARG, "n_chunks (%d) must lie in [1, %d]", n_chunks, kMaxRingChunks);
  if (order != MLA_RING_ORDER && order != MLA_RING_BALANCED)
    return fail(MLA_ERR_INVALID_ARG, "order (%d) must be MLA_RING_ORDER or MLA_RING_BALANCED", order);
  if (dq != 576 || dv != kRingDv)
    return fail(MLA_ERR_UNSUPPORTED, "the ring is built for dq = 576, dv = %d (got %d, %d)", kRingDv, dq, dv);
  if (!q || !kv || !out || !lse) return fail(MLA_ERR_INVALID_ARG, "q, kv, out and lse must be given");
  const size_t need = mla_ring_workspace_size(B, H, N, n_chunks);
  if (need && !workspace) return fail(MLA_ERR_INVALID_ARG, "the ring needs a workspace of mla_ring_workspace_size() bytes");
  if (need && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (need == SIZE_MAX) return fail(MLA_ERR_UNSUPPORTED, "the ring's workspace size overflows (N = %lld)", (long long)N);
  if (workspace_bytes < need)
    return fail(MLA_ERR_INVALID_ARG, "workspace_bytes (%zu) is below mla_ring_workspace_size() (%zu)", workspace_bytes, need);
  const int P = n_chunks;
  const int64_t C = (N + P - 1) / P;  // chunk r holds rows [r C, min((r + 1) C, N))
  auto len = [&](int r) { return std::max<int64_t>(0, std::min<int64_t>(C, N - r * C)); };
  int32_t launch_of[kMaxRingChunks * (kMaxRingChunks + 1) / 2];
  const int n_launches = ring_schedule(P, order, launch_of);

  // Views of every call (they must outlive the preparation below).  Query
  // chunk r's running result between its calls: the float32 slice r of the
  // workspace, [B, H, C, dv] contiguous.
  const int n_calls = P * (P + 1) / 2;
  std::vector<mla_rows> views(5 * (size_t)n_calls);
  std::vector<mla_fwd_call> calls(n_calls);
  std::vector<int> seen(P, 0);
  auto shift = [](const mla_rows* r, int64_t t0, int elem) {
    mla_rows v = *r;
    if (v.data) v.data = static_cast<char*>(v.data) + t0 * r->stride_t * elem;
    return v;
  };
  int ci = 0;
  for (int L = 0; L < n_launches; ++L)
    for (int r = 0; r < P; ++r)
      for (int k = 0; k <= r; ++k) {
        if (launch_of[r * (r + 1) / 2 + k] != L) continue;
        const bool first = seen[r] == 0, last = seen[r] == r;  // query chunk r makes r + 1 calls
        ++seen[r];
        mla_rows* v = &views[5 * (size_t)ci];
        v[0] = shift(q, r * C, 2);
        v[1] = shift(kv, k * C, 2);
        v[2] = shift(out, r * C, 2);
        v[3] = shift(lse, r * C, 4);
        float* carry_r = workspace ? static_cast<float*>(workspace) + (size_t)r * B * H * C * kRingDv : nullptr;
        v[4] = mla_rows{carry_r, (int64_t)H * C * kRingDv, C * kRingDv, kRingDv};
        mla_fwd_call& c = calls[ci];
        c = mla_fwd_call{};
        c.q = &v[0];
        c.kv = &v[1];
        c.B = B;
        c.Hq = H;
        c.Nq = len(r);
        c.Nkv = len(k);
        c.dq = dq;
        c.dr = 0;
        c.dv = dv;
        c.scale = scale;
        c.flags = MLA_CAUSAL | (last ? 0u : MLA_OUT_F32) | (first ? 0u : MLA_PREV_OUT_F32);
        c.q_offset = r * C;
        c.kv_offset = k * C;
        c.prev_out = first ? nullptr : &v[4];
        c.prev_lse = first ? nullptr : &v[3];
        c.out = last ? &v[2] : &v[4];
        c.lse = &v[3];
        ++ci;
      }
  // Validate every call before anything is launched.
  for (int i = 0; i < n_calls; i += MLA_MAX_GROUP) {
    mla::GroupParams g;
    if (mla_status st = prepare_group(std::min(MLA_MAX_GROUP, n_calls - i), &calls[i], &g)) return st;
  }
  if (B == 0 || N == 0) return MLA_OK;
  if (P == 1) {  // one call, no fold: a plain launch
    mla::GroupParams g;
    if (mla_status st = prepare_group(1, &calls[0], &g)) return st;
    if (g.n == 0) return MLA_OK;
    return hip_status(mla::launch_latent_group(g, static_cast<hipStream_t>(stream)), "ring launch");
  }

  // One launch for all the calls.  The base views are those of chunk 0's
  // only call (the kernel moves them to each call's chunks); each chunk's
  // calls fold in the order of their launch indices in the schedule.
  mla::RingParams rp{};
  {
    int form = FORM_EMPTY;
    if (mla_status st = prepare_fwd(q, nullptr, kv, nullptr, nullptr, B, H, 1, len(0), len(0), dq, 0, dv, nullptr, 0,
                                    scale, MLA_CAUSAL, 0, 0, nullptr, nullptr, out, lse, nullptr, 0, &rp.base, &form))
      return st;
  }
  rp.carry = static_cast<float*>(workspace);
  rp.queue = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + (need - kRingQueueBytes));
  rp.chunk_items = (C + 31) / 32 * (int64_t)rp.base.n_hgrp * B;
  rp.C = C;
  rp.N = N;
  rp.P = P;
  int64_t items = 0;
  for (int j = 0; j < P; ++j) {
    const int r = P - 1 - j;
    rp.chunk_first[j] = (int32_t)items;
    items += (len(r) + 31) / 32 * (int64_t)rp.base.n_hgrp * B;
    if (items > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "the ring has too many work items for one launch");
  }
  rp.chunk_first[P] = (int32_t)items;
  rp.n_items = (int32_t)items;
  for (int r = 0; r < P; ++r) {
    uint8_t* fk = rp.fold_k + r * (r + 1) / 2;
    for (int k = 0; k <= r; ++k) fk[k] = (uint8_t)k;
    std::stable_sort(fk, fk + r + 1, [&](uint8_t a, uint8_t b) {
      return launch_of[r * (r + 1) / 2 + a] < launch_of[r * (r + 1) / 2 + b];
    });
  }
  return hip_status(mla::launch_latent_ring(rp, static_cast<hipStream_t>(stream)), "ring launch");
}

mla_status mla_merge_lse(const mla_rows* out_a, const mla_rows* lse_a, const mla_rows* out_b,
                         const mla_rows* lse_b, int32_t B, int32_t H, int64_t N, int32_t dv,
                         const mla_rows* out, const mla_rows* lse, void* stream) {
  g_last_error.clear();
  mla_status st;
  if (B < 0 || H <= 0 || N < 0 || dv <= 0 || dv % 8)
    return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, H > 0, N >= 0, dv > 0 and a multiple of 8");
  const bool none = B == 0 || N == 0;  // no rows: the views may be NULL
  if ((st = check_rows(out_a, "out_a", true, none)) || (st = check_rows(out_b, "out_b", true, none)) ||
      (st = check_rows(out, "out", true, none)))
    return st;
  if ((st = check_lse(lse_a, "lse_a", none)) || (st = check_lse(lse_b, "lse_b", none))) return st;
  if (lse && (st = check_lse(lse, "lse", none))) return st;
  if (none) return MLA_OK;
  if ((out->data == out_a->data && !same_view(out, out_a)) || (out->data == out_b->data && !same_view(out, out_b)))
    return fail(MLA_ERR_INVALID_ARG, "out may alias out_a/out_b only as the identical view");
  if (lse && ((lse->data == lse_a->data && !same_view(lse, lse_a)) || (lse->data == lse_b->data && !same_view(lse, lse_b))))
    return fail(MLA_ERR_INVALID_ARG, "lse may alias lse_a/lse_b only as the identical view");
  if (!fits_grid({B, H, N / 4 + (N % 4 != 0)})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
  mla::MergeParams p{};
  p.oa = rc(out_a);
  p.ob = rc(out_b);
  p.la = lc(lse_a);
  p.lb = lc(lse_b);
  p.out = rm(out);
  p.lse = lm(lse);
  p.B = B;
  p.H = H;
  p.N = N;
  p.dv = dv;
  return hip_status(mla::launch_merge(p, static_cast<hipStream_t>(stream)), "merge launch");
}

mla_status mla_sparse_fwd(const mla_rows* q_lift, const mla_rows* q_pe, const mla_rows* c_kv,
                          const mla_rows* k_pe, const int32_t* topk_idx, int32_t B, int64_t S,
                          int64_t S_kv, int32_t H, int32_t L, int32_t R, int32_t K, float scale,
                          uint32_t flags, const mla_rows* out, const mla_rows* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st;
  if (B < 0 || S < 0 || S_kv <= 0 || H <= 0 || K <= 0)
    return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, S >= 0, S_kv > 0, H > 0, K > 0");
  if (L != 512 || R != 64) return fail(MLA_ERR_UNSUPPORTED, "sparse kernel is built for L = 512, R = 64 (got %d, %d)", L, R);
  if (H > 128) return fail(MLA_ERR_UNSUPPORTED, "sparse kernel handles up to 128 heads per query (got %d)", H);
  if (K > mla::kSparseMaxTopk)
    return fail(MLA_ERR_UNSUPPORTED, "sparse kernel handles up to %d indices per query (got %d)", mla::kSparseMaxTopk, K);
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARG, "scale must be finite");
  if (flags & ~(MLA_OUT_MX4 | MLA_OUT_F32))
    return fail(MLA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~(MLA_OUT_MX4 | MLA_OUT_F32));
  const bool out_f32 = flags & MLA_OUT_F32;
  if (out_f32 && (flags & MLA_OUT_MX4))
    return fail(MLA_ERR_UNSUPPORTED, "MLA_OUT_MX4 is built for bf16 output only (not with MLA_OUT_F32)");
  if ((st = check_workspace(workspace, workspace_bytes))) return st;
  const bool no_q = B == 0 || S == 0;  // no queries: the query-side views may be NULL
  if ((st = check_rows(q_lift, "q_lift", true, no_q)) || (st = check_rows(q_pe, "q_pe", true, no_q)) ||
      (st = out_f32 ? check_rows_f32(out, "out", no_q) : check_rows(out, "out", true, no_q)))
    return st;
  if ((st = check_rows(c_kv, "c_kv", false, B == 0)) || (st = check_rows(k_pe, "k_pe", false, B == 0))) return st;
  if ((!topk_idx && !no_q) || (reinterpret_cast<uintptr_t>(topk_idx) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "topk_idx: missing or not 4-byte aligned");
  if (lse && (st = check_lse(lse, "lse", no_q))) return st;
  if (no_q) return MLA_OK;
  if (!fits_grid({B, S})) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
  if (!fits_grid({S_kv, c_kv->stride_t, 2}) || !fits_grid({S_kv, k_pe->stride_t, 2}))
    return fail(MLA_ERR_UNSUPPORTED, "one batch of the cache must span less than 2 GiB (row offsets are 32-bit)");
  mla::AttnParams p{};
  p.qa = rc(q_lift);
  p.qb = rc(q_pe);
  p.ka = rc(c_kv);
  p.kb = rc(k_pe);
  p.out = rm(out);
  p.lse = lm(lse);
  p.idx = topk_idx;
  p.da = L;
  p.B = B;
  p.Hq = H;
  p.group = H;
  p.Nq = S;
  p.Nkv = S_kv;
  p.topk = K;
  p.scale_log2 = scale * kLog2e;
  p.mx4 = (flags & MLA_OUT_MX4) ? 1 : 0;
  p.out_f32 = out_f32 ? 1 : 0;
  p.queue = static_cast<unsigned*>(workspace);
  if (S == 0 || B == 0) return MLA_OK;
  return hip_status(mla::launch_latent_sparse(p, static_cast<hipStream_t>(stream)), "sparse attention launch");
}

size_t mla_decode_workspace_size(int32_t B, int32_t H, int64_t Nkv, int32_t n_splits) {
  int32_t S = 0, chunk = 0;
  if (B < 0 || H <= 0 || Nkv < 0 || n_splits < 0 || !decode_split(B, Nkv, n_splits, &S, &chunk)) return 0;
  size_t ol, oo;
  return decode_ws_bytes(B, H, S, 512, &ol, &oo);
}

}  // extern "C"

namespace {

// mla_decode_fwd with its workspace: `scratch` true when the workspace is the
// library's static one (mla_decode_fwd_noalloc), which bounds the sizes.
mla_status decode_fwd(const mla_rows* q, const mla_rows* q_rope, const mla_rows* kv, const mla_rows* k_rope,
                      const int32_t* kv_lens, const int32_t* kv_slots, int32_t n_slots, int32_t B, int32_t H,
                      int64_t Nkv, int32_t dq, int32_t dr, int32_t dv, float scale, int32_t n_splits,
                      const mla_rows* out, const mla_rows* lse, void* workspace, size_t workspace_bytes,
                      bool scratch, void* stream) {
  mla_status st;
  if (B < 0 || H <= 0 || Nkv < 0 || n_splits < 0)
    return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, H > 0, Nkv >= 0, n_splits >= 0");
  if (dq + dr != 576 || dv != 512 || !(dr == 0 || dr == 64))
    return fail(MLA_ERR_UNSUPPORTED, "decode is built for dq + dr = 576 (dr = 0 or 64), dv = 512 (got %d, %d, %d)",
                dq, dr, dv);
  if (H > 128) return fail(MLA_ERR_UNSUPPORTED, "decode handles up to 128 heads per sequence (got %d)", H);
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARG, "scale must be finite");
  if ((q_rope == nullptr) != (k_rope == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "q_rope and k_rope must both be given or both be NULL");
  if ((q_rope == nullptr) != (dr == 0))
    return fail(MLA_ERR_INVALID_ARG, "dr must be 0 exactly when q_rope/k_rope are NULL");
  // no sequences: every view may be NULL; no cache rows: the cache may be
  const bool no_b = B == 0, no_kv = B == 0 || Nkv == 0;
  if ((st = check_rows(q, "q", true, no_b)) || (st = check_rows(kv, "kv", false, no_kv)) ||
      (st = check_rows(out, "out", true, no_b)))
    return st;
  if (q_rope && ((st = check_rows(q_rope, "q_rope", true, no_b)) || (st = check_rows(k_rope, "k_rope", false, no_kv))))
    return st;
  if (lse && (st = check_lse(lse, "lse", no_b))) return st;
  if (kv_lens && (reinterpret_cast<uintptr_t>(kv_lens) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "kv_lens must be 4-byte aligned");
  if (kv_slots && (reinterpret_cast<uintptr_t>(kv_slots) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "kv_slots must be 4-byte aligned");
  if (kv_slots ? n_slots <= 0 : n_slots != 0 && n_slots < B)
    return fail(MLA_ERR_INVALID_ARG, "n_slots: need n_slots > 0 with kv_slots, else 0 or at least B");
  if (!fits_grid({Nkv, kv->stride_t, 2}) || (k_rope && !fits_grid({Nkv, k_rope->stride_t, 2})))
    return fail(MLA_ERR_UNSUPPORTED, "one sequence of the cache must span less than 2 GiB (row offsets are 32-bit)");
  int32_t S = 0, chunk = 0;
  if (!decode_split(B, Nkv, n_splits, &S, &chunk))
    return fail(n_splits > 0 ? MLA_ERR_INVALID_ARG : MLA_ERR_UNSUPPORTED,
                "no split of %lld rows fits (at most 64 splits of at most 2048 rows; n_splits = %d)",
                (long long)Nkv, n_splits);
  size_t off_l, off_o;
  const size_t need = decode_ws_bytes(B, H, S, dv, &off_l, &off_o);
  if ((int64_t)B * S > kMaxGrid) return fail(MLA_ERR_UNSUPPORTED, "problem too large for one launch");
  if (scratch) {
    if (need > mla::kDecodeScratchBytes)
      return fail(MLA_ERR_UNSUPPORTED,
                  "decode without allocation: %d sequences x %d heads x %d key ranges need %zu bytes of "
                  "partial results, above the library's %zu-byte device scratch (use mla_decode_fwd with a "
                  "workspace, or fewer sequences or ranges)",
                  B, H, S, need, (size_t)mla::kDecodeScratchBytes);
    if (B == 0) return MLA_OK;
    if ((st = hip_status(mla::decode_scratch(&workspace), "decode scratch lookup"))) return st;
    workspace_bytes = mla::kDecodeScratchBytes;
  } else {
    if (!workspace) return fail(MLA_ERR_INVALID_ARG, "decode needs a workspace of mla_decode_workspace_size() bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MLA_ERR_INVALID_ARG, "workspace_bytes (%zu) is below mla_decode_workspace_size() (%zu)",
                  workspace_bytes, need);
  }
  if (B == 0) return MLA_OK;

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* part_l = reinterpret_cast<float*>(ws + off_l);
  float* part_o = reinterpret_cast<float*>(ws + off_o);
  mla::AttnParams p{};
  // one query per sequence: the t stride is 0, so every split of a sequence
  // reads the same query row
  p.qa = mla::RowsC{static_cast<const uint16_t*>(q->data), q->stride_b, q->stride_h, 0};
  p.qb = q_rope ? mla::RowsC{static_cast<const uint16_t*>(q_rope->data), q_rope->stride_b, q_rope->stride_h, 0}
                : mla::RowsC{p.qa.p + (dq - 64), q->stride_b, q->stride_h, 0};
  p.ka = mla::RowsC{static_cast<const uint16_t*>(kv->data), kv->stride_b, 0, kv->stride_t};
  p.kb = k_rope ? mla::RowsC{static_cast<const uint16_t*>(k_rope->data), k_rope->stride_b, 0, k_rope->stride_t}
                : mla::RowsC{p.ka.p ? p.ka.p + (dq - 64) : nullptr, kv->stride_b, 0, kv->stride_t};
  p.da = dr == 0 ? dq - 64 : dq;
  p.B = B;
  p.Hq = H;
  p.group = H;
  p.Nq = S;        // the items of a sequence are its splits
  p.Nkv = Nkv;
  p.topk = chunk;
  p.scale_log2 = scale * kLog2e;
  p.decode = 1;
  p.kv_lens = kv_lens;
  p.kv_slots = kv_slots;
  p.n_slots = kv_slots ? n_slots : B;
  p.queue = reinterpret_cast<unsigned*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla::RowsM o_final{static_cast<uint16_t*>(out->data), out->stride_b, out->stride_h, 0};
  const mla::LseM l_final{lse ? static_cast<float*>(lse->data) : nullptr, lse ? lse->stride_b : 0,
                          lse ? lse->stride_h : 0, 0};
  if (S == 1) {
    p.out = o_final;
    p.lse = l_final;
    return hip_status(mla::launch_decode(p, B, s), "decode launch");
  }
  // split s of sequence b writes its fp32 partial at ((b * S + s) * H + h) * dv
  p.out = mla::RowsM{reinterpret_cast<uint16_t*>(part_o), (int64_t)S * H * dv, dv, (int64_t)H * dv};
  p.out_f32 = 1;
  p.lse = mla::LseM{part_l, (int64_t)S * H, 1, H};
  if ((st = hip_status(mla::launch_decode(p, (int64_t)B * S, s), "decode launch"))) return st;
  mla::CombineParams c{};
  c.po = part_o;
  c.pl = part_l;
  c.B = B;
  c.H = H;
  c.S = S;
  c.dv = dv;
  c.out = o_final;
  c.lse = l_final;
  return hip_status(mla::launch_combine(c, s), "decode combine launch");
}

}  // namespace

extern "C" {

mla_status mla_decode_fwd(const mla_rows* q, const mla_rows* q_rope, const mla_rows* kv,
                          const mla_rows* k_rope, const int32_t* kv_lens, const int32_t* kv_slots,
                          int32_t n_slots, int32_t B, int32_t H,
                          int64_t Nkv, int32_t dq, int32_t dr, int32_t dv, float scale,
                          int32_t n_splits, const mla_rows* out, const mla_rows* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return decode_fwd(q, q_rope, kv, k_rope, kv_lens, kv_slots, n_slots, B, H, Nkv, dq, dr, dv, scale, n_splits,
                    out, lse, workspace, workspace_bytes, false, stream);
}

mla_status mla_decode_fwd_noalloc(const mla_rows* q, const mla_rows* q_rope, const mla_rows* kv,
                                  const mla_rows* k_rope, const int32_t* kv_lens, const int32_t* kv_slots,
                                  int32_t n_slots, int32_t B, int32_t H,
                                  int64_t Nkv, int32_t dq, int32_t dr, int32_t dv, float scale,
                                  int32_t n_splits, const mla_rows* out, const mla_rows* lse, void* stream) {
  g_last_error.clear();
  return decode_fwd(q, q_rope, kv, k_rope, kv_lens, kv_slots, n_slots, B, H, Nkv, dq, dr, dv, scale, n_splits,
                    out, lse, nullptr, 0, true, stream);
}

mla_status mla_vup(const mla_rows* o, const void* w_uv, int32_t B, int32_t H, int64_t T, int32_t L, int32_t dvh,
                   uint32_t flags, const mla_rows* out, void* stream) {
  g_last_error.clear();
  mla_status st;
  if (B < 0 || H <= 0 || T < 0) return fail(MLA_ERR_INVALID_ARG, "sizes: need B >= 0, H > 0, T >= 0");
  if (L != 512 || dvh != 128)
    return fail(MLA_ERR_UNSUPPORTED, "V-up is built for L = 512, dvh = 128 (got %d, %d)", L, dvh);
  if (flags & ~MLA_OUT_MX4) return fail(MLA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~MLA_OUT_MX4);
  const bool none = B == 0 || T == 0;  // no rows: o and out may be NULL
  if ((st = check_rows(o, "o", true, none)) || (st = check_rows(out, "out", true, none))) return st;
  if (!w_uv || !aligned16(w_uv)) return fail(MLA_ERR_INVALID_ARG, "w_uv: missing or not 16-byte aligned");
  if (none) return MLA_OK;
  if ((int64_t)H * 512 > kMaxGrid) return fail(MLA_ERR_UNSUPPORTED, "too many heads for one launch");
  mla::VupParams p{};
  p.o = rc(o);
  p.w = static_cast<const uint16_t*>(w_uv);
  p.out = rm(out);
  p.B = B;
  p.H = H;
  p.T = T;
  p.mx4 = (flags & MLA_OUT_MX4) ? 1 : 0;
  return hip_status(mla::launch_vup(p, static_cast<hipStream_t>(stream)), "V-up launch");
}

mla_status mla_debug_gather(const mla_rows* c_kv, const mla_rows* k_pe, const int32_t* idx, int32_t b,
                            int64_t S_kv, int32_t L, int32_t R, int32_t K, uint16_t* rows_out,
                            void* stream) {
  g_last_error.clear();
  mla_status st;
  if (L != 512 || R != 64) return fail(MLA_ERR_UNSUPPORTED, "gather is built for L = 512, R = 64");
  if (b < 0 || S_kv <= 0 || K < 0) return fail(MLA_ERR_INVALID_ARG, "sizes: need b >= 0, S_kv > 0, K >= 0");
  if ((st = check_rows(c_kv, "c_kv", false)) || (st = check_rows(k_pe, "k_pe", false))) return st;
  if (!idx || (reinterpret_cast<uintptr_t>(idx) & 3u)) return fail(MLA_ERR_INVALID_ARG, "idx: missing or misaligned");
  if (!rows_out || !aligned16(rows_out)) return fail(MLA_ERR_INVALID_ARG, "rows_out: missing or not 16-byte aligned");
  if (!fits_grid({S_kv, c_kv->stride_t, 2}) || !fits_grid({S_kv, k_pe->stride_t, 2}))
    return fail(MLA_ERR_UNSUPPORTED, "one batch of the cache must span less than 2 GiB (row offsets are 32-bit)");
  mla::GatherParams p{};
  p.ka = rc(c_kv);
  p.kb = rc(k_pe);
  p.idx = idx;
  p.b = b;
  p.Nkv = S_kv;
  p.K = K;
  p.rows_out = rows_out;
  return hip_status(mla::launch_debug_gather(p, static_cast<hipStream_t>(stream)), "gather launch");
}

}  // extern "C"
