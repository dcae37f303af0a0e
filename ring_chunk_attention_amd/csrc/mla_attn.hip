// HIP kernels (gfx950) for shared-latent MLA attention forward, the split
// query/key ring step and the top-k sparse latent variant.
//
// What is computed (TT-NN ttnn.transformer.ring_mla, description; Ascend
// RingMLAOperation member table; NKI mla_sparse_attention_cte_kernel,
// "Parameters"): for every query row, softmax over the visible keys of
// scale * q.k, times V, plus the natural log-sum-exp of the scaled scores,
// optionally folded into a previous (out, LSE) pair (Ascend prevOut/prevLse).
//
// Design (one workgroup = 4 waves = 128 query rows, one wave per SIMD):
//  * Rows: 32 per wave, the MFMA N dimension.  In the shared-latent form the
//    four waves are four heads of the same 32 queries (all heads share the one
//    KV head), in the sparse form they are 128 heads of one query (all share
//    its index list), in the split form 128 queries of one head.  Either way
//    every key tile is fetched into LDS once per workgroup.
//  * Key tiles of 32 rows are fetched straight into LDS with buffer loads
//    (buffer_load_dwordx4 ... lds: no VGPR staging, 32-bit offsets, and the
//    buffer range check zero-fills rows past the end), double buffered.  A
//    tile is stored as two sub-tiles, the first DA columns and the last 64
//    (latent | RoPE, or nope | RoPE), each row's 16-byte chunks XOR-swizzled
//    so that both read patterns below are free of bank conflicts.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K fragments come from LDS,
//    the wave's Q rows stay in VGPRs for the whole key loop.  Transposing the
//    product puts one query row per lane (16 keys per lane, the other 16 in
//    lane +-32), so the row max and sum need one cross-half exchange.
//  * Softmax in base 2 against a per-row reference max fixed at the row's
//    first visible tile.  Numerator and denominator share the reference, so
//    the result is exact; it only has to stay within fp32 range, which holds
//    while no later score exceeds the reference by more than 2^30.  If one
//    does, the workgroup runs the key loop a second time with the exact row
//    max it has just seen.  The accumulators are therefore never rescaled
//    inside the loop and stay in AGPRs, written only by MFMA.
//  * P (bf16) is shared through LDS, and each wave accumulates O^T = V^T P^T
//    for all 128 rows over its own quarter of the V columns.  V fragments are
//    read from the key tile already in LDS (the value is the key row's
//    prefix) with ds_read_b64_tr_b16, which transposes 4x16 bf16 blocks on the
//    way from LDS, so one tile serves both products.  Sharing P cuts the V
//    traffic from LDS by 4x against each wave doing P.V for its own rows.
//  * Causal: tiles wholly in the future are never loaded; only tiles that cut
//    the diagonal (or the ragged end) are masked.  Workgroups are issued
//    longest-first.
//  * Epilogue: row stats are exchanged through LDS, the fold with the
//    previous (out, LSE) pair happens in fp32 before the single bf16 rounding.
#include "mla_internal.h"

#include <math.h>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int WAVES = 4;
constexpr int ROWS = 128;     // rows per workgroup
constexpr int BN = 32;        // keys per tile
constexpr int DB = 64;        // columns of the second (RoPE) part of a key row
constexpr float TAU = 30.0f;  // allowed growth of a row max over its reference, log2 units
constexpr float LN2 = 0.693147180559945309f;
constexpr unsigned kRsrcFlags = 0x00020000u;  // raw buffer resource word 3 on gfx9
constexpr unsigned kOob = 0x80000000u;        // offset past any valid record: reads zeros

enum Mode { LATENT = 0, SPLIT = 1, SPARSE = 2 };

struct LatentCfg {
  static constexpr int DA = 512, DV = 512;
  static constexpr bool VLAT = true;   // V = first DV columns of the key tile
};
struct SplitCfg {
  static constexpr int DA = 128, DV = 128;
  static constexpr bool VLAT = false;  // separate V tile
};

// Physical 16-byte chunk of logical chunk `c` in tile row `r`: the low three
// bits are XORed with f(r) = 2*(r%4) + (r/4)%2, a permutation of 0..7 over
// any 8 aligned rows (conflict-free 16-byte reads of 8 rows at one column)
// whose values over 4 aligned rows are all even or all odd (conflict-free
// 8-byte transposed reads of 4 rows x 32 bytes).
__device__ __forceinline__ int swz_f(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int swz(int c, int r) { return c ^ swz_f(r); }

template <class C>
struct Smem {
  static constexpr int AROWB = C::DA * 2;          // bytes per row, first part
  static constexpr int BROWB = DB * 2;             // bytes per row, RoPE part
  static constexpr int VROWB = C::DV * 2;
  static constexpr int ATILE = BN * AROWB, BTILE = BN * BROWB;
  static constexpr int VTILE = C::VLAT ? 16 : BN * VROWB;
  alignas(16) unsigned char a[2][ATILE];
  alignas(16) unsigned char b[2][BTILE];
  alignas(16) unsigned char v[2][VTILE];
  alignas(16) unsigned char p[WAVES][2][64 * 16];  // P^T fragments per wave, per 16-key half
  alignas(16) float wprev[ROWS];
  alignas(16) float wcur[ROWS];
  int redo;
};

__device__ __forceinline__ float xhalf_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float xhalf_sum(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcFlags);
}

// One wave-wide 16-byte-per-lane copy into LDS: lane l's 16 bytes at
// rsrc + voffset + soffset land at lds_base + 16*l.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds_base, uint32_t voffset,
                                            uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, (int)voffset, (int)soffset, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// V^T fragment (MFMA A operand, 32 value columns x 16 keys) for value-column
// block `db` (32 columns) and key half `c` (keys 16c..16c+15) of a tile whose
// rows are `rowb` bytes apart.  Lane l receives column 32*db + l%32 for the
// keys 16c + (j/4)*8 + 4*(l/32) + j%4, j = 0..7, which is the key order the
// S^T accumulator leaves in lane l.
__device__ __forceinline__ bf16x8 read_vt(const unsigned char* tile, int rowb, int db, int c, int lane) {
  const int g16 = lane >> 4, i = lane & 15;
  const int hh = g16 >> 1, dvh = g16 & 1, jr = i >> 2, cq = i & 3;
  const int col = 32 * db + 16 * dvh + 4 * cq;
  const int lc = col >> 3, within = (col & 7) * 2;
  const int key0 = 16 * c + 4 * hh + jr;
  const int key1 = key0 + 8;
  const unsigned char* a0 = tile + key0 * rowb + swz(lc, key0) * 16 + within;
  const unsigned char* a1 = tile + key1 * rowb + swz(lc, key1) * 16 + within;
  s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a0);
  s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a1);
  s16x8 x = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// Tile loader.  Wave w copies rows 8w..8w+7 of each sub-tile.  A sub-tile of
// `ch` 16-byte chunks per row is copied in 64-chunk wave instructions, so one
// instruction covers 64/ch rows; lane l handles chunk l % ch of row
// (64/ch)*i + l/ch and fetches the logical chunk that the swizzle places
// there.  `roff(r)` gives the byte offset of tile row r in its source buffer
// (kOob for a row that must read as zeros).
template <int CH, class RowOff>
__device__ __forceinline__ void load_subtile(__amdgpu_buffer_rsrc_t rs, unsigned char* tile, int w, int lane,
                                             RowOff roff) {
  constexpr int RPI = 64 / CH;       // rows per instruction
  constexpr int NI = 8 / RPI;        // instructions per wave (8 rows)
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = 8 * w + RPI * i + lane / CH;
    const int pc = lane % CH;
    const int lcn = swz(pc, r);
    const uint32_t ro = roff(r);
    const uint32_t off = ro == kOob ? kOob : ro + (uint32_t)lcn * 16u;
    copy_to_lds(rs, tile + (8 * w + RPI * i) * CH * 16, off, 0);
  }
}

// Per-workgroup context: which rows it owns and where keys come from.
struct Ctx {
  int b;
  int64_t kv_len;     // valid key rows
  int64_t kv_end;     // keys the workgroup visits: [0, kv_end)
  int64_t t0;         // first token of the sequence (split varlen)
  int64_t q_len;      // valid query rows of the sequence / batch
  int64_t q0;         // first query of the workgroup (latent/split), query index (sparse)
  int hbase;          // first head (latent), head (split)
};

template <class C, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_kernel(const AttnParams p) {
  constexpr int DA = C::DA, DV = C::DV;
  constexpr int DK = DA + DB;
  constexpr int KS = DK / 16;          // MFMA k-steps of Q.K
  constexpr int KSA = DA / 16;         // k-steps served by the first sub-tile
  constexpr int NDVB = DV / 32 / WAVES;  // 32-column value blocks per wave
  constexpr int AROWB = Smem<C>::AROWB, BROWB = Smem<C>::BROWB;
  static_assert(KS - KSA == 4, "second part is 64 columns");

  __shared__ Smem<C> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5, lr = lane & 31;

  // ---------------------------------------------------------------- rows
  Ctx cx;
  cx.t0 = 0;
  if constexpr (MODE == LATENT) {
    const int per = p.n_hgrp * p.B;
    const int id = blockIdx.x;
    const int qblk = p.n_qblk - 1 - id / per;  // longest causal rows first
    const int rem = id % per;
    cx.hbase = (rem % p.n_hgrp) * WAVES;
    cx.b = rem / p.n_hgrp;
    cx.q0 = (int64_t)qblk * 32;
    cx.q_len = p.Nq;
    cx.kv_len = p.Nkv;
    const int64_t last_q = min(p.Nq - 1, cx.q0 + 31);
    cx.kv_end = p.causal ? max<int64_t>(0, min<int64_t>(p.Nkv, p.q_offset + last_q - p.kv_offset + 1)) : p.Nkv;
  } else if constexpr (MODE == SPLIT) {
    const int id = blockIdx.x;
    cx.hbase = id % p.Hq;
    const int qb_lin = id / p.Hq;
    if (p.seq_lens) {
      int64_t cum = 0, t0 = 0, qb = 0, len = 0;
      bool found = false;
      for (int s = 0; s < p.n_seqs; ++s) {
        int64_t L = p.seq_lens[s];
        L = max<int64_t>(0, min<int64_t>(L, p.Nq - t0));
        const int64_t nb = (L + ROWS - 1) / ROWS;
        if (qb_lin < cum + nb) { found = true; qb = qb_lin - cum; len = L; break; }
        cum += nb;
        t0 += L;
      }
      if (!found) return;  // whole workgroup, before any barrier
      cx.b = 0;
      cx.t0 = t0;
      cx.q_len = len;
      cx.kv_len = len;
      cx.q0 = qb * ROWS;
    } else {
      const int64_t nb = (p.Nq + ROWS - 1) / ROWS;
      cx.b = (int)(qb_lin / nb);
      cx.q0 = (nb - 1 - qb_lin % nb) * ROWS;  // longest causal rows first
      cx.q_len = p.Nq;
      cx.kv_len = p.Nkv;
    }
    const int64_t last_q = min(cx.q_len - 1, cx.q0 + ROWS - 1);
    cx.kv_end = p.causal ? max<int64_t>(0, min<int64_t>(cx.kv_len, p.q_offset + last_q - p.kv_offset + 1)) : cx.kv_len;
  } else {  // SPARSE
    const int64_t id = blockIdx.x;
    cx.b = (int)(id / p.Nq);
    cx.q0 = id % p.Nq;
    cx.hbase = 0;
    cx.q_len = p.Nq;
    cx.kv_len = p.topk;
    cx.kv_end = p.topk;
  }

  auto row_head = [&](int rb) -> int {
    if constexpr (MODE == LATENT) return cx.hbase + rb;
    else if constexpr (MODE == SPLIT) return cx.hbase;
    else return rb * 32 + lr;
  };
  auto row_query = [&](int rb) -> int64_t {
    if constexpr (MODE == LATENT) return cx.q0 + lr;
    else if constexpr (MODE == SPLIT) return cx.q0 + rb * 32 + lr;
    else return cx.q0;
  };
  auto row_valid = [&](int rb) -> bool { return row_head(rb) < p.Hq && row_query(rb) < cx.q_len; };
  auto qtok = [&](int64_t q) -> int64_t { return cx.t0 + q; };

  // ------------------------------------------------------------ Q -> VGPR
  bf16x8 qf[KS];
  {
    const int hq = row_head(w) < p.Hq ? row_head(w) : 0;
    const int64_t t = qtok(row_query(w) < cx.q_len ? row_query(w) : 0);
    const uint16_t* ra = p.qa.p + cx.b * p.qa.sb + hq * p.qa.sh + t * p.qa.st;
    const uint16_t* rb = p.qb.p + cx.b * p.qb.sb + hq * p.qb.sh + t * p.qb.st;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const int d = 16 * c + 8 * h;
      qf[c] = c < KSA ? load16(ra + d) : load16(rb + (d - DA));
    }
  }

  // ---------------------------------------------------------- key sources
  const int kvh = (MODE == SPARSE) ? 0 : row_head(0) / p.group;
  const uint16_t* kA = p.ka.p + cx.b * p.ka.sb + (int64_t)kvh * p.ka.sh + cx.t0 * p.ka.st;
  const uint16_t* kB = p.kb.p + cx.b * p.kb.sb + (int64_t)kvh * p.kb.sh + cx.t0 * p.kb.st;
  const uint16_t* vS = C::VLAT ? kA : p.v.p + cx.b * p.v.sb + (int64_t)kvh * p.v.sh + cx.t0 * p.v.st;
  const uint32_t stA = (uint32_t)(p.ka.st * 2), stB = (uint32_t)(p.kb.st * 2), stV = (uint32_t)(p.v.st * 2);
  const int32_t* idx_row = (MODE == SPARSE) ? p.idx + ((int64_t)cx.b * p.Nq + cx.q0) * p.topk : nullptr;

  // sparse: this lane's entry (row lr) of the index list of tile t
  auto load_idx = [&](int t) -> int {
    const int64_t k = (int64_t)t * BN + lr;
    return k < p.topk ? idx_row[k] : -1;
  };
  auto idx_ok = [&](int r) -> bool { return r >= 0 && r < p.Nkv; };

  auto issue_tile = [&](int t, int buf, int idx_lane) {
    const int64_t k0 = (int64_t)t * BN;
    if constexpr (MODE == SPARSE) {
      // the whole cache is the buffer; a row's offset comes from its index
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(kA, (uint32_t)(p.Nkv * stA));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(kB, (uint32_t)(p.Nkv * stB));
      auto roffA = [&](int r) -> uint32_t {
        const int ix = __builtin_amdgcn_readlane(idx_lane, r);
        return idx_ok(ix) ? (uint32_t)ix * stA : kOob;
      };
      auto roffB = [&](int r) -> uint32_t {
        const int ix = __shfl(idx_lane, r);
        return idx_ok(ix) ? (uint32_t)ix * stB : kOob;
      };
      load_subtile<DA / 8>(ra, sm.a[buf], w, lane, roffA);
      load_subtile<DB / 8>(rb, sm.b[buf], w, lane, roffB);
    } else {
      // the buffer is the tile's rows [k0, min(k0 + BN, kv_len)); rows past it read zeros
      const int64_t nrows = min<int64_t>(BN, cx.kv_len - k0);
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(kA + k0 * p.ka.st, (uint32_t)(nrows * stA));
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(kB + k0 * p.kb.st, (uint32_t)(nrows * stB));
      load_subtile<DA / 8>(ra, sm.a[buf], w, lane, [&](int r) -> uint32_t { return (uint32_t)r * stA; });
      load_subtile<DB / 8>(rb, sm.b[buf], w, lane, [&](int r) -> uint32_t { return (uint32_t)r * stB; });
      if constexpr (!C::VLAT) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vS + k0 * p.v.st, (uint32_t)(nrows * stV));
        load_subtile<DV / 8>(rv, sm.v[buf], w, lane, [&](int r) -> uint32_t { return (uint32_t)r * stV; });
      }
    }
  };

  // LDS byte offsets of this lane's K fragments
  const int f_lr = swz_f(lr);
  int koffA[4], koffB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    koffA[j] = lr * AROWB + (((2 * j + h) ^ f_lr) * 16);
    koffB[j] = lr * BROWB + (((2 * j + h) ^ f_lr) * 16);
  }

  const int n_tiles = (int)((cx.kv_end + BN - 1) / BN);
  const int64_t my_qpos = p.q_offset + row_query(w);          // causal position of this lane's row
  const int64_t wave_min_qpos = p.q_offset + row_query(w) - lr;  // smallest position of the wave's rows

  f32x16 O[WAVES][NDVB];
  float m_ref = -INFINITY;  // reference max of this lane's row (log2 units)
  float m_run = -INFINITY;  // running exact max
  float l_part = 0.f;       // this lane's share of the row sum, relative to m_ref
  float l_rnd = 0.f;        // the same over the bf16-rounded weights
  if (tid == 0) sm.redo = 0;

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!sm.redo) break;   // workgroup-uniform: read after a barrier
      m_ref = m_run;         // exact row max: every weight is <= 1
      l_part = 0.f;
      l_rnd = 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < WAVES; ++rb)
#pragma unroll
      for (int j = 0; j < NDVB; ++j) O[rb][j] = f32x16{};

    int idx_cur = -1, idx_nxt = -1;
    if (n_tiles > 0) {
      if constexpr (MODE == SPARSE) {
        idx_cur = load_idx(0);
        idx_nxt = n_tiles > 1 ? load_idx(1) : -1;
        wait_vmem();
      }
      issue_tile(0, 0, idx_cur);
      wait_vmem();
    }
    __syncthreads();

    bool over = false;
    for (int t = 0; t < n_tiles; ++t) {
      const int buf = t & 1;
      int idx_nn = -1;
      if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1, idx_nxt);
      if constexpr (MODE == SPARSE) {
        if (t + 2 < n_tiles) idx_nn = load_idx(t + 2);
      }
      const int64_t k0 = (int64_t)t * BN;

      // S^T = K Q^T  (lane: query row lr; keys (r/4)*8 + 4h + r%4)
      f32x16 s = f32x16{};
      const unsigned char* ta = sm.a[buf];
      const unsigned char* tb = sm.b[buf];
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const bf16x8 kf = c < KSA
            ? *reinterpret_cast<const bf16x8*>(ta + koffA[c & 3] + (c >> 2) * 128)
            : *reinterpret_cast<const bf16x8*>(tb + koffB[c - KSA]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s, 0, 0, 0);
      }

      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * p.scale_log2;

      bool need_mask;
      unsigned vbits = 0xffffffffu;
      if constexpr (MODE == SPARSE) {
        vbits = (unsigned)__ballot(idx_ok(idx_cur));
        need_mask = vbits != 0xffffffffu;
      } else {
        need_mask = (k0 + BN > cx.kv_len) || (p.causal && p.kv_offset + k0 + BN - 1 > wave_min_qpos);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = (r >> 2) * 8 + 4 * h + (r & 3);
          bool ok;
          if constexpr (MODE == SPARSE) {
            ok = (vbits >> kk) & 1u;
          } else {
            const int64_t key = k0 + kk;
            ok = key < cx.kv_len && (!p.causal || p.kv_offset + key <= my_qpos);
          }
          x[r] = ok ? x[r] : -INFINITY;
        }
      }

      float mt = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
      mt = xhalf_max(mt);
      m_run = fmaxf(m_run, mt);
      if (m_ref == -INFINITY) m_ref = mt;        // the row's first visible tile (pass 0)
      over |= m_run > m_ref + TAU;
      const float mu = m_ref == -INFINITY ? 0.f : m_ref;
      f32x8 p0, p1;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p0[r] = __builtin_amdgcn_exp2f(x[r] - mu);
        p1[r] = __builtin_amdgcn_exp2f(x[r + 8] - mu);
      }
      const bf16x8 b0 = __builtin_convertvector(p0, bf16x8);
      const bf16x8 b1 = __builtin_convertvector(p1, bf16x8);
      // two row sums: the exact one gives the LSE; the one of the weights as
      // the P.V product sees them (rounded to bf16) normalises O, so that its
      // weights sum to one
      float ps = 0.f, pr = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ps += p0[r] + p1[r];
        pr += (float)b0[r] + (float)b1[r];
      }
      l_part += ps;
      l_rnd += pr;

      *reinterpret_cast<bf16x8*>(sm.p[w][0] + lane * 16) = b0;
      *reinterpret_cast<bf16x8*>(sm.p[w][1] + lane * 16) = b1;
      __syncthreads();

      // O^T += V^T P^T over this wave's value columns for all 128 rows
      const unsigned char* vt = C::VLAT ? sm.a[buf] : sm.v[buf];
      constexpr int VROWB = C::VLAT ? AROWB : Smem<C>::VROWB;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pb[WAVES];
#pragma unroll
        for (int rb = 0; rb < WAVES; ++rb) pb[rb] = *reinterpret_cast<const bf16x8*>(sm.p[rb][c] + lane * 16);
#pragma unroll
        for (int j = 0; j < NDVB; ++j) {
          const bf16x8 vf = read_vt(vt, VROWB, w * NDVB + j, c, lane);
#pragma unroll
          for (int rb = 0; rb < WAVES; ++rb)
            O[rb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[rb], O[rb][j], 0, 0, 0);
        }
      }
      wait_vmem();
      __syncthreads();
      idx_cur = idx_nxt;
      idx_nxt = idx_nn;
    }
    if (pass == 0) {
      if (__ballot(over) != 0ull && lane == 0) sm.redo = 1;
      __syncthreads();
    }
  }

  // ------------------------------------------------------------- epilogue
  {
    const float l_row = xhalf_sum(l_part);
    const float l_row_rnd = xhalf_sum(l_rnd);
    const float lse_cur = l_row > 0.f ? (m_ref + log2f(l_row)) * LN2 : -INFINITY;
    const float inv = l_row_rnd > 0.f ? 1.f / l_row_rnd : 0.f;
    const bool ok = row_valid(w);
    float lp = -INFINITY;
    const int hq = row_head(w);
    const int64_t tq = qtok(row_query(w));
    if (p.prev_lse.p && ok) lp = p.prev_lse.p[cx.b * p.prev_lse.sb + hq * p.prev_lse.sh + tq * p.prev_lse.st];
    const float mx = fmaxf(lp, lse_cur);
    float L, wp, wc;
    if (mx == -INFINITY) {
      L = -INFINITY; wp = 0.f; wc = 0.f;
    } else {
      const float ea = lp == -INFINITY ? 0.f : expf(lp - mx);
      const float eb = lse_cur == -INFINITY ? 0.f : expf(lse_cur - mx);
      const float z = ea + eb;
      L = mx + logf(z);
      wp = ea / z;
      wc = eb / z * inv;
    }
    if (h == 0) {
      sm.wprev[w * 32 + lr] = wp;
      sm.wcur[w * 32 + lr] = wc;
      if (p.lse.p && ok) p.lse.p[cx.b * p.lse.sb + hq * p.lse.sh + tq * p.lse.st] = L;
    }
  }
  __syncthreads();

#pragma unroll
  for (int rb = 0; rb < WAVES; ++rb) {
    if (!row_valid(rb)) continue;
    const float wp = sm.wprev[rb * 32 + lr];
    const float wc = sm.wcur[rb * 32 + lr];
    const int hq = row_head(rb);
    const int64_t tq = qtok(row_query(rb));
    const int64_t oel = cx.b * p.out.sb + hq * p.out.sh + tq * p.out.st;
    const int64_t pel = cx.b * p.prev_out.sb + hq * p.prev_out.sh + tq * p.prev_out.st;
    const bool fold = p.prev_out.p && wp != 0.f;
#pragma unroll
    for (int j = 0; j < NDVB; ++j) {
      const int dvb = 32 * (w * NDVB + j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dvb + 8 * g + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = wc * O[rb][j][4 * g + e];
        if (fold) {
          if (p.prev_f32) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.prev_out.p) + pel + d);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] += wp * pv[e];
          } else {
            const u32x2 pv = *reinterpret_cast<const u32x2*>(p.prev_out.p + pel + d);
            y[0] += wp * __uint_as_float(pv[0] << 16);
            y[1] += wp * __uint_as_float(pv[0] & 0xffff0000u);
            y[2] += wp * __uint_as_float(pv[1] << 16);
            y[3] += wp * __uint_as_float(pv[1] & 0xffff0000u);
          }
        }
        if (p.out_f32) {
          const f32x4 st = {y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out.p) + oel + d) = st;
        } else {
          const u32x2 st = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<u32x2*>(p.out.p + oel + d) = st;
        }
      }
    }
  }
}

// Debug gather: one workgroup stages the listed rows tile by tile through the
// same swizzled buffer->LDS copy as the sparse kernel and writes them back in
// natural order.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void debug_gather_kernel(const GatherParams p) {
  constexpr int DA = 512;
  __shared__ alignas(16) unsigned char ta[BN * DA * 2];
  __shared__ alignas(16) unsigned char tb[BN * DB * 2];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31;
  const uint16_t* kA = p.ka.p + p.b * p.ka.sb;
  const uint16_t* kB = p.kb.p + p.b * p.kb.sb;
  const uint32_t stA = (uint32_t)(p.ka.st * 2), stB = (uint32_t)(p.kb.st * 2);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(kA, (uint32_t)(p.Nkv * stA));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(kB, (uint32_t)(p.Nkv * stB));
  const int n_tiles = (p.K + BN - 1) / BN;
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN;
    const int ix = (k0 + lr < p.K) ? p.idx[k0 + lr] : -1;
    auto ok = [&](int r) { return r >= 0 && r < p.Nkv; };
    load_subtile<DA / 8>(ra, ta, w, lane, [&](int r) -> uint32_t {
      const int v = __builtin_amdgcn_readlane(ix, r);
      return ok(v) ? (uint32_t)v * stA : kOob;
    });
    load_subtile<DB / 8>(rb, tb, w, lane, [&](int r) -> uint32_t {
      const int v = __shfl(ix, r);
      return ok(v) ? (uint32_t)v * stB : kOob;
    });
    wait_vmem();
    __syncthreads();
    for (int e = tid; e < BN * (DA + DB) / 8; e += 256) {
      const int r = e / ((DA + DB) / 8), c = e % ((DA + DB) / 8);
      if (k0 + r >= p.K) continue;
      const u32x4 val = c < DA / 8 ? *reinterpret_cast<const u32x4*>(ta + r * DA * 2 + swz(c, r) * 16)
                                   : *reinterpret_cast<const u32x4*>(tb + r * DB * 2 + swz(c - DA / 8, r) * 16);
      *reinterpret_cast<u32x4*>(p.rows_out + (int64_t)(k0 + r) * (DA + DB) + c * 8) = val;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_latent_dense(const AttnParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.n_qblk * p.n_hgrp * p.B;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<LatentCfg, LATENT>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_latent_sparse(const AttnParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.Nq;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<LatentCfg, SPARSE>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_split(const AttnParams& p, hipStream_t s) {
  int64_t qblocks;
  if (p.seq_lens) qblocks = (p.Nq + ROWS - 1) / ROWS + p.n_seqs;  // upper bound; extra groups exit
  else qblocks = (p.Nq + ROWS - 1) / ROWS * p.B;
  const int64_t blocks = qblocks * p.Hq;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<SplitCfg, SPLIT>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_debug_gather(const GatherParams& p, hipStream_t s) {
  if (p.K == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
