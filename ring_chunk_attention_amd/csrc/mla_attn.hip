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

#include <atomic>
#include <utility>

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

// SPARSE: top-k lists up to 4096 entries, beside-P.V softmax loop;
// SPARSE_PIPE: lists up to 2048 entries, the tile-step loop of the latent form
enum Mode { LATENT = 0, SPLIT = 1, SPARSE = 2, SPARSE_PIPE = 3 };
constexpr int KMAX_IDX_PIPE = 2048;

struct LatentCfg {
  static constexpr int DA = 512, DV = 512;
  static constexpr bool VLAT = true;   // V = first DV columns of the key tile
};
struct SplitCfg {
  static constexpr int DA = 128, DV = 128;
  static constexpr bool VLAT = false;  // separate V tile
};

// Row swizzle of the LDS tiles: logical 16-byte chunk c of tile row r sits at
// position c ^ g(r) within its 128-byte group, with g(r) = 4*((r/2)%2) +
// (r/4)%4.  The LDS has 64 four-byte banks and serves 16 lanes of a 16-byte
// read per cycle.  Over any 16 aligned rows, g is a permutation of 0..7 on the
// even rows and on the odd rows, so 16 rows read at one column fall on 16
// distinct 16-byte bank groups (rows of a block are 128 bytes apart, so even
// and odd rows use opposite halves of the 256-byte bank window); and within 4
// aligned rows the two rows of equal parity differ in bit 2, so the 8-byte
// transposed reads of 4 rows x 32 bytes are conflict-free as well.
__device__ __forceinline__ int swz_f(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

constexpr int KMAX_IDX = kSparseMaxTopk;  // sparse: longest index list staged in LDS

// Sub-tile layout.  A sub-tile with NG 64-column groups per row is stored as
// blocks of 8 rows x 8 chunks (16 bytes each) = 1 KB: block (r/8, g) at byte
// ((r/8)*NG + g)*1024, row r%8 at +128*(r%8), and logical chunk q of group g
// at position (q%8) ^ f(r%8).  One wave instruction of a global->LDS copy
// fills one block, so every lane's source offset is the same for all groups
// and tiles, and the instruction offset selects the group.
__device__ __forceinline__ int tile_off(int NG, int r, int q) {
  return (((r >> 3) * NG + (q >> 3)) << 10) + ((r & 7) << 7) + (((q & 7) ^ swz_f(r & 15)) << 4);
}

// NB buffers for the first sub-tile (and V), NBB for the 64-column one, which
// only the Q.K chain reads; KIDX entries of the sparse index list
template <class C, int NB, int NBB, int KIDX>
struct Smem {
  static constexpr int ATILE = BN * C::DA * 2, BTILE = BN * DB * 2;
  static constexpr int VTILE = C::VLAT ? 0 : BN * C::DV * 2;
  // 1 KB aligned (the tiles are multiples of 1 KB): a fragment address
  // differs from its k-step-0 neighbour only in bits 5-6 (see frag_addrs)
  alignas(1024) unsigned char a[NB][ATILE];
  alignas(1024) unsigned char b[NBB][BTILE];
  alignas(16) unsigned char v[NB][VTILE];
  alignas(16) int idx[KIDX];                          // sparse: the query's index list
  union {
    alignas(16) unsigned char p[2][WAVES][2][64 * 16];  // P^T fragments: buffer, wave, 16-key half
    struct {                                            // after the key loop
      float wprev[ROWS];
      float wcur[ROWS];
      int flag[WAVES];
      int item;                                         // the work item (with a queue)
    } epi;
  };
};

// Combine lane l with lane l^32: v_permlane32_swap exchanges the upper half
// of one register with the lower half of another; with both operands equal
// to x the two results hold x and its partner value in either order.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Raw buffer resource (4 scalar words) over `bytes` bytes at `base`: stride
// 0, so an offset at or past `bytes` is out of range and reads zeros.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcFlags;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// One wave-wide copy into LDS (buffer_load_dwordx4 ... lds): lane l's 16 bytes
// at rsrc + voffset + IMM land at lds_base + 16*l.  The LDS address is M0 +
// IMM + 16*l (the immediate offset applies to both sides), so M0 is set to
// lds_base - IMM; the nop covers the M0 write -> LDS-DMA read hazard.  The
// copy is issued from asm so that the compiler does not make later LDS reads
// of the other tile buffers wait for it: the kernel waits for its copies
// itself (vmcnt) before the barrier that publishes a tile.  M0 is a reserved
// register, so the asm restores it.
template <int IMM>
__device__ __forceinline__ void copy_to_lds(const u32x4& r, uint32_t lds, uint32_t voffset) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n"
      "s_mov_b32 m0, %[m0]\n"
      "s_nop 0\n"
      "buffer_load_dwordx4 %[vo], %[rs], 0 offen offset:%[imm] lds\n"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [m0] "s"(lds - IMM), [vo] "v"(voffset), [rs] "s"(r), [imm] "n"(IMM)
      : "memory");
}

// Copy column groups [G0, G1) of a block row (8 rows x NG column groups) of a
// sub-tile at LDS byte address `tile`: one instruction per column group.
template <int NG, int G0 = 0, int G1 = NG>
__device__ __forceinline__ void copy_rows(const u32x4& r, uint32_t tile, int w, uint32_t voffset) {
#pragma unroll
  for (int g = G0; g < G1; ++g) {
    const uint32_t dst = tile + (uint32_t)(w * NG + g) * 1024u;
    switch (g) {  // the group offset is an instruction immediate
      case 0: copy_to_lds<0>(r, dst, voffset); break;
      case 1: copy_to_lds<128>(r, dst, voffset); break;
      case 2: copy_to_lds<256>(r, dst, voffset); break;
      case 3: copy_to_lds<384>(r, dst, voffset); break;
      case 4: copy_to_lds<512>(r, dst, voffset); break;
      case 5: copy_to_lds<640>(r, dst, voffset); break;
      case 6: copy_to_lds<768>(r, dst, voffset); break;
      default: copy_to_lds<896>(r, dst, voffset); break;
    }
  }
}

#include "mla_qk_chain.inc"

// f(integral_constant<int, I>) for I = 0..N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wait until at most `tiles` tiles' copies (KI copy instructions each, issued
// by this wave) are in flight; loads complete in order.
template <int KI>
__device__ __forceinline__ void wait_tiles(int tiles) {
  if (tiles <= 0) wait_vmem_n<0>();
  else if (tiles == 1) wait_vmem_n<KI>();
  else wait_vmem_n<2 * KI>();
}

// Byte offset, within a sub-tile with NG column groups, of the first of the two
// transposed reads read_vt makes for value block db and key half c (half 0)
// or of the second (half 1).
template <int NG>
__device__ __forceinline__ uint32_t vt_off(int db, int c, int lane, int half) {
  const int g16 = lane >> 4, i = lane & 15;
  const int hh = g16 >> 1, dvh = g16 & 1, jr = i >> 2, cq = i & 3;
  const int col = 32 * db + 16 * dvh + 4 * cq;
  const int key0 = 16 * c + 4 * hh + jr + 8 * half;
  return (uint32_t)(tile_off(NG, key0, col >> 3) + (col & 7) * 2);
}

// V^T fragment (MFMA A operand, 32 value columns x 16 keys) for value-column
// block `db` (32 columns) and key half `c` (keys 16c..16c+15) of a sub-tile
// with NG column groups.  Lane l receives column 32*db + l%32 for the keys
// 16c + (j/4)*8 + 4*(l/32) + j%4, j = 0..7, the key order the S^T
// accumulator leaves in lane l.
template <int NG>
__device__ __forceinline__ bf16x8 read_vt(const unsigned char* tile, int db, int c, int lane) {
  const int g16 = lane >> 4, i = lane & 15;
  const int hh = g16 >> 1, dvh = g16 & 1, jr = i >> 2, cq = i & 3;
  const int col = 32 * db + 16 * dvh + 4 * cq;
  const int key0 = 16 * c + 4 * hh + jr;
  const unsigned char* a0 = tile + tile_off(NG, key0, col >> 3) + (col & 7) * 2;
  const unsigned char* a1 = tile + tile_off(NG, key0 + 8, col >> 3) + (col & 7) * 2;
  s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a0);
  s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a1);
  s16x8 x = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  return __builtin_bit_cast(bf16x8, x);
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

// The latent and sparse forms use the whole register file and LDS of a CU
// (one workgroup per CU); the split form needs about 200 registers and, with
// three tile buffers, 76 KB of LDS, so two of its workgroups share a CU and
// each hides the other's waits.
template <int MODE>
constexpr int kWavesPerEU = MODE == 1 ? 2 : 1;

template <class C, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, kWavesPerEU<MODE>)))
void attn_fwd_kernel(const AttnParams p) {
  constexpr bool SP = MODE == SPARSE || MODE == SPARSE_PIPE;
  constexpr int DA = C::DA, DV = C::DV;
  constexpr int DK = DA + DB;
  constexpr int KS = DK / 16;            // MFMA k-steps of Q.K
  constexpr int KSA = DA / 16;           // k-steps served by the first sub-tile
  constexpr int NGA = DA / 64;           // column groups of the first sub-tile
  constexpr int NGV = C::VLAT ? NGA : DV / 64;
  constexpr int NDVB = DV / 32 / WAVES;  // 32-column value blocks per wave
  constexpr int KI = NGA + 1 + (C::VLAT ? 0 : NGV);  // copy instructions per wave per tile
  // the latent form (and the sparse one for lists up to 2048) runs the
  // softmax of tile t+1 inside the Q.K chain of tile t+2 (see the main
  // loop) with four key-tile buffers; the others compute it beside P.V with
  // three (the sparse form keeps its index list in LDS instead of a fourth)
  constexpr bool SM_IN_QK = MODE == LATENT || MODE == SPARSE_PIPE;
  constexpr int NB = SM_IN_QK ? 4 : 3;
  // 64-column sub-tile buffers: only the Q.K chain reads them, so two are
  // enough in the tile-step loop (the one being read and the one in flight);
  // the pipelined sparse form needs that room for its index list
  constexpr int NBB = MODE == SPARSE_PIPE ? 2 : NB;
  constexpr int KIDX = MODE == SPARSE ? KMAX_IDX : MODE == SPARSE_PIPE ? KMAX_IDX_PIPE : 0;
  using SM = Smem<C, NB, NBB, KIDX>;
  static_assert(KS - KSA == 4, "second part is 64 columns");
  static_assert(NB - 2 <= 2, "wait_tiles covers at most two tiles in flight");

  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, h = lane >> 5, lr = lane & 31;  // (recomputed past the key loop)
  __builtin_assume(w >= 0 && w < WAVES);

  // ---------------------------------------------------------------- rows
  // Work item: latent, a block of 32 query rows of WAVES heads, longest
  // causal rows first; sparse, one query with all its heads.  With a queue
  // the workgroup takes the next item from a device counter instead of its
  // own index.  The hardware hands the workgroups of a launch to the XCDs in
  // equal shares, whatever their clocks; through the counter a faster XCD
  // also takes items sooner, and so the longer ones, and all finish
  // together.
  int64_t item = blockIdx.x;
  if constexpr (MODE == LATENT || MODE == SPARSE_PIPE) {
    if (p.queue) {
      if (tid == 0) sm.epi.item = (int)atomicAdd(p.queue, 1u);
      __syncthreads();
      item = sm.epi.item;  // (P, which shares this space, is first written past a barrier)
    }
  }
  Ctx cx;
  cx.t0 = 0;
  if constexpr (MODE == LATENT) {
    const int per = p.n_hgrp * p.B;
    const int id = (int)item;
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
    const int64_t id = item;
    cx.b = (int)(id / p.Nq);
    cx.q0 = id % p.Nq;
    cx.hbase = 0;
    cx.q_len = p.Nq;
    cx.kv_len = p.topk;
    cx.kv_end = p.topk;
    if (p.decode) {  // the part of split q0's range inside the valid rows
      int64_t len = p.kv_lens ? (int64_t)p.kv_lens[cx.b] : p.Nkv;
      len = max<int64_t>(0, min<int64_t>(len, p.Nkv));
      cx.kv_len = cx.kv_end = max<int64_t>(0, min<int64_t>(p.topk, len - cx.q0 * p.topk));
    }
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
  const int kvh = SP ? 0 : row_head(0) / p.group;
  const uint16_t* kA = p.ka.p + cx.b * p.ka.sb + (int64_t)kvh * p.ka.sh + cx.t0 * p.ka.st;
  const uint16_t* kB = p.kb.p + cx.b * p.kb.sb + (int64_t)kvh * p.kb.sh + cx.t0 * p.kb.st;
  const uint16_t* vS = C::VLAT ? kA : p.v.p + cx.b * p.v.sb + (int64_t)kvh * p.v.sh + cx.t0 * p.v.st;
  const uint32_t stA = (uint32_t)(p.ka.st * 2), stB = (uint32_t)(p.kb.st * 2), stV = (uint32_t)(p.v.st * 2);

  if constexpr (SP) {  // stage the query's index list in LDS
    if (p.decode) {    // token generation: the rows of split q0, -1 past the valid ones
      const int s0 = (int)(cx.q0 * p.topk), n = (int)cx.kv_end;
      for (int k = tid; k < p.topk; k += 256) sm.idx[k] = k < n ? s0 + k : -1;
    } else {
      const int32_t* idx_row = p.idx + ((int64_t)cx.b * p.Nq + cx.q0) * p.topk;
      for (int k = tid; k < p.topk; k += 256) sm.idx[k] = idx_row[k];
    }
    __syncthreads();
  }
  auto idx_ok = [&](int r) -> bool { return r >= 0 && r < p.Nkv; };

  // loader: wave w copies rows 8w..8w+7 of every sub-tile; lane l handles
  // row 8w + l/8, chunk position l%8
  const int lrow = 8 * w + (lane >> 3);
  const uint32_t lchunk = (uint32_t)(((lane & 7) ^ swz_f(lrow & 15)) << 4);
  const uint32_t voA = (uint32_t)lrow * stA + lchunk;
  const uint32_t voB = (uint32_t)lrow * stB + lchunk;
  const uint32_t voV = (uint32_t)lrow * stV + lchunk;

  // LDS byte addresses of the tile buffers (buffer i at + i * tile size)
  const uint32_t lds_a = lds_addr(&sm.a[0][0]), lds_b = lds_addr(&sm.b[0][0]);
  const uint32_t lds_v = C::VLAT ? lds_a : lds_addr(&sm.v[0][0]);

  // Copies of one key tile: KI wave instructions, one per 64-column group of
  // each sub-tile (A groups, then the B sub-tile, then the V groups).  The
  // sources are worked out once per tile (tile_src); issue_copy<I> issues
  // instruction I, so that the copies can be spread over the MFMA stream.
  struct TileSrc {
    u32x4 ra, rb, rv;
    uint32_t oa, ob, la, lb, lv;
  };
  auto tile_src = [&](int t, int buf) __attribute__((always_inline)) -> TileSrc {
    TileSrc c;
    const int64_t k0 = (int64_t)t * BN;
    // buf: the slot of the tile in the ring of buffers (the A buffer; the B
    // buffer is the same slot modulo NBB)
    c.la = lds_a + buf * SM::ATILE;
    c.lb = lds_b + (buf % NBB) * SM::BTILE;
    c.lv = lds_v + buf * SM::VTILE;
    if constexpr (SP) {
      const int r = (int)k0 + lrow;
      const int ix = r < p.topk ? sm.idx[r] : -1;
      const bool ok = idx_ok(ix);
      c.ra = make_rsrc(kA, (uint32_t)(p.Nkv * stA));
      c.rb = make_rsrc(kB, (uint32_t)(p.Nkv * stB));
      c.oa = ok ? (uint32_t)ix * stA + lchunk : kOob;
      c.ob = ok ? (uint32_t)ix * stB + lchunk : kOob;
    } else {
      // the buffer is the tile's rows [k0, min(k0 + BN, kv_len)); rows past it read zeros
      const uint32_t nrows = (uint32_t)min<int64_t>(BN, cx.kv_len - k0);
      c.ra = make_rsrc(kA + k0 * p.ka.st, nrows * stA);
      c.rb = make_rsrc(kB + k0 * p.kb.st, nrows * stB);
      if constexpr (!C::VLAT) c.rv = make_rsrc(vS + k0 * p.v.st, nrows * stV);
      c.oa = voA;
      c.ob = voB;
    }
    return c;
  };
  auto issue_copy = [&](const TileSrc& c, auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    if constexpr (i < NGA) copy_rows<NGA, i, i + 1>(c.ra, c.la, w, c.oa);
    else if constexpr (i == NGA) copy_rows<1>(c.rb, c.lb, w, c.ob);
    else copy_rows<NGV, i - NGA - 1, i - NGA>(c.rv, c.lv, w, voV);
  };
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const TileSrc c = tile_src(t, buf);
    unroll<KI>([&](auto I) __attribute__((always_inline)) { issue_copy(c, I); });
  };

  // LDS byte offsets of this lane's K fragments (k-step c: + (c/4) KB)
  // (k-step c: chunk 2(c%4) + h of column group c/4; the chunk index is
  // XORed with the row swizzle, so k-step c%4 = k flips bits 5-6 by k)
  const int koffA = tile_off(NGA, lr, h), koffB = tile_off(1, lr, h);

  const int n_tiles = (int)((cx.kv_end + BN - 1) / BN);
  // key rows visible to this lane's row: [0, vis_end), relative to the
  // workgroup's key range (a key's position is kv_offset + its index)
  int32_t vis_end, wave_vis_end;
  {
    const int64_t row_pos = p.q_offset + row_query(w);
    const int64_t wave_pos = row_pos - lr;                // first row of the wave
    int64_t ve = cx.kv_len, we = cx.kv_len;
    if (p.causal && !SP) {
      ve = min<int64_t>(ve, max<int64_t>(0, row_pos - p.kv_offset + 1));
      we = min<int64_t>(we, max<int64_t>(0, wave_pos - p.kv_offset + 1));
    }
    vis_end = (int32_t)ve;        // <= kv_len, which fits 32 bits
    wave_vis_end = __builtin_amdgcn_readfirstlane((int32_t)we);  // visible to every row of the wave
  }

  f32x16 O[WAVES][NDVB];
  float m_ref = -INFINITY;  // reference max of this lane's row (log2 units)
  float m_run = -INFINITY;  // running exact max
  float l_part = 0.f;       // this lane's share of the row sum, relative to m_ref
  float l_rnd = 0.f;        // the same over the bf16-rounded weights
  bool over = false;

  // S^T = K Q^T for one tile (lane: query row lr; keys (r/4)*8 + 4h + r%4)
  // LDS byte addresses of this lane's K fragments in tile buffer `buf`
  auto frag_addrs = [&](int buf, uint32_t* a, uint32_t* b) __attribute__((always_inline)) {
    const uint32_t ta = lds_a + buf * SM::ATILE, tb = lds_b + (buf % NBB) * SM::BTILE;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = (ta + koffA) ^ (uint32_t)(k << 5);
      b[k] = (tb + koffB) ^ (uint32_t)(k << 5);
    }
  };
  auto qk = [&](int buf) __attribute__((always_inline)) -> f32x16 {
    f32x16 s;
    if constexpr (KS == 36) {
      uint32_t a[4], b[4];
      frag_addrs(buf, a, b);
      qk_chain(s, qf, a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
    } else {
      s = f32x16{};
      const unsigned char* ta = sm.a[buf];
      const unsigned char* tb = sm.b[buf];
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const bf16x8 kf = c < KSA ? *reinterpret_cast<const bf16x8*>(ta + (koffA ^ ((c & 3) << 5)) + (c >> 2) * 1024)
                                  : *reinterpret_cast<const bf16x8*>(tb + (koffB ^ ((c - KSA) << 5)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s, 0, 0, 0);
      }
    }
    return s;
  };

  // softmax, first half: scale to log2 units, mask, row max, reference max.
  // `live` false: no tile (all scores masked).
  auto scores = [&](const f32x16& s, int t, bool live, float* x) __attribute__((always_inline)) {
    const int k0 = t * BN;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = s[r] * p.scale_log2;
    bool need_mask;
    unsigned vbits = 0xffffffffu;
    if constexpr (SP) {
      const int k = k0 + lr;
      vbits = (unsigned)__ballot(live && k < p.topk && idx_ok(sm.idx[k < p.topk ? k : 0]));
      need_mask = vbits != 0xffffffffu;
    } else {
      need_mask = !live || k0 + BN > wave_vis_end;
    }
    if (need_mask) {
      // key kk of the tile (kk = (r/4)*8 + 4h + r%4) is visible iff
      // k0 + kk < vis_end, i.e. (r/4)*8 + r%4 < vis_end - k0 - 4h
      const int bound = live ? vis_end - k0 - 4 * h : -1000;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok;
        if constexpr (SP) {
          ok = (vbits >> ((r >> 2) * 8 + 4 * h + (r & 3))) & 1u;
        } else {
          ok = (r >> 2) * 8 + (r & 3) < bound;
        }
        x[r] = ok ? x[r] : -INFINITY;
      }
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = xhalf_max(mt);
    m_run = fmaxf(m_run, mt);
    if (m_ref == -INFINITY) m_ref = mt;  // the row's first visible tile (pass 0)
    over |= m_run > m_ref + TAU;
  };

  // softmax, second half, one quarter (4 of the lane's 16 scores) at a time,
  // so that it can be spread over the P.V MFMAs: weights against the
  // reference mu, row sums, and bf16 P^T fragments to LDS (a 16-key half
  // once its two quarters are done).  The exact row sum gives the LSE; the
  // sum of the weights as the P.V product sees them (rounded to bf16)
  // normalises O, so its weights sum to one.
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  auto weights_q = [&](const float* x, int pb, float mu, bf16x4* bq, auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    f32x4 pq;
#pragma unroll
    for (int r = 0; r < 4; ++r) pq[r] = __builtin_amdgcn_exp2f(x[4 * q + r] - mu);
    bq[q] = __builtin_convertvector(pq, bf16x4);
    l_part += (pq[0] + pq[1]) + (pq[2] + pq[3]);
    l_rnd += ((float)bq[q][0] + (float)bq[q][1]) + ((float)bq[q][2] + (float)bq[q][3]);
    if constexpr (q & 1) {
      const bf16x8 b = {bq[q - 1][0], bq[q - 1][1], bq[q - 1][2], bq[q - 1][3], bq[q][0], bq[q][1], bq[q][2], bq[q][3]};
      *reinterpret_cast<bf16x8*>(sm.p[pb][w][q >> 1] + lane * 16) = b;
    }
  };
  auto mu_of = [&]() __attribute__((always_inline)) { return m_ref == -INFINITY ? 0.f : m_ref; };

  // O^T += V^T P^T over this wave's value columns for all 128 rows
  // hook(integral_constant<int, g>) runs after MFMA group g (one value-column
  // block of one 16-key half), g = 0 .. 2*NDVB-1.  The fragments of group
  // g+1 are read before the MFMAs of group g: the hook may hold copies into
  // LDS, which the compiler does not move LDS reads across.
  auto pv = [&](int buf, int pb, auto&& hook) __attribute__((always_inline)) {
    const unsigned char* vt = C::VLAT ? sm.a[buf] : sm.v[buf];
    bf16x8 pf[WAVES];
#pragma unroll
    for (int rb = 0; rb < WAVES; ++rb) pf[rb] = *reinterpret_cast<const bf16x8*>(sm.p[pb][rb][0] + lane * 16);
    bf16x8 vf = read_vt<NGV>(vt, w * NDVB, 0, lane);
    unroll<2 * NDVB>([&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value, c = g / NDVB, j = g % NDVB;
      bf16x8 vn = vf;
      if constexpr (g + 1 < 2 * NDVB) vn = read_vt<NGV>(vt, w * NDVB + (g + 1) % NDVB, (g + 1) / NDVB, lane);
#pragma unroll
      for (int rb = 0; rb < WAVES; ++rb)
        O[rb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb], O[rb][j], 0, 0, 0);
      // interleave the VALU work of the previous hook (softmax) with these
      // MFMAs: the MFMA unit runs each for several VALU issue slots
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int rb = 0; rb < WAVES; ++rb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      // and keep the row sums of that work here rather than sunk to the barrier
      asm volatile("" ::"v"(l_part), "v"(l_rnd));
      if constexpr (g == NDVB - 1) {
#pragma unroll
        for (int rb = 0; rb < WAVES; ++rb) pf[rb] = *reinterpret_cast<const bf16x8*>(sm.p[pb][rb][1] + lane * 16);
      }
      hook(G);
      vf = vn;
      (void)c;
    });
  };

  // Scores S(tp) = x ready for the chain's softmax, which neither scales nor
  // masks: a tile that needs a mask (a key past the causal bound or the
  // end, or an index outside the cache) or a scale that is not positive is
  // scaled and masked here, and the chain then runs with scale 1 (returned).
  auto prep_scores = [&](f32x16& x, int tp) __attribute__((always_inline)) -> float {
    const int k0 = tp * BN;
    bool mask;
    unsigned vbits = 0xffffffffu;
    if constexpr (SP) {
      const int k = k0 + lr;  // key lr of the tile (lanes 32-63 repeat 0-31)
      const int ix = sm.idx[k < p.topk ? k : 0];
      vbits = (unsigned)__ballot((k < p.topk) & (ix >= 0) & (ix < p.Nkv));
      mask = vbits != 0xffffffffu;
    } else {
      mask = k0 + BN > wave_vis_end;
    }
    mask = mask || !(p.scale_log2 > 0.f);  // wave-uniform
    float sc = p.scale_log2;
    if (mask) {
      const int bound = vis_end - k0 - 4 * h;
      const unsigned vb = vbits >> (4 * h);  // bit (r/4)*8 + r%4: this lane's key r
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bool ok;
        if constexpr (SP) {
          ok = (vb >> ((r >> 2) * 8 + (r & 3))) & 1u;
        } else {
          ok = (r >> 2) * 8 + (r & 3) < bound;
        }
        x[r] = ok ? x[r] * p.scale_log2 : -INFINITY;
      }
      sc = 1.f;
    }
    return sc;
  };
  // Softmax of S(tp) = x to P buffer tp&1 inside the Q.K chain of tile tq;
  // x returns S(tq).
  auto chain_sm = [&](f32x16& x, int tp, int tq) __attribute__((always_inline)) {
    if constexpr (KS == 36) {
      const float sc = prep_scores(x, tp);
      uint32_t a[4], b[4];
      frag_addrs(tq & (NB - 1), a, b);
      qk_chain_softmax(x, qf, a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], sc, m_ref, m_run, l_part, l_rnd,
                       lds_addr(sm.p[tp & 1][w][0]) + lane * 16);
    }
  };

  // ------------------------------------------------------------ main loop
  // Iteration t computes S(t+1) = K(t+1) Q^T, then P(t) V(t) with the
  // softmax of S(t+1) in between, and ends on the one barrier of the
  // iteration.  Tiles t, t+1 and t+2 are resident (t+2 landed by the end of
  // the iteration); the copies of tile t+NB-1 go into the buffer tile t-1
  // left, spread over the P.V MFMAs.  P is double buffered.
  constexpr int NPV = 2 * NDVB;  // MFMA groups of one P.V
  bool redo = false;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!redo) break;      // workgroup-uniform
      m_ref = m_run;         // exact row max: every weight is <= 1
      l_part = 0.f;
      l_rnd = 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < WAVES; ++rb)
#pragma unroll
      for (int j = 0; j < NDVB; ++j) O[rb][j] = f32x16{};

    if constexpr (SM_IN_QK) {
      // Iteration t: P(t) V(t) with the copies of tile t+3 (into the buffer
      // tile t-1 left) spread over its MFMAs; then the Q.K chain of tile t+2
      // with the softmax of S(t+1) inside it, which writes P(t+1); then the
      // one barrier.  Tiles t..t+2 are resident, t+3 lands by the barrier.
      // Unrolled twice so that the two score accumulators trade roles
      // instead of being copied; the last two tiles have no chain.
      auto pv_copy = [&](int t) __attribute__((always_inline)) {
        const bool copy = t + NB - 1 < n_tiles;
        const TileSrc src = tile_src(min(t + NB - 1, n_tiles - 1), (t + NB - 1) & (NB - 1));
        pv(t & (NB - 1), t & 1, [&](auto G) __attribute__((always_inline)) {
          constexpr int g = decltype(G)::value;
          if (copy) {
            unroll<(g + 1) * KI / NPV - g * KI / NPV>([&](auto I) __attribute__((always_inline)) {
              issue_copy(src, std::integral_constant<int, g * KI / NPV + decltype(I)::value>{});
            });
          }
        });
      };
      // Past the last tile the chain still runs: the scores of tile n_tiles
      // are all masked (-inf), which leaves the row stats as they are, and
      // the tile it multiplies is stale and unused; copies past the last
      // tile read zeros (an empty buffer range) into a free buffer.
      if (n_tiles > 0) {
        const int pre = min(n_tiles, NB - 1);
        f32x16 sc;
        if constexpr (NBB >= NB - 1) {
          for (int u = 0; u < pre; ++u) issue_tile(u, u);
          wait_tiles<KI>(0);
          __syncthreads();
          sc = qk(0);
          chain_sm(sc, 0, 1);
          __syncthreads();
        } else {
          // two 64-column buffers: tile 2's goes into tile 0's once every
          // wave has read that in Q.K(0)
          for (int u = 0; u < min(pre, 2); ++u) issue_tile(u, u);
          const TileSrc c2 = tile_src(min(2, n_tiles - 1), 2);
          if (pre > 2) unroll<NGA>([&](auto I) __attribute__((always_inline)) { issue_copy(c2, I); });
          wait_tiles<KI>(0);
          __syncthreads();
          sc = qk(0);
          __syncthreads();
          if (pre > 2) issue_copy(c2, std::integral_constant<int, NGA>{});
          chain_sm(sc, 0, 1);
          wait_tiles<KI>(0);
          __syncthreads();
        }
        // this lane's V fragment offsets for value blocks 4w and 4w+1, key
        // half 0 (other blocks and halves are instruction offsets)
        uint32_t vbo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) vbo[k] = vt_off<NGA>(w * NDVB + (k >> 1), 0, lane, k & 1);
        for (int t = 0; t < n_tiles; ++t) {  // sc = S(t+1)
          const float scl = prep_scores(sc, t + 1);
          uint32_t a[4], b[4], vb[4];
          frag_addrs((t + 2) & (NB - 1), a, b);
          const uint32_t vtile = lds_a + (t & (NB - 1)) * SM::ATILE;
#pragma unroll
          for (int k = 0; k < 4; ++k) vb[k] = vtile + vbo[k];
          TileSrc src = tile_src(min(t + NB - 1, n_tiles - 1), (t + NB - 1) & (NB - 1));
          if (t + NB - 1 >= n_tiles) {
            src.ra[2] = 0;
            src.rb[2] = 0;
          }
          tile_step(sc, O, qf, a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], scl, m_ref, m_run, l_part, l_rnd,
                    lds_addr(sm.p[(t + 1) & 1][w][0]) + lane * 16, lds_addr(sm.p[t & 1][0][0]) + lane * 16, vb,
                    src.oa, src.ob, src.ra, src.rb, src.la + (uint32_t)(w * NGA) * 1024u, src.lb + (uint32_t)w * 1024u);
          wait_tiles<KI>(0);  // tile t+3
          __syncthreads();
        }
        // the step's last MFMAs write O (AGPRs) without the wait states that
        // a following VALU access of O needs
        asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
      }
    } else {
      if (n_tiles > 0) {
        const int pre = min(n_tiles, NB - 1);
        for (int u = 0; u < pre; ++u) issue_tile(u, u);
        wait_tiles<KI>(pre - min(pre, 2));   // tiles 0 and 1 have landed
        __syncthreads();
        {
          float x[16];
          scores(qk(0), 0, true, x);
          const float mu = mu_of();
          bf16x4 bq[4];
          unroll<4>([&](auto Q) __attribute__((always_inline)) { weights_q(x, 0, mu, bq, Q); });
        }
        __syncthreads();
        int buf = 0;
        for (int t = 0; t < n_tiles; ++t) {
          const int nbuf = buf == NB - 1 ? 0 : buf + 1;
          const int cbuf = buf == 0 ? NB - 1 : buf - 1;
          const bool live = t + 1 < n_tiles;
          f32x16 s = f32x16{};
          if (live) s = qk(nbuf);
          float x[16];
          float mu = 0.f;
          bf16x4 bq[4];
          const bool copy = t + NB - 1 < n_tiles;
          const TileSrc src = tile_src(min(t + NB - 1, n_tiles - 1), cbuf);
          // P(t) V(t); along the way the copies of tile t+NB-1 and the softmax
          // of S(t+1): its first half after MFMA group 0, its quarters after
          // groups NPV/5, 2NPV/5, 3NPV/5 and 4NPV/5
          pv(buf, t & 1, [&](auto G) __attribute__((always_inline)) {
            constexpr int g = decltype(G)::value;
            if (copy) {
              unroll<(g + 1) * KI / NPV - g * KI / NPV>([&](auto I) __attribute__((always_inline)) {
                issue_copy(src, std::integral_constant<int, g * KI / NPV + decltype(I)::value>{});
              });
            }
            if constexpr (g == 0) {
              scores(s, t + 1, live, x);
              mu = mu_of();
            }
            unroll<4>([&](auto Q) __attribute__((always_inline)) {
              if constexpr ((decltype(Q)::value + 1) * NPV / 5 == g) weights_q(x, (t + 1) & 1, mu, bq, Q);
            });
          });
          // tile t+2 must have landed; the copies of tile t+NB-1 may stay in flight
          wait_tiles<KI>(min(n_tiles - 1, t + NB - 1) - (t + 2));
          __syncthreads();
          buf = nbuf;
        }
      }
    }
    if (pass == 0) {
      over |= m_run > m_ref + TAU;  // (the softmax in the Q.K chain tracks only m_run)
      // the P buffers are idle now: their space carries the overflow flags
      const bool any = __ballot(over) != 0ull;
      if (lane == 0) sm.epi.flag[w] = any;
      __syncthreads();
      redo = (sm.epi.flag[0] | sm.epi.flag[1] | sm.epi.flag[2] | sm.epi.flag[3]) != 0;
    }
  }

  // Lane-derived values are recomputed here rather than held across the key
  // loop, where the register pressure would spill them to be reloaded one
  // after another, each reload a round trip to memory.
  {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    lane = t & 63;
    h = lane >> 5;
    lr = lane & 31;
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
      sm.epi.wprev[w * 32 + lr] = wp;
      sm.epi.wcur[w * 32 + lr] = wc;
      if (p.lse.p && ok) p.lse.p[cx.b * p.lse.sb + hq * p.lse.sh + tq * p.lse.st] = L;
    }
  }
  __syncthreads();

  if (!p.prev_out.p && !p.out_f32) {
    // Plain bf16 output: O^T sits in the accumulators with one output row per
    // lane, so direct stores would be 8-byte pieces of 32 rows each.  Instead
    // the scaled bf16 rows go through LDS (the idle tile buffers; the row
    // stride is padded by 16 bytes to spread the banks) and leave as whole
    // rows, 16 bytes a lane.
    constexpr int RS = DV * 2 + 16;           // LDS row stride, bytes
    constexpr int LPR = DV * 2 / 16;          // lanes per output row
    constexpr int RPI = 64 / LPR;             // rows per store instruction
    // staging space: the tile buffers and what follows them up to P
    constexpr int CAP = (int)(sizeof(sm.a) + sizeof(sm.b) + sizeof(sm.v) + sizeof(sm.idx));
    constexpr int NPASS = ROWS * RS <= CAP ? 1 : 2;  // halves of the rows at a time
    static_assert(ROWS * RS <= 2 * CAP, "half of the rows fits the staging space");
    constexpr int RBP = WAVES / NPASS;        // row blocks per pass
    const uint32_t stage = lds_addr(&sm.a[0][0]);
    // output row rl of row block rb (workgroup row 32 rb + rl) is at element
    // out_off + rb * o_srb + rl * o_srl; it exists iff rb < o_nrb and
    // rl < o_nrl (latent) or 32 rb + rl < o_nr (split, sparse)
    int64_t out_off, o_srb, o_srl;
    int o_nrb = 0, o_nrl = 0, o_nr = 0;
    if constexpr (MODE == LATENT) {
      out_off = cx.b * p.out.sb + cx.hbase * p.out.sh + qtok(cx.q0) * p.out.st;
      o_srb = p.out.sh;
      o_srl = p.out.st;
      o_nrb = p.Hq - cx.hbase;
      o_nrl = (int)min<int64_t>(32, cx.q_len - cx.q0);
    } else if constexpr (MODE == SPLIT) {
      out_off = cx.b * p.out.sb + cx.hbase * p.out.sh + qtok(cx.q0) * p.out.st;
      o_srb = 32 * p.out.st;
      o_srl = p.out.st;
      o_nr = (int)min<int64_t>(ROWS, cx.q_len - cx.q0);
    } else {
      out_off = cx.b * p.out.sb + qtok(cx.q0) * p.out.st;
      o_srb = 32 * p.out.sh;
      o_srl = p.out.sh;
      o_nr = p.Hq;
    }
#pragma unroll
    for (int pass_ = 0; pass_ < NPASS; ++pass_) {
#pragma unroll
      for (int rbl = 0; rbl < RBP; ++rbl) {
        const int rb = pass_ * RBP + rbl;
        const float wc = sm.epi.wcur[rb * 32 + lr];
        const uint32_t row = stage + (uint32_t)(rbl * 32 + lr) * RS;
#pragma unroll
        for (int j = 0; j < NDVB; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = 32 * (w * NDVB + j) + 8 * g + 4 * h;
            const u32x2 v = {pack_bf16x2(wc * O[rb][j][4 * g], wc * O[rb][j][4 * g + 1]),
                             pack_bf16x2(wc * O[rb][j][4 * g + 2], wc * O[rb][j][4 * g + 3])};
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)(row + d * 2)) = v;
          }
        }
      }
      __syncthreads();
      // this wave stores staged rows w*RPI + k*WAVES*RPI (+ lane/LPR), k < NST,
      // reading a batch of them from LDS before storing the batch.  Staged
      // row k sits in row block rb0 + k/KB of the workgroup at row
      // rl0 + (k%KB)*WAVES*RPI of the block.
      constexpr int NST = RBP * 32 / (WAVES * RPI);
      constexpr int BATCH = NST < 8 ? NST : 8;
      constexpr int KB = 32 / (WAVES * RPI);
      static_assert(NST % BATCH == 0 && 32 % (WAVES * RPI) == 0, "store batches");
      const int rb0 = pass_ * RBP, rl0 = w * RPI + lane / LPR;
      // this lane's element address in the output, stepped along the rows in
      // vector registers (the scalar ones are all taken here)
      int64_t orow = out_off + (int64_t)rb0 * o_srb + (int64_t)rl0 * o_srl + (lane % LPR) * 8;
      int64_t ostep = (int64_t)(WAVES * RPI) * o_srl, oblk = o_srb - (int64_t)KB * ostep;
      asm volatile("" : "+v"(orow), "+v"(ostep), "+v"(oblk));
#pragma unroll
      for (int k0 = 0; k0 < NST; k0 += BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int rs = (w + (k0 + k) * WAVES) * RPI + lane / LPR;
          v[k] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              (uintptr_t)(stage + (uint32_t)rs * RS + (lane % LPR) * 16));
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const int kk = k0 + k, rb = rb0 + kk / KB, rl = rl0 + (kk % KB) * (WAVES * RPI);
          const bool ok = MODE == LATENT ? rb < o_nrb && rl < o_nrl : rb * 32 + rl < o_nr;
          if (ok) *reinterpret_cast<u32x4*>(p.out.p + orow) = v[k];
          orow += (kk + 1) % KB ? ostep : ostep + oblk;
        }
      }
      if (NPASS > 1 && pass_ + 1 < NPASS) __syncthreads();
    }
    return;
  }

#pragma unroll
  for (int rb = 0; rb < WAVES; ++rb) {
    if (!row_valid(rb)) continue;
    const float wp = sm.epi.wprev[rb * 32 + lr];
    const float wc = sm.epi.wcur[rb * 32 + lr];
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
            const f32x4 pv4 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.prev_out.p) + pel + d);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] += wp * pv4[e];
          } else {
            const u32x2 pv2 = *reinterpret_cast<const u32x2*>(p.prev_out.p + pel + d);
            y[0] += wp * __uint_as_float(pv2[0] << 16);
            y[1] += wp * __uint_as_float(pv2[0] & 0xffff0000u);
            y[2] += wp * __uint_as_float(pv2[1] << 16);
            y[3] += wp * __uint_as_float(pv2[1] & 0xffff0000u);
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
  constexpr int DA = 512, NGA = DA / 64;
  __shared__ alignas(16) unsigned char ta[BN * DA * 2];
  __shared__ alignas(16) unsigned char tb[BN * DB * 2];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const uint16_t* kA = p.ka.p + p.b * p.ka.sb;
  const uint16_t* kB = p.kb.p + p.b * p.kb.sb;
  const uint32_t stA = (uint32_t)(p.ka.st * 2), stB = (uint32_t)(p.kb.st * 2);
  const u32x4 ra = make_rsrc(kA, (uint32_t)(p.Nkv * stA));
  const u32x4 rb = make_rsrc(kB, (uint32_t)(p.Nkv * stB));
  const int lrow = 8 * w + (lane >> 3);
  const uint32_t lchunk = (uint32_t)(((lane & 7) ^ swz_f(lrow & 15)) << 4);
  auto ok = [&](int r) { return r >= 0 && r < p.Nkv; };
  const int n_tiles = (p.K + BN - 1) / BN;
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN;
    const int ix = (k0 + lrow < p.K) ? p.idx[k0 + lrow] : -1;
    copy_rows<NGA>(ra, lds_addr(ta), w, ok(ix) ? (uint32_t)ix * stA + lchunk : kOob);
    copy_rows<1>(rb, lds_addr(tb), w, ok(ix) ? (uint32_t)ix * stB + lchunk : kOob);
    wait_vmem();
    __syncthreads();
    for (int e = tid; e < BN * (DA + DB) / 8; e += 256) {
      const int r = e / ((DA + DB) / 8), c = e % ((DA + DB) / 8);
      if (k0 + r >= p.K) continue;
      const u32x4 val = c < DA / 8 ? *reinterpret_cast<const u32x4*>(ta + tile_off(NGA, r, c))
                                   : *reinterpret_cast<const u32x4*>(tb + tile_off(1, r, c - DA / 8));
      *reinterpret_cast<u32x4*>(p.rows_out + (int64_t)(k0 + r) * (DA + DB) + c * 8) = val;
    }
    __syncthreads();
  }
}

__global__ void queue_reset_kernel(unsigned* q) { q[0] = 0u; }

// Compute units of the current device, cached per device (0 if unknown).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One workgroup per item of a latent or sparse kernel (each fills a CU's
// LDS).  The item queue pays off only when the items outnumber the CUs
// several times over (a launch that fits the chip at once has no tail to
// balance); then the counter is reset first, on the same stream.
template <int MODE>
hipError_t launch_items(AttnParams p, int64_t items, hipStream_t s) {
  const int ncu = p.queue ? cu_count() : 0;
  if (ncu > 0 && items > 4 * (int64_t)ncu) hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(1), 0, s, p.queue);
  else p.queue = nullptr;
  hipLaunchKernelGGL((attn_fwd_kernel<LatentCfg, MODE>), dim3((unsigned)items), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_latent_dense(const AttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.n_qblk * p.n_hgrp * p.B;
  if (items == 0) return hipSuccess;
  return launch_items<LATENT>(p, items, s);
}

hipError_t launch_latent_sparse(const AttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.Nq;
  if (items == 0) return hipSuccess;
  if (p.topk <= KMAX_IDX_PIPE) return launch_items<SPARSE_PIPE>(p, items, s);
  AttnParams q = p;
  q.queue = nullptr;
  hipLaunchKernelGGL((attn_fwd_kernel<LatentCfg, SPARSE>), dim3((unsigned)items), dim3(256), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnParams& p, int64_t items, hipStream_t s) {
  if (items == 0) return hipSuccess;
  return launch_items<SPARSE_PIPE>(p, items, s);
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
