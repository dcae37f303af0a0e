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
  int kv_slot;        // decode: the cache slot of the sequence
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
  const int64_t call_item = blockIdx.x;
#include "mla_attn_body.inc"
}

// Several calls in one launch.  Calls with equal item counts (the query
// chunks of a ring step) take workgroups in turn, so that the launch runs
// the longest items of every call first; otherwise call k takes the
// workgroups [first[k], first[k+1]).
template <class C, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, kWavesPerEU<MODE>)))
void attn_fwd_group_kernel(const GroupParams g) {
  int call = 0;
  int64_t call_item;
  if (g.interleave) {
    call = (int)(blockIdx.x % (unsigned)g.n);
    call_item = blockIdx.x / (unsigned)g.n;
  } else {
    for (int i = 1; i < kMaxGroup; ++i)
      if (i < g.n && (int)blockIdx.x >= g.first[i]) call = i;
    call_item = (int64_t)blockIdx.x - g.first[call];
  }
  const AttnParams& p = g.sub[call];
#include "mla_attn_body.inc"
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

// Compute units of the current device, cached per device.
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

hipError_t launch_latent_dense(const AttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.n_qblk * p.n_hgrp * p.B;
  if (items == 0) return hipSuccess;
  return launch_items<LATENT>(p, items, s);
}

hipError_t launch_latent_group(const GroupParams& g, hipStream_t s) {
  const int64_t items = g.first[g.n];
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_group_kernel<LatentCfg, LATENT>), dim3((unsigned)items), dim3(256), 0, s, g);
  return hipGetLastError();
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
  // no item queue here: its counter round trip at the start of each of the
  // many short workgroups cost more (+4.6%) than the balance it brings
  AttnParams q = p;
  q.queue = nullptr;
  hipLaunchKernelGGL((attn_fwd_kernel<SplitCfg, SPLIT>), dim3((unsigned)blocks), dim3(256), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_debug_gather(const GatherParams& p, hipStream_t s) {
  if (p.K == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
