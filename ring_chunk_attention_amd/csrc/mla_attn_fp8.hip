// The FP8 form of the shared-latent attention forward (TensorRT-LLM mla.py,
// forward_absorption_context: the fused FP8 query and the FP8 latent cache,
// float8_e4m3fn, with the BMM1 and BMM2 scales; the output stays bf16).
//
// q8 [B, H, N, 576] and kv8 [B, 1, Nkv, 576] are OCP e4m3 codes, dequantised
// by one scale each.  Both products run on gfx950's 8-bit MFMA
// (v_mfma_*_f32_32x32x64_f8f6f4, e4m3 x e4m3 -> fp32, twice the rate of the
// bf16 32x32x16 form per flop):
//  * S^T = K Q^T over 576 columns: nine k-steps of 64, for each of the two
//    32-key halves of a 64-key tile.  The wave's 32 Q rows (4 heads x the same
//    32 queries per workgroup, as in the bf16 form) stay in 72 VGPRs.
//  * O^T += V^T P^T: P is rounded to e4m3 against the row's reference max
//    (a weight is at most 2^8 = 256, inside e4m3's range of 448), shared
//    through LDS, and each wave multiplies it for all 128 rows over its own
//    128 of the 512 value columns.  The V^T operand comes straight from the
//    key tile in LDS through ds_read_b64_tr_b8, which hands lane i of each
//    group of 16 the byte i % 8 of the 8-byte rows addressed by lanes
//    2e + i / 8 (e = 0..7): the even lanes address 8 columns of 8 key rows,
//    the odd lanes the next 8 columns of the same rows.
//  * Softmax in base 2 against a per-row reference max fixed at the row's
//    first visible tile, with an exact second pass when a later score
//    exceeds it by more than 8 (log2 units); O is divided by the sum of the
//    rounded weights (the weights as the product sees them), the LSE takes
//    the exact fp32 sum.
// A key tile is 64 rows x 576 bytes = 36 KB (the same bytes as the bf16
// form's 32-row tile), copied HBM -> LDS by buffer_load ... lds with a row
// swizzle under which both LDS read patterns are free of bank conflicts.
#include "mla_attn_kernels.inc"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int F8_BN = 64;                 // keys per tile: the K of the P.V product
constexpr int F8_ROWB = 576;              // bytes of a key row: 512 latent + 64 RoPE
constexpr int F8_TILE = F8_BN * F8_ROWB;  // 36 KB
constexpr int F8_ROPE = 32768;            // offset of the RoPE sub-tile within a tile
constexpr int F8_NB = 4;                  // tile buffers: t (P.V), t+1 (Q.K), t+2 and t+3 in flight
constexpr int F8_KS = 9;                  // k-steps of 64 columns in Q.K
constexpr int F8_KI = 9;                  // copy instructions per wave per tile
constexpr float F8_TAU = 8.0f;            // allowed growth of a row max over its reference (log2 units)

struct SmemF8 {
  alignas(1024) unsigned char t[F8_NB][F8_TILE];
  union {
    alignas(16) unsigned char p[2][WAVES][2][64 * 16];  // P^T operands: buffer, row block, 16-byte half
    struct {                                            // after the key loop (and the queue's item)
      float wcur[ROWS];
      int flag[WAVES];
      int item;
    } epi;
  };
};
static_assert(sizeof(SmemF8) <= 160 * 1024, "one workgroup's LDS");

// Latent sub-tile: blocks of 8 rows x 8 chunks of 16 bytes (1 KB), block
// (r / 8, g) at ((r / 8) * 4 + g) KB, row r % 8 at + 128 (r % 8), logical
// chunk q of group g at position (q % 8) ^ f(r).  With f(r) = 2 ((r / 2) % 4)
// + (r / 8) % 2: 16 consecutive rows at one chunk (the Q.K operand reads,
// 16 lanes of 16 bytes) land on 16 distinct 16-byte bank groups, and 8
// consecutive rows at two neighbouring chunks (the transposed V reads, 32
// lanes of 8 bytes) on 16 distinct ones as well.
__device__ __forceinline__ int f8_swz(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
// RoPE sub-tile: blocks of 16 rows x 4 chunks (1 KB) at 32 KB + (r / 16) KB,
// row r % 16 at + 64 (r % 16), chunk q at position q ^ ((r / 4) % 4).

__device__ __forceinline__ i32x4 lds16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>((uintptr_t)addr);
}
__device__ __forceinline__ i32x2 lds_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<__attribute__((address_space(3))) i32x2*>((uintptr_t)addr));
}
__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // e4m3 x e4m3 (format 0 for both operands), no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The same product with the accumulator in VGPRs (the Q.K scores): the
// output accumulators take all 256 AGPRs, and through the builtin the
// compiler put the scores in AGPRs too and moved a quarter of O out to VGPRs
// and back on every tile.  Consecutive products into one accumulator need no
// wait states; a VALU read of the result does (s_nop block below).
__device__ __forceinline__ void mfma8_v0(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_v(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// max of three by one v_max3_f32, without the quieting of signalling NaN
// inputs that fmaxf asks for (MFMA results are never signalling)
__device__ __forceinline__ float f8_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_fp8_kernel(const AttnParams p) {
  __shared__ SmemF8 sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, h = lane >> 5, lr = lane & 31;
  __builtin_assume(w >= 0 && w < WAVES);

  // ------------------------------------------------------------ work item
  // 32 queries x 4 heads, longest causal rows first (or from the queue)
  int64_t item = blockIdx.x;
  if (p.queue) {
    if (tid == 0) sm.epi.item = (int)atomicAdd(p.queue, 1u);
    __syncthreads();
    item = sm.epi.item;  // (P, which shares this space, is first written past a barrier)
  }
  const int per = p.n_hgrp * p.B;
  const int qblk = p.n_qblk - 1 - (int)(item / per);
  const int rem = (int)(item % per);
  const int hbase = (rem % p.n_hgrp) * WAVES;
  const int b = rem / p.n_hgrp;
  const int64_t q0 = (int64_t)qblk * 32;
  const int64_t q_len = p.Nq, kv_len = p.Nkv;
  const int64_t last_q = min(q_len - 1, q0 + 31);
  const int64_t kv_end = p.causal ? max<int64_t>(0, min<int64_t>(kv_len, p.q_offset + last_q - p.kv_offset + 1))
                                  : kv_len;
  const int n_tiles = (int)((kv_end + F8_BN - 1) / F8_BN);

  const uint8_t* Qb = reinterpret_cast<const uint8_t*>(p.qa.p);
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(p.ka.p) + b * p.ka.sb;
  const int64_t stK = p.ka.st;  // bytes

  // ------------------------------------------------------------ Q -> VGPR
  // B operand of k-step c: row lr of the wave, bytes 64c + 32h .. +31
  i32x8 qf[F8_KS];
  {
    const int hq = hbase + w < p.Hq ? hbase + w : 0;
    const int64_t t = q0 + lr < q_len ? q0 + lr : 0;
    const uint8_t* row = Qb + b * p.qa.sb + hq * p.qa.sh + t * p.qa.st + 32 * h;
#pragma unroll
    for (int c = 0; c < F8_KS; ++c) {
      const i32x4 x0 = *reinterpret_cast<const i32x4*>(row + 64 * c);
      const i32x4 x1 = *reinterpret_cast<const i32x4*>(row + 64 * c + 16);
      qf[c] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  }

  // ---------------------------------------------------------- tile copies
  // Wave w fills latent row blocks w and w + 4 (four 1 KB groups each) and
  // RoPE block w: lane l fetches the 16-byte chunk that belongs at position
  // l of the 1 KB block.  Rows past the key range read zeros.
  const uint32_t lds_t = lds_addr(&sm.t[0][0]);
  uint32_t voA0, voA1, voB;
  {
    const int r0 = 8 * w + (lane >> 3), r1 = 8 * (w + 4) + (lane >> 3), rb = 16 * w + (lane >> 2);
    voA0 = (uint32_t)(r0 * stK) + 16u * (uint32_t)((lane & 7) ^ f8_swz(r0));
    voA1 = (uint32_t)(r1 * stK) + 16u * (uint32_t)((lane & 7) ^ f8_swz(r1));
    voB = (uint32_t)(rb * stK) + 16u * (uint32_t)((lane & 3) ^ ((rb >> 2) & 3));
  }
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)t * F8_BN;
    // rows [k0, min(k0 + BN, kv_end)): those past it, which no row of the
    // workgroup sees, read zeros (whatever they hold stays out of P.V)
    const uint32_t nrows = (uint32_t)min<int64_t>(F8_BN, kv_end - k0);
    const u32x4 rs = make_rsrc(Kb + k0 * stK, nrows * (uint32_t)stK);
    const uint32_t base = lds_t + (uint32_t)buf * F8_TILE;
    copy_rows<4>(rs, base, w, voA0);
    copy_rows<4>(rs, base, w + 4, voA1);
    copy_to_lds<512>(rs, base + F8_ROPE + (uint32_t)w * 1024u, voB);
  };

  // ------------------------------------------------- LDS operand addresses
  // Q.K A operand, k-step c < 8: row lr of the key half, chunks 4c + 2h + e
  // (e = 0, 1): + (c / 2) KB + 16 KB per key half; k-step 8 (RoPE): + 2 KB
  // per key half.
  uint32_t koff[2][2], kropw[2];
  {
    const int fk = f8_swz(lr);
    const uint32_t a0 = (uint32_t)((lr >> 3) * 4) * 1024u + 128u * (uint32_t)(lr & 7);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
      for (int cp = 0; cp < 2; ++cp) koff[e][cp] = a0 + 16u * (uint32_t)(((2 * h + e) + 4 * cp) ^ fk);
      kropw[e] = F8_ROPE + (uint32_t)(lr >> 4) * 1024u + 64u * (uint32_t)(lr & 15) +
                 16u * (uint32_t)((2 * h + e) ^ ((lr >> 2) & 3));
    }
  }
  // P.V A operand (V^T, value columns 32 (4w + j) .. +31, keys 32h + 8rr + e):
  // + 4 KB per rr, the XOR selects j and rr % 2 (see f8_swz)
  uint32_t vaddr[4][2];
  {
    const int i = lane & 15, gg = (lane >> 4) & 1, s = (i >> 2) & 3;
    const uint32_t vb = (uint32_t)h * 16384u + (uint32_t)w * 1024u + 128u * (uint32_t)(i >> 1) +
                        8u * (uint32_t)(i & 1) + 32u * (uint32_t)s + 16u * (uint32_t)gg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) vaddr[j][q] = vb ^ (uint32_t)(32 * j + 16 * q);
  }
  const uint32_t lds_pl = lds_addr(&sm.p[0][0][0][0]) + (uint32_t)lane * 16u;  // this lane's slot of the P operands

  f32x16 O[WAVES][4];
  float m_ref = -INFINITY, m_run = -INFINITY, l_part = 0.f, l_rnd = 0.f;
  float mu_fix = 0.f;  // the weights' reference past tile 0
  bool over = false;

  // S^T halves of tile `buf` (lane: query row lr; keys 32kh + 8(r/4) + 4h + r%4).
  // The lane's fragment bases are formed once per tile; the k-step and key
  // half become instruction offsets.
  // pk_prev: the previous softmax's packed e4m3 weights, whose sum (the
  // rounded row sum) is taken here, between the products, where the VALU is
  // otherwise idle.
  auto qk = [&](int buf, f32x16& s0, f32x16& s1, const int (&pk_prev)[2][4]) __attribute__((always_inline)) {
    const uint32_t tb = lds_t + (uint32_t)buf * F8_TILE;
    uint32_t kb[2][2], kr[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kb[e][0] = tb + koff[e][0];
      kb[e][1] = tb + koff[e][1];
      kr[e] = tb + kropw[e];
    }
    auto frags = [&](int c, i32x8* a) __attribute__((always_inline)) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        i32x4 x0, x1;
        if (c < 8) {
          x0 = lds16(kb[0][c & 1] + (uint32_t)((c >> 1) * 1024 + kh * 16384));
          x1 = lds16(kb[1][c & 1] + (uint32_t)((c >> 1) * 1024 + kh * 16384));
        } else {
          x0 = lds16(kr[0] + (uint32_t)(kh * 2048));
          x1 = lds16(kr[1] + (uint32_t)(kh * 2048));
        }
        a[kh] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    };
    // the fragments of k-step c+1 are read before the products of k-step c
    i32x8 acur[2], anext[2];
    frags(0, acur);
    unroll<F8_KS>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = decltype(C)::value;
      if constexpr (c + 1 < F8_KS) frags(c + 1, anext);
      if constexpr (c == 0) {
        mfma8_v0(s0, acur[0], qf[c]);
        mfma8_v0(s1, acur[1], qf[c]);
      } else {
        mfma8_v(s0, acur[0], qf[c]);
        mfma8_v(s1, acur[1], qf[c]);
      }
      if constexpr (c < 8) {
        const int v = pk_prev[c >> 2][c & 3];
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
        l_rnd += (lo[0] + lo[1]) + (hi[0] + hi[1]);
        asm volatile("" ::"v"(l_rnd));
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (c + 1 < F8_KS) {
        acur[0] = anext[0];
        acur[1] = anext[1];
      }
    });
    // the wait states a VALU read of an 8-bit 32x32x64 product's result needs
    asm("s_nop 7\n s_nop 7\n s_nop 7" : "+v"(s0), "+v"(s1));
  };

  // key rows visible to this lane's row: [0, vis_end); to every row of the wave: [0, wave_vis_end)
  int32_t vis_end, wave_vis_end;
  {
    const int64_t row_pos = p.q_offset + q0 + lr;
    int64_t ve = kv_len, we = kv_len;
    if (p.causal) {
      ve = min<int64_t>(ve, max<int64_t>(0, row_pos - p.kv_offset + 1));
      we = min<int64_t>(we, max<int64_t>(0, row_pos - lr - p.kv_offset + 1));
    }
    vis_end = (int32_t)ve;
    wave_vis_end = __builtin_amdgcn_readfirstlane((int32_t)we);
  }

  const float sm_scale = p.scale_log2 > 0.f ? p.scale_log2 : 1.f;

  // The scores of one tile as this lane's 32 values (half kh: x[16 kh + r]),
  // scaled when the scale is not positive, and masked (-inf) where the tile
  // cuts the causal bound or the end of the keys (live == false: no tile).
  auto prep = [&](const f32x16& s0, const f32x16& s1, int t, bool live, float* x) __attribute__((always_inline)) {
    const int k0 = t * F8_BN;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = s0[r];
      x[16 + r] = s1[r];
    }
    if (!(p.scale_log2 > 0.f)) {
#pragma unroll
      for (int r = 0; r < 32; ++r) x[r] *= p.scale_log2;
    }
    if (!live || k0 + F8_BN > wave_vis_end) {
      // key 32kh + 8(r/4) + 4h + r%4 of the tile is visible iff it is < vis_end - k0
      const int bound = live ? vis_end - k0 - 4 * h : -1000;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int kk = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + (r & 3);
        x[r] = kk < bound ? x[r] : -INFINITY;
      }
    }
  };

  // Softmax of prepared scores: row max and reference, weights, their exact
  // and rounded sums, and the e4m3 P^T operand of this wave's rows written
  // to P buffer pb.  Branch-free, so that it can be spread over the P.V
  // products.
  auto softmax = [&](float* x, int pb, int (&pk)[2][4]) __attribute__((always_inline)) {
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 32; ++r) mt = fmaxf(mt, x[r]);
    mt = xhalf_max(mt) * sm_scale;
    m_run = fmaxf(m_run, mt);
    m_ref = m_ref == -INFINITY ? mt : m_ref;
    over |= m_run > m_ref + F8_TAU;
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
    // pk[key half][a]: bytes d = keys 8a + 4h + d of the half (summed by the next Q.K chain)
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float e[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) e[d] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[16 * kh + 4 * a + d], sm_scale, -mu));
        l_part += (e[0] + e[1]) + (e[2] + e[3]);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], v, true);
        pk[kh][a] = v;
      }
    }
    // lanes n and n + 32 hold 16 keys each of both halves of row n; after the
    // swap lane n holds the 32 keys of half 0 and lane n + 32 those of half 1
    int xa[4], ya[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const auto r = __builtin_amdgcn_permlane32_swap((unsigned)pk[0][a], (unsigned)pk[1][a], false, false);
      xa[a] = (int)r[0];
      ya[a] = (int)r[1];
    }
    const uint32_t dst = lds_pl + (uint32_t)(pb * WAVES + w) * 2048u;
    *reinterpret_cast<__attribute__((address_space(3))) i32x4*>((uintptr_t)dst) = i32x4{xa[0], ya[0], xa[1], ya[1]};
    *reinterpret_cast<__attribute__((address_space(3))) i32x4*>((uintptr_t)(dst + 1024)) =
        i32x4{xa[2], ya[2], xa[3], ya[3]};
  };

  // O^T += V^T P^T over this wave's 128 value columns for all 128 rows of
  // tile `buf` with P buffer pb, and beside it the softmax of the next tile's
  // prepared scores x into P buffer pbn.  With one wave per SIMD the
  // instructions issue in order, so the softmax is cut into 16 stages, one
  // after each product, and a scheduling fence after each keeps that order;
  // each value-column block's V^T is read one block ahead.
  auto pv_softmax = [&](int buf, int pb, float* x, int pbn, int (&pk)[2][4]) __attribute__((always_inline)) {
    const uint32_t tb = lds_t + (uint32_t)buf * F8_TILE;
    const uint32_t pr = lds_pl + (uint32_t)pb * (uint32_t)(WAVES * 2048);
    i32x8 pf[WAVES];
#pragma unroll
    for (int rb = 0; rb < WAVES; ++rb) {
      const i32x4 x0 = lds16(pr + (uint32_t)(rb * 2048)), x1 = lds16(pr + (uint32_t)(rb * 2048 + 1024));
      pf[rb] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
    auto read_v = [&](int j) __attribute__((always_inline)) -> i32x8 {
      uint32_t v0 = tb + vaddr[j][0], v1 = tb + vaddr[j][1];
      asm("" : "+v"(v0), "+v"(v1));  // keep the block offsets as instruction offsets
      i32x8 vf;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const i32x2 v = lds_tr8((rr & 1 ? v1 : v0) + (uint32_t)(rr * 4096));
        vf[2 * rr] = v[0];
        vf[2 * rr + 1] = v[1];
      }
      return vf;
    };
    i32x8 vcur = read_v(0), vnext;
    // softmax state across the stages
    float mp[4], mu = 0.f;
    float e[32];
    unroll<16>([&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value, j = g / 4, rb = g % 4;
      if constexpr (rb == 0 && j < 3) vnext = read_v(j + 1);
      O[rb][j] = mfma8(vcur, pf[rb], O[rb][j]);
      if constexpr (g < 4) {
        // partial maxima of 8 scores each
        float m = f8_max3(x[8 * g], x[8 * g + 1], x[8 * g + 2]);
        m = f8_max3(m, x[8 * g + 3], x[8 * g + 4]);
        m = f8_max3(m, x[8 * g + 5], x[8 * g + 6]);
        mp[g] = f8_max3(m, x[8 * g + 7], x[8 * g + 7]);
        if constexpr (g == 3) {
          float mt = f8_max3(f8_max3(mp[0], mp[1], mp[2]), mp[3], mp[3]);
          mt = xhalf_max(mt) * sm_scale;
          // Past tile 0 the reference is fixed (a row that sees any key
          // sees key 0) and m_run only grows: the overflow check waits for
          // the end of the tile loop.
          m_run = f8_max3(m_run, mt, mt);
          mu = mu_fix;
        }
      } else if constexpr (g < 12) {
        // four weights, their exact sum and the e4m3 pair packing
        constexpr int q = g - 4;  // 0..7: weights 4q .. 4q+3 (half q / 4, a = q % 4)
#pragma unroll
        for (int d = 0; d < 4; ++d) e[4 * q + d] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[4 * q + d], sm_scale, -mu));
        l_part += (e[4 * q] + e[4 * q + 1]) + (e[4 * q + 2] + e[4 * q + 3]);
        // (the pair conversions write one half each, so the register's old
        // value, the previous tile's weights already summed, is overwritten
        // whole: no zeroing move)
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * q], e[4 * q + 1], pk[q / 4][q % 4], false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * q + 2], e[4 * q + 3], v, true);
        pk[q / 4][q % 4] = v;
      } else {
        // the lane exchange and the P write (the rounded weights are summed
        // in the next Q.K chain)
        constexpr int q = g - 12;  // 0..3
        if constexpr (q == 3) {
          // lanes n and n + 32 hold 16 keys each of both halves of row n; after
          // the swap lane n holds the 32 keys of half 0 and lane n + 32 those of half 1
          int xa[4], ya[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const auto r = __builtin_amdgcn_permlane32_swap((unsigned)pk[0][a], (unsigned)pk[1][a], false, false);
            xa[a] = (int)r[0];
            ya[a] = (int)r[1];
          }
          const uint32_t dst = lds_pl + (uint32_t)(pbn * WAVES + w) * 2048u;
          *reinterpret_cast<__attribute__((address_space(3))) i32x4*>((uintptr_t)dst) = i32x4{xa[0], ya[0], xa[1], ya[1]};
          *reinterpret_cast<__attribute__((address_space(3))) i32x4*>((uintptr_t)(dst + 1024)) =
              i32x4{xa[2], ya[2], xa[3], ya[3]};
        }
      }
      if constexpr (rb == 3 && j < 3) vcur = vnext;
      // keep the row sums of this stage here rather than sunk to the loop's end
      asm volatile("" ::"v"(l_part));
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ------------------------------------------------------------ main loop
  bool redo = false;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!redo) break;  // workgroup-uniform
      m_ref = m_run;     // exact row max: every weight <= 1
      l_part = 0.f;
      l_rnd = 0.f;
    }
#pragma unroll
    for (int rb = 0; rb < WAVES; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) O[rb][j] = f32x16{};
    if (n_tiles > 0) {
      const int pre = min(n_tiles, F8_NB - 1);
      for (int u = 0; u < pre; ++u) issue_tile(u, u);
      wait_tiles<F8_KI>(pre - min(pre, 2));  // tiles 0 and 1 have landed
      __syncthreads();
      int pk[2][4] = {};  // packed e4m3 weights of the last softmax, not yet summed
      {
        f32x16 s0, s1;
        float x[32];
        qk(0, s0, s1, pk);  // (pk holds zeros: adds nothing)
        prep(s0, s1, 0, true, x);
        softmax(x, 0, pk);
      }
      mu_fix = m_ref == -INFINITY ? 0.f : m_ref;
      __syncthreads();
      for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & (F8_NB - 1), nbuf = (t + 1) & (F8_NB - 1), cbuf = (t + F8_NB - 1) & (F8_NB - 1);
        const bool live = t + 1 < n_tiles;
        // tile t+3 into the buffer tile t-1 left (free since the last barrier)
        if (t + F8_NB - 1 < n_tiles) issue_tile(t + F8_NB - 1, cbuf);
        // past the last tile the product runs on a stale buffer and its scores are all masked
        f32x16 s0, s1;
        float x[32];
        qk(nbuf, s0, s1, pk);
        prep(s0, s1, t + 1, live, x);
        pv_softmax(buf, t & 1, x, (t + 1) & 1, pk);
        // tile t+2 must have landed; later copies may stay in flight
        wait_tiles<F8_KI>(min(n_tiles - 1, t + F8_NB - 1) - (t + 2));
        __syncthreads();
      }
      asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
      // the last softmax's weights (all masked past the last tile: they add 0)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int v = pk[q >> 2][q & 3];
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
        l_rnd += (lo[0] + lo[1]) + (hi[0] + hi[1]);
      }
      over |= m_run > m_ref + F8_TAU;
    }
    if (pass == 0) {
      const bool any = __ballot(over) != 0ull;
      if (lane == 0) sm.epi.flag[w] = any;
      __syncthreads();
      redo = (sm.epi.flag[0] | sm.epi.flag[1] | sm.epi.flag[2] | sm.epi.flag[3]) != 0;
    }
  }

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
    const float lse = l_row > 0.f ? (m_ref + log2f(l_row)) * LN2 : -INFINITY;
    const float wc = l_row_rnd > 0.f ? p.v_scale / l_row_rnd : 0.f;
    const int hq = hbase + w;
    const int64_t tq = q0 + lr;
    if (h == 0) {
      sm.epi.wcur[w * 32 + lr] = wc;
      if (p.lse.p && hq < p.Hq && tq < q_len) p.lse.p[b * p.lse.sb + hq * p.lse.sh + tq * p.lse.st] = lse;
    }
  }
  __syncthreads();

  // bf16 rows staged through the idle tile buffers (row stride padded by 16
  // bytes), then stored as whole 1 KB rows, 16 bytes a lane
  constexpr int RS = 512 * 2 + 16;
  constexpr int LPR = 512 * 2 / 16;  // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per store instruction
  static_assert(ROWS * RS <= (int)sizeof(sm.t), "the rows fit the tile buffers");
  const uint32_t stage = lds_t;
#pragma unroll
  for (int rb = 0; rb < WAVES; ++rb) {
    const float wc = sm.epi.wcur[rb * 32 + lr];
    const uint32_t row = stage + (uint32_t)(rb * 32 + lr) * RS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * (w * 4 + j) + 8 * g + 4 * h;
        const u32x2 v = {pack_bf16x2(wc * O[rb][j][4 * g], wc * O[rb][j][4 * g + 1]),
                         pack_bf16x2(wc * O[rb][j][4 * g + 2], wc * O[rb][j][4 * g + 3])};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)(row + d * 2)) = v;
      }
    }
  }
  __syncthreads();
  const int o_nrb = p.Hq - hbase;
  const int o_nrl = (int)min<int64_t>(32, q_len - q0);
  constexpr int NST = ROWS / (WAVES * RPI);  // store instructions per wave
  constexpr int KB = 32 / (WAVES * RPI);     // of them per row block
#pragma unroll 8
  for (int k = 0; k < NST; ++k) {
    const int rs = (w + k * WAVES) * RPI + lane / LPR;  // staged row
    const int rb = k / KB, rl = w * RPI + lane / LPR + (k % KB) * (WAVES * RPI);
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (uintptr_t)(stage + (uint32_t)rs * RS + (lane % LPR) * 16));
    if (rb < o_nrb && rl < o_nrl) {
      uint16_t* o = p.out.p + b * p.out.sb + (hbase + rb) * p.out.sh + (q0 + rl) * p.out.st + (lane % LPR) * 8;
      *reinterpret_cast<u32x4*>(o) = v;
    }
  }
}

__global__ void fp8_queue_reset_kernel(unsigned* q) { q[0] = 0u; }

}  // namespace

hipError_t launch_latent_fp8(const AttnParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.n_qblk * p.n_hgrp * p.B;
  if (items == 0) return hipSuccess;
  AttnParams q = p;
  const int ncu = q.queue ? cu_count() : 0;
  if (ncu > 0 && items > 4 * (int64_t)ncu) hipLaunchKernelGGL(fp8_queue_reset_kernel, dim3(1), dim3(1), 0, s, q.queue);
  else q.queue = nullptr;
  hipLaunchKernelGGL(attn_fwd_fp8_kernel, dim3((unsigned)items), dim3(256), 0, s, q);
  return hipGetLastError();
}

}  // namespace mla
