// LSE merge of two partial attention results over disjoint key sets
// (TensorRT-LLM mla.py, forward_context_with_chunked_prefill: partial outputs
// merged with their softmax stats; Ascend RingMLAOperation prevOut/prevLse).
//
// HBM-bound elementwise kernel: a wave folds two output rows; each lane
// moves 16 bytes of each operand per row, so a 512-column bf16 row is one
// fully coalesced 1 KB access per operand.  Both rows' pieces and LSE values
// are loaded before any is used (a side whose LSE is -inf is loaded and then
// given weight 0 by a select, never multiplied), so that a wave waits for
// one memory round trip for four rows of input.  (Measured at
// [1, 16, 1024, 512]: one row a wave 12.7 us, two 12.4, four 13.1, eight
// over 20.)  A row's
// two LSE values are read by every lane before lane 0 writes the merged LSE,
// and every output element is read and written by the same lane, so out/lse
// may alias the a or b side.
#include "mla_internal.h"

#include <math.h>

namespace mla {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

constexpr int kMergeRowsPerWave = 2;

__device__ __forceinline__ void fold_piece(const u32x4& va, const u32x4& vb, float wa, float wb, uint16_t* dst) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // a side of weight 0 contributes exactly 0, whatever its row holds
    const float a0 = wa * __uint_as_float(va[e] << 16), a1 = wa * __uint_as_float(va[e] & 0xffff0000u);
    const float b0 = wb * __uint_as_float(vb[e] << 16), b1 = wb * __uint_as_float(vb[e] & 0xffff0000u);
    y[2 * e] = (wa != 0.f ? a0 : 0.f) + (wb != 0.f ? b0 : 0.f);
    y[2 * e + 1] = (wa != 0.f ? a1 : 0.f) + (wb != 0.f ? b1 : 0.f);
  }
  const u32x4 o = {pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
  *reinterpret_cast<u32x4*>(dst) = o;
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void merge_kernel(const MergeParams p) {
  constexpr int R = kMergeRowsPerWave;
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int lane = threadIdx.x & 63;
  if (row0 >= rows) return;
  const bool first = lane * 8 < p.dv;  // this lane's piece of the first 512 columns

  const uint16_t* ra[R];
  const uint16_t* rb[R];
  uint16_t* ro[R];
  float* rl[R];
  u32x4 va[R], vb[R];
  float la[R], lb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = min(row0 + r, rows - 1);  // a tail wave repeats its last row (not stored)
    const int64_t t = row % p.N, bh = row / p.N;
    const int64_t hh = bh % p.H, b = bh / p.H;
    ra[r] = p.oa.p + b * p.oa.sb + hh * p.oa.sh + t * p.oa.st;
    rb[r] = p.ob.p + b * p.ob.sb + hh * p.ob.sh + t * p.ob.st;
    ro[r] = p.out.p + b * p.out.sb + hh * p.out.sh + t * p.out.st;
    rl[r] = p.lse.p ? p.lse.p + b * p.lse.sb + hh * p.lse.sh + t * p.lse.st : nullptr;
    va[r] = vb[r] = u32x4{0u, 0u, 0u, 0u};
    if (first) {
      va[r] = *reinterpret_cast<const u32x4*>(ra[r] + lane * 8);
      vb[r] = *reinterpret_cast<const u32x4*>(rb[r] + lane * 8);
    }
    la[r] = p.la.p[b * p.la.sb + hh * p.la.sh + t * p.la.st];
    lb[r] = p.lb.p[b * p.lb.sb + hh * p.lb.sh + t * p.lb.st];
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (row0 + r >= rows) break;
    const float mx = fmaxf(la[r], lb[r]);
    float L, wa, wb;
    if (mx == -INFINITY) {
      L = -INFINITY; wa = 0.f; wb = 0.f;
    } else {
      const float ea = la[r] == -INFINITY ? 0.f : expf(la[r] - mx);
      const float eb = lb[r] == -INFINITY ? 0.f : expf(lb[r] - mx);
      const float z = ea + eb;
      L = mx + logf(z);
      wa = ea / z;
      wb = eb / z;
    }
    if (first) fold_piece(va[r], vb[r], wa, wb, ro[r] + lane * 8);
    for (int c = lane + 64; c * 8 < p.dv; c += 64)  // columns past 512
      fold_piece(*reinterpret_cast<const u32x4*>(ra[r] + c * 8), *reinterpret_cast<const u32x4*>(rb[r] + c * 8),
                 wa, wb, ro[r] + c * 8);
    if (lane == 0 && rl[r]) *rl[r] = L;
  }
}

// Split-K reduction of token generation (Mojo mha_single_batch_pipelined,
// token-generation description: the partial results of a key split are
// combined afterwards by a kernel of their own): for each (b, h),
// L = log sum_s exp(L_s) and out = sum_s exp(L_s - L) O_s over the S
// partial results (a partial with L_s = -inf has weight 0).  HBM-bound: one
// wave per row; lane s holds split s's LSE for the
// wave reductions, then each lane sums 8 columns over the splits (two
// 16-byte reads per split, a coalesced 2 KB per split and row).
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void combine_kernel(const CombineParams p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)p.B * p.H) return;  // whole wave
  const int64_t b = row / p.H, hh = row % p.H;
  const float ls = lane < p.S ? p.pl[(b * p.S + lane) * p.H + hh] : -INFINITY;
  float mx = ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float e = ls == -INFINITY ? 0.f : expf(ls - mx);
  float z = e;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  const bool live = mx != -INFINITY;
  const float L = live ? mx + logf(z) : -INFINITY;
  const float wgt = live ? e / z : 0.f;  // this lane's split's weight
  uint16_t* ro = p.out.p + b * p.out.sb + hh * p.out.sh;
  for (int c = lane; c * 8 < p.dv; c += 64) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = 0.f;
    // every partial row is written by the attention kernel (an empty range
    // as 0 with weight 0), so the loop reads them all, four splits' loads
    // in flight at a time
    const float* src = p.po + (b * p.S * p.H + hh) * p.dv + c * 8;
    const int64_t sstep = (int64_t)p.H * p.dv;
#pragma unroll 4
    for (int sp = 0; sp < p.S; ++sp) {
      const float ws = __shfl(wgt, sp);
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + sp * sstep);
      const f32x4 a2 = *reinterpret_cast<const f32x4*>(src + sp * sstep + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[k] += ws * a[k];
        y[4 + k] += ws * a2[k];
      }
    }
    u32x4 o = {pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
    *reinterpret_cast<u32x4*>(ro + c * 8) = o;
  }
  if (lane == 0 && p.lse.p) p.lse.p[b * p.lse.sb + hh * p.lse.sh] = L;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  if (rows == 0) return hipSuccess;
  const int64_t per_block = 4 * kMergeRowsPerWave;
  const int64_t blocks = (rows + per_block - 1) / per_block;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
