// LSE merge of two partial attention results over disjoint key sets
// (TensorRT-LLM mla.py, forward_context_with_chunked_prefill: partial outputs
// merged with their softmax stats; Ascend RingMLAOperation prevOut/prevLse).
//
// HBM-bound elementwise kernel: one wave per output row, each lane moves
// 16 bytes of each operand per step, so a 512-column bf16 row is one fully
// coalesced 1 KB access per operand.  The row's two LSE values are read by
// every lane before lane 0 writes the merged LSE, and every output element is
// read and written by the same lane, so out/lse may alias the a or b side.
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

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void merge_kernel(const MergeParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t t = row % p.N;
  const int64_t bh = row / p.N;
  const int64_t hh = bh % p.H, b = bh / p.H;

  const float la = p.la.p[b * p.la.sb + hh * p.la.sh + t * p.la.st];
  const float lb = p.lb.p[b * p.lb.sb + hh * p.lb.sh + t * p.lb.st];
  const float mx = fmaxf(la, lb);
  float L, wa, wb;
  if (mx == -INFINITY) {
    L = -INFINITY; wa = 0.f; wb = 0.f;
  } else {
    const float ea = la == -INFINITY ? 0.f : expf(la - mx);
    const float eb = lb == -INFINITY ? 0.f : expf(lb - mx);
    const float z = ea + eb;
    L = mx + logf(z);
    wa = ea / z;
    wb = eb / z;
  }
  const uint16_t* ra = p.oa.p + b * p.oa.sb + hh * p.oa.sh + t * p.oa.st;
  const uint16_t* rb = p.ob.p + b * p.ob.sb + hh * p.ob.sh + t * p.ob.st;
  uint16_t* ro = p.out.p + b * p.out.sb + hh * p.out.sh + t * p.out.st;
  for (int c = lane; c * 8 < p.dv; c += 64) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.f;
    if (wa != 0.f) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(ra + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] += wa * __uint_as_float(va[e] << 16);
        y[2 * e + 1] += wa * __uint_as_float(va[e] & 0xffff0000u);
      }
    }
    if (wb != 0.f) {
      const u32x4 vb = *reinterpret_cast<const u32x4*>(rb + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] += wb * __uint_as_float(vb[e] << 16);
        y[2 * e + 1] += wb * __uint_as_float(vb[e] & 0xffff0000u);
      }
    }
    u32x4 o = {pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
    *reinterpret_cast<u32x4*>(ro + c * 8) = o;
  }
  if (lane == 0 && p.lse.p) p.lse.p[b * p.lse.sb + hh * p.lse.sh + t * p.lse.st] = L;
}

// Split-K reduction of token generation (Mojo mha_single_batch_pipelined: a
// split over the keys needs a separate reduction kernel at the end): for
// each (b, h), L = log sum_s exp(L_s) and out = sum_s exp(L_s - L) O_s over
// the S partial results (a partial with L_s = -inf has weight 0).  HBM-bound: one wave per row; lane s holds split s's LSE for the
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
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
