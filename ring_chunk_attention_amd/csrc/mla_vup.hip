// V-up projection of the latent attention output (TensorRT-LLM mla.py,
// forward_absorption_context and forward_absorption_generation: after the
// attention over the shared latent rows, a per-head batched product
// [heads, tokens, kv_lora_rank] x [heads, kv_lora_rank, v_head_dim] gives the
// per-head values that o_proj reads):
//
//   out[b, h, t, c] = sum_l o[b, h, t, l] * w[h, c, l],   l < 512, c < 128
//
// The product does 2 * 128 = 256 flops per element of o (128 per byte), far
// below the ~315 flop/byte at which the chip turns MFMA-bound, so the kernel
// is bound by reading o from HBM.  Design:
//  * One workgroup (8 waves, two per SIMD) serves one head and a range of
//    32-row blocks of that head.  The head's 128 x 512 weight (128 KB) is
//    copied into LDS once per workgroup; rows are padded by 16 bytes so that
//    the 32 rows an MFMA fragment read touches start 4 banks apart.
//  * Each wave takes row blocks in turn: its 32 rows (32 KB) go straight from
//    HBM into VGPRs as the B operand of v_mfma_f32_32x32x16_bf16, and
//    out^T = W o^T is 4 column blocks x 32 k-steps = 128 MFMA with the weight
//    rows as the A operand from LDS.  Two waves per SIMD let one wave's loads
//    overlap the other's products.
//  * The accumulator holds one output row per lane (4 consecutive columns per
//    register group).  Stored from there, every store instruction would
//    write 16 bytes into each of 32 rows; instead the rows pass through a
//    small per-wave LDS area, 8 at a time, and leave as whole 256-byte rows
//    (16 lanes a row), which measured 15% faster for the whole kernel.
//  * MX 4-pack input (the sparse kernel's optional column order): the
//    contraction order is free, so the weight is staged with its columns in
//    the same order and the main loop is unchanged.
#include "mla_internal.h"

#include <algorithm>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int VL = 512;              // latent columns (the contraction)
constexpr int VC = 128;              // value columns per head
constexpr int VWAVES = 8;            // waves per workgroup
constexpr int WROW = VL * 2 + 16;    // LDS bytes per staged weight row
constexpr int OROWS = 8;             // output rows staged per wave and pass
constexpr int OSTG = OROWS * VC * 2; // LDS bytes of a wave's output staging

__device__ __forceinline__ unsigned pack2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint32_t a) {
  return reinterpret_cast<__attribute__((address_space(3))) T*>((uintptr_t)a);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
void vup_kernel(const VupParams p) {
  __shared__ alignas(16) unsigned char wl[VC * WROW + VWAVES * OSTG];
  const int h = (int)(blockIdx.x % (unsigned)p.H);
  const int64_t part = blockIdx.x / (unsigned)p.H;
  const int64_t M = (int64_t)p.B * p.T;              // rows of one head
  const int64_t nblk = (M + 31) / 32;
  const int64_t blk0 = part * p.blocks_per_part;
  const int64_t blk1 = min(nblk, blk0 + p.blocks_per_part);
  if (blk0 >= blk1) return;                          // the whole workgroup

  // the head's weight -> LDS (16 bytes a lane, coalesced along the rows)
  const uint16_t* wh = p.w + (int64_t)h * VC * VL;
  for (int i = threadIdx.x; i < VC * VL / 8; i += VWAVES * 64) {
    const int c = i / (VL / 8), l0 = (i % (VL / 8)) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(wh + c * VL + l0);
    const uint32_t row = lds_addr(&wl[0]) + c * WROW;
    if (!p.mx4) {
      *lds_ptr<u32x4>(row + l0 * 2) = v;
    } else {
      // natural column l = 4 * group + sub sits at sub * VL / 4 + group of o
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int l = l0 + e;
        *lds_ptr<uint16_t>(row + ((l % 4) * (VL / 4) + l / 4) * 2) = (uint16_t)(v[e / 2] >> (16 * (e % 2)));
      }
    }
  }
  __syncthreads();

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, hi = lane >> 5;
  // this lane's A fragments: weight row 32 * cb + lr, columns 16 * ks + 8 * hi
  const uint32_t wbase = lds_addr(&wl[0]) + lr * WROW + hi * 16;
  for (int64_t blk = blk0 + wv; blk < blk1; blk += VWAVES) {
    const int64_t m = blk * 32 + lr;
    const bool ok = m < M;
    const int64_t mm = ok ? m : blk * 32;            // rows past the end read the block's first
    const int64_t b = mm / p.T, t = mm % p.T;
    const uint16_t* orow = p.o.p + b * p.o.sb + h * p.o.sh + t * p.o.st + hi * 8;
    // out row of this lane's row m (rows past the end: the block's first row, never stored)
    uint16_t* dst = p.out.p + b * p.out.sb + h * p.out.sh + t * p.out.st;
    bf16x8 ob[VL / 16];
#pragma unroll
    for (int ks = 0; ks < VL / 16; ++ks)
      ob[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(orow + 16 * ks));
    f32x16 acc[VC / 32];
#pragma unroll
    for (int cb = 0; cb < VC / 32; ++cb) acc[cb] = f32x16{};
    // weight fragments one k-step ahead of the products; the scheduling
    // barriers keep the compiler from hoisting all 128 LDS reads at once
    bf16x8 a[2][VC / 32];
#pragma unroll
    for (int cb = 0; cb < VC / 32; ++cb) a[0][cb] = __builtin_bit_cast(bf16x8, *lds_ptr<u32x4>(wbase + cb * 32 * WROW));
#pragma unroll
    for (int ks = 0; ks < VL / 16; ++ks) {
      if (ks + 1 < VL / 16) {
#pragma unroll
        for (int cb = 0; cb < VC / 32; ++cb)
          a[(ks + 1) % 2][cb] = __builtin_bit_cast(bf16x8, *lds_ptr<u32x4>(wbase + cb * 32 * WROW + (ks + 1) * 32));
      }
#pragma unroll
      for (int cb = 0; cb < VC / 32; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % 2][cb], ob[ks], acc[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage OROWS rows at a time in LDS (16-byte chunks XOR-swizzled by row
    // against bank conflicts) and store them as whole 256-byte rows, 16
    // lanes a row.  The lane numbers are laundered here, so that the compiler
    // computes the staging addresses in the loop instead of holding all of
    // them live across it.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr2 = ln & 31, hi2 = ln >> 5;
    const uint32_t stg = lds_addr(&wl[0]) + VC * WROW + wv * OSTG;
#pragma unroll
    for (int pass = 0; pass < 32 / OROWS; ++pass) {
      const int r = lr2 - pass * OROWS;
      if (r >= 0 && r < OROWS) {
#pragma unroll
        for (int cb = 0; cb < VC / 32; ++cb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2 v = {pack2(acc[cb][4 * g], acc[cb][4 * g + 1]), pack2(acc[cb][4 * g + 2], acc[cb][4 * g + 3])};
            const int chunk = (4 * cb + g) ^ r;
            *lds_ptr<u32x2>(stg + r * (VC * 2) + chunk * 16 + hi2 * 8) = v;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < OROWS / 4; ++k) {
        const int rr = 4 * k + ln / 16, chunk = ln % 16;
        const u32x4 v = *lds_ptr<u32x4>(stg + rr * (VC * 2) + (chunk ^ rr) * 16);
        const int src = pass * OROWS + rr;  // lane that owns the row
        const uint64_t d = ((uint64_t)__shfl((int)((uint64_t)dst >> 32), src) << 32) |
                           (uint32_t)__shfl((int)(uint32_t)(uint64_t)dst, src);
        const bool rok = blk * 32 + src < M;
        if (rok) *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(d) + chunk * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace

hipError_t launch_vup(const VupParams& p0, hipStream_t s) {
  VupParams p = p0;
  const int64_t nblk = ((int64_t)p.B * p.T + 31) / 32;
  if (nblk == 0 || p.H == 0) return hipSuccess;
  // about one workgroup per CU over all heads (a workgroup's 130 KB of LDS
  // leaves room for one: a second round would stage every head's weight
  // again; one round measured 2% faster than two), each with at least 16
  // row blocks (two per wave) so that the weight copy stays a small part
  const int ncu = cu_count() > 0 ? cu_count() : 256;
  int64_t parts = ((int64_t)ncu + p.H - 1) / p.H;
  parts = std::max<int64_t>(1, std::min<int64_t>(parts, (nblk + 15) / 16));
  p.blocks_per_part = (nblk + parts - 1) / parts;
  parts = (nblk + p.blocks_per_part - 1) / p.blocks_per_part;
  hipLaunchKernelGGL(vup_kernel, dim3((unsigned)(parts * p.H)), dim3(VWAVES * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
