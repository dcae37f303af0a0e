// Launchers of the shared-latent, sparse and decode forms of the attention
// kernel (mla_attn_kernels.inc), the sparse gather test kernel and the item
// queue's reset.  The split form is built in mla_attn_split.hip.
#include "mla_attn_kernels.inc"

#include <algorithm>

namespace mla {
namespace {

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

hipError_t launch_latent_ring(const RingParams& g, hipStream_t s) {
  if (g.n_items == 0) return hipSuccess;
  // one workgroup per CU (each fills a CU's LDS), or fewer when the items are fewer
  const int ncu = cu_count();
  const int grid = std::min(g.n_items, ncu > 0 ? ncu : 256);
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(1), 0, s, g.queue);
  hipLaunchKernelGGL((attn_fwd_ring_kernel<LatentCfg, LATENT>), dim3((unsigned)grid), dim3(256), 0, s, g);
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

hipError_t launch_debug_gather(const GatherParams& p, hipStream_t s) {
  if (p.K == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
