// The split query/key form of the attention kernel (Ascend RingMLAOperation:
// separate nope and RoPE parts of q and k, a separate V, varlen seqLen, the
// prevOut/prevLse fold), in a translation unit of its own so that it can be
// built with the MFMA accumulators in ordinary VGPRs
// (-mllvm=-amdgpu-mfma-vgpr-form, device side only).  The form is held to
// 256 registers (two waves per SIMD), which the score accumulators of two
// key tiles and the output accumulators fit; with the score accumulator in
// AGPRs, as the compiler otherwise placed it, every key tile cost 16
// AGPR->VGPR reads before the softmax and 16 AGPR writes to clear it.  The
// latent and sparse forms keep their output accumulators in AGPRs
// (mla_attn.hip).
#include "mla_attn_kernels.inc"

namespace mla {

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

}  // namespace mla
