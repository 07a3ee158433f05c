// The head_dim 128 instance of the bf16 attention kernel (uf_attn_bf16.h), in a translation
// unit of its own: the library builds it with the LLVM AMDGPU scheduling strategy "max-ilp".
// Measured side by side, that schedule runs the 2K, 1K, 480P and decoder steps 1.3-2.3%
// faster than the default; for the head_dim 64 and FP8 kernels it is slower.  Both loops of the
// kernel are built here: one sub-tile per step, and the software-pipelined one.
#include <hip/hip_runtime.h>

#include "uf_attn_bf16.h"
#include "uf_internal.h"

namespace uf {

hipError_t launch_attention_d128(const AttnParams& p, hipStream_t stream) {
  const int items = p.n_qblk * p.n_hgrp * p.splits;
  if (p.pipelined)
    hipLaunchKernelGGL((attn_kernel<128, true>), dim3(items), dim3(kAttnThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_kernel<128, false>), dim3(items), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace uf
