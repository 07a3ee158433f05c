// The head_dim 64 instance of the bf16 attention kernel (uf_attn_bf16.h), in a translation
// unit of its own: the library builds it with the LLVM AMDGPU scheduling strategy
// "iterative-ilp", which runs the decoder-XL and refine-XL steps 1-2% faster than the default
// (measured side by side; "max-ilp", the head_dim 128 choice, is slower here).  Only the loop
// with one sub-tile per step is built at head_dim 64: the software-pipelined one needs more than
// the 128 registers per wave that four work-groups per CU leave.
#include <hip/hip_runtime.h>

#include "uf_attn_bf16.h"
#include "uf_internal.h"

namespace uf {

hipError_t launch_attention_d64(const AttnParams& p, hipStream_t stream) {
  const int items = p.n_qblk * p.n_hgrp * p.splits;
  hipLaunchKernelGGL((attn_kernel<64, false>), dim3(items), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace uf
