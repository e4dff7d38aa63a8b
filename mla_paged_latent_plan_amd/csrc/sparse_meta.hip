// Metadata of the sparse prefill's flat-buffer view (FlashMLA wrapper, flash_mla_sparse_fwd: every
// query token attends over rows of one flat latent buffer named by its own index list). The
// prefill runs as one request whose positions are the buffer's rows: its length is s_kv and its
// page table maps page i to page i. Both are written here, on the stream, so that the whole call
// stays free of host copies and can be graph-captured.
#include "layer_internal.h"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void sparse_meta_kernel(int32_t* meta, int32_t s_kv, int32_t pages) {
  const int32_t i = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (i == 0) meta[0] = s_kv;              // the request's length
  if (i < pages) meta[1 + i] = i;           // identity page table
}

}  // namespace

hipError_t launch_sparse_meta(int32_t* meta, int32_t s_kv, int32_t pages, hipStream_t s) {
  const int blocks = (pages + 255) / 256;
  hipLaunchKernelGGL(sparse_meta_kernel, dim3(blocks), dim3(256), 0, s, meta, s_kv, pages);
  return hipGetLastError();
}

}  // namespace mla
