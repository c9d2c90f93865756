// The ends of the decode step on the GPU: the embedding gather (the raw bf16
// row of each token, converted to fp32, with no sqrt(hidden) scale and no
// norm: docs.rs turbospark-runtime 0.3.0, src/families/spark/mod.rs,
// `produce_real_spark_inner`).  The final RMSNorm and the tied head reuse the
// norm and GEMV kernels of gqa_kernels.hip.
#include "gqa_internal.h"

namespace gqa {
namespace {

// Workgroup b copies row ids[b] of the table into h[b]: each thread moves
// 8 columns (16 bytes of bf16 in, 32 bytes of fp32 out) per step.
__global__ __launch_bounds__(256) void embed_gather_kernel(const EmbedParams p) {
  const int b = blockIdx.x;
  const uint4 *src = reinterpret_cast<const uint4 *>(p.table + (size_t)p.ids[b] * p.hidden);
  float4 *dst = reinterpret_cast<float4 *>(p.h + (size_t)b * p.hidden);
  for (int g = threadIdx.x; g < p.hidden / 8; g += 256) {
    const uint4 w = src[g];
    dst[2 * g] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                             __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    dst[2 * g + 1] = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                                 __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u));
  }
}

}  // namespace

hipError_t launch_embed_gather(const EmbedParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(embed_gather_kernel, dim3((unsigned)p.count), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
