// Elementwise passes of the backward ("Retentive Network: A Successor to
// Transformer...", Elamur summary, Summary: the parallel form is the
// training form). Every matrix product of the gradient is again a causal
// retention product, which the forward kernels compute; the gradient through
// the swish gate and the per-head GroupNorm is formed in the epilogue of the
// recomputed forward. The products with the transposed decay mask run on
// reversed sequences, where that mask is causal again: the retention
// kernels read their reversed operands in reversed order (or take the copy
// the rotation pass writes), turn their stored rows back by the rotation's
// angles and store them at reversed positions. What is left here:
//   * state_map_kernel: per-head scaled (and transposed) copies of carried
//     states.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

// Per (sequence, head) D x D fp32 states: dst = scale_h * src, or its
// transpose; the scale per head comes from the host.
struct StateMapParams {
  const float* src;
  float* dst;
  int heads, transpose;
  int64_t total;  // batch * heads * D * D
  float scale[kMaxHeads];
};

template <int D>
__global__ __launch_bounds__(256) void state_map_kernel(StateMapParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.total) return;
  const int64_t mat = i / (D * D);
  const int r = (int)((i / D) % D), c = (int)(i % D);
  const float x = p.src[i] * p.scale[mat % p.heads];
  p.dst[p.transpose ? mat * D * D + (int64_t)c * D + r : i] = x;
}

hipError_t launch_state_map(const Shape& s, const float* src, float* dst, bool transpose, const float* scale,
                            hipStream_t stream) {
  StateMapParams p;
  p.src = src;
  p.dst = dst;
  p.heads = s.heads;
  p.transpose = transpose ? 1 : 0;
  p.total = (int64_t)s.batch * s.heads * s.d * s.d;
  for (int h = 0; h < kMaxHeads; ++h) p.scale[h] = h < s.heads ? scale[h] : 0.f;
  const unsigned blocks = (unsigned)((p.total + 255) / 256);
  switch (s.d) {
    case 64: hipLaunchKernelGGL(state_map_kernel<64>, dim3(blocks), dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(state_map_kernel<128>, dim3(blocks), dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL(state_map_kernel<256>, dim3(blocks), dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


}  // namespace ret
