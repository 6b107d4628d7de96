// Position-rotation table for the xPos-like encoding of queries and keys
// ("Retentive Network: A Successor to Transformer...", Elamur summary,
// Summary): entry [n][j] = (cos, sin) of (pos_offset + n) * base^(-2j/d).
// Angles are formed and reduced in fp64 and rounded to fp32 once, so a
// position of several thousand radians keeps full fp32 accuracy.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

__global__ __launch_bounds__(256) void rotary_table_kernel(float2* __restrict__ table, int seqlen, int half,
                                                           double base, int64_t pos_offset, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)seqlen * half) return;
  const int n = (int)(idx / half), j = (int)(idx % half);
  const double theta = pow(base, -2.0 * j / d);
  const double phi = (double)(pos_offset + n) * theta;
  double s, c;
  sincos(phi, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rotary_table(float2* table, int seqlen, int d, double base, int64_t pos_offset,
                               hipStream_t stream) {
  const int half = d / 2;
  const int64_t total = (int64_t)seqlen * half;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(rotary_table_kernel, dim3(blocks), dim3(256), 0, stream, table, seqlen, half, base,
                     pos_offset, d);
  return hipGetLastError();
}

}  // namespace ret
