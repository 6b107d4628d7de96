// Position rotation of queries and keys, the xPos-like encoding of
// "Retentive Network: A Successor to Transformer..." (Elamur summary,
// Summary). Two passes, or both in one launch (rotate_keys_table_kernel):
//   * a table [n][j] = (cos, sin) of (pos_offset + n) * base^(-2j/d), the
//     angle formed and reduced in fp64 and rounded to fp32 once, so a
//     position of several thousand radians keeps full fp32 accuracy;
//   * a streaming pass that turns every adjacent pair (x_2j, x_2j+1) of q and
//     k by its angle and stores the rotated copies in the input dtype, once,
//     so the retention kernels read them as plain tiles.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

// One thread per pair j and kRotPositions consecutive positions: the
// frequency base^(-2j/d) is formed once per thread, the angles per position.
constexpr int kRotPositions = 4;
__global__ __launch_bounds__(256) void rotary_table_kernel(float2* __restrict__ table, int seqlen, int half,
                                                           double base, int64_t pos_offset, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t groups = (seqlen + kRotPositions - 1) / kRotPositions;
  if (idx >= groups * half) return;
  const int j = (int)(idx % half);
  const int n0 = (int)(idx / half) * kRotPositions;
  const double theta = pow(base, -2.0 * j / d);
#pragma unroll
  for (int i = 0; i < kRotPositions; ++i) {
    const int n = n0 + i;
    if (n >= seqlen) break;
    const double phi = (double)(pos_offset + n) * theta;
    double s, c;
    sincos(phi, &s, &c);
    table[(int64_t)n * half + j] = make_float2((float)c, (float)s);
  }
}

hipError_t launch_rotary_table(float2* table, int seqlen, int d, double base, int64_t pos_offset,
                               hipStream_t stream) {
  const int half = d / 2;
  const int64_t total = (int64_t)((seqlen + kRotPositions - 1) / kRotPositions) * half;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(rotary_table_kernel, dim3(blocks), dim3(256), 0, stream, table, seqlen, half, base,
                     pos_offset, d);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void rotate_keys_kernel(const T* __restrict__ k, T* __restrict__ kr,
                                                           T* __restrict__ krev, const float2* __restrict__ table,
                                                           int64_t chunks, int seqlen, int heads, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-element chunk
  if (idx >= chunks) return;
  const int cpr = d / 8;                                     // chunks per head vector
  const int64_t vec = idx / cpr;                             // (b, n, h) row
  const int c8 = (int)(idx % cpr);
  const int n = (int)((vec / heads) % seqlen);
  const CS4 cs = ld_cs4(table + (int64_t)n * (d / 2) + c8 * 4);
  const int64_t off = idx * 8;
  F8 y = unpack8(ld_raw8(k + off));
  rotate4(y, cs);
  if (kr) store8(kr + off, y);
  if (krev) {  // the same row at the reversed position of its sequence
    const int64_t b = vec / heads / seqlen;
    const int h = (int)(vec % heads);
    store8(krev + ((b * seqlen + (seqlen - 1 - n)) * heads + h) * d + c8 * 8, y);
  }
}

// The table and the pass above in one launch: each block takes
// kFusedPositions consecutive positions, forms their table rows first (the
// same fp64 formula as rotary_table_kernel, so the same bits), writes them
// for the retention kernels' query rotation and keeps them in LDS, then turns
// every (sequence, head) row at those positions. A position's rows of one
// sequence are contiguous (heads x d elements), so consecutive threads take
// consecutive 16-byte chunks.
constexpr int kFusedPositions = 2;
template <typename T>
__global__ __launch_bounds__(256) void rotate_keys_table_kernel(const T* __restrict__ k, T* __restrict__ kr,
                                                                 T* __restrict__ krev, float2* __restrict__ table,
                                                                 int batch, int seqlen, int heads, int d,
                                                                 double base, int64_t pos_offset) {
  __shared__ __attribute__((aligned(16))) float2 cs[kFusedPositions][128];
  const int n0 = (int)blockIdx.x * kFusedPositions;
  const int half = d / 2;
  for (int i = threadIdx.x; i < kFusedPositions * half; i += 256) {
    const int p = i / half, j = i % half, n = n0 + p;
    if (n >= seqlen) continue;
    const double theta = pow(base, -2.0 * j / d);
    const double phi = (double)(pos_offset + n) * theta;
    double sn, c;
    sincos(phi, &sn, &c);
    const float2 v = make_float2((float)c, (float)sn);
    cs[p][j] = v;
    table[(int64_t)n * half + j] = v;
  }
  __syncthreads();
  const int cpr = d / 8;  // chunks per head vector
  const int per_seq = heads * cpr;
  const int per_pos = batch * per_seq;
  for (int i = threadIdx.x; i < kFusedPositions * per_pos; i += 256) {
    const int p = i / per_pos, r = i % per_pos, n = n0 + p;
    if (n >= seqlen) continue;
    const int b = r / per_seq, hc = r % per_seq, c8 = hc % cpr;
    const int64_t row = (int64_t)b * seqlen + n;
    const int64_t off = row * heads * d + (int64_t)hc * 8;
    const CS4 t = ld_cs4(&cs[p][4 * c8]);
    F8 y = unpack8(ld_raw8(k + off));
    rotate4(y, t);
    if (kr) store8(kr + off, y);
    if (krev) store8(krev + ((int64_t)b * seqlen + (seqlen - 1 - n)) * heads * d + (int64_t)hc * 8, y);
  }
}

hipError_t launch_rotate_keys_table(const void* k, void* kr, float2* table, int batch, int seqlen, int heads, int d,
                                    int dtype, double base, int64_t pos_offset, hipStream_t stream, void* krev) {
  if (d / 2 > 128) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((seqlen + kFusedPositions - 1) / kFusedPositions);
  if (dtype == 1)
    hipLaunchKernelGGL(rotate_keys_table_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, (const bf16*)k,
                       (bf16*)kr, (bf16*)krev, table, batch, seqlen, heads, d, base, pos_offset);
  else
    hipLaunchKernelGGL(rotate_keys_table_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)k,
                       (float*)kr, (float*)krev, table, batch, seqlen, heads, d, base, pos_offset);
  return hipGetLastError();
}

// Packed sequences: blocks of one sequence each (per_seq blocks per
// sequence), thread = one 8-element chunk of the sequence's rows.
template <typename T>
__global__ __launch_bounds__(256) void rotate_keys_packed_kernel(const T* __restrict__ k, T* __restrict__ kr,
                                                                 const float2* __restrict__ table,
                                                                 const int* __restrict__ cu, int per_seq, int total,
                                                                 int maxlen, int heads, int d) {
  const int b = uniform_i((int)(blockIdx.x / per_seq));
  int tok0, len;
  packed_span(cu, b, total, maxlen, tok0, len);  // a clamp is reported by the chunkwise kernel
  const int cpr = d / 8;  // chunks per head vector
  const int64_t idx = (int64_t)(blockIdx.x % per_seq) * 256 + threadIdx.x;
  if (idx >= (int64_t)len * heads * cpr) return;
  const int n = (int)(idx / ((int64_t)heads * cpr));
  const int c8 = (int)(idx % cpr);
  const CS4 cs = ld_cs4(table + (int64_t)n * (d / 2) + c8 * 4);
  const int64_t off = ((int64_t)tok0 * heads * cpr + idx) * 8;
  F8 y = unpack8(ld_raw8(k + off));
  rotate4(y, cs);
  store8(kr + off, y);
}

hipError_t launch_rotate_keys_packed(const void* k, void* kr, const float2* table, const int* cu, int batch,
                                     int total, int maxlen, int heads, int d, int dtype, hipStream_t stream) {
  const int64_t per = ((int64_t)maxlen * heads * (d / 8) + 255) / 256;
  if (per < 1 || per * batch > 0x7fffffff) return hipErrorInvalidConfiguration;
  const unsigned blocks = (unsigned)(per * batch);
  if (dtype == 1)
    hipLaunchKernelGGL(rotate_keys_packed_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, (const bf16*)k,
                       (bf16*)kr, table, cu, (int)per, total, maxlen, heads, d);
  else
    hipLaunchKernelGGL(rotate_keys_packed_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)k,
                       (float*)kr, table, cu, (int)per, total, maxlen, heads, d);
  return hipGetLastError();
}

hipError_t launch_rotate_keys(const void* k, void* kr, const float2* table, int batch, int seqlen, int heads, int d,
                              int dtype, hipStream_t stream, void* krev) {
  const int64_t chunks = (int64_t)batch * seqlen * heads * (d / 8);
  const unsigned blocks = (unsigned)((chunks + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(rotate_keys_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, (const bf16*)k, (bf16*)kr,
                       (bf16*)krev, table, chunks, seqlen, heads, d);
  else
    hipLaunchKernelGGL(rotate_keys_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)k, (float*)kr,
                       (float*)krev, table, chunks, seqlen, heads, d);
  return hipGetLastError();
}

}  // namespace ret
