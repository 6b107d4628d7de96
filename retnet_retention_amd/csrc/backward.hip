// Elementwise passes of the parallel form's backward ("Retentive Network: A
// Successor to Transformer...", Elamur summary, Summary: the parallel form is
// the training form). Every matrix product of the gradient is again a causal
// retention product, which the forward kernel computes; these kernels do the
// rest:
//   * gate_norm_bwd_kernel: gradient through the swish gate and the per-head
//     GroupNorm (one wave per token and head, wave reductions over dv);
//   * reverse_tokens_kernel: a copy with the token order of every sequence
//     reversed (the products with the transposed decay mask run on reversed
//     sequences, where that mask is causal again), for inputs that no other
//     pass already writes reversed.
// The rotation's gradient (each pair turned back by its angle) and the
// reversal of the products' outputs happen in the retention kernels' stores.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

// One (token, head) row of D values per D/EPL lanes, EPL elements (16
// bytes) per lane, so a wave takes 64/(D/EPL) rows with 16-byte accesses.
// With y = (o - mean) / sigma, sigma = sqrt(var + eps), s(x) = sigmoid(x):
//   dg = dout * y * s(g) (1 + g (1 - s(g)))
//   dy = dout * g s(g)
//   do = (dy - mean(dy) - y mean(dy y)) / sigma
// dO goes to dov and/or dov_rev (either may be null), the latter at each
// sequence's reversed token positions.
template <typename T, int D>
__global__ __launch_bounds__(256) void gate_norm_bwd_kernel(const T* __restrict__ o, const T* __restrict__ g,
                                                            const T* __restrict__ dout, T* __restrict__ dov,
                                                            T* __restrict__ dg, T* __restrict__ dov_rev,
                                                            int64_t rows, int seqlen, int heads, float eps) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane
  constexpr int LPR = D / EPL;              // lanes per row
  constexpr int RPW = 64 / LPR;             // rows per wave
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  if (row0 >= rows) return;  // whole waves leave together
  const int64_t row = row0 + lane / LPR;
  const bool valid = row < rows;  // the last wave may hold fewer rows: the rest recompute a row and store nothing
  const int64_t rr = valid ? row : rows - 1;
  const int64_t base = rr * D + (lane % LPR) * EPL;
  auto row_sum = [](float v) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 1; w < LPR; w *= 2) v += __shfl_xor(v, w, 64);
    return v;
  };
  float x[EPL], gv[EPL], d[EPL];
  load16f(o + base, x);
  load16f(g + base, gv);
  load16f(dout + base, d);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s += x[i];
  const float mean = row_sum(s) * (1.0f / D);
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s2 += (x[i] - mean) * (x[i] - mean);
  const float rsig = rsqrtf(row_sum(s2) * (1.0f / D) + eps);
  float sdy = 0.f, sdyy = 0.f, dgv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float y = (x[i] - mean) * rsig;
    const float sg = 1.0f / (1.0f + __expf(-gv[i]));
    dgv[i] = d[i] * y * (sg * (1.0f + gv[i] * (1.0f - sg)));
    d[i] = d[i] * gv[i] * sg;  // dy
    x[i] = y;
    sdy += d[i];
    sdyy += d[i] * y;
  }
  const float mdy = row_sum(sdy) * (1.0f / D), mdyy = row_sum(sdyy) * (1.0f / D);
  if (!valid) return;
#pragma unroll
  for (int i = 0; i < EPL; ++i) d[i] = (d[i] - mdy - x[i] * mdyy) * rsig;
  store16f(dg + base, dgv);
  if (dov) store16f(dov + base, d);
  if (dov_rev) {
    const int64_t tok = row / heads, b = tok / seqlen, n = tok % seqlen;
    store16f(dov_rev + ((b * seqlen + (seqlen - 1 - n)) * heads + row % heads) * D + (lane % LPR) * EPL, d);
  }
}

// dst[b][n] = src[b][seqlen - 1 - n], 16 bytes per thread
__global__ __launch_bounds__(256) void reverse_tokens_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             int64_t vecs, int64_t per_tok, int seqlen) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= vecs) return;
  const int64_t tok = i / per_tok, c = i % per_tok;  // tok = b * seqlen + n
  const int64_t b = tok / seqlen, n = tok % seqlen;
  dst[(b * seqlen + (seqlen - 1 - n)) * per_tok + c] = src[i];
}

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

hipError_t launch_gate_norm_bwd(const Shape& s, const void* o, const void* g, const void* dout, void* dov, void* dg,
                                float eps, hipStream_t stream, void* dov_rev) {
  const int64_t rows = (int64_t)s.batch * s.seqlen * s.heads;
  // rows per block: 4 waves of 64 / (D / (16 / element size)) rows
  const int64_t per_block = 4 * 64 / (s.d / (s.dtype == 1 ? 8 : 4));
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
#define RET_GN_BWD(TT, DD)                                                                                       \
  hipLaunchKernelGGL((gate_norm_bwd_kernel<TT, DD>), dim3(blocks), dim3(256), 0, stream, (const TT*)o,          \
                     (const TT*)g, (const TT*)dout, (TT*)dov, (TT*)dg, (TT*)dov_rev, rows, s.seqlen, s.heads, eps)
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: RET_GN_BWD(bf16, 64); break;
      case 128: RET_GN_BWD(bf16, 128); break;
      case 256: RET_GN_BWD(bf16, 256); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (s.d) {
      case 64: RET_GN_BWD(float, 64); break;
      case 128: RET_GN_BWD(float, 128); break;
      case 256: RET_GN_BWD(float, 256); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef RET_GN_BWD
  return hipGetLastError();
}

hipError_t launch_reverse_tokens(const Shape& s, const void* src, void* dst, hipStream_t stream) {
  const int64_t per_tok = (int64_t)s.heads * s.d * (s.dtype == 1 ? 2 : 4) / 16;
  const int64_t vecs = (int64_t)s.batch * s.seqlen * per_tok;
  const unsigned blocks = (unsigned)((vecs + 255) / 256);
  hipLaunchKernelGGL(reverse_tokens_kernel, dim3(blocks), dim3(256), 0, stream, (const uint4*)src, (uint4*)dst, vecs,
                     per_tok, s.seqlen);
  return hipGetLastError();
}

}  // namespace ret
