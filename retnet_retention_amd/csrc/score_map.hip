// Retention score map of one query token ("Visualization of the retention
// mechanism", SpiralAI model card page: the magnitude of each head's
// query-key dot product, summed across heads; here with the parallel form's
// per-head decay of the distance):
//     w[b, m] = sum_h g_h^(n-m) |q'_{b,n,h} . k'_{b,m,h}|   for m <= n, else 0.
// A pure stream over k (each key token read once) against one query row per
// (sequence, head). One wave per (sequence, key token): lanes take 8
// consecutive elements of one head, D/8 lanes per head, so a wave covers
// 64/(D/8) heads per pass with 16-byte loads; the per-head inner products
// reduce inside their lane groups, the heads' weighted magnitudes across the
// wave.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

struct ScoreParams {
  const void* q;
  const void* k;
  const float2* table;  // (cos, sin) [seqlen][D/2] of the rotation, or null
  float* out;
  int batch, seqlen, heads, qpos;
  float log2g[kMaxHeads];
};

template <typename T, int D>
__global__ __launch_bounds__(256) void score_map_kernel(ScoreParams p) {
  constexpr int LPH = D / 8;    // lanes per head
  constexpr int HPW = 64 / LPH;  // heads per wave pass
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * seqlen + m
  if (tok >= (int64_t)p.batch * p.seqlen) return;  // whole waves leave together
  const int m = (int)(tok % p.seqlen);
  const int64_t b = tok / p.seqlen;
  if (m > p.qpos) {
    if (lane == 0) p.out[tok] = 0.f;
    return;
  }
  const int hl = lane / LPH, e0 = (lane % LPH) * 8;
  const T* K = reinterpret_cast<const T*>(p.k) + tok * p.heads * D;
  const T* Q = reinterpret_cast<const T*>(p.q) + (b * p.seqlen + p.qpos) * p.heads * D;
  float acc = 0.f;
  for (int h0 = 0; h0 < p.heads; h0 += HPW) {
    const int h = h0 + hl;
    float dot = 0.f;
    if (h < p.heads) {
      F8 kv = unpack8(ld_raw8(K + h * D + e0));
      F8 qv = unpack8(ld_raw8(Q + h * D + e0));
      if (p.table) {
        rotate4(kv, ld_cs4(p.table + (int64_t)m * (D / 2) + e0 / 2));
        rotate4(qv, ld_cs4(p.table + (int64_t)p.qpos * (D / 2) + e0 / 2));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += qv.x[i] * kv.x[i];
    }
#pragma unroll
    for (int w = 1; w < LPH; w *= 2) dot += __shfl_xor(dot, w, 64);
    if (h < p.heads && lane % LPH == 0)
      acc += __builtin_amdgcn_exp2f((float)(p.qpos - m) * p.log2g[h]) * fabsf(dot);
  }
  acc = sum64(acc);
  if (lane == 0) p.out[tok] = acc;
}

hipError_t launch_score_map(const Shape& s, const void* q, const void* k, const float2* table, int qpos, float* out,
                            hipStream_t stream) {
  ScoreParams p;
  p.q = q;
  p.k = k;
  p.table = table;
  p.out = out;
  p.batch = s.batch;
  p.seqlen = s.seqlen;
  p.heads = s.heads;
  p.qpos = qpos;
  for (int h = 0; h < kMaxHeads; ++h) p.log2g[h] = h < s.heads ? s.log2g[h] : 0.f;
  const int64_t waves = (int64_t)s.batch * s.seqlen;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
#define RET_SCORE(TT, DD) \
  hipLaunchKernelGGL((score_map_kernel<TT, DD>), dim3(blocks), dim3(256), 0, stream, p)
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: RET_SCORE(bf16, 64); break;
      case 128: RET_SCORE(bf16, 128); break;
      case 256: RET_SCORE(bf16, 256); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (s.d) {
      case 64: RET_SCORE(float, 64); break;
      case 128: RET_SCORE(float, 128); break;
      case 256: RET_SCORE(float, 256); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef RET_SCORE
  return hipGetLastError();
}

}  // namespace ret
