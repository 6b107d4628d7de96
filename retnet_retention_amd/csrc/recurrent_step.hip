// Recurrent form, one decode step ("Retentive Network: A Successor to
// Transformer...", Elamur summary, Summary: the recurrent form costs O(1) per
// token and needs no KV cache):
//     S <- g S + k^T v,   o = q S,   then GroupNorm + swish gate.
// The step is a pure stream over the fp32 state: 4 * dk * dv bytes read and
// written per (sequence, head) against ~5 * dk * dv flops, so it is bound by
// HBM bandwidth. One workgroup of 512 threads owns one (sequence, head);
// each wave sweeps whole state rows with 16-byte accesses (a 256-wide row is
// one wave-wide 1 KiB access), eight consecutive rows per workgroup sweep, and
// the row loop is unrolled so that many loads are in flight. (512 threads
// reached 6.07 TB/s on the 1 GiB state of batch 256 against 5.43 TB/s with
// 256: more rows of one state in flight at once.)
#include "common.hpp"
#include "launch.hpp"

namespace ret {

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  void* o;
  float* state;
  int heads;
  int rotary;
  double base;
  int64_t pos;
  const int64_t* positions;  // device [batch]: each sequence's own position, or null (all at pos)
  float eps;
  float gam[kMaxHeads];
};

template <typename T> __device__ __forceinline__ float ld1(const T* p, int i) { return (float)p[i]; }

// STREAM: non-temporal state accesses, for states too large to stay in the
// caches from one step to the next.
template <typename T, int D, bool STREAM>
__global__ __launch_bounds__(512) void recurrent_step_kernel(StepParams p) {
  constexpr int CT = D / 4;       // threads across one state row (float4 each)
  constexpr int RPI = 512 / CT;   // rows per sweep iteration
  __shared__ __attribute__((aligned(16))) float sq[D], sk[D], sv[D];
  __shared__ __attribute__((aligned(16))) float part[RPI][D];
  __shared__ float so[D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int h = bh % p.heads;
  const float gam = p.gam[h];
  const int64_t vec = (int64_t)bh * D;  // token row of this (sequence, head): seqlen is 1
  const T* q = reinterpret_cast<const T*>(p.q) + vec;
  const T* k = reinterpret_cast<const T*>(p.k) + vec;
  const T* v = reinterpret_cast<const T*>(p.v) + vec;
  // per-sequence positions: a negative one marks an inactive slot of the
  // batch (its state stays as it is, its output is zero)
  if (p.positions && p.positions[bh / p.heads] < 0) {
    T* o = reinterpret_cast<T*>(p.o) + vec;
    for (int i = tid; i < D; i += 512) o[i] = (T)0.f;
    return;  // uniform for the workgroup
  }

  for (int i = tid; i < D; i += 512) {
    sq[i] = ld1(q, i);
    sk[i] = ld1(k, i);
    sv[i] = ld1(v, i);
  }
  __syncthreads();
  if (p.rotary) {
    const int64_t pos = p.positions ? p.positions[bh / p.heads] : p.pos;
    for (int j = tid; j < D / 2; j += 512) {
      const double theta = pow(p.base, -2.0 * j / D);
      double s, c;
      sincos((double)pos * theta, &s, &c);
      const float cf = (float)c, sf = (float)s;
      const float q0 = sq[2 * j], q1 = sq[2 * j + 1], k0 = sk[2 * j], k1 = sk[2 * j + 1];
      sq[2 * j] = q0 * cf - q1 * sf;
      sq[2 * j + 1] = q0 * sf + q1 * cf;
      sk[2 * j] = k0 * cf - k1 * sf;
      sk[2 * j + 1] = k0 * sf + k1 * cf;
    }
    __syncthreads();
  }

  const int c4 = tid % CT, r0 = tid / CT;
  const float4 vv = *reinterpret_cast<const float4*>(&sv[c4 * 4]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float* S = p.state + (int64_t)bh * D * D + c4 * 4;
  constexpr int kUnroll = STREAM ? 16 : 8;  // loads in flight per thread
#pragma unroll kUnroll
  for (int r = r0; r < D; r += RPI) {
    f32x4* sp = reinterpret_cast<f32x4*>(S + (int64_t)r * D);
    f32x4 s = STREAM ? __builtin_nontemporal_load(sp) : *sp;
    const float kr = sk[r], qr = sq[r];
    s[0] = gam * s[0] + kr * vv.x;
    s[1] = gam * s[1] + kr * vv.y;
    s[2] = gam * s[2] + kr * vv.z;
    s[3] = gam * s[3] + kr * vv.w;
    if constexpr (STREAM)
      __builtin_nontemporal_store(s, sp);
    else
      *sp = s;
    acc.x += qr * s[0];
    acc.y += qr * s[1];
    acc.z += qr * s[2];
    acc.w += qr * s[3];
  }
  *reinterpret_cast<float4*>(&part[r0][c4 * 4]) = acc;
  __syncthreads();
  for (int j = tid; j < D; j += 512) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPI; ++r) s += part[r][j];
    so[j] = s;
  }
  __syncthreads();

  if (tid < 64) {
    constexpr int PER = D / 64;
    float x[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) x[m] = so[tid + 64 * m];
    T* o = reinterpret_cast<T*>(p.o) + vec;
    if (p.g) {
      const T* gp = reinterpret_cast<const T*>(p.g) + vec;
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < PER; ++m) sum += x[m];
      const float mean = sum64(sum) * (1.0f / D);
      float sq2 = 0.f;
#pragma unroll
      for (int m = 0; m < PER; ++m) sq2 += (x[m] - mean) * (x[m] - mean);
      const float rstd = rsqrtf(sum64(sq2) * (1.0f / D) + p.eps);
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const float gv = ld1(gp, tid + 64 * m);
        o[tid + 64 * m] = (T)((x[m] - mean) * rstd * swish(gv));
      }
    } else {
#pragma unroll
      for (int m = 0; m < PER; ++m) o[tid + 64 * m] = (T)x[m];
    }
  }
}

// States above this size do not stay in the caches between steps.
constexpr size_t kStreamStateBytes = size_t(512) << 20;

template <typename T, int D>
static hipError_t launch_step_t(const Shape& s, const StepParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)s.batch * (unsigned)s.heads;
  if ((size_t)blocks * D * D * sizeof(float) > kStreamStateBytes)
    hipLaunchKernelGGL((recurrent_step_kernel<T, D, true>), dim3(blocks), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_step_kernel<T, D, false>), dim3(blocks), dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_recurrent_step(const Shape& s, const void* q, const void* k, const void* v, const void* g,
                                 void* o, float* state, double rotary_base, int64_t pos, float eps,
                                 hipStream_t stream, const int64_t* positions) {
  StepParams p;
  p.positions = positions;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.o = o;
  p.state = state;
  p.heads = s.heads;
  p.rotary = rotary_base != 0.0;
  p.base = rotary_base;
  p.pos = pos;
  p.eps = eps;
  for (int h = 0; h < kMaxHeads; ++h) p.gam[h] = h < s.heads ? s.gam[h] : 0.f;
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_step_t<bf16, 64>(s, p, stream);
      case 128: return launch_step_t<bf16, 128>(s, p, stream);
      case 256: return launch_step_t<bf16, 256>(s, p, stream);
    }
  } else {
    switch (s.d) {
      case 64: return launch_step_t<float, 64>(s, p, stream);
      case 128: return launch_step_t<float, 128>(s, p, stream);
      case 256: return launch_step_t<float, 256>(s, p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ret
