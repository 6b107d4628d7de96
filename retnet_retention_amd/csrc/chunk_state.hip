// Cross-chunk state of the chunkwise form ("Retentive Network: A Successor
// to Transformer...", Elamur summary, Summary: the chunkwise form passes the
// recurrent state between chunks):
//     R_i = K_i^T (V_i (.) zeta) + g^b R_{i-1},   zeta_r = g^(b-1-r)
// R_{-1} is the carried-in state (or zero). For every chunk i the kernel
// stores R_{i-1} -- transposed to [dv][dk] and rounded to the input element
// type -- for the output kernel's (Q_i R_{i-1}) product, and at the end the
// fp32 R of the last chunk as the state output.
//
// One workgroup owns a TK x 64 tile of R for one (sequence, head) and walks
// the chunks in order, keeping its tile in fp32 accumulator registers; the
// contraction over the chunk's keys runs on the matrix cores with both
// operands read from natural [key][d] LDS tiles by the gfx950 transpose read.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

template <typename T, int D>
struct StTile {
  static constexpr int TK = D < 128 ? D : 128;  // dk rows of R per workgroup
  static constexpr int TV = 64;                 // dv columns of R per workgroup
  static constexpr int WAVES = TK / 32;         // each wave owns 32 dk rows
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BK = 64;                 // keys per LDS stage
  static constexpr int NBV = TV / 16;
  static constexpr int E = sizeof(T);
  static constexpr int KSTR = TK + 32 / E;  // transpose reads: stride = 32 * odd bytes
  static constexpr int VSTR = TV + 32 / E;
  static constexpr int TILES = (D / TK) * (D / TV);
};

struct StateParams {
  const void* k;
  const void* v;
  const float* state_in;
  float* state_out;
  void* snap;
  int batch, seqlen, heads, chunk, nchunks, swizzle;
  float log2g[kMaxHeads];
};

__device__ __forceinline__ void store4(bf16* p, const f32x4& x) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)x[i];
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, const f32x4& x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

template <typename T, int D>
__global__ __launch_bounds__((StTile<T, D>::THREADS)) void chunk_state_kernel(StateParams p) {
  using C = StTile<T, D>;
  __shared__ __attribute__((aligned(16))) T ks[C::BK * C::KSTR];
  __shared__ __attribute__((aligned(16))) T vs[C::BK * C::VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int bid = blockIdx.x;
  int bh, tile;
  if (p.swizzle) {  // the tiles of one (sequence, head) share K and V through one XCD's L2
    const int xcd = bid & 7, slot = bid >> 3;
    bh = xcd + 8 * (slot / C::TILES);
    tile = slot % C::TILES;
  } else {
    bh = bid / C::TILES;
    tile = bid % C::TILES;
  }
  const int tk0 = (tile / (D / C::TV)) * C::TK;
  const int tv0 = (tile % (D / C::TV)) * C::TV;
  const int h = bh % p.heads, b = bh / p.heads;
  const float lg = p.log2g[h];
  const int64_t tstride = (int64_t)p.heads * D;
  const int64_t head0 = ((int64_t)b * p.seqlen * p.heads + h) * D;
  const T* K = reinterpret_cast<const T*>(p.k) + head0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;

  // accumulator element (rr, nb, i) of lane (g, c): R[dk][dv] with
  const int dkw = tk0 + wave * 32 + 4 * g;  // + rr*16 + i
  const int dvl = tv0 + c;                  // + nb*16
  f32x4 racc[2][C::NBV];
  const float* S0 = p.state_in ? p.state_in + (int64_t)bh * D * D : nullptr;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int nb = 0; nb < C::NBV; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        racc[rr][nb][i] = S0 ? S0[(int64_t)(dkw + rr * 16 + i) * D + dvl + nb * 16] : 0.f;

  for (int ci = 0; ci < p.nchunks; ++ci) {
    // R_{ci-1}, transposed, for the output kernel
    T* sn = reinterpret_cast<T*>(p.snap) + ((int64_t)bh * p.nchunks + ci) * D * D;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb) store4(sn + (int64_t)(dvl + nb * 16) * D + dkw + rr * 16, racc[rr][nb]);

    const int cs = ci * p.chunk;
    const int blen = min(p.chunk, p.seqlen - cs);
    const int cend = cs + blen;
    const float dec = gpow((float)blen, lg);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb) racc[rr][nb] *= dec;

    for (int kb0 = cs; kb0 < cend; kb0 += C::BK) {
      // all global loads of the stage first (rows clamped in range), then the
      // LDS writes; keys past the chunk are zeroed (K) and dropped (V * 0).
      constexpr int KI = C::BK * (C::TK / 8) / C::THREADS;
      constexpr int VI = C::BK * (C::TV / 8) / C::THREADS;
      Raw8<T> kr[KI], vr[VI];
#pragma unroll
      for (int it = 0; it < KI; ++it) {
        const int idx = tid + C::THREADS * it;
        const int r = idx / (C::TK / 8), c8 = idx % (C::TK / 8);
        const int key = min(kb0 + r, cend - 1);
        kr[it] = ld_raw8(K + key * tstride + tk0 + c8 * 8);
      }
#pragma unroll
      for (int it = 0; it < VI; ++it) {
        const int idx = tid + C::THREADS * it;
        const int r = idx / (C::TV / 8), c8 = idx % (C::TV / 8);
        const int key = min(kb0 + r, cend - 1);
        vr[it] = ld_raw8(V + key * tstride + tv0 + c8 * 8);
      }
      __syncthreads();  // previous stage's LDS reads are done
#pragma unroll
      for (int it = 0; it < KI; ++it) {
        const int idx = tid + C::THREADS * it;
        const int r = idx / (C::TK / 8), c8 = idx % (C::TK / 8);
        const bool keep = kb0 + r < cend;
        st_raw8(ks + r * C::KSTR + c8 * 8, kr[it], keep);
      }
#pragma unroll
      for (int it = 0; it < VI; ++it) {
        const int idx = tid + C::THREADS * it;
        const int r = idx / (C::TV / 8), c8 = idx % (C::TV / 8);
        const int key = kb0 + r;
        F8 x = unpack8(vr[it]);
        const float z = gpow((float)(cend - 1 - key), lg);
#pragma unroll
        for (int e = 0; e < 8; ++e) x.x[e] *= z;
        zero_unless(x, key < cend);
        store8(vs + r * C::VSTR + c8 * 8, x);
      }
      __syncthreads();
#pragma unroll
      for (int kq = 0; kq < C::BK / 32; ++kq) {
        frag_t<T> afr[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) afr[rr] = lds_col8(ks + kq * 32 * C::KSTR + wave * 32 + rr * 16, C::KSTR, lane);
#pragma unroll
        for (int nb = 0; nb < C::NBV; ++nb) {
          const frag_t<T> bfr = lds_col8(vs + kq * 32 * C::VSTR + nb * 16, C::VSTR, lane);
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) racc[rr][nb] = mma(afr[rr], bfr, racc[rr][nb]);
        }
      }
    }
  }

  if (p.state_out) {
    float* SO = p.state_out + (int64_t)bh * D * D;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) SO[(int64_t)(dkw + rr * 16 + i) * D + dvl + nb * 16] = racc[rr][nb][i];
  }
}

template <typename T, int D>
static hipError_t launch_state_t(const Shape& s, const StateParams& p0, hipStream_t stream) {
  using C = StTile<T, D>;
  StateParams p = p0;
  const int bhs = s.batch * s.heads;
  p.swizzle = (bhs % 8) == 0;
  const int64_t blocks = (int64_t)bhs * C::TILES;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((chunk_state_kernel<T, D>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Shape& s, int chunk, const void* k, const void* v, const float* state_in,
                              float* state_out, void* snap, hipStream_t stream) {
  StateParams p;
  p.k = k;
  p.v = v;
  p.state_in = state_in;
  p.state_out = state_out;
  p.snap = snap;
  p.batch = s.batch;
  p.seqlen = s.seqlen;
  p.heads = s.heads;
  p.chunk = chunk;
  p.nchunks = (s.seqlen + chunk - 1) / chunk;
  p.swizzle = 0;
  for (int h = 0; h < kMaxHeads; ++h) p.log2g[h] = h < s.heads ? s.log2g[h] : 0.f;
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_state_t<bf16, 64>(s, p, stream);
      case 128: return launch_state_t<bf16, 128>(s, p, stream);
      case 256: return launch_state_t<bf16, 256>(s, p, stream);
    }
  } else {
    switch (s.d) {
      case 64: return launch_state_t<float, 64>(s, p, stream);
      case 128: return launch_state_t<float, 128>(s, p, stream);
      case 256: return launch_state_t<float, 256>(s, p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ret
