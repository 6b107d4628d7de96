// Retention output for the parallel and the chunkwise forms
// ("Retentive Network: A Successor to Transformer...", Elamur summary,
// Summary; the parallel form is the chunkwise form with one chunk that spans
// the whole sequence and no carried state):
//     O = xi (.) (Q R_{i-1})  +  (Q K^T (.) D) V        within one chunk
// then GroupNorm + swish gate, fused. Q and K arrive already rotated.
//
// Work unit: one workgroup = 4 waves = 128 consecutive query rows of one
// chunk of one (sequence, head); each wave owns 32 query rows and the full
// dv-wide fp32 output tile in registers.
//
// Data movement: every tile (a 64-key block of K and of V, or a dk slice of
// R_{i-1}^T) is brought into LDS by direct global->LDS loads into one of two
// stage buffers, so the loads of item j+1 run while the matrix cores work on
// item j, with one barrier per item. Tiles are XOR-swizzled instead of padded.
//
// Per key block:
//   * S^T = K Q^T on the matrix cores (Q fragments live in registers), so
//     each lane holds the scores of one query for 8 keys, which is exactly
//     the A fragment of the next product: no LDS round trip for P;
//   * the decay g^(q-k) is generated in registers and masked above the
//     diagonal;
//   * O += P V with V fragments read by the gfx950 LDS transpose read.
// The epilogue normalises each row with 16-lane reductions, goes through LDS
// once to reach row-contiguous order, applies the gate and stores with
// 16-byte accesses.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ret {

template <typename T, int D>
struct OutTile {
  static constexpr int E = sizeof(T);
  static constexpr int WAVES = 4;
  static constexpr int QW = 32;  // query rows per wave
  static constexpr int BM = WAVES * QW;
  static constexpr int BN = E == 2 ? 64 : 32;  // keys per block
  static constexpr int KK = BN / 16;           // 16-key score blocks per key block
  static constexpr int K2 = BN / 32;           // P V contraction steps per key block
  static constexpr int KS = D / 32;            // contraction steps over dk
  static constexpr int NB = D / 16;            // 16-wide output column blocks
  // dk columns per R^T slice; always an even number of slices, so that key
  // blocks start in stage 0 whether or not there is a cross term
  static constexpr int RS = D / 2 < 256 / E ? D / 2 : 256 / E;
  static constexpr int NRS = D / RS;
  using KT = PTile<T, BN, D, 16>;   // K block, row fragments
  using VT = PTile<T, BN, D, 32>;   // V block, column (transpose) fragments
  using RT = PTile<T, D, RS, 16>;   // R^T slice (dv rows x RS dk), row fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
  static constexpr int STAGE = KVB > RT::BYTES ? KVB : RT::BYTES;
  static constexpr int YSTR = D + 4;  // epilogue rows (fp32), two waves per stage buffer
  static_assert(2 * 16 * YSTR * 4 <= STAGE, "epilogue buffer");
  static_assert(NRS % 2 == 0 && NRS <= 4, "even slice count");
};

struct OutParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  void* o;
  const void* snap;
  int batch, seqlen, heads, chunk, nchunks, qblocks;
  int has_state0, swizzle;
  float eps;
  float log2g[kMaxHeads];
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void retention_out_kernel(OutParams p) {
  using C = OutTile<T, D>;
  // two stage buffers as distinct objects: the compiler can then tell the
  // reads of one from the in-flight direct loads into the other
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int g = lane >> 4, c = lane & 15;

  int group, qb;
  const int bid = blockIdx.x;
  if (p.swizzle) {  // keep the query blocks of one chunk on one XCD (shared L2)
    const int xcd = bid & 7, slot = bid >> 3;
    group = xcd + 8 * (slot / p.qblocks);
    qb = p.qblocks - 1 - slot % p.qblocks;
  } else {
    group = bid / p.qblocks;
    qb = p.qblocks - 1 - bid % p.qblocks;
  }
  const int ci = group % p.nchunks;
  const int bh = group / p.nchunks;
  const int h = bh % p.heads, b = bh / p.heads;
  const int c0 = ci * p.chunk;
  const int cend = min(c0 + p.chunk, p.seqlen);
  const int q0 = c0 + qb * C::BM;
  if (q0 >= cend) return;  // uniform for the whole workgroup

  const float lg = p.log2g[h];
  const int64_t tstride = (int64_t)p.heads * D;  // elements between tokens
  const int64_t head0 = ((int64_t)b * p.seqlen * p.heads + h) * D;
  const T* Q = reinterpret_cast<const T*>(p.q) + head0;
  const T* K = reinterpret_cast<const T*>(p.k) + head0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  const T* G = p.g ? reinterpret_cast<const T*>(p.g) + head0 : nullptr;
  T* O = reinterpret_cast<T*>(p.o) + head0;
  const T* R = p.snap ? reinterpret_cast<const T*>(p.snap) + ((int64_t)bh * p.nchunks + ci) * D * D : nullptr;

  const int qw0 = q0 + wave * C::QW;
  const int kend = min(q0 + C::BM, cend);
  const int nkb = (kend - c0 + C::BN - 1) / C::BN;
  const bool cross = R && (ci > 0 || p.has_state0);
  const int nr = cross ? C::NRS : 0;
  const int nitems = nr + nkb;

  // Items: R^T dk slices first (cross term), then key blocks. Item j lives
  // in stage (j & 1); the loads of item j+1 overlap the work on item j.
  auto issue = [&](int j, char* buf) __attribute__((always_inline)) {
    if (j < nr) {
      async_tile<T, typename C::RT, C::WAVES>(buf, R + j * C::RS, D, 0, D - 1, wave, lane);
    } else {
      const int kb0 = c0 + (j - nr) * C::BN;
      async_tile<T, typename C::KT, C::WAVES>(buf, K, tstride, kb0, cend - 1, wave, lane);
      async_tile<T, typename C::VT, C::WAVES>(buf + C::KT::BYTES, V, tstride, kb0, cend - 1, wave, lane);
    }
  };
  issue(0, stage0);

  // Query fragments, kept in registers for the whole workgroup life. Rows
  // past the chunk load a clamped in-range row: their outputs are never
  // stored.
  frag_t<T> qf[2][C::KS];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int row = min(qw0 + qq * 16 + c, cend - 1);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qf[qq][s] = to_frag(unpack8(ld_raw8(Q + row * tstride + s * 32 + 8 * g)), (T*)nullptr);
  }

  f32x4 oacc[2][C::NB];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) oacc[qq][nb] = zero4();

  // Cross-chunk term: slice SL of xi (.) (Q R_{i-1}), then the xi row scale
  // after the last slice.
  auto cross_slice = [&](auto sl_c, const char* buf) __attribute__((always_inline)) {
    constexpr int SL = decltype(sl_c)::value;
    {  // R^T fragments prefetched two steps ahead of their products
      constexpr int NT = (C::RS / 32) * C::NB;
      auto rload = [&](int t) __attribute__((always_inline)) {
        return tile_row8<typename C::RT>(buf, (t % C::NB) * 16 + c, (t / C::NB) * 32 + 8 * g, (T*)nullptr);
      };
      frag_t<T> rb[3];
      rb[0] = rload(0);
      rb[1] = rload(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 2 < NT) rb[(t + 2) % 3] = rload(t + 2);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
          oacc[qq][t % C::NB] = mma(qf[qq][SL * (C::RS / 32) + t / C::NB], rb[t % 3], oacc[qq][t % C::NB]);
      }
    }
    if (SL == C::NRS - 1) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = qw0 + qq * 16 + 4 * g + i;
          const float xi = gpow((float)(row - c0 + 1), lg);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) oacc[qq][nb][i] *= xi;
        }
      }
    }
  };

  // Intra-chunk term (Q K^T (.) D) V over key blocks up to the diagonal; the
  // decay g^(q-k) = exp2((q-k) log2 g) is formed per score (exact integer
  // distance, one multiply, one exp2) and masked above the diagonal.
  auto key_block = [&](int kb0, const char* kt) __attribute__((always_inline)) {
    if (kb0 > qw0 + C::QW - 1 || qw0 >= cend) return;  // block above this wave's diagonal
    const char* vt = kt + C::KT::BYTES;
    f32x4 st[2][C::KK];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) st[qq][kk] = zero4();
    {  // K fragments prefetched two steps ahead of their products
      constexpr int NT = C::KS * C::KK;
      auto kload = [&](int t) __attribute__((always_inline)) {
        return tile_row8<typename C::KT>(kt, (t % C::KK) * 16 + c, (t / C::KK) * 32 + 8 * g, (T*)nullptr);
      };
      frag_t<T> kb[3];
      kb[0] = kload(0);
      kb[1] = kload(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 2 < NT) kb[(t + 2) % 3] = kload(t + 2);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) st[qq][t % C::KK] = mma(kb[t % 3], qf[qq][t / C::KK], st[qq][t % C::KK]);
      }
    }
    frag_t<T> pf[2][C::K2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int qrow = qw0 + qq * 16 + c;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dist = qrow - (kb0 + kk * 16 + 4 * g + i);
          const float val = st[qq][kk][i] * gpow((float)dist, lg);
          st[qq][kk][i] = dist < 0 ? 0.f : val;
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < C::K2; ++k2) pf[qq][k2] = acc_to_frag(st[qq][2 * k2], st[qq][2 * k2 + 1], (T*)nullptr);
    }
    {  // V fragments prefetched two steps ahead of their products
      constexpr int NT = C::K2 * C::NB;
      auto vload = [&](int t) __attribute__((always_inline)) {
        return tile_col8<typename C::VT>(vt, (t / C::NB) * 32, (t % C::NB) * 16, lane, (T*)nullptr);
      };
      frag_t<T> vb[3];
      vb[0] = vload(0);
      vb[1] = vload(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 2 < NT) vb[(t + 2) % 3] = vload(t + 2);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
          oacc[qq][t % C::NB] = mma(pf[qq][t / C::NB], vb[t % 3], oacc[qq][t % C::NB]);
      }
    }
  };

  // One pipeline step: wait for item j, release the other stage, prefetch
  // item j+1 into it, work on item j.
  auto sync_and_prefetch = [&](int j, char* nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of item j have landed
    __syncthreads();                // everyone's have; the other stage is free
    if (j + 1 < nitems) issue(j + 1, nxt);
  };
  if (cross) {
#pragma unroll
    for (int sl = 0; sl < C::NRS; sl += 2) {
      sync_and_prefetch(sl, stage1);
      if (sl == 0) cross_slice(std::integral_constant<int, 0>{}, stage0);
      if constexpr (C::NRS > 2) if (sl == 2) cross_slice(std::integral_constant<int, 2>{}, stage0);
      sync_and_prefetch(sl + 1, stage0);
      if (sl == 0) cross_slice(std::integral_constant<int, 1>{}, stage1);
      if constexpr (C::NRS > 2) if (sl == 2) cross_slice(std::integral_constant<int, 3>{}, stage1);
    }
  }
  for (int j = nr; j < nitems; j += 2) {
    sync_and_prefetch(j, stage1);
    key_block(c0 + (j - nr) * C::BN, stage0);
    if (j + 1 < nitems) {
      sync_and_prefetch(j + 1, stage0);
      key_block(c0 + (j + 1 - nr) * C::BN, stage1);
    }
  }

  // Epilogue: GroupNorm over dv per (token, head), swish gate, store.
  __syncthreads();
  float* yw = reinterpret_cast<float*>(wave < 2 ? stage0 : stage1) + (wave & 1) * 16 * C::YSTR;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    constexpr int EI = 16 * (D / 8) / 64;
    Raw8<T> gr[EI];
    if (G) {
#pragma unroll
      for (int e = 0; e < EI; ++e) {
        const int idx = lane + 64 * e;
        const int r = idx / (D / 8), c8 = idx % (D / 8);
        const int tok = min(qw0 + qq * 16 + r, cend - 1);
        gr[e] = ld_raw8(G + tok * tstride + c8 * 8);
      }
    }
    float mean[4], rstd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mean[i] = 0.f;
      rstd[i] = 1.f;
    }
    if (G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = 0.f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) s += oacc[qq][nb][i];
        mean[i] = sum16(s) * (1.0f / D);
        float s2 = 0.f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const float d = oacc[qq][nb][i] - mean[i];
          s2 += d * d;
        }
        rstd[i] = rsqrtf(sum16(s2) * (1.0f / D) + p.eps);
      }
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) yw[(4 * g + i) * C::YSTR + nb * 16 + c] = (oacc[qq][nb][i] - mean[i]) * rstd[i];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EI; ++e) {
      const int idx = lane + 64 * e;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      const int tok = qw0 + qq * 16 + r;
      const float* yp = yw + r * C::YSTR + c8 * 8;
      const f32x4 ya = reinterpret_cast<const f32x4*>(yp)[0];
      const f32x4 yb = reinterpret_cast<const f32x4*>(yp)[1];
      F8 y{{ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]}};
      if (G) {
        const F8 gv = unpack8(gr[e]);
#pragma unroll
        for (int k = 0; k < 8; ++k) y.x[k] *= swish(gv.x[k]);
      }
      if (tok < cend) store8(O + tok * tstride + c8 * 8, y);
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_out_t(const Shape& s, int chunk, const OutParams& p0, hipStream_t stream) {
  using C = OutTile<T, D>;
  OutParams p = p0;
  p.qblocks = (chunk + C::BM - 1) / C::BM;
  const int groups = s.batch * s.heads * p.nchunks;
  p.swizzle = (groups % 8) == 0;
  const int64_t blocks = (int64_t)groups * p.qblocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((retention_out_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_retention_out(const Shape& s, int chunk, const void* q, const void* k, const void* v,
                                const void* g, void* o, const void* snap, int has_state0, float eps,
                                hipStream_t stream) {
  OutParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.o = o;
  p.snap = snap;
  p.batch = s.batch;
  p.seqlen = s.seqlen;
  p.heads = s.heads;
  p.chunk = chunk;
  p.nchunks = (s.seqlen + chunk - 1) / chunk;
  p.qblocks = 0;
  p.has_state0 = has_state0;
  p.swizzle = 0;
  p.eps = eps;
  for (int h = 0; h < kMaxHeads; ++h) p.log2g[h] = h < s.heads ? s.log2g[h] : 0.f;
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_out_t<bf16, 64>(s, chunk, p, stream);
      case 128: return launch_out_t<bf16, 128>(s, chunk, p, stream);
      case 256: return launch_out_t<bf16, 256>(s, chunk, p, stream);
    }
  } else {
    switch (s.d) {
      case 64: return launch_out_t<float, 64>(s, chunk, p, stream);
      case 128: return launch_out_t<float, 128>(s, chunk, p, stream);
      case 256: return launch_out_t<float, 256>(s, chunk, p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ret
