// Parallel and chunkwise forms of retention ("Retentive Network: A Successor
// to Transformer...", Elamur summary, Summary: the parallel form for
// training; the chunkwise form computes each chunk in parallel and passes the
// recurrent state between chunks). For chunk i of length b:
//     O_i = (Q_i K_i^T (.) D) V_i  +  xi (.) (Q_i R_{i-1})       xi_r = g^(r+1)
//     R_i = g^b R_{i-1} + K_i^T (V_i (.) zeta)                    zeta_r = g^(b-1-r)
// followed by GroupNorm + swish gate. The parallel form is one chunk that
// spans the whole sequence with no carried state. Q and K arrive rotated.
//
// Two workgroup roles share one kernel for the chunkwise form:
//   * output role: 4 waves, 128 query rows of one chunk of one (sequence,
//     head); each wave owns 32 rows and the full dv-wide fp32 output tile in
//     registers. It streams the chunk's K and V blocks up to its diagonal
//     through two LDS stages (direct global->LDS loads, the next block's
//     loads overlapping the matrix-core work on the current one), computes
//     S^T = K Q^T, the decay mask and O += P V, then -- last -- waits for
//     R_{i-1} and adds the cross-chunk term, then GroupNorm + gate.
//   * state role: 4 waves, one chunk of one (sequence, head); accumulates
//     dR_i = K_i^T (V_i (.) zeta) over the chunk's keys (fp32, in registers),
//     waits for R_{i-1} from the previous chunk's state workgroup, forms
//     R_i = g^b R_{i-1} + dR_i and publishes it: fp32 for the next state
//     workgroup, transposed in the input dtype for the next chunk's output
//     workgroups, and as the state output after the last chunk.
// Workgroups take their role from an atomic ticket in chunk-major order, so
// a workgroup only ever waits for workgroups that hold smaller tickets and
// are therefore already running: the waits always end. Every wait is also
// bounded; on expiry it sets an error word in the control block and goes on.
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
  // dk columns per R^T slice; slices are loaded two at a time
  static constexpr int RS = D / 2 < 256 / E ? D / 2 : 256 / E;
  static constexpr int NRS = D / RS;
  using KT = PTile<T, BN, D, 16>;   // K block, row fragments
  using VT = PTile<T, BN, D, 32>;   // V block, column (transpose) fragments
  using RT = PTile<T, D, RS, 16>;   // R^T slice (dv rows x RS dk), row fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
  static constexpr int YSTR = D + 4;  // epilogue rows (fp32), two waves per stage buffer
  static_assert(NRS % 2 == 0, "slices come in pairs");
};

template <typename T, int D>
struct StTile {
  static constexpr int SPLIT = 2;               // state workgroups per chunk, one per dv half
  static constexpr int BK = OutTile<T, D>::BN;  // keys per block
  static constexpr int RB = D / 64;             // 16-row dk blocks per wave (wave owns D/4 dk rows)
  static constexpr int NB = D / 16 / SPLIT;     // 16-wide dv blocks of this half
  using KT = PTile<T, BK, D, 32>;               // K block, column fragments (K^T operand)
  using VT = PTile<T, BK, D, 32>;               // V block, column fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
};

template <typename T, int D>
struct Stage {
  using O = OutTile<T, D>;
  using S = StTile<T, D>;
  static constexpr int A = O::KVB > O::RT::BYTES ? O::KVB : O::RT::BYTES;
  static constexpr int BYTES = A > S::KVB ? A : S::KVB;
  static_assert(2 * 16 * O::YSTR * 4 <= BYTES, "epilogue buffer");
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  void* o;
  const float* state_in;
  float* state_out;
  void* snap;    // [BH][nchunks][dv][dk] of T: R_{i-1}^T for chunk i
  float* chain;  // [BH][2][dk][dv] fp32: R_i handed to the next state workgroup
  int* ctrl;     // [0] ticket, [1] error, [2 + (bh*(nchunks+1) + i)*2 + half]: "half of R_{i-1} ready"
  int batch, seqlen, heads, chunk, nchunks, qblocks;
  int has_state0, xcd_order;
  float eps;
  float log2g[kMaxHeads];
};

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off.
//
// The handed-off data (fp32 chain, per-chunk states) is written with sc1
// stores (relaxed agent-scope atomics: written through to the point where all
// XCDs see the same value) and read with sc1 loads or sc0|sc1 direct loads, so
// no L2 writeback or invalidation of a whole XCD cache is ever needed. The
// producer waits until its stores are acknowledged (vmcnt 0) in every wave
// before one thread raises the flag; the consumer spins on the flag with sc1
// loads, then a barrier orders every wave's reads after it.
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 22;  // ~2^22 x 512 cycles: about a second
constexpr int kCoherent = 17;        // sc0 | sc1 cache policy for direct loads

__device__ __forceinline__ void wait_flag(const int* flag, int* err) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(const_cast<int*>(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      __builtin_amdgcn_s_sleep(8);
      if (++spins > kSpinLimit) {
        atomicOr(err, 1);
        break;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void release_flag(int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent stores are acknowledged
  __syncthreads();                // ... in every wave
  if (threadIdx.x == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// coherent (sc1) stores and loads of handed-off values
__device__ __forceinline__ void store4_coherent(bf16* p, const f32x4& x) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)x[i];
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, o), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store4_coherent(float* p, const f32x4& x) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 a = {x[0], x[1]}, b = {x[2], x[3]};
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, a), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p + 2), __builtin_bit_cast(uint64_t, b), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store1_coherent(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load1_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Output role.
// ---------------------------------------------------------------------------
template <typename T, int D>
__device__ __forceinline__ void out_role(const FwdParams& p, int bh, int ci, int qb, bool chunked, char* stage0,
                                         char* stage1) {
  using C = OutTile<T, D>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;

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

  const int qw0 = q0 + wave * C::QW;
  const int kend = min(q0 + C::BM, cend);
  const int nkb = (kend - c0 + C::BN - 1) / C::BN;

  auto issue_kv = [&](int j, char* buf) __attribute__((always_inline)) {
    const int kb0 = c0 + j * C::BN;
    async_tile<T, typename C::KT, C::WAVES>(buf, K, tstride, kb0, cend - 1, wave, lane);
    async_tile<T, typename C::VT, C::WAVES>(buf + C::KT::BYTES, V, tstride, kb0, cend - 1, wave, lane);
  };
  issue_kv(0, stage0);

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

  // One pipeline step: wait for block j, release the other stage, prefetch
  // block j+1 into it. The stages are distinct LDS objects and the loop is
  // unrolled by two, so the compiler can tell the reads of one stage from
  // the in-flight loads into the other.
  auto sync_and_prefetch = [&](int j, char* nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkb) issue_kv(j + 1, nxt);
  };
  for (int j = 0; j < nkb; j += 2) {
    sync_and_prefetch(j, stage1);
    key_block(c0 + j * C::BN, stage0);
    if (j + 1 < nkb) {
      sync_and_prefetch(j + 1, stage0);
      key_block(c0 + (j + 1) * C::BN, stage1);
    }
  }

  // Cross-chunk term, added last: O = xi (.) (O_intra / xi + Q R_{i-1}).
  // Rows whose xi is below 2^-100 skip it (their Q fragment is zeroed and
  // their scale is 1): the term is then far below fp32 resolution.
  if (chunked && (ci > 0 || p.has_state0)) {
    int* flags = p.ctrl + 2 + (bh * (p.nchunks + 1) + ci) * 2;
    __syncthreads();  // both stages are free
    wait_flag(flags + 0, p.ctrl + 1);
    wait_flag(flags + 1, p.ctrl + 1);
    const T* R = reinterpret_cast<const T*>(p.snap) + ((int64_t)bh * p.nchunks + ci) * D * D;  // [dv][dk]
    float inv[2][4];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xi = gpow((float)(qw0 + qq * 16 + 4 * g + i - c0 + 1), lg);
        inv[qq][i] = xi >= 7.888609e-31f ? __builtin_amdgcn_rcpf(xi) : 1.f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) oacc[qq][nb][i] *= inv[qq][i];
      }
      const float xq = gpow((float)(qw0 + qq * 16 + c - c0 + 1), lg);
      if (!(xq >= 7.888609e-31f)) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[qq][s] = zero_frag<T>();
      }
    }
    auto cross_slice = [&](auto sl_c, const char* buf) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value;
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
    };
    auto slice_pair = [&](auto sl_c) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value;
      async_tile<T, typename C::RT, C::WAVES, kCoherent>(stage0, R + SL * C::RS, D, 0, D - 1, wave, lane);
      async_tile<T, typename C::RT, C::WAVES, kCoherent>(stage1, R + (SL + 1) * C::RS, D, 0, D - 1, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cross_slice(std::integral_constant<int, SL>{}, stage0);
      cross_slice(std::integral_constant<int, SL + 1>{}, stage1);
      __syncthreads();
    };
    slice_pair(std::integral_constant<int, 0>{});
    if constexpr (C::NRS > 2) slice_pair(std::integral_constant<int, 2>{});
    static_assert(C::NRS <= 4, "at most four R^T slices");
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xi = inv[qq][i] == 1.f ? 1.f : gpow((float)(qw0 + qq * 16 + 4 * g + i - c0 + 1), lg);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) oacc[qq][nb][i] *= xi;
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

// ---------------------------------------------------------------------------
// State role.
// ---------------------------------------------------------------------------
// Scale a column fragment by one factor per key; keys past the chunk
// (keep = false) become exact zeros whatever the clamped row held.
__device__ __forceinline__ void scale_frag(bf16x8& f, const float* z, const bool* keep) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)(keep[j] ? (float)f[j] * z[j] : 0.f);
}
__device__ __forceinline__ void scale_frag(f32x8& f, const float* z, const bool* keep) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = keep[j] ? f[j] * z[j] : 0.f;
}

template <typename T, int D>
__device__ __forceinline__ void state_issue(char* buf, const T* K, const T* V, int64_t tstride, int kb0, int rmax,
                                            int wave, int lane) {
  using KT = typename StTile<T, D>::KT;
  using VT = typename StTile<T, D>::VT;
  async_tile<T, KT, 4>(buf, K, tstride, kb0, rmax, wave, lane);
  async_tile<T, VT, 4>(buf + KT::BYTES, V, tstride, kb0, rmax, wave, lane);
}

template <typename T, int D>
__device__ __forceinline__ void state_role(const FwdParams& p, int bh, int ci, int half, char* stage0,
                                           char* stage1) {
  using SC = StTile<T, D>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int h = bh % p.heads, b = bh / p.heads;
  const float lg = p.log2g[h];
  const int c0 = ci * p.chunk;
  const int cend = min(c0 + p.chunk, p.seqlen);
  const int nkb = (cend - c0 + SC::BK - 1) / SC::BK;
  const int64_t tstride = (int64_t)p.heads * D;
  const int64_t head0 = ((int64_t)b * p.seqlen * p.heads + h) * D;
  const T* K = reinterpret_cast<const T*>(p.k) + head0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  // flag of (chunk index j, this half)
  auto flag_of = [&](int j) __attribute__((always_inline)) { return p.ctrl + 2 + (bh * (p.nchunks + 1) + j) * 2 + half; };

  // accumulator element (a, nb, j) of lane (g, c) is R[dk][dv] with
  const int dkw = wave * (D / 4) + 4 * g;  // + 16 a + j
  const int dv0 = half * (D / SC::SPLIT) + c;  // + 16 nb
  T* snap_next = reinterpret_cast<T*>(p.snap) + ((int64_t)bh * p.nchunks + ci + 1) * D * D;
  auto write_snapshot = [&](T* sn, const f32x4 (&acc)[SC::RB][SC::NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
        store4_coherent(sn + (int64_t)(dv0 + nb * 16) * D + dkw + 16 * a, acc[a][nb]);
  };

  f32x4 racc[SC::RB][SC::NB];
  if (ci == 0 && p.state_in) {
    // R_{-1} = state_in: publish it for the output workgroups of chunk 0
    const float* S0 = p.state_in + (int64_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) racc[a][nb][j] = S0[(int64_t)(dkw + 16 * a + j) * D + dv0 + nb * 16];
    write_snapshot(reinterpret_cast<T*>(p.snap) + (int64_t)bh * p.nchunks * D * D, racc);
    release_flag(flag_of(0));
  }
#pragma unroll
  for (int a = 0; a < SC::RB; ++a)
#pragma unroll
    for (int nb = 0; nb < SC::NB; ++nb) racc[a][nb] = zero4();

  auto issue_kv = [&](int j, char* buf) __attribute__((always_inline)) {
    state_issue<T, D>(buf, K, V, tstride, c0 + j * SC::BK, cend - 1, wave, lane);
  };
  // dR += K_blk^T (V_blk (.) zeta): zeta is applied to the K^T fragments (one
  // factor per key), keys past the chunk get zero.
  auto block = [&](int kb0, const char* kt) __attribute__((always_inline)) {
    const char* vt = kt + SC::KT::BYTES;
#pragma unroll
    for (int ks = 0; ks < SC::BK / 32; ++ks) {
      float z[8];
      bool keep[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kb0 + ks * 32 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
        keep[j] = key < cend;
        z[j] = gpow((float)(cend - 1 - key), lg);
      }
      frag_t<T> af[SC::RB];
#pragma unroll
      for (int a = 0; a < SC::RB; ++a) {
        af[a] = tile_col8<typename SC::KT>(kt, ks * 32, wave * (D / 4) + 16 * a, lane, (T*)nullptr);
        scale_frag(af[a], z, keep);
      }
      constexpr int NT = SC::NB;
      auto vload = [&](int t) __attribute__((always_inline)) {
        return tile_col8<typename SC::VT>(vt, ks * 32, half * (D / SC::SPLIT) + t * 16, lane, (T*)nullptr);
      };
      frag_t<T> vb[3];
      vb[0] = vload(0);
      vb[1] = vload(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + 2 < NT) vb[(t + 2) % 3] = vload(t + 2);
#pragma unroll
        for (int a = 0; a < SC::RB; ++a) racc[a][t] = mma(af[a], vb[t % 3], racc[a][t]);
      }
    }
  };
  issue_kv(0, stage0);
  auto sync_and_prefetch = [&](int j, char* nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkb) issue_kv(j + 1, nxt);
  };
  for (int j = 0; j < nkb; j += 2) {
    sync_and_prefetch(j, stage1);
    block(c0 + j * SC::BK, stage0);
    if (j + 1 < nkb) {
      sync_and_prefetch(j + 1, stage0);
      block(c0 + (j + 1) * SC::BK, stage1);
    }
  }

  // R_i = g^b R_{i-1} + dR_i
  const float* Rprev = nullptr;
  if (ci > 0) {
    wait_flag(flag_of(ci), p.ctrl + 1);
    Rprev = p.chain + ((int64_t)bh * 2 + ((ci - 1) & 1)) * D * D;
  } else if (p.state_in) {
    Rprev = p.state_in + (int64_t)bh * D * D;
  }
  if (Rprev) {
    const float dec = gpow((float)(cend - c0), lg);
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          racc[a][nb][j] += dec * (ci > 0 ? load1_coherent(Rprev + (int64_t)(dkw + 16 * a + j) * D + dv0 + nb * 16)
                                          : Rprev[(int64_t)(dkw + 16 * a + j) * D + dv0 + nb * 16]);
  }
  if (ci + 1 < p.nchunks) {
    float* Rn = p.chain + ((int64_t)bh * 2 + (ci & 1)) * D * D;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) store1_coherent(Rn + (int64_t)(dkw + 16 * a + j) * D + dv0 + nb * 16, racc[a][nb][j]);
    write_snapshot(snap_next, racc);
    release_flag(flag_of(ci + 1));
  } else if (p.state_out) {
    float* SO = p.state_out + (int64_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) SO[(int64_t)(dkw + 16 * a + j) * D + dv0 + nb * 16] = racc[a][nb][j];
  }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 1) void retention_parallel_kernel(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  __shared__ __attribute__((aligned(1024))) char stage0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[Stage<T, D>::BYTES];
  int bh, qb;
  const int bid = blockIdx.x;
  const int groups = p.batch * p.heads;
  if (groups % 8 == 0) {  // the query blocks of one (sequence, head) share K and V through one XCD's L2
    const int xcd = bid & 7, slot = bid >> 3;
    bh = xcd + 8 * (slot / p.qblocks);
    qb = p.qblocks - 1 - slot % p.qblocks;
  } else {
    bh = bid / p.qblocks;
    qb = p.qblocks - 1 - bid % p.qblocks;
  }
  out_role<T, D>(p, bh, 0, qb, false, stage0, stage1);
#endif
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void retention_chunkwise_kernel(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  __shared__ __attribute__((aligned(1024))) char stage0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[Stage<T, D>::BYTES];
  __shared__ int s_ticket;
  if (threadIdx.x == 0) s_ticket = atomicAdd(p.ctrl, 1);
  __syncthreads();
  const int t = s_ticket;
  const int bhs = p.batch * p.heads;
  constexpr int SPLIT = StTile<T, D>::SPLIT;
  const int roles = SPLIT + p.qblocks;  // workgroups per (sequence, head, chunk)
  const int ci = t / (bhs * roles);
  int r = t % (bhs * roles);
  int bh, role;  // role < SPLIT: state half; else query block qblocks-1-(role-SPLIT)
  if (p.xcd_order) {
    // blocks of 8 (sequence, head) pairs: slot r -> lane of 8 = likely XCD
    // (workgroups are dispatched round-robin over the 8 XCDs), so the state
    // and output workgroups of one pair tend to share an XCD and its L2
    const int blk = r / (8 * roles), sidx = r % (8 * roles);
    bh = blk * 8 + (sidx & 7);
    role = sidx >> 3;
  } else {
    bh = r / roles;
    role = r % roles;
  }
  const int qb = role < SPLIT ? -1 : p.qblocks - 1 - (role - SPLIT);
  if (qb < 0)
    state_role<T, D>(p, bh, ci, role, stage0, stage1);
  else
    out_role<T, D>(p, bh, ci, qb, true, stage0, stage1);
#endif
}

__global__ void reset_ctrl_kernel(int* ctrl, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) ctrl[i] = 0;
}

template <typename T, int D>
static hipError_t launch_fwd_t(const Shape& s, int chunk, FwdParams p, bool chunked, hipStream_t stream) {
  using C = OutTile<T, D>;
  p.qblocks = (chunk + C::BM - 1) / C::BM;
  const int bhs = s.batch * s.heads;
  if (!chunked) {
    const int64_t blocks = (int64_t)bhs * p.qblocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((retention_parallel_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t nctrl = 2 + (int64_t)bhs * (p.nchunks + 1) * 2;
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3((unsigned)((nctrl + 255) / 256 < 1024 ? (nctrl + 255) / 256 : 1024)),
                     dim3(256), 0, stream, p.ctrl, (int)nctrl);
  p.xcd_order = bhs % 8 == 0;
  const int64_t blocks = (int64_t)p.nchunks * bhs * (StTile<T, D>::SPLIT + p.qblocks);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((retention_chunkwise_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

size_t chunkwise_ctrl_bytes(int batch, int heads, int nchunks) {
  return ((size_t)2 + (size_t)batch * heads * (nchunks + 1) * 2) * sizeof(int);
}

hipError_t launch_retention_fwd(const Shape& s, int chunk, bool chunked, const void* q, const void* k, const void* v,
                                const void* g, void* o, const float* state_in, float* state_out, void* snap,
                                float* chain, int* ctrl, float eps, hipStream_t stream) {
  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.o = o;
  p.state_in = state_in;
  p.state_out = state_out;
  p.snap = snap;
  p.chain = chain;
  p.ctrl = ctrl;
  p.batch = s.batch;
  p.seqlen = s.seqlen;
  p.heads = s.heads;
  p.chunk = chunk;
  p.nchunks = (s.seqlen + chunk - 1) / chunk;
  p.qblocks = 0;
  p.has_state0 = state_in != nullptr;
  p.xcd_order = 0;
  p.eps = eps;
  for (int h = 0; h < kMaxHeads; ++h) p.log2g[h] = h < s.heads ? s.log2g[h] : 0.f;
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_fwd_t<bf16, 64>(s, chunk, p, chunked, stream);
      case 128: return launch_fwd_t<bf16, 128>(s, chunk, p, chunked, stream);
      case 256: return launch_fwd_t<bf16, 256>(s, chunk, p, chunked, stream);
    }
  } else {
    switch (s.d) {
      case 64: return launch_fwd_t<float, 64>(s, chunk, p, chunked, stream);
      case 128: return launch_fwd_t<float, 128>(s, chunk, p, chunked, stream);
      case 256: return launch_fwd_t<float, 256>(s, chunk, p, chunked, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ret
