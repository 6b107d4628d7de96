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
// Workgroups take their role from an atomic ticket in chunk-major order (one
// ticket counter per class of workgroups when the classes can own disjoint
// (sequence, head) pairs), so a workgroup only ever waits for workgroups of
// its class that hold smaller tickets and are therefore already running or
// done: the waits always end. Every wait is also
// bounded; on expiry it sets an error word in the control block and goes on.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ret {

// FAST: every head's decay over the span that one workgroup's decay factors
// cover stays within 2^64 (see kFastSpanLog2); the scores then take one factor
// per key and the rows one factor at the end.
template <typename T, int D, bool FAST = true>
struct OutTile {
  static constexpr int E = sizeof(T);
  static constexpr int WAVES = 4;
  // Query rows per wave, in groups of 16: 48 rows for bf16 on the fast path
  // (the wave's fp32 output tile, 48 x D, and its query fragments stay in
  // registers with room for the fragment pipeline), 32 otherwise (fp32
  // fragments take twice the registers). Every K and V fragment read from
  // LDS feeds QG products. Group i of wave w holds rows 16 (w + WAVES i) ..
  // +15 of the block: every wave spans the whole block, so the causal work is
  // shared evenly.
  static constexpr int QG = E == 2 && FAST ? 3 : 2;
  static constexpr int QW = 16 * QG;
  static constexpr int BM = WAVES * QW;
  static constexpr int BN = E == 2 ? 64 : 32;  // keys per block
  static constexpr int K2 = BN / 32;           // 32-key steps per key block
  static constexpr int KS = D / 32;            // contraction steps over dk
  static constexpr int NB = D / 16;            // 16-wide output column blocks
  // dk columns per R^T slice; the slices stream through the two stages
  static constexpr int RS = D / 2 < 256 / E ? D / 2 : 256 / E;
  static constexpr int NRS = D / RS;
  using KT = PTile<T, BN, D, 16>;   // K block, row fragments
  using VT = PTile<T, BN, D, 32>;   // V block, column (transpose) fragments
  using RT = PTile<T, D, RS, 16>;   // R^T slice (dv rows x RS dk), row fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
  static constexpr int YSTR = D + 4;  // epilogue rows (fp32), two waves per stage buffer
};

// Fast path: with a reference row r0 (the row before the chunk, or before the
// parallel form's query block) the decay factors split as
//     g^(q-k) = g^(q - r0) * g^(r0 - k):
// the products P' = S g^(r0 - k) accumulate O' = P' V (+ Q R_{i-1}, whose row
// scale xi_q = g^(q - r0) is then the same row factor), and O = g^(q - r0) O'.
// Keys reach at most kFastSpan rows past r0, so |log2 g| * span <= 64 keeps
// every factor within 2^+-64 (factors of far keys underflow towards zero,
// which is what they are worth).
constexpr double kFastSpanLog2 = 64.0;

template <typename T, int D>
struct StTile {
  // State workgroups per chunk: one per 128 dk rows of R (one for D <= 128).
  // The four waves split the workgroup's rows; each holds its rows x D of R
  // in fp32 registers. Fewer rows per workgroup shorten the serial chunk-to-
  // chunk hand-off; more rows cost fewer K reads per chunk.
  static constexpr int SPLIT = D > 128 ? D / 128 : 1;
  static constexpr int ROWS = D / SPLIT;        // dk rows per workgroup
  static constexpr int BK = OutTile<T, D>::BN;  // keys per block
  static constexpr int RB = ROWS / 64;          // 16-row dk blocks per wave
  static constexpr int NB = D / 16;             // 16-wide dv blocks
  using KT = PTile<T, BK, ROWS, 32>;            // this workgroup's dk columns of K (K^T operand)
  using VT = PTile<T, BK, D, 32>;               // V block, column fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
};
// per (sequence, head, chunk j) and state part q two ready flags: rows of
// R_{j-1} in the fp32 chain (for chunk j's state workgroup of part q) and in
// the snapshot (for chunk j's output workgroups)
constexpr int kMaxSplit = 2;
constexpr int kFlagsPerChunk = 2 * kMaxSplit;

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
  float* chain;  // [BH][2][D*D] fp32: R_i handed to the next state workgroup (fragment order)
  int* ctrl;     // [0] count, [1] error, [8..15] tickets, [16 + (bh*(nchunks+1) + i)*4 + kind*2 + part]: R_{i-1} ready
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
[[maybe_unused]] constexpr int kCoherent = 17;        // sc0 | sc1 cache policy for direct loads
[[maybe_unused]] constexpr int kTicketWord = 8;       // control block: ticket counters at words 8..15
constexpr int kCtrlHead = 16;        // ... and the ready flags from word 16 on

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
__device__ __forceinline__ f32x4 load4_coherent(const float* p) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
  const f32x2 a = __builtin_bit_cast(f32x2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const f32x2 b = __builtin_bit_cast(f32x2, __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4{a[0], a[1], b[0], b[1]};
}

// ---------------------------------------------------------------------------
// Output role.
// ---------------------------------------------------------------------------
template <typename T, int D, bool FAST>
__device__ __forceinline__ void out_role(const FwdParams& p, int bh, int ci, int qb, bool chunked, char* stage0,
                                         char* stage1) {
  using C = OutTile<T, D, FAST>;
  constexpr int QG = C::QG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;

  const int h = bh % p.heads, b = bh / p.heads;
  const int c0 = ci * p.chunk;
  const int cend = min(c0 + p.chunk, p.seqlen);
  const int q0 = c0 + qb * C::BM;
  if (q0 >= cend) return;  // uniform for the whole workgroup

  const float lg = p.log2g[h];
  const int ref = chunked ? c0 - 1 : q0 - 1;  // reference row of the fast path
  const int64_t tstride = (int64_t)p.heads * D;  // elements between tokens
  const int64_t head0 = ((int64_t)b * p.seqlen * p.heads + h) * D;
  const T* Q = reinterpret_cast<const T*>(p.q) + head0;
  const T* K = reinterpret_cast<const T*>(p.k) + head0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  const T* G = p.g ? reinterpret_cast<const T*>(p.g) + head0 : nullptr;
  T* O = reinterpret_cast<T*>(p.o) + head0;

  // first row of this wave's group i
  auto grow = [&](int i) __attribute__((always_inline)) { return q0 + 16 * (wave + C::WAVES * i); };
  const int kend = min(q0 + C::BM, cend);
  const int nkb = (kend - c0 + C::BN - 1) / C::BN;

  auto issue_kv = [&](int j, char* buf) __attribute__((always_inline)) {
    const int kb0 = c0 + j * C::BN;
    async_tile<T, typename C::KT, C::WAVES>(buf, K, tstride, kb0, cend - 1, wave, lane);
    async_tile<T, typename C::VT, C::WAVES>(buf + C::KT::BYTES, V, tstride, kb0, cend - 1, wave, lane);
  };
  const bool cross = chunked && (ci > 0 || p.has_state0);
  const T* R = cross ? reinterpret_cast<const T*>(p.snap) + ((int64_t)bh * p.nchunks + ci) * D * D : nullptr;
  // R^T slice s ([dv][RS dk columns]) into an LDS stage; waits (once) for
  // the snapshot of R_{i-1} to be published
  auto issue_slice = [&](int sl, char* buf) __attribute__((always_inline)) {
    if (sl == 0) {
      const int* flags = p.ctrl + kCtrlHead + (bh * (p.nchunks + 1) + ci) * kFlagsPerChunk + kMaxSplit;
#pragma unroll
      for (int q = 0; q < StTile<T, D>::SPLIT; ++q) wait_flag(flags + q, p.ctrl + 1);
    }
    async_tile<T, typename C::RT, C::WAVES, kCoherent>(buf, R + sl * C::RS, D, 0, D - 1, wave, lane);
  };
  issue_kv(0, stage0);

  // Query fragments, kept in registers for the whole workgroup life. Rows
  // past the chunk load a clamped in-range row: their outputs are never
  // stored.
  frag_t<T> qf[QG][C::KS];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    const int row = min(grow(i) + c, cend - 1);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qf[i][s] = to_frag(unpack8(ld_raw8(Q + row * tstride + s * 32 + 8 * g)), (T*)nullptr);
  }

  f32x4 oacc[QG][C::NB];
#pragma unroll
  for (int i = 0; i < QG; ++i)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) oacc[i][nb] = zero4();

  // Intra-chunk term (Q K^T (.) D) V over key blocks up to the diagonal, 32
  // keys at a time: S^T = K Q^T for 16 keys per group, decay and causal
  // mask, then O += P V. Only groups 0 .. HI-1 hold rows of the chunk. The K
  // and V fragments of a 32-key step form one sequence of LDS reads with a
  // two-deep prefetch ring.
  constexpr int U = 2 * C::KS + C::NB;  // fragment reads per 32-key step
  float bkl[4];  // g^-(4 g + e): this lane's part of the per-key factors
#pragma unroll
  for (int e = 0; e < 4; ++e) bkl[e] = FAST ? gpow(-(float)(4 * g + e), lg) : 0.f;
  auto key_block = [&](auto hi_c, int kb0, const char* kt) __attribute__((always_inline)) {
    constexpr int HI = decltype(hi_c)::value;
    const char* vt = kt + C::KT::BYTES;
    const bool diag = kb0 + C::BN - 1 > q0;  // some key may follow some row (uniform)
    auto load = [&](auto t_c) __attribute__((always_inline)) {
      constexpr int t = decltype(t_c)::value, kh = t / U, u = t % U;
      if constexpr (u < 2 * C::KS)  // key group 2 kh + u % 2, contraction step u / 2
        return tile_row8<typename C::KT>(kt, (2 * kh + u % 2) * 16 + c, (u / 2) * 32 + 8 * g, (T*)nullptr);
      else
        return tile_col8<typename C::VT>(vt, kh * 32, (u - 2 * C::KS) * 16, lane, (T*)nullptr);
    };
    frag_t<T> ring[3];
    ring[0] = load(std::integral_constant<int, 0>{});
    ring[1] = load(std::integral_constant<int, 1>{});
    f32x4 st[QG][2];
    frag_t<T> pf[QG];
    static_for<C::K2 * U>([&](auto t_c) __attribute__((always_inline)) {
      constexpr int t = decltype(t_c)::value, kh = t / U, u = t % U;
      if constexpr (t + 2 < C::K2 * U) ring[(t + 2) % 3] = load(std::integral_constant<int, t + 2>{});
      if constexpr (u < 2 * C::KS) {
        // the two 16-key groups of the step alternate, so that consecutive
        // products go to different accumulators
        constexpr int k2 = u % 2, s = u / 2;
        if constexpr (s == 0) {
#pragma unroll
          for (int i = 0; i < HI; ++i) st[i][k2] = zero4();
        }
#pragma unroll
        for (int i = 0; i < HI; ++i) st[i][k2] = mma(ring[t % 3], qf[i][s], st[i][k2]);
        if constexpr (u == 2 * C::KS - 1) {
          // decay g^(q-k) and causal mask over the 32 keys, which become P;
          // only the diagonal blocks need the mask
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int k0 = 32 * kh + 16 * h2 + 4 * g;  // key - kb0 of element 0
            if constexpr (FAST) {
              // g^(r0 - k) = g^(r0 - kb0 - 32 kh - 16 h2) * g^-(4 g + e)
              const float sb = gpow((float)(ref - kb0 - 32 * kh - 16 * h2), lg);
              float bk[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) bk[e] = sb * bkl[e];
              if (diag) {
#pragma unroll
                for (int i = 0; i < HI; ++i)
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const float val = st[i][h2][e] * bk[e];
                    st[i][h2][e] = grow(i) + c - kb0 < k0 + e ? 0.f : val;
                  }
              } else {
#pragma unroll
                for (int i = 0; i < HI; ++i)
#pragma unroll
                  for (int e = 0; e < 4; ++e) st[i][h2][e] *= bk[e];
              }
            } else {
#pragma unroll
              for (int i = 0; i < HI; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int dist = grow(i) + c - kb0 - k0 - e;
                  const float val = st[i][h2][e] * gpow((float)dist, lg);
                  st[i][h2][e] = dist < 0 ? 0.f : val;
                }
            }
          }
#pragma unroll
          for (int i = 0; i < HI; ++i) pf[i] = acc_to_frag(st[i][0], st[i][1], (T*)nullptr);
        }
      } else {
        constexpr int nb = u - 2 * C::KS;
#pragma unroll
        for (int i = 0; i < HI; ++i) oacc[i][nb] = mma(pf[i], ring[t % 3], oacc[i][nb]);
      }
      // keep each step's prefetch where it is: two steps ahead of its use
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // One pipeline step: wait for block j, release the other stage, prefetch
  // block j+1 into it -- or, after the last key block, the first R^T slice.
  // The stages are distinct LDS objects and the loop is unrolled by two, so
  // the compiler can tell the reads of one stage from the in-flight loads
  // into the other.
  auto sync_and_prefetch = [&](int j, char* nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkb)
      issue_kv(j + 1, nxt);
    else if (cross)
      issue_slice(0, nxt);
  };
  auto key_loop = [&](auto hi_c) __attribute__((always_inline)) {
    for (int j = 0; j < nkb; j += 2) {
      sync_and_prefetch(j, stage1);
      key_block(hi_c, c0 + j * C::BN, stage0);
      if (j + 1 < nkb) {
        sync_and_prefetch(j + 1, stage0);
        key_block(hi_c, c0 + (j + 1) * C::BN, stage1);
      }
    }
  };
  // groups that hold rows of the chunk (group i starts at row 64 i of the block)
  const int hi = min(QG, (cend - q0 + 16 * C::WAVES - 1) / (16 * C::WAVES));
  static_assert(QG == 2 || QG == 3, "two or three row groups per wave");
  if (hi == QG)
    key_loop(std::integral_constant<int, QG>{});
  else if (hi == QG - 1)
    key_loop(std::integral_constant<int, QG - 1>{});
  else
    key_loop(std::integral_constant<int, 1>{});

  // Gate values, one 16-row group at a time (8-value groups per lane).
  constexpr int EI = 16 * (D / 8) / 64;
  auto load_gate = [&](int i, Raw8<T> (&dst)[EI]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < EI; ++e) {
      const int idx = lane + 64 * e;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      const int tok = min(grow(i) + r, cend - 1);
      dst[e] = ld_raw8(G + tok * tstride + c8 * 8);
    }
  };

  // Cross-chunk term, added last. Fast path: O' += Q R_{i-1} (its row scale
  // xi is the final row factor). Otherwise O = xi (.) (O_intra / xi + Q R):
  // rows whose xi is below 2^-100 skip it (their Q fragment is zeroed, their
  // scale is 1), the term being far below fp32 resolution there. The R^T
  // slices stream through the two stages, the first one already in flight.
  if (cross) {
    float inv[QG][4];
    if constexpr (!FAST) {
#pragma unroll
      for (int i = 0; i < QG; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xi = gpow((float)(grow(i) + 4 * g + e - c0 + 1), lg);
          inv[i][e] = xi >= 7.888609e-31f ? __builtin_amdgcn_rcpf(xi) : 1.f;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) oacc[i][nb][e] *= inv[i][e];
        }
        const float xq = gpow((float)(grow(i) + c - c0 + 1), lg);
        if (!(xq >= 7.888609e-31f)) {
#pragma unroll
          for (int s = 0; s < C::KS; ++s) qf[i][s] = zero_frag<T>();
        }
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
        for (int i = 0; i < QG; ++i)
          oacc[i][t % C::NB] = mma(qf[i][SL * (C::RS / 32) + t / C::NB], rb[t % 3], oacc[i][t % C::NB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // slice SL sits in stage `sa`; slice SL+1 goes into stage `sb` meanwhile
    auto slices = [&](char* sa, char* sb) __attribute__((always_inline)) {
      auto step = [&](auto sl_c, char* cur, char* nxt) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (SL + 1 < C::NRS) issue_slice(SL + 1, nxt);
        cross_slice(sl_c, cur);
      };
      step(std::integral_constant<int, 0>{}, sa, sb);
      step(std::integral_constant<int, 1>{}, sb, sa);
      if constexpr (C::NRS > 2) {
        step(std::integral_constant<int, 2>{}, sa, sb);
        step(std::integral_constant<int, 3>{}, sb, sa);
      }
    };
    static_assert(C::NRS == 2 || C::NRS == 4, "two or four R^T slices");
    // the last key block used stage0 when nkb is odd, so slice 0 is in stage1
    if (nkb & 1)
      slices(stage1, stage0);
    else
      slices(stage0, stage1);
    if constexpr (!FAST) {
#pragma unroll
      for (int i = 0; i < QG; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xi = inv[i][e] == 1.f ? 1.f : gpow((float)(grow(i) + 4 * g + e - c0 + 1), lg);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) oacc[i][nb][e] *= xi;
        }
    }
  }

  // Epilogue: GroupNorm over dv per (token, head), swish gate, store. Each
  // wave stages one 16-row group at a time through its own LDS area to turn
  // the accumulator layout into row-contiguous stores. The gate of the next
  // group loads while the current one is processed (bf16; fp32 gates take
  // twice the registers and load per group).
  constexpr bool kGatePipe = sizeof(T) == 2;
  Raw8<T> gbuf[kGatePipe ? 2 : 1][EI];
  if (kGatePipe && G) load_gate(0, gbuf[0]);
  __syncthreads();  // every wave is done with the stages
  float* yw = reinterpret_cast<float*>(wave < 2 ? stage0 : stage1) + (wave & 1) * 16 * C::YSTR;
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    Raw8<T>(&gq)[EI] = gbuf[kGatePipe ? (i & 1) : 0];
    if (G) {
      if constexpr (kGatePipe) {
        if (i + 1 < QG) load_gate(i + 1, gbuf[(i + 1) & 1]);
      } else {
        load_gate(i, gq);
      }
    }
    // row factor of the fast path (1 otherwise): o = f o'. GroupNorm of f o'
    // is (o' - mean') f / sqrt(f^2 var' + eps), so the statistics are taken
    // on o' and the factor joins the scale.
    float mean[4], rstd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = FAST ? gpow((float)(grow(i) + 4 * g + e - ref), lg) : 1.f;
      mean[e] = 0.f;
      rstd[e] = f;
      if (G) {
        float s = 0.f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) s += oacc[i][nb][e];
        mean[e] = sum16(s) * (1.0f / D);
        float s2 = 0.f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const float d = oacc[i][nb][e] - mean[e];
          s2 += d * d;
        }
        rstd[e] = f * rsqrtf(f * f * (sum16(s2) * (1.0f / D)) + p.eps);
      }
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) yw[(4 * g + e) * C::YSTR + nb * 16 + c] = (oacc[i][nb][e] - mean[e]) * rstd[e];
    // the slab is private to this wave: its own LDS writes are done before
    // it reads them back
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < EI; ++e) {
      const int idx = lane + 64 * e;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      const int tok = grow(i) + r;
      const float* yp = yw + r * C::YSTR + c8 * 8;
      const f32x4 ya = reinterpret_cast<const f32x4*>(yp)[0];
      const f32x4 yb = reinterpret_cast<const f32x4*>(yp)[1];
      F8 y{{ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]}};
      if (G) {
        const F8 gv = unpack8(gq[e]);
#pragma unroll
        for (int k = 0; k < 8; ++k) y.x[k] *= swish(gv.x[k]);
      }
      if (tok < cend) store8(O + tok * tstride + c8 * 8, y);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the slab's reads are done before it is rewritten
    __builtin_amdgcn_wave_barrier();
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

// State role: rows dk0 .. dk0+ROWS-1 (dk0 = ROWS part) of R_i for one chunk
// of one (sequence, head). Accumulates
// dR = K^T (V (.) zeta) over the chunk's keys, waits for R_{i-1} in the fp32
// chain from the previous chunk's workgroup, forms R_i = g^b R_{i-1} + dR,
// hands it on in the chain and then publishes its snapshot R_i^T for the next
// chunk's output workgroups.
template <typename T, int D>
__device__ __forceinline__ void state_role(const FwdParams& p, int bh, int ci, int part, char* stage0,
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
  const int dk0 = part * SC::ROWS;
  const T* K = reinterpret_cast<const T*>(p.k) + head0 + dk0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  // flags of chunk index j for this part: kind 0 = chain, 1 = snapshot
  auto flag_of = [&](int j, int kind) __attribute__((always_inline)) {
    return p.ctrl + kCtrlHead + (bh * (p.nchunks + 1) + j) * kFlagsPerChunk + kind * kMaxSplit + part;
  };

  // accumulator element (a, nb, j) of lane (g, c) is R[dk][dv] with
  const int dkl = dk0 + wave * (SC::ROWS / 4) + 4 * g;  // + 16 a + j
  const int dvl = c;                        // + 16 nb
  T* snap_next = reinterpret_cast<T*>(p.snap) + ((int64_t)bh * p.nchunks + ci + 1) * D * D;
  auto write_snapshot = [&](T* sn, const f32x4 (&acc)[SC::RB][SC::NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
        store4_coherent(sn + (int64_t)(dvl + nb * 16) * D + dkl + 16 * a, acc[a][nb]);
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
        for (int j = 0; j < 4; ++j) racc[a][nb][j] = S0[(int64_t)(dkl + 16 * a + j) * D + dvl + nb * 16];
    write_snapshot(reinterpret_cast<T*>(p.snap) + (int64_t)bh * p.nchunks * D * D, racc);
    release_flag(flag_of(0, 1));
  }
#pragma unroll
  for (int a = 0; a < SC::RB; ++a)
#pragma unroll
    for (int nb = 0; nb < SC::NB; ++nb) racc[a][nb] = zero4();

  auto issue_kv = [&](int j, char* buf) __attribute__((always_inline)) {
    state_issue<T, D>(buf, K, V, tstride, c0 + j * SC::BK, cend - 1, wave, lane);
  };
  // zeta_k = g^(cend-1-k) for key k = kb0 + 32 ks + koff(j), with koff(j) the
  // column-fragment key order {4g..4g+3, 16+4g..16+4g+3}
  float zl[8];  // this lane's part: g^-koff(j)
#pragma unroll
  for (int j = 0; j < 8; ++j) zl[j] = gpow(-(float)(j < 4 ? 4 * g + j : 16 + 4 * g + j - 4), lg);
  // dR += K_blk^T (V_blk (.) zeta): zeta is applied to the K^T fragments (one
  // factor per key), keys past the chunk get zero.
  auto block = [&](int kb0, const char* kt) __attribute__((always_inline)) {
    const char* vt = kt + SC::KT::BYTES;
    const bool ragged = kb0 + SC::BK > cend;  // keys past the chunk in this block (uniform)
#pragma unroll
    for (int ks = 0; ks < SC::BK / 32; ++ks) {
      float z[8];
      bool keep[8];
      if (ragged || lg < -1.5f) {  // exact per key (vanishing decays, ragged block)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = kb0 + ks * 32 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
          keep[j] = key < cend;
          z[j] = gpow((float)(cend - 1 - key), lg);
        }
      } else {
        const float zs = gpow((float)(cend - 1 - kb0 - ks * 32), lg);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          keep[j] = true;
          z[j] = zs * zl[j];
        }
      }
      frag_t<T> af[SC::RB];
#pragma unroll
      for (int a = 0; a < SC::RB; ++a) {
        af[a] = tile_col8<typename SC::KT>(kt, ks * 32, wave * (SC::ROWS / 4) + 16 * a, lane, (T*)nullptr);
        if (ragged)
          scale_frag(af[a], z, keep);
        else
          scale_frag(af[a], z);
      }
      auto vload = [&](int t) __attribute__((always_inline)) {
        return tile_col8<typename SC::VT>(vt, ks * 32, t * 16, lane, (T*)nullptr);
      };
      frag_t<T> vb[3];
      vb[0] = vload(0);
      vb[1] = vload(1);
#pragma unroll
      for (int t = 0; t < SC::NB; ++t) {
        if (t + 2 < SC::NB) vb[(t + 2) % 3] = vload(t + 2);
#pragma unroll
        for (int a = 0; a < SC::RB; ++a) racc[a][t] = mma(af[a], vb[t % 3], racc[a][t]);
        __builtin_amdgcn_sched_barrier(0);
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

  // R_i = g^b R_{i-1} + dR_i. The fp32 chain keeps R in this role's
  // accumulator layout (four contiguous floats per lane and fragment), so
  // the next chunk's workgroup reads it back coalesced.
  auto chain_frag = [&](int slot, int a, int nb) __attribute__((always_inline)) {
    return p.chain + ((int64_t)bh * 2 + slot) * D * D +
           ((((part * 4 + wave) * SC::RB + a) * SC::NB + nb) * 64 + lane) * 4;
  };
  const float dec = gpow((float)(cend - c0), lg);
  if (ci > 0) {
    wait_flag(flag_of(ci, 0), p.ctrl + 1);
    const int slot = (ci - 1) & 1;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb) {
        const f32x4 r = load4_coherent(chain_frag(slot, a, nb));
#pragma unroll
        for (int j = 0; j < 4; ++j) racc[a][nb][j] += dec * r[j];
      }
  } else if (p.state_in) {
    const float* S0 = p.state_in + (int64_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) racc[a][nb][j] += dec * S0[(int64_t)(dkl + 16 * a + j) * D + dvl + nb * 16];
  }
  if (ci + 1 < p.nchunks) {
    // the next state workgroup needs only the chain: release it first
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb) store4_coherent(chain_frag(ci & 1, a, nb), racc[a][nb]);
    release_flag(flag_of(ci + 1, 0));
    write_snapshot(snap_next, racc);
    release_flag(flag_of(ci + 1, 1));
  } else if (p.state_out) {
    float* SO = p.state_out + (int64_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < SC::RB; ++a)
#pragma unroll
      for (int nb = 0; nb < SC::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) SO[(int64_t)(dkl + 16 * a + j) * D + dvl + nb * 16] = racc[a][nb][j];
  }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------
template <typename T, int D, bool FAST>
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
  out_role<T, D, FAST>(p, bh, 0, qb, false, stage0, stage1);
#endif
}

template <typename T, int D, bool FAST>
__global__ __launch_bounds__(256, 1) void retention_chunkwise_kernel(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  __shared__ __attribute__((aligned(1024))) char stage0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[Stage<T, D>::BYTES];
  __shared__ int s_ticket;
  constexpr int SPLIT = StTile<T, D>::SPLIT;
  const int bhs = p.batch * p.heads;
  const int roles = SPLIT + p.qblocks;  // workgroups per (sequence, head, chunk)
  // class of this workgroup: blockIdx mod 8, which is also the XCD it runs on
  // when workgroups are dealt round-robin over the 8 XCDs
  const int cls = p.xcd_order ? (int)(blockIdx.x & 7) : 0;
  if (threadIdx.x == 0) {
    atomicAdd(p.ctrl, 1);  // workgroups that ran
    s_ticket = p.xcd_order ? atomicAdd(p.ctrl + kTicketWord + cls, 1) : atomicAdd(p.ctrl + kTicketWord, 1);
  }
  __syncthreads();
  const int t = s_ticket;
  int ci, bh, role;  // role < SPLIT: state part; else query block qblocks-1-(role-SPLIT)
  if (p.xcd_order) {
    // Class c owns the (sequence, head) pairs bh = 8j + c and takes them
    // chunk-major, role-major: every dependency stays inside the class, and
    // the workgroups of one chunk share an XCD and its L2 when the class is
    // the XCD. Each class has exactly total/8 workgroups and items.
    const int nbl = bhs / 8;
    ci = t / (nbl * roles);
    const int r = t % (nbl * roles);
    role = r / nbl;
    bh = (r % nbl) * 8 + cls;
  } else {
    ci = t / (bhs * roles);
    const int r = t % (bhs * roles);
    bh = r / roles;
    role = r % roles;
  }
  const int qb = role < SPLIT ? -1 : p.qblocks - 1 - (role - SPLIT);
  if (qb < 0)
    state_role<T, D>(p, bh, ci, role, stage0, stage1);
  else
    out_role<T, D, FAST>(p, bh, ci, qb, true, stage0, stage1);
#endif
}

__global__ void reset_ctrl_kernel(int* ctrl, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) ctrl[i] = 0;
}

template <typename T, int D, bool FAST>
static hipError_t launch_fwd_impl(const Shape& s, int chunk, FwdParams p, bool chunked, hipStream_t stream) {
  using C = OutTile<T, D, FAST>;
  p.qblocks = (chunk + C::BM - 1) / C::BM;
  const int bhs = s.batch * s.heads;
  if (!chunked) {
    const int64_t blocks = (int64_t)bhs * p.qblocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((retention_parallel_kernel<T, D, FAST>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t nctrl = kCtrlHead + (int64_t)bhs * (p.nchunks + 1) * kFlagsPerChunk;
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3((unsigned)((nctrl + 255) / 256 < 1024 ? (nctrl + 255) / 256 : 1024)),
                     dim3(256), 0, stream, p.ctrl, (int)nctrl);
  p.xcd_order = bhs % 8 == 0;
  const int64_t blocks = (int64_t)p.nchunks * bhs * (StTile<T, D>::SPLIT + p.qblocks);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((retention_chunkwise_kernel<T, D, FAST>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The fast path applies when every head's decay over the span of one
// workgroup's factors (the chunk, or the parallel form's query block) stays
// within 2^64.
template <typename T, int D>
static hipError_t launch_fwd_t(const Shape& s, int chunk, FwdParams p, bool chunked, hipStream_t stream) {
  const double span = chunked ? chunk : OutTile<T, D, true>::BM;
  bool fast = true;
  for (int h = 0; h < s.heads; ++h) fast = fast && -(double)s.log2g[h] * span <= kFastSpanLog2;
  return fast ? launch_fwd_impl<T, D, true>(s, chunk, p, chunked, stream)
              : launch_fwd_impl<T, D, false>(s, chunk, p, chunked, stream);
}

size_t chunkwise_ctrl_bytes(int batch, int heads, int nchunks) {
  return ((size_t)kCtrlHead + (size_t)batch * heads * (nchunks + 1) * kFlagsPerChunk) * sizeof(int);
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
