// Parallel and chunkwise forms of retention ("Retentive Network: A Successor
// to Transformer...", Elamur summary, Summary: the parallel form for
// training; the chunkwise form computes each chunk in parallel and passes the
// recurrent state between chunks). For chunk i of length b:
//     O_i = (Q_i K_i^T (.) D) V_i  +  xi (.) (Q_i R_{i-1})       xi_r = g^(r+1)
//     R_i = g^b R_{i-1} + K_i^T (V_i (.) zeta)                    zeta_r = g^(b-1-r)
// followed by GroupNorm + swish gate. The parallel form is one chunk that
// spans the whole sequence with no carried state. K arrives rotated; q is
// turned by the angle table as the output role loads it.
//
// Two workgroup roles share one kernel for the chunkwise form:
//   * output role: 8 waves for bf16 (4 for fp32), 32 query rows each, so 256
//     (128) rows of one chunk of one (sequence, head); each wave owns the
//     full dv-wide fp32 output tile of its rows in registers. It streams the
//     chunk's K and V blocks up to its diagonal through two LDS stages
//     (direct global->LDS loads, the next block's loads overlapping the
//     matrix-core work on the current one), computes S^T = K Q^T, the decay
//     mask and O += P V, then -- last -- waits for R_{i-1} and adds the
//     cross-chunk term, then GroupNorm + gate.
//   * state role: one workgroup per chunk of one (sequence, head) for bf16
//     (two, one per 128 dk rows, for fp32 at D = 256); accumulates
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
// The backward's products use separate instantiations (XF) that can read q
// (and, with KVR, k and v) in reversed token order and store their output
// reversed and turned back by the rotation; GBW forms the gradient through
// the gate and GroupNorm in the recomputed forward's epilogue; the forward
// instantiations carry none of that code.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace ret {

// FAST: every head's decay over the span that one workgroup's decay factors
// cover stays within 2^64 (see kFastSpanLog2); the scores then take one factor
// per key and the rows one factor at the end.
// Waves per workgroup: eight for bf16 (two per SIMD: the direct loads of a
// compute unit run faster with more waves issuing them, and one wave's LDS
// and matrix work overlaps the other's), four for fp32, whose fragments take
// twice the registers.
template <typename T> constexpr int kWaves = sizeof(T) == 2 ? 8 : 4;

template <typename T, int D, bool FAST = true>
struct OutTile {
  static constexpr int E = sizeof(T);
  static constexpr int WAVES = kWaves<T>;
  // 32-row query tiles per wave. Every K, V and R^T fragment read from LDS
  // feeds QT products; two tiles would halve the LDS traffic per product but
  // need more than a wave's registers at D = 256 (O^T and Q alone take 384).
  static constexpr int QT = 1;
  static constexpr int QW = 32 * QT;           // query rows per wave
  static constexpr int BM = WAVES * QW;        // query rows per workgroup
  static constexpr int BN = E == 2 ? 64 : 32;  // keys per block
  static constexpr int KH = BN / 32;           // 32-key steps per block
  static constexpr int KS = D / 16;            // contraction steps over dk
  static constexpr int NT = D / 32;            // 32-wide dv tiles
  // dk columns per R^T slice (32 KiB at most); the slices stream through
  // two LDS arrays
  static constexpr int RS = D / 2 < 128 / E ? D / 2 : 128 / E;
  static constexpr int NRS = D / RS;
  using KT = LTile<T, BN, D, kRowTile>;  // K block, row fragments
  using VT = LTile<T, BN, D, kColTile>;  // V block, column (transpose) fragments
  // R^T slice: RS dk columns x D dv rows, stored (in HBM and LDS alike) in
  // fragment order: [dk step s][dv tile t][lane][8 elements], lane (n, h)
  // holding R^T[32 t + n][16 s + 8 h .. +7] -- the A operand of the cross term
  static constexpr int RT_BYTES = RS * D * E;
  static constexpr int KVB = KT::BYTES + VT::BYTES;
};

// Fast path: with a reference row r0 (the row before the chunk, or before the
// parallel form's query block) the decay factors split as
//     g^(q-k) = g^(q - r0) * g^(r0 - k):
// the products P' = S g^(r0 - k) accumulate O' = P' V (+ Q R_{i-1}, whose row
// scale xi_q = g^(q - r0) is then the same row factor), and O = g^(q - r0) O'.
// Keys reach at most one span past r0, so |log2 g| * span <= 64 keeps every
// factor within 2^+-64 (factors of far keys underflow towards zero, which is
// what they are worth).
constexpr double kFastSpanLog2 = 64.0;

// chunkwise grids of at most this many workgroups (one and a half per CU)
// split each chunk's state over two workgroups (bf16, d = 256): measured on
// 384 workgroups (-3%) and against it on 480 (+11%), where the extra state
// workgroups no longer fit beside the others
constexpr int64_t kSmallGrid = 384;

// SPL: state workgroups per chunk (the default, or two for a small grid)
template <typename T, int D, int SPL = (kWaves<T> < 8 && D > 128 ? D / 128 : 1)>
struct StTile {
  // State workgroups per chunk: one (eight waves), or one per 128 dk rows of
  // R (four waves, D = 256). Fewer rows per workgroup shorten the serial
  // chunk-to-chunk hand-off; more rows read V once for more of R and give
  // each block more work to hide the loads of the next. The waves form a
  // WR x WC grid over the workgroup's 32 x 32 tiles of R (rows x dv), each
  // holding MTW x NTW tiles in fp32 registers; waves past the tiles (D = 64)
  // stay idle.
  static constexpr int NW = kWaves<T>;
  static constexpr int SPLIT = SPL;
  static constexpr int ROWS = D / SPLIT;        // dk rows per workgroup
  static constexpr int BK = 32 / (int)sizeof(T) * 2;  // keys per block: 32 (bf16), 16 (fp32)
  static constexpr int MTA = ROWS / 32, NTA = D / 32;   // tiles of the workgroup
  // wave columns: with eight waves two wave rows, so that a wave's 4 tiles
  // take 2 K^T and 2 V fragments per step (4 x 1 tiles would take 5)
  static constexpr int WC = NW >= 8 && NTA >= NW / 2 && MTA >= 2 ? NW / 2 : (NW < NTA ? NW : NTA);
  static constexpr int WR = NW / WC;                    // wave rows
  static constexpr int NTW = NTA / WC;                  // dv tiles per wave
  static constexpr int MTW = MTA / WR > 0 ? MTA / WR : 1;  // row tiles per wave
  static constexpr int ACTIVE = (MTA / MTW) * WC;       // waves with tiles
  using KT = LTile<T, BK, ROWS, kColTile>;      // this workgroup's dk columns of K (K^T operand)
  using VT = LTile<T, BK, D, kColTile>;         // V block, column fragments
  static constexpr int KVB = KT::BYTES + VT::BYTES;
  static_assert(WC * NTW == NTA && (MTA / MTW) * MTW == MTA, "the waves cover every tile");
};
// per (sequence, head, chunk j) and state part q two ready flags: rows of
// R_{j-1} in the fp32 chain (for chunk j's state workgroup of part q) and in
// the snapshot (for chunk j's output workgroups)
constexpr int kMaxSplit = 2;
constexpr int kFlagsPerChunk = 2 * kMaxSplit;

template <typename T, int D>
struct Stage {
  // Four LDS arrays of BYTES each. The output role's two stages are arrays
  // (0, 1) and (2, 3) (K tile, V tile), its R^T slices alternate between
  // arrays 2 and 0; the state role keeps four stages, one per array, with
  // up to three blocks in flight.
  using O = OutTile<T, D>;
  using S = StTile<T, D>;
  static constexpr int max2(int a, int b) { return a > b ? a : b; }
  // output epilogue: each wave stages its 32 rows, HALF dv columns at a
  // time, as fp32 rows of EROW bytes (padded against bank conflicts); two
  // waves share an array
  static constexpr int HALF = D < 128 ? D : 128;
  static constexpr int EROW = HALF * 4 + 16;
  static constexpr int BYTES =
      max2(max2(max2(O::KT::BYTES, O::VT::BYTES), max2(O::RT_BYTES, S::KVB)), 2 * 32 * EROW);
  static_assert(O::WAVES <= 8, "two waves per array");
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  void* o;
  const float* state_in;
  float* state_out;
  void* snap;    // [BH][nchunks][D*D] of T: R_{i-1}^T for chunk i (output fragment order)
  float* chain;  // [BH][2][D*D] fp32: R_i handed to the next state workgroup (fragment order)
  int* ctrl;     // [0] count, [1] error, [8..15] tickets, [16 + (bh*(nchunks+1) + i)*4 + kind*2 + part]: R_{i-1} ready
  // ints from ctrl to this product's ready flags' block (0 but for the
  // second and third products of a launch of several, which share the first
  // one's count, tickets and error word)
  int fbase;
  const float2* rot;  // (cos, sin) per position and pair [seqlen][D/2]: q is turned on load; null: no rotation
  // parallel form only (the backward's products): read q with each sequence's
  // token order reversed; store the output reversed, and/or turned back by
  // out_rot's angles of the stored position (null: as computed)
  int q_rev, out_rev;
  const float2* out_rot;
  // the recomputed forward of the backward (GBW instantiations): dout, and
  // the gate's gradient dg ([batch][seqlen][heads][d], input dtype)
  const void* gb_dout;
  void* gb_dg;
  // (backward instantiations) read k, v with each sequence's token order
  // reversed: the reversed copies that two gradient products take as keys
  // or values, read from the forward-order tensor instead of copied
  int k_rev, v_rev;
  // (the chunkwise multi-product kernel) state workgroups per chunk of this
  // product: the state role's split, or 0 for a product whose snapshots
  // another product's state workgroups write (raising this product's flags),
  // or an earlier launch wrote (snap_ready: nothing to wait for)
  int sroles, snap_ready;
  // (instantiations with the partner snapshot) the snapshots of a partner
  // product whose state is the transpose of this one, written by this
  // product's state workgroups beside their own (null: none), and the ints
  // from ctrl to the partner's ready flags (-1: raise none)
  void* xsnap;
  int xfbase;
  // packed sequences of different lengths (chunkwise form only): sequence b
  // holds rows cu[b] .. cu[b+1]-1 of `total`, seqlen bounds every length;
  // null: batch sequences of seqlen tokens each
  const int* cu;
  int total;
  // their schedule: per ticket class, the (chunk, pair, role) of every
  // workgroup with work in ticket order, then entries with chunk -1
  const int4* sched;
  int per_class;
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

// coherent (sc1) stores and loads of handed-off values, as buffer accesses:
// a scalar descriptor, a per-lane byte offset and a wave-uniform byte offset
// (no per-lane 64-bit addresses to keep in registers)
constexpr int kSc1 = 16;  // cache policy bits: sc1
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, bf16*,
                                                const f32x4& x) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)x[i];
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), rs, voff, soff, kSc1);
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, float*,
                                                const f32x4& x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, voff, soff, kSc1);
}
// volatile (bit 31 of the policy word, a compiler-side flag): the loads keep
// their place relative to scheduling barriers
__device__ __forceinline__ u32x4 load4_coherent(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kSc1 | (int)0x80000000u);
}

// First row and length of sequence b: b * seqlen and seqlen for a batch of
// equal lengths; packed sequences take theirs from cu, clamped into the
// tensor, and a clamp sets bit 2 of the error word (the output is then not
// valid).
__device__ __forceinline__ int seq_rows(const FwdParams& p, int b, int64_t& tok0) {
  if (!p.cu) {
    tok0 = (int64_t)b * p.seqlen;
    return p.seqlen;
  }
  int t0, len;
  if (!packed_span(p.cu, b, p.total, p.seqlen, t0, len) && threadIdx.x == 0) atomicOr(p.ctrl + 1, 2);
  tok0 = t0;
  return len;
}

// ---------------------------------------------------------------------------
// Output role.
// ---------------------------------------------------------------------------
// CROSS: the chunk has a previous state R_{i-1} (chunkwise form, chunk > 0
// or an initial state); the parallel form and chunk 0 without one have none.
// XF: the instantiations that may read q reversed and store their output
// reversed and/or turned back (the backward's products: one launch of the
// parallel or chunkwise multi-product kernel, and the recomputed forward);
// the forward kernels carry none of that code.
// GBW (with XF): the backward's recomputed forward. In place of the forward
// epilogue it forms the gradient through the swish gate and the GroupNorm
// (from the gate g, the caller's dout and the recomputed output, still in
// registers): dg, stored in token order, and dO, stored at each sequence's
// reversed token positions.
// KVR (with XF): k and/or v may be read in reversed token order (p.k_rev,
// p.v_rev).
// SPL: the state workgroups per chunk whose snapshots the cross term waits for.
template <typename T, int D, bool FAST, bool CROSS, bool XF = false, bool GBW = false, bool KVR = false,
          int SPL = StTile<T, D>::SPLIT>
__device__ __forceinline__ void out_role(const FwdParams& p, int bh, int ci, int qb, bool chunked, char* l0, char* l1,
                                         char* l2, char* l3) {
  using C = OutTile<T, D, FAST>;
  constexpr int QT = C::QT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;  // column / half of the 32x32 layout

  // integer division runs on the vector unit: bring the uniform results back
  // to scalar registers
  const int h = uniform_i(bh % p.heads), b = uniform_i(bh / p.heads);
  int64_t tok0;
  const int len = seq_rows(p, b, tok0);
  const int c0 = ci * p.chunk;
  const int cend = min(c0 + p.chunk, len);
  const int q0 = c0 + qb * C::BM;
  if (q0 >= cend) return;  // uniform for the whole workgroup

  const float lg = p.log2g[h];
  const int ref = chunked ? c0 - 1 : q0 - 1;  // reference row of the fast path
  const int64_t tstride = (int64_t)p.heads * D;  // elements between tokens
  const int64_t head0 = (tok0 * p.heads + h) * D;
  const T* Q = reinterpret_cast<const T*>(p.q) + head0;
  const T* K = reinterpret_cast<const T*>(p.k) + head0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  const T* G = p.g ? reinterpret_cast<const T*>(p.g) + head0 : nullptr;
  T* O = reinterpret_cast<T*>(p.o) + head0;

  const int qw0 = q0 + wave * C::QW;  // first row of this wave
  // this lane's query row in the wave's query tile r: qw0 + 32 r + n
  const int kend = min(q0 + C::BM, cend);
  const int nkb = (kend - c0 + C::BN - 1) / C::BN;

  TileLoads<T, typename C::KT, C::WAVES> kload;
  TileLoads<T, typename C::VT, C::WAVES> vload;
  const bool krev = KVR && p.k_rev, vrev = KVR && p.v_rev;  // uniform
  if (krev)
    kload.init_rev(tstride, lane);
  else
    kload.init(tstride, lane);
  if (vrev)
    vload.init_rev(tstride, lane);
  else
    vload.init(tstride, lane);
  auto issue_kv = [&](int j, char* kbuf, char* vbuf) __attribute__((always_inline)) {
    const int kb0 = c0 + j * C::BN;
    if constexpr (KVR) {
      if (kb0 + C::BN <= cend) {
        if (krev) kload.issue_rev(kbuf, K, tstride, len, kb0, wave);
        else kload.issue(kbuf, K, tstride, kb0, wave);
        if (vrev) vload.issue_rev(vbuf, V, tstride, len, kb0, wave);
        else vload.issue(vbuf, V, tstride, kb0, wave);
      } else {
        if (krev) kload.issue_clamped_rev(kbuf, K, tstride, len, kb0, cend - 1, wave);
        else kload.issue_clamped(kbuf, K, tstride, kb0, cend - 1, wave);
        if (vrev) vload.issue_clamped_rev(vbuf, V, tstride, len, kb0, cend - 1, wave);
        else vload.issue_clamped(vbuf, V, tstride, kb0, cend - 1, wave);
      }
      return;
    }
    if (kb0 + C::BN <= cend) {
      kload.issue(kbuf, K, tstride, kb0, wave);
      vload.issue(vbuf, V, tstride, kb0, wave);
    } else {
      kload.issue_clamped(kbuf, K, tstride, kb0, cend - 1, wave);
      vload.issue_clamped(vbuf, V, tstride, kb0, cend - 1, wave);
    }
  };
  const T* R = CROSS ? reinterpret_cast<const T*>(p.snap) + ((int64_t)bh * p.nchunks + ci) * D * D : nullptr;
  // R^T slice s ([dv][RS dk columns]) into an LDS stage; waits (once) for
  // the snapshot of R_{i-1} to be published
  auto issue_slice = [&](int sl, char* buf) __attribute__((always_inline)) {
    if (sl == 0 && !(XF && p.snap_ready)) {
      const int* flags = p.ctrl + p.fbase + kCtrlHead + (bh * (p.nchunks + 1) + ci) * kFlagsPerChunk + kMaxSplit;
#pragma unroll
      for (int q = 0; q < SPL; ++q) wait_flag(flags + q, p.ctrl + 1);
    }
    async_flat<T, C::RT_BYTES, C::WAVES, kCoherent>(buf, R + (int64_t)sl * C::RS * D, wave, lane);
  };
  issue_kv(0, l2, l3);

  // Query fragments of this lane's rows, kept in registers for the whole
  // workgroup life: qf[r][s] = Q[qw0 + 32 r + n][16 s + 8 hh .. +7]. Rows
  // past the chunk load a clamped in-range row: their outputs are never
  // stored. With the position rotation on, each adjacent pair of the 8
  // elements (pairs 8 s + 4 hh .. +3) is turned by its row's angles here, in
  // fp32, before the one rounding to the fragment type.
  frag_t<T> qf[QT][C::KS];
#pragma unroll
  for (int r = 0; r < QT; ++r) {
    const int qrow = min(qw0 + 32 * r + n, cend - 1);
    const T* qr = Q + (int64_t)(XF && p.q_rev ? p.seqlen - 1 - qrow : qrow) * tstride + 8 * hh;
    if (p.rot) {
      const float2* cs = p.rot + (int64_t)qrow * (D / 2) + 4 * hh;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        F8 x = unpack8(ld_raw8(qr + 16 * s));
        rotate4(x, ld_cs4(cs + 8 * s));
        qf[r][s] = to_frag(x, (T*)nullptr);
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) qf[r][s] = to_frag(unpack8(ld_raw8(qr + 16 * s)), (T*)nullptr);
    }
  }

  // O^T accumulators: oacc[r][t] element i is O'[qw0 + 32 r + n][32 t + 8 (i/4) + 4 hh + i%4]
  f32x16 oacc[QT][C::NT];
#pragma unroll
  for (int r = 0; r < QT; ++r)
#pragma unroll
    for (int t = 0; t < C::NT; ++t) oacc[r][t] = zero16();

  // per-key decay factors of the fast path: accumulator element i is key
  // 8 (i/4) + 4 hh + i%4 of a 32-key step, with factor
  // g^-(8 (i/4)) g^-(i%4) g^-(4 hh); the first two are wave-uniform (kept in
  // scalar registers), the last one is this lane's.
  float g8[4], g1[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    g8[a] = uniform_f(FAST ? gpow(-(float)(8 * a), lg) : 0.f);
    g1[a] = uniform_f(FAST ? gpow(-(float)a, lg) : 0.f);
  }
  const float ghh = FAST ? gpow(-(float)(4 * hh), lg) : 0.f;

  // Intra-chunk term over key blocks up to the diagonal, 32 keys at a time:
  // S^T = K Q^T (16 products per query tile), decay and causal mask, then
  // O^T += V^T P^T (NT x 2 products per query tile). Every K and V fragment
  // read from LDS feeds the QT query tiles; the fragments of a step form one
  // sequence of LDS reads with a two-deep prefetch ring.
  constexpr int U = C::KS + 2 * C::NT;  // fragment reads per 32-key step
  auto key_block = [&](int kb0, const char* kt, const char* vt) __attribute__((always_inline)) {
    if (kb0 > qw0 + C::QW - 1) return;  // block above this wave's rows (uniform)
    const bool diag = kb0 + C::BN - 1 > qw0;  // some key may follow some row (uniform)
    auto load = [&](auto t_c) __attribute__((always_inline)) {
      constexpr int t = decltype(t_c)::value, kh = t / U, u = t % U;
      if constexpr (u < C::KS)  // K rows 32 kh + n, dk 16 u + 8 hh
        return tile_row8<typename C::KT>(kt, 32 * kh + n, 16 * u + 8 * hh, (T*)nullptr);
      else  // V keys 32 kh + 16 (u' % 2) + {..}, dv 32 (u' / 2) + n
        return tile_col8w<typename C::VT>(vt, 32 * kh + 16 * ((u - C::KS) % 2), 32 * ((u - C::KS) / 2), lane,
                                          (T*)nullptr);
    };
    frag_t<T> ring[3];
    ring[0] = load(std::integral_constant<int, 0>{});
    ring[1] = load(std::integral_constant<int, 1>{});
    f32x16 st[QT];
    frag_t<T> pf[QT][2];
    static_for<C::KH * U>([&](auto t_c) __attribute__((always_inline)) {
      constexpr int t = decltype(t_c)::value, kh = t / U, u = t % U;
      if constexpr (t + 2 < C::KH * U) ring[(t + 2) % 3] = load(std::integral_constant<int, t + 2>{});
      if constexpr (u < C::KS) {
        // The score products run at raised wave priority, the decay below at
        // the normal one: after each block's barrier the two waves of a SIMD
        // start in step, and this lets one wave's products issue while the
        // other does its decay's vector work (measured: 3B parallel -1.1 to
        // -1.4%, 7B/8k chunkwise -0.5%).
        if constexpr (u == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int r = 0; r < QT; ++r) st[r] = mma32(ring[t % 3], qf[r][u], u == 0 ? zero16() : st[r]);
        if constexpr (u == C::KS - 1) __builtin_amdgcn_s_setprio(0);
        if constexpr (u == C::KS - 1) {
          // decay g^(q-k) and causal mask; element i is key kb0 + 32 kh + k_i
          const int kk0 = kb0 + 32 * kh;
#pragma unroll
          for (int r = 0; r < QT; ++r) {
            const int qrow = qw0 + 32 * r + n;
            if constexpr (FAST) {
              const float sb = gpow((float)(ref - kk0), lg) * ghh;  // g^(r0 - kk0 - 4 hh)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                if (i % 4 != 0) st[r][i] *= g1[i % 4];
                st[r][i] *= (i / 4 == 0 ? sb : sb * g8[i / 4]);
              }
              if (diag) {
                // key kk0 + 4 hh + o_i follows the row when o_i > dq: one
                // compare with a constant per score
                const int dq = qrow - kk0 - 4 * hh;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                  if (8 * (i / 4) + (i % 4) > dq) st[r][i] = 0.f;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int dist = qrow - (kk0 + 8 * (i / 4) + 4 * hh + (i % 4));
                const float val = st[r][i] * gpow((float)dist, lg);
                st[r][i] = dist < 0 ? 0.f : val;
              }
            }
            pf[r][0] = acc_frag<0>(st[r], (T*)nullptr);
            pf[r][1] = acc_frag<1>(st[r], (T*)nullptr);
          }
        }
      } else {
        constexpr int v = u - C::KS, tt = v / 2, sl = v % 2;
#pragma unroll
        for (int r = 0; r < QT; ++r) oacc[r][tt] = mma32(ring[t % 3], pf[r][sl], oacc[r][tt]);
      }
      // keep each step's prefetch where it is: two steps ahead of its use
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // One pipeline step: wait for block j, release the other stage, prefetch
  // block j+1 into it. Block j sits in stage (2, 3) for even j, (0, 1) for
  // odd j, so that after an even number of blocks the last step prefetches
  // the first R^T slice into array 2 (after an odd number the slice is
  // loaded once the last block is done). The arrays are distinct LDS objects
  // and the loop is unrolled by two, so the compiler can tell the reads of
  // one stage from the in-flight loads into the other.
  auto sync_and_prefetch = [&](int j, char* nk, char* nv, auto slice_c) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nkb)
      issue_kv(j + 1, nk, nv);
    else if constexpr (CROSS && decltype(slice_c)::value)
      issue_slice(0, nk);
  };
  for (int j = 0; j < nkb; j += 2) {
    sync_and_prefetch(j, l0, l1, std::false_type{});
    key_block(c0 + j * C::BN, l2, l3);
    if (j + 1 < nkb) {
      sync_and_prefetch(j + 1, l2, l3, std::true_type{});
      key_block(c0 + (j + 1) * C::BN, l0, l1);
    }
  }

  // Cross-chunk term, added last. Fast path: O'^T += R^T Q^T (its row scale
  // xi is the final row factor). Otherwise O = xi (.) (O_intra / xi + Q R):
  // a row whose xi is below 2^-100 skips it (its Q fragments are zeroed and
  // its scale is 1), the term being far below fp32 resolution there. The R^T
  // slices stream through two LDS arrays, the first one already in flight;
  // every R^T fragment feeds the QT query tiles.
  if constexpr (CROSS) {
    if (nkb & 1) {  // the last key block sat in arrays 2 and 3
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      issue_slice(0, l2);
    }
    float inv[QT];
#pragma unroll
    for (int r = 0; r < QT; ++r) {
      inv[r] = 1.f;
      if constexpr (!FAST) {
        const float xi = gpow((float)(qw0 + 32 * r + n - c0 + 1), lg);
        if (xi >= 7.888609e-31f) {
          inv[r] = __builtin_amdgcn_rcpf(xi);
        } else {
#pragma unroll
          for (int s = 0; s < C::KS; ++s) qf[r][s] = zero_frag<T>();
        }
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[r][t][i] *= inv[r];
      }
    }
    auto cross_slice = [&](auto sl_c, const char* buf) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value;
      constexpr int SS = C::RS / 16;  // dk steps per slice
      constexpr int NTT = SS * C::NT;
      auto rload = [&](int t) __attribute__((always_inline)) {  // step t / NT, dv tile t % NT
        return *reinterpret_cast<const frag_t<T>*>(buf + (t * 64 + lane) * (int)sizeof(frag_t<T>));
      };
      frag_t<T> rb[3];
      rb[0] = rload(0);
      rb[1] = rload(1);
#pragma unroll
      for (int t = 0; t < NTT; ++t) {
        if (t + 2 < NTT) rb[(t + 2) % 3] = rload(t + 2);
#pragma unroll
        for (int r = 0; r < QT; ++r)
          oacc[r][t % C::NT] = mma32(rb[t % 3], qf[r][SL * SS + t / C::NT], oacc[r][t % C::NT]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // slice SL sits in array 2 (even SL) or 0 (odd SL); slice SL+1 goes into
    // the other one meanwhile
    static_for<C::NRS>([&](auto sl_c) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value;
      char* cur = SL % 2 == 0 ? l2 : l0;
      char* nxt = SL % 2 == 0 ? l0 : l2;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (SL + 1 < C::NRS) issue_slice(SL + 1, nxt);
      cross_slice(sl_c, cur);
    });
    if constexpr (!FAST) {
#pragma unroll
      for (int r = 0; r < QT; ++r) {
        const float xi = inv[r] == 1.f ? 1.f : gpow((float)(qw0 + 32 * r + n - c0 + 1), lg);
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[r][t][i] *= xi;
      }
    }
  }
  // Epilogue. GroupNorm over dv per (token, head) from the registers (each
  // lane holds half of one query row per tile, the other half in lane ^ 32)
  // -- with the fast path's row factor f: GN(f o') = (o' - mean') f /
  // sqrt(f^2 var' + eps) --, then the swish gate. The normalized rows pass
  // through the wave's own LDS area, HALF dv columns at a time, so that the
  // gate loads and the output stores run along rows: LPR lanes cover the
  // HALF columns of one row with 16-byte accesses.
  using SG = Stage<T, D>;
  constexpr int CPL = 16 / (int)sizeof(T);  // columns per lane access
  constexpr int LPR = SG::HALF / CPL;       // lanes per row
  constexpr int RPA = 64 / LPR;             // rows per access
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the LDS arrays
  char* stg = (wave >> 1) == 0 ? l0 : (wave >> 1) == 1 ? l1 : (wave >> 1) == 2 ? l2 : l3;
  stg += (wave & 1) * 32 * SG::EROW;
#pragma unroll
  for (int r = 0; r < QT; ++r) {
    const int qrow = qw0 + 32 * r + n;
    const float f = FAST ? gpow((float)(qrow - ref), lg) : 1.f;
    float mean = 0.f, scale = f;
    if (G) {
      float s1 = 0.f;
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s1 += oacc[r][t][i];
      mean = sum_pair32(s1) * (1.0f / D);
      float s2 = 0.f;
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float d = oacc[r][t][i] - mean;
          s2 += d * d;
        }
      scale = f * rsqrtf(f * f * (sum_pair32(s2) * (1.0f / D)) + p.eps);
    }
    const float shift = -mean * scale;  // normalized value: o scale + shift
    if constexpr (GBW) {
      // With y the normalized row (y = (o - mean) / sigma, sigma =
      // sqrt(var + eps); here y = o' scale + shift) and s = sigmoid(g):
      //   dg = dout y s (1 + g (1 - s)),  dy = dout g s,
      //   dO = (dy - mean(dy) - y mean(dy y)) / sigma.
      // Whole rows pass through the wave's LDS area, PR rows at a time, so
      // that every access holds complete rows: LPR2 lanes per row, 16
      // bytes each, and the two row means reduce across those lanes before
      // the same access forms dO.
      constexpr int CPL = 16 / (int)sizeof(T);
      constexpr int EROW2 = D * 4 + 16;
      constexpr int PR = (32 * SG::EROW) / EROW2 < 32 ? (32 * SG::EROW) / EROW2 : 32;
      constexpr int LPR2 = D / CPL, RPA2 = 64 / LPR2;
      static_assert(PR % RPA2 == 0 && 32 % PR == 0 && PR * EROW2 <= 32 * SG::EROW, "whole rows per pass");
      const float rsr = scale / f;  // 1 / sigma of this lane's row (f > 0 by the fast path's span rule)
      const T* DO = reinterpret_cast<const T*>(p.gb_dout) + head0;
      T* DG = reinterpret_cast<T*>(p.gb_dg) + head0;
      static_for<32 / PR>([&](auto p_c) __attribute__((always_inline)) {
        constexpr int P0 = decltype(p_c)::value * PR;  // first row of the pass within the tile
        if (n >= P0 && n < P0 + PR) {
#pragma unroll
          for (int t = 0; t < C::NT; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<f32x4*>(stg + (n - P0) * EROW2 + (32 * t + 8 * a + 4 * hh) * 4) =
                  f32x4{__builtin_fmaf(oacc[r][t][4 * a], scale, shift),
                        __builtin_fmaf(oacc[r][t][4 * a + 1], scale, shift),
                        __builtin_fmaf(oacc[r][t][4 * a + 2], scale, shift),
                        __builtin_fmaf(oacc[r][t][4 * a + 3], scale, shift)};
        }
        // the pass's gate and dout values, KG accesses at a time, all in
        // flight before the first is used (64 registers for bf16)
        constexpr int NK = PR / RPA2, KG = sizeof(T) == 2 ? NK : (NK < 4 ? NK : 4);
        static_assert(NK % KG == 0, "whole groups");
        const int grow0 = min(qw0 + 32 * r + P0, cend - 1);
        const __amdgpu_buffer_rsrc_t grs = scalar_rsrc(G + (int64_t)grow0 * tstride);
        const __amdgpu_buffer_rsrc_t drs = scalar_rsrc(DO + (int64_t)grow0 * tstride);
#pragma unroll
        for (int k0 = 0; k0 < NK; k0 += KG) {
          u32x4b graw[KG], draw[KG];
#pragma unroll
          for (int kk = 0; kk < KG; ++kk) {
            const int orow = qw0 + 32 * r + P0 + (k0 + kk) * RPA2 + lane / LPR2;
            const int grow = min(orow, cend - 1);  // rows past the chunk load a clamped row and store nothing
            const uint32_t off = (uint32_t)(((grow - grow0) * tstride + (lane % LPR2) * CPL) * (int)sizeof(T));
            graw[kk] = __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0);
            draw[kk] = __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0);
          }
#pragma unroll
          for (int kk = 0; kk < KG; ++kk) {
            const int k = k0 + kk;
            const int rr = k * RPA2 + lane / LPR2, col = (lane % LPR2) * CPL;
            const int orow = qw0 + 32 * r + P0 + rr;
            const float rs = __shfl(rsr, P0 + rr, 64);
            float y[CPL], gv[CPL], dv[CPL];
#pragma unroll
            for (int e = 0; e < CPL; e += 4) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(stg + rr * EROW2 + (col + e) * 4);
#pragma unroll
              for (int i = 0; i < 4; ++i) y[e + i] = x[i];
            }
            load16f_raw(graw[kk], gv, (T*)nullptr);
            load16f_raw(draw[kk], dv, (T*)nullptr);
            float dg[CPL], s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
              const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv[e]));
              dg[e] = dv[e] * y[e] * (sg * __builtin_fmaf(gv[e], 1.0f - sg, 1.0f));
              dv[e] = dv[e] * gv[e] * sg;  // dy
              s1 += dv[e];
              s2 = __builtin_fmaf(dv[e], y[e], s2);
            }
            s1 = sum_lanes<LPR2>(s1);
            s2 = sum_lanes<LPR2>(s2);
            const float m1 = s1 * (1.0f / D), m2 = s2 * (1.0f / D);
#pragma unroll
            for (int e = 0; e < CPL; ++e) dv[e] = (dv[e] - m1 - y[e] * m2) * rs;
            if (orow < cend) {
              store16f(DG + (int64_t)orow * tstride + col, dg);
              store16f(O + (int64_t)(p.seqlen - 1 - orow) * tstride + col, dv);
            }
          }
        }
      });
      continue;
    }
    // The rows of this tile: gate loads and output stores as buffer
    // accesses from a wave-uniform base (the tile's first row) and a 32-bit
    // lane offset. The forward's stores go through a descriptor whose size
    // ends at the chunk's last row, so the stores of rows past it are
    // dropped by the hardware instead of branched around.
    const int row0 = qw0 + 32 * r;
    // rows of the tile inside the chunk: none for a wave past a short last
    // chunk's end (its gate rows clamp to the chunk's last row, and nothing
    // of it is stored)
    const int rows_in = cend - row0;
    const int grow0 = min(row0, cend - 1);  // gate base row: every clamped row is at or after it
    constexpr uint32_t RB = (uint32_t)sizeof(T);
    static_for<D / SG::HALF>([&](auto h_c) __attribute__((always_inline)) {
      constexpr int H = decltype(h_c)::value;
      // this pass's gate values, 16 bytes per row access, ahead of their use
      const int lrow = lane / LPR, lcol = (lane % LPR) * CPL;
      float g[32 / RPA][CPL];
      if (G) {
        const __amdgpu_buffer_rsrc_t grs = scalar_rsrc(G + (int64_t)grow0 * tstride + H * SG::HALF);
#pragma unroll
        for (int k = 0; k < 32 / RPA; ++k) {
          const int grow = min(row0 + k * RPA + lrow, cend - 1);
          const uint32_t off = (uint32_t)(((grow - grow0) * tstride + lcol) * RB);
          load16f_raw(__builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0), g[k], (T*)nullptr);
        }
      }
      // normalized values of dv tiles H HALF/32 .. into the staging rows
#pragma unroll
      for (int t = H * SG::HALF / 32; t < (H + 1) * SG::HALF / 32; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = 32 * t - H * SG::HALF + 8 * a + 4 * hh;
          *reinterpret_cast<f32x4*>(stg + n * SG::EROW + col * 4) =
              f32x4{__builtin_fmaf(oacc[r][t][4 * a], scale, shift), __builtin_fmaf(oacc[r][t][4 * a + 1], scale, shift),
                    __builtin_fmaf(oacc[r][t][4 * a + 2], scale, shift),
                    __builtin_fmaf(oacc[r][t][4 * a + 3], scale, shift)};
        }
      // along the rows: gate, store; the descriptor covers rows row0 ..
      // cend - 1 (the last row only up to this half's end: its bytes past
      // that belong to the next head)
      [[maybe_unused]] __amdgpu_buffer_rsrc_t ors;
      if constexpr (!XF)
        ors = scalar_rsrc(O + (int64_t)grow0 * tstride + H * SG::HALF,
                          rows_in > 0 ? (uint32_t)(((rows_in - 1) * tstride + SG::HALF) * RB) : 0u);
#pragma unroll
      for (int k = 0; k < 32 / RPA; ++k) {
        const int rr = k * RPA + lrow, orow = qw0 + 32 * r + rr;
        float y[CPL];
#pragma unroll
        for (int e = 0; e < CPL; e += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rr * SG::EROW + (lcol + e) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) y[e + i] = v[i];
        }
        if (G) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) y[e] *= swish(g[k][e]);
        }
        if constexpr (XF) {
          if (orow < cend) {
            int mrow = orow;  // stored position
            if (p.out_rev) mrow = p.seqlen - 1 - orow;
            if (p.out_rot) unrotate_pairs<CPL>(y, p.out_rot + (int64_t)mrow * (D / 2) + (H * SG::HALF + lcol) / 2);
            store16f(O + (int64_t)mrow * tstride + H * SG::HALF + lcol, y);
          }
        } else {
          store16f_raw(ors, (uint32_t)((rr * tstride + lcol) * RB), y, (T*)nullptr);
        }
      }
    });
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

// State role: rows dk0 .. dk0+ROWS-1 (dk0 = ROWS part) of R_i for one chunk
// of one (sequence, head). Accumulates dR = K^T (V (.) zeta) over the chunk's
// keys, waits for those rows of R_{i-1} in the fp32 chain from the previous
// chunk's workgroup, forms R_i = g^b R_{i-1} + dR, hands it on in the chain
// and then publishes its snapshot R_i^T for the next chunk's output
// workgroups. Wave (wr, wc) owns row tiles wr MTW .. +MTW-1 and dv tiles
// wc NTW .. +NTW-1.
// XS: the instantiations that may also write a partner product's snapshots
// (p.xsnap), the backward's: the state of the dv gradient product is the
// transpose of the dk product's, and that of the dq product the transpose
// of the recomputed forward's (same decays, same chunks, transposed initial
// states), so one state workgroup serves both.
template <typename T, int D, bool KVR = false, int SPL = StTile<T, D>::SPLIT, bool XS = false>
__device__ __forceinline__ void state_role(const FwdParams& p, int bh, int ci, int part, char* l0, char* l1,
                                           char* l2, char* l3) {
  using SC = StTile<T, D, SPL>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  // integer division runs on the vector unit: bring the uniform results back
  // to scalar registers
  const int h = uniform_i(bh % p.heads), b = uniform_i(bh / p.heads);
  int64_t tok0;
  const int len = seq_rows(p, b, tok0);
  // chunks of this sequence (an empty one still carries state_in to state_out
  // in its chunk 0); the workgroups of the chunks past them have no work
  const int nch = len > 0 ? (len + p.chunk - 1) / p.chunk : 1;
  if (ci >= nch) return;
  const float lg = p.log2g[h];
  const int c0 = ci * p.chunk;
  const int cend = min(c0 + p.chunk, len);
  const int nkb = (cend - c0 + SC::BK - 1) / SC::BK;
  const int64_t tstride = (int64_t)p.heads * D;
  const int64_t head0 = (tok0 * p.heads + h) * D;
  const int dk0 = part * SC::ROWS;
  const T* K = reinterpret_cast<const T*>(p.k) + head0 + dk0;
  const T* V = reinterpret_cast<const T*>(p.v) + head0;
  // flags of chunk index j for this part: kind 0 = chain, 1 = snapshot
  auto flag_of = [&](int j, int kind) __attribute__((always_inline)) {
    return p.ctrl + p.fbase + kCtrlHead + (bh * (p.nchunks + 1) + j) * kFlagsPerChunk + kind * kMaxSplit + part;
  };
  // rows 4 hh + {0..3} + 8 a (a = 0..3) of the wave's row tile mt hold
  // accumulator elements 4a .. 4a+3; the columns are dv = dvw + 32 nt + n
  const int wr = wave / SC::WC, wc = wave % SC::WC;
  const int dvw = wc * SC::NTW * 32;
  const int mt0 = wr * SC::MTW;       // first row tile of the wave
  const bool active = wave < SC::ACTIVE;  // uniform
  auto dk_of = [&](int mt, int a) __attribute__((always_inline)) {
    return dk0 + 32 * (mt0 + mt) + 8 * a + 4 * hh;
  };
  T* snap_next = reinterpret_cast<T*>(p.snap) + ((int64_t)bh * p.nchunks + ci + 1) * D * D;
  // Snapshot R^T in the output role's fragment order (see OutTile): the 4
  // values of (tile mt, nt, row group a) of lane (n, hh) are rows
  // dk = 16 S + 8 (a%2) + 4 hh + e of column dv = 32 t + n, i.e. half hh of
  // the fragment of lane (n, a%2) at step S, tile t. One store per lane writes
  // 8 bytes; a wave writes 512 contiguous bytes.
  using OT = OutTile<T, D>;
  auto write_snapshot = [&](T* sn, const f32x16 (&acc)[SC::MTW][SC::NTW]) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(sn);
    const uint32_t voff = (uint32_t)((n * 8 + 4 * hh) * (int)sizeof(T));  // this lane's part
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int S = (dk0 + 32 * (mt0 + mt)) / 16 + a / 2;  // dk step (uniform)
          const int t = (dvw + 32 * nt) / 32;                   // dv tile (uniform)
          const int soff = (S / (OT::RS / 16)) * OT::RS * D + (((S % (OT::RS / 16)) * OT::NT + t) * 64 + 32 * (a % 2)) * 8;
          store4_coherent(rs, voff, (uint32_t)(soff * (int)sizeof(T)), (T*)nullptr,
                          f32x4{acc[mt][nt][4 * a], acc[mt][nt][4 * a + 1], acc[mt][nt][4 * a + 2], acc[mt][nt][4 * a + 3]});
        }
  };
  // The partner's snapshot (XS, p.xsnap set). Its state R' is R^T, so the
  // snapshot it reads, R'^T in the fragment order above, is R itself: the 8
  // elements of the fragment slot of lane (n, h) at step S, tile t are
  // R[32 t + n][16 S + 8 h .. +7], 8 consecutive dv of one dk row. The
  // workgroup's rows of R pass through LDS as T, row-major, each row padded
  // by 16 bytes (the 16-byte reads of one instruction, 32 rows, then hit
  // distinct banks), 32-row tiles TPA to an array; each lane then reads and
  // stores whole slots, a wave 1 KiB of contiguous snapshot per store.
  constexpr int XROWB = D * (int)sizeof(T) + 16;
  constexpr int XTILEB = 32 * XROWB;
  constexpr int XTPA = Stage<T, D>::BYTES / XTILEB;
  static_assert(!XS || SC::MTA <= 4 * XTPA, "the workgroup's rows of R fit the four arrays");
  auto xs_tile = [&](int tl) __attribute__((always_inline)) {
    const int ai = tl / XTPA;  // uniform
    char* a = ai == 0 ? l0 : ai == 1 ? l1 : ai == 2 ? l2 : l3;
    return a + (tl % XTPA) * XTILEB;
  };
  auto xs_stage = [&](const f32x16 (&acc)[SC::MTW][SC::NTW]) __attribute__((always_inline)) {
    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt) {
      char* tile = xs_tile(mt0 + mt);
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          *reinterpret_cast<T*>(tile + (8 * (i / 4) + 4 * hh + i % 4) * XROWB + (dvw + 32 * nt + n) * (int)sizeof(T)) =
              (T)acc[mt][nt][i];
    }
  };
  // after a barrier that follows xs_stage: the slots of this workgroup's rows
  // (tiles t = dk0/32 + tl) into the partner snapshot sn
  auto xs_store = [&](T* sn) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(sn);
    constexpr int NS = D / 16;                 // steps S per tile
    constexpr int EL = 16 / (int)sizeof(T);    // elements per 16 bytes
#pragma unroll 2
    for (int x = wave; x < SC::MTA * NS; x += SC::NW) {
      const int tl = x / NS, S = x % NS;  // uniform
      const int t = dk0 / 32 + tl;
      const char* src = xs_tile(tl) + n * XROWB + (16 * S + 8 * hh) * (int)sizeof(T);
      const int soff = (S / (OT::RS / 16)) * OT::RS * D + ((S % (OT::RS / 16)) * OT::NT + t) * 64 * 8;
#pragma unroll
      for (int c = 0; c < 8 / EL; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src + 16 * c), rs,
                                               (uint32_t)(lane * 8 * (int)sizeof(T) + 16 * c),
                                               (uint32_t)(soff * (int)sizeof(T)), kSc1);
    }
  };
  auto xflag_of = [&](int j) __attribute__((always_inline)) {
    return p.ctrl + p.xfbase + kCtrlHead + (bh * (p.nchunks + 1) + j) * kFlagsPerChunk + kMaxSplit + part;
  };
  const bool xs = XS && p.xsnap != nullptr;  // uniform

  // R_i accumulates from g^b R_{i-1}: for chunk 0 with an initial state that
  // term is added here (R_{-1} = state_in, also published for the output
  // workgroups of chunk 0); for later chunks after the keys, from the chain
  const float dec = gpow((float)(cend - c0), lg);
  f32x16 racc[SC::MTW][SC::NTW];
  if (ci == 0 && p.state_in && active) {
    const float* S0 = p.state_in + (int64_t)bh * D * D;
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          racc[mt][nt][i] = S0[(int64_t)(dk_of(mt, i / 4) + i % 4) * D + dvw + 32 * nt + n];
    write_snapshot(reinterpret_cast<T*>(p.snap) + (int64_t)bh * p.nchunks * D * D, racc);
    if (xs) xs_stage(racc);
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) racc[mt][nt][i] *= dec;
  } else {
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt) racc[mt][nt] = zero16();
  }
  if (ci == 0 && p.state_in) {
    if (xs) {
      __syncthreads();  // the staged rows of R_{-1}
      xs_store(reinterpret_cast<T*>(p.xsnap) + (int64_t)bh * p.nchunks * D * D);
    }
    // every wave's snapshot stores (and its LDS reads, before the key blocks
    // refill the arrays) are done: both snapshots' flags
    release_flag(flag_of(0, 1));
    if (xs && p.xfbase >= 0 && threadIdx.x == 0)
      __hip_atomic_store(xflag_of(0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  TileLoads<T, typename SC::KT, SC::NW> kload;
  TileLoads<T, typename SC::VT, SC::NW> vload;
  const bool krev = KVR && p.k_rev, vrev = KVR && p.v_rev;  // uniform
  if (krev)
    kload.init_rev(tstride, lane);
  else
    kload.init(tstride, lane);
  if (vrev)
    vload.init_rev(tstride, lane);
  else
    vload.init(tstride, lane);
  auto issue_kv = [&](int j, char* buf) __attribute__((always_inline)) {  // K^T then V tile
    const int kb0 = c0 + j * SC::BK;
    char* vbuf = buf + SC::KT::BYTES;
    if constexpr (KVR) {
      if (kb0 + SC::BK <= cend) {
        if (krev) kload.issue_rev(buf, K, tstride, len, kb0, wave);
        else kload.issue(buf, K, tstride, kb0, wave);
        if (vrev) vload.issue_rev(vbuf, V, tstride, len, kb0, wave);
        else vload.issue(vbuf, V, tstride, kb0, wave);
      } else {
        if (krev) kload.issue_clamped_rev(buf, K, tstride, len, kb0, cend - 1, wave);
        else kload.issue_clamped(buf, K, tstride, kb0, cend - 1, wave);
        if (vrev) vload.issue_clamped_rev(vbuf, V, tstride, len, kb0, cend - 1, wave);
        else vload.issue_clamped(vbuf, V, tstride, kb0, cend - 1, wave);
      }
      return;
    }
    if (kb0 + SC::BK <= cend) {
      kload.issue(buf, K, tstride, kb0, wave);
      vload.issue(vbuf, V, tstride, kb0, wave);
    } else {
      kload.issue_clamped(buf, K, tstride, kb0, cend - 1, wave);
      vload.issue_clamped(vbuf, V, tstride, kb0, cend - 1, wave);
    }
  };
  // zeta_k = g^(cend-1-k); fragment element j is key k0 + kj(j) with
  // kj(j) = 4 hh + j (j < 4), 8 + 4 hh + j - 4 (j >= 4)
  float zl[8];  // this lane's part: g^-kj(j)
#pragma unroll
  for (int j = 0; j < 8; ++j) zl[j] = gpow(-(float)(j < 4 ? 4 * hh + j : 8 + 4 * hh + j - 4), lg);
  // dR += K_blk^T (V_blk (.) zeta): zeta scales the V fragments (one factor
  // per key); keys past the chunk get zero.
  auto block = [&](int kb0, const char* kt) __attribute__((always_inline)) {
    if (!active) return;
    const char* vt = kt + SC::KT::BYTES;
    const bool ragged = kb0 + SC::BK > cend;  // keys past the chunk in this block (uniform)
#pragma unroll
    for (int ks = 0; ks < SC::BK / 16; ++ks) {
      const int k0 = kb0 + 16 * ks;
      float z[8];
      bool keep[8];
      if (ragged || lg < -1.5f) {  // exact per key (vanishing decays, ragged block)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = k0 + (j < 4 ? 4 * hh + j : 8 + 4 * hh + j - 4);
          keep[j] = key < cend;
          z[j] = gpow((float)(cend - 1 - key), lg);
        }
      } else {
        const float zs = gpow((float)(cend - 1 - k0), lg);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          keep[j] = true;
          z[j] = zs * zl[j];
        }
      }
      frag_t<T> af[SC::MTW];
#pragma unroll
      for (int mt = 0; mt < SC::MTW; ++mt)
        af[mt] = tile_col8w<typename SC::KT>(kt, 16 * ks, 32 * (mt0 + mt), lane, (T*)nullptr);
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt) {
        // zeta scales this wave's own V fragments (fewer than its K^T ones)
        frag_t<T> vb = tile_col8w<typename SC::VT>(vt, 16 * ks, dvw + 32 * nt, lane, (T*)nullptr);
        if (ragged)
          scale_frag(vb, z, keep);
        else
          scale_frag(vb, z);
#pragma unroll
        for (int mt = 0; mt < SC::MTW; ++mt) racc[mt][nt] = mma32(af[mt], vb, racc[mt][nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Four stages (one LDS array each), up to three blocks in flight: block j
  // sits in array j % 4. Before block j is read every wave waits until at
  // most its loads of the (up to two) later blocks are outstanding; the
  // barrier then frees array (j - 1) % 4 for block j + 3. With an uneven
  // split of the loads over the waves each step waits for all of them.
  constexpr int LPB = TileLoads<T, typename SC::KT, SC::NW>::PER + TileLoads<T, typename SC::VT, SC::NW>::PER;
  constexpr bool EVEN = SC::KT::NINST % SC::NW == 0 && SC::VT::NINST % SC::NW == 0;
  auto arr = [&](auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value % 4;
    if constexpr (S == 0) return l0;
    else if constexpr (S == 1) return l1;
    else if constexpr (S == 2) return l2;
    else return l3;
  };
  auto wait_landed = [&](int later) __attribute__((always_inline)) {
    // vmcnt <= later * LPB, lgkmcnt 0 (this wave's reads of the array about
    // to be refilled are done), expcnt left alone
    constexpr int kOthers = 0x7 << 4;
    if (EVEN && later >= 2)
      __builtin_amdgcn_s_waitcnt(kOthers | ((2 * LPB) & 15) | (((2 * LPB) >> 4) << 14));
    else if (EVEN && later == 1)
      __builtin_amdgcn_s_waitcnt(kOthers | (LPB & 15) | ((LPB >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0);
  };
  static_assert(2 * LPB < 64, "vmcnt range");
  if (0 < nkb) issue_kv(0, arr(std::integral_constant<int, 0>{}));
  if (1 < nkb) issue_kv(1, arr(std::integral_constant<int, 1>{}));
  if (2 < nkb) issue_kv(2, arr(std::integral_constant<int, 2>{}));
  for (int j = 0; j < nkb; j += 4) {
    static_for<4>([&](auto u_c) __attribute__((always_inline)) {
      constexpr int u = decltype(u_c)::value;
      const int jj = j + u;
      if (jj < nkb) {
        wait_landed(min(2, nkb - 1 - jj));
        bare_barrier();
        if (jj + 3 < nkb) issue_kv(jj + 3, arr(std::integral_constant<int, u + 3>{}));
        block(c0 + jj * SC::BK, arr(u_c));
      }
    });
  }

  // R_i = g^b R_{i-1} + dR_i. The fp32 chain keeps R in this role's
  // accumulator layout (16 contiguous floats per lane and tile), so the next
  // chunk's workgroup of the same part reads it back coalesced: element
  // group q (4 floats) of tile (mt, nt) of a wave sits at a wave-uniform
  // offset, its lanes' 16-byte accesses covering 1 KiB of contiguous bytes.
  auto chain_rsrc = [&](int slot) __attribute__((always_inline)) {
    return scalar_rsrc(p.chain + ((int64_t)bh * 2 + slot) * D * D);
  };
  auto chain_soff = [&](int mt, int nt, int q) __attribute__((always_inline)) {
    return (uint32_t)((((((part * SC::NW + wave) * SC::MTW + mt) * SC::NTW + nt) * 4 + q) * 64) * 16);
  };
  const uint32_t chain_voff = (uint32_t)lane * 16u;
  if (ci > 0) {
    wait_flag(flag_of(ci, 0), p.ctrl + 1);
    if (active) {
      const __amdgpu_buffer_rsrc_t rs = chain_rsrc((ci - 1) & 1);
      // one 32-row tile at a time, every load of the tile in flight before
      // the first use (the compiler would otherwise wait on each in turn)
#pragma unroll
      for (int mt = 0; mt < SC::MTW; ++mt) {
        u32x4 r[SC::NTW][4];
#pragma unroll
        for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) r[nt][q] = load4_coherent(rs, chain_voff, chain_soff(mt, nt, q));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 x = __builtin_bit_cast(f32x4, r[nt][q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) racc[mt][nt][4 * q + e] += dec * x[e];
          }
        __builtin_amdgcn_sched_barrier(0);  // the next tile's loads stay behind this one's uses
      }
    }
  }
  if (ci + 1 < nch) {
    // the next state workgroup needs only the chain: release it first
    if (active) {
      const __amdgpu_buffer_rsrc_t rs = chain_rsrc(ci & 1);
#pragma unroll
      for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store4_coherent(rs, chain_voff, chain_soff(mt, nt, q), (float*)nullptr,
                            f32x4{racc[mt][nt][4 * q], racc[mt][nt][4 * q + 1], racc[mt][nt][4 * q + 2],
                                  racc[mt][nt][4 * q + 3]});
    }
    release_flag(flag_of(ci + 1, 0));
    if (active) write_snapshot(snap_next, racc);
    if (xs) xs_stage(racc);  // the key blocks' reads of the arrays ended before the release's barrier
    release_flag(flag_of(ci + 1, 1));  // its barrier also covers the staged rows
    if (xs) {
      xs_store(reinterpret_cast<T*>(p.xsnap) + ((int64_t)bh * p.nchunks + ci + 1) * D * D);
      if (p.xfbase >= 0) release_flag(xflag_of(ci + 1));
    }
  } else if (p.state_out && active) {
    float* SO = p.state_out + (int64_t)bh * D * D;
#pragma unroll
    for (int mt = 0; mt < SC::MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < SC::NTW; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) SO[(int64_t)(dk_of(mt, i / 4) + i % 4) * D + dvw + 32 * nt + n] = racc[mt][nt][i];
  }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------
// XF: the instantiation with reversed query reads and transforming stores;
// GBW: the backward's recomputed forward (gradient through the gate and
// GroupNorm in the epilogue). The forward's carries none of that code.
template <typename T, int D, bool FAST, bool XF = false, bool GBW = false>
__global__ __launch_bounds__(kWaves<T> * 64, 1) void retention_parallel_kernel(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  __shared__ __attribute__((aligned(1024))) char l0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l1[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l2[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l3[Stage<T, D>::BYTES];
  // Workgroups are dealt out longest first: a query block's work grows with
  // its index (it reads every key up to its diagonal), so the last query
  // blocks of all (sequence, head) pairs go first and the short ones fill the
  // tail. When the pairs divide evenly over the 8 XCDs, the query blocks of
  // one pair stay on one XCD (blockIdx mod 8), sharing its K and V through
  // that XCD's L2.
  int bh, qb;
  const int bid = blockIdx.x;
  const int groups = p.batch * p.heads;
  if (groups % 8 == 0) {
    const int xcd = bid & 7, slot = bid >> 3, per = groups / 8;
    bh = xcd + 8 * (slot % per);
    qb = p.qblocks - 1 - slot / per;
  } else {
    bh = bid % groups;
    qb = p.qblocks - 1 - bid / groups;
  }
  out_role<T, D, FAST, false, XF, GBW>(p, bh, 0, qb, false, l0, l1, l2, l3);
#endif
}

// Several parallel-form products of one shape in one grid (the backward's
// three gradient products, none of which reads another's output): dealt
// out longest query block first across all of them, so that
// the long blocks of every product start at once and the short blocks of all
// fill the end, instead of each launch ending on its own long blocks.
constexpr int kMaxProducts = 3;
struct MultiParams {
  FwdParams p[kMaxProducts];
  int nprod;
};

template <typename T, int D, bool FAST, bool KVR>
__global__ __launch_bounds__(kWaves<T> * 64, 1) void retention_parallel_multi_kernel(MultiParams mp) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char l0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l1[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l2[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l3[Stage<T, D>::BYTES];
  const int nprod = mp.nprod;
  const int groups = mp.p[0].batch * mp.p[0].heads;
  const int bid = blockIdx.x;
  int prod, bh, qb;
  if (groups % 8 == 0) {  // a pair's query blocks stay on one XCD, as in the single launch
    const int xcd = bid & 7, slot = bid >> 3, per = groups / 8;
    qb = mp.p[0].qblocks - 1 - slot / (per * nprod);
    const int r = slot % (per * nprod);
    prod = r / per;
    bh = xcd + 8 * (r % per);
  } else {
    qb = mp.p[0].qblocks - 1 - bid / (groups * nprod);
    const int r = bid % (groups * nprod);
    prod = r / groups;
    bh = r % groups;
  }
  prod = uniform_i(prod);
  out_role<T, D, FAST, false, true, false, KVR>(mp.p[prod], uniform_i(bh), 0, uniform_i(qb), false, l0, l1, l2, l3);
#endif
}

// A workgroup's item: chunk ci of pair bh, role slot `role` of the chunk
// (the dispatch is written out in both chunkwise kernels: as a called
// function, even inlined, it cost the kernel registers). Role order inside a
// chunk: the longest query block first (it pulls the chunk's K and V from
// HBM while the state workgroups follow into L2), the state parts, then the
// other query blocks. Every wait must be for a
// workgroup with an earlier ticket, which is already running, so that no
// number of waiting workgroups can fill the chip: in chunk 0 with a
// carried-in state, whose output workgroups wait for the state parts to
// publish R_{-1}, the state parts come first.
template <typename T, int D, bool FAST, bool XF = false, bool GBW = false, int SPL = StTile<T, D>::SPLIT>
__global__ __launch_bounds__(kWaves<T> * 64, 1) void retention_chunkwise_kernel(FwdParams p) {
  constexpr bool KVR = false;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  __shared__ __attribute__((aligned(1024))) char l0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l1[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l2[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l3[Stage<T, D>::BYTES];
  __shared__ int s_ticket;
  constexpr int SPLIT = SPL;
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
  const int t = __builtin_amdgcn_readfirstlane(s_ticket);  // uniform: scalar registers for all it derives
  int ci, bh, role;  // role slot inside the chunk
  if (p.sched) {
    // packed sequences: the schedule skips the chunks past each sequence's
    // end, so the workgroups without work come last
    const int4 e = p.sched[(int64_t)cls * p.per_class + t];
    ci = uniform_i(e.x);
    if (ci < 0) return;
    bh = e.y;
    role = e.z;
  } else if (p.xcd_order) {
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
  ci = uniform_i(ci);
  bh = uniform_i(bh);
  role = uniform_i(role);
  const bool state_first = ci == 0 && p.has_state0;
  const int qb = state_first ? (role < SPLIT ? -1 : p.qblocks - 1 - (role - SPLIT))
                             : (role == 0 ? p.qblocks - 1 : role <= SPLIT ? -1 : p.qblocks - 1 - (role - SPLIT));
  if (qb < 0)
    state_role<T, D, KVR, SPL, GBW>(p, bh, ci, state_first ? role : role - 1, l0, l1, l2, l3);
  else if (ci > 0 || p.has_state0)
    out_role<T, D, FAST, true, XF, GBW, KVR, SPL>(p, bh, ci, qb, true, l0, l1, l2, l3);
  else
    out_role<T, D, FAST, false, XF, GBW, KVR, SPL>(p, bh, ci, qb, true, l0, l1, l2, l3);
#endif
}

// Several chunkwise products of one shape in one grid (the backward's three
// gradient products): one ticket sequence for all of them, chunk-major with
// the products in order inside each chunk, so every wait is still for an
// earlier ticket (of the same product, or of an earlier product that writes
// this one's snapshots), and the products' last chunks end together instead
// of each launch ending on its own. Each product has its own ready flags,
// chain and snapshots; the tickets, the count and the error word are those
// of the first product's control block. A product with sroles = 0 has no
// state workgroups: its chunks hold only output blocks, longest first.
template <typename T, int D, bool FAST, bool KVR>
__global__ __launch_bounds__(kWaves<T> * 64, 1) void retention_chunkwise_multi_kernel(MultiParams mp) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char l0[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l1[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l2[Stage<T, D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char l3[Stage<T, D>::BYTES];
  __shared__ int s_ticket;
  constexpr int SPLIT = StTile<T, D>::SPLIT;
  const FwdParams& p0 = mp.p[0];
  const int nprod = mp.nprod;
  const int bhs = p0.batch * p0.heads;
  const int cls = p0.xcd_order ? (int)(blockIdx.x & 7) : 0;
  if (threadIdx.x == 0) {
    atomicAdd(p0.ctrl, 1);
    s_ticket = p0.xcd_order ? atomicAdd(p0.ctrl + kTicketWord + cls, 1) : atomicAdd(p0.ctrl + kTicketWord, 1);
  }
  __syncthreads();
  const int t = __builtin_amdgcn_readfirstlane(s_ticket);
  // the pairs a ticket sequence serves, and each product's items per chunk
  const int nbl = p0.xcd_order ? bhs / 8 : bhs;
  int per[kMaxProducts], all = 0;
#pragma unroll
  for (int i = 0; i < kMaxProducts; ++i) {
    per[i] = i < nprod ? nbl * (mp.p[i].sroles + p0.qblocks) : 0;
    all += per[i];
  }
  const int ci = uniform_i(t / all);
  int r = t % all, prod = 0;
  if (r >= per[0]) {
    r -= per[0];
    prod = 1;
    if (r >= per[1]) {
      r -= per[1];
      prod = 2;
    }
  }
  prod = uniform_i(prod);
  const FwdParams& p = mp.p[prod];
  const int roles = p.sroles + p.qblocks;
  int bh, role;
  if (p0.xcd_order) {
    role = r / nbl;
    bh = (r % nbl) * 8 + cls;
  } else {
    bh = r / roles;
    role = r % roles;
  }
  bh = uniform_i(bh);
  role = uniform_i(role);
  constexpr bool XF = true, GBW = false;
  const int sr = p.sroles;
  const bool state_first = ci == 0 && p.has_state0;
  const int qb = sr == 0        ? p.qblocks - 1 - role
                 : state_first ? (role < sr ? -1 : p.qblocks - 1 - (role - sr))
                               : (role == 0 ? p.qblocks - 1 : role <= sr ? -1 : p.qblocks - 1 - (role - sr));
  if (qb < 0)
    state_role<T, D, KVR, SPLIT, true>(p, bh, ci, state_first ? role : role - 1, l0, l1, l2, l3);
  else if (ci > 0 || p.has_state0)
    out_role<T, D, FAST, true, XF, GBW, KVR>(p, bh, ci, qb, true, l0, l1, l2, l3);
  else
    out_role<T, D, FAST, false, XF, GBW, KVR>(p, bh, ci, qb, true, l0, l1, l2, l3);
#endif
}

// Schedule of a packed batch, one workgroup per slot and ticket class (8
// classes with the XCD order, else 1). Each sequence's chunks are spread evenly over the
// launch's nc slots: with n chunks, chunk ci sits in slot
// floor((2 ci + 1) nc / (2 n)), one slot apart for the longest sequences,
// further apart for shorter ones. So the longest chains of chunks, which set
// the critical path, advance from the first tickets on while the other
// sequences' chunks fill the chip beside them, instead of all sequences
// crowding the first slots and the longest chain running alone at the end.
// Slots go in order; inside a slot the entries keep the equal-length
// mapping's order (role-major over the class's pairs, or pair-major over all
// pairs), and the rest of the class's share of the grid gets chunk -1. Every
// wait stays on an earlier ticket: a chunk's predecessor sits in an earlier
// slot (nc / n >= 1), and inside chunk 0 the roles keep their order.
constexpr int kSchedCache = 8192;  // pairs whose chunk counts the schedule kernel keeps in LDS

__global__ __launch_bounds__(256) void varlen_schedule_kernel(FwdParams p, int4* sched, int roles, int classes) {
  __shared__ int s_part[4];
  __shared__ int s_nch[kSchedCache];
  // one workgroup per (slot, class): the slots' entries are written in parallel
  const int cls = blockIdx.x % classes, sl = blockIdx.x / classes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bhs = p.batch * p.heads;
  const int npairs = p.xcd_order ? bhs / 8 : bhs;
  int4* out = sched + (int64_t)cls * p.per_class;
  // chunks of pair j's sequence
  auto chunks_of = [&](int j) {
    const int bh = p.xcd_order ? j * 8 + cls : j;
    const int b = bh / p.heads;
    int tok0, len;
    clamp_span(p.cu[b], p.cu[b + 1], p.total, p.seqlen, tok0, len);
    return len > 0 ? (len + p.chunk - 1) / p.chunk : 1;
  };
  for (int j = tid; j < min(npairs, kSchedCache); j += 256) s_nch[j] = chunks_of(j);
  __syncthreads();
  auto nch_of = [&](int j) { return j < kSchedCache ? s_nch[j] : chunks_of(j); };
  // of a pair with n chunks: the chunks in slots before sl, i.e. those with
  // (2 ci + 1) nc < 2 n sl; that count is also the index of its first chunk
  // at or after slot sl, which lies in sl when (2 ci + 1) nc < 2 n (sl + 1)
  const int64_t nc = p.nchunks;
  auto before = [&](int n) {
    const int64_t num = 2 * (int64_t)n * sl - nc;
    return num <= 0 ? 0 : (int)min((num + 2 * nc - 1) / (2 * nc), (int64_t)n);
  };
  auto chunk_here = [&](int n) {
    const int ci = before(n);
    return ci < n && (2 * (int64_t)ci + 1) * nc < 2 * (int64_t)n * (sl + 1) ? ci : -1;
  };
  // block-wide sum of one int per thread
  auto block_sum = [&](int x) {
    x = (int)sum64((float)x);  // exact: far below 2^24 per wave
    __syncthreads();
    if (lane == 0) s_part[wave] = x;
    __syncthreads();
    return s_part[0] + s_part[1] + s_part[2] + s_part[3];
  };
  int cb = 0, cc = 0, ct = 0;  // this thread's pairs: chunks before the slot, in it, in all
  for (int j = tid; j < npairs; j += 256) {
    const int n = nch_of(j);
    cb += before(n);
    cc += chunk_here(n) >= 0 ? 1 : 0;
    ct += n;
  }
  const int base = roles * block_sum(cb);
  const int count = block_sum(cc);
  const int total = roles * block_sum(ct);
  if (count > 0) {
    int rank0 = 0;  // pairs with work before this tile
    for (int j0 = 0; j0 < npairs; j0 += 256) {
      const int j = j0 + tid;
      const int ci = j < npairs ? chunk_here(nch_of(j)) : -1;
      const bool real = ci >= 0;
      const uint64_t m = __ballot(real);
      const int below = __builtin_popcountll(m & ((uint64_t(1) << lane) - 1));
      __syncthreads();
      if (lane == 0) s_part[wave] = __builtin_popcountll(m);
      __syncthreads();
      int rank = rank0 + below;
      for (int w = 0; w < wave; ++w) rank += s_part[w];
      if (real) {
        const int bh = p.xcd_order ? j * 8 + cls : j;
        for (int r = 0; r < roles; ++r) {
          const int pos = p.xcd_order ? base + r * count + rank : base + rank * roles + r;
          out[pos] = make_int4(ci, bh, r, 0);
        }
      }
      rank0 += s_part[0] + s_part[1] + s_part[2] + s_part[3];
    }
  }
  // the class's entries past its last item, shared among its slots' workgroups
  for (int i = total + sl * 256 + tid; i < p.per_class; i += 256 * p.nchunks) out[i] = make_int4(-1, 0, 0, 0);
}

// Zero the control block before a chunkwise launch; keep_err leaves word 1
// (the error word) as it is, so that a call made of several launches (the
// backward's products) reports an error of any of them.
__global__ void reset_ctrl_kernel(int* ctrl, int n, int keep_err) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    if (!(keep_err && i == 1)) ctrl[i] = 0;
}

// One int copied on the device (a caller's copy of the error word).
__global__ void copy_word_kernel(const int* src, int* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

hipError_t launch_copy_word(const int* src, int* dst, hipStream_t stream) {
  hipLaunchKernelGGL(copy_word_kernel, dim3(1), dim3(64), 0, stream, src, dst);
  return hipGetLastError();
}

template <typename T, int D, bool FAST>
static hipError_t launch_fwd_impl(const Shape& s, int chunk, FwdParams p, bool chunked, hipStream_t stream,
                                  hipEvent_t before, hipEvent_t after, bool keep_err) {
  using C = OutTile<T, D, FAST>;
  p.qblocks = (chunk + C::BM - 1) / C::BM;
  const int bhs = s.batch * s.heads;
  if (!chunked) {
    const int64_t blocks = (int64_t)bhs * p.qblocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (before && hipEventRecord(before, stream) != hipSuccess) return hipErrorInvalidValue;
    if (p.gb_dout)
      hipLaunchKernelGGL((retention_parallel_kernel<T, D, FAST, true, true>), dim3((unsigned)blocks),
                         dim3(64 * C::WAVES), 0, stream, p);
    else if (p.q_rev || p.out_rev || p.out_rot)
      hipLaunchKernelGGL((retention_parallel_kernel<T, D, FAST, true>), dim3((unsigned)blocks), dim3(64 * C::WAVES), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((retention_parallel_kernel<T, D, FAST>), dim3((unsigned)blocks), dim3(64 * C::WAVES), 0,
                         stream, p);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && after && hipEventRecord(after, stream) != hipSuccess) return hipErrorInvalidValue;
    return e;
  }
  const int64_t nctrl = kCtrlHead + (int64_t)bhs * (p.nchunks + 1) * kFlagsPerChunk;
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3((unsigned)((nctrl + 255) / 256 < 1024 ? (nctrl + 255) / 256 : 1024)),
                     dim3(256), 0, stream, p.ctrl, (int)nctrl, keep_err ? 1 : 0);
  p.xcd_order = bhs % 8 == 0;
  // A grid of few workgroups per CU is not filled by the chunks'
  // independent work: the state chain (one link per chunk) sets its length.
  // There (bf16, d = 256, batch form) each chunk's state splits over two
  // workgroups of 128 rows, which halves a link's products, combine and
  // publish.
  constexpr int SPL1 = StTile<T, D>::SPLIT;
  constexpr bool CAN2 = sizeof(T) == 2 && D == 256 && SPL1 == 1;
  const bool two = CAN2 && !p.cu && !p.q_rev && !p.out_rev && !p.out_rot && !p.gb_dout &&
                   (int64_t)p.nchunks * bhs * (SPL1 + p.qblocks) <= kSmallGrid;
  const int roles = (two ? 2 : SPL1) + p.qblocks;
  const int64_t blocks = (int64_t)p.nchunks * bhs * roles;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (p.cu) {
    const int classes = p.xcd_order ? 8 : 1;
    p.per_class = (int)(blocks / classes);
    hipLaunchKernelGGL(varlen_schedule_kernel, dim3((unsigned)(classes * p.nchunks)), dim3(256), 0, stream, p,
                       const_cast<int4*>(p.sched), roles, classes);
  }
  if (before && hipEventRecord(before, stream) != hipSuccess) return hipErrorInvalidValue;
  if (p.gb_dout)
    hipLaunchKernelGGL((retention_chunkwise_kernel<T, D, FAST, true, true>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, p);
  else if (p.q_rev || p.out_rev || p.out_rot)
    hipLaunchKernelGGL((retention_chunkwise_kernel<T, D, FAST, true>), dim3((unsigned)blocks), dim3(64 * C::WAVES), 0,
                       stream, p);
  else if (CAN2 && two)
    hipLaunchKernelGGL((retention_chunkwise_kernel<T, D, FAST, false, false, CAN2 ? 2 : SPL1>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, p);
  else
    hipLaunchKernelGGL((retention_chunkwise_kernel<T, D, FAST>), dim3((unsigned)blocks), dim3(64 * C::WAVES), 0,
                       stream, p);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && after && hipEventRecord(after, stream) != hipSuccess) return hipErrorInvalidValue;
  return e;
}

// The fast path applies when every head's decay over the span of one
// workgroup's factors (the chunk, or the parallel form's query block) stays
// within 2^64.
template <typename T, int D>
static hipError_t launch_fwd_t(const Shape& s, int chunk, FwdParams p, bool chunked, hipStream_t stream,
                               hipEvent_t before, hipEvent_t after, bool keep_err) {
  const double span = chunked ? chunk : OutTile<T, D, true>::BM;
  bool fast = true;
  for (int h = 0; h < s.heads; ++h) fast = fast && -(double)s.log2g[h] * span <= kFastSpanLog2;
  return fast ? launch_fwd_impl<T, D, true>(s, chunk, p, chunked, stream, before, after, keep_err)
              : launch_fwd_impl<T, D, false>(s, chunk, p, chunked, stream, before, after, keep_err);
}

size_t chunkwise_sched_bytes(const Shape& s, int chunk) {
  const int nchunks = (s.seqlen + chunk - 1) / chunk;
  const int bm = s.dtype == 1 ? OutTile<bf16, 64, true>::BM : OutTile<float, 64, true>::BM;
  int split = 1;
  if (s.dtype == 1)
    split = s.d == 256 ? StTile<bf16, 256>::SPLIT : s.d == 128 ? StTile<bf16, 128>::SPLIT : StTile<bf16, 64>::SPLIT;
  else
    split = s.d == 256 ? StTile<float, 256>::SPLIT : s.d == 128 ? StTile<float, 128>::SPLIT : StTile<float, 64>::SPLIT;
  const size_t roles = (size_t)split + (chunk + bm - 1) / bm;
  return (size_t)nchunks * s.batch * s.heads * roles * sizeof(int4);
}

size_t chunkwise_ctrl_bytes(int batch, int heads, int nchunks) {
  return ((size_t)kCtrlHead + (size_t)batch * heads * (nchunks + 1) * kFlagsPerChunk) * sizeof(int);
}

// Kernel parameters of one launch (see launch_retention_fwd for the fields'
// meaning); qblocks and xcd_order are set by the launcher.
static FwdParams make_params(const Shape& s, int chunk, const void* q, const void* k, const void* v, const void* g,
                             void* o, const float* state_in, float* state_out, void* snap, float* chain, int* ctrl,
                             const float2* rot, float eps, bool q_rev, bool out_rev, const float2* out_rot,
                             const int* cu, int total, void* sched) {
  FwdParams p;
  p.cu = cu;
  p.total = total;
  p.sched = cu ? static_cast<const int4*>(sched) : nullptr;
  p.per_class = 0;
  p.rot = rot;
  p.q_rev = q_rev;
  p.out_rev = out_rev;
  p.out_rot = out_rot;
  p.gb_dout = nullptr;
  p.gb_dg = nullptr;
  p.k_rev = 0;
  p.v_rev = 0;
  p.sroles = 0;
  p.snap_ready = 0;
  p.xsnap = nullptr;
  p.xfbase = -1;
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
  p.fbase = 0;
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
  return p;
}

hipError_t launch_retention_fwd(const Shape& s, int chunk, bool chunked, const void* q, const void* k, const void* v,
                                const void* g, void* o, const float* state_in, float* state_out, void* snap,
                                float* chain, int* ctrl, const float2* rot, float eps, hipStream_t stream,
                                hipEvent_t before, hipEvent_t after, bool q_rev, bool out_rev,
                                const float2* out_rot, const int* cu, int total, void* sched, bool keep_err,
                                const void* gb_dout, void* gb_dg, void* xsnap) {
  if (rot && q_rev) return hipErrorInvalidValue;  // q's angles are those of its own positions
  // the recomputed forward of the backward: gate, dout and dg given, dO
  // stored reversed, nothing else transformed, batch form; the partner
  // snapshots only there
  if ((gb_dout != nullptr) != (gb_dg != nullptr) ||
      (gb_dout && (!g || !out_rev || q_rev || out_rot || cu)) || (xsnap && (!gb_dout || !chunked)))
    return hipErrorInvalidValue;
  // packed sequences: chunkwise form, forward only, with a schedule buffer
  if (cu && (!chunked || q_rev || out_rev || out_rot || !sched)) return hipErrorInvalidValue;
  FwdParams p = make_params(s, chunk, q, k, v, g, o, state_in, state_out, snap, chain, ctrl, rot, eps, q_rev, out_rev,
                            out_rot, cu, total, sched);
  p.gb_dout = gb_dout;
  p.gb_dg = gb_dg;
  p.xsnap = xsnap;  // no flags: the later launch reads these snapshots as ready
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_fwd_t<bf16, 64>(s, chunk, p, chunked, stream, before, after, keep_err);
      case 128: return launch_fwd_t<bf16, 128>(s, chunk, p, chunked, stream, before, after, keep_err);
      case 256: return launch_fwd_t<bf16, 256>(s, chunk, p, chunked, stream, before, after, keep_err);
    }
  } else {
    switch (s.d) {
      case 64: return launch_fwd_t<float, 64>(s, chunk, p, chunked, stream, before, after, keep_err);
      case 128: return launch_fwd_t<float, 128>(s, chunk, p, chunked, stream, before, after, keep_err);
      case 256: return launch_fwd_t<float, 256>(s, chunk, p, chunked, stream, before, after, keep_err);
    }
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, bool FAST>
static hipError_t launch_multi_impl(const Shape& s, MultiParams& mp, hipStream_t stream) {
  using C = OutTile<T, D, FAST>;
  const int qblocks = (s.seqlen + C::BM - 1) / C::BM;
  for (int i = 0; i < mp.nprod; ++i) mp.p[i].qblocks = qblocks;
  const int64_t blocks = (int64_t)s.batch * s.heads * qblocks * mp.nprod;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  bool kvr = false;
  for (int i = 0; i < mp.nprod; ++i) kvr = kvr || mp.p[i].k_rev || mp.p[i].v_rev;
  if (kvr)
    hipLaunchKernelGGL((retention_parallel_multi_kernel<T, D, FAST, true>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, mp);
  else
    hipLaunchKernelGGL((retention_parallel_multi_kernel<T, D, FAST, false>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, mp);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_multi_t(const Shape& s, MultiParams& mp, hipStream_t stream) {
  bool fast = true;
  for (int h = 0; h < s.heads; ++h) fast = fast && -(double)s.log2g[h] * OutTile<T, D, true>::BM <= kFastSpanLog2;
  return fast ? launch_multi_impl<T, D, true>(s, mp, stream) : launch_multi_impl<T, D, false>(s, mp, stream);
}

template <typename T, int D, bool FAST>
static hipError_t launch_cmulti_impl(const Shape& s, int chunk, MultiParams& mp, int* ctrl0, int64_t stride,
                                     hipStream_t stream, bool keep_err) {
  using C = OutTile<T, D, FAST>;
  const int bhs = s.batch * s.heads;
  const int nchunks = (s.seqlen + chunk - 1) / chunk;
  const int64_t nctrl = kCtrlHead + (int64_t)bhs * (nchunks + 1) * kFlagsPerChunk;
  if (stride < nctrl) return hipErrorInvalidValue;
  const int64_t all = stride * (mp.nprod - 1) + nctrl;  // every product's block, from the first one's start
  if (all > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(reset_ctrl_kernel, dim3((unsigned)((all + 255) / 256 < 1024 ? (all + 255) / 256 : 1024)),
                     dim3(256), 0, stream, ctrl0, (int)all, keep_err ? 1 : 0);
  const int qblocks = (chunk + C::BM - 1) / C::BM;
  int64_t roles = 0;  // workgroups per (sequence, head, chunk) over the products
  for (int i = 0; i < mp.nprod; ++i) {
    mp.p[i].qblocks = qblocks;
    mp.p[i].xcd_order = bhs % 8 == 0;
    mp.p[i].ctrl = ctrl0;
    mp.p[i].fbase = (int)(stride * i);
    // sroles arrives as 1 (state workgroups) or 0, xfbase as the partner's index
    mp.p[i].sroles = mp.p[i].sroles ? StTile<T, D>::SPLIT : 0;
    if (mp.p[i].xfbase >= 0) mp.p[i].xfbase = (int)(stride * mp.p[i].xfbase);
    roles += mp.p[i].sroles + qblocks;
  }
  const int64_t blocks = (int64_t)nchunks * bhs * roles;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipGetLastError();
  bool kvr = false;
  for (int i = 0; i < mp.nprod; ++i) kvr = kvr || mp.p[i].k_rev || mp.p[i].v_rev;
  if (kvr)
    hipLaunchKernelGGL((retention_chunkwise_multi_kernel<T, D, FAST, true>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, mp);
  else
    hipLaunchKernelGGL((retention_chunkwise_multi_kernel<T, D, FAST, false>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, mp);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_cmulti_t(const Shape& s, int chunk, MultiParams& mp, int* ctrl0, int64_t stride,
                                  hipStream_t stream, bool keep_err) {
  bool fast = true;
  for (int h = 0; h < s.heads; ++h) fast = fast && -(double)s.log2g[h] * chunk <= kFastSpanLog2;
  return fast ? launch_cmulti_impl<T, D, true>(s, chunk, mp, ctrl0, stride, stream, keep_err)
              : launch_cmulti_impl<T, D, false>(s, chunk, mp, ctrl0, stride, stream, keep_err);
}

hipError_t launch_chunkwise_products(const Shape& s, int chunk, int n, const ChunkProduct* pr, int* ctrl,
                                     int64_t ctrl_stride, float eps, hipStream_t stream, bool keep_err) {
  if (n < 1 || n > kMaxProducts || chunk < 1 || !ctrl) return hipErrorInvalidValue;
  // Products without state workgroups: snapshots from an earlier launch, or
  // from exactly one earlier product of this one (every wait then stays on
  // an earlier ticket); no chain, no final state.
  int writer[kMaxProducts] = {-1, -1, -1};
  for (int i = 0; i < n; ++i) {
    const int x = pr[i].xprod;
    if (x < 0) continue;
    if (x <= i || x >= n || !pr[i].state_wgs || pr[x].state_wgs || pr[x].snap_ready || writer[x] >= 0)
      return hipErrorInvalidValue;
    writer[x] = i;
  }
  for (int i = 0; i < n; ++i)
    if (pr[i].state_wgs ? pr[i].snap_ready
                        : pr[i].state_out || pr[i].state_in || pr[i].snap_ready == (writer[i] >= 0))
      return hipErrorInvalidValue;
  MultiParams mp;
  mp.nprod = n;
  for (int i = 0; i < kMaxProducts; ++i) {
    const ChunkProduct& x = pr[i < n ? i : 0];
    mp.p[i] = make_params(s, chunk, x.q, x.k, x.v, nullptr, x.o, x.state_in, x.state_out, x.snap, x.chain, ctrl,
                          nullptr, eps, x.q_rev, x.out_rev, x.out_rot, nullptr, 0, nullptr);
    mp.p[i].k_rev = x.k_rev;
    mp.p[i].v_rev = x.v_rev;
    mp.p[i].has_state0 = x.state_in != nullptr || x.cross0;
    mp.p[i].sroles = x.state_wgs ? 1 : 0;  // the state split is set per instantiation
    mp.p[i].snap_ready = x.snap_ready;
    mp.p[i].xsnap = x.xprod >= 0 ? pr[x.xprod].snap : nullptr;
    mp.p[i].xfbase = x.xprod;  // the partner's index until its flags' offset is known
  }
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_cmulti_t<bf16, 64>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
      case 128: return launch_cmulti_t<bf16, 128>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
      case 256: return launch_cmulti_t<bf16, 256>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
    }
  } else {
    switch (s.d) {
      case 64: return launch_cmulti_t<float, 64>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
      case 128: return launch_cmulti_t<float, 128>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
      case 256: return launch_cmulti_t<float, 256>(s, chunk, mp, ctrl, ctrl_stride, stream, keep_err);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_parallel_products(const Shape& s, int n, const ParallelProduct* pr, float eps,
                                    hipStream_t stream) {
  if (n < 1 || n > kMaxProducts) return hipErrorInvalidValue;
  MultiParams mp;
  mp.nprod = n;
  for (int i = 0; i < kMaxProducts; ++i) {
    const ParallelProduct& x = pr[i < n ? i : 0];
    mp.p[i] = make_params(s, s.seqlen, x.q, x.k, x.v, nullptr, x.o, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, eps, x.q_rev, x.out_rev, x.out_rot, nullptr, 0, nullptr);
    mp.p[i].k_rev = x.k_rev;
    mp.p[i].v_rev = x.v_rev;
  }
  if (s.dtype == 1) {
    switch (s.d) {
      case 64: return launch_multi_t<bf16, 64>(s, mp, stream);
      case 128: return launch_multi_t<bf16, 128>(s, mp, stream);
      case 256: return launch_multi_t<bf16, 256>(s, mp, stream);
    }
  } else {
    switch (s.d) {
      case 64: return launch_multi_t<float, 64>(s, mp, stream);
      case 128: return launch_multi_t<float, 128>(s, mp, stream);
      case 256: return launch_multi_t<float, 256>(s, mp, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ret
