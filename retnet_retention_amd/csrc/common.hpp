// Device helpers shared by the retention kernels (gfx950 / CDNA4 only).
//
// Matrix-core convention used everywhere (checked on gfx950 hardware):
//   one 16x16 output block, contraction step of 32 ("k-step"):
//   lane l, g = l/16, c = l%16
//     A fragment: A[c][k0 + 8g + j]   j = 0..7
//     B fragment: B[k0 + 8g + j][c]
//     C/D accum:  C[4g + i][c]        i = 0..3
//   bf16 runs one v_mfma_f32_16x16x32_bf16; fp32 runs eight
//   v_mfma_f32_16x16x4_f32, instruction s feeding logical k = 8g + s, which
//   keeps the per-lane data layout identical for both element types.
//
// A contraction is blind to the order of its k index as long as A and B use
// the same order. Fragments whose k runs down a column of a row-major LDS
// tile ("column fragments") use the order
//   j = 0..3 -> row k0 + 4g + j,   j = 4..7 -> row k0 + 16 + 4g + (j - 4)
// which is exactly the row order of two stacked 16x16 accumulator blocks, so
// an accumulator tile can feed the next contraction straight from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ret {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = 128;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), inlined
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { using type = bf16x8; };
template <> struct FragOf<float> { using type = f32x8; };
template <typename T> using frag_t = typename FragOf<T>::type;

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// 32x32 tiles, contraction step 16 (checked on gfx950 hardware):
//   lane l, n = l % 32, h = l / 32
//     A fragment: A[n][k0 + 8h + j]   j = 0..7
//     B fragment: B[k0 + 8h + j][n]
//     C/D accum:  C[8(i/4) + 4h + (i%4)][n]   i = 0..15
//   bf16 runs one v_mfma_f32_32x32x16_bf16, which issues at the full matrix
//   rate from a single wave (the 16x16x32 form does not); fp32 runs eight
//   v_mfma_f32_32x32x2_f32, instruction j pairing element j of both halves.
// Column fragments (k down a column of a row-major tile) use the key order
//   j = 0..3 -> row k0 + 4h + j,   j = 4..7 -> row k0 + 8 + 4h + (j - 4)
// which is the row order of accumulator elements 0..7 (and, 16 rows on,
// 8..15): a 32x32 accumulator feeds the next contraction as two fragments
// without leaving its lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
// accumulator elements 8 sl .. 8 sl + 7 as a fragment (rows 16 sl .. 16 sl + 15
// in the column-fragment order)
template <int SL>
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& c, bf16*) {
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (bf16)c[8 * SL + j];
  return f;
}
template <int SL>
__device__ __forceinline__ f32x8 acc_frag(const f32x16& c, float*) {
  f32x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = c[8 * SL + j];
  return f;
}

// ---------------------------------------------------------------------------
// 8-element vectors in registers, as fp32, loaded from / stored to T memory.
// ---------------------------------------------------------------------------
struct F8 { float x[8]; };

__device__ __forceinline__ F8 load8(const bf16* p) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  F8 r;
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.x[2 * i] = __uint_as_float(u[i] << 16);
    r.x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ F8 load8(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  return F8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}

// 16 bytes of T (8 bf16 or 4 fp32 elements) to and from floats
__device__ __forceinline__ void load16f(const bf16* p, float* v) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}
__device__ __forceinline__ void load16f(const float* p, float* v) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = x[i];
}
__device__ __forceinline__ void store16f(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store16f(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void store8(bf16* p, const F8& v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v.x[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}

__device__ __forceinline__ void store8(float* p, const F8& v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v.x[0], v.x[1], v.x[2], v.x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v.x[4], v.x[5], v.x[6], v.x[7]);
}

// Four consecutive elements (8 bytes of bf16, 16 of fp32) to and from floats.
// Bare workgroup barrier: no wait of any kind is attached (a fence would
// also wait for the direct loads still in flight into other LDS buffers).
// The caller waits for what the barrier must cover (s_waitcnt); the memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// a wave-uniform int held in a scalar register
__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Rows of sequence b in a packed (varlen) tensor whose sequence boundaries
// are cu[0..batch]: first row tok0 and length len, clamped into the tensor's
// `total` rows and to at most `maxlen` tokens. b must be wave-uniform; the
// results are. Returns false when a clamp changed the boundaries (the caller
// reports it), so every access stays inside the tensor for any cu.
__device__ __forceinline__ bool clamp_span(int a, int e, int total, int maxlen, int& tok0, int& len) {
  const int a2 = min(max(a, 0), total);
  const int e2 = min(max(e, a2), total);
  tok0 = a2;
  len = min(e2 - a2, maxlen);
  return a2 == a && e2 == e && e2 - a2 <= maxlen;
}
__device__ __forceinline__ bool packed_span(const int* cu, int b, int total, int maxlen, int& tok0, int& len) {
  return clamp_span(uniform_i(cu[b]), uniform_i(cu[b + 1]), total, maxlen, tok0, len);
}

// a wave-uniform float held in a scalar register
__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// four consecutive elements, raw
template <typename T> struct Vec4Of;
template <> struct Vec4Of<bf16> { using type = bf16x4; };
template <> struct Vec4Of<float> { using type = f32x4; };
template <typename T> using vec4_t = typename Vec4Of<T>::type;

__device__ __forceinline__ void load4(const bf16* p, float* v) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = x[e];
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (bf16)v[e];
  *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void store8_zero(bf16* p) { *reinterpret_cast<uint4*>(p) = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void store8_zero(float* p) {
  reinterpret_cast<float4*>(p)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
  reinterpret_cast<float4*>(p)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// raw 8-element copy (no conversion)
__device__ __forceinline__ void copy8(bf16* dst, const bf16* src) {
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void copy8(float* dst, const float* src) {
  reinterpret_cast<float4*>(dst)[0] = reinterpret_cast<const float4*>(src)[0];
  reinterpret_cast<float4*>(dst)[1] = reinterpret_cast<const float4*>(src)[1];
}

// Raw 8-element chunk as loaded (no conversion), so that a batch of global
// loads can be issued back to back before any of them is consumed.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { u32x4 w; };
template <> struct Raw8<float> { f32x4 a, b; };

__device__ __forceinline__ Raw8<bf16> ld_raw8(const bf16* p) { return Raw8<bf16>{*reinterpret_cast<const u32x4*>(p)}; }
__device__ __forceinline__ Raw8<float> ld_raw8(const float* p) {
  return Raw8<float>{reinterpret_cast<const f32x4*>(p)[0], reinterpret_cast<const f32x4*>(p)[1]};
}
// store, or zeros when !keep (a select: no branch around the store)
__device__ __forceinline__ void st_raw8(bf16* p, const Raw8<bf16>& r, bool keep) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(p) = keep ? r.w : z;
}
__device__ __forceinline__ void st_raw8(float* p, const Raw8<float>& r, bool keep) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  reinterpret_cast<f32x4*>(p)[0] = keep ? r.a : z;
  reinterpret_cast<f32x4*>(p)[1] = keep ? r.b : z;
}
__device__ __forceinline__ F8 unpack8(const Raw8<bf16>& r) {
  F8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.x[2 * i] = __uint_as_float(r.w[i] << 16);
    o.x[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
  }
  return o;
}
__device__ __forceinline__ F8 unpack8(const Raw8<float>& r) {
  return F8{{r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3]}};
}
__device__ __forceinline__ void zero_unless(F8& v, bool keep) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v.x[i] = keep ? v.x[i] : 0.f;
}

// (cos, sin) of 4 consecutive pairs, as two 16-byte loads
// N consecutive elements (N/2 adjacent pairs) turned back by the angles at
// cs[0 .. N/2): (x c + y s, -x s + y c), the transpose of the rotation
template <int N>
__device__ __forceinline__ void unrotate_pairs(float* v, const float2* cs) {
#pragma unroll
  for (int j = 0; j < N / 2; j += 2) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(cs + j);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float c = t[2 * u], s = t[2 * u + 1];
      const float e = v[2 * (j + u)], o = v[2 * (j + u) + 1];
      v[2 * (j + u)] = e * c + o * s;
      v[2 * (j + u) + 1] = -e * s + o * c;
    }
  }
}

struct CS4 { f32x4 a, b; };
__device__ __forceinline__ CS4 ld_cs4(const float2* p) {
  return CS4{reinterpret_cast<const f32x4*>(p)[0], reinterpret_cast<const f32x4*>(p)[1]};
}
__device__ __forceinline__ void rotate4(F8& v, const CS4& t) {
  const float c[4] = {t.a[0], t.a[2], t.b[0], t.b[2]};
  const float s[4] = {t.a[1], t.a[3], t.b[1], t.b[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e = v.x[2 * j], o = v.x[2 * j + 1];
    v.x[2 * j] = e * c[j] - o * s[j];
    v.x[2 * j + 1] = e * s[j] + o * c[j];
  }
}

// Rotate 4 adjacent pairs (x[2j], x[2j+1]) by the angles whose (cos, sin) are cs[0..3].
__device__ __forceinline__ void rotate4(F8& v, const float2* cs) {
  const float4 a = reinterpret_cast<const float4*>(cs)[0];
  const float4 b = reinterpret_cast<const float4*>(cs)[1];
  const float c[4] = {a.x, a.z, b.x, b.z};
  const float s[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e = v.x[2 * j], o = v.x[2 * j + 1];
    v.x[2 * j] = e * c[j] - o * s[j];
    v.x[2 * j + 1] = e * s[j] + o * c[j];
  }
}

__device__ __forceinline__ bf16x8 to_frag(const F8& v, bf16*) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v.x[i];
  return o;
}
__device__ __forceinline__ f32x8 to_frag(const F8& v, float*) {
  f32x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = v.x[i];
  return o;
}

template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() {
  frag_t<T> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (T)0.f;
  return f;
}

// ---------------------------------------------------------------------------
// LDS fragment loads.
// ---------------------------------------------------------------------------
// Row fragment: 8 consecutive elements of one row (k contiguous).
__device__ __forceinline__ bf16x8 lds_row8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 lds_row8(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Column fragment of a row-major tile whose element [k0][n0] is at `base`
// (row stride `stride` elements): lane (g, i) receives rows
// k0 + {4g..4g+3, 16+4g..16+4g+3} of column n0 + i.
// bf16 uses the gfx950 transpose read ds_read_b64_tr_b16: inside each group of
// 16 lanes, lane m fetches 4 elements of row (m/4) at column 4(m%4), and lane
// i ends up with column i of those four rows.
__device__ __forceinline__ bf16x8 lds_col8(const bf16* base, int stride, int lane) {
  const int g = (lane >> 4) & 3, i = lane & 15;
  const bf16* p = base + (4 * g + (i >> 2)) * stride + 4 * (i & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * stride));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ f32x8 lds_col8(const float* base, int stride, int lane) {
  const int g = (lane >> 4) & 3, i = lane & 15;
  const float* p = base + 4 * g * stride + i;
  f32x8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = p[j * stride];
    f[4 + j] = p[(16 + j) * stride];
  }
  return f;
}

// Two stacked 16x16 accumulator blocks (rows k0..k0+15 and k0+16..k0+31 of a
// 32-deep contraction) become one A fragment in the column-fragment k order.
__device__ __forceinline__ bf16x8 acc_to_frag(const f32x4& lo, const f32x4& hi, bf16*) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = (bf16)lo[i];
    o[4 + i] = (bf16)hi[i];
  }
  return o;
}
__device__ __forceinline__ f32x8 acc_to_frag(const f32x4& lo, const f32x4& hi, float*) {
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Multiply element j of a fragment by z[j] (bf16 fragments round back).
__device__ __forceinline__ void scale_frag(bf16x8& f, const float* z) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)((float)f[i] * z[i]);
}
__device__ __forceinline__ void scale_frag(f32x8& f, const float* z) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] *= z[i];
}
// Multiply every element of a fragment by x (bf16 fragments round back).
__device__ __forceinline__ void scale_frag(bf16x8& f, float x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)((float)f[i] * x);
}
__device__ __forceinline__ void scale_frag(f32x8& f, float x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] *= x;
}
// One half (H = 0: rows k0..k0+15, H = 1: k0+16..k0+31) of such a fragment.
template <int H>
__device__ __forceinline__ void set_half(bf16x8& f, const f32x4& x, std::integral_constant<int, H>) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[4 * H + i] = (bf16)x[i];
}
template <int H>
__device__ __forceinline__ void set_half(f32x8& f, const f32x4& x, std::integral_constant<int, H>) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[4 * H + i] = x[i];
}

// ---------------------------------------------------------------------------
// LDS tiles filled by direct global->LDS loads.
//
// global_load_lds_dwordx4 / buffer_load ... lds write lane i's 16 bytes to
// LDS base + 16 i (M0 holds the base): one wave-wide load fills 1 KiB of
// consecutive LDS. A tile of ROWS rows of COLS elements (row bytes ROWB a
// power of two, 128 .. 1024) is stored load by load: load n holds rows
// n RPI .. n RPI + RPI-1 (RPI = 1024 / ROWB) at LDS offset n (1024 + PADL),
// and inside it the rows' 16-byte chunks are interleaved in groups of G:
// chunk c of row lr sits at chunk position (c / G) G RPI + lr G + c % G.
// A lane's global offset is then the same for every load up to a
// wave-uniform row step, a fragment read is a per-lane base plus an
// immediate offset (the constant part of its chunk index being a multiple of
// G), and G and PADL put the reads of one instruction in distinct banks (64
// banks of 4 bytes):
//   row tiles (16 lanes read one chunk of 16 consecutive rows);
//   column tiles (transposed reads: 32 lanes read 4 chunks of 4 aligned rows).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

enum TileKind { kRowTile, kColTile };

template <typename T, int ROWS, int COLS, TileKind KIND>
struct LTile {
  static constexpr int ROWB = COLS * (int)sizeof(T);  // row bytes
  static constexpr int CPR = ROWB / 16;               // chunks per row
  static constexpr int RPI = 1024 / ROWB;             // rows per wave-wide load
  static_assert(ROWB >= 128 && ROWB <= 1024 && (ROWB & (ROWB - 1)) == 0, "power-of-two rows of 128..1024 bytes");
  static_assert(ROWS % RPI == 0, "whole loads");
  // (G, PADL) by row bytes 128 / 256 / 512 / 1024
  static constexpr int G = KIND == kRowTile ? (ROWB == 128 ? 2 : 1) : (ROWB == 128 ? 4 : 1);
  static constexpr int PADL = KIND == kRowTile ? (ROWB == 128 ? 16 : ROWB == 256 ? 64 : ROWB == 512 ? 32 : 16)
                                               : (ROWB <= 256 ? 0 : ROWB == 512 ? 128 : 64);
  static constexpr int LSTRIDE = 1024 + PADL;  // LDS bytes per load
  static constexpr int NINST = ROWS / RPI;     // wave-wide loads
  static constexpr int BYTES = NINST * LSTRIDE;
  __device__ static __forceinline__ int off(int r, int col) {
    const int byte = col * (int)sizeof(T), c = byte >> 4;
    return (r / RPI) * LSTRIDE + (((c / G) * G * RPI + (r % RPI) * G + c % G) << 4) + (byte & 15);
  }
  // byte step of DR rows (a multiple of RPI): the same chunk positions
  static constexpr int row_step(int dr) { return (dr / RPI) * LSTRIDE; }
};

// Direct loads of tile TL spread over NW waves (wave w issues loads w, w+NW,
// ...). The lane's offset is worked out once: loads of rows that all exist
// take it plus a scalar row step, as buffer loads from a scalar descriptor
// (no vector arithmetic per load); loads of a tile with rows past rmax clamp
// each lane's row. Completion: s_waitcnt vmcnt + barrier.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer descriptor, gfx9 family

// buffer descriptor of a wave-uniform base address, in scalar registers;
// accesses at byte offsets from `bytes` on are dropped (stores) or read as
// zero (loads) by the hardware
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const void* base, uint32_t bytes = 0xffffffffu) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kBufferWord3);
}

// 16 loaded bytes of T (8 bf16 or 4 fp32 elements) to floats, and floats
// to 16 bytes of T stored through a buffer descriptor
typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load16f_raw(u32x4b w, float* v, bf16*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load16f_raw(u32x4b w, float* v, float*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ void store16f_raw(__amdgpu_buffer_rsrc_t rs, uint32_t off, const float* v, bf16*) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4b, o), rs, off, 0, 0);
}
__device__ __forceinline__ void store16f_raw(__amdgpu_buffer_rsrc_t rs, uint32_t off, const float* v, float*) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4b{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                __float_as_uint(v[3])},
                                         rs, off, 0, 0);
}

template <typename T, typename TL, int NW>
struct TileLoads {
  static constexpr int PER = (TL::NINST + NW - 1) / NW;
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  uint32_t off;  // byte offset of this lane's chunk from the load's first row
  // chunk position `lane` of a load: row (lane / G) % RPI, chunk
  // (lane / (G RPI)) G + lane % G
  __device__ static __forceinline__ int lane_row(int lane) { return (lane / TL::G) % TL::RPI; }
  __device__ static __forceinline__ int lane_chunk(int lane) {
    return (lane / (TL::G * TL::RPI)) * TL::G + lane % TL::G;
  }
  __device__ __forceinline__ void init(int64_t gstride, int lane) {
    off = (uint32_t)((lane_row(lane) * (int)gstride + lane_chunk(lane) * EPC) * (int)sizeof(T));
  }
  // For the reversed loads below: a load's rows run downwards in g.
  __device__ __forceinline__ void init_rev(int64_t gstride, int lane) {
    off = (uint32_t)(((TL::RPI - 1 - lane_row(lane)) * (int)gstride + lane_chunk(lane) * EPC) * (int)sizeof(T));
  }
  // Reversed token order (after init_rev): tile row r holds row
  // len - 1 - (row0 + r) of g, for rows row0 .. row0 + ROWS - 1 all below len
  // (the lowest row of g read, len - row0 - ROWS, is wave-uniform: the
  // descriptor's base; load n starts NINST - 1 - n loads above it).
  __device__ __forceinline__ void issue_rev(char* lds, const T* g, int64_t gstride, int len, int row0,
                                            int wave) const {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(g + (int64_t)(len - row0 - TL::NINST * TL::RPI) * gstride);
    const uint32_t step = (uint32_t)(TL::RPI * gstride * (int64_t)sizeof(T));
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int n = wave + m * NW;
      if (TL::NINST % NW != 0 && m == PER - 1 && n >= TL::NINST) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + n * TL::LSTRIDE), 16, off,
                                               (TL::NINST - 1 - n) * step, 0, 0);
    }
  }
  // The same with every row past rmax (rmax >= row0, below len) replaced by
  // row rmax: tile row r holds row len - 1 - min(row0 + r, rmax).
  __device__ __forceinline__ void issue_clamped_rev(char* lds, const T* g, int64_t gstride, int len, int row0,
                                                    int rmax, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(g + (int64_t)(len - 1 - rmax) * gstride);
    const int lane = threadIdx.x & 63, lr = lane_row(lane), lc = lane_chunk(lane);
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int n = wave + m * NW;
      if (TL::NINST % NW != 0 && m == PER - 1 && n >= TL::NINST) break;
      const int r = min(n * TL::RPI + lr, rmax - row0);  // row relative to row0
      const uint32_t o = (uint32_t)(((rmax - row0 - r) * (int)gstride + lc * EPC) * (int)sizeof(T));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + n * TL::LSTRIDE), 16, o, 0, 0, 0);
    }
  }
  // rows row0 .. row0 + ROWS - 1 of g, all in range (g + row0 gstride is
  // wave-uniform)
  __device__ __forceinline__ void issue(char* lds, const T* g, int64_t gstride, int row0, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(g + row0 * gstride);
    const uint32_t step = (uint32_t)(TL::RPI * gstride * (int64_t)sizeof(T));  // bytes per load
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int n = wave + m * NW;  // wave-uniform; below NINST except maybe in the last load
      if (TL::NINST % NW != 0 && m == PER - 1 && n >= TL::NINST) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + n * TL::LSTRIDE), 16, off, n * step, 0, 0);
    }
  }
  // rows row0 .. row0 + ROWS - 1 of g with every row past rmax replaced by
  // row rmax (rmax >= row0)
  __device__ __forceinline__ void issue_clamped(char* lds, const T* g, int64_t gstride, int row0, int rmax,
                                                int wave) const {
    const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(g + row0 * gstride);
    const int lane = threadIdx.x & 63, lr = lane_row(lane), lc = lane_chunk(lane);
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int n = wave + m * NW;
      if (TL::NINST % NW != 0 && m == PER - 1 && n >= TL::NINST) break;
      const int r = min(n * TL::RPI + lr, rmax - row0);  // row relative to row0
      const uint32_t o = (uint32_t)((r * (int)gstride + lc * EPC) * (int)sizeof(T));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + n * TL::LSTRIDE), 16, o, 0, 0, 0);
    }
  }
};

// A contiguous block of BYTES (a multiple of 1 KiB) copied into LDS by NW
// waves, one 16-byte chunk per lane and load (g wave-uniform). CPOL: cache
// policy (0: default; 17 = sc0|sc1: read coherently data that another XCD
// wrote with sc1 stores).
template <typename T, int BYTES, int NW, int CPOL = 0>
__device__ __forceinline__ void async_flat(char* lds, const T* g, int wave, int lane) {
  static_assert(BYTES % 1024 == 0, "whole wave-wide loads");
  constexpr int NINST = BYTES / 1024;
  const __amdgpu_buffer_rsrc_t rs = scalar_rsrc(g);
#pragma unroll
  for (int m = 0; m < (NINST + NW - 1) / NW; ++m) {
    const int n = wave + m * NW;  // wave-uniform
    if (NINST % NW != 0 && n >= NINST) break;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + n * 1024), 16, (uint32_t)lane * 16u,
                                             (uint32_t)n * 1024u, 0, CPOL);
  }
}

// Row fragment: elements (r, col .. col+7).
template <typename TL>
__device__ __forceinline__ bf16x8 tile_row8(const char* t, int r, int col, bf16*) {
  return *reinterpret_cast<const bf16x8*>(t + TL::off(r, col));
}
template <typename TL>
__device__ __forceinline__ f32x8 tile_row8(const char* t, int r, int col, float*) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(t + TL::off(r, col));
  const f32x4 b = *reinterpret_cast<const f32x4*>(t + TL::off(r, col + 4));
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Column fragment for 32x32 tiles: lane (n = l%32, h = l/32) receives rows
// k0 + {4h..4h+3, 8+4h..8+4h+3} of column n0 + n (k0 a multiple of 16). bf16:
// per 16-lane group (h = group/2, 16 columns from n0 + 16 (group%2)) lane m
// fetches 4 elements of row k0 + 4h + m/4 at column 4(m%4), and the transpose
// read hands lane m column m of those four rows; a second read 8 rows on
// gives the rest.
template <typename TL>
__device__ __forceinline__ bf16x8 tile_col8w(const char* t, int k0, int n0, int lane, bf16*) {
  const int grp = lane >> 4, m = lane & 15, h = grp >> 1;
  const char* p = t + TL::off(k0 + 4 * h + (m >> 2), n0 + 16 * (grp & 1) + 4 * (m & 3));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + TL::row_step(8)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}
template <typename TL>
__device__ __forceinline__ f32x8 tile_col8w(const char* t, int k0, int n0, int lane, float*) {
  const int n = lane & 31, h = lane >> 5;
  f32x8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = *reinterpret_cast<const float*>(t + TL::off(k0 + 4 * h + j, n0 + n));
    f[4 + j] = *reinterpret_cast<const float*>(t + TL::off(k0 + 8 + 4 * h + j, n0 + n));
  }
  return f;
}

// ---------------------------------------------------------------------------
// Reductions.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes that share g (lanes 16g .. 16g+15): butterflies
// within the row of 16 lanes (quad xor 1, quad xor 2, mirror in 8, mirror in
// 16); every lane ends with the full sum.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Sum over each group of N consecutive lanes (N = 2 .. 64, a power of two),
// in every lane of the group: the butterflies of sum16 up to N, then lane
// exchanges across 16-lane rows.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "power-of-two lane group");
  x += dpp<0xB1>(x);
  if constexpr (N >= 4) x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Sum of the two lanes l and l ^ 32.
__device__ __forceinline__ float sum_pair32(float x) { return x + __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float sum64(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// swish(x) = x * sigmoid(x) with the hardware exp2 and reciprocal (about 1 ulp
// each): exp2(-x log2 e) saturates to +inf for very negative x, giving -0.
__device__ __forceinline__ float swish(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// g^e for a decay g given as log2(g): exp2(e * log2 g).
// The hardware exp2 flushes results below the normal range to zero, which is
// the right answer for a decay factor that small.
__device__ __forceinline__ float gpow(float e, float log2g) { return __builtin_amdgcn_exp2f(e * log2g); }

}  // namespace ret
