// C-ABI host layer: argument validation (before any HIP call), per-head decay
// table, workspace carving and kernel launches on the caller's stream.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "retention.h"

namespace {

using ret::Shape;

constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t elem_size(int32_t dtype) { return dtype == RET_BF16 ? 2 : 4; }

// Decay of head h: the caller's value, or g_h = 1 - 2^(-5-h) (per-head decay
// of "Retentive Network: A Successor to Transformer...", Elamur summary,
// Key points, fifth item).
double head_gamma(const ret_desc_t* d, int h) { return d->gamma ? d->gamma[h] : 1.0 - std::ldexp(1.0, -5 - h); }

ret_status_t check_desc(const ret_desc_t* d) {
  if (!d) return RET_ERR_NULL;
  if (d->batch < 1 || d->seqlen < 1 || d->heads < 1 || d->heads > ret::kMaxHeadsHost) return RET_ERR_SHAPE;
  // every launch grid is bounded by batch * heads * seqlen workgroups; the
  // product is formed in two steps so that it cannot overflow int64 itself
  const int64_t bh = (int64_t)d->batch * d->heads;
  if (bh > INT32_MAX || bh * d->seqlen > INT32_MAX) return RET_ERR_SHAPE;
  // kernels address within one sequence with 32-bit element offsets
  if ((int64_t)d->seqlen * d->heads * (d->dk > d->dv ? d->dk : d->dv) >= INT32_MAX) return RET_ERR_SHAPE;
  if (d->dtype != RET_F32 && d->dtype != RET_BF16) return RET_ERR_UNSUPPORTED;
  if (d->dk != d->dv || (d->dk != 64 && d->dk != 128 && d->dk != 256)) return RET_ERR_UNSUPPORTED;
  if (d->gamma) {
    for (int h = 0; h < d->heads; ++h) {
      const double g = d->gamma[h];
      if (!(std::isfinite(g) && g > 0.0 && g <= 1.0)) return RET_ERR_GAMMA;
    }
  }
  if (!(std::isfinite(d->rotary_base) && d->rotary_base >= 0.0)) return RET_ERR_ARG;
  if (d->pos_offset < 0 || d->pos_offset > (int64_t(1) << 52)) return RET_ERR_ARG;
  return RET_OK;
}

ret_status_t check_eps(const ret_desc_t* d, const void* g) {
  if (g && !(std::isfinite(d->gn_eps) && d->gn_eps > 0.0f)) return RET_ERR_ARG;
  return RET_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// bytes of one [batch][seqlen][heads][d] tensor and of one fp32 state
size_t tensor_bytes(const ret_desc_t* d) {
  return (size_t)d->batch * d->seqlen * d->heads * d->dk * elem_size(d->dtype);
}
size_t state_bytes_exact(const ret_desc_t* d) { return (size_t)d->batch * d->heads * d->dk * d->dv * 4; }

// the decode step's state (read and written in place) overlaps none of q, k,
// v, g, o
ret_status_t check_step_state(const ret_desc_t* d, const void* q, const void* k, const void* v, const void* g,
                              const void* o, const float* state) {
  const size_t n = tensor_bytes(d), ns = state_bytes_exact(d);
  if (overlaps(state, ns, q, n) || overlaps(state, ns, k, n) || overlaps(state, ns, v, n) ||
      overlaps(state, ns, g, n) || overlaps(state, ns, o, n))
    return RET_ERR_ALIAS;
  return RET_OK;
}

ret_status_t check_tensors(const ret_desc_t* d, const void* q, const void* k, const void* v, const void* g,
                           const void* o) {
  if (!q || !k || !v || !o) return RET_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (g && !aligned16(g)))
    return RET_ERR_ALIGN;
  const size_t n = (size_t)d->batch * d->seqlen * d->heads * d->dk * elem_size(d->dtype);
  if (overlaps(o, n, q, n) || overlaps(o, n, k, n) || overlaps(o, n, v, n) || overlaps(o, n, g, n))
    return RET_ERR_ALIAS;
  return RET_OK;
}

Shape make_shape(const ret_desc_t* d) {
  Shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = d->batch;
  s.seqlen = d->seqlen;
  s.heads = d->heads;
  s.d = d->dk;
  s.dtype = d->dtype;
  for (int h = 0; h < d->heads; ++h) {
    const double g = head_gamma(d, h);
    s.log2g[h] = (float)(std::log1p(g - 1.0) / std::log(2.0));
    s.gam[h] = (float)g;
  }
  return s;
}

// Rotation needs the angle table and a rotated copy of k.
size_t rot_bytes(const ret_desc_t* d) {
  if (d->rotary_base == 0.0) return 0;
  const size_t kb = (size_t)d->batch * d->seqlen * d->heads * d->dk * elem_size(d->dtype);
  return align_up((size_t)d->seqlen * (d->dk / 2) * sizeof(float2)) + align_up(kb);
}

// Launch the table and key rotation passes when rotation is on: k is replaced
// by its rotated copy in the workspace and *table is set for the retention
// kernel, which turns q as it loads it (null when rotation is off).
// Packed sequences (cu set): k holds `total` rows, sequence b the rows
// cu[b] .. cu[b+1]-1, each token turned by its position in its sequence.
bool rotate_inputs(const ret_desc_t* d, const void*& k, const float2** table, void* workspace, hipStream_t stream,
                   const int32_t* cu = nullptr, int total = 0) {
  *table = nullptr;
  if (d->rotary_base == 0.0) return true;
  char* ws = static_cast<char*>(workspace);
  float2* tab = reinterpret_cast<float2*>(ws);
  char* kr = ws + align_up((size_t)d->seqlen * (d->dk / 2) * sizeof(float2));
  if (cu) {
    if (ret::launch_rotary_table(tab, d->seqlen, d->dk, d->rotary_base, d->pos_offset, stream) != hipSuccess ||
        ret::launch_rotate_keys_packed(k, kr, tab, cu, d->batch, total, d->seqlen, d->heads, d->dk, d->dtype,
                                       stream) != hipSuccess)
      return false;
  } else if (ret::launch_rotate_keys_table(k, kr, tab, d->batch, d->seqlen, d->heads, d->dk, d->dtype,
                                           d->rotary_base, d->pos_offset, stream) != hipSuccess) {
    return false;
  }
  k = kr;
  *table = tab;
  return true;
}

int32_t eff_chunk(const ret_desc_t* d, int32_t chunk) { return chunk < d->seqlen ? chunk : d->seqlen; }

size_t nchunks_of(const ret_desc_t* d, int32_t chunk) {
  const int32_t c = eff_chunk(d, chunk);
  return ((size_t)d->seqlen + c - 1) / c;
}

// Chunkwise workspace: control block | rotation (optional) | fp32 state chain
// (two slots per sequence and head) | per-chunk states R_{i-1}^T.
size_t ctrl_bytes(const ret_desc_t* d, int32_t chunk) {
  return align_up(ret::chunkwise_ctrl_bytes(d->batch, d->heads, (int)nchunks_of(d, chunk)));
}
size_t chain_bytes(const ret_desc_t* d) { return align_up((size_t)d->batch * d->heads * 2 * d->dk * d->dv * 4); }
size_t snap_bytes(const ret_desc_t* d, int32_t chunk) {
  return align_up((size_t)d->batch * d->heads * nchunks_of(d, chunk) * d->dk * d->dv * elem_size(d->dtype));
}


// Backward of the parallel form. Workspace slots, each one tensor
// [batch][seqlen][heads][d] rounded up to 256 bytes: the angle table and the
// rotated q', k' and reversed q' with rotation (none without: the products
// read q reversed); with a gate the reversed dO, written by the recomputed
// forward's epilogue (none without: the products read dout reversed).
size_t bwd_tensor_bytes(const ret_desc_t* d) {
  return align_up((size_t)d->batch * d->seqlen * d->heads * d->dk * elem_size(d->dtype));
}
size_t bwd_table_bytes(const ret_desc_t* d) {
  return d->rotary_base == 0.0 ? 0 : align_up((size_t)d->seqlen * (d->dk / 2) * sizeof(float2));
}
size_t bwd_bytes(const ret_desc_t* d, bool gate) {
  const int slots = (d->rotary_base == 0.0 ? 0 : 3) + (gate ? 1 : 0);
  return bwd_table_bytes(d) + slots * bwd_tensor_bytes(d);
}


// Backward of the chunkwise form: the chunkwise kernel's own workspace for
// each of the three gradient products, which run in one launch (three
// control blocks, then three state chains, then three sets of per-chunk
// states; the recomputed forward uses the first chain and the third set),
// the parallel backward's table and tensor slots, then with a carried state
// three fp32 states (S0^T; dS^T / g for the reversed dk product; its final
// state).
constexpr int kBwdProducts = 3;
size_t state_bytes(const ret_desc_t* d) { return align_up((size_t)d->batch * d->heads * d->dk * d->dv * 4); }
size_t cbwd_bytes(const ret_desc_t* d, int32_t chunk, bool gate, bool states) {
  return kBwdProducts * (ctrl_bytes(d, chunk) + chain_bytes(d) + snap_bytes(d, chunk)) + bwd_bytes(d, gate) +
         (states ? 3 * state_bytes(d) : 0);
}

// Chunkwise forward: every check that does not involve the workspace.
ret_status_t check_chunkwise_args(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                  const void* v, const void* g, const void* o, const float* state_in,
                                  const float* state_out) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (chunk < 1) return RET_ERR_SHAPE;
  if ((st = check_tensors(desc, q, k, v, g, o)) != RET_OK) return st;
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out))) return RET_ERR_ALIGN;
  // the written buffers (o, state_out) overlap nothing else; state_in ==
  // state_out exactly is allowed (the kernel reads every state_in value
  // before the last chunk writes state_out)
  const size_t n = tensor_bytes(desc), ns = state_bytes_exact(desc);
  if (overlaps(o, n, state_in, ns) || overlaps(o, n, state_out, ns)) return RET_ERR_ALIAS;
  if (overlaps(state_out, ns, q, n) || overlaps(state_out, ns, k, n) || overlaps(state_out, ns, v, n) ||
      overlaps(state_out, ns, g, n) || (state_out != state_in && overlaps(state_out, ns, state_in, ns)))
    return RET_ERR_ALIAS;
  return RET_OK;
}

// Workspace bytes of the chunkwise forward: control block | rotation
// (optional) | fp32 state chain | per-chunk states.
size_t chunkwise_bytes(const ret_desc_t* desc, int32_t chunk) {
  return ctrl_bytes(desc, chunk) + rot_bytes(desc) + chain_bytes(desc) + snap_bytes(desc, chunk);
}

// The chunkwise forward's launches over a checked workspace `ws` of at
// least chunkwise_bytes() bytes.
ret_status_t launch_chunkwise(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k, const void* v,
                              const void* g, void* o, const float* state_in, float* state_out, char* ws,
                              hipStream_t stream, hipEvent_t before, hipEvent_t after) {
  const size_t cb = ctrl_bytes(desc, chunk), rb = rot_bytes(desc), hb = chain_bytes(desc);
  const Shape s = make_shape(desc);
  const int32_t c = eff_chunk(desc, chunk);
  int* ctrl = reinterpret_cast<int*>(ws);
  const float2* table;
  if (!rotate_inputs(desc, k, &table, ws + cb, stream)) return RET_ERR_HIP;
  float* chain = reinterpret_cast<float*>(ws + cb + rb);
  void* snap = ws + cb + rb + hb;
  if (ret::launch_retention_fwd(s, c, true, q, k, v, g, o, state_in, state_out, snap, chain, ctrl, table,
                                desc->gn_eps, stream, before, after) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of retention_chunkwise_fwd_noalloc, for callers that cannot
// allocate device memory. Each device the library runs on holds one copy of
// this array for the life of the process. Host code never uses the array's
// name as an address (on the host it names a stand-in, not device memory):
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that pointer is passed on.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until looked up

// The scratch's device address on the device of `stream` (the current device
// for the null stream).
ret_status_t scratch_for(hipStream_t stream, char** out) {
  int dev = 0;
  if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return RET_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RET_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return RET_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return RET_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return RET_ERR_HIP;
    if (e != hipSuccess || !p) return RET_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return RET_OK;
}

ret_status_t chunkwise_bwd_impl(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k, const void* v,
                                const void* g, const void* dout, const float* state_in, const float* d_state_out,
                                void* dq, void* dk, void* dv, void* dg, float* d_state_in, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (chunk < 1) return RET_ERR_SHAPE;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return RET_ERR_NULL;
  if ((g == nullptr) != (dg == nullptr) || (state_in == nullptr) != (d_state_in == nullptr)) return RET_ERR_NULL;
  const void* ins[] = {q, k, v, g, dout, state_in, d_state_out};
  void* outs[] = {dq, dk, dv, dg, d_state_in};
  for (const void* p : ins)
    if (p && !aligned16(p)) return RET_ERR_ALIGN;
  for (const void* p : outs)
    if (p && !aligned16(p)) return RET_ERR_ALIGN;
  const size_t n = (size_t)desc->batch * desc->seqlen * desc->heads * desc->dk * elem_size(desc->dtype);
  const size_t ns = (size_t)desc->batch * desc->heads * desc->dk * desc->dv * 4;
  const size_t in_n[] = {n, n, n, n, n, ns, ns};
  const size_t out_n[] = {n, n, n, n, ns};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return RET_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return RET_ERR_ALIAS;
  }
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  // the dS terms enter the reversed products as state_in = dS / g: keep 1/g
  // within fp32 range
  if (d_state_out)
    for (int h = 0; h < desc->heads; ++h)
      if (head_gamma(desc, h) < std::ldexp(1.0, -60)) return RET_ERR_GAMMA;
  const bool states = state_in || d_state_out;
  const size_t need = cbwd_bytes(desc, chunk, g != nullptr, states);
  if (!workspace || workspace_bytes < need) return RET_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RET_ERR_ALIGN;
  for (int j = 0; j < 7; ++j)
    if (overlaps(workspace, need, ins[j], in_n[j])) return RET_ERR_ALIAS;
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, need, outs[i], out_n[i])) return RET_ERR_ALIAS;

  const Shape s = make_shape(desc);
  const int32_t c = eff_chunk(desc, chunk);
  char* ws = static_cast<char*>(workspace);
  const size_t cb = ctrl_bytes(desc, chunk), hb = chain_bytes(desc), sb = snap_bytes(desc, chunk);
  int* ctrl = reinterpret_cast<int*>(ws);
  auto chain_of = [&](int i) { return reinterpret_cast<float*>(ws + kBwdProducts * cb + i * hb); };
  auto snap_of = [&](int i) { return static_cast<void*>(ws + kBwdProducts * (cb + hb) + i * sb); };
  float* chain = chain_of(0);
  void* snap = snap_of(0);
  char* tab_at = ws + kBwdProducts * (cb + hb + sb);
  const size_t tb = bwd_tensor_bytes(desc);
  char* next = tab_at + bwd_table_bytes(desc);
  auto slot = [&]() { char* p = next; next += tb; return p; };
  char* st_at = tab_at + bwd_bytes(desc, g != nullptr);
  auto state_slot = [&](int i) { return reinterpret_cast<float*>(st_at + i * state_bytes(desc)); };
  // The call's first chunkwise launch clears the control block's error word,
  // the later one keeps it, so the word reports an error of either.
  bool first = true;
  // Initial states of the products (per head g): S0^T for dq, dS^T / g for
  // the reversed dk product (its g^(m'+1) then makes g^(N-1-m)); the reversed
  // dv product's is dS / g, the transpose, and so are all its states: the dk
  // product's state workgroups write its snapshots too. In the same way the
  // dq product's states are the recomputed forward's transposed (with a gate,
  // which recomputes it). The dk product's final state Z gives dS0 = g Z^T.
  float ones[ret::kMaxHeadsHost], inv[ret::kMaxHeadsHost], gam[ret::kMaxHeadsHost];
  for (int h = 0; h < desc->heads; ++h) {
    ones[h] = 1.f;
    inv[h] = (float)(1.0 / head_gamma(desc, h));
    gam[h] = (float)head_gamma(desc, h);
  }
  float *s0t = nullptr, *xs = nullptr, *zs = nullptr;
  if (state_in) {
    zs = state_slot(2);
    if (!g) {
      s0t = state_slot(0);
      if (ret::launch_state_map(s, state_in, s0t, true, ones, stream) != hipSuccess) return RET_ERR_HIP;
    }
  }
  if (d_state_out) {
    xs = state_slot(1);
    if (ret::launch_state_map(s, d_state_out, xs, true, inv, stream) != hipSuccess) return RET_ERR_HIP;
  }
  // q', k' and the reversed q'
  const float2* table = nullptr;
  const void *qr = q, *kr = k;
  void* qrev = nullptr;
  if (desc->rotary_base != 0.0) {
    float2* tab = reinterpret_cast<float2*>(tab_at);
    void* qs = slot();
    void* ks = slot();
    qrev = slot();
    if (ret::launch_rotate_keys_table(q, qs, tab, desc->batch, desc->seqlen, desc->heads, desc->dk, desc->dtype,
                                      desc->rotary_base, desc->pos_offset, stream, qrev) != hipSuccess ||
        ret::launch_rotate_keys(k, ks, tab, desc->batch, desc->seqlen, desc->heads, desc->dk, desc->dtype,
                                stream) != hipSuccess)
      return RET_ERR_HIP;
    table = tab;
    qr = qs;
    kr = ks;
  }
  // without rotation the products read q in reversed order where they need
  // it reversed (no copy)
  // dO and its reversed copy
  const void* dov = dout;
  void* dorev = nullptr;
  if (g) {
    // the recomputed forward forms dg and dO (stored reversed) in its
    // epilogue, from the gate, dout and its output in registers, and writes
    // the dq product's snapshots beside its own (in the third product's
    // area, which that launch then refills); it clears the error word, the
    // products' launch keeps it
    dorev = slot();
    first = false;
    if (ret::launch_retention_fwd(s, c, true, qr, kr, v, g, dorev, state_in, nullptr, snap_of(2), chain, ctrl,
                                  nullptr, desc->gn_eps, stream, nullptr, nullptr, false, true, nullptr, nullptr, 0,
                                  nullptr, false, dout, dg, snap) != hipSuccess)
      return RET_ERR_HIP;
    dov = nullptr;  // the dq product reads the reversed copy back in order
  }
  // without a gate the products read dout in reversed order where they need
  // it reversed (no copy)
  const void* qr_rev = qrev ? qrev : q;      // reversed q': the rotation pass's copy, or q read reversed
  const void* do_rev = dorev ? dorev : dout;  // reversed dO: the recompute's copy, or dout read reversed
  const bool rq = qrev == nullptr, rdo = dorev == nullptr;
  // the parallel backward's three products, each run as the chunkwise form
  // (the same function), storing straight into the caller's tensors, in one
  // launch
  ret::ChunkProduct prods[kBwdProducts] = {
      {dov ? dov : dorev, v, kr, dq, s0t, nullptr, snap_of(0), chain_of(0), dov == nullptr, false, table, false,
       false},
      {v, do_rev, qr_rev, dk, xs, zs, snap_of(1), chain_of(1), true, true, table, rdo, rq},
      {kr, qr_rev, do_rev, dv, nullptr, nullptr, snap_of(2), nullptr, true, true, nullptr, rq, rdo},
  };
  if (g) {  // the dq product's snapshots are the recompute's
    prods[0].state_wgs = false;
    prods[0].snap_ready = true;
    prods[0].cross0 = state_in != nullptr;
    prods[0].chain = nullptr;
  }
  prods[1].xprod = 2;  // the dk product's state workgroups write the dv product's snapshots
  prods[2].state_wgs = false;
  prods[2].cross0 = d_state_out != nullptr;
  const bool keep = !first;  // a recomputed forward before them cleared the error word
  if (ret::launch_chunkwise_products(s, c, kBwdProducts, prods, ctrl, (int64_t)(cb / sizeof(int)), desc->gn_eps,
                                     stream, keep) != hipSuccess)
    return RET_ERR_HIP;
  if (state_in && ret::launch_state_map(s, zs, d_state_in, true, gam, stream) != hipSuccess) return RET_ERR_HIP;
  return RET_OK;
}

}  // namespace

extern "C" {

int32_t retention_abi_version(void) { return 1; }

const char* retention_status_string(ret_status_t s) {
  // a C caller may pass any int: read it as one (a C++ load of an enum
  // outside its enumerators' range is undefined)
  static_assert(sizeof(ret_status_t) == sizeof(int32_t), "ret_status_t is a 32-bit int in the C ABI");
  int32_t code;
  std::memcpy(&code, &s, sizeof(code));
  switch (code) {
    case RET_OK: return "ok";
    case RET_ERR_NULL: return "a required pointer is NULL";
    case RET_ERR_SHAPE: return "batch, seqlen, heads or chunk out of range";
    case RET_ERR_UNSUPPORTED: return "unsupported dk/dv/dtype (need dk == dv in {64,128,256}, fp32 or bf16)";
    case RET_ERR_GAMMA: return "decay outside (0, 1]";
    case RET_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RET_ERR_WORKSPACE: return "workspace NULL or too small";
    case RET_ERR_HIP: return "HIP runtime error at kernel launch";
    case RET_ERR_ALIAS: return "output overlaps an input";
    case RET_ERR_ARG: return "invalid scalar argument (gn_eps, rotary_base or pos_offset)";
    case RET_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds (128 MiB)";
  }
  return "unknown status";
}

size_t retention_parallel_workspace_bytes(const ret_desc_t* desc) {
  if (check_desc(desc) != RET_OK) return 0;
  return rot_bytes(desc);
}

ret_status_t retention_parallel_fwd(const ret_desc_t* desc, const void* q, const void* k, const void* v,
                                    const void* g, void* o, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if ((st = check_tensors(desc, q, k, v, g, o)) != RET_OK) return st;
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  const size_t need = rot_bytes(desc);
  if (need && (!workspace || workspace_bytes < need)) return RET_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return RET_ERR_ALIGN;
  if (need) {
    const size_t n = tensor_bytes(desc);
    if (overlaps(workspace, need, q, n) || overlaps(workspace, need, k, n) || overlaps(workspace, need, v, n) ||
        overlaps(workspace, need, g, n) || overlaps(workspace, need, o, n))
      return RET_ERR_ALIAS;
  }

  const Shape s = make_shape(desc);
  const float2* table;
  if (!rotate_inputs(desc, k, &table, workspace, stream)) return RET_ERR_HIP;
  if (ret::launch_retention_fwd(s, desc->seqlen, false, q, k, v, g, o, nullptr, nullptr, nullptr, nullptr, nullptr,
                                table, desc->gn_eps, stream) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

size_t retention_parallel_bwd_workspace_bytes(const ret_desc_t* desc, int32_t has_gate) {
  if (check_desc(desc) != RET_OK) return 0;
  return bwd_bytes(desc, has_gate != 0);
}

ret_status_t retention_parallel_bwd(const ret_desc_t* desc, const void* q, const void* k, const void* v,
                                    const void* g, const void* dout, void* dq, void* dk, void* dv, void* dg,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return RET_ERR_NULL;
  if ((g == nullptr) != (dg == nullptr)) return RET_ERR_NULL;
  const void* ins[] = {q, k, v, g, dout};
  void* outs[] = {dq, dk, dv, dg};
  for (const void* p : ins)
    if (p && !aligned16(p)) return RET_ERR_ALIGN;
  for (const void* p : outs)
    if (p && !aligned16(p)) return RET_ERR_ALIGN;
  const size_t n = (size_t)desc->batch * desc->seqlen * desc->heads * desc->dk * elem_size(desc->dtype);
  for (int i = 0; i < 4; ++i) {
    for (const void* p : ins)
      if (overlaps(outs[i], n, p, n)) return RET_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], n, outs[j], n)) return RET_ERR_ALIAS;
  }
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  const size_t need = bwd_bytes(desc, g != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need)) return RET_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return RET_ERR_ALIGN;
  if (overlaps(workspace, need, q, n) || overlaps(workspace, need, k, n) || overlaps(workspace, need, v, n) ||
      overlaps(workspace, need, g, n) || overlaps(workspace, need, dout, n) || overlaps(workspace, need, dq, n) ||
      overlaps(workspace, need, dk, n) || overlaps(workspace, need, dv, n) || overlaps(workspace, need, dg, n))
    return RET_ERR_ALIAS;

  const Shape s = make_shape(desc);
  const size_t tb = bwd_tensor_bytes(desc);
  char* ws = static_cast<char*>(workspace);
  char* next = ws + bwd_table_bytes(desc);
  auto slot = [&]() { char* p = next; next += tb; return p; };
  // q' and k' (rotated when rotation is on) and q' with each sequence's
  // token order reversed
  const float2* table = nullptr;
  const void *qr = q, *kr = k;
  void* qrev = nullptr;
  if (desc->rotary_base != 0.0) {
    float2* tab = reinterpret_cast<float2*>(ws);
    void* qs = slot();
    void* ks = slot();
    qrev = slot();
    if (ret::launch_rotate_keys_table(q, qs, tab, desc->batch, desc->seqlen, desc->heads, desc->dk, desc->dtype,
                                      desc->rotary_base, desc->pos_offset, stream, qrev) != hipSuccess ||
        ret::launch_rotate_keys(k, ks, tab, desc->batch, desc->seqlen, desc->heads, desc->dk, desc->dtype,
                                stream) != hipSuccess)
      return RET_ERR_HIP;
    table = tab;
    qr = qs;
    kr = ks;
  }
  // without rotation the products read q in reversed order where they need
  // it reversed (no copy)
  // dO, the gradient of the retention output before the epilogue (through
  // the gate and GroupNorm, from the recomputed raw output, or dout itself),
  // and its reversed copy
  // (with a gate only the reversed copy is written: the dq product reads it
  // back in forward order)
  const void* dov = dout;
  void* dorev = nullptr;
  if (g) {
    // the recomputed forward forms dg and dO (stored reversed) in its
    // epilogue, from the gate, dout and its output in registers
    dorev = slot();
    if (ret::launch_retention_fwd(s, desc->seqlen, false, qr, kr, v, g, dorev, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, desc->gn_eps, stream, nullptr, nullptr, false, true, nullptr,
                                  nullptr, 0, nullptr, false, dout, dg) != hipSuccess)
      return RET_ERR_HIP;
    dov = nullptr;
  }
  // without a gate the products read dout in reversed order where they need
  // it reversed (no copy)
  const void* qr_rev = qrev ? qrev : q;
  const void* do_rev = dorev ? dorev : dout;
  const bool rq = qrev == nullptr, rdo = dorev == nullptr;
  // Three forward products, each storing its gradient straight into the
  // caller's tensor (turned back by the rotation where it applies), in one
  // grid:
  //   dq = rot^T(P(dO, V, K'));
  //   dk = rot^T(rev P(rev V, rev dO, rev Q')), the transposed mask made
  //        causal by reversing every sequence (q read reversed, output
  //        stored reversed);
  //   dv = rev P(rev K', rev Q', rev dO).
  const ret::ParallelProduct prods[3] = {
      {dov ? dov : dorev, v, kr, dq, dov == nullptr, false, table, false, false},
      {v, do_rev, qr_rev, dk, true, true, table, rdo, rq},
      {kr, qr_rev, do_rev, dv, true, true, nullptr, rq, rdo},
  };
  if (ret::launch_parallel_products(s, 3, prods, desc->gn_eps, stream) != hipSuccess) return RET_ERR_HIP;
  return RET_OK;
}

size_t retention_chunkwise_bwd_workspace_bytes(const ret_desc_t* desc, int32_t chunk, int32_t has_gate) {
  if (check_desc(desc) != RET_OK || chunk < 1) return 0;
  return cbwd_bytes(desc, chunk, has_gate != 0, false);
}

ret_status_t retention_chunkwise_bwd(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                     const void* v, const void* g, const void* dout, void* dq, void* dk, void* dv,
                                     void* dg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return chunkwise_bwd_impl(desc, chunk, q, k, v, g, dout, nullptr, nullptr, dq, dk, dv, dg, nullptr, workspace,
                            workspace_bytes, stream);
}

size_t retention_chunkwise_bwd_state_workspace_bytes(const ret_desc_t* desc, int32_t chunk, int32_t has_gate) {
  if (check_desc(desc) != RET_OK || chunk < 1) return 0;
  return cbwd_bytes(desc, chunk, has_gate != 0, true);
}

ret_status_t retention_chunkwise_bwd_state(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                           const void* v, const void* g, const void* dout, const float* state_in,
                                           const float* d_state_out, void* dq, void* dk, void* dv, void* dg,
                                           float* d_state_in, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  return chunkwise_bwd_impl(desc, chunk, q, k, v, g, dout, state_in, d_state_out, dq, dk, dv, dg, d_state_in,
                            workspace, workspace_bytes, stream);
}

size_t retention_chunkwise_workspace_bytes(const ret_desc_t* desc, int32_t chunk) {
  if (check_desc(desc) != RET_OK || chunk < 1) return 0;
  return chunkwise_bytes(desc, chunk);
}

ret_status_t retention_chunkwise_fwd_timed(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                           const void* v, const void* g, void* o, const float* state_in,
                                           float* state_out, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t before, hipEvent_t after) {
  ret_status_t st = check_chunkwise_args(desc, chunk, q, k, v, g, o, state_in, state_out);
  if (st != RET_OK) return st;
  const size_t need = chunkwise_bytes(desc, chunk);
  if (!workspace || workspace_bytes < need) return RET_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RET_ERR_ALIGN;
  {
    const size_t n = tensor_bytes(desc), ns = state_bytes_exact(desc);
    const void* all[] = {q, k, v, g, o, state_in, state_out};
    const size_t all_n[] = {n, n, n, n, n, ns, ns};
    for (int j = 0; j < 7; ++j)
      if (overlaps(workspace, need, all[j], all_n[j])) return RET_ERR_ALIAS;
  }
  return launch_chunkwise(desc, chunk, q, k, v, g, o, state_in, state_out, static_cast<char*>(workspace), stream,
                          before, after);
}

ret_status_t retention_chunkwise_fwd_noalloc(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                             const void* v, const void* g, void* o, const float* state_in,
                                             float* state_out, int32_t* error_word, hipStream_t stream) {
  ret_status_t st = check_chunkwise_args(desc, chunk, q, k, v, g, o, state_in, state_out);
  if (st != RET_OK) return st;
  if (chunkwise_bytes(desc, chunk) > kScratchBytes) return RET_ERR_SCRATCH;
  if (error_word) {
    if ((reinterpret_cast<uintptr_t>(error_word) & 3u) != 0) return RET_ERR_ALIGN;
    const size_t n = tensor_bytes(desc), ns = state_bytes_exact(desc);
    const void* all[] = {q, k, v, g, o, state_in, state_out};
    const size_t all_n[] = {n, n, n, n, n, ns, ns};
    for (int j = 0; j < 7; ++j)
      if (overlaps(error_word, sizeof(int32_t), all[j], all_n[j])) return RET_ERR_ALIAS;
  }
  char* ws = nullptr;
  if ((st = scratch_for(stream, &ws)) != RET_OK) return st;
  if ((st = launch_chunkwise(desc, chunk, q, k, v, g, o, state_in, state_out, ws, stream, nullptr, nullptr)) !=
      RET_OK)
    return st;
  if (error_word && ret::launch_copy_word(reinterpret_cast<const int*>(ws) + 1, error_word, stream) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

ret_status_t retention_chunkwise_fwd(const ret_desc_t* desc, int32_t chunk, const void* q, const void* k,
                                     const void* v, const void* g, void* o, const float* state_in,
                                     float* state_out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  return retention_chunkwise_fwd_timed(desc, chunk, q, k, v, g, o, state_in, state_out, workspace, workspace_bytes,
                                       stream, nullptr, nullptr);
}

// Packed sequences of different lengths (prefill of a ragged batch): the
// chunkwise form per sequence, the sequences' boundaries in a device array
// the host never reads. Workspace: the chunkwise layout for batch sequences
// of up to seqlen tokens, then the launch schedule.
size_t retention_chunkwise_varlen_workspace_bytes(const ret_desc_t* desc, int32_t chunk) {
  if (check_desc(desc) != RET_OK || chunk < 1) return 0;
  return retention_chunkwise_workspace_bytes(desc, chunk) +
         align_up(ret::chunkwise_sched_bytes(make_shape(desc), eff_chunk(desc, chunk)));
}

ret_status_t retention_chunkwise_varlen_fwd(const ret_desc_t* desc, int32_t chunk, const int32_t* cu_seqlens,
                                            int64_t total_tokens, const void* q, const void* k, const void* v,
                                            const void* g, void* o, const float* state_in, float* state_out,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (chunk < 1) return RET_ERR_SHAPE;
  if (total_tokens < 0 || total_tokens > (int64_t)desc->batch * desc->seqlen) return RET_ERR_SHAPE;
  if (!cu_seqlens || !q || !k || !v || !o) return RET_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return RET_ERR_ALIGN;
  const void* tens[] = {q, k, v, g, o, state_in, state_out};
  for (const void* t : tens)
    if (t && !aligned16(t)) return RET_ERR_ALIGN;
  const size_t n = (size_t)total_tokens * desc->heads * desc->dk * elem_size(desc->dtype);
  const size_t ns = (size_t)desc->batch * desc->heads * desc->dk * desc->dv * 4;
  const size_t cb = ((size_t)desc->batch + 1) * sizeof(int32_t);
  if (overlaps(o, n, q, n) || overlaps(o, n, k, n) || overlaps(o, n, v, n) || overlaps(o, n, g, n) ||
      overlaps(o, n, state_in, ns) || overlaps(o, n, state_out, ns) || overlaps(o, n, cu_seqlens, cb) ||
      overlaps(state_out, ns, cu_seqlens, cb))
    return RET_ERR_ALIAS;
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  const Shape s = make_shape(desc);
  const int32_t c = eff_chunk(desc, chunk);
  const size_t rb = rot_bytes(desc), kb = ctrl_bytes(desc, chunk), hb = chain_bytes(desc);
  const size_t sb = snap_bytes(desc, chunk);
  const size_t need = kb + rb + hb + sb + align_up(ret::chunkwise_sched_bytes(s, c));
  if (!workspace || workspace_bytes < need) return RET_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RET_ERR_ALIGN;
  const void* ins[] = {q, k, v, g, o, state_in, state_out, cu_seqlens};
  const size_t in_n[] = {n, n, n, n, n, ns, ns, cb};
  for (int j = 0; j < 8; ++j)
    if (overlaps(workspace, need, ins[j], in_n[j])) return RET_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  int* ctrl = reinterpret_cast<int*>(ws);
  const float2* table;
  if (!rotate_inputs(desc, k, &table, ws + kb, stream, cu_seqlens, (int)total_tokens)) return RET_ERR_HIP;
  if (ret::launch_retention_fwd(s, c, true, q, k, v, g, o, state_in, state_out, ws + kb + rb + hb,
                                reinterpret_cast<float*>(ws + kb + rb), ctrl, table, desc->gn_eps, stream, nullptr,
                                nullptr, false, false, nullptr, cu_seqlens, (int)total_tokens,
                                ws + kb + rb + hb + sb) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

ret_status_t retention_recurrent_step(const ret_desc_t* desc, const void* q, const void* k, const void* v,
                                      const void* g, void* o, float* state, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (desc->seqlen != 1) return RET_ERR_SHAPE;
  if ((st = check_tensors(desc, q, k, v, g, o)) != RET_OK) return st;
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  if (!state) return RET_ERR_NULL;
  if (!aligned16(state)) return RET_ERR_ALIGN;
  if ((st = check_step_state(desc, q, k, v, g, o, state)) != RET_OK) return st;
  const Shape s = make_shape(desc);
  if (ret::launch_recurrent_step(s, q, k, v, g, o, state, desc->rotary_base, desc->pos_offset, desc->gn_eps,
                                 stream) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

size_t retention_score_map_workspace_bytes(const ret_desc_t* desc) {
  if (check_desc(desc) != RET_OK) return 0;
  return bwd_table_bytes(desc);
}

ret_status_t retention_score_map(const ret_desc_t* desc, const void* q, const void* k, int32_t query,
                                 float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (!q || !k || !scores) return RET_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores)) return RET_ERR_ALIGN;
  if (query < -1 || query >= desc->seqlen) return RET_ERR_ARG;
  const size_t n = (size_t)desc->batch * desc->seqlen * desc->heads * desc->dk * elem_size(desc->dtype);
  const size_t ns = (size_t)desc->batch * desc->seqlen * sizeof(float);
  if (overlaps(scores, ns, q, n) || overlaps(scores, ns, k, n)) return RET_ERR_ALIAS;
  const size_t need = bwd_table_bytes(desc);
  if (need && (!workspace || workspace_bytes < need)) return RET_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return RET_ERR_ALIGN;
  if (need && (overlaps(workspace, need, q, n) || overlaps(workspace, need, k, n) ||
               overlaps(workspace, need, scores, ns)))
    return RET_ERR_ALIAS;
  const Shape s = make_shape(desc);
  float2* table = nullptr;
  if (need) {
    table = static_cast<float2*>(workspace);
    if (ret::launch_rotary_table(table, desc->seqlen, desc->dk, desc->rotary_base, desc->pos_offset, stream) !=
        hipSuccess)
      return RET_ERR_HIP;
  }
  if (ret::launch_score_map(s, q, k, table, query < 0 ? desc->seqlen - 1 : query, scores, stream) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

ret_status_t retention_recurrent_step_positions(const ret_desc_t* desc, const void* q, const void* k,
                                                const void* v, const void* g, void* o, float* state,
                                                const int64_t* positions, hipStream_t stream) {
  ret_status_t st = check_desc(desc);
  if (st != RET_OK) return st;
  if (desc->seqlen != 1) return RET_ERR_SHAPE;
  if ((st = check_tensors(desc, q, k, v, g, o)) != RET_OK) return st;
  if ((st = check_eps(desc, g)) != RET_OK) return st;
  if (!state || !positions) return RET_ERR_NULL;
  if (!aligned16(state) || (reinterpret_cast<uintptr_t>(positions) & 7u) != 0) return RET_ERR_ALIGN;
  if ((st = check_step_state(desc, q, k, v, g, o, state)) != RET_OK) return st;
  if (overlaps(positions, (size_t)desc->batch * 8, o, tensor_bytes(desc)) ||
      overlaps(positions, (size_t)desc->batch * 8, state, state_bytes_exact(desc)))
    return RET_ERR_ALIAS;
  const Shape s = make_shape(desc);
  if (ret::launch_recurrent_step(s, q, k, v, g, o, state, desc->rotary_base, desc->pos_offset, desc->gn_eps,
                                 stream, positions) != hipSuccess)
    return RET_ERR_HIP;
  return RET_OK;
}

ret_status_t retention_chunkwise_error(const void* workspace, size_t workspace_bytes, int32_t* error_word,
                                       hipStream_t stream) {
  if (!workspace || !error_word) return RET_ERR_NULL;
  if (workspace_bytes < 2 * sizeof(int32_t)) return RET_ERR_WORKSPACE;
  if (!aligned16(workspace)) return RET_ERR_ALIGN;
  int32_t word = 0;
  const int32_t* src = static_cast<const int32_t*>(workspace) + 1;
  if (hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return RET_ERR_HIP;
  *error_word = word;
  return RET_OK;
}

}  // extern "C"
