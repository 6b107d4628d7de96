// Internal launcher interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ret {

constexpr int kMaxHeadsHost = 128;

// Shared by every launcher: shapes, dtype and the fp32 log2 of each decay
// (computed on the host in fp64).
struct Shape {
  int batch, seqlen, heads, d;  // d = dk = dv
  int dtype;                    // 0 fp32, 1 bf16
  float log2g[kMaxHeadsHost];  // log2 of each decay, fp64 on the host, then rounded
  float gam[kMaxHeadsHost];    // each decay rounded to fp32
};

// cos/sin table [seqlen][d/2] (float2) for positions pos_offset + n.
hipError_t launch_rotary_table(float2* table, int seqlen, int d, double base, int64_t pos_offset,
                               hipStream_t stream);

// Rotated copy kr of k ([batch][seqlen][heads][d], same dtype); the
// queries are turned by the retention kernels as they load them. `krev`
// (may be null) also receives the rotated rows with each sequence's token
// order reversed; kr may be null when only that copy is wanted.
hipError_t launch_rotate_keys(const void* k, void* kr, const float2* table, int batch, int seqlen, int heads, int d,
                              int dtype, hipStream_t stream, void* krev = nullptr);
// The same rotation for packed sequences: sequence b holds rows cu[b] ..
// cu[b+1]-1 of `total` (clamped as the chunkwise kernel clamps them), token n
// of a sequence turns by the table's row n; at most maxlen tokens each.
// the table and the rotation of k (and its reversed copy) in one launch
hipError_t launch_rotate_keys_table(const void* k, void* kr, float2* table, int batch, int seqlen, int heads, int d,
                                    int dtype, double base, int64_t pos_offset, hipStream_t stream,
                                    void* krev = nullptr);
hipError_t launch_rotate_keys_packed(const void* k, void* kr, const float2* table, const int* cu, int batch,
                                     int total, int maxlen, int heads, int d, int dtype, hipStream_t stream);

// Parallel form (chunked == false: chunk == seqlen, no state) or chunkwise
// form (chunked == true) in one launch. Chunkwise needs: snap [BH][nchunks]
// [d][d] of the input dtype, chain [BH][2][d][d] fp32 and a control block of
// chunkwise_ctrl_bytes() ints, all device memory owned by the caller.
size_t chunkwise_ctrl_bytes(int batch, int heads, int nchunks);
// Schedule buffer of a packed (varlen) chunkwise launch: one 16-byte entry
// per workgroup of the grid (s.seqlen bounds every sequence's length).
size_t chunkwise_sched_bytes(const Shape& s, int chunk);
// `rot` (may be null): the cos/sin table of launch_rotary_table, with which
// the kernels turn q as they load it (k must then arrive rotated). For the
// backward's products: `q_rev` reads q
// with each sequence's token order reversed (not with `rot`), `out_rev`
// stores the output reversed, `out_rot` (may be null) turns each stored
// output row back by its stored position's angles.
// `before`/`after` (may be null) are recorded around the main kernel.
// keep_err: the control block's reset leaves its error word (word 1) as it
// is, for the second and later launches of one call.
// gb_dout, gb_dg (both or neither; batch form, with g and out_rev, without
// q_rev or out_rot): the backward's recomputed forward, which
// stores dg (the gate's gradient) and, in o at reversed positions, dO (the
// gradient reaching the retention output through the gate and GroupNorm)
// instead of the forward's output. xsnap (chunkwise, with gb_dout; may be
// null): per-chunk states of the same layout as snap that also receive the
// transpose of each R_{i-1}, the snapshots of a later product whose state
// is that transpose (the dq gradient product's).
hipError_t launch_retention_fwd(const Shape& s, int chunk, bool chunked, const void* q, const void* k, const void* v,
                                const void* g, void* o, const float* state_in, float* state_out, void* snap,
                                float* chain, int* ctrl, const float2* rot, float eps, hipStream_t stream,
                                hipEvent_t before = nullptr, hipEvent_t after = nullptr, bool q_rev = false,
                                bool out_rev = false, const float2* out_rot = nullptr, const int* cu = nullptr,
                                int total = 0, void* sched = nullptr, bool keep_err = false,
                                const void* gb_dout = nullptr, void* gb_dg = nullptr, void* xsnap = nullptr);

// Up to three parallel-form products of shape s with no state in one grid
// (q_rev, out_rev, out_rot as above; no rotation of q on load): the
// backward's gradient products, none of which reads another's output.
struct ParallelProduct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  bool q_rev, out_rev;
  const float2* out_rot;
  bool k_rev, v_rev;  // read k / v with each sequence's token order reversed
};
hipError_t launch_parallel_products(const Shape& s, int n, const ParallelProduct* products, float eps,
                                    hipStream_t stream);

// Up to three chunkwise products of shape s in one grid (the chunkwise
// backward's gradient products): each with its own snapshots (snap), chain
// and control block, the blocks ctrl_stride ints apart from `ctrl` on (each
// at least chunkwise_ctrl_bytes() / 4 ints); the first block's error word
// reports every product's errors. keep_err as for launch_retention_fwd.
// A product whose state is the transpose of an earlier one's needs no state
// workgroups of its own (state_wgs false): either the earlier product of the
// launch names it as xprod, and its state workgroups write this product's
// snapshots too and raise its flags, or an earlier launch wrote them all
// (snap_ready). Such a product has no chain and no state_out; cross0 says
// whether its chunk 0 has a previous state (a snapshot of R_{-1}).
struct ChunkProduct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* state_in;
  float* state_out;
  void* snap;
  float* chain;
  bool q_rev, out_rev;
  const float2* out_rot;
  bool k_rev, v_rev;  // read k / v with each sequence's token order reversed
  bool state_wgs = true;
  bool snap_ready = false;
  bool cross0 = false;
  int xprod = -1;
};
hipError_t launch_chunkwise_products(const Shape& s, int chunk, int n, const ChunkProduct* products, int* ctrl,
                                     int64_t ctrl_stride, float eps, hipStream_t stream, bool keep_err);

// *dst = *src on the device, in stream order (one int).
hipError_t launch_copy_word(const int* src, int* dst, hipStream_t stream);

// States [batch][heads][d][d] fp32: dst = scale[h] * src (transposed per
// matrix when asked); scale: HOST array [heads].
hipError_t launch_state_map(const Shape& s, const float* src, float* dst, bool transpose, const float* scale,
                            hipStream_t stream);

// Score map of query token `qpos`: out [batch][seqlen] fp32 (zeros past
// qpos); `table` (may be null) the rotation's cos/sin table.
hipError_t launch_score_map(const Shape& s, const void* q, const void* k, const float2* table, int qpos, float* out,
                            hipStream_t stream);

// One decode step, in place on `state`. `positions` (device, [batch], may
// be null): each sequence's rotation position instead of `pos`.
hipError_t launch_recurrent_step(const Shape& s, const void* q, const void* k, const void* v, const void* g,
                                 void* o, float* state, double rotary_base, int64_t pos, float eps,
                                 hipStream_t stream, const int64_t* positions = nullptr);

}  // namespace ret
