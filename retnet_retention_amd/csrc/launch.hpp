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

// Rotated copies qr, kr of q, k ([batch][seqlen][heads][d], same dtype).
hipError_t launch_rotate_qk(const void* q, const void* k, void* qr, void* kr, const float2* table, int batch,
                            int seqlen, int heads, int d, int dtype, hipStream_t stream);

// Per-chunk states: snap[b][h][i] = R_{i-1} transposed ([dv][dk], element
// type = dtype), state_out = R_last (fp32 [dk][dv]) when non-null.
hipError_t launch_chunk_state(const Shape& s, int chunk, const void* k, const void* v, const float* state_in,
                              float* state_out, void* snap, hipStream_t stream);

// Output of the parallel form (snap == nullptr, chunk == seqlen) or of the
// chunkwise form (snap from launch_chunk_state).
hipError_t launch_retention_out(const Shape& s, int chunk, const void* q, const void* k, const void* v,
                                const void* g, void* o, const void* snap, int has_state0, float eps,
                                hipStream_t stream);

// One decode step, in place on `state`.
hipError_t launch_recurrent_step(const Shape& s, const void* q, const void* k, const void* v, const void* g,
                                 void* o, float* state, double rotary_base, int64_t pos, float eps,
                                 hipStream_t stream);

}  // namespace ret
