// Stand-ins for the kernel launchers (launch.hpp) in the sanitizer build of
// the C-ABI layer: the driver's calls all fail validation first, so reaching
// any of these is itself an error.
#include <cstdio>
#include <cstdlib>

#include "launch.hpp"

namespace ret {
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "a kernel launcher was reached: %s\n", what);
  std::abort();
}
hipError_t launch_rotary_table(float2*, int, int, double, int64_t, hipStream_t) { reached("rotary_table"); }
hipError_t launch_rotate_keys(const void*, void*, const float2*, int, int, int, int, int, hipStream_t, void*) {
  reached("rotate_keys");
}
hipError_t launch_rotate_keys_table(const void*, void*, float2*, int, int, int, int, int, double, int64_t, hipStream_t,
                                    void*) {
  reached("rotate_keys_table");
}
hipError_t launch_rotate_keys_packed(const void*, void*, const float2*, const int*, int, int, int, int, int, int,
                                     hipStream_t) {
  reached("rotate_keys_packed");
}
// Workspace layout sizes (host arithmetic, no device call). The driver only
// compares a workspace with what the same build asks for, so these need to be
// self-consistent, not equal to the kernels' own layout.
size_t chunkwise_ctrl_bytes(int batch, int heads, int nchunks) {
  return (16 + (size_t)batch * heads * (nchunks + 1) * 4) * sizeof(int);
}
size_t chunkwise_sched_bytes(const Shape& s, int chunk) {
  const size_t nchunks = ((size_t)s.seqlen + chunk - 1) / chunk;
  return nchunks * s.batch * s.heads * 3 * 16;
}
hipError_t launch_retention_fwd(const Shape&, int, bool, const void*, const void*, const void*, const void*, void*,
                                const float*, float*, void*, float*, int*, const float2*, float, hipStream_t,
                                hipEvent_t, hipEvent_t, bool, bool, const float2*, const int*, int, void*, bool,
                                const void*, void*, void*) {
  reached("retention_fwd");
}
hipError_t launch_parallel_products(const Shape&, int, const ParallelProduct*, float, hipStream_t) {
  reached("parallel_products");
}
hipError_t launch_chunkwise_products(const Shape&, int, int, const ChunkProduct*, int*, int64_t, float, hipStream_t,
                                     bool) {
  reached("chunkwise_products");
}
hipError_t launch_copy_word(const int*, int*, hipStream_t) { reached("copy_word"); }
hipError_t launch_state_map(const Shape&, const float*, float*, bool, const float*, hipStream_t) {
  reached("state_map");
}
hipError_t launch_score_map(const Shape&, const void*, const void*, const float2*, int, float*, hipStream_t) {
  reached("score_map");
}
hipError_t launch_recurrent_step(const Shape&, const void*, const void*, const void*, const void*, void*, float*,
                                 double, int64_t, float, hipStream_t, const int64_t*) {
  reached("recurrent_step");
}
}  // namespace ret
