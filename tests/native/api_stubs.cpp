// Stand-ins for the kernel launchers of libbra, for the host-only build of
// the C-ABI front end under the sanitizers.  No call of that check passes
// validation, so reaching any of these is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "bra_internal.h"

namespace bra {
namespace {
[[noreturn]] void reached(const char* name) {
  std::printf("FAIL %s reached: a call passed validation\n", name);
  std::exit(2);
}
}  // namespace

hipError_t launch_pool(const void*, const void*, double*, double*, const Shape&, bool, hipStream_t) {
  reached("launch_pool");
}
hipError_t launch_linear(const void*, int, int, const void*, const float*, int, void* const*, int,
                         bool, hipStream_t, int, const void*) {
  reached("launch_linear");
}
hipError_t launch_mlp(const void*, long long, int, int, const void*, const float*, const void*,
                      const float*, const void*, void*, hipStream_t) {
  reached("launch_mlp");
}
hipError_t launch_block_tail(const void*, const void*, long long, int, int, const void*,
                             const float*, const float*, const float*, float, const void*,
                             const float*, const void*, const float*, void*, void*, void*,
                             hipStream_t) {
  reached("launch_block_tail");
}
hipError_t launch_pos_conv(const void*, const float*, const float*, const Shape&, bool, void*,
                           hipStream_t, const float*, const float*, float, void*) {
  reached("launch_pos_conv");
}
hipError_t launch_backward(const void*, const void*, const void*, const int32_t*, const void*,
                           const Shape&, float, const float*, int, void*, void*, void*, float*,
                           float*, void*, hipStream_t) {
  reached("launch_backward");
}
hipError_t launch_layer_norm(const void*, long long, int, const float*, const float*, float, bool,
                             void*, hipStream_t) {
  reached("launch_layer_norm");
}
hipError_t launch_means_proj(const double*, int, int, const void*, const float*, bool, double*,
                             double*, hipStream_t) {
  reached("launch_means_proj");
}
hipError_t launch_pool_route(const void*, const void*, double*, double*, const Shape&, bool, double,
                             int32_t*, float*, hipStream_t) {
  reached("launch_pool_route");
}
hipError_t launch_route(const double*, const double*, const Shape&, double, int32_t*, float*,
                        hipStream_t) {
  reached("launch_route");
}
hipError_t launch_attend(const void*, const void*, const void*, const int32_t*, const Shape&, bool,
                         float, const float*, const float*, int, void*, hipStream_t) {
  reached("launch_attend");
}
bool attend_xproj_ok(const Shape&, const float*, int) { return false; }
hipError_t launch_attend_xproj(const void*, const void*, const float*, const int32_t*,
                               const Shape&, float, const float*, const float*, int, void*,
                               hipStream_t) {
  reached("launch_attend_xproj");
}
hipError_t launch_attend_region(const void*, const void*, const void*, const int32_t*,
                                const Shape&, float, const float*, const float*, int, void*,
                                hipStream_t) {
  reached("launch_attend_region");
}
hipError_t scratch_buffer(void**) { reached("scratch_buffer"); }
hipError_t launch_lepe(const void*, const float*, const float*, int, const Shape&, bool, void*,
                       hipStream_t) {
  reached("launch_lepe");
}
}  // namespace bra
