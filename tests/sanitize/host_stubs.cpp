// Host-only stand-ins for the kernel launchers and device queries that the C
// front end (kda_api.cpp) calls, so that it can be built with g++ under the
// host sanitizers and driven by tests/test_abi.py on a machine without a GPU.
// A launch does nothing and succeeds; there is no device, so the device
// queries report none; the last backward plan is kept for inspection.  Not
// part of the library.
#include "kda_launch.h"

namespace kda {

int device_compute_units() { return 0; }

int scratch_buffer(void** ptr) {
  *ptr = nullptr;
  return 100;  // hipErrorNoDevice
}

int launch_chunk_forward(int, int, int, int, int, const SegPlan&, float, int, const ChunkInputs&, const float*,
                         const int32_t*, void*, float*, float*, int, void*, void*, void* const*) {
  return 0;
}

// the plan of the last backward call, for tests of the host plan
static BwdPlan g_last_bwd;

int launch_chunk_backward(int, int, int, int, int, const BwdPlan& bp, float, int, const ChunkInputs&, const float*,
                          const int32_t*, const void*, const float*, void*, void*, void*, void*, float*, float*, void*,
                          void*, void* const*, const AuxStream*) {
  g_last_bwd = bp;
  return 0;
}

int launch_decode_step(int, int, int, int, float, int, const void*, const void*, const void*, const void*,
                       const float*, float*, void*, void*) {
  return 0;
}

}  // namespace kda

// The window width, area slots and workspace bytes of the last backward
// call's plan (test hook of this stand-in library only).
extern "C" int kda_stub_last_backward_plan(long long* width, long long* n_area, unsigned long long* ws_bytes) {
  *width = kda::g_last_bwd.width;
  *n_area = kda::g_last_bwd.n_area;
  *ws_bytes = kda::g_last_bwd.ws_bytes;
  return 0;
}
