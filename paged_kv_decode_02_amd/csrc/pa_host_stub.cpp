// Host-only stand-ins for the device side of libpa, used only by the
// sanitizer build of the host code (pa_host.cpp, pa_api.cpp compiled with
// g++ -fsanitize=address,undefined; paged_kv_decode_02_amd/build.py,
// build_host_sanitized).  Every launch reports that no device is present,
// so validation and planning run in full and nothing reaches a GPU.  The
// product library is built from the .hip sources instead.
#include "pa_internal.h"

namespace pa {

namespace {
int no_device(const char* who) { return fail(PA_EHIP, std::string(who) + ": host-only build, no device"); }
}  // namespace

int device_cu_count() { return 0; }
int launch_decode(const DecodeLaunch&) { return no_device("decode"); }
int launch_decode_multi(const DecodeLaunch&, const MultiPlan&) { return no_device("decode_multi"); }
int launch_stream(const DecodeLaunch&, const int32_t*, float*, const int32_t*, bool, StreamPlan*) {
  return no_device("stream");
}
int launch_stream_merge(const DecodeLaunch&, const int32_t*, int64_t) { return no_device("stream merge"); }
int launch_cascade(const CascadeLaunch&) { return no_device("cascade"); }
int launch_mixed(const MixedLaunch&) { return no_device("mixed"); }
int launch_append(const AppendLaunch&) { return no_device("append"); }
int launch_append_fp8(const AppendFp8Launch&) { return no_device("append_fp8"); }
void profile_before(void*) {}
void profile_after(void*) {}

}  // namespace pa

extern "C" int pa_decode_noalloc(void*, float*, const void*, const void*, const void*, const int32_t*, int32_t,
                                 const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int64_t,
                                 float, pa_dtype, int32_t, void*) {
  pa::clear_error();
  return pa::fail(PA_EHIP, "pa_decode_noalloc: host-only build, no current device");
}
extern "C" int pa_profile_enable(int32_t) { return pa::fail(PA_EHIP, "pa_profile_enable: host-only build"); }
extern "C" int pa_profile_collect(float*, int32_t) { return pa::fail(PA_EHIP, "pa_profile_collect: host-only build"); }
