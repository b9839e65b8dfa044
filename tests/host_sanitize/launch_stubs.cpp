// Stand-ins for the device side of libsvga, for a host-only build of its C ABI
// (api.cpp, tilemap_host.cpp, plan_host.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer. Every launcher and HIP runtime call answers
// "no device": the sanitized tests exercise argument checking, the host tile
// map builder and the host planning code, and reach no launch.
#include "svga_internal.h"

extern "C" {
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "no device (host-only sanitizer build)"; }
}

namespace svga {

hipError_t launch_attn_fwd(const AttnLaunch& a, hipStream_t, bool* supported) {
    *supported = attn_supported(a.head_dim, a.bq, a.bkv);
    return hipErrorNoDevice;
}
hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    return hipErrorNoDevice;
}
hipError_t launch_permute(const void*, void*, const uint8_t*, int32_t, const Geo&, int32_t, bool, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_build_tilemap(const Geo&, int32_t, int32_t, int32_t, unsigned char*, const MapLayout&,
                                const svga_tilemap_header&, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_route(const RouteLaunch&, hipStream_t) { return hipErrorNoDevice; }

}  // namespace svga
