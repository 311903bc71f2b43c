// Stand-ins for the kernel launchers of libbsta, for the host-only
// sanitizer build of the C ABI's argument validation (bsta_api.hip): each
// counts its calls and launches nothing, so the driver can check that a
// rejected call never reaches a launch and that an accepted one does.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsta_common.hpp"

namespace {
int g_launches = 0;
}

int stub_launches() { return g_launches; }

namespace bsta {
hipError_t launch_permute(const Geo&, const void*, void*, bool, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_tile_pool(const Geo&, const void*, void*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_pool1(const Geo&, const void*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_pool(const Geo&, const void*, const void*, float*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_scores(const Geo&, const float*, const float*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_topk(const Geo&, int, const float*, uint8_t*, int32_t*, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sta(const Geo&, const int32_t*, uint8_t*, int32_t*, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_cumulative(const Geo&, float, int, float*, uint8_t*, int32_t*, int32_t*,
                              hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_packed_select(const Geo&, const PackedSpans&, const float*, uint8_t*, int32_t*,
                                int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t bwd_scratch(void** out) {
    static char fake_scratch[64];
    *out = fake_scratch;
    return hipSuccess;
}
hipError_t launch_attn_bwd(const Geo&, const void*, const void*, const void*, const void*,
                           const void*, const float*, const int32_t*, const int32_t*, int64_t,
                           float, void*, void*, void*, float*, int32_t*, int32_t*, int32_t*,
                           hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attn_fwd(const Geo&, const void*, const void*, const void*, const int32_t*,
                           const int32_t*, int64_t, float, void*, float*, const uint64_t*, int,
                           bool, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prune(const Geo&, const void*, double, uint64_t*, int32_t*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
}  // namespace bsta
