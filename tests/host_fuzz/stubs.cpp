// Host-only stand-ins for the kernel launchers: validation is what is under test.
#include "gdn_internal.h"
int g_launches = 0;
namespace gdn {
hipError_t launch_conv_tree_step(const Dims &, const float *, const float *, const float *, const int32_t *,
                                 const int32_t *, const int32_t *, float *, float *, int32_t *, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_tree_verify(const VerifyArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_replay_commit(const Dims &, int, const LayerPtrs &, const int32_t *, const int32_t *,
                                const int32_t *, const int32_t *, int32_t *, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_conv_step(const Dims &, const float *, const float *, float *, const int32_t *, float *, int32_t *,
                            hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_decode_step(const Dims &, const float *, const float *, const float *, int64_t, const float *,
                              const float *, float *, const int32_t *, float *, int32_t *, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_conv_decode_step(const Dims &, const float *, const float *, float *, const float *, const float *,
                                   int64_t, const float *, const float *, float *, const int32_t *, int32_t *, float *,
                                   int32_t *, hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t launch_prefill(const Dims &, int, const float *, const float *, const float *, int64_t, const float *,
                          const float *, float *, const int32_t *, const float *, int, float *, float *, int32_t *,
                          hipStream_t) {
    ++g_launches; return hipSuccess;
}
hipError_t static_scratch(hipStream_t, float **ptr) {
    *ptr = reinterpret_cast<float *>(0x7E0000000000ull);  // a stand-in, never dereferenced
    return hipSuccess;
}
}  // namespace gdn
