// Test-only stand-ins for the kernel launchers, linked into the host-sanitizer build
// of api.hip: they record that validation let a call through and return a sentinel
// status, touching none of their pointer arguments.  Never part of the library.
#include "ps_internal.h"

extern "C" int ps_stub_calls = 0;
constexpr int kReached = 77;

namespace ps {

int launch_maxpool2d(const float *, float *, int, int, int, int, int, int, int, int, int, int,
                     hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_conv_pool(const void *, const void *, const float *, const float *, void *, int, int,
                     int, int, int, int, int, int, int, float, int, int, int, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_conv_general(const void *, const void *, const float *, const float *, void *, int,
                        int, int, int, int, int, int, int, int, int, int, int, int, int, float,
                        int, int, int, int, int, int, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_convT_softmax(const float *, const float *, const float *, const float *, float *, int,
                         int, int, int, int, int, int, int, float, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_convT_softmax_bf16(const uint16_t *, const uint16_t *, const float *, const float *,
                              uint16_t *, int, int, int, int, int, int, int, int, float,
                              hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_convT(const float *, const float *, const float *, float *, int, int, int, int, int,
                 int, int, int, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_tanh_scale_bias_maxpool(const void *, const float *, void *, int, int, int, int, int,
                                   int, int, float, int, int, int, int, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}
int launch_softmax_bias_scale_sigmoid(const float *, const float *, float *, int, int, int, int,
                                      float, hipStream_t) {
    ++ps_stub_calls;
    return kReached;
}

}  // namespace ps
