// multipass.hip -- placeholder launchers for N > 16384 (multi-pass path).
#include "fftconv_internal.hpp"

namespace fftconv {

hipError_t launch_multipass_conv(int, int, const void *, void *, const void *, const float *,
                                 const uint8_t *, void *, int64_t, int64_t, int64_t, int64_t,
                                 hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_multipass_prepare(int, int, const void *, int64_t, void *, const float *, void *,
                                    int64_t, int64_t, int64_t, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace fftconv
