// One variant of the decode kernels per object: PKV_STREAM (non-temporal K/V
// loads), PKV_STEP (the decode step with its cache writes), PKV_HALF (blocks of 8
// tokens).  The build compiles this file once per variant; without the macros it
// instantiates all eight.

#include "decode_kernels.h"

namespace pkv {

#if defined(PKV_STREAM) && defined(PKV_STEP) && defined(PKV_HALF)
template hipError_t launch_decode_variant<PKV_STREAM, PKV_STEP, PKV_HALF>(int, int, bool, const DecodeArgs&,
                                                                          int, hipStream_t);
#else
template hipError_t launch_decode_variant<false, false, false>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<false, false, true>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<false, true, false>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<false, true, true>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<true, false, false>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<true, false, true>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<true, true, false>(int, int, bool, const DecodeArgs&, int, hipStream_t);
template hipError_t launch_decode_variant<true, true, true>(int, int, bool, const DecodeArgs&, int, hipStream_t);
#endif

}  // namespace pkv
