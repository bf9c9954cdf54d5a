// Decode launch entry: picks the compiled variant of the decode kernels (declared
// in pagedkv_internal.h, instantiated by decode_variant.hip) for a call's load
// policy, mode and block size.

#include "pagedkv_internal.h"

namespace pkv {

namespace {

template <bool Step>
hipError_t dispatch(int dtype, int head_dim, bool group, const DecodeArgs& a, int passes,
                    hipStream_t st) {
    const bool stream = !a.keep_cached;
    if (a.block_size == 8)
        return stream ? launch_decode_variant<true, Step, true>(dtype, head_dim, group, a, passes, st)
                      : launch_decode_variant<false, Step, true>(dtype, head_dim, group, a, passes, st);
    return stream ? launch_decode_variant<true, Step, false>(dtype, head_dim, group, a, passes, st)
                  : launch_decode_variant<false, Step, false>(dtype, head_dim, group, a, passes, st);
}

}  // namespace

hipError_t launch_decode_step(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                              hipStream_t stream) {
    return dispatch<true>(dtype, head_dim, use_group_kernel, a, 4, stream);
}

hipError_t launch_decode(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                         int passes, hipStream_t stream) {
    return dispatch<false>(dtype, head_dim, use_group_kernel, a, passes, stream);
}

}  // namespace pkv
