// Dtype dispatch of the decode launchers. The decode kernels of each dtype live in their
// own translation unit (pkv_decode.hip compiled with -DPKV_DECODE_DTYPE=0, 1, 2).

#include "pkv_internal.h"

namespace pkv {

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d_head, int group,
                         hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_decode_dtype<0>(a, d_head, group, stream);
    case 1: return launch_decode_dtype<1>(a, d_head, group, stream);
    case 2: return launch_decode_dtype<2>(a, d_head, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_quantized(const DecodeArgs& a, int dtype, int kv_format, int d_head,
                                   int group, hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_decode_quantized_dtype<1>(a, kv_format, d_head, group, stream);
    case 2: return launch_decode_quantized_dtype<2>(a, kv_format, d_head, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared_prefix(const DecodeArgs& a, int dtype, int d_head, int group,
                                hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_shared_prefix_dtype<0>(a, d_head, group, stream);
    case 1: return launch_shared_prefix_dtype<1>(a, d_head, group, stream);
    case 2: return launch_shared_prefix_dtype<2>(a, d_head, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
