// Decode kernels instantiated for 8 query head(s) per workgroup.
#include "kvq_decode_impl.hpp"

namespace kvq {
template hipError_t launch_decode_hg<8>(const DecodeArgs &, hipStream_t, hipEvent_t, hipEvent_t);
}  // namespace kvq
