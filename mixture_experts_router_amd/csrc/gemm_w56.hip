// Batched GEMM launches for 5- and 6-bit affine codes.
#include "gemm_kernel.hpp"

namespace moe {

template hipError_t launch_bits<5>(GemmMode, int, const GemmParams&, hipStream_t);
template hipError_t launch_bits<6>(GemmMode, int, const GemmParams&, hipStream_t);

}  // namespace moe
