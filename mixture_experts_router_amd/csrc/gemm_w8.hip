// Batched GEMM launches for 8-bit affine codes.
#include "gemm_kernel.hpp"

namespace moe {

template hipError_t launch_bits<8>(GemmMode, int, const GemmParams&, hipStream_t);

}  // namespace moe
