// Batched GEMM launches for 4-bit affine codes.
#include "gemm_kernel.hpp"

namespace moe {

template hipError_t launch_bits<4>(GemmMode, int, const GemmParams&, hipStream_t);

}  // namespace moe
