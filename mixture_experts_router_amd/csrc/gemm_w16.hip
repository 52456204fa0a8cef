// Batched GEMM launches for fp16 weights.
#include "gemm_kernel.hpp"

namespace moe {

template hipError_t launch_bits<16>(GemmMode, int, const GemmParams&, hipStream_t);

}  // namespace moe
