// Batched GEMM launches for NVFP4 codes.
#include "gemm_kernel.hpp"

namespace moe {

template hipError_t launch_bits<NVF4>(GemmMode, int, const GemmParams&, hipStream_t);

}  // namespace moe
