// Tiled int8 sparse GEMM, requantized int8 output (the kernel is in gemm_i8_tiled_impl.h).
#include "gemm_i8_tiled_impl.h"

namespace sp24 {
namespace tiled_i8 {
template hipError_t launch_out<OUT_I8>(const GemmArgs&, hipStream_t);
}  // namespace tiled_i8
}  // namespace sp24
