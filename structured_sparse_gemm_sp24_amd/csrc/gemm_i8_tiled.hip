// Tiled int8 sparse GEMM: the shape check and the dispatch over output kinds. The kernel is in
// gemm_i8_tiled_impl.h; the int32 and fp32 outputs are instantiated here, bf16 and int8 in
// gemm_i8_tiled_bf16.hip and gemm_i8_tiled_i8.hip (separate files compile in parallel).
#include "gemm_i8_tiled_impl.h"

namespace sp24 {
namespace tiled_i8 {
extern template hipError_t launch_out<OUT_BF16>(const GemmArgs&, hipStream_t);
extern template hipError_t launch_out<OUT_I8>(const GemmArgs&, hipStream_t);
template hipError_t launch_out<OUT_I32>(const GemmArgs&, hipStream_t);
template hipError_t launch_out<OUT_F32>(const GemmArgs&, hipStream_t);
}  // namespace tiled_i8

bool gemm_i8_tiled_ok(const GemmArgs& g) {
    // 16-byte X rows in every batch entry; 32-bit load offsets stay below bit 31, which marks the
    // loads past the last stage: 128 rows of X (128 * ldx), token-major 64 rows from a wave's first,
    // and 16 row blocks of compressed tiles (16 * K / 128 * 1 KB)
    const bool x_ok = g.ldx % 16 == 0 && (reinterpret_cast<uintptr_t>(g.X) & 15) == 0 && (g.batch == 1 || g.sx % 16 == 0);
    const bool tm_ok = !g.tm || g.K % 128 == 0;
    const int64_t tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
    return x_ok && tm_ok && g.N > 64 && g.ldx < ((int64_t)1 << 24) && g.K < ((int64_t)1 << 22) && tiles < (1 << 30);
}

hipError_t launch_gemm_i8_tiled(const GemmArgs& g, hipStream_t s) {
    switch (g.out_kind) {
    case OUT_I32: return tiled_i8::launch_out<OUT_I32>(g, s);
    case OUT_F32: return tiled_i8::launch_out<OUT_F32>(g, s);
    case OUT_BF16: return tiled_i8::launch_out<OUT_BF16>(g, s);
    default: return tiled_i8::launch_out<OUT_I8>(g, s);
    }
}

}  // namespace sp24
