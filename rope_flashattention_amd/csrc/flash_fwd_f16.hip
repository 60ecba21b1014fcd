// Instantiation of the 16-bit fused RoPE + FlashAttention kernels for _Float16
// (one translation unit per element type, compiled in parallel).
#include "flash_fwd.h"

namespace ropefa {

void launch_flash16_f16(const FaArgs& a, int hp, int D, int rot, dim3 grid, hipStream_t stream) {
    launch16_hp<_Float16>(a, hp, D, rot, grid, stream);
}

}  // namespace ropefa
