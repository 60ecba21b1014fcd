// Instantiation of the 16-bit fused RoPE + FlashAttention kernels for __bf16
// (one translation unit per element type, compiled in parallel).
#include "flash_fwd.h"

namespace ropefa {

void launch_flash16_bf16(const FaArgs& a, int hp, int D, int rot, dim3 grid, hipStream_t stream) {
    launch16_hp<__bf16>(a, hp, D, rot, grid, stream);
}

}  // namespace ropefa
