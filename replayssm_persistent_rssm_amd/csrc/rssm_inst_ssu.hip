// rssm_inst_ssu.hip -- compiled instances of the decode-step kernel: state
// and input dtypes f32 / bf16 / f16, up to 4 and up to 8 new tokens.
#include "ssu_kernel.h"

namespace rssm {

namespace {

template <int ST, int IT>
const void* pick(int tokens) {
  if (tokens <= 4) return reinterpret_cast<const void*>(&ssu_decode_kernel<ST, IT, 4>);
  return reinterpret_cast<const void*>(&ssu_decode_kernel<ST, IT, 8>);
}

template <int ST>
const void* pick_input(int input_dtype, int tokens) {
  switch (input_dtype) {
    case kF32: return pick<ST, kF32>(tokens);
    case kBF16: return pick<ST, kBF16>(tokens);
    case kF16: return pick<ST, kF16>(tokens);
    default: return nullptr;
  }
}

}  // namespace

// NULL when no instance covers the combination.
const void* ssu_kernel_for(int state_dtype, int input_dtype, int tokens) {
  if (tokens < 1 || tokens > 8) return nullptr;
  switch (state_dtype) {
    case kF32: return pick_input<kF32>(input_dtype, tokens);
    case kBF16: return pick_input<kBF16>(input_dtype, tokens);
    case kF16: return pick_input<kF16>(input_dtype, tokens);
    default: return nullptr;
  }
}

}  // namespace rssm
