// rssm_inst_f32.hip -- compiled instances of the materialize and encode
// kernels for f32 state (one translation unit per state dtype so they build
// in parallel).
#include "rssm_instances.h"

namespace rssm {

static const KernelEntry kKernels[] = {
    RSSM_KENTRY(kF32, kF32, 16, 16, 8, 0)
    RSSM_KENTRY(kF32, kF32, 16, 16, 16, 0)
    RSSM_KENTRY(kF32, kBF16, 16, 16, 8, 0)
    RSSM_KENTRY(kF32, kBF16, 16, 16, 16, 0)
    RSSM_KENTRY(kF32, kF16, 16, 16, 8, 0)
    RSSM_KENTRY(kF32, kF16, 16, 16, 16, 0)
    RSSM_KENTRY(kF32, kF32, 64, 128, 8, 0)
    RSSM_KENTRY(kF32, kF32, 64, 128, 16, 0)
    RSSM_KENTRY(kF32, kBF16, 64, 128, 8, 0)
    RSSM_KENTRY(kF32, kBF16, 64, 128, 16, 0)
    RSSM_KENTRY(kF32, kF16, 64, 128, 8, 0)
    RSSM_KENTRY(kF32, kF16, 64, 128, 16, 0)
    RSSM_MENTRY(kF32, kF32, 64, 128, 8, 0)
    RSSM_MENTRY(kF32, kF32, 64, 128, 16, 0)
    RSSM_MENTRY(kF32, kBF16, 64, 128, 8, 0)
    RSSM_MENTRY(kF32, kBF16, 64, 128, 16, 0)
    RSSM_MENTRY(kF32, kF16, 64, 128, 8, 0)
    RSSM_MENTRY(kF32, kF16, 64, 128, 16, 0)
};

static const EncodeEntry kEncoders[] = {
    RSSM_EENTRY(kF32, 16, 0)
    RSSM_EENTRY(kF32, 128, 0)
};

const KernelEntry* kernels_f32(int* n) {
  *n = static_cast<int>(sizeof(kKernels) / sizeof(kKernels[0]));
  return kKernels;
}

const EncodeEntry* encoders_f32(int* n) {
  *n = static_cast<int>(sizeof(kEncoders) / sizeof(kEncoders[0]));
  return kEncoders;
}

}  // namespace rssm
