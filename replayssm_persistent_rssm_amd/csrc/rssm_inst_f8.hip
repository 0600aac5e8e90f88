// rssm_inst_f8.hip -- compiled instances of the materialize and encode
// kernels for f8 state (one translation unit per state dtype so they build
// in parallel).
#include "rssm_kernel.h"

namespace rssm {

#define RSSM_KENTRY(ST, IT, D, S, KM, SR)                                              \
  {ST, IT, D, S, KM, SR, 1, reinterpret_cast<const void*>(&materialize_kernel<ST, IT, D, S, KM, (SR != 0)>), \
   "materialize<" #ST "," #IT "," #D "x" #S ",kmax" #KM ",sr" #SR ">"},
// Multi-checkpoint instances (up to kMaxCheckpoints per request).
#define RSSM_MENTRY(ST, IT, D, S, KM, SR)                                              \
  {ST, IT, D, S, KM, SR, kMaxCheckpoints,                                             \
   reinterpret_cast<const void*>(&materialize_kernel<ST, IT, D, S, KM, (SR != 0), kMaxCheckpoints>), \
   "materialize_checkpoints<" #ST "," #IT "," #D "x" #S ",kmax" #KM ",sr" #SR ">"},
#define RSSM_EENTRY(ST, S, SR)                                                           \
  {ST, S, SR, reinterpret_cast<const void*>(&encode_rows_kernel<ST, S, (SR != 0)>),     \
   "encode_rows<" #ST ",dstate" #S ",sr" #SR ">"},

static const KernelEntry kKernels[] = {
    RSSM_KENTRY(kF8, kF32, 64, 128, 8, 0)
    RSSM_KENTRY(kF8, kF32, 64, 128, 8, 1)
    RSSM_KENTRY(kF8, kF32, 64, 128, 16, 0)
    RSSM_KENTRY(kF8, kF32, 64, 128, 16, 1)
    RSSM_KENTRY(kF8, kBF16, 64, 128, 8, 0)
    RSSM_KENTRY(kF8, kBF16, 64, 128, 8, 1)
    RSSM_KENTRY(kF8, kBF16, 64, 128, 16, 0)
    RSSM_KENTRY(kF8, kBF16, 64, 128, 16, 1)
    RSSM_KENTRY(kF8, kF16, 64, 128, 8, 0)
    RSSM_KENTRY(kF8, kF16, 64, 128, 8, 1)
    RSSM_KENTRY(kF8, kF16, 64, 128, 16, 0)
    RSSM_KENTRY(kF8, kF16, 64, 128, 16, 1)
    RSSM_MENTRY(kF8, kF32, 64, 128, 8, 0)
    RSSM_MENTRY(kF8, kF32, 64, 128, 8, 1)
    RSSM_MENTRY(kF8, kF32, 64, 128, 16, 0)
    RSSM_MENTRY(kF8, kF32, 64, 128, 16, 1)
    RSSM_MENTRY(kF8, kBF16, 64, 128, 8, 0)
    RSSM_MENTRY(kF8, kBF16, 64, 128, 8, 1)
    RSSM_MENTRY(kF8, kBF16, 64, 128, 16, 0)
    RSSM_MENTRY(kF8, kBF16, 64, 128, 16, 1)
    RSSM_MENTRY(kF8, kF16, 64, 128, 8, 0)
    RSSM_MENTRY(kF8, kF16, 64, 128, 8, 1)
    RSSM_MENTRY(kF8, kF16, 64, 128, 16, 0)
    RSSM_MENTRY(kF8, kF16, 64, 128, 16, 1)
};

static const EncodeEntry kEncoders[] = {
    RSSM_EENTRY(kF8, 128, 0)
    RSSM_EENTRY(kF8, 128, 1)
};

const KernelEntry* kernels_f8(int* n) {
  *n = static_cast<int>(sizeof(kKernels) / sizeof(kKernels[0]));
  return kKernels;
}

const EncodeEntry* encoders_f8(int* n) {
  *n = static_cast<int>(sizeof(kEncoders) / sizeof(kEncoders[0]));
  return kEncoders;
}

}  // namespace rssm
