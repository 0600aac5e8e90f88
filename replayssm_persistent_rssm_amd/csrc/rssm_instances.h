// rssm_instances.h -- registry-entry macros shared by the per-dtype instance
// files (rssm_inst_<dtype>.hip).  Each file lists the compiled template
// instances of its state dtype in a table the host launcher searches.
#pragma once

#include "rssm_kernel.h"

// Single-checkpoint materialize instance.
#define RSSM_KENTRY(ST, IT, D, S, KM, SR)                                              \
  {ST, IT, D, S, KM, SR, 1, reinterpret_cast<const void*>(&materialize_kernel<ST, IT, D, S, KM, (SR != 0)>), \
   "materialize<" #ST "," #IT "," #D "x" #S ",kmax" #KM ",sr" #SR ">"},
// Multi-checkpoint instance (up to kMaxCheckpoints per request).
#define RSSM_MENTRY(ST, IT, D, S, KM, SR)                                              \
  {ST, IT, D, S, KM, SR, kMaxCheckpoints,                                             \
   reinterpret_cast<const void*>(&materialize_kernel<ST, IT, D, S, KM, (SR != 0), kMaxCheckpoints>), \
   "materialize_checkpoints<" #ST "," #IT "," #D "x" #S ",kmax" #KM ",sr" #SR ">"},
// Encode test hook instance.
#define RSSM_EENTRY(ST, S, SR)                                                           \
  {ST, S, SR, reinterpret_cast<const void*>(&encode_rows_kernel<ST, S, (SR != 0)>),     \
   "encode_rows<" #ST ",dstate" #S ",sr" #SR ">"},
