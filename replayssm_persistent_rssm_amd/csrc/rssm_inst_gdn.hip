// rssm_inst_gdn.hip -- compiled instances of the gated-delta-rule commit
// kernel: windows of up to 8 and up to 16 tokens.
#include "gdn_kernel.h"

namespace rssm {

const void* gdn_kernel_for(int window) {
  if (window <= 8) return reinterpret_cast<const void*>(&gdn_commit_kernel<8>);
  return reinterpret_cast<const void*>(&gdn_commit_kernel<16>);
}

}  // namespace rssm
