// Persistent layer chain with K-chunked MFMA stages (an ablation: slower than
// the default stage kernels): the instantiations for MT = 2 m-tiles (M = 17
// to 32) with (unpaired, paired) tiles per item of (4, 6) and (2, 6).  Three
// and four m-tiles do not fit the register file next to the chain's state
// (the kernel is in chain_body.h).
#include <hip/hip_runtime.h>

#include "chain_body.h"

namespace sg {

ChainKernel chain_kernel_kc(int mt, int code) {
  switch (mt * 100 + code) {
    case 2 * 100 + 46: return k_chain<3, 2, 46>;
    case 2 * 100 + 26: return k_chain<3, 2, 26>;
    default: return nullptr;
  }
}

}  // namespace sg
