// Persistent layer chain with K-chunked MFMA stages: the instantiations for
// MT = 2 and 3 m-tiles with (unpaired, paired) tiles per item of (4, 6) and
// (2, 6), and (4, 4) at four m-tiles, where six paired tiles would not fit
// the register file (the kernel is in chain_body.h).
#include <hip/hip_runtime.h>

#include "chain_body.h"

namespace sg {

ChainKernel chain_kernel_kc(int mt, int code) {
  switch (mt * 100 + code) {
    case 2 * 100 + 46: return k_chain<3, 2, 46>;
    case 2 * 100 + 26: return k_chain<3, 2, 26>;
    case 3 * 100 + 46: return k_chain<3, 3, 46>;
    case 3 * 100 + 26: return k_chain<3, 3, 26>;
    case 4 * 100 + 44: return k_chain<3, 4, 44>;
    default: return nullptr;
  }
}

}  // namespace sg
