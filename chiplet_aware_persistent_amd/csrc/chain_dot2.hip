// Persistent layer chain with dot2 stages (M < 16): the instantiations for
// M = 1..15 rows and G = 2 or 4 weight rows per wave (the kernel is in
// chain_body.h).
#include <hip/hip_runtime.h>

#include "chain_body.h"

namespace sg {

template <int M>
static ChainKernel dot2_for(int g) {
  if (g == 2) return k_chain<0, M, 2>;
  if (g == 4) return k_chain<0, M, 4>;
  return nullptr;
}

ChainKernel chain_kernel_dot2(int m, int g) {
  switch (m) {
    case 1: return dot2_for<1>(g);
    case 2: return dot2_for<2>(g);
    case 3: return dot2_for<3>(g);
    case 4: return dot2_for<4>(g);
    case 5: return dot2_for<5>(g);
    case 6: return dot2_for<6>(g);
    case 7: return dot2_for<7>(g);
    case 8: return dot2_for<8>(g);
    case 9: return dot2_for<9>(g);
    case 10: return dot2_for<10>(g);
    case 11: return dot2_for<11>(g);
    case 12: return dot2_for<12>(g);
    case 13: return dot2_for<13>(g);
    case 14: return dot2_for<14>(g);
    case 15: return dot2_for<15>(g);
    default: return nullptr;
  }
}

}  // namespace sg
