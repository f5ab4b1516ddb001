// Row kernel instantiations: MXFP8 scores with the bf16 reference row.
#include "rowstats_impl.h"

namespace kvp {

hipError_t launch_row_stats_mx(const RowStatsParams& p, int tpw, hipStream_t s) {
  switch (tpw) {
    case 2: return launch_t<2, KSRC_BF16, true>(p, s);
    case 4: return launch_t<4, KSRC_BF16, true>(p, s);
    case 8: return launch_t<8, KSRC_BF16, true>(p, s);
    case 16: return launch_t<16, KSRC_BF16, true>(p, s);
    case 24: return launch_t<24, KSRC_BF16, true>(p, s);
    case 32: return launch_t<32, KSRC_BF16, true>(p, s);
    case 40: return launch_t<40, KSRC_BF16, true>(p, s);
    case 50: return launch_t<50, KSRC_BF16, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvp
