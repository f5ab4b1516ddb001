// Row kernel instantiations: scores against packed 4-bit K/V.
#include "rowstats_impl.h"

namespace kvp {

hipError_t launch_row_stats_int4(const RowStatsParams& p, int tpw, hipStream_t s) {
  switch (tpw) {
    case 1: return launch_t<1, KSRC_INT4, false>(p, s);
    case 2: return launch_t<2, KSRC_INT4, false>(p, s);
    case 4: return launch_t<4, KSRC_INT4, false>(p, s);
    case 8: return launch_t<8, KSRC_INT4, false>(p, s);
    case 16: return launch_t<16, KSRC_INT4, false>(p, s);
    case 24: return launch_t<24, KSRC_INT4, false>(p, s);
    case 32: return launch_t<32, KSRC_INT4, false>(p, s);
    case 40: return launch_t<40, KSRC_INT4, false>(p, s);
    case 49: return launch_t<49, KSRC_INT4, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvp
