// Row kernel dispatch: tile counts per key count and the per-mode launchers.
#include "kvprof_internal.h"

namespace kvp {

constexpr int kWaves = 8;  // waves per row-kernel workgroup (16 keys per tile)

int row_stats_tpw_for(int n_k, bool mx) {
  const int need = (n_k + kWaves * 16 - 1) / (kWaves * 16);
  static const int kT[] = {1, 2, 4, 8, 16, 24, 32, 40, 49};
  static const int kTmx[] = {2, 4, 8, 16, 24, 32, 40, 50};  // even: 32-key P blocks never straddle waves
  if (mx) {
    for (int t : kTmx)
      if (t >= need) return t;
    return -1;
  }
  for (int t : kT)
    if (t >= need) return t;
  return -1;
}

hipError_t launch_row_stats(const RowStatsParams& p, int tpw, int ksrc, bool mx, hipStream_t s) {
  if (mx) return launch_row_stats_mx(p, tpw, s);
  if (ksrc == KSRC_INT4) return launch_row_stats_int4(p, tpw, s);
  return launch_row_stats_bf16(p, tpw, s);
}

}  // namespace kvp
