// arnfp8_rows_e4m3.hip -- the fused row kernel instances for e4m3fn (per-row fp32 scale) output.
#include "arnfp8_tables.hpp"

namespace arnfp8 {

RowKernel row_table_e4m3(int P, int vpt, bool res_in, bool res_out, bool sc1) {
  return RowTable<kFmtE4m3>::get(P, vpt, res_in, res_out, sc1);
}

}  // namespace arnfp8
