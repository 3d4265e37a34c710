// arnfp8_rows_e5m2.hip -- the fused row kernel instances for e5m2 (per-row fp32 scale) output.
#include "arnfp8_tables.hpp"

namespace arnfp8 {

RowKernel row_table_e5m2(int P, int vpt, bool res_in, bool res_out, bool sc1) {
  return RowTable<kFmtE5m2>::get(P, vpt, res_in, res_out, sc1);
}

}  // namespace arnfp8
