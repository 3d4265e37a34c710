// arnfp8_rows_mxfp8.hip -- the fused row kernel instances for MXFP8 (E8M0 scale per 32 values) output.
#include "arnfp8_tables.hpp"

namespace arnfp8 {

RowKernel row_table_mxfp8(int P, int vpt, bool res_in, bool res_out, bool sc1) {
  return RowTable<kFmtMx>::get(P, vpt, res_in, res_out, sc1);
}

}  // namespace arnfp8
