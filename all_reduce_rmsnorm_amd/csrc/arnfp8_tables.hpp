// arnfp8_tables.hpp -- launch tables of the fused row kernel, one per output
// format.  Each table is defined in its own translation unit
// (arnfp8_rows_<format>.hip), which instantiates that format's kernels, so
// the three formats compile in parallel.
#pragma once

#include "arnfp8_kernels.hpp"

namespace arnfp8 {

typedef void (*RowKernel)(RowArgs);

// The kernel instance for (P in 1..8, chunks per lane in {1, 2, 4, 8, 16},
// residual read, residual written, sc1 stores).
RowKernel row_table_e4m3(int P, int vpt, bool res_in, bool res_out, bool sc1);
RowKernel row_table_e5m2(int P, int vpt, bool res_in, bool res_out, bool sc1);
RowKernel row_table_mxfp8(int P, int vpt, bool res_in, bool res_out, bool sc1);

typedef void (*SplitKernel)(SplitArgs);

// The split-row kernel instance for (P in 1..8, residual read, residual
// written); e4m3fn output (arnfp8_split.hip).
SplitKernel split_table(int P, bool res_in, bool res_out);

// Builds one format's table from its kernel template instances.
template <int FMT>
struct RowTable {
  template <int P, int VPT, bool SC1>
  static RowKernel by_res(bool res_in, bool res_out) {
    if (res_in)
      return res_out ? arnfp8_row_kernel<FMT, P, VPT, true, true, SC1>
                     : arnfp8_row_kernel<FMT, P, VPT, true, false, SC1>;
    return res_out ? arnfp8_row_kernel<FMT, P, VPT, false, true, SC1>
                   : arnfp8_row_kernel<FMT, P, VPT, false, false, SC1>;
  }
  template <int P, int VPT>
  static RowKernel by_policy(bool res_in, bool res_out, bool sc1) {
    return sc1 ? by_res<P, VPT, true>(res_in, res_out) : by_res<P, VPT, false>(res_in, res_out);
  }
  template <int P>
  static RowKernel by_vpt(int vpt, bool res_in, bool res_out, bool sc1) {
    switch (vpt) {
      case 1: return by_policy<P, 1>(res_in, res_out, sc1);
      case 2: return by_policy<P, 2>(res_in, res_out, sc1);
      case 4: return by_policy<P, 4>(res_in, res_out, sc1);
      case 8: return by_policy<P, 8>(res_in, res_out, sc1);
      default: return by_policy<P, 16>(res_in, res_out, sc1);
    }
  }
  static RowKernel get(int P, int vpt, bool res_in, bool res_out, bool sc1) {
    switch (P) {
      case 1: return by_vpt<1>(vpt, res_in, res_out, sc1);
      case 2: return by_vpt<2>(vpt, res_in, res_out, sc1);
      case 3: return by_vpt<3>(vpt, res_in, res_out, sc1);
      case 4: return by_vpt<4>(vpt, res_in, res_out, sc1);
      case 5: return by_vpt<5>(vpt, res_in, res_out, sc1);
      case 6: return by_vpt<6>(vpt, res_in, res_out, sc1);
      case 7: return by_vpt<7>(vpt, res_in, res_out, sc1);
      default: return by_vpt<8>(vpt, res_in, res_out, sc1);
    }
  }
};

}  // namespace arnfp8
