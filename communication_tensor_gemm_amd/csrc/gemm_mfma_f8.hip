// Instantiations of the tile GEMM for e4m3 inputs (32 x 32 x 64 f8f6f4
// MFMA), plus the launch entry points that dispatch on the element types.
// Built with the compiler's default MFMA register form, under which this
// family does not spill.
#include "fused_run.h"

namespace dg {

hipError_t launch_gemm_mfma16(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream);
hipError_t launch_fused_mfma16(int in_kind, int out_kind, const FusedArgs& a, int grid,
                               hipStream_t stream);

hipError_t launch_gemm(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream) {
  using namespace tile;
  if (p.M <= 0 || p.N <= 0 || p.L <= 0) return hipSuccess;
  if (in_kind == IN_E4M3 && out_kind == OUT_BF16) return launch_t<IN_E4M3, OUT_BF16>(p, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_F32) return launch_t<IN_E4M3, OUT_F32>(p, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_E4M3) return launch_t<IN_E4M3, OUT_E4M3>(p, stream);
  return launch_gemm_mfma16(in_kind, out_kind, p, stream);
}

hipError_t launch_fused(int in_kind, int out_kind, const FusedArgs& a, int grid, hipStream_t stream) {
  using namespace tile;
  if (grid <= 0) return hipSuccess;
  if (in_kind == IN_E4M3 && out_kind == OUT_BF16) return launch_fused_t<IN_E4M3, OUT_BF16>(a, grid, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_F32) return launch_fused_t<IN_E4M3, OUT_F32>(a, grid, stream);
  if (in_kind == IN_E4M3 && out_kind == OUT_E4M3) return launch_fused_t<IN_E4M3, OUT_E4M3>(a, grid, stream);
  return launch_fused_mfma16(in_kind, out_kind, a, grid, stream);
}

}  // namespace dg
