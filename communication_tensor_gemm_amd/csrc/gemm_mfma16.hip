// Instantiations of the tile GEMM for the 16 x 16 MFMA family (bf16 and
// fp32 inputs), as per-step launches and as the single-launch run.  A unit
// of its own because the fp32 half slab needs a higher unroll threshold.
#include "fused_run.h"

namespace dg {

hipError_t launch_gemm_mfma16(int in_kind, int out_kind, const GemmParams& p,
                              hipStream_t stream) {
  using namespace tile;
  if (in_kind == IN_F32 && out_kind == OUT_F32) return launch_t<IN_F32, OUT_F32>(p, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_F32) return launch_t<IN_BF16, OUT_F32>(p, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_BF16) return launch_t<IN_BF16, OUT_BF16>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fused_mfma16(int in_kind, int out_kind, const FusedArgs& a, int grid,
                               hipStream_t stream) {
  using namespace tile;
  if (in_kind == IN_F32 && out_kind == OUT_F32) return launch_fused_t<IN_F32, OUT_F32>(a, grid, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_F32) return launch_fused_t<IN_BF16, OUT_F32>(a, grid, stream);
  if (in_kind == IN_BF16 && out_kind == OUT_BF16)
    return launch_fused_t<IN_BF16, OUT_BF16>(a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace dg
