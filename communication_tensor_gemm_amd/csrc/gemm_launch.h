// Internal interface between the step scheduler and the gfx950 GEMM kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Element type of A/B, and of C/D.
enum InKind { IN_F32 = 0, IN_BF16 = 1, IN_E4M3 = 2 };
enum OutKind { OUT_F32 = 0, OUT_BF16 = 1 };

// One GEMM over an (M x N) block of D, full K:
//   D[i][j] = alpha * sum_k A[i][k] * B[j][k] + beta * C[i][j]
// A rows are lda apart, B rows (the N index) ldb apart, both K-contiguous.
// Strides and leading dimensions are in elements of the operand's type.
struct GemmParams {
  const void* A;
  const void* B;
  const void* C;  // read only when beta != 0
  void* D;
  int64_t lda, ldb, ldc, ldd;
  int64_t sA, sB, sC, sD;  // batch strides
  int32_t M, N, K, L;
  float alpha, beta;
};

// Macro tile of one workgroup, and the bytes of one operand row per K tile.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowBytes = 128;

inline int in_elem_size(int in_kind) { return in_kind == IN_F32 ? 4 : (in_kind == IN_BF16 ? 2 : 1); }
inline int out_elem_size(int out_kind) { return out_kind == OUT_F32 ? 4 : 2; }

// Enqueue one GEMM on `stream`.  The caller has validated the shapes:
// K * elem_size % 16 == 0, 256 * lda * elem_size < 2^31 (same for ldb).
hipError_t launch_gemm(int in_kind, int out_kind, const GemmParams& p, hipStream_t stream);

}  // namespace dg
