// Device-side arguments of the block GEMM and its workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4nx {

struct GemmArgs {
  const uint8_t* w;
  const uint16_t* X;
  float* Y;
  float* partial;   // [n_blocks][S][64][8*32] fp32 when S > 1
  uint32_t* cnt;    // [n_blocks] parts arrived; zero between calls
  int32_t TR, TC, M, S;
};

// Tile rows per workgroup of the block GEMM.
constexpr int kGemmRowsPerWg = 8;

// K parts for a weight of TR x TC tiles: enough workgroups to give every CU
// dequantisation work (about 384 workgroups), but at least 4 tile columns per
// part so the fp32 partial tiles stay small next to the weights they summarise.
inline int gemm_parts(int TR, int TC) {
  const int nb = (TR + kGemmRowsPerWg - 1) / kGemmRowsPerWg;
  int S = (384 + nb - 1) / nb;
  const int lim = TC / 4 > 0 ? TC / 4 : 1;
  if (S > lim) S = lim;
  if (S < 1) S = 1;
  return S;
}

inline size_t gemm_ws_bytes(int TR, int TC) {
  const int S = gemm_parts(TR, TC);
  if (S == 1) return 0;
  const size_t nb = (TR + kGemmRowsPerWg - 1) / kGemmRowsPerWg;
  const size_t cnt = (nb * 4 + 255) & ~(size_t)255;
  return cnt + nb * S * 64 * kGemmRowsPerWg * 32 * 4;
}

hipError_t launch_gemm(int kind, const GemmArgs& a, hipStream_t s);

}  // namespace q4nx
