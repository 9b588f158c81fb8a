// Q-Cal: the low-rank query calibration of the HiLS paper (paperglide,
// "Implementation and Training Recipes", Q-Cal; dev.to "Engineering
// Details": delta_q = W_up W_down h). The calibrated query only feeds the
// chunk scores, so it is produced in fp32:
//   u[t, h*r + j] = sum_D h[t, D] W_down[h, j, D]   (bf16 MFMA, exact products,
//                                                   fp32 accumulation)
//   q_hat[b, h, i, :] = q[b, h, i, :] + W_up[h] u[t, h*r : h*r + r]   (fp32 FMA)
// One workgroup computes 64 tokens x 64 columns of u (64 / r heads) with four
// waves in a 2 x 2 arrangement of 32 x 32 sub-tiles, then the heads' q_hat.
#include "hils_common.h"
#include "hils_internal.h"

namespace hils {

template <typename T>
__global__ __launch_bounds__(256) void k_qcal(const T* __restrict__ q, const T* __restrict__ hs,
                                              const T* __restrict__ Wd, const T* __restrict__ Wu,
                                              float* __restrict__ qhat, float* __restrict__ u_out,
                                              int ntok, int Nq, int Hq, int d, int D, int r) {
  typedef typename Frag<T>::type FT;
  __shared__ float us[64][65];
  extern __shared__ float wu_s[];  // [nh][d][r + 1]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int ncol = Hq * r;

  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero4();

  const T* arow[2];
  const T* brow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    int t = t0 + 32 * wm + 16 * mb + (lane & 15);
    t = t < ntok ? t : ntok - 1;
    arow[mb] = hs + (size_t)t * D + 8 * (lane >> 4);
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int c = c0 + 32 * wn + 16 * nb + (lane & 15);
    brow[nb] = Wd + (size_t)c * D + 8 * (lane >> 4);
  }
  for (int k0 = 0; k0 < D; k0 += 32) {
    FT A0 = ld8<T>(arow[0] + k0), A1 = ld8<T>(arow[1] + k0);
    FT B0 = ld8<T>(brow[0] + k0), B1 = ld8<T>(brow[1] + k0);
    acc[0][0] = mma16(A0, B0, acc[0][0]);
    acc[0][1] = mma16(A0, B1, acc[0][1]);
    acc[1][0] = mma16(A1, B0, acc[1][0]);
    acc[1][1] = mma16(A1, B1, acc[1][1]);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
        const int col = 32 * wn + 16 * nb + (lane & 15);
        us[row][col] = acc[mb][nb][i];
        if (u_out != nullptr && t0 + row < ntok) u_out[(size_t)(t0 + row) * ncol + c0 + col] = acc[mb][nb][i];
      }
  // stage W_up of this tile's heads as fp32, rows padded to r + 1
  const int nh = 64 / r, h0 = c0 / r;
  for (int x = threadIdx.x; x < nh * d * r; x += 256) {
    const int j = x % r, dd = (x / r) % d, hl = x / (r * d);
    wu_s[(hl * d + dd) * (r + 1) + j] = to_f<T>(Wu[((size_t)(h0 + hl) * d + dd) * r + j]);
  }
  __syncthreads();
  const int total = 64 * nh * d;
  for (int x = threadIdx.x; x < total; x += 256) {
    const int dd = x % d, hl = (x / d) % nh, tok = x / (d * nh);
    const int t = t0 + tok;
    if (t >= ntok) continue;
    const float* wrow = wu_s + (hl * d + dd) * (r + 1);
    const float* urow = &us[tok][hl * r];
    float s = 0.f;
    for (int j = 0; j < r; ++j) s = fmaf(wrow[j], urow[j], s);
    const int bb = t / Nq, i = t - bb * Nq;
    const size_t off = (((size_t)bb * Hq + h0 + hl) * Nq + i) * d + dd;
    qhat[off] = to_f<T>(q[off]) + s;
  }
}

hipError_t launch_qcal(const Dims& p, int Nq, const void* q, const void* h, const void* W_down,
                       const void* W_up, float* q_hat, float* u, hipStream_t st) {
  const int ntok = p.B * Nq;
  dim3 grid((ntok + 63) / 64, p.Hq * p.r / 64);
  const size_t lds = (size_t)(64 / p.r) * p.d * (p.r + 1) * sizeof(float);
  if (p.dtype == 1)
    hipLaunchKernelGGL(k_qcal<uint16_t>, grid, dim3(256), lds, st, (const uint16_t*)q,
                       (const uint16_t*)h, (const uint16_t*)W_down, (const uint16_t*)W_up, q_hat,
                       u, ntok, Nq, p.Hq, p.d, p.D, p.r);
  else
    hipLaunchKernelGGL(k_qcal<float>, grid, dim3(256), lds, st, (const float*)q, (const float*)h,
                       (const float*)W_down, (const float*)W_up, q_hat, u, ntok, Nq, p.Hq, p.d,
                       p.D, p.r);
  return hipGetLastError();
}

}  // namespace hils
