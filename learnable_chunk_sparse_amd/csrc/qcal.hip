// Q-Cal: the low-rank query calibration of the HiLS paper (paperglide,
// "Implementation and Training Recipes", Q-Cal; dev.to "Engineering
// Details": delta_q = W_up W_down h). The calibrated query only feeds the
// chunk scores, so it is produced in fp32:
//   u[t, h*r + j] = sum_D h[t, D] W_down[h, j, D]        (GEMM 1)
//   q_hat[b, h, i, :] = q[b, h, i, :] + W_up[h] u[t, h*r : h*r + r]   (GEMM 2)
// One workgroup owns 128 tokens x 128 columns of u (128 / r heads). The
// column blocks of one token block run back to back on one XCD, so the
// hidden-state tile comes from HBM once and from that XCD's L2 after.
// GEMM 1 runs on 16x16x32 bf16 MFMAs (exact products, fp32 accumulation)
// over LDS tiles of KS-deep k steps (64 for bf16 where D allows: each row of
// a step is then one whole 128-byte line, loaded by eight lanes), with the
// next steps' global loads prefetched into registers while the current one
// is multiplied. GEMM 2
// (k = r) reuses the u tile from LDS, split into hi + lo bf16 halves so that
// the fp32 u keeps ~16 significant bits, and adds q in the epilogue. With no
// q_hat output only u is produced (GEMM 1 alone).
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

namespace {
constexpr int QT_M = 128, QT_N = 128;
constexpr int QT_UP = QT_N + 4;     // pitch of the fp32 u tile
}

template <typename T, int DH, int NS, int KS>
__global__ __launch_bounds__(256) void k_qcal(const T* __restrict__ q, const T* __restrict__ hs,
                                              const T* __restrict__ Wd, const T* __restrict__ Wu,
                                              float* __restrict__ qhat, float* __restrict__ u_out,
                                              int ntok, int Nq, int Hq, int d, int D, int r) {
  typedef typename Frag<T>::type FT;
  constexpr int KP = KS + 8;  // padded k pitch of the operand tiles (elements)
  // LDS: two k-step tiles of A (tokens) and B (u columns), later reused for u
  extern __shared__ __align__(16) unsigned char smem[];
  T* As = reinterpret_cast<T*>(smem);            // [QT_M][KP]
  T* Bs = As + QT_M * KP;                        // [QT_N][KP]
  float* us = reinterpret_cast<float*>(smem);    // [QT_M][QT_UP] after the k loop

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int wm = w & 1, wn = w >> 1;
  const int ncol = Hq * r;
  int t0, c0;
  {
    // 1-D grid, column block fastest; each XCD walks one contiguous range
    const int ncb = (ncol + QT_N - 1) / QT_N, nwg = gridDim.x, L = blockIdx.x;
    const int xcd = L % NXCD, kx = L / NXCD, qx = nwg / NXCD, rem = nwg % NXCD;
    const int Lp = xcd * qx + min(xcd, rem) + kx;
    t0 = (Lp / ncb) * QT_M;
    c0 = (Lp % ncb) * QT_N;
  }

  // global -> register prefetch: KS / 8 lanes share one row of a k step,
  // each moving 8 consecutive elements, so a row's step is read contiguously;
  // NV passes of 256 / (KS / 8) rows cover the 128 rows of A and of B
  constexpr int VEC = 8, LPR = KS / VEC, RPP = 256 / LPR, NV = QT_M / RPP;
  static_assert(QT_M % RPP == 0 && QT_N == QT_M, "loader covers whole tiles");
  const int lrow = tid / LPR, lk = (tid % LPR) * VEC;  // first row and k of this thread
  const T* asrc[NV];
  const T* bsrc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int ta = min(t0 + lrow + RPP * v, ntok - 1);
    const int cb = min(c0 + lrow + RPP * v, ncol - 1);  // columns past Hq*r are never stored
    asrc[v] = hs + (size_t)ta * D + lk;
    bsrc[v] = Wd + (size_t)cb * D + lk;
  }
  // NS k-steps in flight in a register ring (the loop is unrolled by NS, so
  // the ring indices are fixed; fetches past the end re-read the last step)
  FT ra[NS][NV], rbv[NS][NV];
  auto fetch = [&](int s, int k0) __attribute__((always_inline)) {
    k0 = min(k0, D - KS);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ra[s][v] = ld8<T>(asrc[v] + k0);
      rbv[s][v] = ld8<T>(bsrc[v] + k0);
    }
  };
  auto stash = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      *reinterpret_cast<FT*>(As + (lrow + RPP * v) * KP + lk) = ra[s][v];
      *reinterpret_cast<FT*>(Bs + (lrow + RPP * v) * KP + lk) = rbv[s][v];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b2 = 0; b2 < 4; ++b2) acc[a][b2] = zero4();

#pragma unroll
  for (int s = 0; s < NS; ++s) fetch(s, s * KS);
  for (int k0 = 0; k0 < D; k0 += NS * KS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      __syncthreads();
      stash(s);
      __syncthreads();
      fetch(s, k0 + (s + NS) * KS);
#pragma unroll
      for (int kk = 0; kk < KS; kk += 32) {
        FT af[4], bfr[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          af[mb] = *reinterpret_cast<const FT*>(As + (64 * wm + 16 * mb + col) * KP + kk + 8 * grp);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          bfr[nb] = *reinterpret_cast<const FT*>(Bs + (64 * wn + 16 * nb + col) * KP + kk + 8 * grp);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mma16(af[mb], bfr[nb], acc[mb][nb]);
      }
    }
  }
  __syncthreads();
  // u tile -> LDS (fp32), and optionally to global
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        us[(64 * wm + 16 * mb + 4 * grp + i) * QT_UP + 64 * wn + 16 * nb + col] = acc[mb][nb][i];
  __syncthreads();
  if (u_out != nullptr) {
    for (int x = tid; x < QT_M * QT_N; x += 256) {
      const int rr = x / QT_N, cc = x - rr * QT_N;
      if (t0 + rr < ntok && c0 + cc < ncol) u_out[(size_t)(t0 + rr) * ncol + c0 + cc] = us[rr * QT_UP + cc];
    }
  }

  // GEMM 2, transposed so that every lane ends with 4 consecutive dims of one
  // token: q_hat^T[dims][tokens] = W_up[h] u_h^T + q^T. Wave w takes the
  // tile's heads w, w + 4, ...; W_up[h] is the A operand (16 dims x 32 of r,
  // loaded once per head), u^T the B operand read from LDS and split into hi
  // + lo bf16 halves (fp32 u keeps ~16 significant bits); the q values for
  // the next 16 tokens are fetched while the current ones are multiplied.
  if (qhat == nullptr) return;  // u only (routing folds W_up into the landmark side)
  const int h0 = c0 / r, nh = min(QT_N / r, Hq - h0);
  const int nks = (r + 31) / 32;
  for (int hl = w; hl < nh; hl += 4) {
    const int h = h0 + hl;
    constexpr int NBM = DH / 16;  // 16-dim blocks
    constexpr int nnb = NBM;
    // W_up[h] fragments: loaded unguarded from clamped columns, then zeroed
    // where the 32-wide k step runs past r (no per-element branches around
    // loads)
    FT wa[NBM][2];
#pragma unroll
    for (int nb = 0; nb < NBM; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bool kin = ks < nks && 32 * ks + 8 * grp < r;
        const int kc = kin ? 32 * ks + 8 * grp : 0;
        const FT raw = ld8<T>(Wu + ((size_t)h * d + 16 * nb + col) * r + kc);
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = kin ? (float)raw[j] : 0.f;
        wa[nb][ks] = pack8<T>(z);
      }
    // q^T fragments of token block mb: 4 consecutive dims per (lane, nb)
    typedef typename std::conditional<sizeof(T) == 2, u16x4, f32x4>::type QV;
    auto qrow = [&](int mb) __attribute__((always_inline)) {
      const int t = min(t0 + 16 * mb + col, ntok - 1);
      const int bb = t / Nq, ii = t - bb * Nq;
      return (((size_t)bb * Hq + h) * Nq + ii) * d + 4 * grp;
    };
    QV qv[NBM], qn[NBM];
    {
      const size_t ro = qrow(0);
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) qv[nb] = *reinterpret_cast<const QV*>(q + ro + 16 * nb);
    }
    for (int mb = 0; mb < QT_M / 16; ++mb) {
      {
        const size_t rn = qrow(min(mb + 1, QT_M / 16 - 1));
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) qn[nb] = *reinterpret_cast<const QV*>(q + rn + 16 * nb);
      }
      f32x4 acc[NBM];
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) acc[nb] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks >= nks) break;  // uniform; ks stays a constant index into wa
        const bool kv = 32 * ks + 8 * grp < r;
        const float* ur = us + (16 * mb + col) * QT_UP + hl * r + (kv ? 32 * ks + 8 * grp : 0);
        float x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = kv ? ur[j] : 0.f;
        const FT bhi = pack8<T>(x);
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb)
          if (nb < nnb) acc[nb] = mma16(wa[nb][ks], bhi, acc[nb]);
        if constexpr (sizeof(T) == 2) {
          const u16x8 hb = __builtin_bit_cast(u16x8, bhi);
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = x[j] - bf2f(hb[j]);
          const FT blo = pack8<T>(y);
#pragma unroll
          for (int nb = 0; nb < NBM; ++nb)
            if (nb < nnb) acc[nb] = mma16(wa[nb][ks], blo, acc[nb]);
        }
      }
      // D layout: dims 16 nb + 4 grp + i of token 16 mb + col
      const int t = t0 + 16 * mb + col;
      if (t < ntok) {
        const size_t ro = qrow(mb);
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
          if (nb >= nnb) continue;
          f32x4 o = acc[nb];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] += to_f<T>(qv[nb][i]);
          *reinterpret_cast<f32x4*>(qhat + ro + 16 * nb) = o;
        }
      }
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) qv[nb] = qn[nb];
    }
  }
}

hipError_t launch_qcal(const Dims& p, int Nq, const void* q, const void* h, const void* W_down,
                       const void* W_up, float* q_hat, float* u, hipStream_t st) {
  const int ntok = p.B * Nq;
  dim3 grid((unsigned)(((ntok + QT_M - 1) / QT_M) * ((p.Hq * p.r + QT_N - 1) / QT_N)));
  const size_t el = p.dtype == 1 ? 2 : 4;
  auto go = [&](auto kern, auto tq, int ks) -> hipError_t {
    typedef decltype(tq) TT;
    const size_t lds = std::max<size_t>((size_t)(QT_M + QT_N) * (ks + 8) * el, (size_t)QT_M * QT_UP * 4);
    if (lds > 64 * 1024) {  // beyond the default dynamic LDS limit only
      hipError_t e2 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e2 != hipSuccess) return e2;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, (const TT*)q, (const TT*)h, (const TT*)W_down,
                       (const TT*)W_up, q_hat, u, ntok, Nq, p.Hq, p.d, p.D, p.r);
    return hipGetLastError();
  };
  // bf16: 64-deep k steps (whole 128-byte rows), two in flight when D is a
  // multiple of 128; fp32 rows of a 32-deep step are already 128 bytes, four
  // in flight when D is a multiple of 128. D is a multiple of 32 (checked by
  // the caller), the fallback steps.
  const bool deep = p.D % 128 == 0;
  if (p.dtype == 1) {
    if (p.D % 64 != 0) {
      if (p.d == 64) return go(k_qcal<uint16_t, 64, 1, 32>, uint16_t(), 32);
      return go(k_qcal<uint16_t, 128, 1, 32>, uint16_t(), 32);
    }
    if (p.d == 64) return deep ? go(k_qcal<uint16_t, 64, 2, 64>, uint16_t(), 64) : go(k_qcal<uint16_t, 64, 1, 64>, uint16_t(), 64);
    return deep ? go(k_qcal<uint16_t, 128, 2, 64>, uint16_t(), 64) : go(k_qcal<uint16_t, 128, 1, 64>, uint16_t(), 64);
  }
  if (p.d == 64) return deep ? go(k_qcal<float, 64, 4, 32>, float(), 32) : go(k_qcal<float, 64, 1, 32>, float(), 32);
  return deep ? go(k_qcal<float, 128, 4, 32>, float(), 32) : go(k_qcal<float, 128, 1, 32>, float(), 32);
}

// ---------------------------------------------------------------- shared pair
// One Q-Cal pair for all heads: the per-head kernels read a copy per head
// (16-byte vectors; blockIdx.y = head), and the per-head weight gradients
// are summed over the heads afterwards.
__global__ __launch_bounds__(256) void k_repeat_heads(const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst, long nvec) {
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x < nvec) dst[(long)blockIdx.y * nvec + x] = src[x];
}

__global__ __launch_bounds__(256) void k_sum_heads(const float* __restrict__ src,
                                                   float* __restrict__ dst, long n, int Hq) {
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  float a = 0.f;
  for (int h = 0; h < Hq; ++h) a += src[(long)h * n + x];
  dst[x] = a;
}

hipError_t launch_repeat_heads(const void* src, void* dst, size_t bytes_per_head, int Hq,
                               hipStream_t st) {
  if (bytes_per_head % 16 != 0) return hipErrorInvalidValue;
  const long nvec = (long)(bytes_per_head / 16);
  hipLaunchKernelGGL(k_repeat_heads, dim3((unsigned)((nvec + 255) / 256), (unsigned)Hq), dim3(256), 0,
                     st, (const u32x4*)src, (u32x4*)dst, nvec);
  return hipGetLastError();
}

hipError_t launch_sum_heads(const float* src, float* dst, size_t n, int Hq, hipStream_t st) {
  hipLaunchKernelGGL(k_sum_heads, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst,
                     (long)n, Hq);
  return hipGetLastError();
}

}  // namespace hils
