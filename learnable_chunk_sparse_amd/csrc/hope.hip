// HoPE: partial rotary position encoding of queries and keys.
//
// Paper: "Implementation and Training Recipes" (HoPE keeps the rotary
// frequencies whose period fits the training length and leaves the other
// dimensions without position, NoPE); dev.to summary, "Engineering Details"
// (Hierarchical Positional Encoding: rotary dims inside the pre-training
// window, NoPE beyond it). For row (b, h, n) at position p = pos[b, n] (n when
// no position table is given) and each rotating pair (a, b) of frequency
// theta_j = base^(-2j/d):
//   y_a = x_a cos(p theta_j) - x_b sin(p theta_j)
//   y_b = x_a sin(p theta_j) + x_b cos(p theta_j)
// NoPE pairs are copied unchanged. The inverse (rotation by -p theta_j) is
// the transpose, which carries gradients back.
//
// The angle is reduced in fp64 (turns = p theta_j / 2 pi, minus its nearest
// integer) so positions in the millions keep their low-order bits; sin and cos
// of the reduced turn are taken in fp32. One thread owns 16-byte vectors of
// pairs at one (b, n) and applies them to up to four heads: the angles are
// computed once per position and head group. Consecutive threads cover
// consecutive bytes of a row, then consecutive positions, so every head's
// loads and stores are contiguous runs (an HBM-bound stream: read 2 and write
// 2 elements per pair).
#include "hils_common.h"
#include "hils_internal.h"

#include <math.h>

namespace hils {

// Per-pair turn rate theta_j / 2 pi (negated for the inverse; 0 for NoPE
// pairs) and the rotating-pair mask.
struct HopeTab {
  double rev[64];
  uint64_t rot;
};

// Heads per thread (grid.y covers the rest): enough reuse of the angles, and
// enough threads in flight to keep HBM busy.
constexpr int HOPE_HEADS = 4;

// Pairs j = v VE + i (i < VE) of a unit v: split layout reads the vector at
// v VE and its partner at d/2 + v VE; interleaved layout reads the two
// adjacent vectors at 2 v VE (pair i = elements 2i, 2i + 1 of the 32 bytes).
// x and y may be the same buffer (every element is read and written by one
// thread), so neither is restrict-qualified.
template <typename T, int DH, bool IL>
__global__ __launch_bounds__(256) void k_hope(const T* x, T* y, const int32_t* __restrict__ pos,
                                              int H, int N, int nunits, HopeTab tab) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int UPR = DH / (2 * VE);  // units per row
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= nunits) return;
  const int bn = u / UPR, v = u - bn * UPR;
  const int b = bn / N, n = bn - b * N;
  const double p = pos ? (double)pos[bn] : (double)n;
  float c[VE], s[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) {
    const int j = v * VE + i;
    const double t = p * tab.rev[j];
    const float f = (float)(t - rint(t));  // in [-1/2, 1/2] turns
    sincospif(2.f * f, &s[i], &c[i]);
    if (!((tab.rot >> j) & 1)) {
      c[i] = 1.f;
      s[i] = 0.f;
    }
  }
  const int o0 = IL ? 2 * v * VE : v * VE;
  const int o1 = IL ? o0 + VE : DH / 2 + v * VE;
  // rotate one (first, second) vector pair in place
  auto rotate = [&](T (&a)[VE], T (&bb)[VE]) __attribute__((always_inline)) {
    float xa[VE], xb[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      if constexpr (IL) {
        xa[i] = to_f(i < VE / 2 ? a[2 * i] : bb[2 * i - VE]);
        xb[i] = to_f(i < VE / 2 ? a[2 * i + 1] : bb[2 * i + 1 - VE]);
      } else {
        xa[i] = to_f(a[i]);
        xb[i] = to_f(bb[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      const bool r = (tab.rot >> (v * VE + i)) & 1;
      const float ya = r ? fmaf(xa[i], c[i], -xb[i] * s[i]) : xa[i];
      const float yb = r ? fmaf(xa[i], s[i], xb[i] * c[i]) : xb[i];
      if constexpr (IL) {
        if (i < VE / 2) {
          a[2 * i] = from_f<T>(ya);
          a[2 * i + 1] = from_f<T>(yb);
        } else {
          bb[2 * i - VE] = from_f<T>(ya);
          bb[2 * i + 1 - VE] = from_f<T>(yb);
        }
      } else {
        a[i] = from_f<T>(ya);
        bb[i] = from_f<T>(yb);
      }
    }
  };
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int HU = 4;  // heads whose loads are issued together
  const int hend = min(H, (int)(blockIdx.y + 1) * HOPE_HEADS);
  for (int h0 = blockIdx.y * HOPE_HEADS; h0 < hend; h0 += HU) {
    T va[HU][VE], vb[HU][VE];
#pragma unroll
    for (int k = 0; k < HU; ++k) {
      if (h0 + k < hend) {
        const size_t row = (((size_t)b * H + h0 + k) * N + n) * DH;
        const u32x4v ra = *reinterpret_cast<const u32x4v*>(x + row + o0);
        const u32x4v rb = *reinterpret_cast<const u32x4v*>(x + row + o1);
        __builtin_memcpy(va[k], &ra, 16);
        __builtin_memcpy(vb[k], &rb, 16);
      }
    }
#pragma unroll
    for (int k = 0; k < HU; ++k) {
      if (h0 + k < hend) {
        rotate(va[k], vb[k]);
        const size_t row = (((size_t)b * H + h0 + k) * N + n) * DH;
        u32x4v wa, wb;
        __builtin_memcpy(&wa, va[k], 16);
        __builtin_memcpy(&wb, vb[k], 16);
        *reinterpret_cast<u32x4v*>(y + row + o0) = wa;
        *reinterpret_cast<u32x4v*>(y + row + o1) = wb;
      }
    }
  }
}

template <typename T, int DH>
static hipError_t hope_go(bool il, int B, int H, int N, const void* x, void* y, const int32_t* pos,
                          const HopeTab& tab, hipStream_t st) {
  constexpr int UPR = DH / (2 * (16 / (int)sizeof(T)));
  const long long nu = (long long)B * N * UPR;
  if (nu > 0x7fffff00LL) return hipErrorInvalidValue;
  const int nunits = (int)nu;
  const dim3 grid((nunits + 255) / 256, (H + HOPE_HEADS - 1) / HOPE_HEADS);
  if (il)
    hipLaunchKernelGGL((k_hope<T, DH, true>), grid, dim3(256), 0, st, (const T*)x, (T*)y, pos, H, N,
                       nunits, tab);
  else
    hipLaunchKernelGGL((k_hope<T, DH, false>), grid, dim3(256), 0, st, (const T*)x, (T*)y, pos, H,
                       N, nunits, tab);
  return hipGetLastError();
}

hipError_t launch_hope(int dtype, int B, int H, int N, int d, const void* x, void* y,
                       const int32_t* pos, double base, int train_len, bool interleaved,
                       bool inverse, hipStream_t st) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  HopeTab tab{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int j = 0; j < d / 2; ++j) {
    const double theta = pow(base, -2.0 * j / d);
    if (two_pi / theta <= (double)train_len) {
      tab.rot |= 1ull << j;
      tab.rev[j] = (inverse ? -theta : theta) / two_pi;
    }
  }
  if (B == 0 || H == 0 || N == 0) return hipSuccess;
  if (dtype == 1) {
    return d == 64 ? hope_go<uint16_t, 64>(interleaved, B, H, N, x, y, pos, tab, st)
                   : hope_go<uint16_t, 128>(interleaved, B, H, N, x, y, pos, tab, st);
  }
  return d == 64 ? hope_go<float, 64>(interleaved, B, H, N, x, y, pos, tab, st)
                 : hope_go<float, 128>(interleaved, B, H, N, x, y, pos, tab, st);
}

}  // namespace hils
