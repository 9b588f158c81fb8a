// Routing: surrogate chunk scores, GQA max over the group's heads and a
// running top-K, fused so that the O(N^2 / S) score matrix never leaves the
// chip (paper: surrogate-score step of "The HiLS-Attention Mechanism", the
// GQA max paragraph, top-K selection; nestfrontier "The routing problem" for
// the O(N^2/S) routing term).
//
//   s_{h,c}(i) = scale * q_hat_h(i) . kL_c + e_c  for c < n_dist(i)
//   sel_c(i)   = max_{h in group} s_{h,c}(i)
//   T(i)       = the K best c by (sel desc, c asc)
//
// Workgroup = 4 waves = 64 consecutive positions of one (batch, KV head);
// wave w owns 16 positions x G heads. Scores come from 16x16x32 bf16 MFMAs:
// the fp32 q_hat is split into hi + lo bf16 parts (two products with fp32
// accumulation, landmark keys are exact bf16), which keeps each score within
// ~1e-6 of its fp64 value. Chunks are scanned in ascending order, 16 per step;
// candidates that beat a position's current K-th score are staged in LDS and
// inserted by the lane owning that position, so ties keep the lower index.
#include "hils_common.h"
#include "hils_internal.h"

namespace hils {

template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_route(const QT* __restrict__ qs, const T* __restrict__ kL,
                                               const T* __restrict__ e, int32_t* __restrict__ topk_idx,
                                               float* __restrict__ topk_score, int N, int C, int Hkv,
                                               int K, int W, int S, float scale, int ntiles) {
  typedef typename Frag<T>::type FT;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  constexpr int KS = DH / 32;
  extern __shared__ float lds[];
  const int KP = K + 1;
  float* lst_s = lds;                            // [64][KP]
  int* lst_i = (int*)(lst_s + 64 * KP);          // [64][KP]
  float* lst_h = (float*)(lst_i + 64 * KP);      // [64][KP][G]
  float* thr_s = lst_h + 64 * KP * G;            // [64]
  int* cnt_s = (int*)(thr_s + 64);               // [64]
  float* st = (float*)(cnt_s + 64);              // [4][16][17]
  float* st_h = st + 4 * 16 * 17;                // [4][G][16][17]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tile = ntiles - 1 - blockIdx.x;      // heavy (late) tiles first
  const int bg = blockIdx.y;                      // b * Hkv + g
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * 64;

  if (threadIdx.x < 64) {
    thr_s[threadIdx.x] = NEG_INF;
    cnt_s[threadIdx.x] = 0;
  }

  // A fragments: rows = 16 positions of this wave, one block per head
  FT ahi[G][KS];
  FT alo[G][HAS_LO ? KS : 1];
  {
    int pos = p0 + 16 * w + (lane & 15);
    pos = pos < N ? pos : N - 1;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const QT* src = qs + (((size_t)b * Hq + g * G + hh) * N + pos) * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = to_f<QT>(src[32 * ks + j]);
        ahi[hh][ks] = pack8<T>(x);
        if constexpr (HAS_LO) {
          const u16x8 hb = __builtin_bit_cast(u16x8, ahi[hh][ks]);
          float y[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = x[j] - bf2f(hb[j]);
          alo[hh][ks] = pack8<T>(y);
        }
      }
    }
  }
  __syncthreads();

  const int plast = min(p0 + 16 * w + 15, N - 1);
  const int nd_w = (p0 + 16 * w < N) ? n_distant(plast, W, S) : 0;
  int nd_i[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = p0 + 16 * w + 4 * (lane >> 4) + i;
    nd_i[i] = pos < N ? n_distant(pos, W, S) : 0;
  }
  const T* kLg = kL + (size_t)bg * C * DH;
  const T* eg = e + (size_t)bg * C;
  float* stw = st + w * 16 * 17;
  float* sthw = st_h + w * G * 16 * 17;

  for (int c0 = 0; c0 < nd_w; c0 += 16) {
    const int c = c0 + (lane & 15);
    const int cl = c < nd_w ? c : nd_w - 1;
    FT bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bf[ks] = ld8<T>(kLg + (size_t)cl * DH + 8 * (lane >> 4) + 32 * ks);
    const float ev = to_f<T>(eg[cl]);
    f32x4 acc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      acc[hh] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc[hh] = mma16(ahi[hh][ks], bf[ks], acc[hh]);
        if constexpr (HAS_LO) acc[hh] = mma16(alo[hh][ks], bf[ks], acc[hh]);
      }
    }
    float sel[4];
    bool pass = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float best = NEG_INF;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        acc[hh][i] = fmaf(acc[hh][i], scale, ev);
        best = fmaxf(best, acc[hh][i]);
      }
      sel[i] = (c < nd_i[i]) ? best : NEG_INF;
      pass |= sel[i] > thr_s[16 * w + 4 * (lane >> 4) + i];
    }
    if (__ballot(pass) == 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = 4 * (lane >> 4) + i;
      stw[pr * 17 + (lane & 15)] = sel[i];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) sthw[(hh * 16 + pr) * 17 + (lane & 15)] = acc[hh][i];
    }
    wave_lds_sync();
    if (lane < 16) {
      const int pl = 16 * w + lane;
      float thr = thr_s[pl];
      int n = cnt_s[pl];
      float* ls = lst_s + pl * KP;
      int* li = lst_i + pl * KP;
      float* lh = lst_h + pl * KP * G;
      for (int j = 0; j < 16; ++j) {
        const float v = stw[lane * 17 + j];
        if (!(v > thr)) continue;
        // insert below every entry that scores >= v (earlier chunks win ties)
        int at = n < K ? n : K - 1;
        while (at > 0 && ls[at - 1] < v) {
          ls[at] = ls[at - 1];
          li[at] = li[at - 1];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) lh[at * G + hh] = lh[(at - 1) * G + hh];
          --at;
        }
        ls[at] = v;
        li[at] = c0 + j;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) lh[at * G + hh] = sthw[(hh * 16 + lane) * 17 + j];
        n = n < K ? n + 1 : K;
        if (n == K) thr = ls[K - 1];
      }
      thr_s[pl] = thr;
      cnt_s[pl] = n;
    }
    wave_lds_sync();
  }

  // write this wave's positions: indices ascending, -1 / NaN padded
  if (lane < 16) {
    const int pl = 16 * w + lane;
    const int pos = p0 + pl;
    if (pos < N) {
      const int n = cnt_s[pl];
      int* li = lst_i + pl * KP;
      float* lh = lst_h + pl * KP * G;
      // insertion sort by chunk id (n <= 64)
      for (int a = 1; a < n; ++a) {
        const int key = li[a];
        float hv[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) hv[hh] = lh[a * G + hh];
        int bpos = a;
        while (bpos > 0 && li[bpos - 1] > key) {
          li[bpos] = li[bpos - 1];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) lh[bpos * G + hh] = lh[(bpos - 1) * G + hh];
          --bpos;
        }
        li[bpos] = key;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) lh[bpos * G + hh] = hv[hh];
      }
      int32_t* dst = topk_idx + ((size_t)bg * N + pos) * K;
      for (int k = 0; k < K; ++k) dst[k] = k < n ? li[k] : -1;
      if (topk_score != nullptr) {
        for (int hh = 0; hh < G; ++hh) {
          float* ds = topk_score + (((size_t)b * Hq + g * G + hh) * N + pos) * K;
          for (int k = 0; k < K; ++k) ds[k] = k < n ? lh[k * G + hh] : __builtin_nanf("");
        }
      }
    }
  }
}

static size_t route_lds(int K, int G) {
  const int KP = K + 1;
  return sizeof(float) * (size_t)(64 * KP * 2 + 64 * KP * G + 128 + 4 * 16 * 17 * (1 + G));
}

template <typename T, typename QT, int G, int DH>
static hipError_t route_go(const Dims& p, const void* qs, const void* kL, const void* e,
                           int32_t* idx, float* sc, hipStream_t st) {
  const int ntiles = (p.N + 63) / 64;
  const size_t lds = route_lds(p.K, G);
  auto kern = k_route<T, QT, G, DH>;
  if (lds > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), lds, st, (const QT*)qs,
                     (const T*)kL, (const T*)e, idx, sc, p.N, p.C, p.Hkv, p.K, p.W, p.S, p.scale,
                     ntiles);
  return hipGetLastError();
}

template <typename T, typename QT, int G>
static hipError_t route_d(const Dims& p, const void* qs, const void* kL, const void* e, int32_t* idx,
                          float* sc, hipStream_t st) {
  if (p.d == 64) return route_go<T, QT, G, 64>(p, qs, kL, e, idx, sc, st);
  return route_go<T, QT, G, 128>(p, qs, kL, e, idx, sc, st);
}

template <typename T, typename QT>
static hipError_t route_g(const Dims& p, const void* qs, const void* kL, const void* e, int32_t* idx,
                          float* sc, hipStream_t st) {
  switch (p.G) {
    case 1: return route_d<T, QT, 1>(p, qs, kL, e, idx, sc, st);
    case 2: return route_d<T, QT, 2>(p, qs, kL, e, idx, sc, st);
    case 4: return route_d<T, QT, 4>(p, qs, kL, e, idx, sc, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route(const Dims& p, const void* qs, bool q_is_f32, const void* kL, const void* e,
                        int32_t* topk_idx, float* topk_score, hipStream_t st) {
  if (p.dtype == 1) {
    if (q_is_f32) return route_g<uint16_t, float>(p, qs, kL, e, topk_idx, topk_score, st);
    return route_g<uint16_t, uint16_t>(p, qs, kL, e, topk_idx, topk_score, st);
  }
  return route_g<float, float>(p, qs, kL, e, topk_idx, topk_score, st);
}

}  // namespace hils
