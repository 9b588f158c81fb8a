// HiLS decode step: one new query per sequence (paper Fig. 6 decode latency;
// nestfrontier "The routing problem": score the chunk summaries, keep the top
// K distant chunks, attend inside them and in the local window).
//
// The step is bound by HBM bandwidth: every distant landmark key is read once
// (the O(L/S) per-token retrieval term), then only the K selected chunks and
// the window. Four launches:
//   k_dec_scan    split landmark scan: each workgroup scores CPW chunks of one
//                 (sequence, KV head) with 16x16x32 MFMAs (rows = chunks, columns
//                 = the group's heads, hi and lo halves of the fp32 query), takes
//                 the max over heads, and keeps its own top-K (rank count).
//   k_dec_merge   per (sequence, KV head): bitonic sort of the splits' lists,
//                 final top-K in ascending chunk order.
//   k_dec_attn    one wave per 64-token unit (a selected chunk or a window
//                 block) for all G heads: S^T = K Q^T on MFMA, softmax, O^T =
//                 V^T P^T with V staged transposed in LDS. A chunk unit leaves
//                 (log-weight s_c, weight 1, O_c); a window block leaves its
//                 (max, sum, unnormalised output).
//   k_dec_combine per (sequence, query head): log-sum-exp merge of all units,
//                 which is exactly the fusion softmax over {s_c} and lse_W.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>

namespace hils {

namespace {

constexpr int CPW = 256;  // chunks per scan workgroup
constexpr int VPADD = 8;

__device__ __forceinline__ int seq_n(const int32_t* seq_len, int b, int N) {
  if (seq_len == nullptr) return N;
  int n = seq_len[b];
  return n < 1 ? 1 : (n > N ? N : n);
}

// monotone map of a float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t ord_f(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// sort key: larger score first, then lower chunk index first
__device__ __forceinline__ uint64_t mkkey(float s, int c) {
  return ((uint64_t)ord_f(s) << 32) | (uint32_t)(~(uint32_t)c);
}
constexpr uint64_t EMPTY_KEY = 0;  // below every real key

}  // namespace

// ---------------------------------------------------------------- scan
template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_dec_scan(const QT* __restrict__ qs, const T* __restrict__ kL,
                                                  const T* __restrict__ e,
                                                  const int32_t* __restrict__ seq_len,
                                                  uint64_t* __restrict__ lists, int N, int C, int Hkv,
                                                  int K, int W, int S, float scale, int nsplit) {
  typedef typename Frag<T>::type FT;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  constexpr int KS = DH / 32;
  constexpr int NPART = HAS_LO ? 2 : 1;
  __shared__ float sc_s[CPW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int n = seq_n(seq_len, b, N);
  const int nd = n_distant(n - 1, W, S);
  const int c_lo = split * CPW;
  uint64_t* out = lists + ((size_t)bg * nsplit + split) * K;
  if (c_lo >= nd) {
    for (int k = threadIdx.x; k < K; k += 256) out[k] = EMPTY_KEY;
    return;
  }
  // B operand: column col = part * G + h holds the hi (part 0) or lo (part 1)
  // bf16 half of query head h; other columns are zero.
  FT bq[KS];
  {
    const int col = lane & 15;
    const int h = col % G, part = col / G;
    const bool live = col < NPART * G;
    const QT* src = qs + ((size_t)b * Hq + g * G + h) * DH + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = live ? to_f<QT>(src[32 * ks + j]) : 0.f;
      if constexpr (HAS_LO) {
        const auto hi = pack8<T>(x);
        if (part == 1) {
          const u16x8 hb = __builtin_bit_cast(u16x8, hi);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = x[j] - bf2f(hb[j]);
        }
      }
      bq[ks] = pack8<T>(x);
    }
  }
  const T* kLg = kL + (size_t)bg * C * DH;
  const T* eg = e + (size_t)bg * C;
  // each wave: 4 steps of 16 chunks
#pragma unroll
  for (int st = 0; st < CPW / 64; ++st) {
    const int cb = c_lo + 64 * w + 16 * st;
    const int c = cb + (lane & 15);
    const int cl = c < nd ? c : nd - 1;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mma16(ld8<T>(kLg + (size_t)cl * DH + 8 * (lane >> 4) + 32 * ks), bq[ks], acc);
    // lane holds D[chunk 4*(lane/16)+i][col lane%16]: add hi + lo, max over heads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[i];
      if constexpr (HAS_LO) v += __shfl_xor(v, G, 64);
#pragma unroll
      for (int m = 1; m < G; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
      acc[i] = v;
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = cb + 4 * (lane >> 4) + i;
        sc_s[64 * w + 16 * st + 4 * (lane >> 4) + i] =
            cc < nd ? fmaf(acc[i], scale, to_f<T>(eg[cc])) : NEG_INF;
      }
    }
  }
  __syncthreads();
  // rank count: fewer than K better candidates -> slot = rank
  const int t = threadIdx.x;
  const float my = sc_s[t];
  const int myc = c_lo + t;
  if (t < K) out[t] = EMPTY_KEY;
  __syncthreads();
  if (my != NEG_INF) {
    int rank = 0;
    for (int j = 0; j < CPW; ++j) {
      const float o = sc_s[j];
      rank += (o > my) || (o == my && j < t);
    }
    if (rank < K) out[rank] = mkkey(my, myc);
  }
}

// ---------------------------------------------------------------- merge
__global__ __launch_bounds__(1024) void k_dec_merge(const uint64_t* __restrict__ lists,
                                                    int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ topk_out, int nsplit,
                                                    int K) {
  extern __shared__ uint64_t keys[];
  const int bg = blockIdx.x;
  const int n = nsplit * K;
  int P = 1;
  while (P < n) P <<= 1;
  const uint64_t* src = lists + (size_t)bg * n;
  for (int i = threadIdx.x; i < P; i += blockDim.x) keys[i] = i < n ? src[i] : EMPTY_KEY;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = keys[i], bb = keys[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < bb) : (a > bb)) {
            keys[i] = bb;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // top K in ascending chunk order
  __shared__ int ids[64];
  if (threadIdx.x < K) {
    const uint64_t kk = keys[threadIdx.x];
    ids[threadIdx.x] = kk == EMPTY_KEY ? 0x7FFFFFFF : (int)(~(uint32_t)(kk & 0xFFFFFFFFu));
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int me = ids[threadIdx.x];
    int r = 0;
    for (int j = 0; j < K; ++j) r += ids[j] < me;
    const int v = me == 0x7FFFFFFF ? -1 : me;
    // empties all sort last with equal ids; place them after the real ones
    int slot = r;
    if (me == 0x7FFFFFFF) {
      int before = 0;
      for (int j = 0; j < threadIdx.x; ++j) before += ids[j] == 0x7FFFFFFF;
      slot = r + before;
    }
    sel[(size_t)bg * K + slot] = v;
    if (topk_out != nullptr) topk_out[(size_t)bg * K + slot] = v;
  }
}

// ---------------------------------------------------------------- attention units
// Stage a 64-token V block transposed into vt[DH][64 + VPADD] (one wave).
template <typename T, int DH>
__device__ __forceinline__ void dec_stage_vt(const T* __restrict__ vsrc, int nvalid, T* vt, int lane) {
  const int tp = lane & 31, half = lane >> 5;
  const int t0 = 2 * tp, t1 = 2 * tp + 1;
  const T* r0 = vsrc + (size_t)(t0 < nvalid ? t0 : 0) * DH + half * (DH / 2);
  const T* r1 = vsrc + (size_t)(t1 < nvalid ? t1 : 0) * DH + half * (DH / 2);
  constexpr int VS = 64 + VPADD;
#pragma unroll
  for (int j = 0; j < DH / 2; j += 8) {
    const auto a = ld8<T>(r0 + j);
    const auto bb = ld8<T>(r1 + j);
    if constexpr (sizeof(T) == 2) {
      const u16x8 ua = __builtin_bit_cast(u16x8, a), ub = __builtin_bit_cast(u16x8, bb);
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2)
        *reinterpret_cast<uint32_t*>(vt + (half * (DH / 2) + j + e2) * VS + t0) =
            (uint32_t)ua[e2] | ((uint32_t)ub[e2] << 16);
    } else {
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        float2 pr;
        pr.x = a[e2];
        pr.y = bb[e2];
        *reinterpret_cast<float2*>(vt + (half * (DH / 2) + j + e2) * VS + t0) = pr;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type dec_ld_vt(const T* vt, int mb, int ks, int lane) {
  constexpr int VS = 64 + VPADD;
  const T* p = vt + (16 * mb + (lane & 15)) * VS + 32 * ks + 4 * (lane >> 4);
  if constexpr (sizeof(T) == 2) {
    const u16x4 a = *reinterpret_cast<const u16x4*>(p);
    const u16x4 bb = *reinterpret_cast<const u16x4*>(p + 16);
    u16x8 u;
    u[0] = a[0]; u[1] = a[1]; u[2] = a[2]; u[3] = a[3];
    u[4] = bb[0]; u[5] = bb[1]; u[6] = bb[2]; u[7] = bb[3];
    return __builtin_bit_cast(bf16x8, u);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(p + 16);
    f32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = bb[0]; r[5] = bb[1]; r[6] = bb[2]; r[7] = bb[3];
    return r;
  }
}

// partial layout per (bg, unit, head): [m, l, U[0..DH)]
template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_dec_attn(const T* __restrict__ q, const QT* __restrict__ qs,
                                                  const T* __restrict__ k, const T* __restrict__ v,
                                                  const T* __restrict__ kL, const T* __restrict__ e,
                                                  const int32_t* __restrict__ seq_len,
                                                  const int32_t* __restrict__ sel,
                                                  float* __restrict__ part, int N, int C, int Hkv,
                                                  int K, int W, int S, float scale, int units) {
  typedef typename Frag<T>::type FT;
  constexpr int KS = DH / 32, MB = DH / 16;
  constexpr int VS = 64 + VPADD;
  __shared__ __align__(16) T vt_s[4][DH * VS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + w;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  if (u >= units) return;
  const int n = seq_n(seq_len, b, N);
  const int i = n - 1;
  const int nd = n_distant(i, W, S);
  const int ws = nd * S;
  float* pout = part + ((size_t)bg * units + u) * G * (DH + 2);
  // what this unit covers
  int t0, cnt, chunk = -1;
  if (u < K) {
    chunk = sel[(size_t)bg * K + u];
    t0 = chunk * S;
    cnt = chunk >= 0 ? S : 0;
  } else {
    t0 = ws + 64 * (u - K);
    cnt = min(64, n - t0);
  }
  const int col = lane & 15;
  if (cnt <= 0) {
    if (col < G && (lane >> 4) == 0) {
      pout[col * (DH + 2)] = NEG_INF;
      pout[col * (DH + 2) + 1] = 0.f;
    }
    return;
  }
  // Q^T operand: column col = head col (raw query), zero beyond G
  FT qf[KS];
  {
    const int h = col < G ? col : 0;
    const T* src = q + ((size_t)b * Hq + g * G + h) * DH + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = col < G ? to_f<T>(src[32 * ks + j]) : 0.f;
      qf[ks] = pack8<T>(x);
    }
  }
  const T* kb = k + ((size_t)bg * N + t0) * DH;
  const T* vb = v + ((size_t)bg * N + t0) * DH;
  T* vt = vt_s[w];
  dec_stage_vt<T, DH>(vb, cnt, vt, lane);
  f32x4 sacc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    int tok = 16 * tb + (lane & 15);
    tok = tok < cnt ? tok : 0;
    sacc[tb] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sacc[tb] = mma16(ld8<T>(kb + (size_t)tok * DH + 8 * (lane >> 4) + 32 * ks), qf[ks], sacc[tb]);
  }
  float mx = NEG_INF;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int tok = 16 * tb + 4 * (lane >> 4) + ii;
      const float x = tok < cnt ? sacc[tb][ii] * scale : NEG_INF;
      sacc[tb][ii] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  float ls = 0.f;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float x = sacc[tb][ii];
      const float p = x == NEG_INF ? 0.f : __expf(x - mx);
      sacc[tb][ii] = p;
      ls += p;
    }
  ls += shfl_xor(ls, 16);
  ls += shfl_xor(ls, 32);
  wave_lds_sync();
  f32x4 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = zero4();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float x[8] = {sacc[2 * ks][0], sacc[2 * ks][1], sacc[2 * ks][2], sacc[2 * ks][3],
                  sacc[2 * ks + 1][0], sacc[2 * ks + 1][1], sacc[2 * ks + 1][2], sacc[2 * ks + 1][3]};
    const FT pf = pack8<T>(x);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb] = mma16(dec_ld_vt<T>(vt, mb, ks, lane), pf, oacc[mb]);
  }
  if (col < G) {
    float* ph = pout + col * (DH + 2);
    float mval = mx, lval = ls, coef = 1.f;
    if (chunk >= 0) {
      // a selected chunk enters the fusion as one term: log-weight s_c,
      // weight 1, vector O_c
      const QT* qh = qs + ((size_t)b * Hq + g * G + col) * DH;
      const T* kr = kL + ((size_t)bg * C + chunk) * DH;
      float s = 0.f;
      for (int dd = 0; dd < DH; ++dd) s = fmaf(to_f<QT>(qh[dd]), to_f<T>(kr[dd]), s);
      mval = fmaf(s, scale, to_f<T>(e[(size_t)bg * C + chunk]));
      lval = 1.f;
      coef = 1.f / ls;
    }
    if ((lane >> 4) == 0) {
      ph[0] = mval;
      ph[1] = lval;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) ph[2 + 16 * mb + 4 * (lane >> 4) + ii] = oacc[mb][ii] * coef;
  }
}

// ---------------------------------------------------------------- combine
template <typename T, int DH>
__global__ __launch_bounds__(64) void k_dec_combine(const float* __restrict__ part, T* __restrict__ o,
                                                    float* __restrict__ lse, int Hkv, int G,
                                                    int units) {
  const int bh = blockIdx.x;  // b * Hq + h
  const int Hq = Hkv * G;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / G, hh = h - g * G;
  const int bg = b * Hkv + g;
  const int lane = threadIdx.x;
  float M = NEG_INF;
  for (int u = 0; u < units; ++u) M = fmaxf(M, part[(((size_t)bg * units + u) * G + hh) * (DH + 2)]);
  float Z = 0.f;
  float acc[DH / 64];
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) acc[j] = 0.f;
  for (int u = 0; u < units; ++u) {
    const float* p = part + (((size_t)bg * units + u) * G + hh) * (DH + 2);
    const float m = p[0];
    if (m == NEG_INF) continue;
    const float wgt = __expf(m - M);
    Z += wgt * p[1];
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) acc[j] += wgt * p[2 + lane + 64 * j];
  }
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) o[(size_t)bh * DH + lane + 64 * j] = from_f<T>(acc[j] / Z);
  if (lane == 0) lse[bh] = M + __logf(Z);
}

// ---------------------------------------------------------------- host side
namespace {
struct DecWs {
  float* qhat;
  uint64_t* lists;
  int32_t* sel;
  float* part;
  int nsplit, units;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t carve(const Dims& p, void* base, DecWs* w) {
  char* c = static_cast<char*>(base);
  size_t off = 0;
  w->nsplit = std::max(1, (p.C + CPW - 1) / CPW);
  w->units = p.K + (p.W + p.S - 1 + 63) / 64 + 1;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + off : nullptr;
    off += up256(bytes);
    return ptr;
  };
  w->qhat = (float*)take(p.r > 0 ? (size_t)p.B * p.Hq * p.d * sizeof(float) : 0);
  w->lists = (uint64_t*)take((size_t)p.B * p.Hkv * w->nsplit * p.K * sizeof(uint64_t));
  w->sel = (int32_t*)take((size_t)p.B * p.Hkv * p.K * sizeof(int32_t));
  w->part = (float*)take((size_t)p.B * p.Hkv * w->units * p.G * (p.d + 2) * sizeof(float));
  return off;
}
}  // namespace

size_t decode_workspace(const Dims& p) {
  DecWs w;
  const size_t s = carve(p, nullptr, &w);
  if ((size_t)w.nsplit * p.K > 8192) return (size_t)-1;  // merge sort capacity
  return s;
}

template <typename T, typename QT, int G, int DH>
static hipError_t dec_go(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                         const int32_t* seq_len, const void* kL, const void* e, void* o, float* lse,
                         int32_t* topk_idx, const DecWs& w, hipStream_t st) {
  hipLaunchKernelGGL((k_dec_scan<T, QT, G, DH>), dim3(w.nsplit, p.B * p.Hkv), dim3(256), 0, st,
                     (const QT*)qs, (const T*)kL, (const T*)e, seq_len, w.lists, p.N, p.C, p.Hkv,
                     p.K, p.W, p.S, p.scale, w.nsplit);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int P = 1;
  while (P < w.nsplit * p.K) P <<= 1;
  const size_t lds = (size_t)P * sizeof(uint64_t);
  if (lds > 64 * 1024) {
    err = hipFuncSetAttribute((const void*)k_dec_merge, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_dec_merge, dim3(p.B * p.Hkv), dim3(1024), lds, st, w.lists, w.sel, topk_idx,
                     w.nsplit, p.K);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_attn<T, QT, G, DH>), dim3((w.units + 3) / 4, p.B * p.Hkv), dim3(256), 0,
                     st, (const T*)q, (const QT*)qs, (const T*)k, (const T*)v, (const T*)kL,
                     (const T*)e, seq_len, w.sel, w.part, p.N, p.C, p.Hkv, p.K, p.W, p.S, p.scale,
                     w.units);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_combine<T, DH>), dim3(p.B * p.Hq), dim3(64), 0, st, w.part, (T*)o, lse,
                     p.Hkv, G, w.units);
  return hipGetLastError();
}

template <typename T, typename QT, int G>
static hipError_t dec_d(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const void* kL, const void* e, void* o, float* lse,
                        int32_t* idx, const DecWs& w, hipStream_t st) {
  if (p.d == 64) return dec_go<T, QT, G, 64>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
  return dec_go<T, QT, G, 128>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
}

template <typename T, typename QT>
static hipError_t dec_g(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const void* kL, const void* e, void* o, float* lse,
                        int32_t* idx, const DecWs& w, hipStream_t st) {
  switch (p.G) {
    case 1: return dec_d<T, QT, 1>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 2: return dec_d<T, QT, 2>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 4: return dec_d<T, QT, 4>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 8: return dec_d<T, QT, 8>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Dims& p, const void* qs, bool q_is_f32, const void* q, const void* k,
                         const void* v, const int32_t* seq_len, const void* kL, const void* e,
                         void* o, float* lse, int32_t* topk_idx, void* ws, hipStream_t st) {
  DecWs w;
  carve(p, ws, &w);
  if (p.dtype == 1) {
    if (q_is_f32) return dec_g<uint16_t, float>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
    return dec_g<uint16_t, uint16_t>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
  }
  return dec_g<float, float>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
}

}  // namespace hils
