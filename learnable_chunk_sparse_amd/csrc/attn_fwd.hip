// HiLS prefill forward: sliding-window attention, attention inside each
// selected chunk, and the hierarchical fusion, in one kernel per query tile.
//
// Paper: Fig. 3 (inter-chunk softmax gives each chunk its mass, intra-chunk
// softmax spreads it over the chunk's tokens), the engineersofai abstract
// (each query attends to each retrieved chunk independently; the outputs are
// fused by the retrieval scores), "Limitations of Naive Sparse Attention"
// (local sliding window plus top-K distant chunks). For query row (h, i):
//   O_W, lse_W : exact causal softmax attention over the window [n_dist*S, i]
//   O_c, lse_c : exact softmax attention over the S tokens of chunk c in T(i)
//   L = log(sum_{c in T} exp(s_c) + exp(lse_W))
//   o = sum_{c in T} exp(s_c - L) O_c + exp(lse_W - L) O_W
//
// Tile: R = 64 * CB rows = TP positions x G heads of one (batch, KV head),
// 4 waves. Products use the transposed form S^T = K Q^T (tokens x rows) so
// that the probabilities land in registers exactly where the P^T operand of
// O^T = V^T P^T needs them (the token order inside each 32-token step is
// permuted identically on both operands; V is staged transposed in LDS).
//   Phase A (window): wave w runs a banded flash attention over its own
//     16*CB rows; the fusion normaliser L follows from lse_W and the
//     selected scores, and exp(lse_W - L) O_W seeds an fp32 row accumulator
//     in LDS.
//   Phase B (chunks): the tile's (position, slot) selections are bucketed by
//     chunk id (counting sort in LDS) and cut into groups of up to 16/G
//     positions x G heads sharing one chunk; each group is one 64-token block
//     of MFMA work, and exp(s_c - L) O_c is added to the rows' accumulators
//     with LDS atomics. Compaction keeps MFMA columns busy even when adjacent
//     queries pick different chunks.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>

namespace hils {

constexpr int VPAD = 8;  // Vt row padding (elements)

// In-place exclusive scan of a[0..n) by the whole block; returns the total.
__device__ int block_excl_scan(int* a, int n, int* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int seg = (n + 255) / 256;
  const int lo = min(n, t * seg), hi = min(n, lo + seg);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  int v = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int base = v - s;
  for (int j = 0; j < w; ++j) base += wsum[j];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  for (int i = lo; i < hi; ++i) {
    const int x = a[i];
    a[i] = base;
    base += x;
  }
  __syncthreads();
  return total;
}

// Stage a 64-token block of V ([64][DH] rows starting at vsrc, row stride DH)
// transposed into vt[DH][64 + VPAD]. One wave. Tokens >= nvalid read row 0.
template <typename T, int DH>
__device__ __forceinline__ void stage_vt(const T* __restrict__ vsrc, int nvalid, T* vt, int lane) {
  const int tp = lane & 31, half = lane >> 5;
  const int t0 = 2 * tp, t1 = 2 * tp + 1;
  const T* r0 = vsrc + (size_t)(t0 < nvalid ? t0 : 0) * DH + half * (DH / 2);
  const T* r1 = vsrc + (size_t)(t1 < nvalid ? t1 : 0) * DH + half * (DH / 2);
  constexpr int VS = 64 + VPAD;
#pragma unroll
  for (int j = 0; j < DH / 2; j += 8) {
    const auto a = ld8<T>(r0 + j);
    const auto b = ld8<T>(r1 + j);
    if constexpr (sizeof(T) == 2) {
      const u16x8 ua = __builtin_bit_cast(u16x8, a), ub = __builtin_bit_cast(u16x8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = half * (DH / 2) + j + e;
        *reinterpret_cast<uint32_t*>(vt + dd * VS + t0) = (uint32_t)ua[e] | ((uint32_t)ub[e] << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = half * (DH / 2) + j + e;
        float2 pr;
        pr.x = a[e];
        pr.y = b[e];
        *reinterpret_cast<float2*>(vt + dd * VS + t0) = pr;
      }
    }
  }
}

// V^T fragment (A operand of O^T = V^T P^T): rows d = 16*mb + lane%16, the 8
// tokens {4g..4g+3, 16+4g..16+4g+3} (+32*ks), g = lane/16.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type ld_vt(const T* vt, int mb, int ks, int lane) {
  constexpr int VS = 64 + VPAD;
  const T* p = vt + (16 * mb + (lane & 15)) * VS + 32 * ks + 4 * (lane >> 4);
  if constexpr (sizeof(T) == 2) {
    const u16x4 a = *reinterpret_cast<const u16x4*>(p);
    const u16x4 b = *reinterpret_cast<const u16x4*>(p + 16);
    u16x8 u;
    u[0] = a[0]; u[1] = a[1]; u[2] = a[2]; u[3] = a[3];
    u[4] = b[0]; u[5] = b[1]; u[6] = b[2]; u[7] = b[3];
    return __builtin_bit_cast(bf16x8, u);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
    f32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
  }
}

// P^T fragment (B operand) for token step ks from the S^T accumulators.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type p_frag(const f32x4& s0, const f32x4& s1) {
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  return pack8<T>(x);
}

template <typename T, int G, int DH, int CB>
__global__ __launch_bounds__(256) void k_attn_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v,
                                                  const int32_t* __restrict__ topk_idx,
                                                  const float* __restrict__ topk_score,
                                                  T* __restrict__ o, float* __restrict__ lse,
                                                  int N, int Hkv, int K, int W, int S, float scale,
                                                  int ntiles, int C) {
  typedef typename Frag<T>::type FT;
  constexpr int R = 64 * CB;        // rows per tile
  constexpr int TP = R / G;         // positions per tile
  constexpr int PPG = 16 / G;       // positions per chunk group
  constexpr int KS = DH / 32;
  constexpr int MB = DH / 16;
  constexpr int AS = R + 4;         // accT row stride
  constexpr int VS = 64 + VPAD;
  constexpr int EPT = TP * 32 / 256;  // max entries per thread (K <= 32)

  extern __shared__ __align__(16) unsigned char smem[];
  float* accT = reinterpret_cast<float*>(smem);                 // [DH][AS]
  float* Ls = accT + DH * AS;                                   // [R]
  T* vtb = reinterpret_cast<T*>(Ls + R);                        // [4][DH][VS]
  int* off = reinterpret_cast<int*>(vtb + 4 * DH * VS);         // [C] counts, then offsets
  int* gb = off + C;                                            // [C] group counts, then bases
  int* grp = gb + C;                                            // [2 * NGMAX]
  const int NGMAX = min(TP * K, TP * K / PPG + C + 1);
  uint16_t* ent = reinterpret_cast<uint16_t*>(grp + 2 * NGMAX);  // [TP*K]
  __shared__ int wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tile = ntiles - 1 - blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * TP;
  const int plast = min(p0 + TP - 1, N - 1);
  const int ndmax = n_distant(plast, W, S);  // chunks any row of the tile can select
  const T* kg = k + (size_t)bg * N * DH;
  const T* vg = v + (size_t)bg * N * DH;
  T* vt = vtb + w * DH * VS;

  // ------------------------------------------------ bucket selections by chunk
  for (int x = tid; x < ndmax; x += 256) off[x] = 0;
  __syncthreads();
  int my_c[EPT], my_r[EPT];
  const int E = TP * K;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int x = tid + 256 * j;
    my_c[j] = -1;
    my_r[j] = 0;
    if (x < E) {
      const int pl = x / K, kk = x - pl * K;
      const int pos = p0 + pl;
      const int c = pos < N ? topk_idx[((size_t)bg * N + pos) * K + kk] : -1;
      if (c >= 0 && c < ndmax) {
        my_c[j] = c;
        my_r[j] = atomicAdd(&off[c], 1);
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < ndmax; x += 256) gb[x] = (off[x] + PPG - 1) / PPG;
  __syncthreads();
  const int Etot = block_excl_scan(off, ndmax, wsum);
  const int NG = block_excl_scan(gb, ndmax, wsum);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int c = my_c[j];
    if (c >= 0) {
      const int x = tid + 256 * j;
      const int pl = x / K, kk = x - pl * K;
      const int r = my_r[j];
      ent[off[c] + r] = (uint16_t)((pl << 6) | kk);
      if (r % PPG == 0) {
        const int gi = gb[c] + r / PPG;
        const int n = (c + 1 < ndmax ? off[c + 1] : Etot) - off[c] - r;
        grp[2 * gi] = c;
        grp[2 * gi + 1] = ((off[c] + r) << 5) | (n < PPG ? n : PPG);
      }
    }
  }

  // ------------------------------------------------ phase A: window
  {
    const int rbase = w * 16 * CB;                 // first tile row of this wave
    const int pw_lo = p0 + rbase / G;
    const int pw_hi = min(p0 + (rbase + 16 * CB - 1) / G, N - 1);
    FT qf[CB][KS];
    int prow[CB], wsr[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r = rbase + 16 * cb + (lane & 15);
      const int pos = p0 + r / G, hh = r % G;
      prow[cb] = pos < N ? pos : -1;
      wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
      const int pc = pos < N ? pos : N - 1;
      const T* src = q + (((size_t)b * Hq + g * G + hh) * N + pc) * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = ld8<T>(src + 32 * ks);
    }
    float m[CB], lsum[CB];
    f32x4 oacc[MB][CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      m[cb] = NEG_INF;
      lsum[cb] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] = zero4();
    }
    if (pw_lo < N) {
      const int kv_lo = n_distant(pw_lo, W, S) * S;
      for (int kv0 = kv_lo; kv0 <= pw_hi; kv0 += 64) {
        const int nvalid = min(64, N - kv0);
        f32x4 sacc[4][CB];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          int tok = 16 * tb + (lane & 15);
          tok = tok < nvalid ? tok : 0;
          const T* src = kg + (size_t)(kv0 + tok) * DH + 8 * (lane >> 4);
          FT kf[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kf[ks] = ld8<T>(src + 32 * ks);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            sacc[tb][cb] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[tb][cb] = mma16(kf[ks], qf[cb][ks], sacc[tb][cb]);
          }
        }
        wave_lds_sync();  // previous block's V^T reads are complete
        stage_vt<T, DH>(vg + (size_t)kv0 * DH, nvalid, vt, lane);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          float bmax = NEG_INF;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = kv0 + 16 * tb + 4 * (lane >> 4) + i;
              const bool ok = prow[cb] >= 0 && j <= prow[cb] && j >= wsr[cb];
              const float x = ok ? sacc[tb][cb][i] * scale : NEG_INF;
              sacc[tb][cb][i] = x;
              bmax = fmaxf(bmax, x);
            }
          bmax = fmaxf(bmax, shfl_xor(bmax, 16));
          bmax = fmaxf(bmax, shfl_xor(bmax, 32));
          const float mnew = fmaxf(m[cb], bmax);
          const float alpha = (m[cb] == NEG_INF) ? 0.f : __expf(m[cb] - mnew);
          float ps = 0.f;
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = sacc[tb][cb][i];
              const float pv = (x == NEG_INF) ? 0.f : __expf(x - mnew);
              sacc[tb][cb][i] = pv;
              ps += pv;
            }
          lsum[cb] = lsum[cb] * alpha + ps;
          m[cb] = mnew;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= alpha;
        }
        wave_lds_sync();  // V^T staged
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          FT pf[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) pf[cb] = p_frag<T>(sacc[2 * ks][cb], sacc[2 * ks + 1][cb]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const FT vf = ld_vt<T>(vt, mb, ks, lane);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[mb][cb] = mma16(vf, pf[cb], oacc[mb][cb]);
          }
        }
      }
    }
    // window log-sum-exp, fusion normaliser, window contribution
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float ls = lsum[cb];
      ls += shfl_xor(ls, 16);
      ls += shfl_xor(ls, 32);
      const int r = rbase + 16 * cb + (lane & 15);
      float L = 0.f, coef = 0.f;
      if (prow[cb] >= 0) {
        const float lW = m[cb] + __logf(ls);
        const int hh = r % G;
        const size_t rowoff = ((size_t)b * Hq + g * G + hh) * N + prow[cb];
        const int32_t* ti = topk_idx + ((size_t)bg * N + prow[cb]) * K;
        const float* ts = topk_score + rowoff * K;
        float mx = lW;
        for (int kk = 0; kk < K; ++kk)
          if (ti[kk] >= 0) mx = fmaxf(mx, ts[kk]);
        float tot = __expf(lW - mx);
        for (int kk = 0; kk < K; ++kk)
          if (ti[kk] >= 0) tot += __expf(ts[kk] - mx);
        L = mx + __logf(tot);
        coef = __expf(m[cb] - L);
        if ((lane >> 4) == 0) lse[rowoff] = L;
      }
      if ((lane >> 4) == 0) Ls[r] = L;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) accT[(16 * mb + 4 * (lane >> 4) + i) * AS + r] = oacc[mb][cb][i] * coef;
    }
  }
  __syncthreads();

  // ------------------------------------------------ phase B: selected chunks
  for (int gi = w; gi < NG; gi += 4) {
    const int c = grp[2 * gi];
    const int gdesc = grp[2 * gi + 1];
    const int st = gdesc >> 5, n = gdesc & 31;
    const int col = lane & 15;
    const int ei = col / G, hh = col % G;
    const bool valid = ei < n;
    const int en = ent[st + (valid ? ei : 0)];
    const int pl = en >> 6, kk = en & 63;
    const int pos = p0 + pl;
    const int row = pl * G + hh;
    const size_t rowoff = ((size_t)b * Hq + g * G + hh) * N + pos;
    FT qf[KS];
    {
      const T* src = q + rowoff * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = ld8<T>(src + 32 * ks);
    }
    const T* kc = kg + (size_t)c * 64 * DH;
    f32x4 sacc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const T* src = kc + (size_t)(16 * tb + (lane & 15)) * DH + 8 * (lane >> 4);
      sacc[tb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[tb] = mma16(ld8<T>(src + 32 * ks), qf[ks], sacc[tb]);
    }
    wave_lds_sync();
    stage_vt<T, DH>(vg + (size_t)c * 64 * DH, 64, vt, lane);
    float mx = NEG_INF;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sacc[tb][i] *= scale;
        mx = fmaxf(mx, sacc[tb][i]);
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    float ps = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __expf(sacc[tb][i] - mx);
        sacc[tb][i] = pv;
        ps += pv;
      }
    ps += shfl_xor(ps, 16);
    ps += shfl_xor(ps, 32);
    wave_lds_sync();
    f32x4 oc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oc[mb] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const FT pf = p_frag<T>(sacc[2 * ks], sacc[2 * ks + 1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oc[mb] = mma16(ld_vt<T>(vt, mb, ks, lane), pf, oc[mb]);
    }
    if (valid) {
      const float s = topk_score[rowoff * K + kk];
      const float alpha = __expf(s - Ls[row]) / ps;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          atomicAdd(&accT[(16 * mb + 4 * (lane >> 4) + i) * AS + row], alpha * oc[mb][i]);
    }
  }
  __syncthreads();

  // ------------------------------------------------ write o
  for (int x = tid; x < R * DH; x += 256) {
    const int dd = x % DH, r = x / DH;
    const int pos = p0 + r / G, hh = r % G;
    if (pos < N) o[(((size_t)b * Hq + g * G + hh) * N + pos) * DH + dd] = from_f<T>(accT[dd * AS + r]);
  }
}

template <typename T, int G, int DH, int CB>
static size_t fwd_lds(const Dims& p) {
  constexpr int R = 64 * CB, TP = R / G, PPG = 16 / G;
  const int ngmax = std::min(TP * p.K, TP * p.K / PPG + p.C + 1);
  size_t s = sizeof(float) * ((size_t)DH * (R + 4) + R);
  s += sizeof(T) * 4 * DH * (64 + VPAD);
  s += sizeof(int) * (2 * (size_t)p.C + 2 * (size_t)ngmax);
  s += sizeof(uint16_t) * (size_t)TP * p.K;
  return (s + 15) & ~(size_t)15;
}

template <typename T, int G, int DH, int CB>
static hipError_t fwd_go(const Dims& p, const void* q, const void* k, const void* v,
                         const int32_t* idx, const float* sc, void* o, float* lse, hipStream_t st) {
  constexpr int TP = 64 * CB / G;
  const int ntiles = (p.N + TP - 1) / TP;
  const size_t lds = fwd_lds<T, G, DH, CB>(p);
  auto kern = k_attn_fwd<T, G, DH, CB>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), lds, st, (const T*)q, (const T*)k,
                     (const T*)v, idx, sc, (T*)o, lse, p.N, p.Hkv, p.K, p.W, p.S, p.scale, ntiles,
                     p.C);
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t fwd_d(const Dims& p, const void* q, const void* k, const void* v, const int32_t* idx,
                        const float* sc, void* o, float* lse, hipStream_t st) {
  constexpr int CB = sizeof(T) == 2 ? 2 : 1;
  if (p.d == 64) return fwd_go<T, G, 64, CB>(p, q, k, v, idx, sc, o, lse, st);
  return fwd_go<T, G, 128, CB>(p, q, k, v, idx, sc, o, lse, st);
}

template <typename T>
static hipError_t fwd_g(const Dims& p, const void* q, const void* k, const void* v, const int32_t* idx,
                        const float* sc, void* o, float* lse, hipStream_t st) {
  switch (p.G) {
    case 1: return fwd_d<T, 1>(p, q, k, v, idx, sc, o, lse, st);
    case 2: return fwd_d<T, 2>(p, q, k, v, idx, sc, o, lse, st);
    case 4: return fwd_d<T, 4>(p, q, k, v, idx, sc, o, lse, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int CB>
static size_t lds_by_g(const Dims& p) {
  switch (p.G) {
    case 1: return p.d == 64 ? fwd_lds<T, 1, 64, CB>(p) : fwd_lds<T, 1, 128, CB>(p);
    case 2: return p.d == 64 ? fwd_lds<T, 2, 64, CB>(p) : fwd_lds<T, 2, 128, CB>(p);
    case 4: return p.d == 64 ? fwd_lds<T, 4, 64, CB>(p) : fwd_lds<T, 4, 128, CB>(p);
    default: return (size_t)-1;
  }
}

size_t attn_fwd_lds_bytes(const Dims& p) {
  // dynamic LDS plus the kernel's static scan scratch
  const size_t stat = 64;
  if (p.dtype == 1) return lds_by_g<uint16_t, 2>(p) + stat;
  return lds_by_g<float, 1>(p) + stat;
}

hipError_t launch_attn_fwd(const Dims& p, const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, const float* topk_score, void* o, float* lse,
                           hipStream_t st) {
  if (p.dtype == 1) return fwd_g<uint16_t>(p, q, k, v, topk_idx, topk_score, o, lse, st);
  return fwd_g<float>(p, q, k, v, topk_idx, topk_score, o, lse, st);
}

}  // namespace hils
