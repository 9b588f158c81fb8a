// Landmark summary of the complete chunks and its backward (paperglide, "The
// HiLS-Attention Mechanism", the landmark worked example: the landmark query
// of a chunk scores the chunk's tokens, the softmax of those scores weights
// the keys into the chunk's summary key, and the entropy of the weights is
// the chunk's bias; the overview derives the pair as the first-order Taylor
// expansion of the chunk's attention mass around the landmark query).
//
//   forward   s_t = scale qL . k_t,  p = softmax(s) over the chunk's S tokens,
//             kL = sum_t p_t k_t,   e = -sum_t p_t log p_t = log Z - sum_t p_t s_t
//   backward  (chain rule; dkL, de given) with sbar = sum_t p_t s_t:
//             ds_t = p_t (dkL . k_t - dkL . kL - de (s_t - sbar))
//             dqL  = scale sum_t ds_t k_t
//             dk_t += scale ds_t qL + p_t dkL
//
// One wave per (b, kv head, chunk). The forward keeps the chunk's keys in
// registers (layout below). The backward runs up to four independent waves per
// workgroup (as many as keep the workgroup's LDS under 48 KB); the chunk's 64
// keys are staged in LDS in their own type (bf16 keys stay bf16: half the
// LDS, twice the resident waves), rows padded so that lane t reading row t
// (scores, dkL . k_t) and lane j reading column j (the key-weighted sums) are
// both free of bank conflicts (bf16: pitch DH + 2, an odd number of words;
// fp32: DH + 1). Lane t owns token t for the scores and the softmax (wave
// reductions); lane j owns dims j and j + 64 for the sums over tokens. All
// arithmetic is fp32.
#include "hils_common.h"
#include "hils_internal.h"

namespace hils {

namespace {
constexpr int LS = 64;  // chunk size (tokens per chunk)

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// LDS row pitch of the staged keys (elements)
template <typename T, int DH>
constexpr int kpitch() { return sizeof(T) == 2 ? DH + 2 : DH + 1; }
// waves (chunks) per workgroup
template <typename T, int DH>
constexpr int lm_waves() {
  constexpr int per = LS * kpitch<T, DH>() * (int)sizeof(T) + (2 * DH + 2 * LS) * 4;
  return per * 4 <= 48 * 1024 ? 4 : per * 2 <= 48 * 1024 ? 2 : 1;
}

// the chunk's keys -> kf[t][j] (pitch kpitch); 16-byte loads
template <typename T, int DH>
__device__ __forceinline__ void stage_keys(const T* __restrict__ kc, T* kf, int lane) {
  constexpr int V = 16 / sizeof(T), PER = LS * DH / (64 * V), P = kpitch<T, DH>();
  // all loads first, then the LDS stores
  T v[PER][V];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int x = (it * 64 + lane) * V;
    if constexpr (sizeof(T) == 2) {
      const u16x8 a = *reinterpret_cast<const u16x8*>(kc + x);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[it][i] = a[i];
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(kc + x);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[it][i] = a[i];
    }
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int x = (it * 64 + lane) * V;
    const int t = x / DH, j = x - t * DH;
    if constexpr (sizeof(T) == 2) {
      // j is a multiple of 8 and the pitch even: 4-byte aligned pairs
#pragma unroll
      for (int i = 0; i < 8; i += 2)
        *reinterpret_cast<uint32_t*>(kf + t * P + j + i) = (uint32_t)v[it][i] | ((uint32_t)v[it][i + 1] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[t * P + j + i] = v[it][i];
    }
  }
}

// scores, softmax weights (to LDS) and the chunk statistics of one chunk
struct ChunkSoftmax {
  float s, p;   // this lane's token
  float logZ;   // log sum_t exp(s_t)
  float sbar;   // sum_t p_t s_t
};
template <typename T, int DH>
__device__ __forceinline__ ChunkSoftmax chunk_softmax(const T* kf, const float* qs, float* ps,
                                                      float scale, int lane) {
  float acc = 0.f;
  const T* kr = kf + lane * kpitch<T, DH>();
#pragma unroll 16
  for (int j = 0; j < DH; ++j) acc = fmaf(qs[j], to_f<T>(kr[j]), acc);
  ChunkSoftmax r;
  r.s = acc * scale;
  const float m = wave_max(r.s);
  const float ex = expf(r.s - m);
  const float Z = wave_sum(ex);
  r.p = ex / Z;
  r.logZ = m + logf(Z);
  r.sbar = wave_sum(r.p * r.s);
  ps[lane] = r.p;
  return r;
}
}  // namespace

// Forward in registers: lane l holds the 16-byte slices l, l + 64, ... of the
// chunk's key block (token tl + TPI it, dims part V .. part V + V - 1 with
// part = l % LPT, tl = l / LPT), so each load round reads 1 KB contiguously.
// Scores: partial dots (bf16: two-element dot instructions on the raw
// words, products exact in fp32) reduced over the LPT lanes of a token;
// softmax statistics and the weighted key sums: reduced over the TPI token
// groups. One wave per chunk, four chunks per workgroup, no LDS (more chunks
// per wave, or a loop with the next chunk's loads in flight, measured slower).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_landmark_fwd(const T* __restrict__ qL, const T* __restrict__ k,
                                                     T* __restrict__ kL, T* __restrict__ e,
                                                     float* __restrict__ kL32, float* __restrict__ e32,
                                                     int N, int C, float scale) {
  constexpr int V = 16 / (int)sizeof(T);  // elements per 16-byte slice
  constexpr int LPT = DH / V;             // lanes per token row
  constexpr int TPI = 64 / LPT;           // tokens per load round
  constexpr int PER = LS / TPI;           // load rounds
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + w, bg = blockIdx.y;
  if (c >= C) return;  // whole waves; the waves share no data
  const int part = lane % LPT, tl = lane / LPT;
  const size_t cr = (size_t)bg * C + c;  // (b, kv head, chunk)
  const T* kc = k + ((size_t)bg * N + (size_t)c * LS) * DH + (size_t)tl * DH + part * V;
  u32x4 raw[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) raw[it] = *reinterpret_cast<const u32x4*>(kc + (size_t)it * TPI * DH);
  const u32x4 rq = *reinterpret_cast<const u32x4*>(qL + cr * DH + part * V);
  auto key = [&](int it, int i) __attribute__((always_inline)) -> float {
    T tk[V];
    __builtin_memcpy(tk, &raw[it], 16);
    return to_f<T>(tk[i]);
  };
  float sc[PER];
  float mx = NEG_INF;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    float a = 0.f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (copies: a bit cast of a vector component would read component 0)
        const uint32_t qi = rq[i], ki = raw[it][i];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qi),
                                            __builtin_bit_cast(bf16x2_t, ki), a, false);
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) a = fmaf(__uint_as_float(rq[i]), key(it, i), a);
    }
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) a += __shfl_xor(a, m, 64);
    sc[it] = a * scale;
    mx = fmaxf(mx, sc[it]);
  }
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  float ex[PER], Z = 0.f;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    ex[it] = expf(sc[it] - mx);
    Z += ex[it];
  }
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1) Z += __shfl_xor(Z, m, 64);
  const float rz = 1.f / Z;
  float acc[V], sbar = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const float p = ex[it] * rz;
    sbar = fmaf(p, sc[it], sbar);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(p, key(it, i), acc[i]);
  }
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1) {
    sbar += __shfl_xor(sbar, m, 64);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += __shfl_xor(acc[i], m, 64);
  }
  if (tl == 0) {
    T o[V];
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] = from_f<T>(acc[i]);
    u32x4 ov;
    __builtin_memcpy(&ov, o, 16);
    *reinterpret_cast<u32x4*>(kL + cr * DH + part * V) = ov;
    if (kL32 != nullptr) {
#pragma unroll
      for (int i = 0; i < V; i += 4)
        *reinterpret_cast<f32x4*>(kL32 + cr * DH + part * V + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
    }
    if (lane == 0) {
      const float ent = mx + logf(Z) - sbar;
      e[cr] = from_f<T>(ent);
      if (e32 != nullptr) e32[cr] = ent;
    }
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_landmark_bwd(const T* __restrict__ qL, const T* __restrict__ k,
                                                     const float* __restrict__ dkL,
                                                     const float* __restrict__ de,
                                                     float* __restrict__ dqL, float* __restrict__ dk,
                                                     int N, int C, float scale) {
  constexpr int P = kpitch<T, DH>(), WB = lm_waves<T, DH>();
  __shared__ __align__(16) T kf_all[WB][LS * P];
  __shared__ float qs_all[WB][DH], gs_all[WB][DH], ps_all[WB][LS], dss_all[WB][LS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * WB + w, bg = blockIdx.y;
  if (c >= C) return;  // whole waves; the waves share no data
  T* kf = kf_all[w];
  float *qs = qs_all[w], *gs = gs_all[w], *ps = ps_all[w], *dss = dss_all[w];
  const size_t cr = (size_t)bg * C + c;
  const size_t t0 = (size_t)bg * N + (size_t)c * LS;  // first token row of the chunk
  stage_keys<T, DH>(k + t0 * DH, kf, lane);
  for (int j = lane; j < DH; j += 64) {
    qs[j] = to_f<T>(qL[cr * DH + j]);
    gs[j] = dkL[cr * DH + j];
  }
  const float dev = de[cr];
  wave_lds_sync();
  const ChunkSoftmax r = chunk_softmax<T, DH>(kf, qs, ps, scale, lane);
  wave_lds_sync();
  // dkL . kL with kL = sum_t p_t k_t (lane j: its dims)
  float gk = 0.f;
#pragma unroll
  for (int j = lane; j < DH; j += 64) {
    float a = 0.f;
#pragma unroll 16
    for (int t = 0; t < LS; ++t) a = fmaf(ps[t], to_f<T>(kf[t * P + j]), a);
    gk = fmaf(gs[j], a, gk);
  }
  gk = wave_sum(gk);
  // ds_t (lane t)
  {
    float g = 0.f;
    const T* kr = kf + lane * P;
#pragma unroll 16
    for (int j = 0; j < DH; ++j) g = fmaf(gs[j], to_f<T>(kr[j]), g);
    dss[lane] = r.p * (g - gk - dev * (r.s - r.sbar));
  }
  wave_lds_sync();
#pragma unroll
  for (int j = lane; j < DH; j += 64) {
    float a = 0.f;
#pragma unroll 16
    for (int t = 0; t < LS; ++t) a = fmaf(dss[t], to_f<T>(kf[t * P + j]), a);
    dqL[cr * DH + j] = a * scale;
    const float qj = qs[j] * scale, gj = gs[j];
    float* dkc = dk + t0 * DH + j;
#pragma unroll 8
    for (int t = 0; t < LS; ++t) dkc[(size_t)t * DH] += fmaf(dss[t], qj, ps[t] * gj);
  }
}

namespace {
template <typename T, int DH>
hipError_t lm_go(const Dims& p, bool bwd, const void* qL, const void* k, void* kL, void* e,
                 float* kL32, float* e32, const float* dkL, const float* de, float* dqL, float* dk,
                 hipStream_t st) {
  constexpr int WB = lm_waves<T, DH>();
  const dim3 grid((unsigned)((p.C + WB - 1) / WB), (unsigned)(p.B * p.Hkv));
  if (!bwd) {
    hipLaunchKernelGGL((k_landmark_fwd<T, DH>), dim3((unsigned)((p.C + 3) / 4), (unsigned)(p.B * p.Hkv)),
                       dim3(256), 0, st, (const T*)qL, (const T*)k, (T*)kL, (T*)e, kL32, e32, p.N,
                       p.C, p.scale);
  } else {
    hipLaunchKernelGGL((k_landmark_bwd<T, DH>), grid, dim3(64 * WB), 0, st, (const T*)qL, (const T*)k,
                       dkL, de, dqL, dk, p.N, p.C, p.scale);
  }
  return hipGetLastError();
}

hipError_t lm_dispatch(const Dims& p, bool bwd, const void* qL, const void* k, void* kL, void* e,
                       float* kL32, float* e32, const float* dkL, const float* de, float* dqL,
                       float* dk, hipStream_t st) {
  if (p.C <= 0) return hipSuccess;
  if (p.dtype == 1) {
    if (p.d == 64) return lm_go<uint16_t, 64>(p, bwd, qL, k, kL, e, kL32, e32, dkL, de, dqL, dk, st);
    return lm_go<uint16_t, 128>(p, bwd, qL, k, kL, e, kL32, e32, dkL, de, dqL, dk, st);
  }
  if (p.d == 64) return lm_go<float, 64>(p, bwd, qL, k, kL, e, kL32, e32, dkL, de, dqL, dk, st);
  return lm_go<float, 128>(p, bwd, qL, k, kL, e, kL32, e32, dkL, de, dqL, dk, st);
}
}  // namespace

hipError_t launch_landmark_fwd(const Dims& p, const void* qL, const void* k, void* kL, void* e,
                               float* kL32, float* e32, hipStream_t st) {
  return lm_dispatch(p, false, qL, k, kL, e, kL32, e32, nullptr, nullptr, nullptr, nullptr, st);
}

hipError_t launch_landmark_bwd(const Dims& p, const void* qL, const void* k, const float* dkL,
                               const float* de, float* dqL, float* dk, hipStream_t st) {
  return lm_dispatch(p, true, qL, k, nullptr, nullptr, nullptr, nullptr, dkL, de, dqL, dk, st);
}

}  // namespace hils
