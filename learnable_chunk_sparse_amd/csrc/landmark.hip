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
// One wave per (b, kv head, chunk), one wave per workgroup. The chunk's 64
// keys are staged in LDS as fp32 rows padded to DH + 1 floats, so lane t
// reading row t (scores, dkL . k_t) and lane j reading column j (the
// key-weighted sums) are both free of bank conflicts. Lane t owns token t for
// the scores and the softmax (wave reductions); lane j owns dims j and
// j + 64 for the sums over tokens. All arithmetic is fp32.
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

// the chunk's keys -> kf[t][j] (fp32, pitch DH + 1); 16-byte loads
template <typename T, int DH>
__device__ __forceinline__ void stage_keys(const T* __restrict__ kc, float* kf, int lane) {
  constexpr int V = 16 / sizeof(T), PER = LS * DH / (64 * V);
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int x = (it * 64 + lane) * V;
    const int t = x / DH, j = x - t * DH;
    if constexpr (sizeof(T) == 2) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(kc + x);
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[t * (DH + 1) + j + i] = bf2f(v[i]);
    } else {
      const f32x4 v = *reinterpret_cast<const f32x4*>(kc + x);
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[t * (DH + 1) + j + i] = v[i];
    }
  }
}

// scores, softmax weights (to LDS) and the chunk statistics of one chunk
struct ChunkSoftmax {
  float s, p;   // this lane's token
  float logZ;   // log sum_t exp(s_t)
  float sbar;   // sum_t p_t s_t
};
template <int DH>
__device__ __forceinline__ ChunkSoftmax chunk_softmax(const float* kf, const float* qs, float* ps,
                                                      float scale, int lane) {
  float acc = 0.f;
  const float* kr = kf + lane * (DH + 1);
#pragma unroll 16
  for (int j = 0; j < DH; ++j) acc = fmaf(qs[j], kr[j], acc);
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

template <typename T, int DH>
__global__ __launch_bounds__(64) void k_landmark_fwd(const T* __restrict__ qL, const T* __restrict__ k,
                                                     T* __restrict__ kL, T* __restrict__ e,
                                                     float* __restrict__ kL32, float* __restrict__ e32,
                                                     int N, int C, float scale) {
  __shared__ float kf[LS * (DH + 1)];
  __shared__ float qs[DH], ps[LS];
  const int lane = threadIdx.x;
  const int c = blockIdx.x, bg = blockIdx.y;
  const size_t cr = (size_t)bg * C + c;  // (b, kv head, chunk)
  stage_keys<T, DH>(k + ((size_t)bg * N + (size_t)c * LS) * DH, kf, lane);
  for (int j = lane; j < DH; j += 64) qs[j] = to_f<T>(qL[cr * DH + j]);
  __syncthreads();
  const ChunkSoftmax r = chunk_softmax<DH>(kf, qs, ps, scale, lane);
  __syncthreads();
#pragma unroll
  for (int j = lane; j < DH; j += 64) {
    float a = 0.f;
#pragma unroll 16
    for (int t = 0; t < LS; ++t) a = fmaf(ps[t], kf[t * (DH + 1) + j], a);
    kL[cr * DH + j] = from_f<T>(a);
    if (kL32 != nullptr) kL32[cr * DH + j] = a;
  }
  if (lane == 0) {
    const float ent = r.logZ - r.sbar;
    e[cr] = from_f<T>(ent);
    if (e32 != nullptr) e32[cr] = ent;
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(64) void k_landmark_bwd(const T* __restrict__ qL, const T* __restrict__ k,
                                                     const float* __restrict__ dkL,
                                                     const float* __restrict__ de,
                                                     float* __restrict__ dqL, float* __restrict__ dk,
                                                     int N, int C, float scale) {
  __shared__ float kf[LS * (DH + 1)];
  __shared__ float qs[DH], gs[DH], ps[LS], dss[LS];
  const int lane = threadIdx.x;
  const int c = blockIdx.x, bg = blockIdx.y;
  const size_t cr = (size_t)bg * C + c;
  const size_t t0 = (size_t)bg * N + (size_t)c * LS;  // first token row of the chunk
  stage_keys<T, DH>(k + t0 * DH, kf, lane);
  for (int j = lane; j < DH; j += 64) {
    qs[j] = to_f<T>(qL[cr * DH + j]);
    gs[j] = dkL[cr * DH + j];
  }
  const float dev = de[cr];
  __syncthreads();
  const ChunkSoftmax r = chunk_softmax<DH>(kf, qs, ps, scale, lane);
  __syncthreads();
  // dkL . kL with kL = sum_t p_t k_t (lane j: its dims)
  float gk = 0.f;
#pragma unroll
  for (int j = lane; j < DH; j += 64) {
    float a = 0.f;
#pragma unroll 16
    for (int t = 0; t < LS; ++t) a = fmaf(ps[t], kf[t * (DH + 1) + j], a);
    gk = fmaf(gs[j], a, gk);
  }
  gk = wave_sum(gk);
  // ds_t (lane t)
  {
    float g = 0.f;
    const float* kr = kf + lane * (DH + 1);
#pragma unroll 16
    for (int j = 0; j < DH; ++j) g = fmaf(gs[j], kr[j], g);
    dss[lane] = r.p * (g - gk - dev * (r.s - r.sbar));
  }
  __syncthreads();
#pragma unroll
  for (int j = lane; j < DH; j += 64) {
    float a = 0.f;
#pragma unroll 16
    for (int t = 0; t < LS; ++t) a = fmaf(dss[t], kf[t * (DH + 1) + j], a);
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
  const dim3 grid((unsigned)p.C, (unsigned)(p.B * p.Hkv));
  if (!bwd)
    hipLaunchKernelGGL((k_landmark_fwd<T, DH>), grid, dim3(64), 0, st, (const T*)qL, (const T*)k,
                       (T*)kL, (T*)e, kL32, e32, p.N, p.C, p.scale);
  else
    hipLaunchKernelGGL((k_landmark_bwd<T, DH>), grid, dim3(64), 0, st, (const T*)qL, (const T*)k,
                       dkL, de, dqL, dk, p.N, p.C, p.scale);
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
