// Batched C (+)= A * B on bf16 MFMA, used by the Q-Cal backward (weight and
// input gradients of the low-rank query calibration).
//
// A is M x K and B is K x N; each may be stored "row-major" (A[m][k],
// B[k][n]) or "k-major" (A[k][m], B[n][k]) through the template flags, so
// the transposed products of a backward pass (X^T dY, dY W^T) need no
// separate transpose. fp32 operands are split into a bf16 hi part and a bf16
// lo part (x = hi + lo + O(2^-16 |x|)); products of the parts are exact in
// the MFMA and accumulate in fp32, which keeps ~16 significant bits per
// product term (hi*hi + hi*lo + lo*hi). bf16 operands are used as they are.
// Tiles of 64 x 64 with a 32-deep k step are staged through LDS in the
// [row][k] layout the fragments read; split-K adds partial tiles atomically.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

template <typename TA, typename TB, bool AKM, bool BKM>
__global__ __launch_bounds__(256) void k_gemm(const TA* __restrict__ A, const TB* __restrict__ B,
                                              float* __restrict__ Cm, int M, int N, int K, long lda,
                                              long ldb, long ldc, long sA1, long sA2, long sB1,
                                              long sB2, long sC1, long sC2, int nz2, int kchunk,
                                              int splits, int accumulate) {
  constexpr bool ALO = sizeof(TA) == 4, BLO = sizeof(TB) == 4;
  constexpr int KP = 40;  // padded k pitch (elements) of the LDS tiles
  __shared__ __align__(16) uint16_t as_hi[64 * KP], bs_hi[64 * KP];
  __shared__ __align__(16) uint16_t as_lo[ALO ? 64 * KP : 8], bs_lo[BLO ? 64 * KP : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int bz = blockIdx.z / splits, sp = blockIdx.z - bz * splits;
  const int z1 = bz / nz2, z2 = bz - z1 * nz2;
  A += z1 * sA1 + z2 * sA2;
  B += z1 * sB1 + z2 * sB2;
  Cm += z1 * sC1 + z2 * sC2;
  const int k_begin = sp * kchunk, k_end = min(K, k_begin + kchunk);
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero4();

  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    // ---- stage A (64 x 32) and B (32 x 64) as [row][k]
    {
      float x[8];
      int r, kk;
      if (!AKM) {  // A[m][k]: thread loads 8 k of one m
        r = tid >> 2;
        kk = (tid & 3) * 8;
        const int m = m0 + r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + kk + j;
          x[j] = (m < M && k < k_end) ? to_f<TA>(A[(long)m * lda + k]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint16_t hi = f2bf(x[j]);
          as_hi[r * KP + kk + j] = hi;
          if constexpr (ALO) as_lo[r * KP + kk + j] = f2bf(x[j] - bf2f(hi));
        }
      } else {  // A[k][m]: thread loads 8 m of one k
        kk = tid >> 3;
        r = (tid & 7) * 8;
        const int k = k0 + kk;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int m = m0 + r + j;
          x[j] = (m < M && k < k_end) ? to_f<TA>(A[(long)k * lda + m]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint16_t hi = f2bf(x[j]);
          as_hi[(r + j) * KP + kk] = hi;
          if constexpr (ALO) as_lo[(r + j) * KP + kk] = f2bf(x[j] - bf2f(hi));
        }
      }
      if (!BKM) {  // B[k][n]: thread loads 8 n of one k
        kk = tid >> 3;
        r = (tid & 7) * 8;
        const int k = k0 + kk;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + r + j;
          x[j] = (n < N && k < k_end) ? to_f<TB>(B[(long)k * ldb + n]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint16_t hi = f2bf(x[j]);
          bs_hi[(r + j) * KP + kk] = hi;
          if constexpr (BLO) bs_lo[(r + j) * KP + kk] = f2bf(x[j] - bf2f(hi));
        }
      } else {  // B[n][k]: thread loads 8 k of one n
        r = tid >> 2;
        kk = (tid & 3) * 8;
        const int n = n0 + r;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + kk + j;
          x[j] = (n < N && k < k_end) ? to_f<TB>(B[(long)n * ldb + k]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint16_t hi = f2bf(x[j]);
          bs_hi[r * KP + kk + j] = hi;
          if constexpr (BLO) bs_lo[r * KP + kk + j] = f2bf(x[j] - bf2f(hi));
        }
      }
    }
    __syncthreads();
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int off = (32 * wm + 16 * mb + (lane & 15)) * KP + 8 * (lane >> 4);
      ah[mb] = *reinterpret_cast<const bf16x8*>(as_hi + off);
      if constexpr (ALO) al[mb] = *reinterpret_cast<const bf16x8*>(as_lo + off);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int off = (32 * wn + 16 * nb + (lane & 15)) * KP + 8 * (lane >> 4);
      bh[nb] = *reinterpret_cast<const bf16x8*>(bs_hi + off);
      if constexpr (BLO) bl[nb] = *reinterpret_cast<const bf16x8*>(bs_lo + off);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        acc[mb][nb] = mma16(ah[mb], bh[nb], acc[mb][nb]);
        if constexpr (BLO) acc[mb][nb] = mma16(ah[mb], bl[nb], acc[mb][nb]);
        if constexpr (ALO) acc[mb][nb] = mma16(al[mb], bh[nb], acc[mb][nb]);
      }
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
        const int n = n0 + 32 * wn + 16 * nb + (lane & 15);
        if (m < M && n < N) {
          float* c = Cm + (long)m * ldc + n;
          if (splits > 1 || accumulate)
            atomicAdd(c, acc[mb][nb][i]);
          else
            *c = acc[mb][nb][i];
        }
      }
}

// Same product for shapes whose M, N, K, leading dimensions and batch strides
// are multiples of 8 elements (16-byte aligned operands): every thread's
// eight elements of a stage are one contiguous vector, loaded without
// per-element branches (a vector is wholly inside or outside the matrix;
// outside ones are clamped and zeroed), and the next k-step's vectors are
// in flight while the current one is multiplied.
template <typename T> struct V8;
template <> struct V8<uint16_t> { typedef u16x8 type; };
template <> struct V8<float> { typedef f32x8 type; };

template <typename T>
__device__ __forceinline__ typename V8<T>::type ldv8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const u16x8*>(p);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}
template <typename T>
__device__ __forceinline__ float v8f(const typename V8<T>::type& v, int j) {
  if constexpr (sizeof(T) == 2)
    return bf2f(v[j]);
  else
    return v[j];
}

template <typename TA, typename TB, bool AKM, bool BKM>
__global__ __launch_bounds__(256) void k_gemm_v(const TA* __restrict__ A, const TB* __restrict__ B,
                                                float* __restrict__ Cm, int M, int N, int K, long lda,
                                                long ldb, long ldc, long sA1, long sA2, long sB1,
                                                long sB2, long sC1, long sC2, int nz2, int kchunk,
                                                int splits, int accumulate) {
  constexpr bool ALO = sizeof(TA) == 4, BLO = sizeof(TB) == 4;
  constexpr int KP = 40;
  __shared__ __align__(16) uint16_t as_hi[64 * KP], bs_hi[64 * KP];
  __shared__ __align__(16) uint16_t as_lo[ALO ? 64 * KP : 8], bs_lo[BLO ? 64 * KP : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int bz = blockIdx.z / splits, sp = blockIdx.z - bz * splits;
  const int z1 = bz / nz2, z2 = bz - z1 * nz2;
  A += z1 * sA1 + z2 * sA2;
  B += z1 * sB1 + z2 * sB2;
  Cm += z1 * sC1 + z2 * sC2;
  const int k_begin = sp * kchunk, k_end = min(K, k_begin + kchunk);
  // this thread's vector of each stage: (row, k offset) for row-major
  // operands, (k offset, row) for k-major ones
  const int ar = AKM ? (tid & 7) * 8 : tid >> 2, ak = AKM ? tid >> 3 : (tid & 3) * 8;
  const int br = BKM ? tid >> 2 : (tid & 7) * 8, bk = BKM ? (tid & 3) * 8 : tid >> 3;
  const bool a_in = m0 + ar < M, b_in = n0 + br < N;
  auto lda_v = [&](int k0, typename V8<TA>::type& x, bool& ok) __attribute__((always_inline)) {
    const int k = k0 + ak;
    ok = a_in && k < k_end;
    const int kc = ok ? k : k_begin, mc = a_in ? m0 + ar : 0;
    x = ldv8<TA>(AKM ? A + (long)kc * lda + mc : A + (long)mc * lda + kc);
  };
  auto ldb_v = [&](int k0, typename V8<TB>::type& x, bool& ok) __attribute__((always_inline)) {
    const int k = k0 + bk;
    ok = b_in && k < k_end;
    const int kc = ok ? k : k_begin, nc = b_in ? n0 + br : 0;
    x = ldv8<TB>(BKM ? B + (long)nc * ldb + kc : B + (long)kc * ldb + nc);
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero4();
  typename V8<TA>::type xa;
  typename V8<TB>::type xb;
  bool oka, okb;
  lda_v(k_begin, xa, oka);
  ldb_v(k_begin, xb, okb);
  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    // publish the stage held in registers as [row][k] bf16 (hi, lo)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = oka ? v8f<TA>(xa, j) : 0.f;
      const uint16_t hi = f2bf(v);
      const int o = AKM ? (ar + j) * KP + ak : ar * KP + ak + j;
      as_hi[o] = hi;
      if constexpr (ALO) as_lo[o] = f2bf(v - bf2f(hi));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = okb ? v8f<TB>(xb, j) : 0.f;
      const uint16_t hi = f2bf(v);
      const int o = BKM ? br * KP + bk + j : (br + j) * KP + bk;
      bs_hi[o] = hi;
      if constexpr (BLO) bs_lo[o] = f2bf(v - bf2f(hi));
    }
    __syncthreads();
    // next stage's vectors in flight during the products
    if (k0 + 32 < k_end) {
      lda_v(k0 + 32, xa, oka);
      ldb_v(k0 + 32, xb, okb);
    }
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int off = (32 * wm + 16 * mb + (lane & 15)) * KP + 8 * (lane >> 4);
      ah[mb] = *reinterpret_cast<const bf16x8*>(as_hi + off);
      if constexpr (ALO) al[mb] = *reinterpret_cast<const bf16x8*>(as_lo + off);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int off = (32 * wn + 16 * nb + (lane & 15)) * KP + 8 * (lane >> 4);
      bh[nb] = *reinterpret_cast<const bf16x8*>(bs_hi + off);
      if constexpr (BLO) bl[nb] = *reinterpret_cast<const bf16x8*>(bs_lo + off);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        acc[mb][nb] = mma16(ah[mb], bh[nb], acc[mb][nb]);
        if constexpr (BLO) acc[mb][nb] = mma16(ah[mb], bl[nb], acc[mb][nb]);
        if constexpr (ALO) acc[mb][nb] = mma16(al[mb], bh[nb], acc[mb][nb]);
      }
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
        const int n = n0 + 32 * wn + 16 * nb + (lane & 15);
        if (m < M && n < N) {
          float* c = Cm + (long)m * ldc + n;
          if (splits > 1 || accumulate)
            atomicAdd(c, acc[mb][nb][i]);
          else
            *c = acc[mb][nb][i];
        }
      }
}

// Products whose operands both have the contraction index outermost (A[k][m]
// and B[k][n]), as in the weight gradients summed over tokens. Tiles of
// 128 x 128 (four waves of 64 x 64), k steps of 32, two LDS buffers, and the
// stage after next held in registers. A thread loads a 4 (k) x 4 (m or n)
// block of each operand and writes it into LDS as four 4-element k runs
// ([row][k] layout, 8-byte stores; with a pitch of 40 elements the 32 lanes of
// a store cover the 64 banks once). The workgroups of one XCD take
// consecutive (split, tile) ids, so a split's operand slices are shared in
// that XCD's L2. Split-K partial tiles go to a workspace slab per split and
// k_gemm_sum adds them (no atomics); without a split the tile goes to C.
template <typename T> struct V4;
template <> struct V4<uint16_t> { typedef u16x4 type; };
template <> struct V4<float> { typedef f32x4 type; };

template <typename TA, typename TB>
__global__ __launch_bounds__(256, 2) void k_gemm_kk(const TA* A, const TB* B,
                                                    float* __restrict__ out, int M, int N, int K,
                                                    long lda, long ldb, long ldo, long slab, int kchunk,
                                                    int ntn, int ntiles, int accumulate) {
  constexpr bool ALO = sizeof(TA) == 4, BLO = sizeof(TB) == 4;
  constexpr int KP = 40, PL = 128 * KP;  // elements of one operand plane
  constexpr int NPL = 2 + ALO + BLO;     // planes per buffer: A hi (lo), B hi (lo)
  extern __shared__ __align__(16) uint16_t sm[];  // [2][NPL][128][KP]
  typedef typename V4<TA>::type VA;
  typedef typename V4<TB>::type VB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  int L, y0;
  xcd_block(L, y0);
  const int sp = L / ntiles, tile = L - sp * ntiles;
  const int mt = tile / ntn, nt = tile - mt * ntn;
  const int m0 = mt * 128, n0 = nt * 128;
  const int k_begin = sp * kchunk, nk = (min(K, k_begin + kchunk) - k_begin) / 32;
  const int kq = tid & 7, rq = tid >> 3;  // this thread's block: k 4 kq + (0..3), row 4 rq + (0..3)
  const TA* ap = A + (long)(k_begin + 4 * kq) * lda + m0 + 4 * rq;
  const TB* bp = B + (long)(k_begin + 4 * kq) * ldb + n0 + 4 * rq;
  VA ra[2][4];
  VB rb[2][4];
  auto load = [&](int set, int s) __attribute__((always_inline)) {
    const long ss = 32 * min(s, nk - 1);  // past the end: a repeated stage, never used
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ra[set][kk] = *reinterpret_cast<const VA*>(ap + (ss + kk) * lda);
      rb[set][kk] = *reinterpret_cast<const VB*>(bp + (ss + kk) * ldb);
    }
  };
  auto put = [&](uint16_t* hi_p, uint16_t* lo_p, auto v, auto lo_on) __attribute__((always_inline)) {
    // v[kk][mm] -> rows 4 rq + mm, k run 4 kq .. 4 kq + 3
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      u16x4 hi, lo;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if constexpr (decltype(lo_on)::value) {
          const float x = v[kk][mm];
          hi[kk] = f2bf(x);
          lo[kk] = f2bf(x - bf2f(hi[kk]));
        } else {
          hi[kk] = v[kk][mm];
        }
      }
      const int o = (4 * rq + mm) * KP + 4 * kq;
      *reinterpret_cast<u16x4*>(hi_p + o) = hi;
      if constexpr (decltype(lo_on)::value) *reinterpret_cast<u16x4*>(lo_p + o) = lo;
    }
  };
  auto store = [&](int set, int buf) __attribute__((always_inline)) {
    uint16_t* base = sm + buf * NPL * PL;
    put(base, base + PL, ra[set], std::integral_constant<bool, ALO>());
    put(base + (1 + ALO) * PL, base + (2 + ALO) * PL, rb[set], std::integral_constant<bool, BLO>());
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint16_t* base = sm + buf * NPL * PL;
    const uint16_t* ah = base;
    const uint16_t* al = base + PL;
    const uint16_t* bh = base + (1 + ALO) * PL;
    const uint16_t* bl = base + (2 + ALO) * PL;
    const int fo = (lane & 15) * KP + 8 * (lane >> 4);
    bf16x8 bhf[4], blf[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int o = (64 * wn + 16 * nb) * KP + fo;
      bhf[nb] = *reinterpret_cast<const bf16x8*>(bh + o);
      if constexpr (BLO) blf[nb] = *reinterpret_cast<const bf16x8*>(bl + o);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int o = (64 * wm + 16 * mb) * KP + fo;
      const bf16x8 ahf = *reinterpret_cast<const bf16x8*>(ah + o);
      bf16x8 alf;
      if constexpr (ALO) alf = *reinterpret_cast<const bf16x8*>(al + o);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[mb][nb] = mma16(ahf, bhf[nb], acc[mb][nb]);
        if constexpr (BLO) acc[mb][nb] = mma16(ahf, blf[nb], acc[mb][nb]);
        if constexpr (ALO) acc[mb][nb] = mma16(alf, bhf[nb], acc[mb][nb]);
      }
    }
  };
  load(0, 0);
  load(1, 1);
  store(0, 0);
  __syncthreads();
  // (the empty asm statements keep the compiler from sinking the loads of
  // the stage after next below the products; A and B are not restrict-
  // qualified so that the statements order them)
  for (int s = 0; s < nk; s += 2) {
    load(0, s + 2);
    asm volatile("" ::: "memory");
    compute(0);
    store(1, 1);
    __syncthreads();
    if (s + 1 >= nk) break;
    load(1, s + 3);
    asm volatile("" ::: "memory");
    compute(1);
    store(0, 0);
    __syncthreads();
  }
  float* o = out + (size_t)sp * slab + (long)(m0 + 64 * wm + 4 * (lane >> 4)) * ldo + n0 + 64 * wn +
             (lane & 15);
  auto emit = [&](auto acc_on) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* c = o + (long)(16 * mb + i) * ldo + 16 * nb;
          if constexpr (decltype(acc_on)::value)
            *c += acc[mb][nb][i];
          else
            *c = acc[mb][nb][i];
        }
  };
  if (accumulate)
    emit(std::true_type());
  else
    emit(std::false_type());
}

// C[m][n] (+)= sum over the splits of the partial slabs P[s][m][n] (pitch N);
// four consecutive n per thread.
__global__ __launch_bounds__(256) void k_gemm_sum(const float* __restrict__ P, float* __restrict__ Cm,
                                                  int M, int N, long ldc, int splits, int accumulate) {
  const long n4 = (long)M * N / 4;
  const long slab = (long)M * N;
  for (long x = blockIdx.x * 256L + threadIdx.x; x < n4; x += (long)gridDim.x * 256) {
    const long e = 4 * x;
    const int m = (int)(e / N), n = (int)(e - (long)m * N);
    f32x4 s = zero4();
    for (int sp = 0; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(P + sp * slab + e);
    f32x4* c = reinterpret_cast<f32x4*>(Cm + (long)m * ldc + n);
    *c = accumulate ? *c + s : s;
  }
}

// Launch shape of the k_gemm_kk path; false when the product does not have
// its form (A k-major, B row-major, one batch, 128-multiples, 4-aligned rows).
static bool kk_plan(const GemmArgs& g, int* splits, int* kchunk) {
  if (!g.akm || g.bkm || g.n1 != 1 || g.n2 != 1) return false;
  if (g.M % 128 || g.N % 128 || g.K % 32 || g.lda % 4 || g.ldb % 4 || g.ldc % 4) return false;
  const int ntiles = (g.M / 128) * (g.N / 128);
  int sp = std::max(1, std::min((512 + ntiles - 1) / ntiles, g.K / 1024));
  int kc = (g.K + sp - 1) / sp;
  kc = (kc + 31) / 32 * 32;
  *splits = (g.K + kc - 1) / kc;
  *kchunk = kc;
  return true;
}

size_t gemm_work_bytes(const GemmArgs& g) {
  int sp, kc;
  if (!kk_plan(g, &sp, &kc) || sp == 1) return 0;
  return (size_t)sp * g.M * g.N * sizeof(float);
}

template <typename TA, typename TB>
static hipError_t gemm_kk_go(const GemmArgs& g, const TA* A, const TB* B, int splits, int kchunk,
                             hipStream_t st) {
  const int ntn = g.N / 128, ntiles = (g.M / 128) * ntn;
  constexpr int NPL = 2 + (sizeof(TA) == 4) + (sizeof(TB) == 4);
  const size_t lds = 2 * NPL * 128 * 40 * sizeof(uint16_t);
  auto kern = k_gemm_kk<TA, TB>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  const bool direct = splits == 1;
  float* out = direct ? g.C : g.work;
  hipLaunchKernelGGL(kern, dim3(ntiles * splits), dim3(256), lds, st, A, B, out, g.M, g.N, g.K, g.lda,
                     g.ldb, direct ? g.ldc : (long)g.N, direct ? 0L : (long)g.M * g.N, kchunk, ntn,
                     ntiles, direct && g.accumulate ? 1 : 0);
  if ((err = hipGetLastError()) != hipSuccess || direct) return err;
  const long n4 = (long)g.M * g.N / 4;
  const unsigned nb = (unsigned)std::min<long>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(k_gemm_sum, dim3(nb), dim3(256), 0, st, g.work, g.C, g.M, g.N, g.ldc, splits,
                     g.accumulate ? 1 : 0);
  return hipGetLastError();
}

// C[z] (+)= A[z] * B[z] over the batch z = (z1, z2), z1 < g.n1, z2 < g.n2.
template <typename TA, typename TB, bool AKM, bool BKM>
static hipError_t gemm_go(const GemmArgs& g, const TA* A, const TB* B, hipStream_t st) {
  int splits = g.splits < 1 ? 1 : g.splits;
  int kchunk = (g.K + splits - 1) / splits;
  kchunk = (kchunk + 31) / 32 * 32;
  splits = (g.K + kchunk - 1) / kchunk;
  if constexpr (AKM && !BKM) {
    int sk, kc;
    if (kk_plan(g, &sk, &kc) && (uintptr_t)A % 16 == 0 && (uintptr_t)B % 16 == 0 &&
        (sk == 1 || g.work != nullptr))
      return gemm_kk_go<TA, TB>(g, A, B, sk, kc, st);
  }
  dim3 grid((g.M + 63) / 64, (g.N + 63) / 64, g.n1 * g.n2 * splits);
  auto m8 = [](long x) { return x % 8 == 0; };
  const bool vec = m8(g.M) && m8(g.N) && m8(g.K) && m8(g.lda) && m8(g.ldb) && m8(g.sA1) && m8(g.sA2) &&
                   m8(g.sB1) && m8(g.sB2) && ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
  if (vec) {
    hipLaunchKernelGGL((k_gemm_v<TA, TB, AKM, BKM>), grid, dim3(256), 0, st, A, B, g.C, g.M, g.N, g.K,
                       g.lda, g.ldb, g.ldc, g.sA1, g.sA2, g.sB1, g.sB2, g.sC1, g.sC2, g.n2, kchunk,
                       splits, g.accumulate ? 1 : 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm<TA, TB, AKM, BKM>), grid, dim3(256), 0, st, A, B, g.C, g.M, g.N, g.K,
                     g.lda, g.ldb, g.ldc, g.sA1, g.sA2, g.sB1, g.sB2, g.sC1, g.sC2, g.n2, kchunk,
                     splits, g.accumulate ? 1 : 0);
  return hipGetLastError();
}

template <typename TA, typename TB>
static hipError_t gemm_t(const GemmArgs& g, const TA* A, const TB* B, hipStream_t st) {
  if (!g.akm && !g.bkm) return gemm_go<TA, TB, false, false>(g, A, B, st);
  if (!g.akm && g.bkm) return gemm_go<TA, TB, false, true>(g, A, B, st);
  if (g.akm && !g.bkm) return gemm_go<TA, TB, true, false>(g, A, B, st);
  return gemm_go<TA, TB, true, true>(g, A, B, st);
}

hipError_t gemm(const GemmArgs& g, const void* A, int a_dtype, const void* B, int b_dtype,
                hipStream_t st) {
  // dtype codes: 0 fp32, 1 bf16
  if (a_dtype == 0 && b_dtype == 0) return gemm_t<float, float>(g, (const float*)A, (const float*)B, st);
  if (a_dtype == 0 && b_dtype == 1) return gemm_t<float, uint16_t>(g, (const float*)A, (const uint16_t*)B, st);
  if (a_dtype == 1 && b_dtype == 0) return gemm_t<uint16_t, float>(g, (const uint16_t*)A, (const float*)B, st);
  return gemm_t<uint16_t, uint16_t>(g, (const uint16_t*)A, (const uint16_t*)B, st);
}

}  // namespace hils
