// Device-side building blocks shared by the HiLS kernels (gfx950 / CDNA4).
//
// MFMA fragment convention used everywhere (checked on the device): for the
// 16x16x32 bf16 product D = A * B (+C),
//   lane l holds A[row = l % 16][k = 8 * (l / 16) + e], e = 0..7,
//             B[k = 8 * (l / 16) + e][col = l % 16],
//             D[row = 4 * (l / 16) + i][col = l % 16], i = 0..3.
// fp32 inputs use eight 16x16x4 fp32 products with the same per-lane
// element layout (element e feeds product e), so every kernel is written
// once over the element type T (uint16_t holding bf16 bits, or float).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float NEG_INF = -__builtin_inff();

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// 2^x with one v_exp_f32 (exp2(-inf) = 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float x) { return f2bf(x); }

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// 8 consecutive elements (16 B for bf16, 32 B for fp32; aligned)
template <typename T> __device__ __forceinline__ typename Frag<T>::type ld8(const T* p);
template <> __device__ __forceinline__ bf16x8 ld8<uint16_t>(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ f32x8 ld8<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// 8 floats -> fragment of T
template <typename T> __device__ __forceinline__ typename Frag<T>::type pack8(const float* x);
template <> __device__ __forceinline__ bf16x8 pack8<uint16_t>(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}
template <> __device__ __forceinline__ f32x8 pack8<float>(const float* x) {
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[j];
  return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// operand whose every element is 1: ones x P^T puts the column sums of P^T
// into every row of the product
__device__ __forceinline__ bf16x8 ones_frag() {
  const __bf16 o = (__bf16)1.0f;
  return bf16x8{o, o, o, o, o, o, o, o};
}

// bf16 fragment times c as a sum of two bf16 fragments (hi + lo carries
// ~16 significant bits of each product)
__device__ __forceinline__ void scale_split(const bf16x8& f, float c, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = (float)f[j] * c;
    hi[j] = (__bf16)x;
    lo[j] = (__bf16)(x - (float)hi[j]);
  }
}

// every element of a fragment times c (rounded back to T)
template <typename T>
__device__ __forceinline__ typename Frag<T>::type scale_frag(const typename Frag<T>::type& f, float c) {
  typename Frag<T>::type r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (sizeof(T) == 2)
      r[j] = (__bf16)((float)f[j] * c);
    else
      r[j] = f[j] * c;
  }
  return r;
}

// two accumulator quads (rows 4 g + i of two 16-row blocks) -> one operand
// fragment; the k order {0..3, 16..19}-style permutation is the same on
// whichever operand is built this way
template <typename T>
__device__ __forceinline__ typename Frag<T>::type pk8(const f32x4& s0, const f32x4& s1) {
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  return pack8<T>(x);
}

// In-place exclusive scan of a[0..n) by the whole block (256 threads);
// returns the total. Contains barriers: call from uniform control flow.
__device__ __forceinline__ int block_excl_scan(int* a, int n, int* wsum) {
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

// Completes this wave's outstanding LDS operations and stops the compiler
// from moving memory accesses across: used where lanes of ONE wave exchange
// data through LDS (the other waves are not involved).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int n_distant(int i, int W, int S) {
  const int x = i - W + 1;
  return x <= 0 ? 0 : x / S;
}

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// linear id. xcd_block renumbers a 2-D grid (x fastest) so that every XCD
// walks one contiguous range of it: the x-neighbours of one y, which read the
// same (b, kv head) keys, values and queries, then share an L2.
constexpr int NXCD = 8;
__device__ __forceinline__ void xcd_block(int& x, int& y) {
  const int gx = gridDim.x;
  const int T = gx * gridDim.y;
  const int L = blockIdx.x + gx * blockIdx.y;
  const int xcd = L % NXCD, k = L / NXCD;
  const int q = T / NXCD, rem = T % NXCD;
  const int Lp = xcd * q + min(xcd, rem) + k;
  y = Lp / gx;
  x = Lp - y * gx;
}

// cross-lane helpers (lanes xor-ed within the wave)
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, WAVE); }

// max / sum over the four lanes l, l^16, l^32, l^48 (one column of an MFMA
// D fragment) with the gfx950 row-swap permutes: swapping a copy of x with
// itself leaves {x[l], x[l^16]} (then {x[l], x[l^32]}) in the two results
__device__ __forceinline__ float col_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// buffer resource over [base, base + bytes): loads past the end return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

}  // namespace hils
