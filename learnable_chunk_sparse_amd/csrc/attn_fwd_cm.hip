// HiLS prefill forward, chunk-major strategy (long sequences).
//
// Paper: Fig. 3 (each selected chunk gets its inter-chunk mass exp(s_c - L),
// spread over its tokens by the intra-chunk softmax), the engineersofai
// abstract (each query attends to each retrieved chunk independently and the
// per-chunk outputs are fused by the retrieval scores), "Limitations of Naive
// Sparse Attention" (local window plus distant chunks); the same result as
// the query-tile strategies of attn_fwd.hip and attn_fwd_sparse.hip.
//
// Why chunk-major: when adjacent queries share few chunks (independent
// queries over thousands of distant chunks), a query tile reuses each chunk
// it loads for about one position, so every (position, chunk) selection costs
// a whole 64-token K and V block of traffic. Here every selected chunk is
// loaded once per (batch, KV head) and serves all the rows that chose it,
// found through the inverse index (inv_index.hip); the price is one per-chunk
// output per (position, slot, head) written and read back once.
//
//   k_fwd_cm_chunks  one workgroup per (chunk, b, KV head); the chunk's K rows
//                    and V^T sit in LDS while the waves take 16-row blocks of
//                    the chunk's rows (16 / G entries x G heads): S^T = K Q^T,
//                    softmax over the 64 tokens, O_c^T = V^T P^T, O_c
//                    normalised and stored in the input dtype at
//                    part[b, g][entry][head], entries in the inverse index's
//                    order (each workgroup writes one contiguous run). A row
//                    is 16-byte pieces, piece 4 x + gl held by lane group gl
//                    (its x-th vector of MFMA output dims), so the four lanes
//                    of a row move 64 contiguous bytes per instruction in
//                    both kernels.
//   k_fwd_cm_window  query tiles of 128 rows (128 / G positions x G heads):
//                    banded flash attention over the window with K / V^T
//                    blocks staged through LDS for the four waves; then
//                    L = log(exp(lse_W) + exp(lse_sel)) and
//                    o = exp(lse_W - L) O_W + sum_k exp(s_k - L) O_{c_k},
//                    each O_{c_k} found through the entry index of
//                    (position, slot k) that the inverse index records.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

namespace {

// ---------------------------------------------------------------- LDS slot
// One 64-token block: K rows and V^T rows (token-permuted), pitches padded by
// 16 bytes so the 16-byte fragment reads of 16 lanes hit distinct banks.
template <typename T, int DH>
struct WSlot {
  static constexpr int VE = 16 / (int)sizeof(T);
  static constexpr int KP = DH + VE;
  static constexpr int VP = 64 + VE;
  static constexpr int KE = 64 * KP;
  static constexpr int ELEMS = KE + DH * VP;
  static constexpr int KV = 64 * DH / VE;
  static constexpr int VPT = 2 * KV / 256;
};

// ---------------------------------------------------------------- chunk pass
template <typename T, int DH>
struct RowBlock {
  typename Frag<T>::type q[DH / 32];
  int pos, slot;  // slot: the row block's entry index within the chunk's list
  bool valid;
};

// The chunk's K and V^T sit in LDS (read as fragments by each row block), so
// that a wave holds only its row blocks: four waves per SIMD at bf16, and the
// queries of the next two row blocks in flight while one is multiplied.
// Work items: a chunk's list cut into pieces of at most CM_ITEM_ROWS rows
// (CM_ITEM_ROWS / G entries), so that a chunk chosen by a large share of the
// positions (a high entropy bias makes some chunks far more popular than
// others) is spread over many workgroups instead of one. One workgroup per
// (b, KV head) lists them in chunk order: item = (chunk, first entry).
constexpr int CM_ITEM_ROWS = 1024;
// the window pass's 128-row tiles: each wave owns one 16-row block (eight
// waves). With two blocks per wave the accumulators, score tiles, query
// fragments and staged blocks needed ~480 registers at d = 128 (one wave per
// SIMD) and 235 at d = 64 (two); with one, 198 and 120 (two and four).
template <int DH>
constexpr int cm_win_cb() { return 1; }
template <int DH>
constexpr int cm_win_rows() { return 128; }  // (64-row tiles at d = 128, two workgroups per CU: no faster)
template <int DH>
constexpr int cm_win_threads() { return cm_win_rows<DH>() / (16 * cm_win_cb<DH>()) * 64; }

__global__ __launch_bounds__(256) void k_cm_items(const int* __restrict__ off, int2* __restrict__ items,
                                                  int* __restrict__ nitems, int* __restrict__ scratch,
                                                  int C, int E, int maxit) {
  __shared__ int wsum[4];
  const int bg = blockIdx.x;
  const int* ob = off + (size_t)bg * (C + 1);
  int* cnt = scratch + (size_t)bg * C;
  for (int c = threadIdx.x; c < C; c += 256) cnt[c] = (ob[c + 1] - ob[c] + E - 1) / E;
  __syncthreads();
  const int tot = block_excl_scan(cnt, C, wsum);
  int2* it = items + (size_t)bg * maxit;
  for (int c = threadIdx.x; c < C; c += 256) {
    const int n = ob[c + 1] - ob[c];
    for (int s0 = 0, j = cnt[c]; s0 < n; s0 += E, ++j) it[j] = int2{c, s0};
  }
  if (threadIdx.x == 0) nitems[bg] = tot;
}

template <typename T, int G, int DH>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? (DH == 64 ? 3 : 2) : 1) void k_fwd_cm_chunks(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int* __restrict__ off, const int* __restrict__ lst, const int2* __restrict__ items,
    const int* __restrict__ nitems, T* __restrict__ part, int N, int Np, int Hkv, int K, int C,
    int maxit, float scale) {
  typedef typename Frag<T>::type FT;
  typedef WSlot<T, DH> SG;
  constexpr int KS = DH / 32;
  constexpr int MB = DH / 16;
  constexpr int EPB = 16 / G;  // entries per 16-row block
  constexpr int E = CM_ITEM_ROWS / G;  // entries per work item
  extern __shared__ __align__(16) unsigned char smem[];
  T* sl = reinterpret_cast<T*>(smem);
  const int bg = blockIdx.y;
  if ((int)blockIdx.x >= nitems[bg]) return;  // uniform over the workgroup
  const int2 item = items[(size_t)bg * maxit + blockIdx.x];
  const int c = item.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int* ob = off + (size_t)bg * (C + 1);
  const int e0 = ob[c] + item.y, n = min(E, ob[c + 1] - e0);
  const int nb = (n + EPB - 1) / EPB;
  const int tid = threadIdx.x, lane = tid & 63, gl = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // stage the chunk's K rows and V^T columns (16-byte vectors)
  {
    const T* kb = k + ((size_t)bg * N + (size_t)c * 64) * DH;
    const T* vb = vt + (size_t)bg * DH * Np + (size_t)c * 64;
#pragma unroll
    for (int s2 = 0; s2 < SG::VPT; ++s2) {
      const int vi = tid + 256 * s2;
      if (s2 < SG::VPT / 2) {
        const int tok = vi / (DH / SG::VE), pt = vi - tok * (DH / SG::VE);
        *reinterpret_cast<u32x4*>(sl + tok * SG::KP + pt * SG::VE) =
            *reinterpret_cast<const u32x4*>(kb + (size_t)tok * DH + pt * SG::VE);
      } else {
        const int vj = vi - SG::KV;
        const int dd = vj / (64 / SG::VE), pt = vj - dd * (64 / SG::VE);
        *reinterpret_cast<u32x4*>(sl + SG::KE + dd * SG::VP + pt * SG::VE) =
            *reinterpret_cast<const u32x4*>(vb + (size_t)dd * Np + pt * SG::VE);
      }
    }
  }
  __syncthreads();
  if (w >= nb) return;  // no barrier below

  const int* lb = lst + (size_t)bg * N * K + e0;
  const int hh = cl % G;
  const float sc2 = scale * LOG2E;

  auto load_rows = [&](RowBlock<T, DH>& r, int j) __attribute__((always_inline)) {
    const int x = j * EPB + cl / G;
    r.valid = x < n;
    const int en = lb[min(x, n - 1)];
    r.pos = en >> 6;
    r.slot = x;  // entry index within the chunk's list
    const T* src = q + (((size_t)b * Hq + g * G + hh) * N + r.pos) * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) r.q[ks] = ld8<T>(src + 32 * ks);
  };
  auto process = [&](const RowBlock<T, DH>& r) __attribute__((always_inline)) {
    f32x4 sacc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      sacc[tb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[tb] = mma16(ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks), r.q[ks], sacc[tb]);
    }
    float mx = NEG_INF;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tb][i]);
    const float mref = col_max4(mx) * sc2;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[tb][i] = fast_exp2(fmaf(sacc[tb][i], sc2, -mref));
    FT pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pf[ks] = pk8<T>(sacc[2 * ks], sacc[2 * ks + 1]);
    float ps;
    if constexpr (sizeof(T) == 2) {
      // the sum of exactly the rounded weights the PV product uses
      f32x4 s4 = mma16(ones_frag(), pf[0], zero4());
      s4 = mma16(ones_frag(), pf[1], s4);
      ps = s4[0];
    } else {
      float s = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += sacc[tb][i];
      ps = col_sum4(s);
    }
    f32x4 oc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oc[mb] = zero4();
    const T* vbs = sl + SG::KE;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        oc[mb] = mma16(ld8<T>(vbs + (16 * mb + cl) * SG::VP + 8 * gl + 32 * ks), pf[ks], oc[mb]);
    if (r.valid) {
      const float inv = 1.0f / ps;
      // vector x of this lane is the row's 16-byte piece 4 x + gl
      u32x4* dst = reinterpret_cast<u32x4*>(part + ((size_t)bg * N * K + e0 + r.slot) * G * DH +
                                            (size_t)hh * DH) + gl;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int m2 = 0; m2 < MB; m2 += 2) {
          u16x8 hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hv[i] = f2bf(oc[m2][i] * inv);
            hv[4 + i] = f2bf(oc[m2 + 1][i] * inv);
          }
          dst[4 * (m2 / 2)] = __builtin_bit_cast(u32x4, hv);
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dst[4 * mb] = __builtin_bit_cast(u32x4, oc[mb] * inv);
      }
    }
  };
  // row blocks w, w + 4, ...: the queries of the next two (d = 64) or the
  // next one (d = 128, register budget) are in flight while one is multiplied
  if constexpr (DH == 64) {
    RowBlock<T, DH> r0, r1, r2;
    load_rows(r0, w);
    if (w + 4 < nb) load_rows(r1, w + 4);
    for (int j = w; j < nb; j += 12) {
      if (j + 8 < nb) load_rows(r2, j + 8);
      process(r0);
      if (j + 4 >= nb) break;
      if (j + 12 < nb) load_rows(r0, j + 12);
      process(r1);
      if (j + 8 >= nb) break;
      if (j + 16 < nb) load_rows(r1, j + 16);
      process(r2);
    }
  } else {
    RowBlock<T, DH> r0, r1;
    load_rows(r0, w);
    for (int j = w; j < nb; j += 8) {
      if (j + 4 < nb) load_rows(r1, j + 4);
      process(r0);
      if (j + 4 >= nb) break;
      if (j + 8 < nb) load_rows(r0, j + 8);
      process(r1);
    }
  }
}

// ---------------------------------------------------------------- window pass
template <typename T, int G, int DH>
__global__ __launch_bounds__(cm_win_threads<DH>(), (cm_win_threads<DH>() == 256 && sizeof(T) == 2) ? 2 : 1) void k_fwd_cm_window(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_score,
    const float* __restrict__ sel_lse, const int* __restrict__ rank, const T* __restrict__ part,
    T* __restrict__ o, float* __restrict__ lse, int N, int Np, int Hkv, int K, int W, int S,
    float scale, int ntiles) {
  typedef typename Frag<T>::type FT;
  typedef WSlot<T, DH> SG;
  constexpr int CB = cm_win_cb<DH>();      // 16-row blocks per wave
  constexpr int RW = 16 * CB;              // rows per wave
  constexpr int NT = cm_win_threads<DH>(); // 128 rows per tile
  constexpr int VPT = 2 * SG::KV / NT;     // staged 16-byte vectors per thread and block
  constexpr int R = cm_win_rows<DH>();
  constexpr int TP = R / G;
  constexpr int KS = DH / 32;
  constexpr int MB = DH / 16;

  extern __shared__ __align__(16) unsigned char smem[];
  T* slots = reinterpret_cast<T*>(smem);  // [2][ELEMS]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gl = lane >> 4, cl = lane & 15;
  int tx, bg;
  xcd_block(tx, bg);
  const int tile = ntiles - 1 - tx;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * TP;
  const int plast = min(p0 + TP - 1, N - 1);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bg * N * DH, N * DH * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vt + (size_t)bg * DH * Np, DH * Np * (int)sizeof(T));

  // wave w owns rows 32 w + 16 cb + cl
  FT qf[CB][KS];
  int prow[CB], wsr[CB];
  float lsel[CB], Lr[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = RW * w + 16 * cb + cl;
    const int pos = p0 + r / G, hh = r % G;
    prow[cb] = pos < N ? pos : -1;
    wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
    const int pc = pos < N ? pos : N - 1;
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pc;
    lsel[cb] = sel_lse[ro];
    const T* src = q + ro * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = ld8<T>(src + 32 * ks);
  }
  const int pw_lo = p0 + RW * w / G;
  const int pw_hi = min(p0 + (RW * w + RW - 1) / G, N - 1);
  const bool wave_live = pw_lo < N;
  const bool all_valid = p0 + (RW * w + RW - 1) / G < N;
  const int ws_lo = wave_live ? n_distant(pw_lo, W, S) * S : 0;
  const int ws_hi = wave_live ? n_distant(pw_hi, W, S) * S : 0;

  float m[CB], lsum[CB];
  f32x4 oacc[MB][CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m[cb] = NEG_INF;
    lsum[cb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] = zero4();
  }
  const float sc2 = scale * LOG2E;

  const int kv_lo = n_distant(p0, W, S) * S;
  const int nW = (plast - kv_lo) / 64 + 1;
  // blocks in flight in registers: two sets (blocks n + 2, n + 3)
  constexpr int NSET = VPT > 4 ? 1 : 2;
  u32x4 stg[2][VPT];
  auto issue = [&](u32x4 (&rg)[VPT], int n) __attribute__((always_inline)) {
    const int kv0 = kv_lo + 64 * min(n, nW - 1);
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int vi = tid + NT * s;
      if (s < VPT / 2) {
        const int tok = vi / (DH / SG::VE), pt = vi - tok * (DH / SG::VE);
        rg[s] = buf_ld16(krs, ((kv0 + tok) * DH + pt * SG::VE) * (int)sizeof(T));
      } else {
        const int vj = vi - SG::KV;
        const int dd = vj / (64 / SG::VE), pt = vj - dd * (64 / SG::VE);
        rg[s] = buf_ld16(vrs, (dd * Np + kv0 + pt * SG::VE) * (int)sizeof(T));
      }
    }
  };
  auto commit = [&](const u32x4 (&rg)[VPT], int slot) __attribute__((always_inline)) {
    T* base = slots + slot * SG::ELEMS;
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int vi = tid + NT * s;
      T* dst;
      if (s < VPT / 2) {
        const int tok = vi / (DH / SG::VE), pt = vi - tok * (DH / SG::VE);
        dst = base + tok * SG::KP + pt * SG::VE;
      } else {
        const int vj = vi - SG::KV;
        const int dd = vj / (64 / SG::VE), pt = vj - dd * (64 / SG::VE);
        dst = base + SG::KE + dd * SG::VP + pt * SG::VE;
      }
      *reinterpret_cast<u32x4*>(dst) = rg[s];
    }
  };

  // banded flash attention of the wave's rows over one staged block; the
  // reference m moves only when a block's scores exceed it by more than 16
  // (log2 units), or on a row's first scores
  auto window_block = [&](const T* sl, int kv0, auto masked) __attribute__((always_inline)) {
    constexpr bool MSK = decltype(masked)::value;
    constexpr float SHIFT_AT = 16.f;
    f32x4 sacc[4][CB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) sacc[tb][cb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FT kf = ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) sacc[tb][cb] = mma16(kf, qf[cb][ks], sacc[tb][cb]);
      }
    }
    float bmx[CB];
    bool shift = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float bmax = NEG_INF;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[tb][cb][i];
          if constexpr (MSK) {
            const int j = kv0 + 16 * tb + 4 * gl + i;
            x = (j <= prow[cb] && j >= wsr[cb]) ? x : NEG_INF;
            sacc[tb][cb][i] = x;
          }
          bmax = fmaxf(bmax, x);
        }
      bmx[cb] = col_max4(bmax) * sc2 - (m[cb] == NEG_INF ? 0.f : m[cb]);
      shift |= bmx[cb] > SHIFT_AT || (m[cb] == NEG_INF && bmx[cb] != NEG_INF);
    }
    if (__ballot(shift) != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bool first = m[cb] == NEG_INF;
        const bool up = bmx[cb] > SHIFT_AT || (first && bmx[cb] != NEG_INF);
        const float dlt = up ? bmx[cb] : 0.f;
        const float alpha = first ? 0.f : fast_exp2(-dlt);
        if (up) m[cb] = (first ? 0.f : m[cb]) + dlt;
        lsum[cb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= alpha;
      }
    }
    FT pf[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float mc = m[cb] == NEG_INF ? 0.f : m[cb];
      float ps = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(sacc[tb][cb][i], sc2, -mc));
          sacc[tb][cb][i] = pv;
          ps += pv;
        }
      lsum[cb] += ps;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[cb][ks] = pk8<T>(sacc[2 * ks][cb], sacc[2 * ks + 1][cb]);
    }
    const T* vb = sl + SG::KE;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const FT vf = ld8<T>(vb + (16 * mb + cl) * SG::VP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[mb][cb] = mma16(vf, pf[cb][ks], oacc[mb][cb]);
      }
  };

  // one step: publish block n + 1 from register set rg into the other slot
  // (whose block n - 1 every wave has finished), reload rg with block n + 3,
  // then multiply block n
  auto wstep = [&](int n, u32x4 (&rg)[VPT]) __attribute__((always_inline)) {
    commit(rg, (n + 1) & 1);
    issue(rg, n + 1 + NSET);
    const T* sl = slots + (n & 1) * SG::ELEMS;
    const int kv0 = kv_lo + 64 * n;
    if (wave_live && kv0 <= pw_hi && kv0 + 63 >= ws_lo) {
      const bool clean = all_valid && kv0 >= ws_hi && kv0 + 63 <= pw_lo;
      if (clean)
        window_block(sl, kv0, std::false_type());
      else
        window_block(sl, kv0, std::true_type());
    }
    __syncthreads();
  };
  int n = 0;
  if constexpr (NSET == 2) {
    issue(stg[0], 0);
    issue(stg[1], 1);
    commit(stg[0], 0);
    issue(stg[0], 2);
    __syncthreads();
    for (; n + 1 < nW; n += 2) {
      wstep(n, stg[1]);
      wstep(n + 1, stg[0]);
    }
    if (n < nW) wstep(n, stg[1]);
  } else {
    issue(stg[0], 0);
    commit(stg[0], 0);
    issue(stg[0], 1);
    __syncthreads();
    for (; n < nW; ++n) wstep(n, stg[0]);
  }

  // fusion normaliser and the window's weight exp(lse_W - L)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float ls = col_sum4(lsum[cb]);
    const float lW = (m[cb] + __log2f(ls)) * LN2;
    const float mx = fmaxf(lW, lsel[cb]);
    const bool live = prow[cb] >= 0;
    const float L = live ? mx + __logf(__expf(lW - mx) + __expf(lsel[cb] - mx)) : 0.f;
    const float coef = live ? fast_exp2(m[cb] - L * LOG2E) : 0.f;
    Lr[cb] = L;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= coef;
  }

  // selected chunks: add exp(s_k - L) O_{c_k} from the chunk pass (this
  // lane's VPS 16-byte vectors are the row's pieces 4 x + gl). Slots go in
  // groups of SLG (32 vectors of partials per lane and group at d = 128,
  // where the window's registers are free by now; 8 at d = 64, within the
  // window's budget of four waves per SIMD, since larger groups cost a wave
  // per SIMD and ran slower): a group's partial loads go out together with
  // the next group's scores, ids and entry indices, so that each group costs
  // one load latency.
  constexpr int VPS = 4 * MB * (int)sizeof(T) / 16;
  constexpr int SLG = (DH == 64 ? 8 : 32) / VPS;
  constexpr int NGM = (32 + SLG - 1) / SLG;  // groups at the largest K (32)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = RW * w + 16 * cb + cl;
    const int hh = r % G;
    const bool live = prow[cb] >= 0;
    const int pc = live ? prow[cb] : N - 1;
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pc;
    const int32_t* ids = topk_idx + ((size_t)bg * N + pc) * K;
    const int* rks = rank + ((size_t)bg * N + pc) * K;
    const float* scs = topk_score + ro * K;
    const T* pb = part + (size_t)bg * N * K * G * DH + (size_t)hh * DH;
    // a group's raw meta: the id (empty slot: negative), score and entry
    int mid[2][SLG], mrk[2][SLG];
    float msc[2][SLG];
    auto meta = [&](int gi, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SLG; ++j) {
        const int kk = min(gi * SLG + j, K - 1);
        mid[set][j] = ids[kk];
        msc[set][j] = scs[kk];
        mrk[set][j] = rks[kk];
      }
    };
    meta(0, 0);
#pragma unroll
    for (int gi = 0; gi < NGM; ++gi) {
      if (gi * SLG >= K) break;  // uniform
      const int set = gi & 1;
      float wk[SLG];
      u32x4 pv[SLG][VPS];
#pragma unroll
      for (int j = 0; j < SLG; ++j) {
        const bool sel = live && gi * SLG + j < K && mid[set][j] >= 0;
        wk[j] = sel ? __expf(msc[set][j] - Lr[cb]) : 0.f;
        const u32x4* src = reinterpret_cast<const u32x4*>(pb + (size_t)(sel ? mrk[set][j] : 0) * G * DH) + gl;
#pragma unroll
        for (int x = 0; x < VPS; ++x) pv[j][x] = sel ? src[4 * x] : u32x4{0u, 0u, 0u, 0u};
      }
      if (gi + 1 < NGM && (gi + 1) * SLG < K) meta(gi + 1, set ^ 1);
#pragma unroll
      for (int j = 0; j < SLG; ++j) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int x = 0; x < VPS; ++x) {
            const u16x8 hv = __builtin_bit_cast(u16x8, pv[j][x]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              oacc[2 * x][cb][i] += wk[j] * bf2f(hv[i]);
              oacc[2 * x + 1][cb][i] += wk[j] * bf2f(hv[4 + i]);
            }
          }
        } else {
#pragma unroll
          for (int x = 0; x < VPS; ++x) oacc[x][cb] += wk[j] * __builtin_bit_cast(f32x4, pv[j][x]);
        }
      }
    }
  }

  // write o and lse
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (prow[cb] < 0) continue;
    const int r = RW * w + 16 * cb + cl;
    const size_t ro = ((size_t)b * Hq + g * G + r % G) * N + prow[cb];
    if (gl == 0) lse[ro] = Lr[cb];
    T* dst = o + ro * DH + 4 * gl;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (sizeof(T) == 2) {
        u16x4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = f2bf(oacc[mb][cb][i]);
        *reinterpret_cast<u16x4*>(dst + 16 * mb) = hv;
      } else {
        *reinterpret_cast<f32x4*>(dst + 16 * mb) = oacc[mb][cb];
      }
    }
  }
}

template <typename T, int DH>
size_t cm_window_lds() {
  return sizeof(T) * 2 * (size_t)WSlot<T, DH>::ELEMS;
}

// an upper bound of the work items of one (b, KV head): the sum over chunks
// of ceil(n_c / E) is at most N K / E + C
int cm_max_items(const Dims& p) {
  const long E = CM_ITEM_ROWS / p.G;
  return (int)(((long)p.N * p.K + E - 1) / E + p.C);
}

template <typename T, int G, int DH>
hipError_t cm_chunks_go(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                        const InvIndex& ix, const CmItems& it, void* part, hipStream_t st) {
  const int maxit = cm_max_items(p);
  const size_t lds = sizeof(T) * (size_t)WSlot<T, DH>::ELEMS;
  auto kern = k_fwd_cm_chunks<T, G, DH>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(maxit, p.B * p.Hkv), dim3(256), lds, st,
                     (const T*)q, (const T*)k, (const T*)vt, ix.off, ix.lst, it.items, it.nitems,
                     (T*)part, p.N, Np, p.Hkv, p.K, p.C, maxit, p.scale);
  return hipGetLastError();
}

template <typename T, int G, int DH>
hipError_t cm_window_go(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                        const int32_t* idx, const float* sc, const float* sl, const int* rank,
                        const void* part, void* o, float* lse, hipStream_t st) {
  constexpr int TP = cm_win_rows<DH>() / G;
  const int ntiles = (p.N + TP - 1) / TP;
  const size_t lds = cm_window_lds<T, DH>();
  auto kern = k_fwd_cm_window<T, G, DH>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(cm_win_threads<DH>()), lds, st, (const T*)q, (const T*)k,
                     (const T*)vt, idx, sc, sl, rank, (const T*)part, (T*)o, lse, p.N, Np, p.Hkv, p.K,
                     p.W, p.S, p.scale, ntiles);
  return hipGetLastError();
}

template <typename T>
hipError_t cm_chunks_t(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                       const InvIndex& ix, const CmItems& it, void* part, hipStream_t st) {
  switch (p.G * 1000 + p.d) {
    case 1064: return cm_chunks_go<T, 1, 64>(p, q, k, vt, Np, ix, it, part, st);
    case 1128: return cm_chunks_go<T, 1, 128>(p, q, k, vt, Np, ix, it, part, st);
    case 2064: return cm_chunks_go<T, 2, 64>(p, q, k, vt, Np, ix, it, part, st);
    case 2128: return cm_chunks_go<T, 2, 128>(p, q, k, vt, Np, ix, it, part, st);
    case 4064: return cm_chunks_go<T, 4, 64>(p, q, k, vt, Np, ix, it, part, st);
    case 4128: return cm_chunks_go<T, 4, 128>(p, q, k, vt, Np, ix, it, part, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t cm_window_t(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                       const int32_t* idx, const float* sc, const float* sl, const int* rank,
                       const void* part, void* o, float* lse, hipStream_t st) {
  switch (p.G * 1000 + p.d) {
    case 1064: return cm_window_go<T, 1, 64>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    case 1128: return cm_window_go<T, 1, 128>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    case 2064: return cm_window_go<T, 2, 64>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    case 2128: return cm_window_go<T, 2, 128>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    case 4064: return cm_window_go<T, 4, 64>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    case 4128: return cm_window_go<T, 4, 128>(p, q, k, vt, Np, idx, sc, sl, rank, part, o, lse, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fwd_cm_ok(const Dims& p) {
  if (!inv_index_ok(p)) return false;
  const size_t lds = p.dtype == 1 ? (p.d == 64 ? cm_window_lds<uint16_t, 64>() : cm_window_lds<uint16_t, 128>())
                                  : (p.d == 64 ? cm_window_lds<float, 64>() : cm_window_lds<float, 128>());
  return lds <= 160 * 1024 && (p.G == 1 || p.G == 2 || p.G == 4);
}

size_t fwd_cm_part_bytes(const Dims& p) {
  return (size_t)p.B * p.Hkv * p.N * p.K * p.G * p.d * (p.dtype == 1 ? 2 : 4);
}

size_t fwd_cm_items_carve(const Dims& p, void* base, CmItems* out) {
  char* c = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + o : nullptr;
    o += (bytes + 255) & ~(size_t)255;
    return ptr;
  };
  const size_t bg = (size_t)p.B * p.Hkv;
  out->items = (int2*)take(bg * (size_t)cm_max_items(p) * sizeof(int2));
  out->nitems = (int*)take(bg * sizeof(int));
  out->scratch = (int*)take(bg * (size_t)p.C * sizeof(int));
  return o;
}

hipError_t launch_cm_items(const Dims& p, const InvIndex& ix, const CmItems& it, hipStream_t st) {
  if (p.C == 0) return hipSuccess;
  hipLaunchKernelGGL(k_cm_items, dim3(p.B * p.Hkv), dim3(256), 0, st, ix.off, it.items, it.nitems,
                     it.scratch, p.C, CM_ITEM_ROWS / p.G, cm_max_items(p));
  return hipGetLastError();
}

hipError_t launch_fwd_cm_chunks(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                                const InvIndex& ix, const CmItems& it, void* part, hipStream_t st) {
  if (p.C == 0) return hipSuccess;
  if (p.dtype == 1) return cm_chunks_t<uint16_t>(p, q, k, vt, Np, ix, it, part, st);
  return cm_chunks_t<float>(p, q, k, vt, Np, ix, it, part, st);
}

hipError_t launch_fwd_cm_window(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                                const int32_t* topk_idx, const float* topk_score,
                                const float* sel_lse, const int* rank, const void* part, void* o,
                                float* lse, hipStream_t st) {
  if (p.dtype == 1)
    return cm_window_t<uint16_t>(p, q, k, vt, Np, topk_idx, topk_score, sel_lse, rank, part, o, lse, st);
  return cm_window_t<float>(p, q, k, vt, Np, topk_idx, topk_score, sel_lse, rank, part, o, lse, st);
}

}  // namespace hils
