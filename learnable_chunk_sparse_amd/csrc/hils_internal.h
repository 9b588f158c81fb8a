// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hils {

struct Dims {
  int dtype;  // 0 fp32, 1 bf16
  int B, Hq, Hkv, G, d;
  int N;      // query/key length (prefill) or cache capacity (decode)
  int S, K, W;
  int C;      // N / S
  int D, r;
  float scale;
  int fwd_strategy = 0;  // prefill forward schedule: 0 by shape, 1 union, 2 compact, 3 chunk-major
};

// Q-Cal: q_hat = q + W_up (W_down h) in fp32; u = W_down h (fp32, optional).
// ntok tokens; token t = b * Nq + i. q: [B, Hq, Nq, d].
hipError_t launch_qcal(const Dims& p, int Nq, const void* q, const void* h, const void* W_down,
                       const void* W_up, float* q_hat, float* u, hipStream_t st);

// Routing over a prefill sequence: scores every distant chunk, GQA max,
// top-K. qs: scoring queries ([B, Hq, N, d], fp32 when q_is_f32 else in the
// input dtype). Writes topk_idx and, if non-null, topk_score.
// u path of the routing (route_u_ok: bf16, G = 1, r in {32, 64}): qs is the raw
// query and u = W_down h [B N, Hq r] fp32 (launch_qcal with no q_hat), klh / klo
// the W_up^T kL planes of launch_route_klp; u == nullptr selects the q_hat path.
struct RouteU {
  const float* u = nullptr;
  const uint16_t* klh = nullptr;
  const uint16_t* kll = nullptr;
};
bool route_u_ok(const Dims& p);
hipError_t launch_route_klp(const Dims& p, const void* W_up, const void* kL, uint16_t* klh,
                            uint16_t* kll, hipStream_t st);
hipError_t launch_route(const Dims& p, const void* qs, bool q_is_f32, const void* kL, const void* e,
                        int32_t* topk_idx, float* topk_score, float* sel_lse, hipStream_t st,
                        const RouteU& ru = RouteU());

// Fused window attention + selected-chunk attention + fusion (the query-major
// strategies). vt: the transposed, token-permuted copy of V that
// launch_vt_perm wrote (attn_fwd_vt_bytes).
hipError_t launch_attn_fwd(const Dims& p, const void* q, const void* k, const void* vt,
                           const int32_t* topk_idx, const float* topk_score, const float* sel_lse,
                           void* o, float* lse, hipStream_t st);
size_t attn_fwd_lds_bytes(const Dims& p);
// the strategy a forward call runs: 1 shared block, 2 bucketed, 3 chunk-major
int fwd_strategy_of(const Dims& p);
// bucketed chunk strategy of the forward (attn_fwd_sparse.hip)
size_t fwd_sparse_lds_bytes(const Dims& p);
hipError_t launch_fwd_sparse(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                             const int32_t* idx, const float* sc, const float* sl, void* o,
                             float* lse, hipStream_t st);
size_t attn_fwd_vt_bytes(const Dims& p);

// Inverse index of a selection (inv_index.hip): per (b, KV head) and chunk,
// the (position << 6 | slot) entries that selected it, ascending by position
// (deterministic). off [B Hkv][C + 1]: first entry of each chunk's list in lst
// [B Hkv][N K]; cnt: per-range counts (scratch).
constexpr int INV_MAX_CHUNKS = 16384;
struct InvIndex {
  int* cnt = nullptr;
  int* off = nullptr;
  int* lst = nullptr;
  int* rank = nullptr;  // optional [B Hkv][N][K]: list index of (position, slot)
  int ns = 1;
};
int inv_ranges(const Dims& p);
bool inv_index_ok(const Dims& p);
size_t inv_index_carve(const Dims& p, void* base, InvIndex* out, bool with_rank = false);
hipError_t launch_inv_index(const Dims& p, const int32_t* topk_idx, const InvIndex& ix,
                            hipStream_t st);

// Chunk-major forward (attn_fwd_cm.hip): each selected chunk is loaded once
// and its selecting rows write their normalised chunk outputs O_c (in the
// input dtype, dims in MFMA-fragment order) to part [B Hkv][entry][G][d] in
// the inverse index's order; the window kernel then computes the window
// attention, the fusion normaliser and o = exp(lse_W - L) O_W +
// sum_k exp(s_k - L) O_{c_k}, finding each entry through ix.rank.
bool fwd_cm_ok(const Dims& p);
size_t fwd_cm_part_bytes(const Dims& p);
// work items of the chunk pass (pieces of the chunks' lists)
struct CmItems {
  int2* items = nullptr;
  int* nitems = nullptr;
  int* scratch = nullptr;
};
size_t fwd_cm_items_carve(const Dims& p, void* base, CmItems* out);
// chunk lists cut into work items (after launch_inv_index)
hipError_t launch_cm_items(const Dims& p, const InvIndex& ix, const CmItems& it, hipStream_t st);
hipError_t launch_fwd_cm_chunks(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                                const InvIndex& ix, const CmItems& it, void* part, hipStream_t st);
hipError_t launch_fwd_cm_window(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                                const int32_t* topk_idx, const float* topk_score,
                                const float* sel_lse, const int* rank, const void* part, void* o,
                                float* lse, hipStream_t st);
hipError_t launch_vt_perm(const Dims& p, const void* v, void* vt, hipStream_t st);

// Decode.
size_t decode_workspace(const Dims& p);
// page_table == nullptr: contiguous caches; otherwise pages of 64 tokens
// (k, v [P, Hkv, 64, d], kL [P, Hkv, d], e [P, Hkv]) with the page of chunk c
// of sequence b at page_table[b * max_pages + c].
hipError_t launch_decode(const Dims& p, const void* q_or_qhat, bool q_is_f32, const void* q,
                         const void* k, const void* v, const int32_t* seq_len,
                         const int32_t* page_table, int max_pages, const void* kL, const void* e,
                         void* o, float* lse, int32_t* topk_idx, void* ws, hipStream_t st);

// Batched GEMM C (+)= A * B on bf16 MFMA (fp32 operands split hi + lo).
// A is M x K: element (m, k) at A[m * lda + k] (akm = false) or A[k * lda + m]
// (akm = true); B is K x N: (k, n) at B[k * ldb + n] (bkm = false) or
// B[n * ldb + k] (bkm = true); C is M x N fp32 at C[m * ldc + n]. Batch
// z = (z1, z2) offsets the operands by z1 * s?1 + z2 * s?2 elements.
// splits > 1 splits K and adds partial tiles atomically (C must be zeroed);
// accumulate adds into C.
struct GemmArgs {
  int M, N, K;
  bool akm, bkm;
  long lda, ldb, ldc;
  int n1 = 1, n2 = 1;
  long sA1 = 0, sA2 = 0, sB1 = 0, sB2 = 0, sC1 = 0, sC2 = 0;
  float* C;
  int splits = 1;
  bool accumulate = false;
  // workspace for split-K partial tiles of the token-major weight-gradient
  // path (gemm_work_bytes); null selects the atomic split-K path
  float* work = nullptr;
};
size_t gemm_work_bytes(const GemmArgs& g);
hipError_t gemm(const GemmArgs& g, const void* A, int a_dtype, const void* B, int b_dtype,
                hipStream_t st);

// Backward.
bool bwd_dq_shared_ok(const Dims& p);
hipError_t launch_bwd_dq_shared(const Dims& p, const void* q, const void* k, const void* v,
                                const void* kt, int Np, const void* dO, const void* kL,
                                const int32_t* topk_idx, const float* sT, const float* lse,
                                float* Dv, float* dq, float* dqhat, float* ds, float* beta,
                                float* delta, hipStream_t st);
size_t bwd_workspace(const Dims& p);
hipError_t launch_bwd(const Dims& p, const void* q, const void* k, const void* v, const void* kL,
                      const void* e, const void* h, const void* W_down, const void* W_up,
                      const void* o, const float* lse, const int32_t* topk_idx, const void* dO,
                      float* dq, float* dk, float* dv, float* dkL, float* de, float* dW_down,
                      float* dW_up, float* dh, void* ws, hipStream_t st);

// Landmark summary (landmark.hip): kL, e of every complete chunk from its
// landmark query, and the backward into the landmark queries and keys.
hipError_t launch_landmark_fwd(const Dims& p, const void* qL, const void* k, void* kL, void* e,
                               float* kL32, float* e32, hipStream_t st);
hipError_t launch_landmark_bwd(const Dims& p, const void* qL, const void* k, const float* dkL,
                               const float* de, float* dqL, float* dk, hipStream_t st);

// HoPE rotation of x [B, H, N, d] into y (may alias x); pos [B, N] or null.
hipError_t launch_hope(int dtype, int B, int H, int N, int d, const void* x, void* y,
                       const int32_t* pos, double base, int train_len, bool interleaved,
                       bool inverse, hipStream_t st);

// One Q-Cal pair shared by all heads: dst = Hq copies of src (bytes_per_head
// a multiple of 16); dst[x] = sum over the Hq blocks of n floats of src.
hipError_t launch_repeat_heads(const void* src, void* dst, size_t bytes_per_head, int Hq,
                               hipStream_t st);
hipError_t launch_sum_heads(const float* src, float* dst, size_t n, int Hq, hipStream_t st);

}  // namespace hils
