// Host-side interface of the backward pass (backward.hip), shared with the C-ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pathattn {

// Device buffers of the backward pass (fp32), carved from its workspace.
struct bwd_buffers {
  float *qt, *kt, *Pm, *Sm, *fl, *ftot;  // per-chunk terms of the forward (scaled as the forward's)
  float *St, *Gst, *Off;                 // per (query chunk, key chunk) pair of one band: states, their gradients,
                                         // FoX offsets
  float *lse2, *Dv, *drow, *dcol;        // per row: log2-unit lse, dO . o, row and column sums of dz
  float *dqt, *dkt, *dPm, *dSm;          // gradients of the per-chunk terms
  float *dva;                            // dv summed over the bands so far (fp32)
  float *Zi;                             // A^{-1} per chunk (bf16 inputs at d = chunk = 64), else unused
};

// The chunk-pair kernels take the query chunks in bands of 4 ceil(sqrt(M)) chunks (M chunks per head) and
// hold the per-pair states of one band at a time, so that the workspace grows as L d sqrt(L / chunk)
// per head rather than as L^2 d / chunk.  (The key-side sums are re-read and re-written once per band:
// bands twice as wide halve that traffic for about twice the states.  At B=8, H=24, L=4096, per call:
// bands of 2, 4 and 8 ceil(sqrt(M)) chunks 6.00, 5.64-5.71 and 5.60-5.65 ms for 4.4, 6.4 and 7.9 GB.)
#ifndef PATHATTN_BAND_FACTOR
#define PATHATTN_BAND_FACTOR 4
#endif
inline int64_t bwd_band_chunks(int64_t M) {
  int64_t b = 1;
  while (b * b < M) ++b;
  return PATHATTN_BAND_FACTOR * b < M ? PATHATTN_BAND_FACTOR * b : (M > 0 ? M : 1);
}
// Pairs (m, n < m) of the largest band: the per-head slab of the pair states.
inline int64_t bwd_band_pairs(int64_t M) {
  const int64_t G = bwd_band_chunks(M);
  int64_t most = 0;
  for (int64_t mb = 0; mb < M; mb += G) {
    const int64_t me = mb + G < M ? mb + G : M;
    const int64_t p = me * (me - 1) / 2 - mb * (mb - 1) / 2;
    most = p > most ? p : most;
  }
  return most;
}

__host__ __device__ inline int64_t pair_index(int64_t m, int64_t n) { return m * (m - 1) / 2 + n; }

// The chunk-pair kernels run one band of query chunks [mb, me) at a time (bands ascending, about
// sqrt(M) chunks each), so that only that band's pair states are held: the states of pair (m, n < m)
// sit in per-head slabs of `stride` pairs, in pair_index order from (mb, 0).  The key-side sums over
// query chunks carry over from band to band in the workspace (fixed order: deterministic).
struct pair_band {
  int64_t mb, me, stride;
  __host__ __device__ size_t slot(int64_t bh, int64_t m, int64_t n) const {
    return (size_t)bh * stride + (size_t)(pair_index(m, n) - pair_index(mb, 0));
  }
};

// Within an XCD the heads are taken in groups of kBwdHeadGroup, and within a group the q-th block of each
// head goes before the (q+1)-th: the blocks resident at a time then share few heads' tile streams in L2
// (measured at B=8, H=24, L=4096, per call: groups of 1, 2, 4, 8 and all 24 heads 6.15, 6.11, 6.19, 6.20
// and 6.37 ms).
#ifndef PATHATTN_BWD_HGROUP
#define PATHATTN_BWD_HGROUP 2
#endif
constexpr int kBwdXcd = 8;
constexpr int64_t kBwdHeadGroup = PATHATTN_BWD_HGROUP;
// Block -> (batch*head, chunk) of the two chunk-pair kernels (1-D grid of kBwdXcd * ceil(BH / kBwdXcd) * M
// blocks): workgroup b runs on XCD b % 8, each with its own L2, so every block of one (batch, head),
// which all read that head's ktilde, v and P tiles, lands on the same XCD; heads are dealt round-robin
// to XCDs and grouped within an XCD as above.  Returns false for the surplus blocks of XCDs with fewer
// heads.
__device__ __forceinline__ bool bwd_pair_block(int64_t BH, int64_t M, int64_t& bh, int64_t& q) {
  const int64_t xcd = blockIdx.x % kBwdXcd, slot = blockIdx.x / kBwdXcd;
  const int64_t heads_here = (BH - xcd + kBwdXcd - 1) / kBwdXcd;
  if (slot >= heads_here * M) return false;
  const int64_t grp = slot / (kBwdHeadGroup * M), in_grp = slot % (kBwdHeadGroup * M);
  const int64_t gh = heads_here - grp * kBwdHeadGroup < kBwdHeadGroup ? heads_here - grp * kBwdHeadGroup : kBwdHeadGroup;
  bh = xcd + kBwdXcd * (grp * kBwdHeadGroup + in_grp % gh);
  q = in_grp / gh;
  return true;
}

// backward_tiles.hip: one band of the chunk-pair kernels for bf16 inputs at d = chunk = 64 (the prefill's
// bf16 per-chunk terms in qt, kt, Pm, Sm; bf16 pair states in St, Gst).
hipError_t bwd_pair_tiles_run(bool fox, const void* v, const void* out, const void* dout, const float* lse,
                              int64_t BH, int64_t L, float scale, pair_band band, const bwd_buffers& b, void* dv,
                              hipStream_t st);
// backward_tiles.hip: per-chunk gradients (dq, dk, dw, dbeta) of bf16 inputs at d = chunk = 64, from the
// chain's d qtilde, d ktilde, dP, dS and the stored A^{-1} (b.Zi)
hipError_t bwd_chunk_grad_tiles_run(const void* q, const void* k, const void* w, const float* beta, int64_t BH,
                                    int64_t L, const bwd_buffers& b, void* dq, void* dk, void* dw, float* dbeta,
                                    hipStream_t st);

hipError_t bwd_run(bool bf16, int d, int chunk, const void* q, const void* k, const void* v, const void* w,
                   const float* beta, const float* logf, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* dw, float* dbeta, float* dlogf, int64_t BH, int64_t L,
                   float scale, const bwd_buffers& b, hipStream_t st);

}  // namespace pathattn
