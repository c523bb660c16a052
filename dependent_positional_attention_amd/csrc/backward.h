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

// The chunk-pair kernels take the query chunks in bands of ceil(sqrt(M)) chunks (M chunks per head) and
// hold the per-pair states of one band at a time, so that the workspace grows as L d sqrt(L / chunk)
// per head rather than as L^2 d / chunk.
inline int64_t bwd_band_chunks(int64_t M) {
  int64_t b = 1;
  while (b * b < M) ++b;
  return b;
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

hipError_t bwd_run(bool bf16, int d, int chunk, const void* q, const void* k, const void* v, const void* w,
                   const float* beta, const float* logf, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* dw, float* dbeta, float* dlogf, int64_t BH, int64_t L,
                   float scale, const bwd_buffers& b, hipStream_t st);

}  // namespace pathattn
