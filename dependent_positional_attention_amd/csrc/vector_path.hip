// Vector-ALU PaTH prefill (fp32 arithmetic throughout).
//
// This path serves dtype fp32 (where the matrix cores' bf16 inputs would not
// meet fp32 accuracy) and the small head dims / chunk sizes outside the
// matrix-core kernels.  It follows the same blockwise scheme as the
// matrix-core path (PaTH summary, gist.science/ko/paper/2505.16381, section 3):
//
//   per chunk c (C tokens, rows w_a, q_a, k_a, strengths beta_a):
//     A      = I + diag(beta) * strict_upper(W W^T)            (unit upper triangular)
//     T^{-1} = A^{-1} diag(beta)                              (compact UT form:
//              H_0 ... H_{C-1} = I - W^T T^{-1} W, and every contiguous sub-range
//              uses the matching principal block of T^{-1})
//     U[t][a] = w_t . q_a for t <= a      R[b][s] = k_b . w_s for s > b
//     X = T^{-1} U     Y = R T^{-1}
//     qtilde_a = q_a - sum_s X[s][a] w_s      = H_0 ... H_a q_a          (chunk prefix)
//     ktilde_b = k_b - sum_t Y[b][t] w_t      = H_{C-1} ... H_{b+1} k_b  (chunk suffix)
//     S[a][b]  = q_a . k_b - (Y U)[b][a]      = k_b^T H_{b+1} ... H_a q_a, b <= a
//     P_c      = I - W^T T^{-1} W             = H_0 ... H_{C-1}
//   per query chunk m (right-to-left scan over key chunks n < m):
//     logits vs chunk n use the running query r, which starts at qtilde and is
//     moved across each finished key chunk by r <- P_n r; online softmax.
//
// PaTH-FoX bias F_i - F_j (F = inclusive prefix sum of f) is formed from
// chunk-local prefix sums plus a running sum of chunk totals, so no long
// prefix sums are ever subtracted from each other.
#include "common.h"

namespace pathattn {

// ------------------------------------------------------------------------------------ prep
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void vec_prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ w, const float* __restrict__ beta,
                                                       const float* __restrict__ logf, int64_t L, int64_t M,
                                                       float qscale, float* __restrict__ qt, float* __restrict__ kt,
                                                       float* __restrict__ Pm, float* __restrict__ Sm,
                                                       float* __restrict__ fl, float* __restrict__ ftot) {
  constexpr int CP = C + 1;
  constexpr int ZS = (C * CP > C * D) ? C * CP : C * D;
  extern __shared__ float smem[];
  float* Ws = smem;        // [C][D]
  float* Qs = Ws + C * D;  // [C][D]
  float* Ks = Qs + C * D;  // [C][D]
  float* Bs = Ks + C * D;  // [C]
  float* Az = Bs + C;      // A [C][CP], later Z2 = T^{-1} W [C][D]
  float* Ti = Az + ZS;     // T^{-1} [C][CP]
  float* Us = Ti + C * CP; // U [C][CP]
  float* RX = Us + C * CP; // R, later X [C][CP]
  float* Ys = RX + C * CP; // Y [C][CP]

  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t Lp = M * C;

  for (int e = tid; e < C * D; e += blockDim.x) {
    const int a = e / D, x = e % D;
    const int64_t i = (int64_t)c * C + a;
    const bool ok = i < L;
    const size_t g = ((size_t)bh * L + (ok ? i : 0)) * D + x;
    Ws[e] = ok ? to_f32(w[g]) : 0.f;
    Qs[e] = ok ? to_f32(q[g]) : 0.f;
    Ks[e] = ok ? to_f32(k[g]) : 0.f;
  }
  for (int a = tid; a < C; a += blockDim.x) {
    const int64_t i = (int64_t)c * C + a;
    Bs[a] = i < L ? beta[bh * L + i] : 0.f;  // padded tokens: identity transitions
  }
  if (logf != nullptr && tid == 0) {
    float s = 0.f;
    for (int a = 0; a < C; ++a) {
      const int64_t i = (int64_t)c * C + a;
      s += i < L ? logf[bh * L + i] : 0.f;
      fl[bh * Lp + i] = s;
    }
    ftot[bh * M + c] = s;
  }
  __syncthreads();

  // A (strict upper, scaled by beta of the row), U (t <= a), R (s > b)
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, s = e % C;
    float g = 0.f, u = 0.f, rr = 0.f;
    for (int x = 0; x < D; ++x) {
      const float wr = Ws[r * D + x];
      g += wr * Ws[s * D + x];
      u += wr * Qs[s * D + x];
      rr += Ks[r * D + x] * Ws[s * D + x];
    }
    Az[r * CP + s] = (r < s) ? Bs[r] * g : 0.f;
    Us[r * CP + s] = (r <= s) ? u : 0.f;
    RX[r * CP + s] = (s > r) ? rr : 0.f;
  }
  __syncthreads();

  // T^{-1} = A^{-1} diag(beta): back substitution, one column per thread.
  if (tid < C) {
    const int j = tid;
    for (int i = C - 1; i > j; --i) Ti[i * CP + j] = 0.f;
    Ti[j * CP + j] = 1.f;
    for (int i = j - 1; i >= 0; --i) {
      float s = 0.f;
      for (int kk = i + 1; kk <= j; ++kk) s += Az[i * CP + kk] * Ti[kk * CP + j];
      Ti[i * CP + j] = -s;
    }
    const float bj = Bs[j];
    for (int i = 0; i <= j; ++i) Ti[i * CP + j] *= bj;
  }
  __syncthreads();

  // Y[b][t] = sum_{s=b+1..t} R[b][s] T^{-1}[s][t]
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int b = e / C, t = e % C;
    float y = 0.f;
    for (int s = b + 1; s <= t; ++s) y += RX[b * CP + s] * Ti[s * CP + t];
    Ys[b * CP + t] = y;
  }
  __syncthreads();

  // S[a][b] for b <= a (written out), X[s][a] = sum_{t=s..a} T^{-1}[s][t] U[t][a] (into RX)
  float* Sc = Sm + ((size_t)bh * M + c) * C * C;
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int a = e / C, b = e % C;
    float sv = 0.f;
    if (b <= a) {
      for (int x = 0; x < D; ++x) sv += Qs[a * D + x] * Ks[b * D + x];
      for (int t = b + 1; t <= a; ++t) sv -= Ys[b * CP + t] * Us[t * CP + a];
    }
    Sc[e] = sv * qscale;
    const int s = e / C, aa = e % C;
    float xv = 0.f;
    for (int t = s; t <= aa; ++t) xv += Ti[s * CP + t] * Us[t * CP + aa];
    RX[s * CP + aa] = xv;
  }
  __syncthreads();

  // qtilde, ktilde, Z2 = T^{-1} W
  float* qtc = qt + ((size_t)bh * Lp + (size_t)c * C) * D;
  float* ktc = kt + ((size_t)bh * Lp + (size_t)c * C) * D;
  for (int e = tid; e < C * D; e += blockDim.x) {
    const int a = e / D, x = e % D;
    float qv = Qs[e], kv = Ks[e], zv = 0.f;
    for (int s = 0; s <= a; ++s) qv -= RX[s * CP + a] * Ws[s * D + x];
    for (int t = a + 1; t < C; ++t) kv -= Ys[a * CP + t] * Ws[t * D + x];
    for (int t = a; t < C; ++t) zv += Ti[a * CP + t] * Ws[t * D + x];
    qtc[e] = qv * qscale;
    ktc[e] = kv;
    Az[e] = zv;  // Z2[a][x]
  }
  __syncthreads();

  // P[x][y] = delta_xy - sum_s W[s][x] Z2[s][y]
  float* Pc = Pm + ((size_t)bh * M + c) * D * D;
  for (int e = tid; e < D * D; e += blockDim.x) {
    const int x = e / D, y = e % D;
    float p = (x == y) ? 1.f : 0.f;
    for (int s = 0; s < C; ++s) p -= Ws[s * D + x] * Az[s * D + y];
    Pc[e] = p;
  }
}

// ------------------------------------------------------------------------------------ attention
// One thread per query row of chunk m; the key chunks of the scan are staged in LDS.
template <typename T, int D, int C>
__global__ __launch_bounds__(C) void vec_attn_kernel(const float* __restrict__ qt, const float* __restrict__ kt,
                                                     const T* __restrict__ v, const float* __restrict__ Pm,
                                                     const float* __restrict__ Sm, const float* __restrict__ fl,
                                                     const float* __restrict__ ftot, T* __restrict__ out,
                                                     float* __restrict__ lse, int64_t L, int64_t M) {
  __shared__ float Kl[C * D];
  __shared__ float Vl[C * D];
  __shared__ float Pl[D * D];
  __shared__ float Fl[C];

  const int64_t m = (int64_t)gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int64_t bh = blockIdx.y;
  const int a = threadIdx.x;
  const int64_t Lp = M * C;
  const int64_t i = m * C + a;
  const bool fox = fl != nullptr;

  float o[D], r[D], z[C];
  for (int x = 0; x < D; ++x) o[x] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  auto stage_values = [&](int64_t n) {
    for (int e = threadIdx.x; e < C * D; e += C) {
      const int64_t j = n * C + e / D;
      Vl[e] = j < L ? to_f32(v[((size_t)bh * L + j) * D + e % D]) : 0.f;
    }
    if (fox) Fl[threadIdx.x] = fl[bh * Lp + n * C + threadIdx.x];
  };
  auto absorb = [&]() {
    float bm = -INFINITY;
    for (int b = 0; b < C; ++b) bm = fmaxf(bm, z[b]);
    const float mnew = fmaxf(mrun, bm);
    const float alpha = fast_exp2(mrun - mnew);
    lrun *= alpha;
    for (int x = 0; x < D; ++x) o[x] *= alpha;
    for (int b = 0; b < C; ++b) {
      const float p = fast_exp2(z[b] - mnew);
      lrun += p;
      for (int x = 0; x < D; ++x) o[x] += p * Vl[b * D + x];
    }
    mrun = mnew;
  };

  // diagonal block: precomputed in-chunk logits
  stage_values(m);
  __syncthreads();
  const float* Srow = Sm + (((size_t)bh * M + m) * C + a) * C;
  for (int b = 0; b < C; ++b) z[b] = (b <= a) ? Srow[b] - (fox ? kLog2e * Fl[b] : 0.f) : -INFINITY;
  absorb();

  for (int x = 0; x < D; ++x) r[x] = qt[((size_t)bh * Lp + i) * D + x];
  float off = 0.f;  // sum of chunk log-forget totals over chunks n..m-1
  for (int64_t n = m - 1; n >= 0; --n) {
    __syncthreads();
    for (int e = threadIdx.x; e < C * D; e += C) Kl[e] = kt[((size_t)bh * Lp + n * C) * D + e];
    for (int e = threadIdx.x; e < D * D; e += C) Pl[e] = Pm[((size_t)bh * M + n) * D * D + e];
    stage_values(n);
    __syncthreads();
    if (fox) off += ftot[bh * M + n];
    for (int b = 0; b < C; ++b) {
      float s = 0.f;
      for (int x = 0; x < D; ++x) s += Kl[b * D + x] * r[x];
      z[b] = s + (fox ? kLog2e * (off - Fl[b]) : 0.f);
    }
    absorb();
    if (n > 0) {
      float nr[D];
      for (int x = 0; x < D; ++x) {
        float s = 0.f;
        for (int y = 0; y < D; ++y) s += Pl[x * D + y] * r[y];
        nr[x] = s;
      }
      for (int x = 0; x < D; ++x) r[x] = nr[x];
    }
  }

  if (i < L) {
    const float inv = 1.f / lrun;
    for (int x = 0; x < D; ++x) out[((size_t)bh * L + i) * D + x] = from_f32<T>(o[x] * inv);
    if (lse != nullptr) {
      const float fa = fox ? fl[bh * Lp + i] : 0.f;
      lse[bh * L + i] = (mrun + fast_log2(lrun)) * kLn2 + fa;
    }
  }
}

// ------------------------------------------------------------------------------------ decode cache
// Prefill -> decode hand-off (inference rule of the same section: a decode cache slot j holds
// H_{L-1} ... H_{j+1} k_j).  With R_n = P_{n+1} ... P_{M-1} (identity for the last chunk), the
// slots of chunk n are the rows ktilde_n R_n; R is carried right to left, R_{n-1} = P_n R_n, in LDS,
// one block per (batch, head).  Values are copied alongside.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void vec_cache_kernel(const float* __restrict__ kt, const float* __restrict__ Pm,
                                                        const T* __restrict__ v, int64_t L, int64_t M, int64_t cap,
                                                        T* __restrict__ kc, T* __restrict__ vc) {
  __shared__ float R[2][D * D];
  const int64_t bh = blockIdx.x, Lp = M * C;
  const int tid = threadIdx.x;
  for (int e = tid; e < D * D; e += blockDim.x) R[0][e] = (e / D == e % D) ? 1.f : 0.f;
  __syncthreads();
  int cur = 0;
  for (int64_t n = M - 1; n >= 0; --n) {
    const float* Rc = R[cur];
    for (int e = tid; e < C * D; e += blockDim.x) {
      const int b = e / D, y = e % D;
      const int64_t j = n * C + b;
      if (j < L) {
        const float* kr = kt + ((size_t)bh * Lp + j) * D;
        float s = 0.f;
        for (int m = 0; m < D; ++m) s += kr[m] * Rc[m * D + y];
        kc[((size_t)bh * cap + j) * D + y] = from_f32<T>(s);
        vc[((size_t)bh * cap + j) * D + y] = v[((size_t)bh * L + j) * D + y];
      }
    }
    if (n > 0) {
      float* Rn = R[cur ^ 1];
      const float* Pn = Pm + ((size_t)bh * M + n) * D * D;
      for (int e = tid; e < D * D; e += blockDim.x) {
        const int x = e / D, y = e % D;
        float s = 0.f;
        for (int m = 0; m < D; ++m) s += Pn[x * D + m] * Rc[m * D + y];
        Rn[e] = s;
      }
    }
    __syncthreads();
    cur ^= 1;
  }
}

// ------------------------------------------------------------------------------------ launch
// phases: bit 0 = per-chunk prep, bit 1 = attention scan (reads what the prep left in the workspace).
template <typename T, int D, int C>
static hipError_t launch_vec(int phases, const void* q, const void* k, const void* v, const void* w,
                             const float* beta, const float* logf, void* out, float* lse, int64_t BH, int64_t L,
                             float scale, float* qt, float* kt, float* Pm, float* Sm, float* fl, float* ftot,
                             hipStream_t st) {
  const int64_t M = (L + C - 1) / C;
  constexpr int CP = C + 1;
  constexpr int ZS = (C * CP > C * D) ? C * CP : C * D;
  constexpr size_t lds = sizeof(float) * (3 * C * D + C + ZS + 4 * C * CP);
  static_assert(lds <= 160 * 1024, "vector prep exceeds LDS");
  dim3 grid((unsigned)M, (unsigned)BH);
  hipError_t e = hipSuccess;
  if (phases & 1) {
    e = hipFuncSetAttribute((const void*)vec_prep_kernel<T, D, C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
    vec_prep_kernel<T, D, C><<<grid, 256, lds, st>>>((const T*)q, (const T*)k, (const T*)w, beta, logf, L, M,
                                                    scale * kLog2e, qt, kt, Pm, Sm, fl, ftot);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    vec_attn_kernel<T, D, C><<<grid, C, 0, st>>>(qt, kt, (const T*)v, Pm, Sm, logf ? fl : nullptr, ftot, (T*)out,
                                                 lse, L, M);
    e = hipGetLastError();
  }
  return e;
}

#define PATHATTN_VEC_CASE(TT, DD, CC)                                                                              \
  if (d == DD && chunk == CC)                                                                                      \
    return launch_vec<TT, DD, CC>(phases, q, k, v, w, beta, logf, out, lse, BH, L, scale, qt, kt, Pm, Sm, fl, ftot, \
                                  st);

template <typename T>
static hipError_t dispatch_vec(int phases, int d, int chunk, const void* q, const void* k, const void* v,
                               const void* w, const float* beta, const float* logf, void* out, float* lse,
                               int64_t BH, int64_t L, float scale, float* qt, float* kt, float* Pm, float* Sm,
                               float* fl, float* ftot, hipStream_t st) {
  PATHATTN_VEC_CASE(T, 16, 16)
  PATHATTN_VEC_CASE(T, 16, 32)
  PATHATTN_VEC_CASE(T, 16, 64)
  PATHATTN_VEC_CASE(T, 32, 16)
  PATHATTN_VEC_CASE(T, 32, 32)
  PATHATTN_VEC_CASE(T, 32, 64)
  PATHATTN_VEC_CASE(T, 64, 16)
  PATHATTN_VEC_CASE(T, 64, 32)
  PATHATTN_VEC_CASE(T, 64, 64)
  return hipErrorInvalidValue;
}
#undef PATHATTN_VEC_CASE

template <typename T>
static hipError_t dispatch_vec_cache(int d, int chunk, const float* kt, const float* Pm, const void* v, int64_t BH,
                                     int64_t L, int64_t cap, void* kc, void* vc, hipStream_t st) {
  const int64_t M = (L + chunk - 1) / chunk;
#define PATHATTN_VEC_CACHE_CASE(DD, CC)                                                                     \
  if (d == DD && chunk == CC) {                                                                             \
    vec_cache_kernel<T, DD, CC><<<dim3((unsigned)BH), 256, 0, st>>>(kt, Pm, (const T*)v, L, M, cap, (T*)kc, \
                                                                    (T*)vc);                                \
    return hipGetLastError();                                                                               \
  }
  PATHATTN_VEC_CACHE_CASE(16, 16)
  PATHATTN_VEC_CACHE_CASE(16, 32)
  PATHATTN_VEC_CACHE_CASE(16, 64)
  PATHATTN_VEC_CACHE_CASE(32, 16)
  PATHATTN_VEC_CACHE_CASE(32, 32)
  PATHATTN_VEC_CACHE_CASE(32, 64)
  PATHATTN_VEC_CACHE_CASE(64, 16)
  PATHATTN_VEC_CACHE_CASE(64, 32)
  PATHATTN_VEC_CACHE_CASE(64, 64)
#undef PATHATTN_VEC_CACHE_CASE
  return hipErrorInvalidValue;
}

hipError_t vec_cache_run(bool bf16, int d, int chunk, const float* kt, const float* Pm, const void* v, int64_t BH,
                         int64_t L, int64_t cap, void* kc, void* vc, hipStream_t st) {
  if (bf16) return dispatch_vec_cache<__bf16>(d, chunk, kt, Pm, v, BH, L, cap, kc, vc, st);
  return dispatch_vec_cache<float>(d, chunk, kt, Pm, v, BH, L, cap, kc, vc, st);
}

bool vec_supported(int d, int chunk) {
  return (d == 16 || d == 32 || d == 64) && (chunk == 16 || chunk == 32 || chunk == 64);
}

hipError_t vec_run(int phases, bool bf16, int d, int chunk, const void* q, const void* k, const void* v,
                   const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH, int64_t L,
                   float scale, float* qt, float* kt, float* Pm, float* Sm, float* fl, float* ftot, hipStream_t st) {
  if (bf16)
    return dispatch_vec<__bf16>(phases, d, chunk, q, k, v, w, beta, logf, out, lse, BH, L, scale, qt, kt, Pm, Sm, fl,
                                ftot, st);
  return dispatch_vec<float>(phases, d, chunk, q, k, v, w, beta, logf, out, lse, BH, L, scale, qt, kt, Pm, Sm, fl,
                             ftot, st);
}

}  // namespace pathattn
