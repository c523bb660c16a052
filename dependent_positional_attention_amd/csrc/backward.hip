// PaTH / PaTH-FoX backward pass.  fp32 accumulation throughout.  At d = chunk = 64 the 64 x 64 x 64
// products run on the matrix cores: fp32 (16x16x4) for fp32 inputs; bf16 (16x16x32) for bf16 inputs,
// where a product of input values (w, q, k, v, dO are bf16 numbers) is exact and any other fp32 operand
// is split into hi + lo bf16 (hi*hi + hi*lo + lo*hi, about 2^-16 relative).  Other sizes use the fp32
// vector-ALU kernels.
//
// The pages give the forward only (PaTH summary, gist.science/ko/paper/2505.16381, section 3, and the
// lecture notes on PaTH, brianyu43.github.io/gpumode/lecture_074.html, whose "limitations" part only
// says the backward costs more than RoPE's).  This file differentiates the blockwise forward of
// vector_path.hip step by step, chunk size C, head dim D:
//
//   forward per query chunk m:  r^(m-1) = qtilde_m (scaled by scale*log2e),
//                               z_mn = r^(n) ktilde_n^T (+ FoX bias), r^(n-1) = r^(n) P_n^T
//   backward per query chunk m: the states r^(n) are kept (they cannot be recovered from r^(n-1):
//                               P_n is singular when some beta_s = 1; the query chunks go in bands
//                               of about sqrt(M), so only one band's states are held), then, for
//                               n = 0 .. m-1,
//                               dr^(n) = g_mn ktilde_n + dr^(n-1) P_n,   g = ln2 * dz
//   dP_n     = sum_{m > n} dr^(n-1)_m^T r^(n)_m          (d x d, reduced per key chunk)
//   dktilde_n = sum_{m > n} g_mn^T r^(n)_m,  dv_n = sum_{m >= n} p_mn^T dO_m
//   dz_ij    = p_ij (dO_i . v_j - D_i),  D_i = dO_i . o_i,  p_ij = exp2(z2_ij - lse2_i)
//
// then each chunk's UT-transform terms (qtilde, ktilde, P, in-chunk logits S) are differentiated back
// to q, k, w, beta:
//
//   A = I + diag(beta) strict_upper(W W^T),  Ti = A^{-1} diag(beta)
//   U = (W Q^T) on t <= a,  R = (K W^T) on s > b,  X = Ti U,  Y = R Ti
//   qtilde = Q - X^T W,  ktilde = K - Y W,  P = I - W^T Ti W,  S^T = (K Q^T - Y U) on b <= a
//
//   dX = -W dqtilde^T      dY = -dktilde W^T - dS^T U^T      dU = Ti^T dX - (dS Y)^T      dR = dY Ti^T
//   dTi = dX U^T + R^T dY - W dP W^T
//   dA  = -A^{-T} dTi Ti^T (strict upper),  dbeta = diag(A^{-T} dTi) + rowsum(dA o W W^T)
//   dW  = -X dqtilde - Y^T dktilde - Ti W dP^T - Ti^T W dP + dU Q + dR^T K + (dN + dN^T) W,
//         dN = diag(beta) dA
//   dQ  = dqtilde + dS K + dU^T W,   dK = dktilde + dS^T Q + dR W
//
// PaTH-FoX: z_ij carries F_i - F_j, so dF_t = sum_j dz_tj - sum_i dz_it and df_s = sum_{t >= s} dF_t.
#include <type_traits>

#include "backward.h"
#include "common.h"

namespace pathattn {

namespace {

template <int C, int D>
struct BwdShape {
  static constexpr int DP = D + 1, CP = C + 1, CD = C * D, CC = C * C;
  static constexpr int NE = (CD + 255) / 256;  // C x D elements per thread
  static constexpr int NC = (CC + 255) / 256;  // C x C elements per thread
  static constexpr int NDD = (D * D + 255) / 256;
  static constexpr int SL = (C * CP > C * DP ? (C * CP > D * DP ? C * CP : D * DP) : (C * DP > D * DP ? C * DP : D * DP));
  static constexpr size_t lds_query = sizeof(float) * (5 * C * DP + D * DP + C * CP + 4 * C);
  static constexpr size_t lds_key = sizeof(float) * (5 * C * DP + 2 * C * CP + 4 * C);
  static constexpr size_t lds_prep = sizeof(float) * (9 * SL + 2 * C);
};


}  // namespace

// ------------------------------------------------------------------------------- query chunks
// One block per (query chunk m of the band, batch*head).  Writes the states r^(n) and incoming
// gradients dr^(n-1) of every pair (m, n < m), the FoX offsets of each pair, the row statistics, the
// in-chunk logit gradient dS (unscaled units), d qtilde (unscaled) and the row sums of dz.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void bwd_query_kernel(
    const float* __restrict__ qt, const float* __restrict__ kt, const float* __restrict__ Pm,
    const float* __restrict__ Sm, const float* __restrict__ fl, const float* __restrict__ ftot,
    const T* __restrict__ v, const T* __restrict__ out, const T* __restrict__ dout, const float* __restrict__ lse,
    int64_t L, int64_t M, float scale, pair_band band, float* __restrict__ St, float* __restrict__ Gst,
    float* __restrict__ Off, float* __restrict__ lse2w, float* __restrict__ Dw, float* __restrict__ drow,
    float* __restrict__ dqt, float* __restrict__ dSm) {
  using S = BwdShape<C, D>;
  constexpr int DP = S::DP, CP = S::CP, CD = S::CD, NE = S::NE;
  extern __shared__ float sm[];
  float* Rs = sm;           // r^(n)          [C][DP]
  float* Ks = Rs + C * DP;  // ktilde_n       [C][DP]
  float* Vs = Ks + C * DP;  // v_n            [C][DP]
  float* Os = Vs + C * DP;  // dO_m           [C][DP]
  float* Qd = Os + C * DP;  // dr^(n-1)       [C][DP]
  float* Ps = Qd + C * DP;  // P_n            [D][DP]
  float* Gs = Ps + D * DP;  // dz             [C][CP]
  float* l2 = Gs + C * CP;  // lse2 of the rows
  float* Dv = l2 + C;       // D of the rows
  float* Fn = Dv + C;       // local FoX prefix of key chunk n
  float* rs = Fn + C;       // row sums of dz

  const int tid = threadIdx.x;
  const int64_t m = band.me - 1 - blockIdx.x;  // longest rows of the band first
  const int64_t bh = blockIdx.y, Lp = M * C;
  const bool fox = fl != nullptr;
  const size_t row0 = (size_t)bh * Lp + (size_t)m * C;

  auto stage_rows = [&](float* dst, const T* src, int64_t c0) PA_INLINE {
    for (int e = tid; e < CD; e += 256) {
      const int a = e / D, x = e % D;
      const int64_t i = c0 + a;
      dst[a * DP + x] = i < L ? to_f32(src[((size_t)bh * L + i) * D + x]) : 0.f;
    }
  };

  stage_rows(Os, dout, m * C);
  __syncthreads();
  for (int a = tid; a < C; a += 256) {
    const int64_t i = m * C + a;
    float dv = 0.f, l2v = INFINITY;  // padded rows: p = 0
    if (i < L) {
      const T* orow = out + ((size_t)bh * L + i) * D;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) dv += Os[a * DP + x] * to_f32(orow[x]);
      l2v = kLog2e * (lse[bh * L + i] - (fox ? fl[row0 + a] : 0.f));
    }
    Dv[a] = dv;
    l2[a] = l2v;
    rs[a] = 0.f;
    lse2w[row0 + a] = l2v;
    Dw[row0 + a] = dv;
  }

  // pass 1: states r^(n), n = m-1 .. 0, in the forward's order (and its FoX offsets)
  float R[NE], G[NE];
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    R[j] = e < CD ? qt[row0 * D + e] : 0.f;
    G[j] = 0.f;
  }
  float off = 0.f;
  for (int64_t n = m - 1; n >= 0; --n) {
    const size_t pr = band.slot(bh, m, n);
    if (fox) off += ftot[bh * M + n];
    if (tid == 0) Off[pr] = off;
    for (int j = 0; j < NE; ++j) {
      const int e = tid + 256 * j;
      if (e < CD) St[pr * CD + e] = R[j];
    }
    if (n > 0) {
      for (int j = 0; j < NE; ++j) {
        const int e = tid + 256 * j;
        if (e < CD) Rs[(e / D) * DP + e % D] = R[j];
      }
      const float* Pn = Pm + ((size_t)bh * M + n) * D * D;
      for (int e = tid; e < D * D; e += 256) Ps[(e / D) * DP + e % D] = Pn[e];
      __syncthreads();
      for (int j = 0; j < NE; ++j) {
        const int e = tid + 256 * j;
        if (e < CD) {
          const int a = e / D, x = e % D;
          float s = 0.f;
          #pragma unroll 4
          for (int y = 0; y < D; ++y) s += Rs[a * DP + y] * Ps[x * DP + y];
          R[j] = s;
        }
      }
      __syncthreads();
    }
  }

  // in-chunk block: logits from S
  stage_rows(Vs, v, m * C);
  if (fox)
    for (int a = tid; a < C; a += 256) Fn[a] = fl[row0 + a];
  __syncthreads();
  {
    const float* Sc = Sm + ((size_t)bh * M + m) * C * C;
    float* dSc = dSm + ((size_t)bh * M + m) * C * C;
    for (int e = tid; e < C * C; e += 256) {
      const int a = e / C, b = e % C;
      float dz = 0.f;
      if (b <= a) {
        const float z2 = Sc[e] - (fox ? kLog2e * Fn[b] : 0.f);
        const float p = fast_exp2(z2 - l2[a]);
        float dp = 0.f;
        #pragma unroll 4
        for (int x = 0; x < D; ++x) dp += Os[a * DP + x] * Vs[b * DP + x];
        dz = p * (dp - Dv[a]);
      }
      Gs[a * CP + b] = dz;
      dSc[e] = scale * dz;
    }
  }
  __syncthreads();
  for (int a = tid; a < C; a += 256) {
    float s = 0.f;
    #pragma unroll 4
    for (int b = 0; b < C; ++b) s += Gs[a * CP + b];
    rs[a] += s;
  }

  // pass 2: n = 0 .. m-1, gradients flow back up the chain of transports
  for (int64_t n = 0; n < m; ++n) {
    const size_t pr = band.slot(bh, m, n);
    __syncthreads();
    for (int j = 0; j < NE; ++j) {
      const int e = tid + 256 * j;
      if (e < CD) {
        const int a = e / D, x = e % D;
        Rs[a * DP + x] = St[pr * CD + e];
        Ks[a * DP + x] = kt[((size_t)bh * Lp + (size_t)n * C) * D + e];
        if (n > 0) {
          Qd[a * DP + x] = G[j];
          Gst[pr * CD + e] = G[j];
        }
      }
    }
    stage_rows(Vs, v, n * C);
    if (n > 0) {
      const float* Pn = Pm + ((size_t)bh * M + n) * D * D;
      for (int e = tid; e < D * D; e += 256) Ps[(e / D) * DP + e % D] = Pn[e];
    }
    if (fox)
      for (int a = tid; a < C; a += 256) Fn[a] = fl[(size_t)bh * Lp + (size_t)n * C + a];
    const float offn = fox ? Off[pr] : 0.f;
    __syncthreads();
    for (int e = tid; e < C * C; e += 256) {
      const int a = e / C, b = e % C;
      float z2 = fox ? kLog2e * (offn - Fn[b]) : 0.f, dp = 0.f;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) {
        z2 += Rs[a * DP + x] * Ks[b * DP + x];
        dp += Os[a * DP + x] * Vs[b * DP + x];
      }
      const float p = fast_exp2(z2 - l2[a]);
      Gs[a * CP + b] = p * (dp - Dv[a]);
    }
    __syncthreads();
    for (int a = tid; a < C; a += 256) {
      float s = 0.f;
      #pragma unroll 4
      for (int b = 0; b < C; ++b) s += Gs[a * CP + b];
      rs[a] += s;
    }
    for (int j = 0; j < NE; ++j) {
      const int e = tid + 256 * j;
      if (e < CD) {
        const int a = e / D, y = e % D;
        float s = 0.f, t = 0.f;
        if (n > 0)
          #pragma unroll 4
          for (int x = 0; x < D; ++x) s += Qd[a * DP + x] * Ps[x * DP + y];
        #pragma unroll 4
        for (int b = 0; b < C; ++b) t += Gs[a * CP + b] * Ks[b * DP + y];
        G[j] = s + kLn2 * t;
      }
    }
  }

  const float c = scale * kLog2e;  // qtilde entered the scan scaled by c
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) dqt[row0 * D + e] = c * G[j];
  }
  for (int a = tid; a < C; a += 256) drow[row0 + a] = rs[a];
}

// ------------------------------------------------------------------------------- key chunks
// One block per (key chunk n < me, batch*head): the band's share of dv, d ktilde, dP_n and the column
// sums of dz.  The band holding query chunk n starts the sums (with the in-chunk block); later bands add
// to them (dv in fp32 in `dva` until the last band rounds it to the output dtype).
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void bwd_key_kernel(
    const float* __restrict__ kt, const float* __restrict__ Sm, const float* __restrict__ fl,
    const T* __restrict__ v, const T* __restrict__ dout, const float* __restrict__ St, const float* __restrict__ Gst,
    const float* __restrict__ Off, const float* __restrict__ lse2w, const float* __restrict__ Dw, int64_t L,
    int64_t M, pair_band band, T* __restrict__ dv, float* __restrict__ dva, float* __restrict__ dkt,
    float* __restrict__ dPm, float* __restrict__ dcol) {
  using S = BwdShape<C, D>;
  constexpr int DP = S::DP, CP = S::CP, CD = S::CD, NE = S::NE, NDD = S::NDD;
  extern __shared__ float sm[];
  float* Ks = sm;           // ktilde_n  [C][DP]
  float* Vs = Ks + C * DP;  // v_n
  float* Rs = Vs + C * DP;  // r^(n)_m
  float* Os = Rs + C * DP;  // dO_m
  float* Gq = Os + C * DP;  // dr^(n-1)_m
  float* Pp = Gq + C * DP;  // p     [C][CP]
  float* Zs = Pp + C * CP;  // dz    [C][CP]
  float* l2 = Zs + C * CP;
  float* Dv = l2 + C;
  float* Fn = Dv + C;
  float* cs = Fn + C;

  const int tid = threadIdx.x;
  const int64_t n = blockIdx.x, bh = blockIdx.y, Lp = M * C;
  const bool fox = fl != nullptr;
  const size_t rown = (size_t)bh * Lp + (size_t)n * C;
  const bool first = n >= band.mb;  // query chunk n is in this band: the sums start here
  const bool last = band.me == M;   // the sums end here

  auto stage_rows = [&](float* dst, const T* src, int64_t c0) PA_INLINE {
    for (int e = tid; e < CD; e += 256) {
      const int a = e / D, x = e % D;
      const int64_t i = c0 + a;
      dst[a * DP + x] = i < L ? to_f32(src[((size_t)bh * L + i) * D + x]) : 0.f;
    }
  };
  auto stage_stats = [&](int64_t mm) PA_INLINE {
    const size_t r0 = (size_t)bh * Lp + (size_t)mm * C;
    for (int a = tid; a < C; a += 256) {
      l2[a] = lse2w[r0 + a];
      Dv[a] = Dw[r0 + a];
    }
  };

  for (int e = tid; e < CD; e += 256) Ks[(e / D) * DP + e % D] = kt[rown * D + e];
  stage_rows(Vs, v, n * C);
  for (int a = tid; a < C; a += 256) {
    Fn[a] = fox ? fl[rown + a] : 0.f;
    cs[a] = first ? 0.f : dcol[rown + a];
  }
  float aK[NE], aV[NE], aP[NDD];
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    aK[j] = (!first && e < CD) ? dkt[rown * D + e] : 0.f;
    aV[j] = (!first && e < CD) ? dva[rown * D + e] : 0.f;
  }
  for (int j = 0; j < NDD; ++j) {
    const int e = tid + 256 * j;
    aP[j] = (!first && e < D * D) ? dPm[((size_t)bh * M + n) * D * D + e] : 0.f;
  }

  // in-chunk block
  if (first) {
  stage_rows(Os, dout, n * C);
  stage_stats(n);
  __syncthreads();
  {
    const float* Sc = Sm + ((size_t)bh * M + n) * C * C;
    for (int e = tid; e < C * C; e += 256) {
      const int a = e / C, b = e % C;
      float p = 0.f, dz = 0.f;
      if (b <= a) {
        const float z2 = Sc[e] - (fox ? kLog2e * Fn[b] : 0.f);
        p = fast_exp2(z2 - l2[a]);
        float dp = 0.f;
        #pragma unroll 4
        for (int x = 0; x < D; ++x) dp += Os[a * DP + x] * Vs[b * DP + x];
        dz = p * (dp - Dv[a]);
      }
      Pp[a * CP + b] = p;
      Zs[a * CP + b] = dz;
    }
  }
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int b = e / D, x = e % D;
      float s = 0.f;
      #pragma unroll 4
      for (int a = 0; a < C; ++a) s += Pp[a * CP + b] * Os[a * DP + x];
      aV[j] += s;
    }
  }
  for (int b = tid; b < C; b += 256) {
    float s = 0.f;
    #pragma unroll 4
    for (int a = 0; a < C; ++a) s += Zs[a * CP + b];
    cs[b] += s;
  }
  }

  for (int64_t m = (n + 1 > band.mb ? n + 1 : band.mb); m < band.me; ++m) {
    const size_t pr = band.slot(bh, m, n);
    __syncthreads();
    for (int e = tid; e < CD; e += 256) {
      const int a = e / D, x = e % D;
      Rs[a * DP + x] = St[pr * CD + e];
      if (n > 0) Gq[a * DP + x] = Gst[pr * CD + e];
    }
    stage_rows(Os, dout, m * C);
    stage_stats(m);
    const float offn = fox ? Off[pr] : 0.f;
    __syncthreads();
    for (int e = tid; e < C * C; e += 256) {
      const int a = e / C, b = e % C;
      float z2 = fox ? kLog2e * (offn - Fn[b]) : 0.f, dp = 0.f;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) {
        z2 += Rs[a * DP + x] * Ks[b * DP + x];
        dp += Os[a * DP + x] * Vs[b * DP + x];
      }
      const float p = fast_exp2(z2 - l2[a]);
      Pp[a * CP + b] = p;
      Zs[a * CP + b] = p * (dp - Dv[a]);
    }
    __syncthreads();
    for (int j = 0; j < NE; ++j) {
      const int e = tid + 256 * j;
      if (e < CD) {
        const int b = e / D, x = e % D;
        float sv = 0.f, sk = 0.f;
        #pragma unroll 4
        for (int a = 0; a < C; ++a) {
          sv += Pp[a * CP + b] * Os[a * DP + x];
          sk += Zs[a * CP + b] * Rs[a * DP + x];
        }
        aV[j] += sv;
        aK[j] += kLn2 * sk;
      }
    }
    for (int b = tid; b < C; b += 256) {
      float s = 0.f;
      #pragma unroll 4
      for (int a = 0; a < C; ++a) s += Zs[a * CP + b];
      cs[b] += s;
    }
    if (n > 0)
      for (int j = 0; j < NDD; ++j) {
        const int e = tid + 256 * j;
        if (e < D * D) {
          const int x = e / D, y = e % D;
          float s = 0.f;
          #pragma unroll 4
          for (int a = 0; a < C; ++a) s += Gq[a * DP + x] * Rs[a * DP + y];
          aP[j] += s;
        }
      }
  }

  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int b = e / D;
      dkt[rown * D + e] = aK[j];
      if (!last) dva[rown * D + e] = aV[j];
      else if (n * C + b < L) dv[((size_t)bh * L + n * C + b) * D + e % D] = from_f32<T>(aV[j]);
    }
  }
  for (int j = 0; j < NDD; ++j) {
    const int e = tid + 256 * j;
    if (e < D * D) dPm[((size_t)bh * M + n) * D * D + e] = aP[j];
  }
  for (int b = tid; b < C; b += 256) dcol[rown + b] = cs[b];
}

// ------------------------------------------------------------------------------- matrix-core variants
// C = D = 64: the 64 x 64 x 64 products of the chunk-pair kernels run on the matrix cores: the fp32 ones
// (16x16x4, the helpers here) for fp32 inputs, so the fp32 accuracy is kept, and the bf16 ones (16x16x32,
// the helpers further down: exact for products of input values, hi + lo splits otherwise) for bf16
// inputs.  Four waves; wave w owns output rows 16w .. 16w+15.
// Tiles are row-major in LDS with a 68-float row stride (16-byte aligned rows).  In one 16x16x4 step
// lane (r, g) (r = lane % 16, g = lane / 16) brings A[row r][slot g] and B[slot g][col r], and holds
// D[4g + e][r] (e = 0..3) of the accumulator; within 16-wide k blocks slot g of step j is
// k = k0 + 4g + j, so an operand stored k-contiguous is read as one float4.
namespace {

constexpr int kS = 68;  // LDS row stride (floats) of the 64-wide tiles

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc[cb] += sum_{k<64} A(16w + r', k) B(k, 16cb + r'') over the wave's strip; SA, SB are the
// operands' row strides (kS for LDS tiles, 64 for fp32 tiles read straight from global memory).
//   AT = false: A(i, k) = A[i][k] (float4 reads)    AT = true: A(i, k) = A[k][i]
//   BK = false: B(k, j) = B[j][k] (float4 reads)    BK = true: B(k, j) = B[k][j]
// (acc[c] holds column block cb0 + c: a wave may cover NC < 4 of the four)
template <bool AT, bool BK, int SA = kS, int SB = kS, int NC>
__device__ __forceinline__ void mm64(f32x4 (&acc)[NC], const float* __restrict__ A, const float* __restrict__ B,
                                     int w, int lane, int cb0 = 0) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < 64; k0 += 16) {
    float a[4];
    if constexpr (!AT) {
      const float4 v = *reinterpret_cast<const float4*>(A + (16 * w + r) * SA + k0 + 4 * g);
      a[0] = v.x, a[1] = v.y, a[2] = v.z, a[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = A[(k0 + 4 * g + j) * SA + 16 * w + r];
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cb = cb0 + c;
      float b[4];
      if constexpr (!BK) {
        const float4 v = *reinterpret_cast<const float4*>(B + (16 * cb + r) * SB + k0 + 4 * g);
        b[0] = v.x, b[1] = v.y, b[2] = v.z, b[3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = B[(k0 + 4 * g + j) * SB + 16 * cb + r];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[c] = mfma4(a[j], b[j], acc[c]);
    }
  }
}

template <int NC>
__device__ __forceinline__ void zero4(f32x4 (&acc)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// accumulator layout <-> row-major 64 x 64 (LDS stride kS, or global stride 64)
__device__ __forceinline__ void acc_to_lds(const f32x4 (&acc)[4], float* T, int w, int lane, float mul = 1.f) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) T[(16 * w + 4 * g + e) * kS + 16 * cb + r] = mul * acc[cb][e];
}
__device__ __forceinline__ void acc_to_global(const f32x4 (&acc)[4], float* T, int w, int lane, float mul = 1.f) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) T[(16 * w + 4 * g + e) * 64 + 16 * cb + r] = mul * acc[cb][e];
}
template <int NC>
__device__ __forceinline__ void global_to_acc(f32x4 (&acc)[NC], const float* T, int w, int lane, int cb0 = 0) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c][e] = T[(16 * w + 4 * g + e) * 64 + 16 * (cb0 + c) + r];
}

// 64 rows of a [.., L, 64] input starting at row c0 (rows >= L read as zero), widened to fp32.
template <typename T>
__device__ __forceinline__ void tile_rows(float* dst, const T* __restrict__ src, int64_t c0, int64_t L, int tid,
                                          int nt = 256) {
  for (int e = tid; e < 64 * 16; e += nt) {
    const int row = e >> 4, c4 = (e & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c0 + row < L) {
      const T* p = src + (size_t)(c0 + row) * 64 + c4;
      v = make_float4(to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3]));
    }
    *reinterpret_cast<float4*>(dst + row * kS + c4) = v;
  }
}

// Registers <-> 64 x 64 tiles, so that the next chunk pair's tiles can be fetched while the current pair
// computes: thread tid carries rows (tid + 256 i) / 16, columns 4 ((tid + 256 i) % 16) .. +3, i = 0..3.
__device__ __forceinline__ void fetch_tile(f32x4 (&reg)[4], const float* __restrict__ src, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, row = e >> 4, c4 = (e & 15) * 4;
    reg[i] = *reinterpret_cast<const f32x4*>(src + row * 64 + c4);
  }
}
// Rows of a [.., L, 64] input: fetched raw (in the input's type) from a clamped, always valid row, and
// widened and masked (rows >= L read as zero) only when stored, so that no wait for the data is forced
// at the fetch.
template <typename T>
using raw4 = typename std::conditional<std::is_same<T, float>::value, f32x4, bf16x4>::type;
template <typename T>
__device__ __forceinline__ f32x4 widen4(const raw4<T>& x) {
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <typename T>
__device__ __forceinline__ void fetch_rows(raw4<T> (&reg)[4], const T* __restrict__ src, int64_t c0, int64_t L,
                                           int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, row = e >> 4, c4 = (e & 15) * 4;
    const int64_t rr = c0 + row < L ? c0 + row : L - 1;
    reg[i] = *reinterpret_cast<const raw4<T>*>(src + (size_t)rr * 64 + c4);
  }
}
template <typename T>
__device__ __forceinline__ void put_rows(float* dst, const raw4<T> (&reg)[4], int64_t c0, int64_t L, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, row = e >> 4, c4 = (e & 15) * 4;
    const f32x4 v = widen4<T>(reg[i]);
    *reinterpret_cast<f32x4*>(dst + row * kS + c4) = c0 + row < L ? v : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}
__device__ __forceinline__ void put_tile(float* dst, const f32x4 (&reg)[4], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, row = e >> 4, c4 = (e & 15) * 4;
    *reinterpret_cast<f32x4*>(dst + row * kS + c4) = reg[i];
  }
}

// A-operand of mm64 held in registers: a[4 kb + j] = A(16w + r, 16 kb + 4g + j), i.e. the wave's own
// 16 rows of a row-major 64 x 64 operand.
__device__ __forceinline__ void frag_f32(float (&a)[16], const float* __restrict__ src, int w, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (16 * w + r) * 64 + 16 * kb + 4 * g);
    a[4 * kb] = v[0], a[4 * kb + 1] = v[1], a[4 * kb + 2] = v[2], a[4 * kb + 3] = v[3];
  }
}
template <typename T>
__device__ __forceinline__ void frag_rows(float (&a)[16], const T* __restrict__ src, int64_t c0, int64_t L, int w,
                                          int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int64_t row = c0 + 16 * w + r;
  const int64_t rr = row < L ? row : L - 1;  // clamped (valid) row; masked below
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f32x4 v = widen4<T>(*reinterpret_cast<const raw4<T>*>(src + (size_t)rr * 64 + 16 * kb + 4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) a[4 * kb + j] = row < L ? v[j] : 0.f;
  }
}

// acc[cb] += sum_k A(16w + r', k) B(k, 16cb + r'') with A from registers (frag_f32 / frag_rows layout);
// B as in mm64.
template <bool BK, int SB = kS>
__device__ __forceinline__ void mm64_ra(f32x4 (&acc)[4], const float (&a)[16], const float* __restrict__ B,
                                        int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int k0 = 16 * kb;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      float b[4];
      if constexpr (!BK) {
        const float4 v = *reinterpret_cast<const float4*>(B + (16 * cb + r) * SB + k0 + 4 * g);
        b[0] = v.x, b[1] = v.y, b[2] = v.z, b[3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = B[(k0 + 4 * g + j) * SB + 16 * cb + r];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[cb] = mfma4(a[4 * kb + j], b[j], acc[cb]);
    }
  }
}

// bf16x3 products (bf16 inputs): an fp32 operand x = hi + lo with hi = bf16(x), lo = bf16(x - hi); a product
// sums hi*hi + hi*lo + lo*hi on the bf16 matrix cores (about 2^-16 relative; lo*lo dropped).
__device__ __forceinline__ void split8(const f32x4& x, const f32x4& y, bf16x8& h, bf16x8& l) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = i < 4 ? x[i] : y[i - 4];
    const __bf16 hi = (__bf16)v;
    h[i] = hi;
    l[i] = (__bf16)(v - (float)hi);
  }
}

// mm64 on the bf16 matrix cores (bf16 inputs): acc[cb] += sum_k A(16w + r', k) B(k, 16cb + r''), operands as
// in mm64 (AT, BK, row strides SA, SB; LDS tiles or global fp32 tiles).  An operand flagged exact (EA, EB:
// it holds bf16 numbers, i.e. w, q or k of a bf16 input) is converted exactly; any other is split into
// hi + lo bf16, and the product sums hi*hi, hi*lo and lo*hi (about 2^-16 relative; lo*lo dropped).
template <bool KT, int S>
__device__ __forceinline__ void load8(float (&v)[8], const float* __restrict__ M, int rc, int k0) {
  if constexpr (!KT) {  // M[rc][k0 .. k0 + 7]
    const f32x4 x = *reinterpret_cast<const f32x4*>(M + rc * S + k0);
    const f32x4 y = *reinterpret_cast<const f32x4*>(M + rc * S + k0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = x[i], v[4 + i] = y[i];
  } else {  // M[k0 .. k0 + 7][rc]
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = M[(k0 + i) * S + rc];
  }
}
template <bool EXACT>
__device__ __forceinline__ void to_bf8(const float (&v)[8], bf16x8& h, bf16x8& l) {
  if constexpr (EXACT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (__bf16)v[i];
  } else {
    split8(f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]}, h, l);
  }
}
template <bool AT, bool BK, int SA, int SB, bool EA, bool EB, int NC>
__device__ __forceinline__ void mm64_bf(f32x4 (&acc)[NC], const float* __restrict__ A, const float* __restrict__ B,
                                        int w, int lane, int cb0 = 0) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int k0 = 32 * ks + 8 * g;
    float av[8];
    load8<AT, SA>(av, A, 16 * w + r, k0);
    bf16x8 ah, al;
    to_bf8<EA>(av, ah, al);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float bv[8];
      load8<BK, SB>(bv, B, 16 * (cb0 + c) + r, k0);
      bf16x8 bh, bl;
      to_bf8<EB>(bv, bh, bl);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[c], 0, 0, 0);
      if constexpr (!EB) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[c], 0, 0, 0);
      if constexpr (!EA) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[c], 0, 0, 0);
    }
  }
}
// mm64, on the bf16 matrix cores for a bf16 input
template <typename T, bool AT, bool BK, int SA = kS, int SB = kS, bool EA = false, bool EB = false, int NC>
__device__ __forceinline__ void mmx(f32x4 (&acc)[NC], const float* A, const float* B, int w, int lane, int cb0 = 0) {
  if constexpr (std::is_same<T, __bf16>::value) mm64_bf<AT, BK, SA, SB, EA, EB>(acc, A, B, w, lane, cb0);
  else mm64<AT, BK, SA, SB>(acc, A, B, w, lane, cb0);
}

// The next chunk pair's operands of the two chunk-pair kernels, fetched into registers one step ahead
// (plain functions rather than capturing lambdas, so that the arrays stay in registers).
__device__ __forceinline__ void fetch_query_pair(f32x4 (&pK)[4], f32x4 (&pV)[4], f32x4 (&pP)[4], float (&pra)[16],
                                                 float& pF, float& poff, const float* __restrict__ kt,
                                                 const float* __restrict__ vb, const float* __restrict__ Pm,
                                                 const float* __restrict__ St, const float* __restrict__ fl,
                                                 const float* __restrict__ Off, const pair_band& band, int64_t bh,
                                                 int64_t m, int64_t n, int64_t M, int64_t L, int tid, int w,
                                                 int lane) {
  constexpr int C = 64, CD = 64 * 64;
  const int64_t Lp = M * C;
  const size_t pr = band.slot(bh, m, n);
  fetch_tile(pK, kt + ((size_t)bh * Lp + (size_t)n * C) * 64, tid);
  fetch_rows(pV, vb, n * C, L, tid);
  fetch_tile(pP, Pm + ((size_t)bh * M + n) * CD, tid);  // P_0 when n = 0: fetched, not used
  frag_f32(pra, St + pr * CD, w, lane);
  if (fl != nullptr) {
    pF = fl[(size_t)bh * Lp + (size_t)n * C + (tid & 63)];
    poff = Off[pr];
  }
}
__device__ __forceinline__ void fetch_key_pair(f32x4 (&pR)[4], f32x4 (&pG)[4], f32x4 (&pO)[4], float& pl2,
                                               float& pDv, float& poff, const float* __restrict__ St,
                                               const float* __restrict__ Gst, const float* __restrict__ ob,
                                               const float* __restrict__ lse2w, const float* __restrict__ Dw,
                                               const float* __restrict__ Off, bool fox, const pair_band& band,
                                               int64_t bh, int64_t m, int64_t n, int64_t M, int64_t L, int tid) {
  constexpr int C = 64, CD = 64 * 64;
  const int64_t Lp = M * C;
  const size_t pr = band.slot(bh, m, n);
  fetch_tile(pR, St + pr * CD, tid);
  fetch_tile(pG, Gst + pr * CD, tid);  // not written for n = 0 (no transport there): fetched, not used
  fetch_rows(pO, ob, m * C, L, tid);
  const size_t r0 = (size_t)bh * Lp + (size_t)m * C;
  pl2 = lse2w[r0 + (tid & 63)];
  pDv = Dw[r0 + (tid & 63)];
  if (fox) poff = Off[pr];
}


// Both chunk-pair kernels keep four 64 x 64 LDS tiles (about 70 KB, so two blocks share a CU): three
// tiles that every wave reads whole, and one whose rows 16w .. 16w+15 only wave w writes and reads
// (accumulators turned into A-operands), which needs no block barrier.  Operands a wave reads only
// for its own rows stay in registers.
constexpr size_t kLdsPairMfma = sizeof(float) * (4 * 64 * kS + 3 * 64);

}  // namespace

// Query-chunk kernel on the fp32 matrix cores, fp32 inputs (same outputs as bwd_query_kernel<float, 64, 64>;
// bf16 inputs take bwd_query_tile_kernel).
__global__ __launch_bounds__(256, 2) void bwd_query_mfma_kernel(
    const float* __restrict__ qt, const float* __restrict__ kt, const float* __restrict__ Pm,
    const float* __restrict__ Sm, const float* __restrict__ fl, const float* __restrict__ ftot,
    const float* __restrict__ v, const float* __restrict__ out, const float* __restrict__ dout,
    const float* __restrict__ lse, int64_t L, int64_t M, float scale, pair_band band, float* __restrict__ St,
    float* __restrict__ Gst,
    float* __restrict__ Off, float* __restrict__ lse2w, float* __restrict__ Dw, float* __restrict__ drow,
    float* __restrict__ dqt, float* __restrict__ dSm, int64_t BH) {
  constexpr int C = 64, CD = 64 * 64;
  extern __shared__ float sm[];
  float* Ks = sm;           // ktilde_n
  float* Vs = Ks + C * kS;  // v_n
  float* Ps = Vs + C * kS;  // P_n
  float* Xs = Ps + C * kS;  // wave rows: r^(n) (pass 1), dr^(n-1) then ln2 * dz (pass 2)
  float* l2 = Xs + C * kS;
  float* Dv = l2 + C;
  float* Fn = Dv + C;

  int64_t bh, q;
  if (!bwd_pair_block(BH, band.me - band.mb, bh, q)) return;  // whole block
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int64_t m = band.me - 1 - q;  // longest of the band first
  const int64_t Lp = M * C;
  const bool fox = fl != nullptr;
  const size_t row0 = (size_t)bh * Lp + (size_t)m * C;
  const float* vb = v + (size_t)bh * L * 64;

  // dO_m rows of this wave (the A-operand of dO V^T), and D_i = dO_i . o_i
  float oa[16];
  frag_rows(oa, dout + (size_t)bh * L * 64, m * C, L, w, lane);
  {
    float ob[16];
    frag_rows(ob, out + (size_t)bh * L * 64, m * C, L, w, lane);
    float dv = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) dv += oa[x] * ob[x];
    dv += __shfl_xor(dv, 16);
    dv += __shfl_xor(dv, 32);
    if (g == 0) {
      const int a = 16 * w + r;
      const int64_t i = m * C + a;
      const float l2v = i < L ? kLog2e * (lse[bh * L + i] - (fox ? fl[row0 + a] : 0.f)) : INFINITY;  // padded: p = 0
      Dv[a] = dv;
      l2[a] = l2v;
      lse2w[row0 + a] = l2v;
      Dw[row0 + a] = dv;
    }
  }

  // pass 1: states r^(n), n = m-1 .. 0; P_{n} arrives in registers one step ahead
  f32x4 R[4], G[4];
  global_to_acc(R, qt + row0 * 64, w, lane);
  zero4(G);
  // (fetched unconditionally, at a clamped index: a conditionally written register array would be
  // kept in scratch memory)
  f32x4 pP[4];
  fetch_tile(pP, Pm + ((size_t)bh * M + (m > 0 ? m - 1 : 0)) * CD, tid);
  float off = 0.f;
  for (int64_t n = m - 1; n >= 0; --n) {
    const size_t pr = band.slot(bh, m, n);
    if (fox) off += ftot[bh * M + n];
    if (tid == 0) Off[pr] = off;
    acc_to_global(R, St + pr * CD, w, lane);
    if (n > 0) {
      acc_to_lds(R, Xs, w, lane);
      __syncthreads();  // every wave is done with the previous P
      put_tile(Ps, pP, tid);
      __syncthreads();
      fetch_tile(pP, Pm + ((size_t)bh * M + (n > 1 ? n - 1 : 0)) * CD, tid);
      zero4(R);
      mm64<false, false>(R, Xs, Ps, w, lane);  // r P_n^T
    }
  }

  // in-chunk block: logits from S, D = dO_m V_m^T on the matrix cores
  __syncthreads();
  tile_rows(Vs, vb, m * C, L, tid);
  if (fox && tid < C) Fn[tid] = fl[row0 + tid];
  __syncthreads();
  float rsum[4] = {0.f, 0.f, 0.f, 0.f};  // rows 16w + 4g + e, partial over this lane's columns
  {
    f32x4 DP[4];
    zero4(DP);
    mm64_ra<false>(DP, oa, Vs, lane);
    const float* Sc = Sm + ((size_t)bh * M + m) * C * C;
    float* dSc = dSm + ((size_t)bh * M + m) * C * C;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * w + 4 * g + e, b = 16 * cb + r;
        float dz = 0.f;
        if (b <= a) {
          const float z2 = Sc[a * C + b] - (fox ? kLog2e * Fn[b] : 0.f);
          dz = fast_exp2(z2 - l2[a]) * (DP[cb][e] - Dv[a]);
        }
        rsum[e] += dz;
        dSc[a * C + b] = scale * dz;
      }
  }

  // pass 2: n = 0 .. m-1; the next pair's ktilde, v, P (whole tiles) and this wave's rows of r^(n)
  // arrive in registers one step ahead
  if (m > 0) {
  f32x4 pK[4];
  f32x4 pV[4];
  float pra[16], ra[16];
  float pF = 0.f, poff = 0.f;
  fetch_query_pair(pK, pV, pP, pra, pF, poff, kt, vb, Pm, St, fl, Off, band, bh, m, 0, M, L, tid, w, lane);
  for (int64_t n = 0; n < m; ++n) {
    const size_t pr = band.slot(bh, m, n);
    __syncthreads();  // every wave is done with the previous ktilde, v, P, FoX prefix
    put_tile(Ks, pK, tid);
    put_rows<float>(Vs, pV, n * C, L, tid);
    if (n > 0) put_tile(Ps, pP, tid);
    if (fox && tid < C) Fn[tid] = pF;
    const float offn = poff;
#pragma unroll
    for (int x = 0; x < 16; ++x) ra[x] = pra[x];
    if (n > 0) {
      acc_to_lds(G, Xs, w, lane);  // dr^(n-1), this wave's rows
      acc_to_global(G, Gst + pr * CD, w, lane);
    }
    __syncthreads();
    // the last step fetches its own pair again (not used)
    fetch_query_pair(pK, pV, pP, pra, pF, poff, kt, vb, Pm, St, fl, Off, band, bh, m, n + 1 < m ? n + 1 : n, M, L,
                     tid, w, lane);
    f32x4 Z[4], DP[4];
    zero4(G);
    if (n > 0) mm64<false, true>(G, Xs, Ps, w, lane);  // dr^(n-1) P_n
    zero4(Z);
    zero4(DP);
    mm64_ra<false>(Z, ra, Ks, lane);
    mm64_ra<false>(DP, oa, Vs, lane);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * w + 4 * g + e, b = 16 * cb + r;
        const float z2 = Z[cb][e] + (fox ? kLog2e * (offn - Fn[b]) : 0.f);
        const float dz = fast_exp2(z2 - l2[a]) * (DP[cb][e] - Dv[a]);
        rsum[e] += dz;
        Xs[a * kS + b] = kLn2 * dz;  // the wave's own rows; the reads of dr^(n-1) above came first
      }
    mm64<false, true>(G, Xs, Ks, w, lane);  // + g ktilde_n
  }
  }

  acc_to_global(G, dqt + row0 * 64, w, lane, scale * kLog2e);  // qtilde entered the scan scaled
  // row sums: reduce over the 16 lanes that share g
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s = rsum[e];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (r == 0) drow[row0 + 16 * w + 4 * g + e] = s;
  }
}

// Key-chunk kernel on the fp32 matrix cores, fp32 inputs (same outputs as bwd_key_kernel<float, 64, 64>;
// bf16 inputs take bwd_key_tile_kernel).  The logits of a pair are formed transposed (rows = keys of
// chunk n), so that p and g are stored k-contiguous for the products that reduce over the queries.
__global__ __launch_bounds__(256, 2) void bwd_key_mfma_kernel(
    const float* __restrict__ kt, const float* __restrict__ Sm, const float* __restrict__ fl,
    const float* __restrict__ v, const float* __restrict__ dout, const float* __restrict__ St,
    const float* __restrict__ Gst,
    const float* __restrict__ Off, const float* __restrict__ lse2w, const float* __restrict__ Dw, int64_t L,
    int64_t M, pair_band band, float* __restrict__ dv, float* __restrict__ dva, float* __restrict__ dkt,
    float* __restrict__ dPm, float* __restrict__ dcol, int64_t BH) {
  constexpr int C = 64, CD = 64 * 64;
  extern __shared__ float sm[];
  float* Rs = sm;           // r^(n)_m
  float* Os = Rs + C * kS;  // dO_m
  float* Gq = Os + C * kS;  // dr^(n-1)_m
  float* Xs = Gq + C * kS;  // wave rows: p^T, then (ln2 dz)^T  [key][query]
  float* l2 = Xs + C * kS;
  float* Dv = l2 + C;
  float* Fn = Dv + C;

  int64_t bh, n;
  if (!bwd_pair_block(BH, band.me, bh, n)) return;  // whole block; low key chunks first
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int64_t Lp = M * C;
  const bool fox = fl != nullptr;
  const size_t rown = (size_t)bh * Lp + (size_t)n * C;
  const bool first = n >= band.mb;  // query chunk n is in this band: the sums start here (in-chunk block)
  const bool last = band.me == M;   // the sums end here
  const float* vb = v + (size_t)bh * L * 64;
  const float* ob = dout + (size_t)bh * L * 64;

  // this wave's rows of ktilde_n and v_n: the A-operands of the transposed logits and of V dO^T
  float ka[16], va[16];
  frag_f32(ka, kt + rown * 64, w, lane);
  frag_rows(va, vb, n * C, L, w, lane);

  f32x4 aV[4], aK[4], aP[4];
  float csum[4] = {0.f, 0.f, 0.f, 0.f};  // key rows 16w + 4g + e, this band's share
  if (tid < C) Fn[tid] = fox ? fl[rown + tid] : 0.f;
  if (!first) {  // the sums of the earlier bands
    global_to_acc(aV, dva + rown * 64, w, lane);
    global_to_acc(aK, dkt + rown * 64, w, lane);
    global_to_acc(aP, dPm + ((size_t)bh * M + n) * CD, w, lane);
  } else {
  zero4(aV);
  zero4(aK);
  zero4(aP);
  tile_rows(Os, ob, n * C, L, tid);
  if (tid < C) {
    l2[tid] = lse2w[rown + tid];
    Dv[tid] = Dw[rown + tid];
  }
  __syncthreads();

  // in-chunk block (m = n): D^T = V dO^T on the matrix cores, logits from S
  {
    f32x4 DT[4];
    zero4(DT);
    mm64_ra<false>(DT, va, Os, lane);
    const float* Sc = Sm + ((size_t)bh * M + n) * C * C;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 16 * w + 4 * g + e, a = 16 * cb + r;
        float p = 0.f, dz = 0.f;
        if (b <= a) {
          const float z2 = Sc[a * C + b] - (fox ? kLog2e * Fn[b] : 0.f);
          p = fast_exp2(z2 - l2[a]);
          dz = p * (DT[cb][e] - Dv[a]);
        }
        csum[e] += dz;
        Xs[b * kS + a] = p;  // the wave's own rows
      }
  }
  mm64<false, true>(aV, Xs, Os, w, lane);  // dv_n += p^T dO_n
  }

  // the band's query chunks m > n; the next pair's tiles arrive in registers one step ahead
  const int64_t m0 = n + 1 > band.mb ? n + 1 : band.mb;
  if (m0 < band.me) {
  f32x4 pR[4], pG[4];
  f32x4 pO[4];
  float pl2 = 0.f, pDv = 0.f, poff = 0.f;
  fetch_key_pair(pR, pG, pO, pl2, pDv, poff, St, Gst, ob, lse2w, Dw, Off, fox, band, bh, m0, n, M, L, tid);
  for (int64_t m = m0; m < band.me; ++m) {
    __syncthreads();  // every wave is done with the previous r, dO, dr, row statistics
    put_tile(Rs, pR, tid);
    if (n > 0) put_tile(Gq, pG, tid);
    put_rows<float>(Os, pO, m * C, L, tid);
    if (tid < C) {
      l2[tid] = pl2;
      Dv[tid] = pDv;
    }
    const float offn = poff;
    __syncthreads();
    // the last step fetches its own pair again (not used)
    fetch_key_pair(pR, pG, pO, pl2, pDv, poff, St, Gst, ob, lse2w, Dw, Off, fox, band, bh,
                   m + 1 < band.me ? m + 1 : m, n, M, L, tid);
    f32x4 ZT[4], DT[4];
    zero4(ZT);
    zero4(DT);
    mm64_ra<false>(ZT, ka, Rs, lane);  // (r ktilde^T)^T
    mm64_ra<false>(DT, va, Os, lane);  // (dO v^T)^T
    float gz[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 16 * w + 4 * g + e, a = 16 * cb + r;
        const float z2 = ZT[cb][e] + (fox ? kLog2e * (offn - Fn[b]) : 0.f);
        const float p = fast_exp2(z2 - l2[a]);
        const float dz = p * (DT[cb][e] - Dv[a]);
        csum[e] += dz;
        Xs[b * kS + a] = p;
        gz[cb][e] = kLn2 * dz;
      }
    mm64<false, true>(aV, Xs, Os, w, lane);  // dv_n += p^T dO_m
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) Xs[(16 * w + 4 * g + e) * kS + 16 * cb + r] = gz[cb][e];  // after the reads of p
    mm64<false, true>(aK, Xs, Rs, w, lane);           // d ktilde_n += g^T r
    if (n > 0) mm64<true, true>(aP, Gq, Rs, w, lane);  // dP_n += dr^(n-1)^T r
  }
  }

  acc_to_global(aK, dkt + rown * 64, w, lane);
  acc_to_global(aP, dPm + ((size_t)bh * M + n) * CD, w, lane);
  if (!last) {
    acc_to_global(aV, dva + rown * 64, w, lane);
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 16 * w + 4 * g + e;
        if (n * C + b < L) dv[((size_t)bh * L + n * C + b) * 64 + 16 * cb + r] = aV[cb][e];
      }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s = csum[e];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (r == 0) {
      const size_t i = rown + 16 * w + 4 * g + e;
      dcol[i] = (first ? 0.f : dcol[i]) + s;
    }
  }
}

// ------------------------------------------------------------------------------- per-chunk terms, matrix cores
namespace {

constexpr int kT = 64 * kS;                                     // one 64 x 64 LDS tile
constexpr size_t kLdsChunkMfma = sizeof(float) * (9 * kT + 3 * 64);     // gradient kernel
constexpr size_t kLdsChunkFwdMfma = sizeof(float) * (8 * kT + 64);   // forward-terms kernel

// Element (i, j) of the accumulator layout: i = 16w + 4g + e, j = 16cb + r.
template <typename F, int NC>
__device__ __forceinline__ void acc_store(const f32x4 (&acc)[NC], float* T, int w, int lane, F f, int cb0 = 0) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, j = 16 * (cb0 + c) + r;
      T[i * kS + j] = f(i, j, acc[c][e]);
    }
}

template <int NC>
__device__ __forceinline__ void sub4(f32x4 (&acc)[NC], const f32x4 (&t)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] -= t[c];
}

// A = I + diag(beta) strict_upper(W W^T) is read from tile Aa (only r < s), A^{-1} written to Ai
// (unit upper triangular, zeros below) by back substitution, one column per thread.
// The thread's column z stays in registers; the loops run over fixed bounds (z[kk] = 0 below the
// diagonal and z[j] = 1 make the extra terms vanish), and each sum is split over four accumulators
// so that the dependent FMA chains overlap.
__device__ __forceinline__ void unit_upper_inverse(const float* Aa, float* Ai, int tid) {
  if (tid < 64) {
    const int j = tid;
    float z[64];
#pragma unroll
    for (int i = 63; i >= 0; --i) {
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = i + 1; kk < 64; ++kk) s4[(kk - i - 1) & 3] = __builtin_fmaf(Aa[i * kS + kk], z[kk], s4[(kk - i - 1) & 3]);
      const float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      z[i] = i == j ? 1.f : (i < j ? -sum : 0.f);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) Ai[i * kS + j] = z[i];
  }
}

// acc[cb] += sum_k A[16w + r'][k] B[16cb + r''][k] on the bf16 matrix cores, for fp32 LDS tiles (stride
// kS) holding bf16 numbers (w, q, k of a bf16 input): the conversions and the products are exact.
__device__ __forceinline__ bf16x8 row8_bf16(const float* p) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p), y = *reinterpret_cast<const f32x4*>(p + 4);
  return bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                (__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
}
template <int NC>
__device__ __forceinline__ void mm64_rows_bf16(f32x4 (&acc)[NC], const float* __restrict__ A,
                                               const float* __restrict__ B, int w, int lane, int cb0) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 a = row8_bf16(A + (16 * w + r) * kS + 32 * ks + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          a, row8_bf16(B + (16 * (cb0 + c) + r) * kS + 32 * ks + 8 * g), acc[c], 0, 0, 0);
  }
}
// mm64<false, false>, on the bf16 matrix cores when the operands hold bf16 numbers
template <typename T, int NC>
__device__ __forceinline__ void mm64_rows(f32x4 (&acc)[NC], const float* A, const float* B, int w, int lane,
                                          int cb0 = 0) {
  if constexpr (std::is_same<T, __bf16>::value) mm64_rows_bf16(acc, A, B, w, lane, cb0);
  else mm64<false, false>(acc, A, B, w, lane, cb0);
}

// W, Q, K of chunk c (rows >= L zero), beta, then A (into Aa), U (t <= a), R (s > b).  NT threads; each
// wave covers NC column blocks from cb0.
template <typename T, int NC = 4, int NT = 256>
__device__ __forceinline__ void chunk_setup(const T* q, const T* k, const T* w, const float* beta, int64_t bh,
                                            int64_t c, int64_t L, float* Wt, float* Qt, float* Kt, float* Aa,
                                            float* Ut, float* Rt, float* Bs, int tid, int wv, int lane, int cb0 = 0) {
  const size_t base = (size_t)bh * L * 64;
  tile_rows(Wt, w + base, c * 64, L, tid, NT);
  tile_rows(Qt, q + base, c * 64, L, tid, NT);
  tile_rows(Kt, k + base, c * 64, L, tid, NT);
  if (tid < 64) Bs[tid] = c * 64 + tid < L ? beta[bh * L + c * 64 + tid] : 0.f;  // padded: identity
  __syncthreads();
  f32x4 t[NC];
  zero4(t);
  mm64_rows<T>(t, Wt, Wt, wv, lane, cb0);  // w_r . w_s
  acc_store(t, Aa, wv, lane, [&](int i, int j, float x) { return i < j ? Bs[i] * x : 0.f; }, cb0);
  zero4(t);
  mm64_rows<T>(t, Wt, Qt, wv, lane, cb0);  // w_t . q_a
  acc_store(t, Ut, wv, lane, [](int i, int j, float x) { return i <= j ? x : 0.f; }, cb0);
  zero4(t);
  mm64_rows<T>(t, Kt, Wt, wv, lane, cb0);  // k_b . w_s
  acc_store(t, Rt, wv, lane, [](int i, int j, float x) { return j > i ? x : 0.f; }, cb0);
}

}  // namespace

// The forward's per-chunk terms in fp32 (the same outputs as vec_prep_kernel<T, 64, 64>): qtilde and S
// scaled by qscale = scale * log2e, ktilde, P_c, FoX local prefix and chunk totals.
template <typename T>
__global__ __launch_bounds__(256) void bwd_chunk_fwd_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ w, const float* __restrict__ beta,
    const float* __restrict__ logf, int64_t L, int64_t M, float qscale, float* __restrict__ qt,
    float* __restrict__ kt, float* __restrict__ Pm, float* __restrict__ Sm, float* __restrict__ fl,
    float* __restrict__ ftot) {
  extern __shared__ float sm[];
  float* Wt = sm;
  float* Qt = Wt + kT;
  float* Kt = Qt + kT;
  float* Ta = Kt + kT;  // A, then Ti
  float* Ai = Ta + kT;  // A^{-1}, then Y
  float* Ut = Ai + kT;
  float* Rt = Ut + kT;  // R, then Z2 = Ti W
  float* Xt = Rt + kT;
  float* Bs = Xt + kT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t c = blockIdx.x, bh = blockIdx.y, Lp = M * 64;
  const size_t row0 = (size_t)bh * Lp + (size_t)c * 64;

  if (logf != nullptr && tid == 0) {
    float s = 0.f;
    for (int a = 0; a < 64; ++a) {
      const int64_t i = c * 64 + a;
      s += i < L ? logf[bh * L + i] : 0.f;
      fl[row0 + a] = s;
    }
    ftot[bh * M + c] = s;
  }
  chunk_setup(q, k, w, beta, bh, c, L, Wt, Qt, Kt, Ta, Ut, Rt, Bs, tid, wv, lane);
  __syncthreads();
  unit_upper_inverse(Ta, Ai, tid);
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) Ta[(e >> 6) * kS + (e & 63)] = Ai[(e >> 6) * kS + (e & 63)] * Bs[e & 63];
  __syncthreads();
  f32x4 t[4], u[4];
  zero4(t);
  mmx<T, false, true, kS, kS, false, false>(t, Ta, Ut, wv, lane);  // X = Ti U
  acc_store(t, Xt, wv, lane, [](int, int, float x) { return x; });
  zero4(u);
  mmx<T, false, true, kS, kS, false, false>(u, Rt, Ta, wv, lane);  // Y = R Ti
  zero4(t);
  mmx<T, false, true, kS, kS, false, true>(t, Ta, Wt, wv, lane);  // Z2 = Ti W
  __syncthreads();
  acc_store(u, Ai, wv, lane, [](int, int, float x) { return x; });  // Y
  acc_store(t, Rt, wv, lane, [](int, int, float x) { return x; });  // Z2
  __syncthreads();
  // S[a][b] = q_a . k_b - (Y U)[b][a] for b <= a
  zero4(t);
  mm64_rows<T>(t, Qt, Kt, wv, lane);
  zero4(u);
  mmx<T, true, false, kS, kS, false, false>(u, Ut, Ai, wv, lane);
  sub4(t, u);
  {
    const int r = lane & 15, g = lane >> 4;
    float* Sc = Sm + ((size_t)bh * M + c) * 64 * 64;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * wv + 4 * g + e, b = 16 * cb + r;
        Sc[a * 64 + b] = b <= a ? qscale * t[cb][e] : 0.f;
      }
  }
  // qtilde = Q - X^T W (scaled), ktilde = K - Y W, P = I - W^T Z2
  zero4(t);
  mmx<T, true, true, kS, kS, false, true>(t, Xt, Wt, wv, lane);
  {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * wv + 4 * g + e, x = 16 * cb + r;
        qt[(row0 + a) * 64 + x] = qscale * (Qt[a * kS + x] - t[cb][e]);
      }
  }
  zero4(t);
  mmx<T, false, true, kS, kS, false, true>(t, Ai, Wt, wv, lane);
  {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 16 * wv + 4 * g + e, x = 16 * cb + r;
        kt[(row0 + b) * 64 + x] = Kt[b * kS + x] - t[cb][e];
      }
  }
  zero4(t);
  mmx<T, true, true, kS, kS, true, false>(t, Wt, Rt, wv, lane);
  {
    const int r = lane & 15, g = lane >> 4;
    float* Pc = Pm + ((size_t)bh * M + c) * 64 * 64;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = 16 * wv + 4 * g + e, y = 16 * cb + r;
        Pc[x * 64 + y] = (x == y ? 1.f : 0.f) - t[cb][e];
      }
  }
}

// Gradients of the per-chunk terms back to q, k, w, beta (the same outputs as bwd_prep_kernel<T, 64, 64>),
// fp32 inputs (bf16 ones take bwd_chunk_grad_tile_kernel).  d qtilde, d ktilde, dS and dP are read
// straight from global memory (fp32 tiles, row stride 64); A^{-1} is formed here by back substitution.
template <typename T>
__global__ __launch_bounds__(512) void bwd_chunk_grad_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ w, const float* __restrict__ beta,
    const float* __restrict__ dqt, const float* __restrict__ dkt, const float* __restrict__ dPm,
    const float* __restrict__ dSm, int64_t L, int64_t M, T* __restrict__ dq,
    T* __restrict__ dk, T* __restrict__ dw, float* __restrict__ dbeta) {
  extern __shared__ float sm[];
  float* S0 = sm;        // W
  float* S1 = S0 + kT;   // Q
  float* S2 = S1 + kT;   // K
  float* S3 = S2 + kT;   // A, then Ti
  float* S4 = S3 + kT;   // U, dU, dTi
  float* S5 = S4 + kT;   // R, dR, M1
  float* S6 = S5 + kT;   // A^{-1}
  float* S7 = S6 + kT;   // X, dX, W dP, dN
  float* S8 = S7 + kT;   // Y, dY, W dP^T
  float* Bs = S8 + kT;
  float* dB = Bs + 64;  // dbeta partials, one row of 64 per column half (each filled by single waves)
  // eight waves: wave 4h + wv works on rows 16 wv .. 16 wv + 15 and column blocks cb0 = 2h, 2h + 1 of every
  // product (two waves per SIMD with the one block the LDS plan allows per CU)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wv = wave & 3, cb0 = 2 * (wave >> 2);
  const int r = lane & 15, g = lane >> 4;
  const int64_t c = blockIdx.x, bh = blockIdx.y, Lp = M * 64;
  const size_t row0 = (size_t)bh * Lp + (size_t)c * 64;
  const float* dQ = dqt + row0 * 64;                         // d qtilde  [a][x]
  const float* dK = dkt + row0 * 64;                         // d ktilde  [b][x]
  const float* dS = dSm + ((size_t)bh * M + c) * 64 * 64;   // dS        [a][b]
  const float* dP = dPm + ((size_t)bh * M + c) * 64 * 64;   // dP        [x][y]

  if (tid < 128) dB[tid] = 0.f;
  chunk_setup<T, 2, 512>(q, k, w, beta, bh, c, L, S0, S1, S2, S3, S4, S5, Bs, tid, wv, lane, cb0);
  __syncthreads();
  unit_upper_inverse(S3, S6, tid);
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 512) S3[(e >> 6) * kS + (e & 63)] = S6[(e >> 6) * kS + (e & 63)] * Bs[e & 63];
  __syncthreads();

  auto keep = [](int, int, float x) { return x; };
  auto neg = [](int, int, float x) { return -x; };
  f32x4 aq[2], ak[2], aw[2], t[2], u[2], rU[2], rG[2];
  global_to_acc(aq, dQ, wv, lane, cb0);  // dq = d qtilde + ...
  global_to_acc(ak, dK, wv, lane, cb0);  // dk = d ktilde + ...
  zero4(aw);
  zero4(t);
  mmx<T, false, true, kS, kS, false, false>(t, S3, S4, wv, lane, cb0);  // X = Ti U
  acc_store(t, S7, wv, lane, keep, cb0);
  zero4(t);
  mmx<T, false, true, kS, kS, false, false>(t, S5, S3, wv, lane, cb0);  // Y = R Ti
  acc_store(t, S8, wv, lane, keep, cb0);
  mmx<T, false, true, 64, kS, false, true>(aq, dS, S2, wv, lane, cb0);  // dq += dS K
  mmx<T, true, true, 64, kS, false, true>(ak, dS, S1, wv, lane, cb0);   // dk += dS^T Q
  __syncthreads();
  zero4(t);
  mmx<T, false, true, kS, 64, false, false>(t, S7, dQ, wv, lane, cb0);  // X dqtilde
  mmx<T, true, true, kS, 64, false, false>(t, S8, dK, wv, lane, cb0);   // + Y^T dktilde
  sub4(aw, t);
  zero4(u);
  mmx<T, false, false, kS, 64, true, false>(u, S0, dQ, wv, lane, cb0);  // -dX = W dqtilde^T
  zero4(t);
  mmx<T, false, false, 64, kS, false, true>(t, dK, S0, wv, lane, cb0);  // -dY = dktilde W^T
  mmx<T, true, false, 64, kS, false, false>(t, dS, S4, wv, lane, cb0);   //       + dS^T U^T
  zero4(rU);
  mmx<T, true, false, kS, 64, false, false>(rU, S8, dS, wv, lane, cb0);  // (dS Y)^T
  __syncthreads();
  acc_store(u, S7, wv, lane, neg, cb0);  // dX
  acc_store(t, S8, wv, lane, neg, cb0);  // dY
  __syncthreads();
  zero4(u);
  mmx<T, true, true, kS, kS, false, false>(u, S3, S7, wv, lane, cb0);  // dU = Ti^T dX - (dS Y)^T
  sub4(u, rU);
  zero4(rG);
  mmx<T, false, false, kS, kS, false, false>(rG, S7, S4, wv, lane, cb0);  // dTi = dX U^T
  mmx<T, true, true, kS, kS, false, false>(rG, S5, S8, wv, lane, cb0);    //     + R^T dY
  zero4(t);
  mmx<T, false, false, kS, kS, false, false>(t, S8, S3, wv, lane, cb0);  // dR = dY Ti^T
  __syncthreads();
  acc_store(u, S4, wv, lane, [](int i, int j, float x) { return i <= j ? x : 0.f; }, cb0);
  acc_store(t, S5, wv, lane, [](int i, int j, float x) { return j > i ? x : 0.f; }, cb0);
  __syncthreads();
  mmx<T, false, true, kS, kS, false, true>(aw, S4, S1, wv, lane, cb0);  // dW += dU Q
  mmx<T, true, true, kS, kS, false, true>(aw, S5, S2, wv, lane, cb0);   //     + dR^T K
  mmx<T, true, true, kS, kS, false, true>(aq, S4, S0, wv, lane, cb0);   // dq += dU^T W
  mmx<T, false, true, kS, kS, false, true>(ak, S5, S0, wv, lane, cb0);  // dk += dR W
  zero4(t);
  mmx<T, false, true, kS, 64, true, false>(t, S0, dP, wv, lane, cb0);  // W dP
  zero4(u);
  mmx<T, false, false, kS, 64, true, false>(u, S0, dP, wv, lane, cb0);  // W dP^T
  acc_store(t, S7, wv, lane, keep, cb0);
  acc_store(u, S8, wv, lane, keep, cb0);
  __syncthreads();
  zero4(t);
  mmx<T, false, false, kS, kS, false, true>(t, S7, S0, wv, lane, cb0);  // dTi -= W dP W^T
  sub4(rG, t);
  zero4(t);
  mmx<T, false, true, kS, kS, false, false>(t, S3, S8, wv, lane, cb0);  // dW -= Ti W dP^T
  mmx<T, true, true, kS, kS, false, false>(t, S3, S7, wv, lane, cb0);   //      + Ti^T W dP
  sub4(aw, t);
  __syncthreads();
  acc_store(rG, S4, wv, lane, keep, cb0);
  __syncthreads();
  zero4(t);
  mmx<T, true, true, kS, kS, false, false>(t, S6, S4, wv, lane, cb0);  // M1 = A^{-T} dTi; dbeta += diag(M1)
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (16 * wv + 4 * g + e == 16 * (cb0 + cc) + r) atomicAdd(&dB[32 * cb0 + 16 * (cb0 + cc) + r], t[cc][e]);
  acc_store(t, S5, wv, lane, keep, cb0);
  __syncthreads();
  zero4(t);
  mmx<T, false, false, kS, kS, false, false>(t, S5, S3, wv, lane, cb0);  // M1 Ti^T
  zero4(u);
  mm64_rows<T>(u, S0, S0, wv, lane, cb0);  // w_r . w_s
  {
    float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * wv + 4 * g + e, j = 16 * (cb0 + cc) + r;
        const float z = i < j ? -t[cc][e] : 0.f;  // dA[i][j]
        rowp[e] += z * u[cc][e];
        t[cc][e] = Bs[i] * z;  // dN
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = rowp[e];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (r == 0) atomicAdd(&dB[32 * cb0 + 16 * wv + 4 * g + e], x);
    }
  }
  acc_store(t, S7, wv, lane, keep, cb0);
  __syncthreads();
  mmx<T, false, true, kS, kS, false, true>(aw, S7, S0, wv, lane, cb0);  // dW += dN W
  mmx<T, true, true, kS, kS, false, true>(aw, S7, S0, wv, lane, cb0);   //      + dN^T W
  __syncthreads();
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 16 * wv + 4 * g + e, x = 16 * (cb0 + cc) + r;
      const int64_t i = c * 64 + a;
      if (i < L) {
        const size_t o = ((size_t)bh * L + i) * 64 + x;
        dq[o] = from_f32<T>(aq[cc][e]);
        dk[o] = from_f32<T>(ak[cc][e]);
        dw[o] = from_f32<T>(aw[cc][e]);
      }
    }
  if (tid < 64 && c * 64 + tid < L) dbeta[bh * L + c * 64 + tid] = dB[tid] + dB[64 + tid];
}

// ------------------------------------------------------------------------------- UT-transform terms
// One block per (chunk c, batch*head): from d qtilde, d ktilde, dP and dS of the chunk to dq, dk, dw,
// dbeta.  Nine LDS tiles; the C x C intermediates pass through registers where a tile is rewritten.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ w, const float* __restrict__ beta,
    const float* __restrict__ dqt, const float* __restrict__ dkt, const float* __restrict__ dPm,
    const float* __restrict__ dSm, int64_t L, int64_t M, T* __restrict__ dq, T* __restrict__ dk,
    T* __restrict__ dw, float* __restrict__ dbeta) {
  using S = BwdShape<C, D>;
  constexpr int DP = S::DP, CP = S::CP, CD = S::CD, CC = S::CC, NE = S::NE, NC = S::NC, SL = S::SL;
  extern __shared__ float sm[];
  float* Wt = sm;         // W [C][DP]
  float* Qt = Wt + SL;    // Q
  float* Kt = Qt + SL;    // K
  float* Ai = Kt + SL;    // A^{-1} [C][CP] (unit upper triangular; Ti = Ai diag(beta))
  float* Ut = Ai + SL;    // U, later W dP
  float* Rt = Ut + SL;    // R, later W dP^T
  float* X6 = Rt + SL;    // A, dS, dY, dTi
  float* X7 = X6 + SL;    // dktilde, dqtilde, dU, dR, dP, dN
  float* X8 = X7 + SL;    // Y, X, dX, A^{-T} dTi
  float* Bs = X8 + SL;    // beta [C]
  float* dB = Bs + C;     // dbeta [C]

  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x, bh = blockIdx.y, Lp = M * C;
  const size_t row0 = (size_t)bh * Lp + (size_t)c * C;

  for (int e = tid; e < CD; e += 256) {
    const int a = e / D, x = e % D;
    const int64_t i = c * C + a;
    const bool ok = i < L;
    const size_t g = ((size_t)bh * L + (ok ? i : 0)) * D + x;
    Wt[a * DP + x] = ok ? to_f32(w[g]) : 0.f;
    Qt[a * DP + x] = ok ? to_f32(q[g]) : 0.f;
    Kt[a * DP + x] = ok ? to_f32(k[g]) : 0.f;
  }
  for (int a = tid; a < C; a += 256) {
    const int64_t i = c * C + a;
    Bs[a] = i < L ? beta[bh * L + i] : 0.f;
    dB[a] = 0.f;
  }
  __syncthreads();

  // A (into X6), U, R
  for (int e = tid; e < CC; e += 256) {
    const int r = e / C, s = e % C;
    float g = 0.f, u = 0.f, rr = 0.f;
    #pragma unroll 4
    for (int x = 0; x < D; ++x) {
      g += Wt[r * DP + x] * Wt[s * DP + x];
      u += Wt[r * DP + x] * Qt[s * DP + x];
      rr += Kt[r * DP + x] * Wt[s * DP + x];
    }
    X6[r * CP + s] = r < s ? Bs[r] * g : 0.f;
    Ut[r * CP + s] = r <= s ? u : 0.f;
    Rt[r * CP + s] = s > r ? rr : 0.f;
  }
  __syncthreads();
  // A^{-1} by back substitution, one column per thread
  for (int j = tid; j < C; j += 256) {
    for (int i = C - 1; i > j; --i) Ai[i * CP + j] = 0.f;
    Ai[j * CP + j] = 1.f;
    for (int i = j - 1; i >= 0; --i) {
      float s = 0.f;
      for (int kk = i + 1; kk <= j; ++kk) s += X6[i * CP + kk] * Ai[kk * CP + j];
      Ai[i * CP + j] = -s;
    }
  }
  __syncthreads();
  // dS into X6, Y = R Ti into X8
  {
    const float* dSc = dSm + ((size_t)bh * M + c) * CC;
    for (int e = tid; e < CC; e += 256) {
      const int b = e / C, t = e % C;
      X6[b * CP + t] = dSc[e];
      float y = 0.f;
      for (int s = b + 1; s <= t; ++s) y += Rt[b * CP + s] * Ai[s * CP + t];
      X8[b * CP + t] = y * Bs[t];
    }
  }
  __syncthreads();

  float aq[NE], ak[NE], aw[NE], rA[NC], rB[NC];
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    aw[j] = 0.f;
    if (e < CD) {
      const int a = e / D, x = e % D;
      float sq = dqt[row0 * D + e], sk = dkt[row0 * D + e];
      #pragma unroll 4
      for (int b = 0; b < C; ++b) {
        sq += X6[a * CP + b] * Kt[b * DP + x];  // dS K
        sk += X6[b * CP + a] * Qt[b * DP + x];  // dS^T Q
      }
      aq[j] = sq;
      ak[j] = sk;
    }
  }
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    rA[j] = rB[j] = 0.f;
    if (e < CC) {
      const int r = e / C, s = e % C;
      float u = 0.f, y = 0.f;
      #pragma unroll 4
      for (int b = 0; b < C; ++b) {
        u += X6[s * CP + b] * X8[b * CP + r];  // (dS Y)[s][r]   -> dU[r][s]
        y += X6[b * CP + r] * Ut[s * CP + b];  // (dS^T U^T)[r][s] -> dY[r][s]
      }
      rA[j] = -u;
      rB[j] = -y;
    }
  }
  __syncthreads();
  // d ktilde into X7: dW -= Y^T dktilde, dY -= dktilde W^T
  for (int e = tid; e < CD; e += 256) X7[(e / D) * DP + e % D] = dkt[row0 * D + e];
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int t = e / D, x = e % D;
      float s = 0.f;
      #pragma unroll 4
      for (int b = 0; b < C; ++b) s += X8[b * CP + t] * X7[b * DP + x];
      aw[j] -= s;
    }
  }
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int b = e / C, t = e % C;
      float s = 0.f;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) s += X7[b * DP + x] * Wt[t * DP + x];
      rB[j] -= s;
    }
  }
  __syncthreads();
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) X6[(e / C) * CP + e % C] = rB[j];  // dY
  }
  // d qtilde into X7, X = Ti U into X8
  for (int e = tid; e < CD; e += 256) X7[(e / D) * DP + e % D] = dqt[row0 * D + e];
  for (int e = tid; e < CC; e += 256) {
    const int t = e / C, a = e % C;
    float s = 0.f;
    for (int u = t; u <= a; ++u) s += Ai[t * CP + u] * Bs[u] * Ut[u * CP + a];
    X8[t * CP + a] = s;
  }
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int t = e / D, x = e % D;
      float s = 0.f;
      #pragma unroll 4
      for (int a = 0; a < C; ++a) s += X8[t * CP + a] * X7[a * DP + x];
      aw[j] -= s;  // dW -= X dqtilde
    }
  }
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int t = e / C, a = e % C;
      float s = 0.f;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) s += Wt[t * DP + x] * X7[a * DP + x];
      rB[j] = -s;  // dX
    }
  }
  __syncthreads();
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) X8[(e / C) * CP + e % C] = rB[j];  // dX
  }
  __syncthreads();
  // dU = Ti^T dX - (dS Y)^T on t <= a, into X7
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int t = e / C, a = e % C;
      float s = 0.f;
      for (int u = 0; u <= t; ++u) s += Ai[u * CP + t] * X8[u * CP + a];
      X7[t * CP + a] = t <= a ? rA[j] + Bs[t] * s : 0.f;
    }
  }
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int r = e / D, x = e % D;
      float sw = 0.f, sq = 0.f;
      #pragma unroll 4
      for (int a = 0; a < C; ++a) {
        sw += X7[r * CP + a] * Qt[a * DP + x];  // dW += dU Q
        sq += X7[a * CP + r] * Wt[a * DP + x];  // dQ += dU^T W
      }
      aw[j] += sw;
      aq[j] += sq;
    }
  }
  __syncthreads();
  // dR = dY Ti^T on s > b, into X7
  for (int e = tid; e < CC; e += 256) {
    const int b = e / C, s = e % C;
    float acc = 0.f;
    for (int t = s; t < C; ++t) acc += X6[b * CP + t] * Ai[s * CP + t] * Bs[t];
    X7[b * CP + s] = s > b ? acc : 0.f;
  }
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int r = e / D, x = e % D;
      float sk = 0.f, sw = 0.f;
      #pragma unroll 4
      for (int s = 0; s < C; ++s) {
        sk += X7[r * CP + s] * Wt[s * DP + x];  // dK += dR W
        sw += X7[s * CP + r] * Kt[s * DP + x];  // dW += dR^T K
      }
      ak[j] += sk;
      aw[j] += sw;
    }
  }
  // dTi = dX U^T + R^T dY (registers), then - W dP W^T
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int t = e / C, u = e % C;
      float s = 0.f;
      #pragma unroll 4
      for (int a = 0; a < C; ++a) s += X8[t * CP + a] * Ut[u * CP + a] + Rt[a * CP + t] * X6[a * CP + u];
      rA[j] = s;
    }
  }
  __syncthreads();
  {
    const float* dPc = dPm + ((size_t)bh * M + c) * D * D;
    for (int e = tid; e < D * D; e += 256) X7[(e / D) * DP + e % D] = dPc[e];
  }
  __syncthreads();
  for (int e = tid; e < CD; e += 256) {
    const int t = e / D, y = e % D;
    float a1 = 0.f, a2 = 0.f;
    #pragma unroll 4
    for (int x = 0; x < D; ++x) {
      a1 += Wt[t * DP + x] * X7[x * DP + y];  // (W dP)[t][y]
      a2 += Wt[t * DP + x] * X7[y * DP + x];  // (W dP^T)[t][y]
    }
    Ut[t * DP + y] = a1;
    Rt[t * DP + y] = a2;
  }
  __syncthreads();
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int t = e / C, u = e % C;
      float s = 0.f;
      #pragma unroll 4
      for (int y = 0; y < D; ++y) s += Ut[t * DP + y] * Wt[u * DP + y];
      rA[j] -= s;
    }
  }
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int t = e / D, x = e % D;
      float s = 0.f;
      #pragma unroll 4
      for (int u = 0; u < C; ++u)
        s += Ai[t * CP + u] * Bs[u] * Rt[u * DP + x] + Ai[u * CP + t] * Bs[t] * Ut[u * DP + x];
      aw[j] -= s;  // dW -= Ti W dP^T + Ti^T W dP
    }
  }
  __syncthreads();
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) X6[(e / C) * CP + e % C] = rA[j];  // dTi
  }
  __syncthreads();
  // M1 = A^{-T} dTi into X8; dbeta += diag(M1)
  for (int j = 0; j < NC; ++j) {
    const int e = tid + 256 * j;
    if (e < CC) {
      const int r = e / C, s = e % C;
      float acc = 0.f;
      for (int u = 0; u <= r; ++u) acc += Ai[u * CP + r] * X6[u * CP + s];
      X8[r * CP + s] = acc;
      if (r == s) atomicAdd(&dB[r], acc);
    }
  }
  __syncthreads();
  // dA = -M1 Ti^T on r < s; dbeta_r += sum_s dA[r][s] (w_r . w_s); dN = diag(beta) dA into X7
  for (int e = tid; e < CC; e += 256) {
    const int r = e / C, s = e % C;
    float z = 0.f;
    if (r < s) {
      for (int u = s; u < C; ++u) z -= X8[r * CP + u] * Ai[s * CP + u] * Bs[u];
      float g = 0.f;
      #pragma unroll 4
      for (int x = 0; x < D; ++x) g += Wt[r * DP + x] * Wt[s * DP + x];
      atomicAdd(&dB[r], z * g);
    }
    X7[r * CP + s] = Bs[r] * z;
  }
  __syncthreads();
  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int t = e / D, x = e % D;
      float s = 0.f;
      #pragma unroll 4
      for (int u = 0; u < C; ++u) s += (X7[t * CP + u] + X7[u * CP + t]) * Wt[u * DP + x];
      aw[j] += s;
    }
  }

  for (int j = 0; j < NE; ++j) {
    const int e = tid + 256 * j;
    if (e < CD) {
      const int a = e / D, x = e % D;
      const int64_t i = c * C + a;
      if (i < L) {
        const size_t g = ((size_t)bh * L + i) * D + x;
        dq[g] = from_f32<T>(aq[j]);
        dk[g] = from_f32<T>(ak[j]);
        dw[g] = from_f32<T>(aw[j]);
      }
    }
  }
  for (int a = tid; a < C; a += 256) {
    const int64_t i = c * C + a;
    if (i < L) dbeta[bh * L + i] = dB[a];
  }
}

// ------------------------------------------------------------------------------- forget gates
// df_s = sum_{t >= s} (rowsum_t - colsum_t): a suffix sum per (batch, head), one block each.
__global__ __launch_bounds__(256) void bwd_forget_kernel(const float* __restrict__ drow,
                                                         const float* __restrict__ dcol, int64_t L, int64_t Lp,
                                                         float* __restrict__ dlogf) {
  __shared__ float part[256];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t seg = (L + 255) / 256, lo = tid * seg, hi = lo + seg < L ? lo + seg : L;
  const float* r = drow + bh * Lp;
  const float* cc = dcol + bh * Lp;
  float s = 0.f;
  for (int64_t t = lo; t < hi; ++t) s += r[t] - cc[t];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;  // exclusive suffix over the later segments
    for (int u = 255; u >= 0; --u) {
      const float x = part[u];
      part[u] = acc;
      acc += x;
    }
  }
  __syncthreads();
  float acc = part[tid];
  for (int64_t t = hi - 1; t >= lo; --t) {
    acc += r[t] - cc[t];
    dlogf[bh * L + t] = acc;
  }
}

// ------------------------------------------------------------------------------- launch
// mfma_path.hip: the prefill's per-chunk terms (bf16 transport form) for bf16 inputs at d = chunk = 64, plus
// A^{-1} per chunk
hipError_t mfma_prep_bwd_run(const void* q, const void* k, const void* w, const float* beta, const float* logf,
                             int64_t BH, int64_t L, float qs, void* qt, void* kt, void* Pm, float* Sm, float* fl,
                             float* ftot, float* Zi, hipStream_t st);
// vector_path.hip: the forward's per-chunk terms in fp32 (other shapes than d = chunk = 64)
hipError_t vec_run(int phases, bool bf16, int d, int chunk, const void* q, const void* k, const void* v,
                   const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH, int64_t L,
                   float scale, float* qt, float* kt, float* Pm, float* Sm, float* fl, float* ftot, hipStream_t st);

template <typename T, int D, int C>
static hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* w, const float* beta,
                             const float* logf, const void* out, const float* lse, const void* dout, void* dq,
                             void* dk, void* dv, void* dw, float* dbeta, float* dlogf, int64_t BH, int64_t L,
                             float scale, const bwd_buffers& b, hipStream_t st) {
  using S = BwdShape<C, D>;
  static_assert(S::lds_query <= 160 * 1024 && S::lds_key <= 160 * 1024 && S::lds_prep <= 160 * 1024,
                "backward tiles exceed LDS");
  static_assert(kLdsPairMfma <= 160 * 1024 && kLdsChunkMfma <= 160 * 1024, "backward tiles exceed LDS");
  const int64_t M = (L + C - 1) / C;
  const dim3 grid((unsigned)M, (unsigned)BH);
  hipError_t e;
  const bool fox = logf != nullptr;
  auto lds = [](const void* f, size_t bytes) {
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  };
  const int64_t G = bwd_band_chunks(M), NPB = bwd_band_pairs(M);
  if constexpr (D == 64 && C == 64) {  // the matrix cores: bf16 products for bf16 inputs, fp32 ones for fp32
    if constexpr (std::is_same<T, __bf16>::value) {  // the prefill's own per-chunk terms, and the tile kernels
      if ((e = mfma_prep_bwd_run(q, k, w, beta, logf, BH, L, scale * kLog2e, b.qt, b.kt, b.Pm, b.Sm, b.fl, b.ftot,
                                 b.Zi, st)) != hipSuccess)
        return e;
      for (int64_t mb = 0; mb < M; mb += G) {
        const pair_band band{mb, mb + G < M ? mb + G : M, NPB};
        if ((e = bwd_pair_tiles_run(fox, v, out, dout, lse, BH, L, scale, band, b, dv, st)) != hipSuccess) return e;
      }
    } else {
      if ((e = lds((const void*)bwd_chunk_fwd_mfma_kernel<T>, kLdsChunkFwdMfma)) != hipSuccess) return e;
      bwd_chunk_fwd_mfma_kernel<T><<<grid, 256, kLdsChunkFwdMfma, st>>>(
          (const T*)q, (const T*)k, (const T*)w, beta, logf, L, M, scale * kLog2e, b.qt, b.kt, b.Pm, b.Sm, b.fl,
          b.ftot);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = lds((const void*)bwd_query_mfma_kernel, kLdsPairMfma)) != hipSuccess) return e;
      if ((e = lds((const void*)bwd_key_mfma_kernel, kLdsPairMfma)) != hipSuccess) return e;
      const int64_t xh = kBwdXcd * ((BH + kBwdXcd - 1) / kBwdXcd);
      for (int64_t mb = 0; mb < M; mb += G) {
        const pair_band band{mb, mb + G < M ? mb + G : M, NPB};
        bwd_query_mfma_kernel<<<dim3((unsigned)(xh * (band.me - band.mb))), 256, kLdsPairMfma, st>>>(
            b.qt, b.kt, b.Pm, b.Sm, fox ? b.fl : nullptr, b.ftot, (const float*)v, (const float*)out,
            (const float*)dout, lse, L, M, scale, band, b.St, b.Gst, b.Off, b.lse2, b.Dv, b.drow, b.dqt, b.dSm, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        bwd_key_mfma_kernel<<<dim3((unsigned)(xh * band.me)), 256, kLdsPairMfma, st>>>(
            b.kt, b.Sm, fox ? b.fl : nullptr, (const float*)v, (const float*)dout, b.St, b.Gst, b.Off, b.lse2, b.Dv, L,
            M, band, (float*)dv, b.dva, b.dkt, b.dPm, b.dcol, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
    if constexpr (std::is_same<T, __bf16>::value) {
      if ((e = bwd_chunk_grad_tiles_run(q, k, w, beta, BH, L, b, dq, dk, dw, dbeta, st)) != hipSuccess) return e;
    } else {
      if ((e = lds((const void*)bwd_chunk_grad_mfma_kernel<T>, kLdsChunkMfma)) != hipSuccess) return e;
      bwd_chunk_grad_mfma_kernel<T><<<grid, 512, kLdsChunkMfma, st>>>(
          (const T*)q, (const T*)k, (const T*)w, beta, b.dqt, b.dkt, b.dPm, b.dSm, L, M, (T*)dq, (T*)dk,
          (T*)dw, dbeta);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  } else {
    e = vec_run(1, std::is_same<T, __bf16>::value, D, C, q, k, v, w, beta, logf, nullptr, nullptr, BH, L, scale, b.qt,
                b.kt, b.Pm, b.Sm, b.fl, b.ftot, st);
    if (e != hipSuccess) return e;
    if ((e = lds((const void*)bwd_query_kernel<T, D, C>, S::lds_query)) != hipSuccess) return e;
    if ((e = lds((const void*)bwd_key_kernel<T, D, C>, S::lds_key)) != hipSuccess) return e;
    if ((e = lds((const void*)bwd_prep_kernel<T, D, C>, S::lds_prep)) != hipSuccess) return e;
    for (int64_t mb = 0; mb < M; mb += G) {
      const pair_band band{mb, mb + G < M ? mb + G : M, NPB};
      bwd_query_kernel<T, D, C><<<dim3((unsigned)(band.me - band.mb), (unsigned)BH), 256, S::lds_query, st>>>(
          b.qt, b.kt, b.Pm, b.Sm, fox ? b.fl : nullptr, b.ftot, (const T*)v, (const T*)out, (const T*)dout, lse, L,
          M, scale, band, b.St, b.Gst, b.Off, b.lse2, b.Dv, b.drow, b.dqt, b.dSm);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      bwd_key_kernel<T, D, C><<<dim3((unsigned)band.me, (unsigned)BH), 256, S::lds_key, st>>>(
          b.kt, b.Sm, fox ? b.fl : nullptr, (const T*)v, (const T*)dout, b.St, b.Gst, b.Off, b.lse2, b.Dv, L, M,
          band, (T*)dv, b.dva, b.dkt, b.dPm, b.dcol);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    bwd_prep_kernel<T, D, C><<<grid, 256, S::lds_prep, st>>>((const T*)q, (const T*)k, (const T*)w, beta, b.dqt,
                                                            b.dkt, b.dPm, b.dSm, L, M, (T*)dq, (T*)dk, (T*)dw,
                                                            dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (fox) {
    bwd_forget_kernel<<<dim3((unsigned)BH), 256, 0, st>>>(b.drow, b.dcol, L, M * C, dlogf);
    e = hipGetLastError();
  }
  return e;
}

template <typename T>
static hipError_t dispatch_bwd(int d, int chunk, const void* q, const void* k, const void* v, const void* w,
                               const float* beta, const float* logf, const void* out, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* dw, float* dbeta, float* dlogf,
                               int64_t BH, int64_t L, float scale, const bwd_buffers& b, hipStream_t st) {
#define PATHATTN_BWD_CASE(DD, CC)                                                                                 \
  if (d == DD && chunk == CC)                                                                                     \
    return launch_bwd<T, DD, CC>(q, k, v, w, beta, logf, out, lse, dout, dq, dk, dv, dw, dbeta, dlogf, BH, L, scale, \
                                 b, st);
  PATHATTN_BWD_CASE(16, 16)
  PATHATTN_BWD_CASE(16, 32)
  PATHATTN_BWD_CASE(16, 64)
  PATHATTN_BWD_CASE(32, 16)
  PATHATTN_BWD_CASE(32, 32)
  PATHATTN_BWD_CASE(32, 64)
  PATHATTN_BWD_CASE(64, 16)
  PATHATTN_BWD_CASE(64, 32)
  PATHATTN_BWD_CASE(64, 64)
#undef PATHATTN_BWD_CASE
  return hipErrorInvalidValue;
}

hipError_t bwd_run(bool bf16, int d, int chunk, const void* q, const void* k, const void* v, const void* w,
                   const float* beta, const float* logf, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* dw, float* dbeta, float* dlogf, int64_t BH, int64_t L,
                   float scale, const bwd_buffers& b, hipStream_t st) {
  if (bf16)
    return dispatch_bwd<__bf16>(d, chunk, q, k, v, w, beta, logf, out, lse, dout, dq, dk, dv, dw, dbeta, dlogf, BH,
                                L, scale, b, st);
  return dispatch_bwd<float>(d, chunk, q, k, v, w, beta, logf, out, lse, dout, dq, dk, dv, dw, dbeta, dlogf, BH, L,
                             scale, b, st);
}

}  // namespace pathattn
