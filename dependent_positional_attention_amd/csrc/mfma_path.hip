// Matrix-core (bf16 MFMA, fp32 accumulate) PaTH prefill for head dim 64, chunk 64.
//
// Scheme (PaTH summary, gist.science/ko/paper/2505.16381, section 3): each chunk's
// transitions are held in compact UT form, H_0...H_{C-1} = I - W^T T^{-1} W; per
// chunk we precompute boundary-adjusted rows (queries carry the chunk prefix up to
// and including themselves, keys carry the chunk suffix strictly after them), the
// chunk product P_c and the in-chunk logits; the attention kernel then scans key
// chunks right to left, moving its running queries across each finished chunk
// with P_c (the notes on PaTH, "WY" block: a dense d x d matrix per chunk applied
// to the whole query tile, a prefix product between chunks).
//
// Kernel 1 (prep), one workgroup of 4 waves per (b, h, chunk):
//   A = I + diag(beta) strict_upper(W W^T)   (unit upper triangular, fp32)
//   Z = A^{-1} by 16x16-blocked back substitution (fp32), T^{-1} = Z diag(beta)
//   U^T[a][t] = q_a.w_t (t <= a), R[b][s] = k_b.w_s (s > b), X = T^{-1} U, Y = R T^{-1}
//   qtilde = Q - X^T W, ktilde = K - Y W, P = I - W^T (T^{-1} W),
//   S[a][b] = q_a.k_b - (Y U)[b][a]   (b <= a; in-chunk logits before scaling)
// T^{-1} and T^{-1} W enter the matrix cores as hi+lo bf16 pairs so that P is
// accurate enough to be split again into hi+lo for the long-range transport.
//
// Kernel 2 (attention), one workgroup of 4 waves per 4 consecutive query chunks
// (wave w owns chunk 4p+w, 64 queries = four 16-query MFMA column tiles), longest
// rows first.  The waves share one LDS stream of key chunks n = 4p+2 ... 0
// (ktilde_n, V_n^T, P_n, double-buffered); each A-fragment read from LDS feeds
// four MFMAs (one per query tile).  Per key chunk and wave:
//   S^T = ktilde_n Q_run^T       (keys x queries: each lane holds one query column)
//   online softmax (exp2), P^T kept in registers as the PV B-operand
//   O^T += V_n^T P^T
//   Q_run^T <- P_n Q_run^T       (fp32 accumulate, re-rounded to bf16 [hi+lo])
// Column permutation: an MFMA accumulator gives each lane rows 4g..4g+3 of every
// 16-row tile, while a B-operand wants rows 8g..8g+7 of every 32-row k-step.  The
// contraction order is free, so qtilde, ktilde, P (columns) and V^T (key index)
// are stored with stored slot 8g+j of each 32-block holding index 16(j/4)+4g+(j%4);
// accumulators then convert to B-operands in registers with no data movement.
#include "common.h"

namespace pathattn {

namespace {

constexpr int kD = 64;      // head dim
constexpr int kC = 64;      // chunk
constexpr int kLDB = 72;    // bf16 LDS row stride (144 B: conflict-free 16-byte row reads)
constexpr int kLDF = 68;    // fp32 LDS row stride
constexpr int kMat = kC * kLDB;  // elements of one padded 64x64 bf16 LDS matrix

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const __bf16* m, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(m + row * kLDB + col);
}

// acc += X[m0..m0+15][0..63] . Y[n0..n0+15][0..63]^T; lane (r = l%16, g = l/16) receives
// acc[i] = D[m0 + 4g + i][n0 + r].
__device__ __forceinline__ f32x4 mm_tile(const __bf16* X, const __bf16* Y, int m0, int n0, f32x4 acc) {
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    acc = mfma16(lds_frag(X, m0 + r, ks * 32 + g * 8), lds_frag(Y, n0 + r, ks * 32 + g * 8), acc);
  return acc;
}

// Stored slot of original column c (0..63) under the in-block permutation.
__device__ __forceinline__ int perm_pos(int c) {
  const int c32 = c & 31;
  return (c & 32) + ((c32 >> 2) & 3) * 8 + (c32 >> 4) * 4 + (c32 & 3);
}

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return v;
}

__device__ __forceinline__ void split_hi_lo(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

}  // namespace

// =========================================================================== kernel 1: prep
constexpr size_t kPrepLds = 11 * kMat * 2 + 64 * 4 + 2 * kC * kLDF * 4 + 3 * 256 * 4;

__global__ __launch_bounds__(256) void mfma_prep_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ w, const float* __restrict__ beta, const float* __restrict__ logf, int64_t L,
    int64_t M, __bf16* __restrict__ qt, __bf16* __restrict__ kt, __bf16* __restrict__ vt,
    __bf16* __restrict__ p_hi, __bf16* __restrict__ p_lo, float* __restrict__ Sm, float* __restrict__ fl,
    float* __restrict__ ftot) {
  extern __shared__ __align__(16) char smem[];
  __bf16* Ws = reinterpret_cast<__bf16*>(smem);  // W [s][x]
  __bf16* WTs = Ws + kMat;                       // W^T [x][s]
  __bf16* Qs = WTs + kMat;                       // Q [a][x]
  __bf16* Ks = Qs + kMat;                        // K [b][x]
  __bf16* VXs = Ks + kMat;                       // V [b][x], later X^T [a][s]
  __bf16* UTs = VXs + kMat;                      // U^T [a][t]
  __bf16* Rs = UTs + kMat;                       // R [b][s]
  __bf16* TiH = Rs + kMat;                       // T^{-1} [s][t] hi / lo
  __bf16* TiL = TiH + kMat;
  __bf16* TiTH = TiL + kMat;                     // T^{-T} [t][s] hi / lo
  __bf16* TiTL = TiTH + kMat;
  float* Bs = reinterpret_cast<float*>(TiTL + kMat);  // beta [64]
  float* Af = Bs + 64;                                // A [64][kLDF]
  float* Zf = Af + kC * kLDF;                         // Z = A^{-1} [64][kLDF]
  float* Tmp = Zf + kC * kLDF;                        // 3 x 16 x 16 block temporaries
  // After T^{-1} is formed the fp32 A/Z region holds Y and (T^{-1}W)^T hi/lo.
  __bf16* Ys = reinterpret_cast<__bf16*>(Af);  // Y [b][t]
  __bf16* Z2H = Ys + kMat;                      // (T^{-1} W)^T [y][s] hi / lo
  __bf16* Z2L = Z2H + kMat;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t Lp = M * kC;
  const int64_t row0 = (int64_t)c * kC;

  // ---------------------------------------------------------------- A: stage W, W^T, Q, K, V, beta
  for (int e = tid; e < 512; e += 256) {
    const int a = e >> 3, c8 = (e & 7) * 8;
    const int64_t i = row0 + a;
    const bool ok = i < L;
    const size_t go = ((size_t)bh * L + (ok ? i : 0)) * kD + c8;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    const uint4 wv = ok ? *reinterpret_cast<const uint4*>(w + go) : z4;
    *reinterpret_cast<uint4*>(Ws + a * kLDB + c8) = wv;
    *reinterpret_cast<uint4*>(Qs + a * kLDB + c8) = ok ? *reinterpret_cast<const uint4*>(q + go) : z4;
    *reinterpret_cast<uint4*>(Ks + a * kLDB + c8) = ok ? *reinterpret_cast<const uint4*>(k + go) : z4;
    *reinterpret_cast<uint4*>(VXs + a * kLDB + c8) = ok ? *reinterpret_cast<const uint4*>(v + go) : z4;
    const __bf16* wb = reinterpret_cast<const __bf16*>(&wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) WTs[(c8 + j) * kLDB + a] = wb[j];
  }
  if (tid < 64) {
    const int64_t i = row0 + tid;
    Bs[tid] = i < L ? beta[bh * L + i] : 0.f;  // padded tokens: identity transitions
  }
  for (int e = tid; e < kC * kLDF; e += 256) Zf[e] = 0.f;
  if (logf != nullptr && wave == 0) {  // chunk-local inclusive prefix sum of the log-forget gates
    const int64_t i = row0 + l;
    float f = i < L ? logf[bh * L + i] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(f, o, 64);
      if (l >= o) f += y;
    }
    fl[bh * Lp + i] = f;
    if (l == 63) ftot[bh * M + c] = f;
  }
  __syncthreads();

  // ---------------------------------------------------------------- B: V^T out, A, U^T, R, K Q^T
  for (int e = tid; e < 512; e += 256) {
    const int d = e >> 3, ks = (e >> 2) & 1, gg = e & 3;
    bf16x8 o8;
#pragma unroll
    for (int j = 0; j < 8; ++j) o8[j] = VXs[(32 * ks + 16 * (j >> 2) + 4 * gg + (j & 3)) * kLDB + d];
    *reinterpret_cast<bf16x8*>(vt + (((size_t)bh * M + c) * kD + d) * kC + 32 * ks + 8 * gg) = o8;
  }
  f32x4 kq[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // A[s][t] = beta_s (w_s . w_t) for s < t  (rows s in block `wave`)
    f32x4 ga = mm_tile(Ws, Ws, 16 * wave, 16 * nb, zero);
    // D[t][a] = w_t . q_a  ->  U^T[a][t], t <= a
    f32x4 ua = mm_tile(Ws, Qs, 16 * wave, 16 * nb, zero);
    // D[s][b] = w_s . k_b  ->  R[b][s], s > b
    f32x4 ra = mm_tile(Ws, Ks, 16 * wave, 16 * nb, zero);
    const int col = 16 * nb + r;
    float u4[4], r4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * g + i;
      Af[row * kLDF + col] = (row < col) ? Bs[row] * ga[i] : 0.f;
      u4[i] = (row <= col) ? ua[i] : 0.f;
      r4[i] = (row > col) ? ra[i] : 0.f;
    }
    *reinterpret_cast<bf16x4*>(UTs + col * kLDB + 16 * wave + 4 * g) = pack4(u4[0], u4[1], u4[2], u4[3]);
    *reinterpret_cast<bf16x4*>(Rs + col * kLDB + 16 * wave + 4 * g) = pack4(r4[0], r4[1], r4[2], r4[3]);
    // D[b][a] = k_b . q_a for queries a in block `wave`
    kq[nb] = mm_tile(Ks, Qs, 16 * nb, 16 * wave, zero);
  }
  __syncthreads();

  // ---------------------------------------------------------------- C: diagonal 16x16 blocks of Z = A^{-1}
  if (l < 16) {
    const int base = 16 * wave;
    float z[16];
#pragma unroll
    for (int ii = 15; ii >= 0; --ii) {
      float s = 0.f;
#pragma unroll
      for (int kk = ii + 1; kk < 16; ++kk) s += Af[(base + ii) * kLDF + base + kk] * z[kk];
      z[ii] = (ii == l) ? 1.f : (ii < l ? -s : 0.f);
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) Zf[(base + ii) * kLDF + base + l] = z[ii];
  }
  __syncthreads();

  // ---------------------------------------------------------------- D: off-diagonal blocks, by distance
  // Z_IJ = -Z_II sum_{K=I+1..J} A_IK Z_KJ
  for (int lv = 1; lv < 4; ++lv) {
    const int nblk = 4 - lv;
    for (int e = tid; e < nblk * 256; e += 256) {
      const int I = e >> 8, ii = (e >> 4) & 15, jj = e & 15, J = I + lv;
      float s = 0.f;
      for (int K = I + 1; K <= J; ++K)
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) s += Af[(16 * I + ii) * kLDF + 16 * K + kk] * Zf[(16 * K + kk) * kLDF + 16 * J + jj];
      Tmp[e] = s;
    }
    __syncthreads();
    for (int e = tid; e < nblk * 256; e += 256) {
      const int I = e >> 8, ii = (e >> 4) & 15, jj = e & 15, J = I + lv;
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) s += Zf[(16 * I + ii) * kLDF + 16 * I + kk] * Tmp[(I << 8) + (kk << 4) + jj];
      Zf[(16 * I + ii) * kLDF + 16 * J + jj] = -s;
    }
    __syncthreads();
  }

  // T^{-1} = Z diag(beta) as hi/lo bf16, row-major and transposed
  for (int e = tid; e < kC * kC; e += 256) {
    const int s = e >> 6, t = e & 63;
    __bf16 hi, lo;
    split_hi_lo(Zf[s * kLDF + t] * Bs[t], hi, lo);
    TiH[s * kLDB + t] = hi;
    TiL[s * kLDB + t] = lo;
    TiTH[t * kLDB + s] = hi;
    TiTL[t * kLDB + s] = lo;
  }
  __syncthreads();

  // ---------------------------------------------------------------- E: X^T, Y, (T^{-1}W)^T
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int col = 16 * nb + r;
    // D[s][a] = X[s][a]  ->  X^T[a][s]
    f32x4 xa = mm_tile(TiL, UTs, 16 * wave, 16 * nb, mm_tile(TiH, UTs, 16 * wave, 16 * nb, zero));
    *reinterpret_cast<bf16x4*>(VXs + col * kLDB + 16 * wave + 4 * g) = pack4(xa[0], xa[1], xa[2], xa[3]);
    // D[t][b] = Y[b][t]  ->  Y[b][t]
    f32x4 ya = mm_tile(TiTL, Rs, 16 * wave, 16 * nb, mm_tile(TiTH, Rs, 16 * wave, 16 * nb, zero));
    *reinterpret_cast<bf16x4*>(Ys + col * kLDB + 16 * wave + 4 * g) = pack4(ya[0], ya[1], ya[2], ya[3]);
    // D[s][y] = (T^{-1} W)[s][y]  ->  Z2^T[y][s] hi / lo
    f32x4 za = mm_tile(TiL, WTs, 16 * wave, 16 * nb, mm_tile(TiH, WTs, 16 * wave, 16 * nb, zero));
    bf16x4 zh, zl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __bf16 hi, lo;
      split_hi_lo(za[i], hi, lo);
      zh[i] = hi;
      zl[i] = lo;
    }
    *reinterpret_cast<bf16x4*>(Z2H + col * kLDB + 16 * wave + 4 * g) = zh;
    *reinterpret_cast<bf16x4*>(Z2L + col * kLDB + 16 * wave + 4 * g) = zl;
  }
  __syncthreads();

  // ---------------------------------------------------------------- F: outputs
  const size_t chunk_rows = (size_t)bh * Lp + row0;
  const size_t chunk_mat = ((size_t)bh * M + c) * kD * kD;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int x0 = 16 * mb + 4 * g;  // first of this lane's four consecutive columns
    const int a = 16 * wave + r;     // query / key / P-row handled by this lane
    const int pos = perm_pos(x0);
    // qtilde[a][x] = q_a[x] - sum_s X[s][a] w_s[x]
    {
      const f32x4 d4 = mm_tile(WTs, VXs, 16 * mb, 16 * wave, zero);
      const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(Qs + a * kLDB + x0);
      *reinterpret_cast<bf16x4*>(qt + (chunk_rows + a) * kD + pos) =
          pack4((float)q4[0] - d4[0], (float)q4[1] - d4[1], (float)q4[2] - d4[2], (float)q4[3] - d4[3]);
    }
    // ktilde[b][x] = k_b[x] - sum_t Y[b][t] w_t[x]
    {
      const f32x4 d4 = mm_tile(WTs, Ys, 16 * mb, 16 * wave, zero);
      const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(Ks + a * kLDB + x0);
      *reinterpret_cast<bf16x4*>(kt + (chunk_rows + a) * kD + pos) =
          pack4((float)k4[0] - d4[0], (float)k4[1] - d4[1], (float)k4[2] - d4[2], (float)k4[3] - d4[3]);
    }
    // P[x][y] = delta - sum_s w_s[x] Z2[s][y]   (lane: row x = a, columns y = x0..x0+3)
    {
      const f32x4 d4 = mm_tile(Z2L, WTs, 16 * mb, 16 * wave, mm_tile(Z2H, WTs, 16 * mb, 16 * wave, zero));
      bf16x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __bf16 hi, lo;
        split_hi_lo(((x0 + i) == a ? 1.f : 0.f) - d4[i], hi, lo);
        ph[i] = hi;
        pl[i] = lo;
      }
      *reinterpret_cast<bf16x4*>(p_hi + chunk_mat + (size_t)a * kD + pos) = ph;
      if (p_lo != nullptr) *reinterpret_cast<bf16x4*>(p_lo + chunk_mat + (size_t)a * kD + pos) = pl;
    }
    // S[a][b] = q_a.k_b - (Y U)[b][a]   (lane: query a, keys b = x0..x0+3)
    {
      const f32x4 d4 = mm_tile(Ys, UTs, 16 * mb, 16 * wave, zero);
      const float4 s4 = make_float4(kq[mb][0] - d4[0], kq[mb][1] - d4[1], kq[mb][2] - d4[2], kq[mb][3] - d4[3]);
      *reinterpret_cast<float4*>(Sm + (((size_t)bh * M + c) * kC + a) * kC + x0) = s4;
    }
  }
}

// =========================================================================== kernel 2: attention
template <bool FOX, bool X3>
__global__ __launch_bounds__(256, X3 ? 1 : 2) void mfma_attn_kernel(
    const __bf16* __restrict__ qt, const __bf16* __restrict__ kt, const __bf16* __restrict__ vt,
    const __bf16* __restrict__ p_hi, const __bf16* __restrict__ p_lo, const float* __restrict__ Sm,
    const float* __restrict__ fl, const float* __restrict__ ftot, __bf16* __restrict__ out,
    float* __restrict__ lse, int64_t L, int64_t M, float sc) {
  constexpr int NM = X3 ? 4 : 3;  // ktilde, V^T, P hi [, P lo]
  __shared__ __align__(16) __bf16 lds[2][NM][kMat];
  __shared__ float lfl[2][64];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int64_t nP = (M + 3) / 4;
  const int64_t p = nP - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int64_t bh = blockIdx.y;
  const int64_t m = 4 * p + wave;
  const bool active = m < M;
  const int64_t Lp = M * kC;
  const int64_t mtop = (4 * p + 3 < M - 1) ? 4 * p + 3 : M - 1;  // highest query chunk of this block
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  f32x4 o[4][4];
  float mrow[4], lrow[4];
  bf16x8 qb[4][2], ql[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    mrow[a] = -INFINITY;
    lrow[a] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) o[a][b] = zero;
  }

  // Online-softmax update with logits z[kt][qt][i] (log2 units); returns P^T as B-operands.
  auto absorb = [&](f32x4 (&z)[4][4], bf16x8 (&pb)[4][2]) {
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      float mx = -INFINITY;
#pragma unroll
      for (int kti = 0; kti < 4; ++kti)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[kti][qi][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qi], mx);
      const float base = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(mrow[qi] - base);
      lrow[qi] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][qi] *= alpha;
      float ps = 0.f;
#pragma unroll
      for (int kti = 0; kti < 4; ++kti)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(z[kti][qi][i] - base);
          ps += pv;
          pb[qi][kti >> 1][(kti & 1) * 4 + i] = (__bf16)pv;
        }
      lrow[qi] += ps;
      mrow[qi] = mnew;
    }
  };

  // ---------------------------------------------------------------- diagonal block (own chunk)
  if (active) {
    f32x4 z[4][4];
    const float* Sb = Sm + ((size_t)bh * M + m) * kC * kC;
    float fb[4][4];
#pragma unroll
    for (int kti = 0; kti < 4; ++kti)
#pragma unroll
      for (int i = 0; i < 4; ++i) fb[kti][i] = FOX ? kLog2e * fl[bh * Lp + m * kC + 16 * kti + 4 * g + i] : 0.f;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi)
#pragma unroll
      for (int kti = 0; kti < 4; ++kti) {
        const float4 s4 = *reinterpret_cast<const float4*>(Sb + (16 * qi + r) * kC + 16 * kti + 4 * g);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 16 * kti + 4 * g + i, a = 16 * qi + r;
          z[kti][qi][i] = (b <= a) ? sv[i] * sc - fb[kti][i] : -INFINITY;
        }
      }
    bf16x8 pb[4][2];
    absorb(z, pb);
    const __bf16* vtm = vt + ((size_t)bh * M + m) * kD * kC;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vtm + (16 * dt + r) * kC + 32 * ks + 8 * g);
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) o[dt][qi] = mfma16(a, pb[qi][ks], o[dt][qi]);
      }
#pragma unroll
    for (int qi = 0; qi < 4; ++qi)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qb[qi][ks] = *reinterpret_cast<const bf16x8*>(qt + ((size_t)bh * Lp + m * kC + 16 * qi + r) * kD + 32 * ks + 8 * g);
        ql[qi][ks] = bf16x8{};
      }
  }

  // ---------------------------------------------------------------- right-to-left scan over key chunks
  const int64_t nstart = mtop - 1;
  constexpr int NV = NM * 2;  // 16-byte vectors per thread per staged chunk
  uint4 stage[NV];
  float fstage = 0.f;
  auto load_chunk = [&](int64_t n) {
    const __bf16* src[4] = {kt + ((size_t)bh * Lp + n * kC) * kD, vt + ((size_t)bh * M + n) * kD * kC,
                            p_hi + ((size_t)bh * M + n) * kD * kD,
                            X3 ? p_lo + ((size_t)bh * M + n) * kD * kD : nullptr};
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = tid + 256 * h;
        stage[mi * 2 + h] = *reinterpret_cast<const uint4*>(src[mi] + (e >> 3) * 64 + (e & 7) * 8);
      }
    if (FOX && tid < 64) fstage = fl[bh * Lp + n * kC + tid];
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = tid + 256 * h;
        *reinterpret_cast<uint4*>(&lds[buf][mi][(e >> 3) * kLDB + (e & 7) * 8]) = stage[mi * 2 + h];
      }
    if (FOX && tid < 64) lfl[buf][tid] = fstage;
  };

  if (nstart >= 0) {
    load_chunk(nstart);
    store_chunk(0);
  }
  __syncthreads();
  int buf = 0;
  float off = 0.f;
  for (int64_t n = nstart; n >= 0; --n) {
    if (n > 0) load_chunk(n - 1);
    if (active && n < m) {
      const __bf16* Kn = lds[buf][0];
      const __bf16* Vn = lds[buf][1];
      const __bf16* Pn = lds[buf][2];
      // S^T = ktilde_n Q_run^T
      f32x4 z[4][4];
#pragma unroll
      for (int kti = 0; kti < 4; ++kti) {
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) z[kti][qi] = zero;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = lds_frag(Kn, 16 * kti + r, 32 * ks + 8 * g);
#pragma unroll
          for (int qi = 0; qi < 4; ++qi) z[kti][qi] = mfma16(a, qb[qi][ks], z[kti][qi]);
        }
      }
      if (FOX) off += ftot[bh * M + n];
#pragma unroll
      for (int kti = 0; kti < 4; ++kti)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bias = FOX ? kLog2e * (off - lfl[buf][16 * kti + 4 * g + i]) : 0.f;
#pragma unroll
          for (int qi = 0; qi < 4; ++qi) z[kti][qi][i] = z[kti][qi][i] * sc + bias;
        }
      bf16x8 pb[4][2];
      absorb(z, pb);
      // O^T += V_n^T P^T
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = lds_frag(Vn, 16 * dt + r, 32 * ks + 8 * g);
#pragma unroll
          for (int qi = 0; qi < 4; ++qi) o[dt][qi] = mfma16(a, pb[qi][ks], o[dt][qi]);
        }
      // Q_run^T <- P_n Q_run^T
      if (n > 0) {
        f32x4 qn[4][4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
          for (int qi = 0; qi < 4; ++qi) qn[dt][qi] = zero;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = lds_frag(Pn, 16 * dt + r, 32 * ks + 8 * g);
#pragma unroll
            for (int qi = 0; qi < 4; ++qi) qn[dt][qi] = mfma16(a, qb[qi][ks], qn[dt][qi]);
            if (X3) {
              const bf16x8 alo = lds_frag(lds[buf][3], 16 * dt + r, 32 * ks + 8 * g);
#pragma unroll
              for (int qi = 0; qi < 4; ++qi) {
                qn[dt][qi] = mfma16(a, ql[qi][ks], qn[dt][qi]);
                qn[dt][qi] = mfma16(alo, qb[qi][ks], qn[dt][qi]);
              }
            }
          }
        }
#pragma unroll
        for (int qi = 0; qi < 4; ++qi)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float vq = qn[2 * ks + (j >> 2)][qi][j & 3];
              const __bf16 hi = (__bf16)vq;
              qb[qi][ks][j] = hi;
              if (X3) ql[qi][ks][j] = (__bf16)(vq - (float)hi);
            }
      }
    }
    if (n > 0) store_chunk(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    float lt = lrow[qi];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int a = 16 * qi + r;
    const int64_t i = m * kC + a;
    if (active && i < L) {
      const float inv = 1.f / lt;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<bf16x4*>(out + ((size_t)bh * L + i) * kD + 16 * dt + 4 * g) =
            pack4(o[dt][qi][0] * inv, o[dt][qi][1] * inv, o[dt][qi][2] * inv, o[dt][qi][3] * inv);
      if (lse != nullptr && g == 0)
        lse[bh * L + i] = (mrow[qi] + fast_log2(lt)) * kLn2 + (FOX ? fl[bh * Lp + i] : 0.f);
    }
  }
}

// =========================================================================== host
bool mfma_supported(int d, int chunk) { return d == kD && chunk == kC; }

template <bool FOX, bool X3>
static void launch_attn(dim3 grid, hipStream_t st, const __bf16* qt, const __bf16* kt, const __bf16* vt,
                        const __bf16* p_hi, const __bf16* p_lo, const float* Sm, const float* fl, const float* ftot,
                        __bf16* out, float* lse, int64_t L, int64_t M, float sc) {
  mfma_attn_kernel<FOX, X3><<<grid, 256, 0, st>>>(qt, kt, vt, p_hi, p_lo, Sm, fl, ftot, out, lse, L, M, sc);
}

hipError_t mfma_fwd(int chunk, int transport, const void* q, const void* k, const void* v, const void* w,
                    const float* beta, const float* logf, void* out, float* lse, int64_t BH, int64_t L,
                    float scale, void* qt, void* kt, void* vt, void* p_hi, void* p_lo, float* Sm, float* fl,
                    float* ftot, hipStream_t st) {
  if (chunk != kC) return hipErrorInvalidValue;
  const int64_t M = (L + kC - 1) / kC;
  hipError_t e = hipFuncSetAttribute((const void*)mfma_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kPrepLds);
  if (e != hipSuccess) return e;
  const bool x3 = transport == 1;
  mfma_prep_kernel<<<dim3((unsigned)M, (unsigned)BH), 256, kPrepLds, st>>>(
      (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)w, beta, logf, L, M, (__bf16*)qt,
      (__bf16*)kt, (__bf16*)vt, (__bf16*)p_hi, x3 ? (__bf16*)p_lo : nullptr, Sm, fl, ftot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((M + 3) / 4), (unsigned)BH);
  const float sc = scale * kLog2e;
  const bool fox = logf != nullptr;
  auto args = [&](auto fn) {
    fn(grid, st, (const __bf16*)qt, (const __bf16*)kt, (const __bf16*)vt, (const __bf16*)p_hi,
       (const __bf16*)p_lo, Sm, fl, ftot, (__bf16*)out, lse, L, M, sc);
  };
  if (fox && x3) args(launch_attn<true, true>);
  else if (fox) args(launch_attn<true, false>);
  else if (x3) args(launch_attn<false, true>);
  else args(launch_attn<false, false>);
  return hipGetLastError();
}

}  // namespace pathattn
