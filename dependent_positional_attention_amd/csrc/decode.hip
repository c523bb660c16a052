// PaTH decode step (PaTH summary, gist.science/ko/paper/2505.16381, section 3
// "inference"): the cached keys absorb the newest transition in place,
// k_j <- (I - beta_t w_t w_t^T) k_j for every cached j < t, so no transition
// vectors are kept; the new token's key enters untransformed; the query then
// attends over the updated cache with a FlashDecoding-style split over keys.
//
// Kernel 1 (update_attend): grid (splits, B*H).  A workgroup owns the key range
// [j0, j1) of one (b, h) -- ranges are disjoint, so the in-place writes never
// race.  Each key row is read with 16-byte loads by a group of LPK lanes
// (LPK = d / elements-per-16-bytes); the group reduces w.k and q.k with lane
// shuffles, writes the updated key back, and keeps an online-softmax state
// (running max, sum, partial output slice).  Groups are merged through LDS and
// the split's (m, l, o[d]) partial goes to the workspace.
// Kernel 2 (combine): one workgroup per (b, h) merges the splits.
//
// PaTH-FoX (same page, section 2): each slot also carries its forget bias
// sum_{s=j+1..t} f_s as an fp32 value that grows in place by the newest gate,
// exactly like the keys absorb the newest transition; the new slot starts at 0.
// Ragged batches: an optional per-sequence token count replaces the uniform t;
// the split of the key range is sized for the uniform bound.
#include <mutex>

#include "common.h"

namespace pathattn {

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<__bf16> {
  static constexpr int N = 8;
  typedef uint4 raw;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  typedef uint4 raw;
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& r, float* f);
template <>
__device__ __forceinline__ void unpack16<__bf16>(const uint4& r, float* f) {
  const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& r, float* f) {
  f[0] = __uint_as_float(r.x);
  f[1] = __uint_as_float(r.y);
  f[2] = __uint_as_float(r.z);
  f[3] = __uint_as_float(r.w);
}

template <typename T>
__device__ __forceinline__ uint4 pack16(const float* f);
template <>
__device__ __forceinline__ uint4 pack16<__bf16>(const float* f) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 lo = (__bf16)f[2 * i], hi = (__bf16)f[2 * i + 1];
    u[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}
template <>
__device__ __forceinline__ uint4 pack16<float>(const float* f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

// Non-temporal cache accesses for the in-place step, which reads and rewrites every cached key once:
// with both its loads and its stores marked streaming it runs 7% faster at a 64K-token cache (either
// alone changes nothing), while the read-only steps of the deferred kernel are faster with plain loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void stream_store(uint4* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// Sum over the LPK lanes of a key group (groups are aligned runs of LPK lanes).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

constexpr int kDecThreads = 256;
#ifndef PATHATTN_DEC_UNROLL
#define PATHATTN_DEC_UNROLL 4
#endif
constexpr int kDecUnroll = PATHATTN_DEC_UNROLL;

// Merge the key groups' online-softmax states (m, l, o) of one block through LDS and write the
// block's partial (m, l, o[D]) for the combine kernel.
template <int D, int VN, int LPK>
__device__ __forceinline__ void merge_block(float mrun, float lrun, const float (&o)[VN], float* __restrict__ pp) {
  constexpr int GPB = kDecThreads / LPK;
  const int tid = threadIdx.x, grp = tid / LPK, sub = tid % LPK;
  __shared__ float sm[GPB], sl[GPB];
  __shared__ float so[GPB * D];
  if (sub == 0) {
    sm[grp] = mrun;
    sl[grp] = lrun;
  }
#pragma unroll
  for (int x = 0; x < VN; ++x) so[grp * D + sub * VN + x] = o[x];
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
    for (int g = 0; g < GPB; ++g) M = fmaxf(M, sm[g]);
    float Lsum = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int g = 0; g < GPB; ++g) {
        const float f = fast_exp2(sm[g] - M);
        Lsum += sl[g] * f;
        acc += so[g * D + tid] * f;
      }
    }
    pp[2 + tid] = acc;
    if (tid == 0) {
      pp[0] = M;
      pp[1] = Lsum;
    }
  }
}

// Online-softmax update of a group's state with kDecUnroll logits z (log2 units) and their values.
template <int VN>
__device__ __forceinline__ void absorb(float& mrun, float& lrun, float (&o)[VN], const float (&z)[kDecUnroll],
                                       const float (&vf)[kDecUnroll][VN]) {
  float bm = z[0];
#pragma unroll
  for (int u = 1; u < kDecUnroll; ++u) bm = fmaxf(bm, z[u]);
  const float mnew = fmaxf(mrun, bm);
  if (mnew != -INFINITY) {
    const float alpha = fast_exp2(mrun - mnew);
    lrun *= alpha;
#pragma unroll
    for (int x = 0; x < VN; ++x) o[x] *= alpha;
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const float p = fast_exp2(z[u] - mnew);
      lrun += p;
#pragma unroll
      for (int x = 0; x < VN; ++x) o[x] += p * vf[u][x];
    }
    mrun = mnew;
  }
}

// Token count of sequence b: the uniform t, or t_batch[b] when given; -1 marks an entry outside [0, t].
__device__ __forceinline__ int64_t seq_tokens(const int* t_batch, int64_t bh, int H, int64_t t) {
  if (t_batch == nullptr) return t;
  const int64_t tb = t_batch[bh / H];
  return (tb < 0 || tb > t) ? -1 : tb;
}

template <typename T, int D, bool FOX>
__global__ __launch_bounds__(kDecThreads) void decode_update_attend_kernel(
    T* __restrict__ kc, T* __restrict__ vc, float* __restrict__ fc, int64_t cap, int64_t t_max,
    const int* __restrict__ t_batch, int H, const T* __restrict__ q_t, const T* __restrict__ k_t,
    const T* __restrict__ v_t, const T* __restrict__ w_t, const float* __restrict__ beta_t,
    const float* __restrict__ f_t, float scale_log2, int splits, int64_t keys_per_split, float* __restrict__ part) {
  constexpr int VN = Vec16<T>::N;  // elements per 16-byte vector
  constexpr int LPK = D / VN;      // lanes per key
  constexpr int GPB = kDecThreads / LPK;  // key groups per block
  static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "bad lanes per key");

  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int grp = tid / LPK, sub = tid % LPK;

  const int64_t t = seq_tokens(t_batch, bh, H, t_max);  // -1: no keys, nothing written
  const int64_t j0 = (int64_t)split * keys_per_split;
  int64_t j1 = j0 + keys_per_split;
  if (j1 > t + 1) j1 = t + 1;

  float wv[VN], qv[VN];
  {
    const uint4* wp = (const uint4*)(w_t + bh * D) + sub;
    const uint4* qp = (const uint4*)(q_t + bh * D) + sub;
    unpack16<T>(*wp, wv);
    unpack16<T>(*qp, qv);
  }
  const float beta = beta_t[bh];
  T* kb = kc + (size_t)bh * cap * D;
  T* vb = vc + (size_t)bh * cap * D;
  float* fb = FOX ? fc + (size_t)bh * cap : nullptr;
  const float fnew = FOX ? f_t[bh] : 0.f;

  float mrun = -INFINITY, lrun = 0.f, o[VN];
#pragma unroll
  for (int x = 0; x < VN; ++x) o[x] = 0.f;

  for (int64_t base = j0 + grp; base < j1; base += (int64_t)GPB * kDecUnroll) {
    uint4 kr[kDecUnroll], vr[kDecUnroll];
    int64_t jj[kDecUnroll];
    float fb_old[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      jj[u] = base + (int64_t)u * GPB;
      kr[u] = make_uint4(0u, 0u, 0u, 0u);  // keys past the range contribute exp2(-inf) * 0
      vr[u] = make_uint4(0u, 0u, 0u, 0u);
      fb_old[u] = 0.f;
      if (jj[u] < j1) {
        if (jj[u] < t) {
          kr[u] = stream_load((const uint4*)(kb + jj[u] * D) + sub);
          if constexpr (FOX) fb_old[u] = fb[jj[u]];
        } else {  // jj == t: the new token
          kr[u] = *((const uint4*)(k_t + bh * D) + sub);
        }
        vr[u] = (jj[u] < t) ? stream_load((const uint4*)(vb + jj[u] * D) + sub) : *((const uint4*)(v_t + bh * D) + sub);
      }
    }
    float z[kDecUnroll];
    float vf[kDecUnroll][VN];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float kf[VN];
      unpack16<T>(kr[u], kf);
      unpack16<T>(vr[u], vf[u]);
      const bool live = jj[u] < j1;
      float bias = 0.f;  // forget bias of the slot after this step (the new slot: 0)
      if constexpr (FOX) {
        if (live && jj[u] < t) bias = fb_old[u] + fnew;
        if (live && sub == 0) fb[jj[u]] = bias;
      }
      if (live && jj[u] < t) {
        float pd = 0.f;
#pragma unroll
        for (int x = 0; x < VN; ++x) pd += wv[x] * kf[x];
        const float coef = beta * group_sum<LPK>(pd);
#pragma unroll
        for (int x = 0; x < VN; ++x) kf[x] -= coef * wv[x];
        const uint4 nk = pack16<T>(kf);
        stream_store((uint4*)(kb + jj[u] * D) + sub, nk);
        unpack16<T>(nk, kf);  // attend with exactly the stored key
      } else if (live) {  // slot t: the new token, stored untransformed
        *((uint4*)(kb + jj[u] * D) + sub) = kr[u];
        *((uint4*)(vb + jj[u] * D) + sub) = vr[u];
      }
      float sd = 0.f;
#pragma unroll
      for (int x = 0; x < VN; ++x) sd += qv[x] * kf[x];
      sd = group_sum<LPK>(sd);
      z[u] = live ? sd * scale_log2 + (FOX ? bias * kLog2e : 0.f) : -INFINITY;
    }
    absorb<VN>(mrun, lrun, o, z, vf);
  }

  merge_block<D, VN, LPK>(mrun, lrun, o, part + ((size_t)bh * splits + split) * (D + 2));
}

// ------------------------------------------------------------------------------------ deferred updates
// The same step with the key updates deferred: the slots are brought up to date only every `period`
// steps, and in between each step transports its query instead, which leaves the cached keys
// untouched (read once, not read and written).  With t_cur the number of slots that are current
// (they have absorbed every transition of steps < t_cur) and np = t - t_cur pending steps whose
// transitions T_0 .. T_{np-1} (steps t_cur .. t-1) sit in `state`, plus T_np = H_t:
//   slot j <  t_cur:         logit = slot_j . Q_0                  Q_i = T_i T_{i+1} ... T_np q_t
//   slot t_cur <= j < t:     logit = slot_j . Q_{j - t_cur + 1}    (raw key, transitions after it)
//   slot t:                  logit = k_t . q_t                     (Q_{np+1} = q_t)
// which is k_j(t) . q_t for every j, the in-place rule's logit, transition for transition.  On the
// step with np + 1 == period the slots take all pending transitions in order (T_0 first for the
// current slots, T_{j - t_cur + 1} first for the raw ones), are written back, and score against q_t as
// in the in-place kernel.  PaTH-FoX: with G_i = sum of the gates of steps t_cur + i .. t, a current
// slot's bias is its stored value plus G_0 and a raw slot's is G_{j - t_cur + 1}; the update step
// stores them.  State per (b, h): kMaxPeriod directions (fp32, d each), then kMaxPeriod strengths and
// kMaxPeriod gates.
constexpr int kMaxPeriod = 16;

template <typename T, int D, bool FOX>
__global__ __launch_bounds__(kDecThreads) void decode_deferred_kernel(
    T* __restrict__ kc, T* __restrict__ vc, float* __restrict__ fc, int64_t cap, int64_t t, int64_t t_cur,
    int period, float* __restrict__ state, const T* __restrict__ q_t, const T* __restrict__ k_t,
    const T* __restrict__ v_t, const T* __restrict__ w_t, const float* __restrict__ beta_t,
    const float* __restrict__ f_t, float scale_log2, int splits, int64_t keys_per_split, float* __restrict__ part) {
  constexpr int VN = Vec16<T>::N;
  constexpr int LPK = D / VN;
  constexpr int GPB = kDecThreads / LPK;
  constexpr int SS = kMaxPeriod * (D + 2);  // state floats per (b, h)
  __shared__ float Wl[kMaxPeriod][D], Ql[kMaxPeriod + 1][D], Bl[kMaxPeriod], Gl[kMaxPeriod + 1];

  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int grp = tid / LPK, sub = tid % LPK;
  const int np = (int)(t - t_cur);
  const bool flush = np + 1 == period;
  float* st = state + (size_t)bh * SS;

  // transitions T_0 .. T_np, their strengths and gates, and q_t
  for (int e = tid; e < (np + 1) * D; e += kDecThreads) {
    const int i = e / D, x = e % D;
    Wl[i][x] = i < np ? st[i * D + x] : to_f32(w_t[bh * D + x]);
  }
  if (tid <= np) Bl[tid] = tid < np ? st[kMaxPeriod * D + tid] : beta_t[bh];
  if (tid < D) Ql[np + 1][tid] = to_f32(q_t[bh * D + tid]);
  __syncthreads();
  // Q_i = T_i Q_{i+1} for i = np .. 0 (wave 0, two elements per lane), gate suffix sums G_i
  if (tid < 64) {
    float q0 = tid < D ? Ql[np + 1][tid] : 0.f, q1 = tid + 64 < D ? Ql[np + 1][tid + 64] : 0.f;
    float gs = 0.f;
    if (tid == 0) Gl[np + 1] = 0.f;
    for (int i = np; i >= 0; --i) {
      const float w0 = tid < D ? Wl[i][tid] : 0.f, w1 = tid + 64 < D ? Wl[i][tid + 64] : 0.f;
      float dp = w0 * q0 + w1 * q1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) dp += __shfl_xor(dp, o, 64);
      const float c = Bl[i] * dp;
      q0 -= c * w0;
      q1 -= c * w1;
      if (tid < D) Ql[i][tid] = q0;
      if (tid + 64 < D) Ql[i][tid + 64] = q1;
      if constexpr (FOX) {
        gs += i < np ? st[kMaxPeriod * (D + 1) + i] : f_t[bh];
        if (tid == 0) Gl[i] = gs;
      }
    }
  }
  __syncthreads();

  const int64_t j0 = (int64_t)split * keys_per_split;
  int64_t j1 = j0 + keys_per_split;
  if (j1 > t + 1) j1 = t + 1;
  T* kb = kc + (size_t)bh * cap * D;
  T* vb = vc + (size_t)bh * cap * D;
  float* fb = FOX ? fc + (size_t)bh * cap : nullptr;
  // the current slots score against Q_0 (flush: against q_t after their update)
  float qv[VN];
#pragma unroll
  for (int x = 0; x < VN; ++x) qv[x] = Ql[flush ? np + 1 : 0][sub * VN + x];
  const float g0 = FOX ? Gl[0] : 0.f;

  float mrun = -INFINITY, lrun = 0.f, o[VN];
#pragma unroll
  for (int x = 0; x < VN; ++x) o[x] = 0.f;

  for (int64_t base = j0 + grp; base < j1; base += (int64_t)GPB * kDecUnroll) {
    uint4 kr[kDecUnroll], vr[kDecUnroll];
    int64_t jj[kDecUnroll];
    float fb_old[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      jj[u] = base + (int64_t)u * GPB;
      kr[u] = make_uint4(0u, 0u, 0u, 0u);
      vr[u] = make_uint4(0u, 0u, 0u, 0u);
      fb_old[u] = 0.f;
      if (jj[u] < j1) {
        if (jj[u] < t) {
          kr[u] = *((const uint4*)(kb + jj[u] * D) + sub);
          if constexpr (FOX) {
            if (jj[u] < t_cur) fb_old[u] = fb[jj[u]];
          }
        } else {
          kr[u] = *((const uint4*)(k_t + bh * D) + sub);
        }
        vr[u] = (jj[u] < t) ? *((const uint4*)(vb + jj[u] * D) + sub) : *((const uint4*)(v_t + bh * D) + sub);
      }
    }
    float z[kDecUnroll];
    float vf[kDecUnroll][VN], kf[kDecUnroll][VN];
    int i0[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      unpack16<T>(kr[u], kf[u]);
      unpack16<T>(vr[u], vf[u]);
      const int64_t j = jj[u];
      i0[u] = (j >= t_cur && j < t) ? (int)(j - t_cur) + 1 : 0;  // first pending transition of a raw key
    }
    if (flush) {  // every slot below t takes its pending transitions, the four keys interleaved
      for (int i = 0; i <= np; ++i) {
        float w[VN], pd[kDecUnroll];
#pragma unroll
        for (int x = 0; x < VN; ++x) w[x] = Wl[i][sub * VN + x];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
          pd[u] = 0.f;
#pragma unroll
          for (int x = 0; x < VN; ++x) pd[u] += w[x] * kf[u][x];
        }
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) pd[u] = group_sum<LPK>(pd[u]);
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
          if (jj[u] < t && i >= i0[u]) {
            const float c = Bl[i] * pd[u];
#pragma unroll
            for (int x = 0; x < VN; ++x) kf[u][x] -= c * w[x];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int64_t j = jj[u];
      const bool live = j < j1;
      const bool raw = j >= t_cur && j < t;  // key appended since the last update
      float bias = 0.f;
      if constexpr (FOX) bias = j < t_cur ? fb_old[u] + g0 : (raw ? Gl[i0[u]] : 0.f);
      float qj[VN];
#pragma unroll
      for (int x = 0; x < VN; ++x) qj[x] = qv[x];
      if (live && j < t) {
        if (flush) {
          const uint4 nk = pack16<T>(kf[u]);
          *((uint4*)(kb + j * D) + sub) = nk;
          unpack16<T>(nk, kf[u]);  // attend with exactly the stored key
          if constexpr (FOX) {
            if (sub == 0) fb[j] = bias;
          }
        } else if (raw) {
#pragma unroll
          for (int x = 0; x < VN; ++x) qj[x] = Ql[i0[u]][sub * VN + x];
        }
      } else if (live) {  // slot t: the new token, stored untransformed
        *((uint4*)(kb + j * D) + sub) = kr[u];
        *((uint4*)(vb + j * D) + sub) = vr[u];
        if constexpr (FOX) {
          if (sub == 0) fb[j] = 0.f;
        }
#pragma unroll
        for (int x = 0; x < VN; ++x) qj[x] = Ql[np + 1][sub * VN + x];
      }
      float sd = 0.f;
#pragma unroll
      for (int x = 0; x < VN; ++x) sd += qj[x] * kf[u][x];
      sd = group_sum<LPK>(sd);
      z[u] = live ? sd * scale_log2 + (FOX ? bias * kLog2e : 0.f) : -INFINITY;
    }
    absorb<VN>(mrun, lrun, o, z, vf);
  }
  // keep this step's transition for the steps until the next update (one block per (b, h) writes it)
  if (!flush && split == 0) {
    for (int x = tid; x < D; x += kDecThreads) st[np * D + x] = Wl[np][x];
    if (tid == 0) {
      st[kMaxPeriod * D + np] = Bl[np];
      if constexpr (FOX) st[kMaxPeriod * (D + 1) + np] = f_t[bh];
    }
  }
  merge_block<D, VN, LPK>(mrun, lrun, o, part + ((size_t)bh * splits + split) * (D + 2));
}

// Merge of the split partials (m, l, o[D]) of one (b, h): one wave.  Lanes stride over the splits for the
// reference max and the denominator (wave reductions); the weights of each run of 64 splits go through LDS
// once, and each output column sums its partials with independent loads.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part, int splits,
                                                            const int* __restrict__ t_batch, int H, int64_t t_max,
                                                            T* __restrict__ out, float* __restrict__ lse) {
  constexpr int XP = (D + 63) / 64;  // output columns per lane
  __shared__ float wsh[64];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  if (seq_tokens(t_batch, bh, H, t_max) < 0) {  // invalid token count: NaN out, nothing else touched
    for (int x = lane; x < D; x += 64) out[bh * D + x] = from_f32<T>(__builtin_nanf(""));
    if (lse != nullptr && lane == 0) lse[bh] = __builtin_nanf("");
    return;
  }
  const float* pp = part + (size_t)bh * splits * (D + 2);
  float M = -INFINITY;
  for (int s = lane; s < splits; s += 64) M = fmaxf(M, pp[(size_t)s * (D + 2)]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float Lsum = 0.f;
  for (int s = lane; s < splits; s += 64) {
    const float m = pp[(size_t)s * (D + 2)];
    if (m != -INFINITY) Lsum += pp[(size_t)s * (D + 2) + 1] * fast_exp2(m - M);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) Lsum += __shfl_xor(Lsum, o, 64);
  float acc[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 64) {
    const int n = splits - s0 < 64 ? splits - s0 : 64;
    {
      const float m = lane < n ? pp[(size_t)(s0 + lane) * (D + 2)] : -INFINITY;
      wsh[lane] = m != -INFINITY ? fast_exp2(m - M) : 0.f;  // empty splits weigh nothing
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      const int x = lane + 64 * j;
      if (x < D) {
        float a = 0.f;
#pragma unroll 8
        for (int i = 0; i < n; ++i) a += wsh[i] * pp[(size_t)(s0 + i) * (D + 2) + 2 + x];
        acc[j] += a;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  const float inv = 1.f / Lsum;
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    const int x = lane + 64 * j;
    if (x < D) out[bh * D + x] = from_f32<T>(acc[j] * inv);
  }
  if (lse != nullptr && lane == 0) lse[bh] = (M + fast_log2(Lsum)) * kLn2;
}

template <typename T, int D>
static hipError_t launch_decode(void* kc, void* vc, float* fc, int64_t cap, int64_t t, const int* t_batch, int H,
                                const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                                const float* beta_t, const float* f_t, void* out, float* lse, int64_t BH, float scale,
                                int splits, float* part, hipStream_t st) {
  const int64_t keys = t + 1;
  const int64_t kps = (keys + splits - 1) / splits;
  dim3 grid((unsigned)splits, (unsigned)BH);
  if (f_t != nullptr)
    decode_update_attend_kernel<T, D, true><<<grid, kDecThreads, 0, st>>>(
        (T*)kc, (T*)vc, fc, cap, t, t_batch, H, (const T*)q_t, (const T*)k_t, (const T*)v_t, (const T*)w_t, beta_t,
        f_t, scale * kLog2e, splits, kps, part);
  else
    decode_update_attend_kernel<T, D, false><<<grid, kDecThreads, 0, st>>>(
        (T*)kc, (T*)vc, nullptr, cap, t, t_batch, H, (const T*)q_t, (const T*)k_t, (const T*)v_t, (const T*)w_t,
        beta_t, nullptr, scale * kLog2e, splits, kps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<T, D><<<(unsigned)BH, 64, 0, st>>>(part, splits, t_batch, H, t, (T*)out, lse);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_deferred(void* kc, void* vc, float* fc, int64_t cap, int64_t t, int64_t t_cur, int period,
                                  float* state, const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                                  const float* beta_t, const float* f_t, void* out, float* lse, int64_t BH,
                                  float scale, int splits, float* part, hipStream_t st) {
  const int64_t keys = t + 1;
  const int64_t kps = (keys + splits - 1) / splits;
  dim3 grid((unsigned)splits, (unsigned)BH);
  if (f_t != nullptr)
    decode_deferred_kernel<T, D, true><<<grid, kDecThreads, 0, st>>>(
        (T*)kc, (T*)vc, fc, cap, t, t_cur, period, state, (const T*)q_t, (const T*)k_t, (const T*)v_t,
        (const T*)w_t, beta_t, f_t, scale * kLog2e, splits, kps, part);
  else
    decode_deferred_kernel<T, D, false><<<grid, kDecThreads, 0, st>>>(
        (T*)kc, (T*)vc, nullptr, cap, t, t_cur, period, state, (const T*)q_t, (const T*)k_t, (const T*)v_t,
        (const T*)w_t, beta_t, nullptr, scale * kLog2e, splits, kps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<T, D><<<(unsigned)BH, 64, 0, st>>>(part, splits, nullptr, 1, t, (T*)out, lse);
  return hipGetLastError();
}

int decode_max_period() { return kMaxPeriod; }

hipError_t decode_step_deferred(bool bf16, int d, void* kc, void* vc, float* fc, int64_t cap, int64_t t,
                                int64_t t_cur, int period, float* state, const void* q_t, const void* k_t,
                                const void* v_t, const void* w_t, const float* beta_t, const float* f_t, void* out,
                                float* lse, int64_t BH, float scale, int splits, float* part, hipStream_t st) {
#define PATHATTN_DEF_CASE(DD)                                                                                  \
  if (d == DD)                                                                                                 \
    return bf16 ? launch_deferred<__bf16, DD>(kc, vc, fc, cap, t, t_cur, period, state, q_t, k_t, v_t, w_t,    \
                                              beta_t, f_t, out, lse, BH, scale, splits, part, st)              \
                : launch_deferred<float, DD>(kc, vc, fc, cap, t, t_cur, period, state, q_t, k_t, v_t, w_t,     \
                                             beta_t, f_t, out, lse, BH, scale, splits, part, st);
  PATHATTN_DEF_CASE(16)
  PATHATTN_DEF_CASE(32)
  PATHATTN_DEF_CASE(64)
  PATHATTN_DEF_CASE(128)
#undef PATHATTN_DEF_CASE
  return hipErrorInvalidValue;
}

bool decode_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// ------------------------------------------------------------------------------------ fixed scratch
// The split partials of path_decode_step_noalloc live in this file-scope device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy for the life of the process.  In
// host code the array's name is only a stand-in: its device address is resolved once per device with
// hipGetSymbolAddress (with that device current) and that address is what the kernels receive.  Every
// (b, h, split) partial is written by the update/attend kernel before the combine kernel reads it, so the
// array needs no clearing between calls; calls that overlap on one device race on it.
constexpr size_t kScratchFloats = (size_t)8 << 20;  // 32 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t decode_scratch_floats() { return kScratchFloats; }

// Device address of the scratch array on the device that runs `st` (the current device for the null
// stream), resolved on the first call for that device with the device made current for the lookup.
hipError_t decode_scratch(hipStream_t st, float** ptr) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (st != nullptr) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Keys per split chosen automatically: about 1024, so a 64K cache uses 64 splits per (b, h).
int64_t decode_auto_splits(int64_t keys) {
  int64_t s = (keys + 1023) / 1024;
  return s < 1 ? 1 : s;
}

hipError_t decode_step(bool bf16, int d, void* kc, void* vc, float* fc, int64_t cap, int64_t t, const int* t_batch,
                       int H, const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                       const float* beta_t, const float* f_t, void* out, float* lse, int64_t BH, float scale,
                       int splits, float* part, hipStream_t st) {
#define PATHATTN_DEC_CASE(DD)                                                                                    \
  if (d == DD)                                                                                                   \
    return bf16 ? launch_decode<__bf16, DD>(kc, vc, fc, cap, t, t_batch, H, q_t, k_t, v_t, w_t, beta_t, f_t, out, \
                                            lse, BH, scale, splits, part, st)                                   \
                : launch_decode<float, DD>(kc, vc, fc, cap, t, t_batch, H, q_t, k_t, v_t, w_t, beta_t, f_t, out,  \
                                           lse, BH, scale, splits, part, st);
  PATHATTN_DEC_CASE(16)
  PATHATTN_DEC_CASE(32)
  PATHATTN_DEC_CASE(64)
  PATHATTN_DEC_CASE(128)
#undef PATHATTN_DEC_CASE
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------ prompt slot biases
// PaTH-FoX slot biases after a prompt of L tokens: fc[j] = sum_{s=j+1..L-1} f_s.  One block per (b, h):
// thread i sums its contiguous segment, a suffix scan over the 256 segment sums (LDS) gives what lies
// to the right of each segment, and each thread then walks its segment right to left.
__global__ __launch_bounds__(256) void slot_bias_kernel(const float* __restrict__ logf, int64_t L, int64_t cap,
                                                        float* __restrict__ fc) {
  __shared__ float seg[256];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* f = logf + (size_t)bh * L;
  const int64_t per = (L + 255) / 256;
  const int64_t a = (int64_t)tid * per < L ? (int64_t)tid * per : L;
  const int64_t b = a + per < L ? a + per : L;
  float s = 0.f;
  for (int64_t j = a; j < b; ++j) s += f[j];
  seg[tid] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive suffix sums of the segment sums
    const float v = seg[tid] + (tid + off < 256 ? seg[tid + off] : 0.f);
    __syncthreads();
    seg[tid] = v;
    __syncthreads();
  }
  float acc = tid + 1 < 256 ? seg[tid + 1] : 0.f;  // gates after this segment
  float* out = fc + (size_t)bh * cap;
  for (int64_t j = b - 1; j >= a; --j) {
    out[j] = acc;
    acc += f[j];
  }
}

hipError_t slot_bias_run(const float* logf, int64_t BH, int64_t L, int64_t cap, float* fc, hipStream_t st) {
  slot_bias_kernel<<<dim3((unsigned)BH), 256, 0, st>>>(logf, L, cap, fc);
  return hipGetLastError();
}

}  // namespace pathattn
