// C ABI of libpathattn: argument validation, workspace planning and launches.
// Every check runs on the host before anything is enqueued (see path_attn.h).
#include "path_attn.h"

#include "backward.h"
#include "common.h"

namespace pathattn {
// vector_path.hip
bool vec_supported(int d, int chunk);
hipError_t vec_run(int phases, bool bf16, int d, int chunk, const void* q, const void* k, const void* v,
                   const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH, int64_t L,
                   float scale, float* qt, float* kt, float* Pm, float* Sm, float* fl, float* ftot, hipStream_t st);
hipError_t vec_cache_run(bool bf16, int d, int chunk, const float* kt, const float* Pm, const void* v, int64_t BH,
                         int64_t L, int64_t cap, void* kc, void* vc, hipStream_t st);
// mfma_path.hip
bool mfma_supported(int d, int chunk);
hipError_t mfma_run(int phases, int chunk, int transport, const void* q, const void* k, const void* v,
                    const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH,
                    int64_t L, float scale, void* qt, void* qt_lo, void* kt, void* p_hi, void* p_lo, void* kt2,
                    void* p2_hi, void* p2_lo, float* Sm, float* fl, float* ftot, hipStream_t st);
hipError_t mfma_cache_run(int transport, const void* kt, const void* p_hi, const void* p_lo, const void* v,
                          int64_t BH, int64_t L, int64_t cap, void* scratch, void* kc, void* vc, hipStream_t st);
size_t mfma_handoff_scratch_bytes(int64_t BH, int64_t M);
size_t mfma_s_chunk_bytes();
// decode.hip
bool decode_supported(int d);
int64_t decode_auto_splits(int64_t keys);
hipError_t decode_step(bool bf16, int d, void* kc, void* vc, float* fc, int64_t cap, int64_t t, const int* t_batch,
                       int H, const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                       const float* beta_t, const float* f_t, void* out, float* lse, int64_t BH, float scale,
                       int splits, float* part, hipStream_t st);
hipError_t slot_bias_run(const float* logf, int64_t BH, int64_t L, int64_t cap, float* fc, hipStream_t st);
size_t decode_scratch_floats();
hipError_t decode_scratch(hipStream_t st, float** ptr);
int decode_max_period();
hipError_t decode_step_deferred(bool bf16, int d, void* kc, void* vc, float* fc, int64_t cap, int64_t t,
                                int64_t t_cur, int period, float* state, const void* q_t, const void* k_t,
                                const void* v_t, const void* w_t, const float* beta_t, const float* f_t, void* out,
                                float* lse, int64_t BH, float scale, int splits, float* part, hipStream_t st);
}  // namespace pathattn

using namespace pathattn;

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxGridY = 65535;

bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool valid_dtype(int dt) { return dt == PATH_DTYPE_F32 || dt == PATH_DTYPE_BF16; }

// chunk 0 selects the chunk measured fastest for the path and length.  Matrix-core path (bf16, d = 64),
// whole prefill call, chunk 64 / 128 / 256 at about 3.1M tokens per call:
//   L = 512, 1024, 2048, 4096: chunk 64 fastest (the grouping kernel and the partial top group cost more
//                               than the transports they save at 8-64 chunks per sequence; 2-3% at 4096)
//   L = 8192, 16384, 32768:    chunk 256 fastest (3-7% ahead of chunk 64; the scan moves its queries
//                               once per 256 keys)
// so lengths up to kAutoChunkSplit take 64 and longer ones 256.  The vector path takes 64.
constexpr int64_t kAutoChunkSplit = 4096;
int resolve_chunk(int d, int dtype, int chunk, int64_t L) {
  if (chunk != 0) return chunk;
  if (dtype == PATH_DTYPE_BF16 && mfma_supported(d, 256) && L > kAutoChunkSplit) return 256;
  return 64;
}

// Which kernels serve (d, chunk, dtype): the matrix-core path for bf16 when built
// for the shape, the vector path otherwise.
path_status plan_fwd(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype, int transport,
                     path_ws_layout* lay, int64_t* off_handoff = nullptr) {
  chunk = resolve_chunk(d, dtype, chunk, L);
  if (B < 0 || H < 0 || L < 0 || d <= 0 || chunk <= 0) return PATH_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PATH_ERR_UNSUPPORTED;
  if (transport != PATH_TRANSPORT_BF16 && transport != PATH_TRANSPORT_BF16X3) return PATH_ERR_INVALID_ARG;
  const bool bf16 = dtype == PATH_DTYPE_BF16;
  const bool mfma = bf16 && mfma_supported(d, chunk);
  if (!mfma && !vec_supported(d, chunk)) return PATH_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  const int64_t M2 = (L + chunk - 1) / chunk;
  // the matrix-core path builds its per-chunk terms on 64-token (sub-)chunks
  const int sub = mfma ? 64 : chunk;
  const int64_t M = (L + sub - 1) / sub;
  const int64_t Lp = M * sub;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  *lay = path_ws_layout{};
  lay->num_chunks = M2;
  lay->num_sub_chunks = M;
  lay->off_p_lo = -1;
  lay->off_qtilde_lo = -1;
  lay->off_ktilde_c2 = lay->off_p_c2 = lay->off_p_c2_lo = -1;
  if (!mfma) {
    lay->layout_id = 0;
    lay->off_qtilde = take(BH * Lp * d * 4);
    lay->off_ktilde = take(BH * Lp * d * 4);
    lay->off_p = take(BH * M * d * d * 4);
  } else {
    lay->layout_id = chunk > 64 ? 2 : 1;
    lay->off_qtilde = take(BH * Lp * d * 2);
    if (transport == PATH_TRANSPORT_BF16X3) lay->off_qtilde_lo = take(BH * Lp * d * 2);
    lay->off_ktilde = take(BH * Lp * d * 2);
    lay->off_p = take(BH * M * d * d * 2);
    if (transport == PATH_TRANSPORT_BF16X3) lay->off_p_lo = take(BH * M * d * d * 2);
    if (chunk > 64) {  // chunks of G = chunk / 64 sub-chunks: carried keys, products of whole groups
      const int64_t MG = M / (chunk / 64);
      lay->off_ktilde_c2 = take(BH * Lp * d * 2);
      lay->off_p_c2 = take(BH * MG * d * d * 2);
      if (transport == PATH_TRANSPORT_BF16X3) lay->off_p_c2_lo = take(BH * MG * d * d * 2);
    }
  }
  lay->off_s = take(BH * M * (mfma ? (int64_t)mfma_s_chunk_bytes() : (int64_t)sub * sub * 4));
  lay->off_fox_local = take(BH * Lp * 4);
  lay->off_fox_total = take(BH * M * 4);
  const int64_t oh = take(mfma ? (int64_t)mfma_handoff_scratch_bytes(BH, M) : 0);  // hand-off scratch, last
  if (off_handoff != nullptr) *off_handoff = oh;
  lay->total_bytes = off;
  return PATH_OK;
}

path_status from_hip(hipError_t e) { return e == hipSuccess ? PATH_OK : PATH_ERR_HIP; }

}  // namespace

extern "C" {

int path_abi_version(void) { return PATH_ABI_VERSION; }

const char* path_status_string(int status) {
  switch (status) {
    case PATH_OK:
      return "ok";
    case PATH_ERR_INVALID_ARG:
      return "invalid argument";
    case PATH_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case PATH_ERR_HIP:
      return "HIP runtime error";
    case PATH_ERR_SCRATCH:
      return "problem exceeds the library's fixed scratch buffer (use the entry point with a workspace)";
    default:
      return "unknown status";
  }
}

path_status path_attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                          int transport, size_t* bytes) {
  if (bytes == nullptr) return PATH_ERR_INVALID_ARG;
  path_ws_layout lay;
  const path_status s = plan_fwd(B, H, L, d, chunk, dtype, transport, &lay);
  if (s != PATH_OK) return s;
  *bytes = (size_t)lay.total_bytes;
  return PATH_OK;
}

path_status path_attn_workspace_layout(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                       int transport, path_ws_layout* layout) {
  if (layout == nullptr) return PATH_ERR_INVALID_ARG;
  return plan_fwd(B, H, L, d, chunk, dtype, transport, layout);
}

}  // extern "C"

namespace {

constexpr int kPhasePrep = 1, kPhaseScan = 2;

// Shared body of path_attn_prep / path_attn_scan / path_attn_fwd.  The prep phase reads
// q, k, v, w, beta, log_forget; the scan phase reads v (vector path) and log_forget
// (only whether it is NULL) and writes out and lse.
path_status run_fwd(int phases, const void* q, const void* k, const void* v, const void* w, const float* beta,
                    const float* log_forget, void* out, float* lse, int64_t B, int64_t H, int64_t L, int d,
                    int chunk, float scale, int dtype, int transport, void* workspace, size_t workspace_bytes,
                    void* stream) {
  path_ws_layout lay;
  const path_status s = plan_fwd(B, H, L, d, chunk, dtype, transport, &lay);
  if (s != PATH_OK) return s;
  chunk = resolve_chunk(d, dtype, chunk, L);
  const int64_t BH = B * H;
  if (BH == 0 || L == 0) return PATH_OK;
  if (!workspace) return PATH_ERR_INVALID_ARG;
  if ((phases & kPhasePrep) && (!q || !k || !v || !w || !beta)) return PATH_ERR_INVALID_ARG;
  if ((phases & kPhaseScan) && (!out || !v)) return PATH_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(w) || misaligned(beta) ||
      misaligned(log_forget) || misaligned(out) || misaligned(lse) || misaligned(workspace))
    return PATH_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)lay.total_bytes) return PATH_ERR_INVALID_ARG;
  if (BH > kMaxGridY || lay.num_sub_chunks > kMaxGridY) return PATH_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* fl = reinterpret_cast<float*>(ws + lay.off_fox_local);
  float* ftot = reinterpret_cast<float*>(ws + lay.off_fox_total);
  float* Sm = reinterpret_cast<float*>(ws + lay.off_s);
  if (lay.layout_id >= 1) {
    auto at = [&](int64_t o) -> void* { return o >= 0 ? ws + o : nullptr; };
    return from_hip(mfma_run(phases, chunk, transport, q, k, v, w, beta, log_forget, out, lse, BH, L, scale,
                             at(lay.off_qtilde), at(lay.off_qtilde_lo), at(lay.off_ktilde), at(lay.off_p),
                             at(lay.off_p_lo), at(lay.off_ktilde_c2), at(lay.off_p_c2), at(lay.off_p_c2_lo), Sm, fl,
                             ftot, st));
  }
  return from_hip(vec_run(phases, dtype == PATH_DTYPE_BF16, d, chunk, q, k, v, w, beta, log_forget, out, lse, BH, L,
                          scale, reinterpret_cast<float*>(ws + lay.off_qtilde),
                          reinterpret_cast<float*>(ws + lay.off_ktilde), reinterpret_cast<float*>(ws + lay.off_p),
                          Sm, fl, ftot, st));
}

}  // namespace

extern "C" {

path_status path_attn_fwd(const void* q, const void* k, const void* v, const void* w, const float* beta,
                          const float* log_forget, void* out, float* lse, int64_t B, int64_t H, int64_t L,
                          int d, int chunk, float scale, int dtype, int transport, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run_fwd(kPhasePrep | kPhaseScan, q, k, v, w, beta, log_forget, out, lse, B, H, L, d, chunk, scale, dtype,
                 transport, workspace, workspace_bytes, stream);
}

path_status path_attn_prep(const void* q, const void* k, const void* v, const void* w, const float* beta,
                           const float* log_forget, int64_t B, int64_t H, int64_t L, int d, int chunk, float scale,
                           int dtype, int transport, void* workspace, size_t workspace_bytes, void* stream) {
  return run_fwd(kPhasePrep, q, k, v, w, beta, log_forget, nullptr, nullptr, B, H, L, d, chunk, scale, dtype,
                 transport, workspace, workspace_bytes, stream);
}

path_status path_attn_scan(const void* v, const float* log_forget, void* out, float* lse, int64_t B, int64_t H,
                           int64_t L, int d, int chunk, int dtype, int transport, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_fwd(kPhaseScan, nullptr, nullptr, v, nullptr, nullptr, log_forget, out, lse, B, H, L, d, chunk, 1.f,
                 dtype, transport, workspace, workspace_bytes, stream);
}

path_status path_attn_cache_from_prefill(const void* v, const float* log_forget, void* workspace,
                                         size_t workspace_bytes, void* kcache, void* vcache, float* fcache,
                                         int64_t capacity, int64_t B, int64_t H, int64_t L, int d, int chunk,
                                         int dtype, int transport, void* stream) {
  path_ws_layout lay;
  int64_t off_handoff = 0;
  const path_status s = plan_fwd(B, H, L, d, chunk, dtype, transport, &lay, &off_handoff);
  if (s != PATH_OK) return s;
  chunk = resolve_chunk(d, dtype, chunk, L);
  if (capacity < L) return PATH_ERR_INVALID_ARG;
  if ((log_forget == nullptr) != (fcache == nullptr)) return PATH_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  if (BH == 0 || L == 0) return PATH_OK;
  if (!v || !workspace || !kcache || !vcache) return PATH_ERR_INVALID_ARG;
  if (misaligned(v) || misaligned(workspace) || misaligned(kcache) || misaligned(vcache) || misaligned(log_forget) ||
      misaligned(fcache))
    return PATH_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)lay.total_bytes) return PATH_ERR_INVALID_ARG;
  if (BH > (int64_t)0x7fffffff) return PATH_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (lay.layout_id >= 1)
    e = mfma_cache_run(transport, ws + lay.off_ktilde, ws + lay.off_p, lay.off_p_lo >= 0 ? ws + lay.off_p_lo : nullptr,
                       v, BH, L, capacity, ws + off_handoff, kcache, vcache, st);
  else
    e = vec_cache_run(dtype == PATH_DTYPE_BF16, d, chunk, reinterpret_cast<const float*>(ws + lay.off_ktilde),
                      reinterpret_cast<const float*>(ws + lay.off_p), v, BH, L, capacity, kcache, vcache, st);
  if (e == hipSuccess && log_forget != nullptr) e = slot_bias_run(log_forget, BH, L, capacity, fcache, st);
  return from_hip(e);
}

path_status path_decode_workspace_bytes(int64_t B, int64_t H, int d, int64_t capacity, int splits,
                                        size_t* bytes) {
  if (bytes == nullptr || B < 0 || H < 0 || capacity < 0 || splits < 0) return PATH_ERR_INVALID_ARG;
  if (!decode_supported(d)) return PATH_ERR_UNSUPPORTED;
  const int64_t S = splits > 0 ? splits : decode_auto_splits(capacity);
  *bytes = (size_t)(B * H * S * (int64_t)(d + 2) * 4);
  return PATH_OK;
}

path_status path_decode_step(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                             const int* t_batch, const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                             const float* beta_t, const float* log_forget_t, void* out, float* lse, int64_t B,
                             int64_t H, int d, float scale, int dtype, int splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || capacity < 0 || splits < 0) return PATH_ERR_INVALID_ARG;
  if (!valid_dtype(dtype) || !decode_supported(d)) return PATH_ERR_UNSUPPORTED;
  if (t < 0 || t >= capacity) return PATH_ERR_INVALID_ARG;
  if ((log_forget_t == nullptr) != (fcache == nullptr)) return PATH_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  if (BH == 0) return PATH_OK;
  if (!kcache || !vcache || !q_t || !k_t || !v_t || !w_t || !beta_t || !out || !workspace)
    return PATH_ERR_INVALID_ARG;
  if (misaligned(kcache) || misaligned(vcache) || misaligned(q_t) || misaligned(k_t) || misaligned(v_t) ||
      misaligned(w_t) || misaligned(beta_t) || misaligned(out) || misaligned(lse) || misaligned(workspace) ||
      misaligned(fcache) || misaligned(log_forget_t) || misaligned(t_batch))
    return PATH_ERR_UNSUPPORTED;
  if (H > (int64_t)0x7fffffff) return PATH_ERR_UNSUPPORTED;
  const int64_t S = splits > 0 ? splits : decode_auto_splits(t + 1);
  if (S > (int64_t)0x7fffffff) return PATH_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)(BH * S * (int64_t)(d + 2) * 4)) return PATH_ERR_INVALID_ARG;
  if (BH > kMaxGridY) return PATH_ERR_UNSUPPORTED;
  return from_hip(decode_step(dtype == PATH_DTYPE_BF16, d, kcache, vcache, fcache, capacity, t, t_batch, (int)H, q_t,
                              k_t, v_t, w_t, beta_t, log_forget_t, out, lse, BH, scale, (int)S,
                              static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

path_status path_decode_step_noalloc(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                                     const int* t_batch, const void* q_t, const void* k_t, const void* v_t,
                                     const void* w_t, const float* beta_t, const float* log_forget_t, void* out,
                                     float* lse, int64_t B, int64_t H, int d, float scale, int dtype, int splits,
                                     void* stream) {
  if (B < 0 || H < 0 || capacity < 0 || splits < 0) return PATH_ERR_INVALID_ARG;
  if (!valid_dtype(dtype) || !decode_supported(d)) return PATH_ERR_UNSUPPORTED;
  if (t < 0 || t >= capacity) return PATH_ERR_INVALID_ARG;
  if ((log_forget_t == nullptr) != (fcache == nullptr)) return PATH_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  if (BH == 0) return PATH_OK;
  if (!kcache || !vcache || !q_t || !k_t || !v_t || !w_t || !beta_t || !out) return PATH_ERR_INVALID_ARG;
  if (misaligned(kcache) || misaligned(vcache) || misaligned(q_t) || misaligned(k_t) || misaligned(v_t) ||
      misaligned(w_t) || misaligned(beta_t) || misaligned(out) || misaligned(lse) || misaligned(fcache) ||
      misaligned(log_forget_t) || misaligned(t_batch))
    return PATH_ERR_UNSUPPORTED;
  if (H > (int64_t)0x7fffffff || BH > kMaxGridY) return PATH_ERR_UNSUPPORTED;
  const int64_t S = splits > 0 ? splits : decode_auto_splits(t + 1);
  if (S > (int64_t)0x7fffffff) return PATH_ERR_UNSUPPORTED;
  // the split partials must fit the fixed scratch array (checked before anything touches the device)
  if (BH > (int64_t)decode_scratch_floats() / (S * (int64_t)(d + 2))) return PATH_ERR_SCRATCH;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = nullptr;
  if (decode_scratch(st, &part) != hipSuccess) return PATH_ERR_HIP;
  return from_hip(decode_step(dtype == PATH_DTYPE_BF16, d, kcache, vcache, fcache, capacity, t, t_batch, (int)H, q_t,
                              k_t, v_t, w_t, beta_t, log_forget_t, out, lse, BH, scale, (int)S, part, st));
}

size_t path_decode_noalloc_scratch_bytes(void) { return decode_scratch_floats() * sizeof(float); }

path_status path_decode_deferred_state_bytes(int64_t B, int64_t H, int d, size_t* bytes) {
  if (bytes == nullptr || B < 0 || H < 0) return PATH_ERR_INVALID_ARG;
  if (!decode_supported(d)) return PATH_ERR_UNSUPPORTED;
  *bytes = (size_t)(B * H * (int64_t)decode_max_period() * (d + 2) * 4);
  return PATH_OK;
}

path_status path_decode_step_deferred(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                                      int64_t t_cur, int period, float* state, size_t state_bytes,
                                      const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                                      const float* beta_t, const float* log_forget_t, void* out, float* lse,
                                      int64_t B, int64_t H, int d, float scale, int dtype, int splits,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || capacity < 0 || splits < 0) return PATH_ERR_INVALID_ARG;
  if (!valid_dtype(dtype) || !decode_supported(d)) return PATH_ERR_UNSUPPORTED;
  if (t < 0 || t >= capacity || t_cur < 0 || t_cur > t) return PATH_ERR_INVALID_ARG;
  if (period < 1 || period > decode_max_period() || t - t_cur >= period) return PATH_ERR_INVALID_ARG;
  if ((log_forget_t == nullptr) != (fcache == nullptr)) return PATH_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  if (BH == 0) return PATH_OK;
  if (!kcache || !vcache || !state || !q_t || !k_t || !v_t || !w_t || !beta_t || !out || !workspace)
    return PATH_ERR_INVALID_ARG;
  if (misaligned(kcache) || misaligned(vcache) || misaligned(q_t) || misaligned(k_t) || misaligned(v_t) ||
      misaligned(w_t) || misaligned(beta_t) || misaligned(out) || misaligned(lse) || misaligned(workspace) ||
      misaligned(fcache) || misaligned(log_forget_t) || misaligned(state))
    return PATH_ERR_UNSUPPORTED;
  if (state_bytes < (size_t)(BH * (int64_t)decode_max_period() * (d + 2) * 4)) return PATH_ERR_INVALID_ARG;
  const int64_t S = splits > 0 ? splits : decode_auto_splits(t + 1);
  if (S > (int64_t)0x7fffffff) return PATH_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)(BH * S * (int64_t)(d + 2) * 4)) return PATH_ERR_INVALID_ARG;
  if (BH > kMaxGridY) return PATH_ERR_UNSUPPORTED;
  return from_hip(decode_step_deferred(dtype == PATH_DTYPE_BF16, d, kcache, vcache, fcache, capacity, t, t_cur, period,
                                       state, q_t, k_t, v_t, w_t, beta_t, log_forget_t, out, lse, BH, scale, (int)S,
                                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------------------- backward

}  // extern "C"

namespace {

// Byte offsets of the backward's buffers in its workspace (chunk already resolved).
struct bwd_plan {
  int64_t off[19];
  int64_t total;
};

path_status plan_bwd(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype, bwd_plan* p) {
  if (B < 0 || H < 0 || L < 0 || d <= 0 || chunk <= 0) return PATH_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return PATH_ERR_UNSUPPORTED;
  if (!vec_supported(d, chunk)) return PATH_ERR_UNSUPPORTED;
  const int64_t BH = B * H, M = (L + chunk - 1) / chunk, Lp = M * chunk, NPB = bwd_band_pairs(M);
  const int64_t rows = BH * Lp * 4, mat = BH * Lp * d * 4, dd = BH * M * d * d * 4, cc = BH * M * chunk * chunk * 4;
  // one band of query chunks at a time; the matrix-core kernels keep a bf16 input's pair states, ktilde
  // and P in bf16
  const int64_t state_bytes = (dtype == PATH_DTYPE_BF16 && d == 64 && chunk == 64) ? 2 : 4;
  const int64_t pairs = BH * NPB * chunk * d * state_bytes;
  const int64_t zi = state_bytes == 2 ? cc : 0;  // A^{-1} per chunk from the matrix-core forward terms
  // (for those the forward terms are the prefill's own: qtilde too in bf16, the in-chunk logits packed)
  const int64_t qt = BH * Lp * d * state_bytes, kt = qt, pm = BH * M * d * d * state_bytes;
  const int64_t sm = state_bytes == 2 ? BH * M * (int64_t)mfma_s_chunk_bytes() : cc;
  const int64_t sizes[19] = {qt, kt, pm, sm, rows, BH * M * 4,        // qt kt Pm Sm fl ftot
                             pairs, pairs, BH * NPB * 4,              // St Gst Off
                             rows, rows, rows, rows,                  // lse2 Dv drow dcol
                             mat, mat, dd, cc,                        // dqt dkt dPm dSm
                             mat, zi};                                // dva Zi
  int64_t o = 0;
  for (int i = 0; i < 19; ++i) {
    p->off[i] = o;
    o = round_up(o + sizes[i], kAlign);
  }
  p->total = o;
  return PATH_OK;
}

int bwd_chunk(int chunk) { return chunk == 0 ? 64 : chunk; }

}  // namespace

extern "C" {

path_status path_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                          size_t* bytes) {
  if (bytes == nullptr) return PATH_ERR_INVALID_ARG;
  bwd_plan p;
  const path_status s = plan_bwd(B, H, L, d, bwd_chunk(chunk), dtype, &p);
  if (s != PATH_OK) return s;
  *bytes = (size_t)p.total;
  return PATH_OK;
}

path_status path_attn_bwd(const void* q, const void* k, const void* v, const void* w, const float* beta,
                          const float* log_forget, const void* out, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* dw, float* dbeta, float* dlog_forget, int64_t B, int64_t H,
                          int64_t L, int d, int chunk, float scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  chunk = bwd_chunk(chunk);
  bwd_plan p;
  const path_status s = plan_bwd(B, H, L, d, chunk, dtype, &p);
  if (s != PATH_OK) return s;
  if ((log_forget == nullptr) != (dlog_forget == nullptr)) return PATH_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  if (BH == 0 || L == 0) return PATH_OK;
  if (!q || !k || !v || !w || !beta || !out || !lse || !dout || !dq || !dk || !dv || !dw || !dbeta || !workspace)
    return PATH_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(w) || misaligned(beta) ||
      misaligned(log_forget) || misaligned(out) || misaligned(lse) || misaligned(dout) || misaligned(dq) ||
      misaligned(dk) || misaligned(dv) || misaligned(dw) || misaligned(dbeta) || misaligned(dlog_forget) ||
      misaligned(workspace))
    return PATH_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)p.total) return PATH_ERR_INVALID_ARG;
  const int64_t M = (L + chunk - 1) / chunk;
  if (BH > kMaxGridY || M > kMaxGridY) return PATH_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  auto f = [&](int i) { return reinterpret_cast<float*>(ws + p.off[i]); };
  const bwd_buffers b{f(0),  f(1),  f(2),  f(3),  f(4),  f(5),  f(6),  f(7),  f(8), f(9),
                      f(10), f(11), f(12), f(13), f(14), f(15), f(16), f(17), f(18)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == PATH_DTYPE_BF16;
  return from_hip(bwd_run(bf16, d, chunk, q, k, v, w, beta, log_forget, out, lse, dout, dq, dk, dv, dw, dbeta,
                          dlog_forget, BH, L, scale, b, st));
}

}  // extern "C"
