// C ABI of the KDA library: argument validation (host only, before any HIP
// call) and dispatch to the kernel launchers.  See include/kda.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Gate kind and input form: unknown values are invalid.
kda_status_t check_kinds(const kda_shape_t *s) {
  if (s->gate != KDA_GATE_CHANNEL && s->gate != KDA_GATE_HEAD) return KDA_ERR_INVALID_ARGUMENT;
  if (s->input_form != KDA_INPUT_FINAL && s->input_form != KDA_INPUT_PREACT) return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

// alpha holds d_k floats per (token, head) rows of 16 bytes, or one float.
bool alpha_aligned(const kda_shape_t *s, const void *alpha) {
  return s->gate == KDA_GATE_HEAD ? aligned4(alpha) : aligned16(alpha);
}

// Shape checks shared by prefill and its workspace query.
kda_status_t check_prefill_shape(const kda_shape_t *s, bool varlen) {
  if (s == nullptr) return KDA_ERR_INVALID_ARGUMENT;
  if (s->num_seqs < 0 || s->total_tokens < 0 || s->num_heads < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (s->d_k < 1 || s->d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (s->qkv_dtype != KDA_F32 && s->qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (s->gate != KDA_GATE_CHANNEL && s->gate != KDA_GATE_HEAD) return KDA_ERR_INVALID_ARGUMENT;
  if (s->input_form != KDA_INPUT_FINAL && s->input_form != KDA_INPUT_PREACT) return KDA_ERR_INVALID_ARGUMENT;
  if (!varlen) {
    if (s->seq_len < 0) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)s->num_seqs * (int64_t)s->seq_len != s->total_tokens) return KDA_ERR_INVALID_ARGUMENT;
  }
  if (s->d_k != s->d_v || !supported_dim(s->d_k)) return KDA_ERR_UNSUPPORTED;
  if (check_kinds(s) != KDA_OK) return check_kinds(s);
  // Grid limit of the state pass: one workgroup per (sequence, head, 16 value
  // columns), sequences and heads padded to multiples of 8.  (The
  // chunk-local grid, N H W, is kept below 2^31 by the choice of W.)
  if (((int64_t)s->num_seqs * s->num_heads + 7) / 8 * 8 * (s->d_v < 16 ? 1 : s->d_v / 16) >= ((int64_t)1 << 31))
    return KDA_ERR_UNSUPPORTED;
  // The state pass addresses one chunk's rows of v and o with 32-bit offsets.
  if ((int64_t)kda::kChunk * s->num_heads * s->d_v * 4 >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
  // Workspace byte counts (records, checkpoints, partial rows: at most a few
  // KiB per token, head and 16 value columns) are 64-bit: (tokens + 64 N)
  // H d_v/16 stays below 2^40.  (Written with divisions, so that the check
  // itself cannot overflow.)
  const int64_t groups = (int64_t)s->num_heads * (s->d_v < 16 ? 1 : s->d_v / 16);
  const int64_t limit = ((int64_t)1 << 40) / groups;
  if (s->total_tokens >= limit || (int64_t)s->num_seqs * kda::kChunk >= limit - s->total_tokens)
    return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(kda_status_t status) {
  // A C caller may pass any int.  Reading a value outside the enumerators as
  // kda_status_t is undefined in C++, so the argument is read as an int.
  int code;
  static_assert(sizeof(code) == sizeof(status), "kda_status_t is int-sized");
  std::memcpy(&code, &status, sizeof code);
  switch (code) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
  }
  return "KDA_ERR_UNKNOWN";
}

kda_status_t kda_prefill_workspace_size(const kda_shape_t *shape, size_t *bytes) {
  if (bytes == nullptr || shape == nullptr) return KDA_ERR_INVALID_ARGUMENT;
  // The size does not depend on seq_len, so validate as a varlen shape.
  kda_status_t st = check_prefill_shape(shape, /*varlen=*/true);
  if (st != KDA_OK) return st;
  *bytes = kda::prefill_workspace_bytes(*shape);
  return KDA_OK;
}

}  // extern "C"

namespace {

// Validation shared by kda_prefill and its two phases.  `need_*` say which
// pointers the call reads or writes; `one_stripe` asks for a workspace that
// holds every chunk of the batch at once (the phase entry points, which need
// the recommended size).
// On success *plan is the stripe plan for the workspace.
kda_status_t check_prefill_call(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, const int32_t *cu_seqlens,
                                const float *S0, const float *o, const float *S_T,
                                const void *workspace, size_t workspace_bytes, bool need_v,
                                bool need_beta, bool need_o, bool one_stripe, kda::PrefillPlan *plan) {
  const bool varlen = cu_seqlens != nullptr;
  kda_status_t st = check_prefill_shape(shape, varlen);
  if (st != KDA_OK) return st;
  const bool has_tokens = shape->total_tokens > 0;
  if (has_tokens) {
    if (!q || !k || !alpha || (need_v && !v) || (need_beta && !beta) || (need_o && !o))
      return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !alpha_aligned(shape, alpha) || (need_v && !aligned16(v)) ||
        (need_beta && !aligned4(beta)) || (need_o && !aligned16(o)))
      return KDA_ERR_INVALID_ARGUMENT;
  }
  // cu_seqlens is read one int32 at a time: 4-byte alignment, as for kda_backward.
  if ((S0 && !aligned16(S0)) || (S_T && !aligned16(S_T)) || (cu_seqlens && !aligned4(cu_seqlens)))
    return KDA_ERR_INVALID_ARGUMENT;
  if (shape->num_seqs == 0) return has_tokens ? KDA_ERR_INVALID_ARGUMENT : KDA_OK;
  if (workspace == nullptr) return KDA_ERR_WORKSPACE_TOO_SMALL;
  *plan = kda::prefill_plan(*shape, varlen, S_T != nullptr, workspace_bytes);
  if (plan->W <= 0 || (one_stripe && plan->stripes != 1)) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kda::kWorkspaceAlign - 1)) != 0)
    return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

kda_status_t run_prefill(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, const int32_t *cu_seqlens,
                         const float *S0, float *o, float *S_T, void *workspace,
                         size_t workspace_bytes, void *stream, int phases) {
  const bool state = (phases & kda::kPhaseState) != 0;
  const bool local = (phases & kda::kPhaseLocal) != 0;
  kda::PrefillPlan plan{};
  kda_status_t st = check_prefill_call(shape, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace,
                                       workspace_bytes, state, local, state, !(state && local), &plan);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  hipError_t e = kda::launch_prefill(*shape, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, plan,
                                     static_cast<hipStream_t>(stream), phases);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status_t kda_prefill(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, const int32_t *cu_seqlens,
                         const float *S0, float *o, float *S_T, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return run_prefill(shape, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, workspace_bytes,
                     stream, kda::kPhaseLocal | kda::kPhaseState);
}

kda_status_t kda_prefill_chunk_local(const kda_shape_t *shape, const void *q, const void *k,
                                     const float *alpha, const float *beta,
                                     const int32_t *cu_seqlens, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  return run_prefill(shape, q, k, nullptr, alpha, beta, cu_seqlens, nullptr, nullptr, nullptr,
                     workspace, workspace_bytes, stream, kda::kPhaseLocal);
}

kda_status_t kda_prefill_state_pass(const kda_shape_t *shape, const void *q, const void *k,
                                    const void *v, const float *alpha, const int32_t *cu_seqlens,
                                    const float *S0, float *o, float *S_T, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return run_prefill(shape, q, k, v, alpha, nullptr, cu_seqlens, S0, o, S_T, workspace, workspace_bytes,
                     stream, kda::kPhaseState);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kda_prefill_noalloc: kda_prefill with its workspace in a file-scope device
// array, for callers that cannot allocate device memory.  Each GPU the
// library runs on holds its own copy of the array (KDA_NOALLOC_WORKSPACE_BYTES)
// until the process ends.  In host code `scratch` only names the symbol; its
// device address on the current GPU comes from hipGetSymbolAddress, looked
// up once per device and cached.
// ---------------------------------------------------------------------------
__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device; null = not looked up

hipError_t scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & (kda::kWorkspaceAlign - 1)) != 0)
      return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

kda_status_t kda_prefill_noalloc(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta, const int32_t *cu_seqlens,
                                 const float *S0, float *o, float *S_T, void *stream) {
  // Every argument check before the first HIP call (the workspace stands in
  // with a placeholder of the scratch's size and alignment); a shape whose
  // one chunk per (sequence, head) does not fit is rejected.
  kda::PrefillPlan plan{};
  kda_status_t st = check_prefill_call(shape, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T,
                                       reinterpret_cast<const void *>(kda::kWorkspaceAlign),
                                       (size_t)KDA_NOALLOC_WORKSPACE_BYTES, true, true, true, false, &plan);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  // The static workspace is the current device's: a stream of another
  // device would run the kernels there with this device's address.
  if (stream != nullptr) {
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KDA_ERR_LAUNCH;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != cur)
      return KDA_ERR_INVALID_ARGUMENT;
  }
  void *ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
  hipError_t e = kda::launch_prefill(*shape, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, ws, plan,
                                     static_cast<hipStream_t>(stream), kda::kPhaseLocal | kda::kPhaseState);
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Shared by the decode entry points: a dense batch of num_seqs sequences of
// seq_len tokens (seq_len == 1 for kda_decode_step).
kda_status_t check_decode_call(const kda_shape_t *shape, bool one_token, const void *q, const void *k,
                               const void *v, const float *alpha, const float *beta, const float *S,
                               const float *o) {
  if (shape == nullptr) return KDA_ERR_INVALID_ARGUMENT;
  const kda_shape_t &s = *shape;
  if (s.num_seqs < 0 || s.num_heads < 1 || s.seq_len < 1 || (one_token && s.seq_len != 1) ||
      s.total_tokens != (int64_t)s.num_seqs * s.seq_len)
    return KDA_ERR_INVALID_ARGUMENT;
  if (s.qkv_dtype != KDA_F32 && s.qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARGUMENT;
  if (s.d_k < 1 || s.d_v < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (s.gate != KDA_GATE_CHANNEL && s.gate != KDA_GATE_HEAD) return KDA_ERR_INVALID_ARGUMENT;
  if (s.input_form != KDA_INPUT_FINAL && s.input_form != KDA_INPUT_PREACT) return KDA_ERR_INVALID_ARGUMENT;
  if (s.d_k != s.d_v || !supported_dim(s.d_k)) return KDA_ERR_UNSUPPORTED;
  if (s.num_seqs == 0) return KDA_OK;
  if (!q || !k || !v || !alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !alpha_aligned(shape, alpha) || !aligned4(beta) ||
      !aligned16(S) || !aligned16(o))
    return KDA_ERR_INVALID_ARGUMENT;
  // One workgroup per (sequence, head).
  if ((int64_t)s.num_seqs * s.num_heads >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_decode_tokens(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, float *S, float *o, float *S_hist,
                               void *stream) {
  kda_status_t st = check_decode_call(shape, false, q, k, v, alpha, beta, S, o);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  if (S_hist != nullptr && !aligned16(S_hist)) return KDA_ERR_INVALID_ARGUMENT;
  hipError_t e = kda::launch_decode_tokens(*shape, q, k, v, alpha, beta, S, o, S_hist,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_state_commit(const kda_shape_t *shape, float *S, const float *S_hist,
                              const int32_t *accepted, void *stream) {
  if (shape == nullptr) return KDA_ERR_INVALID_ARGUMENT;
  const kda_shape_t &s = *shape;
  if (s.num_seqs < 0 || s.num_heads < 1 || s.seq_len < 1 || s.d_k < 1 || s.d_v < 1)
    return KDA_ERR_INVALID_ARGUMENT;
  if (s.d_k != s.d_v || !supported_dim(s.d_k)) return KDA_ERR_UNSUPPORTED;
  if (s.num_seqs == 0) return KDA_OK;
  if (!S || !S_hist || !accepted || !aligned16(S) || !aligned16(S_hist) || !aligned4(accepted))
    return KDA_ERR_INVALID_ARGUMENT;
  if ((int64_t)s.num_seqs * s.num_heads >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
  hipError_t e = kda::launch_commit(s, S, S_hist, accepted, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_verify_tokens(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, const float *S, float *o, void *stream) {
  kda_status_t st = check_decode_call(shape, false, q, k, v, alpha, beta, S, o);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  hipError_t e = kda::launch_verify_tokens(*shape, q, k, v, alpha, beta, S, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_accept_tokens(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, float *S, const int32_t *accepted,
                               void *stream) {
  // (no outputs: S stands in for o in the shared checks)
  kda_status_t st = check_decode_call(shape, false, q, k, v, alpha, beta, S, S);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  if (accepted == nullptr || !aligned4(accepted)) return KDA_ERR_INVALID_ARGUMENT;
  hipError_t e = kda::launch_accept_tokens(*shape, q, k, v, alpha, beta, S, accepted,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_accept_verify_tokens(const kda_shape_t *shape, const void *q0, const void *k0, const void *v0,
                                      const float *alpha0, const float *beta0, const int32_t *accepted,
                                      const void *q, const void *k, const void *v, const float *alpha,
                                      const float *beta, float *S, float *o, void *stream) {
  kda_status_t st = check_decode_call(shape, false, q, k, v, alpha, beta, S, o);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  // the previous round's tokens: the same shape, so the same checks
  st = check_decode_call(shape, false, q0, k0, v0, alpha0, beta0, S, o);
  if (st != KDA_OK) return st;
  if (accepted == nullptr || !aligned4(accepted)) return KDA_ERR_INVALID_ARGUMENT;
  hipError_t e = kda::launch_accept_verify_tokens(*shape, q0, k0, v0, alpha0, beta0, accepted, q, k, v, alpha,
                                                  beta, S, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_decode_step(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, float *S, float *o,
                             void *stream) {
  kda_status_t st = check_decode_call(shape, true, q, k, v, alpha, beta, S, o);
  if (st != KDA_OK || shape->num_seqs == 0) return st;
  const kda_shape_t &s = *shape;
  hipError_t e = kda::launch_decode(s, q, k, v, alpha, beta, S, o, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_backward_workspace_size(const kda_shape_t *shape, size_t *bytes) {
  if (bytes == nullptr || shape == nullptr) return KDA_ERR_INVALID_ARGUMENT;
  kda_status_t st = check_prefill_shape(shape, /*varlen=*/true);
  if (st != KDA_OK) return st;
  if (shape->input_form != KDA_INPUT_FINAL) return KDA_ERR_UNSUPPORTED;
  *bytes = kda::backward_layout(*shape).bytes;
  return KDA_OK;
}

kda_status_t kda_backward(const kda_shape_t *shape, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          const float *S0, const float *dO, const float *dS_T, float *dq, float *dk,
                          float *dv, float *dalpha, float *dbeta, float *dS0, void *workspace,
                          size_t workspace_bytes, void *stream) {
  const bool varlen = cu_seqlens != nullptr;
  kda_status_t st = check_prefill_shape(shape, varlen);
  if (st != KDA_OK) return st;
  if (shape->input_form != KDA_INPUT_FINAL) return KDA_ERR_UNSUPPORTED;
  const kda_shape_t &s = *shape;
  if (s.total_tokens > 0) {
    if (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk || !dv || !dalpha || !dbeta)
      return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !alpha_aligned(shape, alpha) ||
        !aligned4(beta) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        !alpha_aligned(shape, dalpha) || !aligned4(dbeta))
      return KDA_ERR_INVALID_ARGUMENT;
  }
  if ((S0 && !aligned16(S0)) || (dS_T && !aligned16(dS_T)) || (dS0 && !aligned16(dS0)) ||
      (cu_seqlens && !aligned4(cu_seqlens)))
    return KDA_ERR_INVALID_ARGUMENT;
  if (s.num_seqs == 0) return s.total_tokens > 0 ? KDA_ERR_INVALID_ARGUMENT : KDA_OK;
  // One workgroup per (sequence, head, 16 value columns), the pairs rounded
  // up to a multiple of 8.
  if (((int64_t)s.num_seqs * s.num_heads + 7) / 8 * 8 * (s.d_v < 16 ? 1 : s.d_v / 16) >= ((int64_t)1 << 31))
    return KDA_ERR_UNSUPPORTED;
  if (workspace == nullptr) return KDA_ERR_WORKSPACE_TOO_SMALL;
  const kda::BwdLayout L = kda::backward_plan(s, varlen, workspace_bytes);
  if (L.pieces <= 0) return KDA_ERR_WORKSPACE_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kda::kWorkspaceAlign - 1)) != 0)
    return KDA_ERR_INVALID_ARGUMENT;
  kda::BwdArgs a{q, k, v, alpha, beta, cu_seqlens, S0, dO, dS_T, dq, dk, dv, dalpha, dbeta, dS0, workspace};
  hipError_t e = kda::launch_backward(s, a, L, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"
