// Single-token decode step of the KDA layer (and of its scalar-gate form,
// where every alpha_i of a head is the same one rate).
//
// For one (sequence, head) and one new token (q, k, v, alpha, beta) the
// update rule S' = (I - beta k k^T) Diag(alpha) S + beta k v^T (dimsnsums.com
// "GLM-5.3-FLASH" attention page, section "How can a layer remember without
// rereading?", update rule) is evaluated column by column of S, in one pass
// over the state:
//
//   x_j = sum_i alpha_i k_i S_ij          (k^T Diag(alpha) S)
//   y_j = sum_i alpha_i q_i S_ij          (q^T Diag(alpha) S)
//   w_j = beta (v_j - x_j)
//   S'_ij = alpha_i S_ij + k_i w_j        (written back in place)
//   o_j = y_j + (q.k) w_j                 (= sum_i q_i S'_ij, post-update read-out)
//
// A workgroup owns one head (up to 512 threads): it reads the d x d fp32 state
// once into registers (float4 per lane, each row read by d/4 consecutive
// lanes), reduces x and y over rows with cross-lane shuffles and one LDS
// round, and writes the state back.  Every lane loads alpha_i, k_i, q_i of
// its own rows, and the v_j, beta it needs, before the state, so no load
// waits on another after the state arrives; q.k is summed from the rows in
// registers.  The kernel is bound by HBM:
// 2 x 64 KiB of state traffic per head and step against ~115 kflop.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int D>
struct DecodeCfg {
  static constexpr int TPR = D / 4;                                // lanes per row (float4 each)
  static constexpr int NT = TPR * D < 512 ? TPR * D : 512;         // threads per workgroup
  static constexpr int RPP = NT / TPR;                             // rows per pass
  static constexpr int PASSES = D / RPP;
  static constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0, "workgroup must be whole waves");
  static_assert(D % RPP == 0, "rows must tile evenly");
  static_assert(NT >= D, "one lane per value column in the final step");
};

// Pre-activation inputs (KDA_INPUT_PREACT): alpha = exp(-softplus(a)) =
// 1 / (1 + e^a), beta = sigmoid(b), and q, k scaled by 1 / max(||.||_2, 1e-12).
__device__ __forceinline__ float decay_from_preact(float a) { return 1.f / (1.f + expf(a)); }
__device__ __forceinline__ float strength_from_preact(float b) { return 1.f / (1.f + expf(-b)); }
__device__ __forceinline__ float inv_norm(float ss) { return 1.f / fmaxf(sqrtf(ss), 1e-12f); }

template <int D, typename TIn, int GATE, int FORM>
__global__ __launch_bounds__(DecodeCfg<D>::NT) void decode_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, float *__restrict__ S,
    float *__restrict__ o) {
  using Cfg = DecodeCfg<D>;
  constexpr int TPR = Cfg::TPR, RPP = Cfg::RPP, PASSES = Cfg::PASSES, NW = Cfg::NW;

  __shared__ float s_red[NW][2][D];
  __shared__ float s_qk[NW][3];  // q.k, then ||k||^2, ||q||^2 (pre-activation inputs)
  __shared__ float s_w[D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nh = (int64_t)blockIdx.x;  // flattened (sequence, head)
  const int cq = tid % TPR;                // float4 column
  const int r0 = tid / TPR;                // first row of this lane
  float *Sp = S + nh * (int64_t)(D * D) + cq * 4;

  // Small inputs first (alpha, k, q of this lane's rows; v, beta of the
  // column it finalises; q_i k_i of channel tid), then the state.
  float a[PASSES], kk[PASSES], qq[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = r0 + p * RPP;
    a[p] = GATE == KDA_GATE_HEAD ? alpha[nh] : alpha[nh * D + r];
    kk[p] = to_f32(k[nh * D + r]);
    qq[p] = to_f32(q[nh * D + r]);
  }
  const int cj = tid < D ? tid : 0;
  const float vj = to_f32(v[nh * D + cj]);
  float bt = beta[nh];
  float4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) s[p] = *reinterpret_cast<const float4 *>(Sp + (int64_t)(r0 + p * RPP) * D);
  // Every load is in flight before the first instruction that waits on one
  // (otherwise the scheduler may move the q.k shuffles, which wait for q and
  // k, above the state loads and serialise two memory round trips).
  __builtin_amdgcn_sched_barrier(0);

  constexpr bool kPre = FORM == KDA_INPUT_PREACT;
  if constexpr (kPre) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) a[p] = decay_from_preact(a[p]);
    bt = strength_from_preact(bt);
  }
  // q.k (and the squared norms of raw q and k) from the rows already in
  // registers: the lanes of column group 0 hold every row exactly once.  The
  // unit-length scaling is applied to the reduced sums (x and y are linear
  // in k and q).
  float qk_part = 0.f, kn_part = 0.f, qn_part = 0.f;
  if (cq == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      qk_part += qq[p] * kk[p];
      if constexpr (kPre) {
        kn_part += kk[p] * kk[p];
        qn_part += qq[p] * qq[p];
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    qk_part += __shfl_xor(qk_part, off);
    if constexpr (kPre) {
      kn_part += __shfl_xor(kn_part, off);
      qn_part += __shfl_xor(qn_part, off);
    }
  }
  float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float ka = a[p] * kk[p], qa = a[p] * qq[p];
    x[0] += ka * s[p].x; x[1] += ka * s[p].y; x[2] += ka * s[p].z; x[3] += ka * s[p].w;
    y[0] += qa * s[p].x; y[1] += qa * s[p].y; y[2] += qa * s[p].z; y[3] += qa * s[p].w;
  }
  // Lanes of one wave that share a column group differ in the bits >= TPR.
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] += __shfl_xor(x[j], off);
      y[j] += __shfl_xor(y[j], off);
    }
  }
  if (lane < TPR) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s_red[wave][0][cq * 4 + j] = x[j];
      s_red[wave][1][cq * 4 + j] = y[j];
    }
  }
  if (lane == 0) {
    s_qk[wave][0] = qk_part;
    s_qk[wave][1] = kn_part;
    s_qk[wave][2] = qn_part;
  }
  __syncthreads();

  if (tid < D) {
    float xs = 0.f, ys = 0.f, qk = 0.f, kn = 0.f, qn = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      xs += s_red[w][0][tid];
      ys += s_red[w][1][tid];
      qk += s_qk[w][0];
      if constexpr (kPre) {
        kn += s_qk[w][1];
        qn += s_qk[w][2];
      }
    }
    float ik = 1.f, iq = 1.f;
    if constexpr (kPre) {
      ik = inv_norm(kn);
      iq = inv_norm(qn);
      xs *= ik;
      ys *= iq;
      qk *= ik * iq;
    }
    const float wv = bt * (vj - xs);
    s_w[tid] = kPre ? wv * ik : wv;  // the update adds k_i w_j with unit k
    o[nh * D + tid] = ys + qk * wv;
  }
  __syncthreads();

  const float w0 = s_w[cq * 4 + 0], w1 = s_w[cq * 4 + 1], w2 = s_w[cq * 4 + 2], w3 = s_w[cq * 4 + 3];
  // The new state goes out with non-temporal stores: it is read again only
  // at the next step, after the whole batch has streamed through, so keeping
  // it in the caches only displaces lines still being read.
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = r0 + p * RPP;
    f32x4 n;
    n[0] = a[p] * s[p].x + kk[p] * w0;
    n[1] = a[p] * s[p].y + kk[p] * w1;
    n[2] = a[p] * s[p].z + kk[p] * w2;
    n[3] = a[p] * s[p].w + kk[p] * w3;
    __builtin_nontemporal_store(n, reinterpret_cast<f32x4 *>(Sp + (int64_t)r * D));
  }
}

template <int D, typename TIn, int GATE, int FORM>
hipError_t launch_decode_t(const kda_shape_t &s, const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, float *S, float *o,
                           hipStream_t stream) {
  using Cfg = DecodeCfg<D>;
  const int64_t blocks = (int64_t)s.num_seqs * s.num_heads;
  hipLaunchKernelGGL((decode_kernel<D, TIn, GATE, FORM>), dim3((unsigned)blocks), dim3(Cfg::NT), 0, stream,
                     static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                     static_cast<const TIn *>(v), alpha, beta, S, o);
  return hipGetLastError();
}

template <typename TIn, int GATE, int FORM>
hipError_t dispatch_d(const kda_shape_t &s, const void *q, const void *k, const void *v,
                      const float *alpha, const float *beta, float *S, float *o, hipStream_t st) {
  switch (s.d_k) {
    case 16: return launch_decode_t<16, TIn, GATE, FORM>(s, q, k, v, alpha, beta, S, o, st);
    case 32: return launch_decode_t<32, TIn, GATE, FORM>(s, q, k, v, alpha, beta, S, o, st);
    case 64: return launch_decode_t<64, TIn, GATE, FORM>(s, q, k, v, alpha, beta, S, o, st);
    case 128: return launch_decode_t<128, TIn, GATE, FORM>(s, q, k, v, alpha, beta, S, o, st);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, int FORM>
hipError_t dispatch_gate(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *S, float *o, hipStream_t st) {
  if (s.gate == KDA_GATE_HEAD) return dispatch_d<TIn, KDA_GATE_HEAD, FORM>(s, q, k, v, alpha, beta, S, o, st);
  return dispatch_d<TIn, KDA_GATE_CHANNEL, FORM>(s, q, k, v, alpha, beta, S, o, st);
}

template <typename TIn>
hipError_t dispatch_form(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *S, float *o, hipStream_t st) {
  if (s.input_form == KDA_INPUT_PREACT)
    return dispatch_gate<TIn, KDA_INPUT_PREACT>(s, q, k, v, alpha, beta, S, o, st);
  return dispatch_gate<TIn, KDA_INPUT_FINAL>(s, q, k, v, alpha, beta, S, o, st);
}

}  // namespace

hipError_t launch_decode(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *S, float *o,
                         hipStream_t stream) {
  if (s.qkv_dtype == KDA_BF16) return dispatch_form<__bf16>(s, q, k, v, alpha, beta, S, o, stream);
  return dispatch_form<float>(s, q, k, v, alpha, beta, S, o, stream);
}

}  // namespace kda
