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

#include <type_traits>

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

// Threshold for reading the state with non-temporal loads as well (several
// times the 256 MB Infinity Cache).  The single-token step applies it to the
// state's size: non-temporal stores alone are best at 512 MiB of state (75%
// vs 73.5% of HBM peak with both), both at 2 GiB (72% vs 65%).  The
// multi-token kernel applies it to the bytes it moves (the state read plus
// every state written), which pass it at two tokens with history at B = 256.
constexpr int64_t kStreamStateBytes = (int64_t)1 << 30;

template <int D, typename TIn, int GATE, int FORM, bool NTL>
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
  for (int p = 0; p < PASSES; ++p) {
    const float *src = Sp + (int64_t)(r0 + p * RPP) * D;
    if constexpr (NTL) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
      s[p] = make_float4(x[0], x[1], x[2], x[3]);
    } else {
      s[p] = *reinterpret_cast<const float4 *>(src);
    }
  }
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

// ---------------------------------------------------------------------------
// Several tokens per sequence from the live state (speculative verification
// of drafted tokens, or plain multi-token decode).  One workgroup per
// (sequence, head) as above; the state stays in registers across the
// sequence's tokens, each token's small inputs are loaded while the previous
// token computes.  With a history buffer (HIST) the state after every token is
// written there and S is left as it was (the caller rolls back or commits);
// without one S is advanced in place by all the tokens.
// ---------------------------------------------------------------------------
template <int D, typename TIn>
struct TokenIn {
  using Cfg = DecodeCfg<D>;
  float a[Cfg::PASSES];
  TIn k[Cfg::PASSES], q[Cfg::PASSES];
  TIn v;
  float b;
};

template <int D, typename TIn, int GATE>
__device__ __forceinline__ void load_token_in(TokenIn<D, TIn> &x, const TIn *__restrict__ q,
                                              const TIn *__restrict__ k, const TIn *__restrict__ v,
                                              const float *__restrict__ alpha,
                                              const float *__restrict__ beta, int64_t th, int r0,
                                              int cj) {
  using Cfg = DecodeCfg<D>;
#pragma unroll
  for (int p = 0; p < Cfg::PASSES; ++p) {
    const int r = r0 + p * Cfg::RPP;
    x.a[p] = GATE == KDA_GATE_HEAD ? alpha[th] : alpha[th * D + r];
    x.k[p] = k[th * D + r];
    x.q[p] = q[th * D + r];
  }
  x.v = v[th * D + cj];
  x.b = beta[th];
}

// What a multi-token call does with the state and the outputs.
enum TokMode : int {
  kTokAdvance = 0,  // o for every token; S advanced in place by all of them
  kTokHistory = 1,  // o for every token; the state after each token to hist; S unchanged
  kTokVerify = 2,   // o for every token; S unchanged, nothing else written
  kTokAccept = 3,   // no o; S advanced in place by the first accepted[n] tokens
  kTokAcceptVerify = 4,  // S advanced by the first accepted[n] tokens of the previous round
                         // (prev), then o for every token of this one; S holds the former
};

// One multi-token call: token rows n*ntok .. n*ntok + ntok - 1 of a source
// belong to sequence n.
template <typename TIn>
struct TokSrc {
  const TIn *q, *k, *v;
  const float *alpha, *beta;
};

template <int D, typename TIn, int GATE, int FORM, int MODE, bool NTL>
__global__ __launch_bounds__(DecodeCfg<D>::NT) void decode_tokens_kernel(
    const TokSrc<TIn> in, const TokSrc<TIn> prev, float *__restrict__ S, float *__restrict__ o,
    float *__restrict__ hist, const int32_t *__restrict__ accepted, int ntok, int H) {
  constexpr bool HIST = MODE == kTokHistory;
  using Cfg = DecodeCfg<D>;
  constexpr int TPR = Cfg::TPR, RPP = Cfg::RPP, PASSES = Cfg::PASSES, NW = Cfg::NW;
  constexpr bool kPre = FORM == KDA_INPUT_PREACT;

  __shared__ float s_red[NW][2][D];
  __shared__ float s_qk[NW][3];
  __shared__ float s_w[D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nh = (int64_t)blockIdx.x;  // n * H + h
  const int64_t n = nh / H, h = nh % H;
  const int cq = tid % TPR;
  const int r0 = tid / TPR;
  const int cj = tid < D ? tid : 0;
  // accepted tokens to run first (accept modes): the sequence's count,
  // clamped to [0, ntok]; with none the state is not written
  int na = 0;
  if constexpr (MODE == kTokAccept || MODE == kTokAcceptVerify) {
    const int j = accepted[n];
    na = j < 0 ? 0 : (j > ntok ? ntok : j);
    if constexpr (MODE == kTokAccept) {
      if (na == 0) return;
    }
  }
  // the source of the first tokens run: the accepted ones, or the call's
  const TokSrc<TIn> first = (MODE == kTokAccept || (MODE == kTokAcceptVerify && na > 0)) ? prev : in;

  // The first token's inputs are loaded before the state, so no load waits
  // on another after the state arrives.
  TokenIn<D, TIn> cur, nxt;
  load_token_in<D, TIn, GATE>(cur, first.q, first.k, first.v, first.alpha, first.beta, n * ntok * H + h, r0, cj);
  float *Sp = S + nh * (int64_t)(D * D) + cq * 4;
  float4 s[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const float *src = Sp + (int64_t)(r0 + p * RPP) * D;
    if constexpr (NTL) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
      s[p] = make_float4(x[0], x[1], x[2], x[3]);
    } else {
      s[p] = *reinterpret_cast<const float4 *>(src);
    }
  }
  auto store_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const f32x4 nv = {s[p].x, s[p].y, s[p].z, s[p].w};
      __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(Sp + (int64_t)(r0 + p * RPP) * D));
    }
  };

  // count tokens of src from the state in registers, cur holding the first
  // one's inputs; WO: write their outputs
  auto run = [&](const TokSrc<TIn> &src, int count, auto wo) __attribute__((always_inline)) {
    constexpr bool WO = decltype(wo)::value;
    for (int t = 0; t < count; ++t) {
      const int64_t th = (n * ntok + t) * H + h;  // token row * H + head
      // The next token's inputs (the last token reloads its own: no branch).
      const int tn = t + 1 < count ? t + 1 : t;
      load_token_in<D, TIn, GATE>(nxt, src.q, src.k, src.v, src.alpha, src.beta, (n * ntok + tn) * H + h, r0, cj);

      float a[PASSES], kk[PASSES], qq[PASSES];
  #pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        a[p] = kPre ? decay_from_preact(cur.a[p]) : cur.a[p];
        kk[p] = to_f32(cur.k[p]);
        qq[p] = to_f32(cur.q[p]);
      }
      const float bt = kPre ? strength_from_preact(cur.b) : cur.b;
      const float vj = to_f32(cur.v);

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
        s_w[tid] = kPre ? wv * ik : wv;
        if constexpr (WO) o[th * D + tid] = ys + qk * wv;
      }
      __syncthreads();
      const float w0 = s_w[cq * 4 + 0], w1 = s_w[cq * 4 + 1], w2 = s_w[cq * 4 + 2], w3 = s_w[cq * 4 + 3];
  #pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        s[p].x = a[p] * s[p].x + kk[p] * w0;
        s[p].y = a[p] * s[p].y + kk[p] * w1;
        s[p].z = a[p] * s[p].z + kk[p] * w2;
        s[p].w = a[p] * s[p].w + kk[p] * w3;
      }
      if constexpr (HIST) {
        float *Hp = hist + th * (int64_t)(D * D) + cq * 4;
  #pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          const f32x4 nv = {s[p].x, s[p].y, s[p].z, s[p].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(Hp + (int64_t)(r0 + p * RPP) * D));
        }
      }
      cur = nxt;
    }
  };

  if constexpr (MODE == kTokAccept) {
    run(prev, na, std::false_type{});
    store_state();
  } else if constexpr (MODE == kTokAcceptVerify) {
    if (na > 0) {
      run(prev, na, std::false_type{});
      store_state();
      load_token_in<D, TIn, GATE>(cur, in.q, in.k, in.v, in.alpha, in.beta, n * ntok * H + h, r0, cj);
    }
    run(in, ntok, std::true_type{});
  } else {
    run(in, ntok, std::true_type{});
    if constexpr (MODE == kTokAdvance) store_state();
  }
}

// Rollback / commit: S[n, h] <- hist[n, j - 1, h] with j = accepted[n]
// capped at ntok; j <= 0 leaves S[n, h] as it is.  One workgroup per
// (sequence, head), float4 copies.
template <int D>
__global__ __launch_bounds__(256) void commit_kernel(float *__restrict__ S, const float *__restrict__ hist,
                                                     const int32_t *__restrict__ accepted, int ntok, int H) {
  constexpr int N4 = D * D / 4;                      // 16-byte pieces of one state
  constexpr int U = N4 >= 256 ? N4 / 256 : 1;        // pieces per lane
  const int64_t nh = (int64_t)blockIdx.x;
  const int64_t n = nh / H, h = nh % H;
  int j = accepted[n];
  if (j <= 0) return;
  if (j > ntok) j = ntok;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(hist + ((n * ntok + (j - 1)) * H + h) * (int64_t)(D * D));
  f32x4 *dst = reinterpret_cast<f32x4 *>(S + nh * (int64_t)(D * D));
  // All of a lane's loads in flight before the stores (the trip counts are
  // compile-time, so no guard or loop sits between them to force a wait).
  // The history is read once, with non-temporal loads (132 -> 124 us at
  // B=256, two tokens); non-temporal stores of S measured slower (150 us).
  const int t = (int)threadIdx.x;
  if (N4 < 256 && t >= N4) return;
  f32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + u * 256 + t);
#pragma unroll
  for (int u = 0; u < U; ++u) dst[u * 256 + t] = x[u];
}

// Template dispatch on head size, q/k/v dtype, gate kind and input form: f
// is called with (Int<D>, TypeTag<TIn>, Int<GATE>, Int<FORM>).
template <typename T>
struct TypeTag {
  using type = T;
};
template <int V>
using Int = std::integral_constant<int, V>;

template <typename TIn, int GATE, int FORM, typename F>
hipError_t by_dim(const kda_shape_t &s, F &f) {
  switch (s.d_k) {
    case 16: return f(Int<16>{}, TypeTag<TIn>{}, Int<GATE>{}, Int<FORM>{});
    case 32: return f(Int<32>{}, TypeTag<TIn>{}, Int<GATE>{}, Int<FORM>{});
    case 64: return f(Int<64>{}, TypeTag<TIn>{}, Int<GATE>{}, Int<FORM>{});
    case 128: return f(Int<128>{}, TypeTag<TIn>{}, Int<GATE>{}, Int<FORM>{});
  }
  return hipErrorInvalidValue;
}

template <typename TIn, int FORM, typename F>
hipError_t by_gate(const kda_shape_t &s, F &f) {
  if (s.gate == KDA_GATE_HEAD) return by_dim<TIn, KDA_GATE_HEAD, FORM>(s, f);
  return by_dim<TIn, KDA_GATE_CHANNEL, FORM>(s, f);
}

template <typename TIn, typename F>
hipError_t by_form(const kda_shape_t &s, F &f) {
  if (s.input_form == KDA_INPUT_PREACT) return by_gate<TIn, KDA_INPUT_PREACT>(s, f);
  return by_gate<TIn, KDA_INPUT_FINAL>(s, f);
}

template <typename F>
hipError_t dispatch(const kda_shape_t &s, F &&f) {
  if (s.qkv_dtype == KDA_BF16) return by_form<__bf16>(s, f);
  return by_form<float>(s, f);
}

}  // namespace

hipError_t launch_decode(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *S, float *o,
                         hipStream_t stream) {
  return dispatch(s, [&](auto d, auto t, auto g, auto f) {
    constexpr int D = decltype(d)::value;
    using TIn = typename decltype(t)::type;
    constexpr int G = decltype(g)::value, F = decltype(f)::value;
    const int64_t blocks = (int64_t)s.num_seqs * s.num_heads;
    const bool stream_state = blocks * (int64_t)(D * D) * (int64_t)sizeof(float) > kStreamStateBytes;
    const TIn *qp = static_cast<const TIn *>(q), *kp = static_cast<const TIn *>(k),
              *vp = static_cast<const TIn *>(v);
    if (stream_state)
      hipLaunchKernelGGL((decode_kernel<D, TIn, G, F, true>), dim3((unsigned)blocks), dim3(DecodeCfg<D>::NT), 0,
                         stream, qp, kp, vp, alpha, beta, S, o);
    else
      hipLaunchKernelGGL((decode_kernel<D, TIn, G, F, false>), dim3((unsigned)blocks), dim3(DecodeCfg<D>::NT), 0,
                         stream, qp, kp, vp, alpha, beta, S, o);
    return hipGetLastError();
  });
}

namespace {

// Token sources: the call's tokens (q, k, v, alpha, beta), and the previous
// round's for kTokAcceptVerify (q0 .. beta0; the accept mode runs the call's).
struct TokPtrs {
  const void *q, *k, *v;
  const float *alpha, *beta;
};

hipError_t launch_tokens(const kda_shape_t &s, const TokPtrs &cur, const TokPtrs &prev, float *S, float *o,
                         float *hist, const int32_t *accepted, int mode, hipStream_t stream) {
  return dispatch(s, [&](auto d, auto t, auto g, auto f) {
    constexpr int D = decltype(d)::value;
    using TIn = typename decltype(t)::type;
    constexpr int G = decltype(g)::value, F = decltype(f)::value;
    const int64_t blocks = (int64_t)s.num_seqs * s.num_heads;
    const TokSrc<TIn> in{static_cast<const TIn *>(cur.q), static_cast<const TIn *>(cur.k),
                         static_cast<const TIn *>(cur.v), cur.alpha, cur.beta};
    const TokSrc<TIn> pv{static_cast<const TIn *>(prev.q), static_cast<const TIn *>(prev.k),
                         static_cast<const TIn *>(prev.v), prev.alpha, prev.beta};
    // The state is read once; once the bytes the call moves (that read plus
    // every state written) pass 1 GiB it is read with non-temporal loads too
    // (two tokens with history at B=256, 1.5 GiB: 336 -> 299 us per call).
    const int64_t state_bytes = blocks * (int64_t)(D * D) * (int64_t)sizeof(float);
    const int64_t writes = mode == kTokHistory ? (int64_t)s.seq_len : (mode == kTokVerify ? 0 : 1);
    const bool ntl = state_bytes * (1 + writes) > kStreamStateBytes;
    auto go = [&](auto mode_c, auto ntl_c) {
      constexpr int MO = decltype(mode_c)::value;
      constexpr bool NL = decltype(ntl_c)::value;
      hipLaunchKernelGGL((decode_tokens_kernel<D, TIn, G, F, MO, NL>), dim3((unsigned)blocks),
                         dim3(DecodeCfg<D>::NT), 0, stream, in, pv, S, o, hist, accepted, s.seq_len,
                         s.num_heads);
    };
    auto go_mode = [&](auto mode_c) {
      if (ntl) go(mode_c, std::true_type{});
      else go(mode_c, std::false_type{});
    };
    switch (mode) {
      case kTokAdvance: go_mode(Int<kTokAdvance>{}); break;
      case kTokHistory: go_mode(Int<kTokHistory>{}); break;
      case kTokVerify: go_mode(Int<kTokVerify>{}); break;
      case kTokAccept: go_mode(Int<kTokAccept>{}); break;
      case kTokAcceptVerify: go_mode(Int<kTokAcceptVerify>{}); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_decode_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, float *S, float *o, float *hist,
                                hipStream_t stream) {
  const TokPtrs in{q, k, v, alpha, beta};
  return launch_tokens(s, in, in, S, o, hist, nullptr, hist != nullptr ? kTokHistory : kTokAdvance, stream);
}

hipError_t launch_verify_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, const float *S, float *o,
                                hipStream_t stream) {
  // (the kernel never writes S in this mode)
  const TokPtrs in{q, k, v, alpha, beta};
  return launch_tokens(s, in, in, const_cast<float *>(S), o, nullptr, nullptr, kTokVerify, stream);
}

hipError_t launch_accept_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, float *S, const int32_t *accepted,
                                hipStream_t stream) {
  const TokPtrs in{q, k, v, alpha, beta};
  return launch_tokens(s, in, in, S, nullptr, nullptr, accepted, kTokAccept, stream);
}

hipError_t launch_accept_verify_tokens(const kda_shape_t &s, const void *q0, const void *k0, const void *v0,
                                       const float *alpha0, const float *beta0, const int32_t *accepted,
                                       const void *q, const void *k, const void *v, const float *alpha,
                                       const float *beta, float *S, float *o, hipStream_t stream) {
  const TokPtrs prev{q0, k0, v0, alpha0, beta0}, in{q, k, v, alpha, beta};
  return launch_tokens(s, in, prev, S, o, nullptr, accepted, kTokAcceptVerify, stream);
}

hipError_t launch_commit(const kda_shape_t &s, float *S, const float *hist, const int32_t *accepted,
                         hipStream_t stream) {
  const int64_t blocks = (int64_t)s.num_seqs * s.num_heads;
  switch (s.d_k) {
    case 16:
      hipLaunchKernelGGL(commit_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, S, hist, accepted,
                         s.seq_len, s.num_heads);
      break;
    case 32:
      hipLaunchKernelGGL(commit_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, S, hist, accepted,
                         s.seq_len, s.num_heads);
      break;
    case 64:
      hipLaunchKernelGGL(commit_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, S, hist, accepted,
                         s.seq_len, s.num_heads);
      break;
    case 128:
      hipLaunchKernelGGL(commit_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, S, hist, accepted,
                         s.seq_len, s.num_heads);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
