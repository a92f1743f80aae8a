// Backward pass of the KDA layer (gradients for training).
//
// For the update rule S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
// + beta_t k_t v_t^T and read-out o_t = S_t^T q_t (dimsnsums.com
// "GLM-5.3-FLASH" attention page, section "How can a layer remember without
// rereading?", update rule), given dL/do_t and dL/dS_T: with
// X = Diag(alpha_t) S_{t-1}, w = v_t - X^T k_t (so S_t = X + beta_t k_t w^T)
// and G = dL/dS_t,
//
//   dv_t = beta_t G^T k_t          dbeta_t = (G^T k_t) . w
//   dk_t = beta_t (G w - X G^T k_t) dq_t = S_t dO_t
//   E = G - beta_t k_t (G^T k_t)    dalpha_t = rowsum(E * S_{t-1})
//   dL/dS_{t-1} = Diag(alpha_t) E + q_{t-1} dO_{t-1}^T.
//
// Value columns never mix in G's recurrence, so the work splits by 16 value
// columns: one 256-thread workgroup per (sequence, head, column slice),
// thread (rg, c) holding rows rg*RPT .. +RPT-1 of column c.  Per workgroup:
//   pass 1  the forward recurrence over the sequence from S0, storing the
//           state at the start of every 16-token block (workspace);
//   pass 2  blocks from last to first: re-run the block forward from its
//           checkpoint, keeping every S_{t-1} in LDS (each thread keeps its
//           own elements, so no barrier guards the ring), then the tokens
//           backward with G in registers.
// Column sums (X^T k, G^T k) cross the 16 row groups: two shuffles in the
// wave, one LDS round across the 4 waves (double-buffered, one barrier per
// token).  Row sums over the 16 columns (dk, dq, dalpha) are DPP reductions
// inside a 16-lane row; they are per-slice partials, summed over the slices
// in a fixed order by a second kernel (deterministic results).
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdVW = 16;  // value columns per workgroup

template <int D>
struct BwdCfg {
  static constexpr int VW = kBwdVW < D ? kBwdVW : D;
  static constexpr int SL = D / VW;                // column slices per head
  static constexpr int TPC = kBwdThreads / VW;     // row groups
  static constexpr int RPT = D / TPC;              // rows per thread
  static constexpr int NW = kBwdThreads / 64;
  static_assert(VW == 16 && RPT >= 1 && D % TPC == 0, "layout");
};

// Sum over the 16 lanes of a DPP row (lanes 16j .. 16j+15); the total lands
// in the row's last lane.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));  // row_shr:1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));  // row_shr:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));  // row_shr:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));  // row_shr:8
  return x;
}

template <int D, typename TIn, int GATE>
struct BwdTok {
  using Cf = BwdCfg<D>;
  float a[GATE == KDA_GATE_HEAD ? 1 : Cf::RPT];
  TIn k[Cf::RPT], q[Cf::RPT];
  TIn v;
  float b, dO;
};

// The decay rate of row r0 + i (per key channel), or the head's one rate.
template <int D, typename TIn, int GATE>
__device__ __forceinline__ float rate(const BwdTok<D, TIn, GATE> &x, int i) {
  if constexpr (GATE == KDA_GATE_HEAD) {
    return x.a[0];
  } else {
    return x.a[i];
  }
}

template <int D, typename TIn, int GATE>
__device__ __forceinline__ void load_tok(BwdTok<D, TIn, GATE> &x, const TIn *__restrict__ q,
                                         const TIn *__restrict__ k, const TIn *__restrict__ v,
                                         const float *__restrict__ alpha, const float *__restrict__ beta,
                                         const float *__restrict__ dO, int64_t th, int r0, int col,
                                         bool want_q) {
  using Cf = BwdCfg<D>;
  if constexpr (GATE == KDA_GATE_HEAD) {
    x.a[0] = alpha[th];
  } else {
#pragma unroll
    for (int i = 0; i < Cf::RPT; ++i) x.a[i] = alpha[th * D + r0 + i];
  }
#pragma unroll
  for (int i = 0; i < Cf::RPT; ++i) {
    x.k[i] = k[th * D + r0 + i];
    x.q[i] = want_q ? q[th * D + r0 + i] : x.k[i];
  }
  x.v = v[th * D + col];
  x.b = beta[th];
  x.dO = want_q ? dO[th * D + col] : 0.f;
}

template <int D, typename TIn, int GATE>
__global__ __launch_bounds__(kBwdThreads) void bwd_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    int32_t seq_len, int N, int H, int64_t total, const float *__restrict__ S0,
    const float *__restrict__ dO, const float *__restrict__ dS_T, float *__restrict__ dv,
    float *__restrict__ dS0, float *__restrict__ ckpt, float *__restrict__ part_q,
    float *__restrict__ part_k, float *__restrict__ part_a, float *__restrict__ part_b) {
  using Cf = BwdCfg<D>;
  constexpr int RPT = Cf::RPT, VW = Cf::VW, SL = Cf::SL, NW = Cf::NW;
  constexpr int CK = kBwdBlock;

  __shared__ float s_ring[CK][kBwdThreads][RPT];  // S_{t-1} of the block's tokens, per thread
  __shared__ float s_red[2][NW][2][VW];   // column sums, double-buffered
  __shared__ float s_ah[2][NW];           // scalar gate: dalpha over the rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % VW, rg = tid / VW;
  const int r0 = rg * RPT;
  const int sl = blockIdx.x % SL;
  const int nh = blockIdx.x / SL;
  const int n = nh / H, h = nh % H;
  const int col = sl * VW + c;
  int64_t start, len;
  if (cu != nullptr) {
    start = cu[n];
    len = (int64_t)cu[n + 1] - start;
  } else {
    start = (int64_t)n * seq_len;
    len = seq_len;
  }
  // Clip to the batch (malformed cu_seqlens can never index outside it).
  if (start < 0) start = 0;
  if (start > total) start = total;
  if (len < 0) len = 0;
  if (len > total - start) len = total - start;
  const int64_t nblk = (len + CK - 1) / CK;
  const int64_t blk0 = start / CK + n;  // first checkpoint slot of this sequence
  const int64_t sbase = (((int64_t)n * H + h) * D) * D;  // [n][h] state offset
  auto ck_at = [&](int64_t j) { return ckpt + (((blk0 + j) * H + h) * SL + sl) * (int64_t)(D * VW); };

  int par = 0;
  // Column sums of (x1, x2) over all rows of column c (every thread gets its
  // column's totals).
  auto col_sum2 = [&](float &x1, float &x2) __attribute__((always_inline)) {
    x1 += __shfl_xor(x1, 16);
    x2 += __shfl_xor(x2, 16);
    x1 += __shfl_xor(x1, 32);
    x2 += __shfl_xor(x2, 32);
    if (lane < VW) {
      s_red[par][wave][0][c] = x1;
      s_red[par][wave][1][c] = x2;
    }
    __syncthreads();
    float a1 = 0.f, a2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      a1 += s_red[par][w][0][c];
      a2 += s_red[par][w][1][c];
    }
    x1 = a1;
    x2 = a2;
    par ^= 1;
  };

  // ---- pass 1: forward, checkpoint at every block start -----------------------
  float s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = S0 != nullptr ? S0[sbase + (int64_t)(r0 + i) * D + col] : 0.f;
  auto fwd_step = [&](const BwdTok<D, TIn, GATE> &x) __attribute__((always_inline)) {
    float ak[RPT];
    float xk = 0.f, dummy = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      s[i] *= rate(x, i);
      ak[i] = to_f32(x.k[i]);
      xk += s[i] * ak[i];
    }
    col_sum2(xk, dummy);
    const float w = x.b * (to_f32(x.v) - xk);
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] += ak[i] * w;
  };
  {
    BwdTok<D, TIn, GATE> cur, nxt;
    if (len > 0) load_tok<D, TIn, GATE>(cur, q, k, v, alpha, beta, dO, start * H + h, r0, col, false);
    for (int64_t t = 0; t < len; ++t) {
      const int64_t tn = t + 1 < len ? t + 1 : t;
      load_tok<D, TIn, GATE>(nxt, q, k, v, alpha, beta, dO, (start + tn) * H + h, r0, col, false);
      if (t % CK == 0) {
        float *cp = ck_at(t / CK);
#pragma unroll
        for (int i = 0; i < RPT; ++i) cp[(r0 + i) * VW + c] = s[i];
      }
      fwd_step(cur);
      cur = nxt;
    }
  }
  // Each thread reads back only the checkpoint elements it wrote.
  __threadfence_block();

  // ---- pass 2: backward ---------------------------------------------------------
  float G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) G[i] = dS_T != nullptr ? dS_T[sbase + (int64_t)(r0 + i) * D + col] : 0.f;
  for (int64_t b = nblk - 1; b >= 0; --b) {
    const int64_t tb = b * CK;
    const int nt = (int)(len - tb < CK ? len - tb : CK);
    {
      const float *cp = ck_at(b);
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] = cp[(r0 + i) * VW + c];
    }
    BwdTok<D, TIn, GATE> cur, nxt;
    load_tok<D, TIn, GATE>(cur, q, k, v, alpha, beta, dO, (start + tb) * H + h, r0, col, false);
    for (int j = 0; j < nt; ++j) {
      const int jn = j + 1 < nt ? j + 1 : j;
      load_tok<D, TIn, GATE>(nxt, q, k, v, alpha, beta, dO, (start + tb + jn) * H + h, r0, col, false);
#pragma unroll
      for (int i = 0; i < RPT; ++i) s_ring[j][tid][i] = s[i];
      fwd_step(cur);
      cur = nxt;
    }
    load_tok<D, TIn, GATE>(cur, q, k, v, alpha, beta, dO, (start + tb + nt - 1) * H + h, r0, col, true);
    for (int j = nt - 1; j >= 0; --j) {
      const int64_t th = (start + tb + j) * H + h;
      const int jp = j > 0 ? j - 1 : 0;
      load_tok<D, TIn, GATE>(nxt, q, k, v, alpha, beta, dO, (start + tb + jp) * H + h, r0, col, true);
      float sp[RPT], X[RPT], kf[RPT];
      float xk = 0.f, gk = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float a = rate(cur, i);
        sp[i] = s_ring[j][tid][i];
        kf[i] = to_f32(cur.k[i]);
        G[i] += to_f32(cur.q[i]) * cur.dO;
        X[i] = a * sp[i];
        xk += X[i] * kf[i];
        gk += G[i] * kf[i];
      }
      col_sum2(xk, gk);
      const float bt = cur.b;
      const float w = to_f32(cur.v) - xk;
      if (rg == 0) dv[th * D + col] = bt * gk;
      const float db = row16_sum(gk * w);
      if (tid == VW - 1) part_b[(int64_t)sl * total * H + th] = db;
      float dkp[RPT], dqp[RPT], dap[RPT];
      float da_all = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float a = rate(cur, i);
        const float st = X[i] + bt * kf[i] * w;  // S_t
        dkp[i] = bt * (G[i] * w - X[i] * gk);
        dqp[i] = st * cur.dO;
        const float e = G[i] - bt * kf[i] * gk;
        dap[i] = e * sp[i];
        da_all += dap[i];
        G[i] = a * e;
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        dkp[i] = row16_sum(dkp[i]);
        dqp[i] = row16_sum(dqp[i]);
        if constexpr (GATE != KDA_GATE_HEAD) dap[i] = row16_sum(dap[i]);
      }
      const int64_t po = ((int64_t)sl * total * H + th) * D + r0;
      if (c == VW - 1) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          part_k[po + i] = dkp[i];
          part_q[po + i] = dqp[i];
          if constexpr (GATE != KDA_GATE_HEAD) part_a[po + i] = dap[i];
        }
      }
      if constexpr (GATE == KDA_GATE_HEAD) {
        // one rate per head: dalpha sums over every row and column of the slice
        float t = row16_sum(da_all);
        t = __shfl(t, (lane & ~15) + 15);
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if (lane == 0) s_ah[par][wave] = t;
        __syncthreads();
        if (tid == 0) {
          float u = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) u += s_ah[par][w2];
          part_a[(int64_t)sl * total * H + th] = u;
        }
        par ^= 1;
      }
      cur = nxt;
    }
  }
  if (dS0 != nullptr) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) dS0[sbase + (int64_t)(r0 + i) * D + col] = G[i];
  }
}

// dq, dk, dalpha (and dbeta) = sums of the per-slice partials, slice order fixed.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *__restrict__ part, float *__restrict__ out,
                                                         int64_t n, int slices) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float acc = 0.f;
    for (int s = 0; s < slices; ++s) acc += part[(int64_t)s * n + i];
    out[i] = acc;
  }
}

template <int D, typename TIn, int GATE>
hipError_t launch_bwd_t(const kda_shape_t &s, const BwdArgs &a, hipStream_t stream) {
  using Cf = BwdCfg<D>;
  const BwdLayout L = backward_layout(s);
  char *ws = static_cast<char *>(a.workspace);
  float *ckpt = reinterpret_cast<float *>(ws + L.ckpt_off);
  float *pq = reinterpret_cast<float *>(ws + L.part_q_off);
  float *pk = reinterpret_cast<float *>(ws + L.part_k_off);
  float *pa = reinterpret_cast<float *>(ws + L.part_a_off);
  float *pb = reinterpret_cast<float *>(ws + L.part_b_off);
  const int64_t blocks = (int64_t)s.num_seqs * s.num_heads * Cf::SL;
  hipLaunchKernelGGL((bwd_kernel<D, TIn, GATE>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, stream,
                     static_cast<const TIn *>(a.q), static_cast<const TIn *>(a.k),
                     static_cast<const TIn *>(a.v), a.alpha, a.beta, a.cu, s.seq_len, s.num_seqs, s.num_heads,
                     s.total_tokens, a.S0, a.dO, a.dS_T, a.dv, a.dS0, ckpt, pq, pk, pa, pb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t th = s.total_tokens * s.num_heads;
  const int64_t nd = th * D, na = GATE == KDA_GATE_HEAD ? th : nd;
  struct {
    const float *p;
    float *o;
    int64_t n;
  } jobs[4] = {{pq, a.dq, nd}, {pk, a.dk, nd}, {pa, a.dalpha, na}, {pb, a.dbeta, th}};
  for (const auto &j : jobs) {
    if (j.n == 0) continue;
    const int64_t g = (j.n + 255) / 256 < 8192 ? (j.n + 255) / 256 : 8192;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)g), dim3(256), 0, stream, j.p, j.o, j.n, Cf::SL);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TIn, int GATE>
hipError_t bwd_by_dim(const kda_shape_t &s, const BwdArgs &a, hipStream_t st) {
  switch (s.d_k) {
    case 16: return launch_bwd_t<16, TIn, GATE>(s, a, st);
    case 32: return launch_bwd_t<32, TIn, GATE>(s, a, st);
    case 64: return launch_bwd_t<64, TIn, GATE>(s, a, st);
    case 128: return launch_bwd_t<128, TIn, GATE>(s, a, st);
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t bwd_by_gate(const kda_shape_t &s, const BwdArgs &a, hipStream_t st) {
  if (s.gate == KDA_GATE_HEAD) return bwd_by_dim<TIn, KDA_GATE_HEAD>(s, a, st);
  return bwd_by_dim<TIn, KDA_GATE_CHANNEL>(s, a, st);
}

}  // namespace

hipError_t launch_backward(const kda_shape_t &s, const BwdArgs &a, hipStream_t stream) {
  if (s.qkv_dtype == KDA_BF16) return bwd_by_gate<__bf16>(s, a, stream);
  return bwd_by_gate<float>(s, a, stream);
}

}  // namespace kda
