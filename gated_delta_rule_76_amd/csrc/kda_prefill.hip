// Chunked prefill of the KDA layer on gfx950.
//
// The update rule S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
// + beta_t k_t v_t^T with read-out o_t = S_t^T q_t (dimsnsums.com
// "GLM-5.3-FLASH" attention page, section "How can a layer remember without
// rereading?", update rule) is rewritten exactly, per chunk of C = 64
// tokens r = 1..C with state S0 at the chunk start:
//
//   Gamma_r   = prod_{s<=r} alpha_s                 (per key channel)
//   A_rj      = sum_c k_rc k_jc Gamma_rc/Gamma_jc   (j < r)
//   M_rj      = sum_c q_rc k_jc Gamma_rc/Gamma_jc   (j <= r)
//   T         = (I + Diag(beta) A)^-1 Diag(beta)    (unit lower triangular solve)
//   W         = T (V - Khat S0),  Khat_r = Gamma_r * k_r
//   O         = Qhat S0 + M W,    Qhat_r = Gamma_r * q_r
//   S_C       = Diag(Gamma_C) S0 + Ktil^T W,  Ktil_j = (Gamma_C/Gamma_j) * k_j
//
// (unrolling the recurrence: S_r = Diag(Gamma_r) S0 + sum_{j<=r}
// Diag(Gamma_r/Gamma_j) k_j w_j^T with w_r = beta_r (v_r - k_r^T Diag(alpha_r)
// S_{r-1}); collecting the w_r gives the triangular system above).  A tail
// chunk is padded with alpha = 1, beta = 0, q = k = v = 0, which is an
// exact identity step.
//
// Three kernels:
//   schedule_kernel     varlen packing: chunk counts per sequence -> table
//                       of first-chunk indices (exclusive scan).
//   chunk_local_kernel  one workgroup per (chunk, head), fully parallel:
//                       A and M on the matrix cores, T by a blocked
//                       triangular inverse in fp32; T and M go to the
//                       workspace.
//   chunk_state_kernel  one workgroup per (sequence, head, 16 value
//                       columns), sequential over the chunks of its
//                       sequence: the state slice stays in registers (fp32)
//                       across chunks; every product with S, W and T runs on
//                       the matrix cores.
//
// Decay factors are formed as running products of alpha (never as exp of
// differences of cumulative logs), so no factor exceeds 1 except 1/Gamma
// inside one 16-token block, which is used only when that block's decay
// stays above 2^-100 in every channel; otherwise that diagonal block is
// recomputed directly (see chunk_local_kernel).  alpha = 0 is therefore exact.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = kChunk;          // 64 tokens per chunk
constexpr int NT = 256;            // threads per workgroup (4 waves)
constexpr float kTinyBlock = 7.888609052210118e-31f;  // 2^-100

// ---------------------------------------------------------------------------
// LDS operand planes: a ROWS x COLS fp32 matrix stored either as a bf16
// hi/lo pair (SplitBF16) or as fp32 (F32), padded so that the 16 lanes of a
// fragment read (16 rows, same columns) fall in different banks.
// ---------------------------------------------------------------------------
template <typename P, int ROWS, int COLS>
struct Plane;

template <int ROWS, int COLS>
struct alignas(16) Plane<SplitBF16, ROWS, COLS> {
  static constexpr int PITCH = COLS + 8;
  __bf16 hi[ROWS * PITCH];
  __bf16 lo[ROWS * PITCH];
  __device__ __forceinline__ void store(int r, int c, float x) {
    const __bf16 h = (__bf16)x;
    hi[r * PITCH + c] = h;
    lo[r * PITCH + c] = (__bf16)(x - (float)h);
  }
  __device__ __forceinline__ void store4(int r, int c, const f32x4 &x) {
    bf16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = (__bf16)x[i];
      l[i] = (__bf16)(x[i] - (float)h[i]);
    }
    *reinterpret_cast<bf16x4 *>(&hi[r * PITCH + c]) = h;
    *reinterpret_cast<bf16x4 *>(&lo[r * PITCH + c]) = l;
  }
  __device__ __forceinline__ void store8(int r, int c, const float (&x)[8]) {
    bf16x8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = (__bf16)x[i];
      l[i] = (__bf16)(x[i] - (float)h[i]);
    }
    *reinterpret_cast<bf16x8 *>(&hi[r * PITCH + c]) = h;
    *reinterpret_cast<bf16x8 *>(&lo[r * PITCH + c]) = l;
  }
  __device__ __forceinline__ SplitBF16::Frag load8(int r, int c) const {
    SplitBF16::Frag f;
    f.hi = *reinterpret_cast<const bf16x8 *>(&hi[r * PITCH + c]);
    f.lo = *reinterpret_cast<const bf16x8 *>(&lo[r * PITCH + c]);
    return f;
  }
};

template <int ROWS, int COLS>
struct alignas(16) Plane<F32, ROWS, COLS> {
  static constexpr int PITCH = COLS + 4;
  float f[ROWS * PITCH];
  __device__ __forceinline__ void store(int r, int c, float x) { f[r * PITCH + c] = x; }
  __device__ __forceinline__ void store4(int r, int c, const f32x4 &x) {
    *reinterpret_cast<f32x4 *>(&f[r * PITCH + c]) = x;
  }
  __device__ __forceinline__ void store8(int r, int c, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = x[i];
      b[i] = x[4 + i];
    }
    *reinterpret_cast<f32x4 *>(&f[r * PITCH + c]) = a;
    *reinterpret_cast<f32x4 *>(&f[r * PITCH + c + 4]) = b;
  }
  __device__ __forceinline__ F32::Frag load8(int r, int c) const {
    F32::Frag fr;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(&f[r * PITCH + c]);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(&f[r * PITCH + c + 4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fr.v[j] = a[j];
      fr.v[4 + j] = b[j];
    }
    return fr;
  }
};

// Token range of a chunk.  Sequence n owns tokens [start, start + len); its
// chunk lc covers [start + 64 lc, ...) with `valid` real tokens (clipped to
// the batch, so malformed cu_seqlens can never index outside the tensors).
struct ChunkTok {
  int64_t t0;
  int valid;
};

__device__ __forceinline__ void seq_range(const int32_t *cu, int32_t seq_len, int n, int64_t &start,
                                          int64_t &len) {
  if (cu != nullptr) {
    start = cu[n];
    len = (int64_t)cu[n + 1] - start;
  } else {
    start = (int64_t)n * seq_len;
    len = seq_len;
  }
  if (len < 0) len = 0;
}

__device__ __forceinline__ ChunkTok chunk_tokens(int64_t start, int64_t len, int64_t lc,
                                                 int64_t total_tokens) {
  ChunkTok ct;
  ct.t0 = start + (int64_t)C * lc;
  int64_t v = len - (int64_t)C * lc;
  v = v < C ? v : C;
  const int64_t room = total_tokens - ct.t0;
  v = v < room ? v : room;
  ct.valid = (v > 0 && ct.t0 >= 0) ? (int)v : 0;
  return ct;
}

// Token read for chunk row r: rows past the valid ones re-read the last valid
// row (their values are then replaced by the padding), and every index is
// clamped into [0, total_tokens) so a load can never leave the tensors.
__device__ __forceinline__ int64_t load_token(int64_t t0, int r, int valid, int64_t total_tokens) {
  const int rr = r < valid ? r : (valid > 0 ? valid - 1 : 0);
  int64_t t = t0 + rr;
  t = t < total_tokens ? t : total_tokens - 1;
  return t > 0 ? t : 0;
}

// ---------------------------------------------------------------------------
// Varlen schedule: base[n] = number of chunks of sequences < n, base[N] =
// total chunks.  One workgroup; a block-wide scan per 1024 sequences.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ cu, int N,
                                                        int32_t seq_len, int32_t *__restrict__ base) {
  __shared__ int32_t s_scan[1024];
  const int tid = threadIdx.x;
  int32_t carry = 0;
  for (int start = 0; start < N; start += 1024) {
    const int n = start + tid;
    int32_t cnt = 0;
    if (n < N) {
      int64_t s0, len;
      seq_range(cu, seq_len, n, s0, len);
      cnt = (int32_t)((len + C - 1) / C);
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (n < N) base[n] = carry + s_scan[tid] - cnt;
    carry += s_scan[1023];
    __syncthreads();
  }
  if (tid == 0) base[N] = carry;
}

// Largest n in [0, N) with base[n] <= c (base is non-decreasing, base[0] = 0).
__device__ __forceinline__ int find_seq(const int32_t *base, int N, int64_t c) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)base[mid] <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// chunk_local_kernel: A, M and T of one chunk and head.
//
// The decayed Gram blocks are computed on 16x16 tiles (R, J), J <= R, of
// 16-token blocks.  Per key channel, with bp[r] = product of alpha from the
// start of r's block to r (inclusive), bs[j] = product of alpha after j to
// the end of j's block, bt[b] = decay of the whole block b:
//     Gamma_r / Gamma_j = bp[r] * bs[j] * prod_{J<b<R} bt[b]     (J < R)
//                       = bp[r] / bp[j]                          (J = R, j <= r)
// so each tile is a plain product (x_r * bp_r) . (k_j * left_j) over the key
// channels, done in 32-channel slices on the matrix cores.  In the diagonal
// case 1/bp[j] <= 2^100 is guaranteed by the block test; a block that fails
// it (a channel decaying below 2^-100 within 16 tokens, e.g. alpha = 0) has
// its diagonal tiles recomputed from running products of alpha.
// ---------------------------------------------------------------------------
template <int D>
struct LocalCfg {
  static constexpr int KS = 32;                // channels per slice
  static constexpr int NSL = (D + KS - 1) / KS;
  static constexpr int SP = KS + 4;            // slice pitch (floats)
  static constexpr int MP = C + 1;             // 64x64 matrix pitch
};

// Tiles per wave (5 each): waves 0/1 take block-row 3 plus tile (0,0) of
// A / M, waves 2/3 take block-rows 2 and 1 of A / M.
__device__ __forceinline__ int tile_R(int tsel, int t) { return tsel == 0 ? (t < 4 ? 3 : 0) : (t < 3 ? 2 : 1); }
__device__ __forceinline__ int tile_J(int tsel, int t) { return tsel == 0 ? (t < 4 ? t : 0) : (t < 3 ? t : t - 3); }

template <int D, typename TIn, typename P>
__global__ __launch_bounds__(NT) void chunk_local_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t max_chunks, const int32_t *__restrict__ base,
    float *__restrict__ mats) {
  using L = LocalCfg<D>;
  constexpr int KS = L::KS, SP = L::SP, MP = L::MP;

  __shared__ float s_k[C * SP], s_q[C * SP], s_bp[C * SP], s_bs[C * SP], s_ibp[C * SP];
  __shared__ float s_bt[4 * KS];
  __shared__ float s_A[C * MP], s_M[C * MP], s_X[C * MP];
  __shared__ float s_Y[3 * 16 * 17];
  __shared__ float s_beta[C];
  __shared__ int s_flag[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int64_t c = (int64_t)(blockIdx.x / H);
  const int h = blockIdx.x % H;
  const int64_t nchunks = base[N] < max_chunks ? (int64_t)base[N] : max_chunks;
  if (c >= nchunks) return;
  const int n = find_seq(base, N, c);
  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const ChunkTok ct = chunk_tokens(sstart, slen, c - base[n], total_tokens);
  const int64_t t0 = ct.t0;
  const int nvalid = ct.valid;

  for (int e = tid; e < C * MP; e += NT) {
    s_A[e] = 0.f;
    s_M[e] = 0.f;
    s_X[e] = 0.f;
  }
  if (tid < C) s_beta[tid] = tid < nvalid ? beta[(t0 + tid) * H + h] : 0.f;
  if (tid < 4) s_flag[tid] = 0;

  const int tsel = wave >> 1;
  const bool isM = (wave & 1) != 0;
  f32x4 acc[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) acc[t] = zero4();

  // All of the chunk's q, k and alpha are loaded up front with unconditional
  // vector loads (rows past the valid ones re-read a valid row and are
  // replaced by the padding when written to LDS): per 32-channel slice a
  // thread holds 8 channels of q and k of one row and 2 x 4 channels of
  // alpha of two rows.
  const int kr = tid >> 2, kc = 8 * (tid & 3);       // q/k: row, first channel in slice
  Raw8<TIn> rk[L::NSL], rq[L::NSL];
  float4 ra[L::NSL][2];
  {
    const int64_t tk = load_token(t0, kr, nvalid, total_tokens);
#pragma unroll
    for (int sl = 0; sl < L::NSL; ++sl) {
      const int ch = sl * KS + kc < D - 8 ? sl * KS + kc : D - 8;
      rk[sl].load(k + (tk * H + h) * D + ch);
      rq[sl].load(q + (tk * H + h) * D + ch);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + NT * u, ar = e >> 3, ac = 4 * (e & 7);
        const int cha = sl * KS + ac < D - 4 ? sl * KS + ac : D - 4;
        ra[sl][u] = *reinterpret_cast<const float4 *>(
            alpha + (load_token(t0, ar, nvalid, total_tokens) * H + h) * D + cha);
      }
    }
  }

#pragma unroll
  for (int sl = 0; sl < L::NSL; ++sl) {
    __syncthreads();  // previous slice fully consumed
    {
      const bool okr = kr < nvalid;
      float xk[8], xq[8];
      rk[sl].to_f32(xk);
      rq[sl].to_f32(xq);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = okr && (sl * KS + kc + j < D);
        s_k[kr * SP + kc + j] = ok ? xk[j] : 0.f;
        s_q[kr * SP + kc + j] = ok ? xq[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = tid + NT * u, ar = e >> 3, ac = 4 * (e & 7);
        const float av[4] = {ra[sl][u].x, ra[sl][u].y, ra[sl][u].z, ra[sl][u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = (ar < nvalid) && (sl * KS + ac + j < D);
          s_bp[ar * SP + ac + j] = ok ? av[j] : 1.f;
        }
      }
    }
    __syncthreads();
    if (tid < 4 * KS) {
      const int b = tid / KS, cc = tid % KS;
      float a[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) a[i] = s_bp[(16 * b + i) * SP + cc];
      float p = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p *= a[i];
        s_bp[(16 * b + i) * SP + cc] = p;
      }
      const bool tiny = !(p >= kTinyBlock);
      float sfx = 1.f;
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        s_bs[(16 * b + i) * SP + cc] = sfx;
        sfx *= a[i];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float bpv = s_bp[(16 * b + i) * SP + cc];
        s_ibp[(16 * b + i) * SP + cc] = tiny ? 0.f : 1.0f / bpv;
      }
      s_bt[b * KS + cc] = p;
      if (tiny) atomicOr(&s_flag[b], 1);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const int R = tile_R(tsel, t), J = tile_J(tsel, t);
      const int r = 16 * R + m, jr = 16 * J + m;
      const float *X = isM ? s_q : s_k;
      float xa[8], xb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cc = 8 * g + j;
        xa[j] = X[r * SP + cc] * s_bp[r * SP + cc];
        float left;
        if (J == R) {
          left = s_ibp[jr * SP + cc];
        } else {
          left = s_bs[jr * SP + cc];
          for (int b = J + 1; b < R; ++b) left *= s_bt[b * KS + cc];
        }
        xb[j] = s_k[jr * SP + cc] * left;
      }
      P::mma(acc[t], P::make(xa), P::make(xb));
    }
  }

  // Scatter the tiles (accumulator layout: row 4g+i, column m of the tile),
  // keeping j < r for A and j <= r for M.
  {
    float *dst = isM ? s_M : s_A;
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const int R = tile_R(tsel, t), J = tile_J(tsel, t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * R + 4 * g + i, j = 16 * J + m;
        const bool keep = isM ? (j <= r) : (j < r);
        dst[r * MP + j] = keep ? acc[t][i] : 0.f;
      }
    }
  }
  __syncthreads();

  // Rare path: a 16-token block whose decay underflows 2^-100 in some
  // channel.  Recompute its diagonal tiles of A and M directly:
  //   sum_c x_rc k_jc prod_{j<s<=r} alpha_sc.
  for (int b = 0; b < 4; ++b) {
    if (s_flag[b] == 0) continue;  // uniform across the workgroup
    if (tid < 136) {
      int r = 0, rem = tid;
      while (rem > r) {  // pair index -> (r, j), j <= r, within the block
        rem -= r + 1;
        ++r;
      }
      const int j = rem;
      const int rr = 16 * b + r, jj = 16 * b + j;
      float a_acc = 0.f, m_acc = 0.f;
      if (rr < nvalid && jj < nvalid) {
        for (int ch = 0; ch < D; ++ch) {
          float f = 1.f;
          for (int s = jj + 1; s <= rr; ++s) f *= alpha[((t0 + s) * H + h) * D + ch];
          const int64_t orr = ((t0 + rr) * H + h) * D + ch, ojj = ((t0 + jj) * H + h) * D + ch;
          const float kj = to_f32(k[ojj]) * f;
          a_acc += to_f32(k[orr]) * kj;
          m_acc += to_f32(q[orr]) * kj;
        }
      }
      s_A[rr * MP + jj] = (j < r) ? a_acc : 0.f;
      s_M[rr * MP + jj] = m_acc;
    }
    __syncthreads();
  }

  // L = I + Diag(beta) A (strictly lower part kept in s_A, unit diagonal implied).
  for (int e = tid; e < C * C; e += NT) {
    const int r = e / C, j = e % C;
    if (j < r) s_A[r * MP + j] *= s_beta[r];
  }
  __syncthreads();

  // X = L^-1, blocked by 16.  Diagonal blocks: forward substitution, one
  // column per lane (wave b inverts block b).
  if (lane < 16) {
    const int b = wave, jj = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) s -= s_A[(16 * b + i) * MP + 16 * b + t] * x[t];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s_X[(16 * b + i) * MP + 16 * b + jj] = x[i];
  }
  __syncthreads();
  // Off-diagonal blocks by distance d: X_IJ = -X_II sum_{K=J}^{I-1} L_IK X_KJ.
  for (int d = 1; d < 4; ++d) {
    const int nblk = 4 - d;
    for (int e = tid; e < nblk * 256; e += NT) {
      const int J = e >> 8, rr = (e >> 4) & 15, cc = e & 15, I = J + d;
      float s = 0.f;
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int t = 0; t < 16; ++t) s += s_A[(16 * I + rr) * MP + 16 * K + t] * s_X[(16 * K + t) * MP + 16 * J + cc];
      }
      s_Y[(J * 16 + rr) * 17 + cc] = s;
    }
    __syncthreads();
    for (int e = tid; e < nblk * 256; e += NT) {
      const int J = e >> 8, rr = (e >> 4) & 15, cc = e & 15, I = J + d;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) s += s_X[(16 * I + rr) * MP + 16 * I + t] * s_Y[(J * 16 + t) * 17 + cc];
      s_X[(16 * I + rr) * MP + 16 * J + cc] = -s;
    }
    __syncthreads();
  }

  // T = X Diag(beta); write T then M (64x64 fp32 each, row-major).
  float *outT = mats + ((size_t)c * H + h) * (size_t)(2 * C * C);
  float *outM = outT + C * C;
  for (int e = tid; e < C * C; e += NT) {
    const int r = e / C, j = e % C;
    outT[e] = s_X[r * MP + j] * s_beta[j];
    outM[e] = s_M[r * MP + j];
  }
}

// ---------------------------------------------------------------------------
// chunk_state_kernel: the sequential pass over the chunks of one sequence
// for one head and 16 value columns.
//
// Wave w owns chunk rows 16w..16w+15 for E = Khat S, O = Qhat S + M W and
// W = T (V - E), and state row tiles w, w+4 (16 key channels each) for the
// update S <- Diag(Gamma_C) S + Ktil^T W.  S is kept in fp32 accumulators;
// a copy in operand form (S^T, split for the matrix cores) lives in LDS so
// that every wave can use all key rows.
//
// Per chunk, every thread stages 8 key channels of TPG consecutive tokens:
// q, k, alpha arrive as 16-byte vector loads issued one chunk ahead (the
// next chunk's loads are in flight while this chunk computes), the decay
// factors are running products of alpha along the tokens (a two-level scan:
// inside the thread's tokens, then across token groups through LDS), and
// the operands Khat, Qhat (rows = tokens) and Ktil^T (rows = channels) are
// written to LDS already split for the matrix cores.
//
// blockIdx -> work: consecutive workgroups are dealt round-robin to the 8
// XCDs, so the D/16 workgroups of one (sequence, head) are mapped to block
// indices congruent mod 8: they share an XCD and its L2, and the chunk
// inputs and T/M they all read are fetched from HBM once.
// ---------------------------------------------------------------------------
template <int D>
struct StateCfg {
  static constexpr int G = D / 16;                            // value-column groups per head
  static constexpr int DK = D < 32 ? 32 : D;                  // key width of operand planes
  static constexpr int NKB = DK / 32;                         // 32-wide k-blocks over key channels
  static constexpr int NTILE = D / 16;                        // 16-row tiles of the state
  static constexpr int TPW = (NTILE + 3) / 4;                 // state tiles per wave (max)
  static constexpr int CGR = D / 8;                           // 8-channel groups per token row
  static constexpr int NTG = (NT / CGR) < C ? NT / CGR : C;   // token groups
  static constexpr int TPG = C / NTG;                         // tokens per staging thread
  static constexpr int ACTIVE = CGR * NTG;                    // staging threads
  static_assert(ACTIVE <= NT && C % NTG == 0, "staging layout");
};

template <int D, typename TIn>
struct StateRaw {
  static constexpr int TPG = StateCfg<D>::TPG;
  Raw8<TIn> k[TPG], q[TPG];
  float4 a0[TPG], a1[TPG];
  Raw4<TIn> v;
};

template <int D, typename TIn>
__device__ __forceinline__ void load_state_raw(StateRaw<D, TIn> &R, const TIn *__restrict__ q,
                                               const TIn *__restrict__ k, const TIn *__restrict__ v,
                                               const float *__restrict__ alpha, int64_t t0, int valid,
                                               int64_t total, int h, int H, int col0, int tid) {
  using Cf = StateCfg<D>;
  if (tid < Cf::ACTIVE) {
    const int cg8 = tid % Cf::CGR, tg = tid / Cf::CGR;
#pragma unroll
    for (int i = 0; i < Cf::TPG; ++i) {
      const int64_t off = (load_token(t0, tg * Cf::TPG + i, valid, total) * H + h) * D + 8 * cg8;
      R.k[i].load(k + off);
      R.q[i].load(q + off);
      R.a0[i] = *reinterpret_cast<const float4 *>(alpha + off);
      R.a1[i] = *reinterpret_cast<const float4 *>(alpha + off + 4);
    }
  }
  const int64_t voff = (load_token(t0, tid >> 2, valid, total) * H + h) * D + col0 + 4 * (tid & 3);
  R.v.load(v + voff);
}

template <int D, typename TIn, typename P>
__global__ __launch_bounds__(NT) void chunk_state_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ alpha, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t max_chunks, const int32_t *__restrict__ base,
    const float *__restrict__ mats, const float *__restrict__ S0, float *__restrict__ o,
    float *__restrict__ S_T) {
  using Cf = StateCfg<D>;
  constexpr int G = Cf::G, DK = Cf::DK, NKB = Cf::NKB, NTILE = Cf::NTILE, TPW = Cf::TPW;
  constexpr int CGR = Cf::CGR, NTG = Cf::NTG, TPG = Cf::TPG;

  __shared__ Plane<P, C, DK> Khat;
  __shared__ Plane<P, C, DK> Qhat;
  __shared__ Plane<P, D, C> KtilT;
  __shared__ Plane<P, 16, DK> Sop;
  __shared__ Plane<P, 16, C> Vme;
  __shared__ Plane<P, 16, C> Wop;
  __shared__ float s_v[C * 17];
  __shared__ float s_gam[D];
  __shared__ __attribute__((aligned(16))) float s_pre[NTG * D];  // group totals, then exclusive prefix
  __shared__ __attribute__((aligned(16))) float s_suf[NTG * D];  // exclusive suffix over groups

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;

  const int id = blockIdx.x;
  const int xcd = id & 7, within = id >> 3;
  const int64_t pair = (int64_t)(within / G) * 8 + xcd;
  const int cg = within % G;
  if (pair >= (int64_t)N * H) return;
  const int n = (int)(pair / H), h = (int)(pair % H);
  const int col0 = 16 * cg;

  // Zero the padded key channels of the channel-indexed planes once.
  if constexpr (DK > D) {
    for (int e = tid; e < C * (DK - D); e += NT) {
      const int r = e / (DK - D), cc = D + e % (DK - D);
      Khat.store(r, cc, 0.f);
      Qhat.store(r, cc, 0.f);
      if (r < 16) Sop.store(r, cc, 0.f);
    }
  }

  // Initial state: rows 16t + 4g + i, column col0 + m.
  f32x4 sreg[TPW];
  const float *S0p = S0 ? S0 + (size_t)pair * D * D : nullptr;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + 4 * u;
    sreg[u] = zero4();
    if (t < NTILE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * t + 4 * g + i;
        sreg[u][i] = S0p ? S0p[(size_t)row * D + col0 + m] : 0.f;
      }
      Sop.store4(m, 16 * t + 4 * g, sreg[u]);
    }
  }

  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const int64_t cbeg = base[n];
  int64_t cend = base[n + 1];
  if (cend > max_chunks) cend = max_chunks;
  if (total_tokens <= 0) cend = cbeg;

  const int cg8 = tid % CGR, tg = tid / CGR;
  const int rbase = 16 * wave;
  const int nkb = (wave >> 1) + 1;  // T and M are lower triangular

  // Two register sets for the per-chunk loads (raw inputs and this wave's
  // T/M rows), used alternately: while chunk c is processed from one set,
  // chunk c+1 is loading into the other (the loop is unrolled by two so that
  // no register copy sits between a load and its use).
  StateRaw<D, TIn> bufA, bufB;
  float4 tA[4], mA[4], tB[4], mB[4];
  auto load_tm = [&](int64_t cc, float4 (&tq)[4], float4 (&mq)[4]) {
    const float *src = mats + ((size_t)cc * H + h) * (size_t)(2 * C * C) + (rbase + m) * C + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {  // both k-blocks; above the diagonal T and M are 0
      tq[2 * kb] = *reinterpret_cast<const float4 *>(src + kb * 32);
      tq[2 * kb + 1] = *reinterpret_cast<const float4 *>(src + kb * 32 + 4);
      mq[2 * kb] = *reinterpret_cast<const float4 *>(src + C * C + kb * 32);
      mq[2 * kb + 1] = *reinterpret_cast<const float4 *>(src + C * C + kb * 32 + 4);
    }
  };
  auto prefetch = [&](int64_t cc, StateRaw<D, TIn> &R, float4 (&tq)[4], float4 (&mq)[4]) {
    const ChunkTok cn = chunk_tokens(sstart, slen, cc - cbeg, total_tokens);
    load_state_raw<D, TIn>(R, q, k, v, alpha, cn.t0, cn.valid, total_tokens, h, H, col0, tid);
    load_tm(cc, tq, mq);
  };

  auto process = [&](int64_t c, const StateRaw<D, TIn> &use, const float4 (&tu)[4], const float4 (&mu)[4],
                     int64_t cn, StateRaw<D, TIn> &nb, float4 (&tn)[4], float4 (&mn)[4]) {
    const ChunkTok ct = chunk_tokens(sstart, slen, c - cbeg, total_tokens);
    const int64_t t0 = ct.t0;
    const int nvalid = ct.valid;
    __syncthreads();  // previous chunk's operands fully consumed

    // ---- stage: decay factors and operands --------------------------------
    float av[TPG][8], kv[TPG][8], qv[TPG][8];
    if (tid < Cf::ACTIVE) {
      float tot[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tot[j] = 1.f;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        const bool ok = tg * TPG + i < nvalid;
        use.k[i].to_f32(kv[i]);
        use.q[i].to_f32(qv[i]);
        const float a[8] = {use.a0[i].x, use.a0[i].y, use.a0[i].z, use.a0[i].w,
                            use.a1[i].x, use.a1[i].y, use.a1[i].z, use.a1[i].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          av[i][j] = ok ? a[j] : 1.f;
          kv[i][j] = ok ? kv[i][j] : 0.f;
          qv[i][j] = ok ? qv[i][j] : 0.f;
          tot[j] *= av[i][j];
        }
      }
      *reinterpret_cast<float4 *>(&s_pre[tg * D + 8 * cg8]) = make_float4(tot[0], tot[1], tot[2], tot[3]);
      *reinterpret_cast<float4 *>(&s_pre[tg * D + 8 * cg8 + 4]) = make_float4(tot[4], tot[5], tot[6], tot[7]);
    }
    {
      float vv[4];
      use.v.to_f32(vv);
      const int r = tid >> 2;
      const bool ok = r < nvalid;
#pragma unroll
      for (int j = 0; j < 4; ++j) s_v[r * 17 + 4 * (tid & 3) + j] = ok ? vv[j] : 0.f;
    }
    __syncthreads();
    if (tid < D) {  // exclusive suffix, then exclusive prefix (in place), over token groups
      float sfx = 1.f;
      for (int gg = NTG - 1; gg >= 0; --gg) {
        s_suf[gg * D + tid] = sfx;
        sfx *= s_pre[gg * D + tid];
      }
      float pfx = 1.f;
      for (int gg = 0; gg < NTG; ++gg) {
        const float tv = s_pre[gg * D + tid];
        s_pre[gg * D + tid] = pfx;
        pfx *= tv;
      }
      s_gam[tid] = pfx;  // Gamma_C
    }
    __syncthreads();
    if (tid < Cf::ACTIVE) {
      float ep[8], es[8];
      {
        const float4 p0 = *reinterpret_cast<const float4 *>(&s_pre[tg * D + 8 * cg8]);
        const float4 p1 = *reinterpret_cast<const float4 *>(&s_pre[tg * D + 8 * cg8 + 4]);
        const float4 s0 = *reinterpret_cast<const float4 *>(&s_suf[tg * D + 8 * cg8]);
        const float4 s1 = *reinterpret_cast<const float4 *>(&s_suf[tg * D + 8 * cg8 + 4]);
        ep[0] = p0.x; ep[1] = p0.y; ep[2] = p0.z; ep[3] = p0.w;
        ep[4] = p1.x; ep[5] = p1.y; ep[6] = p1.z; ep[7] = p1.w;
        es[0] = s0.x; es[1] = s0.y; es[2] = s0.z; es[3] = s0.w;
        es[4] = s1.x; es[5] = s1.y; es[6] = s1.z; es[7] = s1.w;
      }
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        float xk[8], xq[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ep[j] *= av[i][j];  // Gamma_r (inclusive)
          xk[j] = ep[j] * kv[i][j];
          xq[j] = ep[j] * qv[i][j];
        }
        Khat.store8(tg * TPG + i, 8 * cg8, xk);
        Qhat.store8(tg * TPG + i, 8 * cg8, xq);
      }
#pragma unroll
      for (int i = TPG - 1; i >= 0; --i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          KtilT.store(8 * cg8 + j, tg * TPG + i, es[j] * kv[i][j]);  // Gamma_C / Gamma_r
          es[j] *= av[i][j];
        }
      }
    }
    prefetch(cn, nb, tn, mn);  // next chunk, into the other register set
    __syncthreads();

    // ---- E = Khat S, O = Qhat S (chunk rows of this wave) ------------------
    f32x4 E = zero4(), O = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const auto B = Sop.load8(m, kb * 32 + 8 * g);
      P::mma(E, Khat.load8(rbase + m, kb * 32 + 8 * g), B);
      P::mma(O, Qhat.load8(rbase + m, kb * 32 + 8 * g), B);
    }
    {
      f32x4 vme;
#pragma unroll
      for (int i = 0; i < 4; ++i) vme[i] = s_v[(rbase + 4 * g + i) * 17 + m] - E[i];
      Vme.store4(m, rbase + 4 * g, vme);
    }
    __syncthreads();

    // ---- W = T (V - E) ------------------------------------------------------
    f32x4 W = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb < nkb) {
        const float x[8] = {tu[2 * kb].x, tu[2 * kb].y, tu[2 * kb].z, tu[2 * kb].w,
                            tu[2 * kb + 1].x, tu[2 * kb + 1].y, tu[2 * kb + 1].z, tu[2 * kb + 1].w};
        P::mma(W, P::make(x), Vme.load8(m, kb * 32 + 8 * g));
      }
    }
    Wop.store4(m, rbase + 4 * g, W);
    __syncthreads();

    // ---- O += M W; store o ----------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb < nkb) {
        const float x[8] = {mu[2 * kb].x, mu[2 * kb].y, mu[2 * kb].z, mu[2 * kb].w,
                            mu[2 * kb + 1].x, mu[2 * kb + 1].y, mu[2 * kb + 1].z, mu[2 * kb + 1].w};
        P::mma(O, P::make(x), Wop.load8(m, kb * 32 + 8 * g));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 4 * g + i;
      if (r < nvalid) o[((t0 + r) * H + h) * D + col0 + m] = O[i];
    }

    // ---- S <- Diag(Gamma_C) S + Ktil^T W (this wave's state tiles) ------------
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + 4 * u;
      if (t < NTILE) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = s_gam[16 * t + 4 * g + i] * sreg[u][i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          P::mma(acc, KtilT.load8(16 * t + m, kb * 32 + 8 * g), Wop.load8(m, kb * 32 + 8 * g));
        sreg[u] = acc;
        Sop.store4(m, 16 * t + 4 * g, acc);
      }
    }
  };

  if (cbeg < cend) prefetch(cbeg, bufA, tA, mA);
  for (int64_t c = cbeg; c < cend; c += 2) {
    // The prefetch is unconditional (the last chunk re-reads itself) so
    // that every wait count stays exact.
    process(c, bufA, tA, mA, c + 1 < cend ? c + 1 : c, bufB, tB, mB);
    if (c + 1 >= cend) break;
    process(c + 1, bufB, tB, mB, c + 2 < cend ? c + 2 : c + 1, bufA, tA, mA);
  }

  if (S_T != nullptr) {
    float *STp = S_T + (size_t)pair * D * D;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + 4 * u;
      if (t < NTILE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) STp[(size_t)(16 * t + 4 * g + i) * D + col0 + m] = sreg[u][i];
      }
    }
  }
}

template <int D, typename TIn, typename P>
hipError_t launch_prefill_t(const kda_shape_t &s, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const int32_t *cu,
                            const float *S0, float *o, float *S_T, void *workspace,
                            hipStream_t stream, int phases) {
  char *ws = static_cast<char *>(workspace);
  int32_t *base = reinterpret_cast<int32_t *>(ws);
  float *mats = reinterpret_cast<float *>(ws + schedule_bytes(s));
  const int N = s.num_seqs, H = s.num_heads;
  const int64_t mc = max_chunks(s);
  const TIn *qp = static_cast<const TIn *>(q), *kp = static_cast<const TIn *>(k),
            *vp = static_cast<const TIn *>(v);
  hipError_t e = hipSuccess;
  if (phases & kPhaseLocal) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, cu, N, s.seq_len, base);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mc > 0) {
      hipLaunchKernelGGL((chunk_local_kernel<D, TIn, P>), dim3((unsigned)(mc * H)), dim3(NT), 0, stream,
                         qp, kp, alpha, beta, cu, s.seq_len, N, H, s.total_tokens, mc, base, mats);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (phases & kPhaseState) {
    const int64_t pairs = (int64_t)N * H;
    const int64_t blocks = (pairs + 7) / 8 * 8 * (D / 16);
    hipLaunchKernelGGL((chunk_state_kernel<D, TIn, P>), dim3((unsigned)blocks), dim3(NT), 0, stream, qp,
                       kp, vp, alpha, cu, s.seq_len, N, H, s.total_tokens, mc, base, mats, S0, o, S_T);
    e = hipGetLastError();
  }
  return e;
}

template <typename TIn>
hipError_t dispatch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const int32_t *cu,
                            const float *S0, float *o, float *S_T, void *ws, hipStream_t st,
                            int ph) {
  // bf16 inputs run the split-bf16 matrix-core path; fp32 inputs (and the
  // 16-wide heads) the fp32 matrix-core path.
  using PB = typename std::conditional<std::is_same<TIn, __bf16>::value, SplitBF16, F32>::type;
  switch (s.d_k) {
    case 16: return launch_prefill_t<16, TIn, F32>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, st, ph);
    case 32: return launch_prefill_t<32, TIn, PB>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, st, ph);
    case 64: return launch_prefill_t<64, TIn, PB>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, st, ph);
    case 128: return launch_prefill_t<128, TIn, PB>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, st, ph);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          const float *S0, float *o, float *S_T, void *workspace,
                          hipStream_t stream, int phases) {
  if (s.qkv_dtype == KDA_BF16)
    return dispatch_prefill<__bf16>(s, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, stream,
                                    phases);
  return dispatch_prefill<float>(s, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, stream,
                                 phases);
}

}  // namespace kda
