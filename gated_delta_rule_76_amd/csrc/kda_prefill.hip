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
  template <int N>
  __device__ __forceinline__ void store_run(int r, int c, const float (&x)[N]) {
    if constexpr (N == 4) {
      f32x4 v;
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
      store4(r, c, v);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) store(r, c + i, x[i]);
    }
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
  template <int N>
  __device__ __forceinline__ void store_run(int r, int c, const float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) store(r, c + i, x[i]);
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
// Chunk records: per (chunk, head), operand fragments in the order the state
// pass consumes them.  Records are head-major (record h * max_chunks + c), so
// the chunks one state-pass workgroup walks through are contiguous in memory.  A fragment is one 16-row x 32-column operand block of
// the matrix-core product (lane 16g+m holds row m, columns 8g..8g+7), 2 KiB:
// for SplitBF16 the bf16 hi plane (lane l at byte 16 l) then the lo plane
// (at 1024 + 16 l); for F32 eight floats per lane (at byte 32 l).
// ---------------------------------------------------------------------------
struct FragRaw {
  uint4 a, b;
};

template <typename P>
struct FragIO;

template <>
struct FragIO<SplitBF16> {
  __device__ __forceinline__ static void store(char *blk, int lane, const float (&x)[8]) {
    bf16x8 h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = (__bf16)x[j];
      l[j] = (__bf16)(x[j] - (float)h[j]);
    }
    *reinterpret_cast<bf16x8 *>(blk + 16 * lane) = h;
    *reinterpret_cast<bf16x8 *>(blk + 1024 + 16 * lane) = l;
  }
  __device__ __forceinline__ static void store_frag(char *blk, int lane, const SplitBF16::Frag &f) {
    *reinterpret_cast<bf16x8 *>(blk + 16 * lane) = f.hi;
    *reinterpret_cast<bf16x8 *>(blk + 1024 + 16 * lane) = f.lo;
  }
  __device__ __forceinline__ static void load(FragRaw &r, const char *blk, int lane) {
    r.a = *reinterpret_cast<const uint4 *>(blk + 16 * lane);
    r.b = *reinterpret_cast<const uint4 *>(blk + 1024 + 16 * lane);
  }
  __device__ __forceinline__ static SplitBF16::Frag frag(const FragRaw &r) {
    SplitBF16::Frag f;
    f.hi = __builtin_bit_cast(bf16x8, r.a);
    f.lo = __builtin_bit_cast(bf16x8, r.b);
    return f;
  }
};

template <>
struct FragIO<F32> {
  __device__ __forceinline__ static void store(char *blk, int lane, const float (&x)[8]) {
    *reinterpret_cast<float4 *>(blk + 32 * lane) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(blk + 32 * lane + 16) = make_float4(x[4], x[5], x[6], x[7]);
  }
  __device__ __forceinline__ static void store_frag(char *blk, int lane, const F32::Frag &f) {
    *reinterpret_cast<float4 *>(blk + 32 * lane) = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
    *reinterpret_cast<float4 *>(blk + 32 * lane + 16) = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
  }
  __device__ __forceinline__ static void load(FragRaw &r, const char *blk, int lane) {
    r.a = *reinterpret_cast<const uint4 *>(blk + 32 * lane);
    r.b = *reinterpret_cast<const uint4 *>(blk + 32 * lane + 16);
  }
  __device__ __forceinline__ static F32::Frag frag(const FragRaw &r) {
    F32::Frag f;
    const float4 a = __builtin_bit_cast(float4, r.a), b = __builtin_bit_cast(float4, r.b);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
};

// hi*b + lo*b for an operand b that is exact in bf16 (v in bf16): the lo part
// of b is zero, so the hi*lo term is skipped.
__device__ __forceinline__ void mma_exact_b(f32x4 &acc, const SplitBF16::Frag &a, const SplitBF16::Frag &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_exact_b(f32x4 &acc, const F32::Frag &a, const F32::Frag &b) {
  F32::mma(acc, a, b);
}

// Fragment indices inside one record.
template <int D>
struct Rec {
  static constexpr int NKB = (D < 32 ? 32 : D) / 32;  // k-blocks over key channels
  static constexpr int NTILE = D / 16;                 // 16-row tiles of key channels
  static constexpr int KHAT = 0;                       // Khat        [row tile][kb]
  static constexpr int QHAT = 4 * NKB;                 // Qhat        [row tile][kb]
  static constexpr int PMAT = 8 * NKB;                 // Ktil^T T    [channel tile][kb of tokens]
  static constexpr int MTM = 8 * NKB + 2 * NTILE;      // M T         non-zero [row tile][kb], 6 blocks
  static constexpr int NFRAG = MTM + 6;
  static constexpr size_t GAM = (size_t)NFRAG * kFragBytes;  // Gamma_C (D floats)
  static constexpr size_t BYTES = (GAM + sizeof(float) * D + kWorkspaceAlign - 1) / kWorkspaceAlign *
                                  kWorkspaceAlign;
  // M T is lower triangular: row tiles 0 and 1 have k-block 0 only.
  __device__ __forceinline__ static int mt_frag(int rt, int kb) { return rt < 2 ? rt : 2 * rt - 2 + kb; }
};

// ---------------------------------------------------------------------------
// chunk_local_kernel: every operand of one chunk and head, computed once.
//
// Wave w holds 16-token block w in registers (lane: TPG consecutive tokens,
// 8 consecutive key channels).  Decay factors are running products of alpha:
// inside a lane, across the block's lanes (shuffles) and across blocks (one
// LDS exchange of the four block totals).
//
// Gram tiles (R, J), J <= R, of A and M over key channels, per channel:
//   Gamma_r / Gamma_j = bp_r bs_j prod_{J<b<R} bt_b      (J < R)
//                     = bp_r / bp_j                      (J = R, j <= r)
// with bp the product from the block start to r, bs the product after j to
// the block end, bt block totals; the in-between block totals are folded
// into the B operand (three extra row blocks).  1/bp is used only when every
// channel's block total is >= 2^-100; otherwise the block's diagonal tiles
// are recomputed directly from running products of alpha.
//
// Then L = I + Diag(beta) A, X = L^-1 (blocked forward substitution in fp32),
// T = X Diag(beta), -T Khat on the matrix cores, and every operand is written
// to the record as fragments.
// ---------------------------------------------------------------------------
template <int D>
struct PrepCfg {
  static constexpr int CGR = D / 8;                               // 8-channel groups per token
  static constexpr int LPB = (64 / CGR) < 16 ? 64 / CGR : 16;     // token lanes per block
  static constexpr int TPG = 16 / LPB;                            // tokens per lane
  static constexpr int ACT = CGR * LPB;                           // active lanes per wave
  static constexpr int DK = D < 32 ? 32 : D;
  static constexpr int PW = DK < 64 ? DK : 64;                    // channels per Gram pass
  static constexpr int NPASS = DK / PW;
  static constexpr int MP = C + 1;
  static_assert(ACT <= 64 && LPB * TPG == 16, "lane layout");
};

// Tiles per wave (5 each): waves 0/1 take block-row 3 plus tile (0,0) of
// A / M, waves 2/3 take block-rows 2 and 1 of A / M.
__device__ __forceinline__ int tile_R(int tsel, int t) { return tsel == 0 ? (t < 4 ? 3 : 0) : (t < 3 ? 2 : 1); }
__device__ __forceinline__ int tile_J(int tsel, int t) { return tsel == 0 ? (t < 4 ? t : 0) : (t < 3 ? t : t - 3); }

template <int D, typename P>
struct PrepLds {
  using Cf = PrepCfg<D>;
  // Gram pass (region G) and output staging (region O) share one buffer.
  struct Gram {
    Plane<P, C, Cf::PW> ka, qa, kb, ki;           // k bp, q bp, k bs, k / bp  (rows = tokens)
    Plane<P, 16, Cf::PW> e0a, e0b, e1;             // block 0 rows x bt1, x bt1 bt2; block 1 x bt2
  };
  struct Out {
    float qn[C * (Cf::DK + 4)];                    // token-major fp32: Qhat, then Khat
    Plane<P, D, C> kt;                             // Ktil^T (rows = channels), then Ktil^T T in fp32
  };
  static_assert(sizeof(Plane<P, D, C>) >= sizeof(float) * D * (C + 4), "Ktil^T T staging");
  static constexpr size_t U = sizeof(Gram) > sizeof(Out) ? sizeof(Gram) : sizeof(Out);
};

template <int D, typename TIn, typename P>
__global__ __launch_bounds__(NT) void chunk_local_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t max_chunks, const int32_t *__restrict__ base, char *__restrict__ recs) {
  using Cf = PrepCfg<D>;
  using Rc = Rec<D>;
  using L = PrepLds<D, P>;
  using IO = FragIO<P>;
  constexpr int CGR = Cf::CGR, LPB = Cf::LPB, TPG = Cf::TPG, DK = Cf::DK, PW = Cf::PW, MP = Cf::MP;
  constexpr int QP = DK + 4;  // pitch of qn

  __shared__ __attribute__((aligned(16))) char s_u[L::U];
  __shared__ float s_L[C * MP], s_M[C * MP], s_X[C * MP];
  __shared__ float s_Y[3 * 16 * 17];
  __shared__ float s_beta[C];
  __shared__ __attribute__((aligned(16))) float s_bt[4 * D];
  __shared__ int s_flag[4];
  auto &G = *reinterpret_cast<typename L::Gram *>(s_u);
  auto &O = *reinterpret_cast<typename L::Out *>(s_u);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int64_t c = (int64_t)(blockIdx.x / H);
  const int h = blockIdx.x % H;
  const int64_t nchunks = base[N] < max_chunks ? (int64_t)base[N] : max_chunks;
  if (c >= nchunks || total_tokens <= 0) return;
  const int n = find_seq(base, N, c);
  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const ChunkTok ct = chunk_tokens(sstart, slen, c - base[n], total_tokens);
  const int64_t t0 = ct.t0;
  const int nvalid = ct.valid;
  char *rec = recs + ((size_t)h * max_chunks + c) * Rc::BYTES;

  // ---- P1: loads (unconditional 16-byte vector loads, clamped rows) ----------
  const int cgl = lane % CGR, tgl = lane / CGR;
  const bool act = lane < Cf::ACT;
  const int r0 = 16 * wave + TPG * tgl;  // first token row of this lane
  Raw8<TIn> kr[TPG], qr[TPG];
  float4 ar0[TPG], ar1[TPG];
  if (act) {
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int64_t off = (load_token(t0, r0 + i, nvalid, total_tokens) * H + h) * D + 8 * cgl;
      kr[i].load(k + off);
      qr[i].load(q + off);
      ar0[i] = *reinterpret_cast<const float4 *>(alpha + off);
      ar1[i] = *reinterpret_cast<const float4 *>(alpha + off + 4);
    }
  }
  if (tid < C) {
    const float bv = beta[load_token(t0, tid, nvalid, total_tokens) * H + h];
    s_beta[tid] = tid < nvalid ? bv : 0.f;
  }
  for (int e = tid; e < C * MP; e += NT) {
    s_L[e] = 0.f;
    s_M[e] = 0.f;
    s_X[e] = 0.f;
  }
  if (tid < 4) s_flag[tid] = 0;

  // ---- P2: block-local decay products ----------------------------------------
  float kv[TPG][8], qv[TPG][8], bp[TPG][8], bs[TPG][8], bt[8];
  bool tiny = false;
  if (act) {
    float av[TPG][8], lt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) lt[j] = 1.f;
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const bool ok = r0 + i < nvalid;
      kr[i].to_f32(kv[i]);
      qr[i].to_f32(qv[i]);
      const float a[8] = {ar0[i].x, ar0[i].y, ar0[i].z, ar0[i].w, ar1[i].x, ar1[i].y, ar1[i].z, ar1[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[i][j] = ok ? a[j] : 1.f;
        kv[i][j] = ok ? kv[i][j] : 0.f;
        qv[i][j] = ok ? qv[i][j] : 0.f;
        lt[j] *= av[i][j];
        bp[i][j] = lt[j];  // prefix inside the lane, completed below
      }
    }
    float y[8], z[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = z[j] = lt[j];
#pragma unroll
    for (int st = 1; st < LPB; st <<= 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = __shfl_up(y[j], CGR * st);
        const float d = __shfl_down(z[j], CGR * st);
        if (tgl >= st) y[j] *= u;
        if (tgl + st < LPB) z[j] *= d;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = __shfl_up(y[j], CGR);
      const float d = __shfl_down(z[j], CGR);
      const float ex = tgl >= 1 ? u : 1.f;       // earlier lanes of the block
      const float sx = tgl + 1 < LPB ? d : 1.f;  // later lanes of the block
      bt[j] = __shfl(y[j], (LPB - 1) * CGR + cgl);
      float suf = sx;
#pragma unroll
      for (int i = TPG - 1; i >= 0; --i) {
        bs[i][j] = suf;  // product after token i to the block end
        suf *= av[i][j];
        bp[i][j] *= ex;  // product from the block start to token i
      }
      tiny = tiny || !(bt[j] >= kTinyBlock);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) bt[j] = 1.f;
  }
  const bool block_tiny = __ballot(tiny) != 0;
  if (lane == 0 && block_tiny) s_flag[wave] = 1;
  if (act && tgl == 0) {
    *reinterpret_cast<float4 *>(&s_bt[wave * D + 8 * cgl]) = make_float4(bt[0], bt[1], bt[2], bt[3]);
    *reinterpret_cast<float4 *>(&s_bt[wave * D + 8 * cgl + 4]) = make_float4(bt[4], bt[5], bt[6], bt[7]);
  }
  __syncthreads();

  // ---- P3: factors from the other blocks ---------------------------------------
  float before[8], after[8], bt1[8], bt2[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) before[j] = after[j] = bt1[j] = bt2[j] = 1.f;
  if (act) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float4 u0 = *reinterpret_cast<const float4 *>(&s_bt[b * D + 8 * cgl]);
      const float4 u1 = *reinterpret_cast<const float4 *>(&s_bt[b * D + 8 * cgl + 4]);
      const float tv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b < wave) before[j] *= tv[j];
        if (b > wave) after[j] *= tv[j];
        if (b == 1) bt1[j] = tv[j];
        if (b == 2) bt2[j] = tv[j];
      }
    }
  }

  // ---- P4: decayed Gram tiles on the matrix cores ----------------------------
  const int tsel = wave >> 1;
  const bool isM = (wave & 1) != 0;
  f32x4 acc[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) acc[t] = zero4();
#pragma unroll
  for (int p = 0; p < Cf::NPASS; ++p) {
    if constexpr (DK > D) {  // channels past D are zero in every operand
      for (int e = tid; e < C * (DK - D); e += NT) {
        const int r = e / (DK - D), cc = D + e % (DK - D);
        G.ka.store(r, cc, 0.f);
        G.qa.store(r, cc, 0.f);
        G.kb.store(r, cc, 0.f);
        G.ki.store(r, cc, 0.f);
        if (r < 16) {
          G.e0a.store(r, cc, 0.f);
          G.e0b.store(r, cc, 0.f);
          G.e1.store(r, cc, 0.f);
        }
      }
    }
    const int c8 = 8 * cgl - p * PW;
    if (act && c8 >= 0 && c8 < PW) {
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        float xa[8], xq[8], xb[8], xi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xa[j] = kv[i][j] * bp[i][j];
          xq[j] = qv[i][j] * bp[i][j];
          xb[j] = kv[i][j] * bs[i][j];
          xi[j] = block_tiny ? 0.f : kv[i][j] * __builtin_amdgcn_rcpf(bp[i][j]);
        }
        const int r = r0 + i;
        G.ka.store8(r, c8, xa);
        G.qa.store8(r, c8, xq);
        G.kb.store8(r, c8, xb);
        G.ki.store8(r, c8, xi);
        if (wave == 0) {
          float x1[8], x2[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x1[j] = xb[j] * bt1[j];
            x2[j] = x1[j] * bt2[j];
          }
          G.e0a.store8(r, c8, x1);
          G.e0b.store8(r, c8, x2);
        } else if (wave == 1) {
          float x1[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x1[j] = xb[j] * bt2[j];
          G.e1.store8(r - 16, c8, x1);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const int R = tile_R(tsel, t), J = tile_J(tsel, t);
#pragma unroll
      for (int kb = 0; kb < PW / 32; ++kb) {
        const int col = kb * 32 + 8 * g;
        const auto A = isM ? G.qa.load8(16 * R + m, col) : G.ka.load8(16 * R + m, col);
        typename P::Frag B;
        if (J == R)
          B = G.ki.load8(16 * J + m, col);
        else if (J == R - 1)
          B = G.kb.load8(16 * J + m, col);
        else if (J == R - 2)
          B = J == 0 ? G.e0a.load8(m, col) : G.e1.load8(m, col);
        else
          B = G.e0b.load8(m, col);
        P::mma(acc[t], A, B);
      }
    }
    __syncthreads();
  }

  // ---- P5: L = I + Diag(beta) A (strictly lower part) and M ----------------------
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const int R = tile_R(tsel, t), J = tile_J(tsel, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * R + 4 * g + i, j = 16 * J + m;
      if (isM)
        s_M[r * MP + j] = (j <= r) ? acc[t][i] : 0.f;
      else
        s_L[r * MP + j] = (j < r) ? acc[t][i] * s_beta[r] : 0.f;
    }
  }
  __syncthreads();

  // Rare path: a 16-token block whose decay underflows 2^-100 in some
  // channel.  Its diagonal tiles of A and M, directly:
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
      s_L[rr * MP + jj] = (j < r) ? a_acc * s_beta[rr] : 0.f;
      s_M[rr * MP + jj] = m_acc;
    }
    __syncthreads();
  }

  // ---- P6: X = L^-1, blocked by 16 ---------------------------------------------
  // Diagonal blocks: forward substitution, one column per lane (wave b
  // inverts block b).
  if (lane < 16) {
    const int b = wave, jj = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) s -= s_L[(16 * b + i) * MP + 16 * b + t] * x[t];
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
        for (int t = 0; t < 16; ++t) s += s_L[(16 * I + rr) * MP + 16 * K + t] * s_X[(16 * K + t) * MP + 16 * J + cc];
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

  // ---- P7: records ------------------------------------------------------------------
  // T = X Diag(beta) is lower triangular; the products Ktil^T T and M T use
  // its column tile ct against token k-block kb only where that block meets
  // rows >= 16 ct: (ct, kb) in {(0,0), (0,1), (1,0), (1,1), (2,1), (3,1)}.
  // Qhat (token-major, fp32) and Ktil^T (channel-major, operand form) to LDS.
  if constexpr (DK > D) {
    for (int e = tid; e < C * (DK - D); e += NT) O.qn[(e / (DK - D)) * QP + D + e % (DK - D)] = 0.f;
  }
  if (act) {
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      float xq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xq[j] = before[j] * bp[i][j] * qv[i][j];  // Gamma_r q_r
      *reinterpret_cast<float4 *>(&O.qn[(r0 + i) * QP + 8 * cgl]) = make_float4(xq[0], xq[1], xq[2], xq[3]);
      *reinterpret_cast<float4 *>(&O.qn[(r0 + i) * QP + 8 * cgl + 4]) = make_float4(xq[4], xq[5], xq[6], xq[7]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float xk[TPG];
#pragma unroll
      for (int i = 0; i < TPG; ++i) xk[i] = bs[i][j] * after[j] * kv[i][j];  // (Gamma_C / Gamma_r) k_r
      O.kt.template store_run<TPG>(8 * cgl + j, r0, xk);
    }
  }
  __syncthreads();
  // Qhat fragments.
#pragma unroll
  for (int kb = 0; kb < Rc::NKB; ++kb) {
    float x[8];
    const float4 u0 = *reinterpret_cast<const float4 *>(&O.qn[(16 * wave + m) * QP + kb * 32 + 8 * g]);
    const float4 u1 = *reinterpret_cast<const float4 *>(&O.qn[(16 * wave + m) * QP + kb * 32 + 8 * g + 4]);
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
    x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
    IO::store(rec + (size_t)(Rc::QHAT + Rc::NKB * wave + kb) * kFragBytes, lane, x);
  }
  // T as a B operand for the six (ct, kb) blocks: rows kb*32 + 8g + j, column 16 ct + m.
  typename P::Frag tb[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int ct = u < 4 ? u >> 1 : u - 2, kb = u < 4 ? u & 1 : 1;
    const float bc = s_beta[16 * ct + m];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s_X[(kb * 32 + 8 * g + j) * MP + 16 * ct + m] * bc;
    tb[u] = P::make(x);
  }
  // Ktil^T T for channel tiles wave, wave + 4 (all four column tiles).
  constexpr int PT = (Rc::NTILE + 3) / 4;
  f32x4 pacc[PT][4];
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) pacc[tt][ct] = zero4();
    const int t = wave + 4 * tt;
    if (t < Rc::NTILE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const auto A = O.kt.load8(16 * t + m, kb * 32 + 8 * g);
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int ct = u < 4 ? u >> 1 : u - 2, ukb = u < 4 ? u & 1 : 1;
          if (ukb == kb) P::mma(pacc[tt][ct], A, tb[u]);
        }
      }
    }
  }
  // M T for row tile wave: column tiles ct <= wave, k-blocks ct/2 .. wave/2.
  f32x4 macc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) macc[ct] = zero4();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (kb <= (wave >> 1)) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s_M[(16 * wave + m) * MP + kb * 32 + 8 * g + j];
      const auto A = P::make(x);
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int ct = u < 4 ? u >> 1 : u - 2, ukb = u < 4 ? u & 1 : 1;
        if (ukb == kb && ct <= wave) P::mma(macc[ct], A, tb[u]);
      }
    }
  }
  __syncthreads();  // Qhat and Ktil^T consumed
  // Khat (token-major) into qn; Ktil^T T (channel-major fp32) over the kt
  // plane; M T into s_L (its strictly upper blocks stay zero from the start).
  float *pm = reinterpret_cast<float *>(&O.kt);
  constexpr int PP = C + 4;
  if (act) {
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      float xk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xk[j] = before[j] * bp[i][j] * kv[i][j];  // Gamma_r k_r
      *reinterpret_cast<float4 *>(&O.qn[(r0 + i) * QP + 8 * cgl]) = make_float4(xk[0], xk[1], xk[2], xk[3]);
      *reinterpret_cast<float4 *>(&O.qn[(r0 + i) * QP + 8 * cgl + 4]) = make_float4(xk[4], xk[5], xk[6], xk[7]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    const int t = wave + 4 * tt;
    if (t < Rc::NTILE) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[(16 * t + 4 * g + i) * PP + 16 * ct + m] = pacc[tt][ct][i];
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    if (ct <= wave) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_L[(16 * wave + 4 * g + i) * MP + 16 * ct + m] = macc[ct][i];
    }
  }
  __syncthreads();
  // Khat, Ktil^T T and M T fragments; Gamma_C.
#pragma unroll
  for (int kb = 0; kb < Rc::NKB; ++kb) {
    float x[8];
    const float4 u0 = *reinterpret_cast<const float4 *>(&O.qn[(16 * wave + m) * QP + kb * 32 + 8 * g]);
    const float4 u1 = *reinterpret_cast<const float4 *>(&O.qn[(16 * wave + m) * QP + kb * 32 + 8 * g + 4]);
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
    x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
    IO::store(rec + (size_t)(Rc::KHAT + Rc::NKB * wave + kb) * kFragBytes, lane, x);
  }
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    const int t = wave + 4 * tt;
    if (t < Rc::NTILE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
        const float4 u0 = *reinterpret_cast<const float4 *>(&pm[(16 * t + m) * PP + kb * 32 + 8 * g]);
        const float4 u1 = *reinterpret_cast<const float4 *>(&pm[(16 * t + m) * PP + kb * 32 + 8 * g + 4]);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
        x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
        IO::store(rec + (size_t)(Rc::PMAT + 2 * t + kb) * kFragBytes, lane, x);
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (kb <= (wave >> 1)) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s_L[(16 * wave + m) * MP + kb * 32 + 8 * g + j];
      IO::store(rec + (size_t)(Rc::MTM + Rc::mt_frag(wave, kb)) * kFragBytes, lane, x);
    }
  }
  if (wave == 0 && act && tgl == 0) {
    float *gam = reinterpret_cast<float *>(rec + Rc::GAM);
    *reinterpret_cast<float4 *>(gam + 8 * cgl) =
        make_float4(bt[0] * after[0], bt[1] * after[1], bt[2] * after[2], bt[3] * after[3]);
    *reinterpret_cast<float4 *>(gam + 8 * cgl + 4) =
        make_float4(bt[4] * after[4], bt[5] * after[5], bt[6] * after[6], bt[7] * after[7]);
  }
}

// ---------------------------------------------------------------------------
// chunk_state_kernel: the sequential pass over the chunks of one sequence for
// one head and 16 value columns, streaming the records.
//
// Eight waves; wave w has row tile rt = w mod 4 (chunk rows 16 rt..+15) and
// owns state row tile w.  Waves 0-3 ("U waves") and 4-7 ("O waves") split
// the two products with S.  Per chunk, with S the d x 16 state slice (fp32
// accumulators, kept across chunks):
//   U waves:  U = V - Khat S       (their row tile; to LDS in operand form)
//   O waves:  O = Qhat S
//   --- barrier ---
//   all:      S <- Diag(Gamma_C) S + (Ktil^T T) U     (state tile w; to LDS)
//   O waves:  o = O + (M T) U
//   --- barrier ---
// Each record fragment is read by one wave of the workgroup.  The record of
// chunk c+1 is loaded into the other register set while chunk c computes
// (the loop is unrolled by two so no copy sits between a load and its use).
//
// blockIdx -> work: consecutive workgroups are dealt round-robin to the 8
// XCDs, so the d/16 workgroups of one (sequence, head) get block indices
// congruent mod 8: they share an XCD and its L2, and every record is fetched
// from HBM once for all of them.
// ---------------------------------------------------------------------------
template <int D>
struct ScanCfg {
  static constexpr int NW = 8;                   // waves per workgroup
  static constexpr int NTH = 64 * NW;
  static constexpr int VW = 16;                  // value columns per workgroup
  static constexpr int G = D / VW;               // workgroups per (sequence, head)
  static constexpr int NKB = Rec<D>::NKB;
  static constexpr int NTILE = Rec<D>::NTILE;    // state row tiles
  static_assert(NTILE <= NW, "shape");
};

template <int D, typename TIn>
struct ScanBuf {
  using Cf = ScanCfg<D>;
  TIn v[4];                 // U waves: V rows 16 rt + 4 g + i, column m
  FragRaw mt[2];            // O waves: M T, row tile rt
  FragRaw a[Cf::NKB];       // Khat (U waves) or Qhat (O waves), row tile rt
  FragRaw p[2];             // Ktil^T T, state tile = wave
  float4 gam;               // Gamma_C, rows of state tile = wave
  uint32_t tch;             // one word of a record two chunks ahead
};

// Loads of one record, in two groups issued in the two phases of the
// previous chunk: the row-tile operands (group 0) and the rest (group 1).
template <int D, typename TIn, typename P>
__device__ __forceinline__ void load_scan_a(ScanBuf<D, TIn> &B, int kk, const char *rec, int wave, int lane,
                                            int rot) {
  using Cf = ScanCfg<D>;
  using Rc = Rec<D>;
  // The workgroups of one head read the same record at the same time; each
  // starts at a different k-block (register slot kk holds k-block
  // (kk + rot) mod NKB).
  const int rt = wave & 3;
  const int abase = wave < 4 ? Rc::KHAT : Rc::QHAT;
  const int kb = (kk + rot) % Cf::NKB;
  FragIO<P>::load(B.a[kk], rec + (size_t)(abase + Cf::NKB * rt + kb) * kFragBytes, lane);
}

template <int D, typename TIn, typename P>
__device__ __forceinline__ void load_scan_b(ScanBuf<D, TIn> &B, const char *rec, const TIn *v,
                                            int64_t vt0, int valid, int64_t total, int h, int H,
                                            int col0, int wave, int lane) {
  using Cf = ScanCfg<D>;
  using Rc = Rec<D>;
  using IO = FragIO<P>;
  // Both roles issue the same loads (V is used by the U waves, M T by the
  // O waves; the partner wave of the same row tile reads the same M T lines):
  // no branch separates the loads, so none of them has to be waited for early.
  const int rt = wave & 3, g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) B.v[i] = v[(load_token(vt0, 16 * rt + 4 * g + i, valid, total) * H + h) * D + col0 + m];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int f = Rc::mt_frag(rt, rt < 2 ? 0 : kb);  // row tiles 0, 1: the k-block 0 block twice
    IO::load(B.mt[kb], rec + (size_t)(Rc::MTM + f) * kFragBytes, lane);
  }
  const int t = wave < Cf::NTILE ? wave : Cf::NTILE - 1;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) IO::load(B.p[kb], rec + (size_t)(Rc::PMAT + 2 * t + kb) * kFragBytes, lane);
  B.gam = *reinterpret_cast<const float4 *>(rec + Rc::GAM + sizeof(float) * (16 * t + 4 * g));
}

// Two waves per SIMD: the two register sets of record fragments take about
// half of each wave's 256 registers.
template <int D, typename TIn, typename P>
__global__ __launch_bounds__(ScanCfg<D>::NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk_state_kernel(
    const TIn *__restrict__ v, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t max_chunks, const int32_t *__restrict__ base,
    const char *__restrict__ recs, const float *__restrict__ S0, float *__restrict__ o,
    float *__restrict__ S_T) {
  using Cf = ScanCfg<D>;
  using Rc = Rec<D>;
  using IO = FragIO<P>;
  using Buf = ScanBuf<D, TIn>;
  constexpr int VW = Cf::VW, G = Cf::G, NKB = Cf::NKB, NTILE = Cf::NTILE, NTH = Cf::NTH;
  constexpr int DK = D < 32 ? 32 : D;

  __shared__ Plane<P, VW, DK> Sop;     // S^T in operand form (rows = value columns)
  __shared__ Plane<P, VW, C> Uop;      // U^T in operand form

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = wave & 3;
  const bool uwave = wave < 4;
  const int m = lane & 15, g = lane >> 4;

  const int id = blockIdx.x;
  const int xcd = id & 7, within = id >> 3;
  const int64_t pair = (int64_t)(within / G) * 8 + xcd;
  const int cg = within % G;
  if (pair >= (int64_t)N * H) return;
  const int n = (int)(pair / H), h = (int)(pair % H);
  const int col0 = VW * cg;

  if constexpr (DK > D) {
    for (int e = tid; e < VW * (DK - D); e += NTH) Sop.store(e / (DK - D), D + e % (DK - D), 0.f);
  }
  f32x4 sreg = zero4();
  const float *S0p = S0 ? S0 + (size_t)pair * D * D : nullptr;
  if (wave < NTILE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sreg[i] = S0p ? S0p[(size_t)(16 * wave + 4 * g + i) * D + col0 + m] : 0.f;
    Sop.store4(m, 16 * wave + 4 * g, sreg);
  }

  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const int64_t cbeg = base[n];
  int64_t cend = base[n + 1];
  if (cend > max_chunks) cend = max_chunks;
  if (total_tokens <= 0) cend = cbeg;

  auto rec_of = [&](int64_t cc) __attribute__((always_inline)) { return recs + ((size_t)h * max_chunks + cc) * Rc::BYTES; };
  // The workgroups of a head split the cache lines of the record two chunks
  // ahead and each reads one word per line, so that the record is in L2 by
  // the time all of them load it in full.
  constexpr int NLINE = (int)(Rc::BYTES / 128);
  constexpr int LPG = (NLINE + G - 1) / G;
  // (threads past the workgroup's share repeat its first line, so each line
  // costs one request)
  auto touch = [&](int64_t cc) __attribute__((always_inline)) {
    const int li = cg * LPG + (tid < LPG ? tid : 0);
    return *reinterpret_cast<const uint32_t *>(rec_of(cc) + 128 * (li < NLINE ? li : NLINE - 1));
  };
  uint32_t sink = 0;

  Buf bufA, bufB;
  auto prefetch_b = [&](int64_t cc, Buf &B) __attribute__((always_inline)) {
    const ChunkTok cn = chunk_tokens(sstart, slen, cc - cbeg, total_tokens);
    load_scan_b<D, TIn, P>(B, rec_of(cc), v, cn.t0, cn.valid, total_tokens, h, H, col0, wave, lane);
  };

  // The loads of the next record are spread over this chunk's two phases,
  // between its matrix-core products, so that each wave keeps computing
  // while its loads queue.
  auto process = [&](int64_t c, const Buf &U, Buf &Nx, int64_t cn) __attribute__((always_inline)) {
    const ChunkTok ct = chunk_tokens(sstart, slen, c - cbeg, total_tokens);
    const char *rn = rec_of(cn);  // unconditional (the last chunk re-reads itself)

    // Khat S (U waves) or Qhat S (O waves) for row tile rt.
    f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int kb = (kk + cg) % NKB;  // the k-block held in register slot kk
      const auto Bs = Sop.load8(m, kb * 32 + 8 * g);
      P::mma((kk & 1) ? acc1 : acc0, IO::frag(U.a[kk]), Bs);
      __builtin_amdgcn_sched_barrier(0);
      load_scan_a<D, TIn, P>(Nx, kk, rn, wave, lane, cg);
      __builtin_amdgcn_sched_barrier(0);
    }
    Nx.tch = touch(cn + 1 < cend ? cn + 1 : cn);
    f32x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = acc0[i] + acc1[i];
    if (uwave) {
      f32x4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        u[i] = (r < ct.valid ? to_f32(U.v[i]) : 0.f) - ov[i];
      }
      Uop.store4(m, 16 * rt + 4 * g, u);
    }
    __syncthreads();

    // U as an operand: rows kb*32 + 8g .. +7 of column m.
    const auto u0 = Uop.load8(m, 8 * g);
    const auto u1 = Uop.load8(m, 32 + 8 * g);
    // S <- Diag(Gamma_C) S + (Ktil^T T) U
    if (wave < NTILE) {
      const float gm[4] = {U.gam.x, U.gam.y, U.gam.z, U.gam.w};
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = gm[i] * sreg[i];
      P::mma(acc, IO::frag(U.p[0]), u0);
      P::mma(acc, IO::frag(U.p[1]), u1);
      sreg = acc;
      Sop.store4(m, 16 * wave + 4 * g, acc);
    }
    // o = Qhat S + (M T) U
    if (!uwave) {
      P::mma(ov, IO::frag(U.mt[0]), u0);
      if (rt >= 2) P::mma(ov, IO::frag(U.mt[1]), u1);
    }
    __builtin_amdgcn_sched_barrier(0);
    prefetch_b(cn, Nx);
    __builtin_amdgcn_sched_barrier(0);
    if (!uwave) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        if (r < ct.valid) o[((ct.t0 + r) * H + h) * D + col0 + m] = ov[i];
      }
    }
    sink += U.tch;
    __syncthreads();
  };

  if (cbeg < cend) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) load_scan_a<D, TIn, P>(bufA, kk, rec_of(cbeg), wave, lane, cg);
    prefetch_b(cbeg, bufA);
    bufA.tch = touch(cbeg);
  }
  __syncthreads();
  for (int64_t c = cbeg; c < cend; c += 2) {
    process(c, bufA, bufB, c + 1 < cend ? c + 1 : c);
    if (c + 1 >= cend) break;
    process(c + 1, bufB, bufA, c + 2 < cend ? c + 2 : c + 1);
  }
  if (N < 0) o[sink & 1] = 0.f;  // never taken (N >= 0): keeps the touches alive

  if (S_T != nullptr && wave < NTILE) {
    float *STp = S_T + (size_t)pair * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) STp[(size_t)(16 * wave + 4 * g + i) * D + col0 + m] = sreg[i];
  }
}

template <int D, typename TIn, typename P>
hipError_t launch_prefill_t(const kda_shape_t &s, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const int32_t *cu,
                            const float *S0, float *o, float *S_T, void *workspace,
                            hipStream_t stream, int phases) {
  char *ws = static_cast<char *>(workspace);
  int32_t *base = reinterpret_cast<int32_t *>(ws);
  char *recs = ws + schedule_bytes(s);
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
                         qp, kp, alpha, beta, cu, s.seq_len, N, H, s.total_tokens, mc, base, recs);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (phases & kPhaseState) {
    const int64_t pairs = (int64_t)N * H;
    const int64_t blocks = (pairs + 7) / 8 * 8 * ScanCfg<D>::G;
    hipLaunchKernelGGL((chunk_state_kernel<D, TIn, P>), dim3((unsigned)blocks), dim3(ScanCfg<D>::NTH), 0, stream,
                       vp, cu,
                       s.seq_len, N, H, s.total_tokens, mc, base, recs, S0, o, S_T);
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
