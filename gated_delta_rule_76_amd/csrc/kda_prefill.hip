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
// S_{r-1}); collecting the w_r gives the triangular system above).  The
// kernels use it re-associated, never forming W:
//
//   U = V - Khat S0,   O = Qhat S0 + (M T) U,   S_C = Diag(Gamma_C) S0 + (Ktil^T T) U
//
// so all that does not depend on S0 is computed once per chunk in parallel.
// A tail chunk is padded with alpha = 1, beta = 0, q = k = v = 0, which is an
// exact identity step.
//
// Three kernels; the last two run per stripe of W consecutive chunks in
// packed order (W follows from the workspace; with the recommended workspace
// the whole batch is one stripe):
//   schedule_kernel     varlen packing: chunk counts per sequence -> table
//                       of first-chunk indices (exclusive scan).
//   chunk_local_kernel  one workgroup per (chunk of the stripe, head), fully
//                       parallel (the stripe's last chunks first):
//                       A and M on the matrix cores, T by a blocked
//                       triangular inverse, Ktil^T T and M T on the matrix
//                       cores; writes the chunk's record (Khat, Qhat,
//                       Ktil^T T, M T, Gamma_C as operand fragments; with
//                       one rate per head and bf16 q/k, exact k and q and
//                       their per-token factors instead of Khat and Qhat).
//   chunk_state_kernel  one workgroup per (sequence, head, 16 or 32 value
//                       columns), sequential over the sequence's chunks in
//                       the stripe: the state slice stays in registers (fp32)
//                       across chunks and is handed to the next stripe
//                       through S_T (or a carry area); every product runs on
//                       the matrix cores with operands streamed from the
//                       records.
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
// Word 3 of a raw (stride 0) buffer descriptor: 32-bit data format; with it
// an access at an offset past num_records is dropped (stores) or reads 0.
constexpr int kBufferWord3 = 0x00020000;
// Busy state-pass workgroups of one 16-column tile above which the state
// pass takes two tiles per workgroup (the 256 CUs of the chip).
constexpr int64_t kStateWideAbove = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Pre-activation inputs (KDA_INPUT_PREACT): decay rate exp(-softplus(a)),
// written as 1 / (1 + e^a) (the same value; 0 for a -> +inf, 1 for
// a -> -inf), and update strength sigmoid(b).
__device__ __forceinline__ float decay_from_preact(float a) { return 1.f / (1.f + expf(a)); }
__device__ __forceinline__ float strength_from_preact(float b) { return 1.f / (1.f + expf(-b)); }
// 1 / max(||x||_2, 1e-12) from the sum of squares.
__device__ __forceinline__ float inv_norm(float ss) { return 1.f / fmaxf(sqrtf(ss), 1e-12f); }

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
  // Columns c0 + 4g .. +3 and c0 + 16 + 4g .. +3 of row r: the k-order of
  // fragments written from matrix-core accumulators.
  __device__ __forceinline__ SplitBF16::Frag load_acc_order(int r, int c0, int g) const {
    const bf16x4 h0 = *reinterpret_cast<const bf16x4 *>(&hi[r * PITCH + c0 + 4 * g]);
    const bf16x4 h1 = *reinterpret_cast<const bf16x4 *>(&hi[r * PITCH + c0 + 16 + 4 * g]);
    const bf16x4 l0 = *reinterpret_cast<const bf16x4 *>(&lo[r * PITCH + c0 + 4 * g]);
    const bf16x4 l1 = *reinterpret_cast<const bf16x4 *>(&lo[r * PITCH + c0 + 16 + 4 * g]);
    SplitBF16::Frag f;
    f.hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    f.lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
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
  __device__ __forceinline__ F32::Frag load_acc_order(int r, int c0, int g) const {
    F32::Frag fr;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(&f[r * PITCH + c0 + 4 * g]);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(&f[r * PITCH + c0 + 16 + 4 * g]);
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
// total chunks.  One workgroup; a block-wide scan per 1024 sequences.  Then
// order[0..N) = the sequences by descending chunk count (ties by index): the
// state pass deals its workgroups out in that order, so the longest chains
// start first and the short ones fill in behind them (longest-first list
// scheduling of the sequential per-sequence passes).  Batches of more than
// 1024 sequences keep the packed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ cu, int N,
                                                        int32_t seq_len, int32_t *__restrict__ base) {
  __shared__ int32_t s_scan[1024];
  __shared__ int32_t s_cnt[1024];
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
    s_cnt[tid] = cnt;
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
  int32_t *order = base + N + 1;
  if (N <= 1024) {
    // (s_cnt holds every sequence's count: one pass of the loop above)
    if (tid < N) {
      const int32_t mine = s_cnt[tid];
      int rank = 0;
      for (int m = 0; m < N; ++m) {
        const int32_t c = s_cnt[m];
        rank += (c > mine) || (c == mine && m < tid);
      }
      order[rank] = tid;
    }
  } else {
    for (int n = tid; n < N; n += 1024) order[n] = n;
  }
}

// A dense batch (no cu_seqlens) needs no table: every sequence has
// ceil(seq_len / 64) chunks, so base[n] = n * that.  The kernels compute it
// and the schedule kernel is not launched.
__device__ __forceinline__ int64_t dense_chunks(int32_t seq_len) {
  return seq_len > 0 ? ((int64_t)seq_len + C - 1) / C : 0;
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



// Packed chunks [first, first + count) of sequence n.
__device__ __forceinline__ void seq_chunk_range(const int32_t *cu, const int32_t *base, int32_t seq_len, int n,
                                                int64_t &first, int64_t &count) {
  if (cu == nullptr) {
    count = dense_chunks(seq_len);
    first = (int64_t)n * count;
  } else {
    first = base[n];
    count = (int64_t)base[n + 1] - first;
  }
}

// ---------------------------------------------------------------------------
// Chunk records: per (chunk, head), operand fragments in the order the state
// pass consumes them.  Records are head-major (slot h W + c - j0 for packed
// chunk c of the stripe that starts at j0), so the chunks one state-pass
// workgroup walks through are contiguous in memory.  A fragment is one 16-row x 32-column operand block of
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

// Byte offsets inside one record.
//
// EXACT (one decay rate per head, bf16 q/k, split-bf16 operands): Khat_r =
// Gamma_r k_r and Qhat_r = Gamma_r q_r are a per-token scalar times a row
// that is exact in bf16 (with pre-activation inputs the scalar also takes
// 1/||k_r|| or 1/||q_r||), so the record holds k and q as single bf16
// fragments (1 KiB) and the two per-token scalars, and the state pass scales
// the rows of Khat S and Qhat S by them: 32 KiB less record per chunk and
// two matrix-core products per k-block instead of three, with no rounding of
// Khat or Qhat.
template <int D, bool EXACT = false>
struct Rec {
  static constexpr int NKB = (D < 32 ? 32 : D) / 32;  // k-blocks over key channels
  static constexpr int NTILE = D / 16;                 // 16-row tiles of key channels
  static constexpr size_t AF = EXACT ? 1024 : kFragBytes;               // bytes of a Khat / Qhat fragment
  static constexpr size_t KHAT = 0;                                     // Khat   [row tile][kb]
  static constexpr size_t QHAT = KHAT + (size_t)4 * NKB * AF;           // Qhat   [row tile][kb]
  static constexpr size_t PMAT = QHAT + (size_t)4 * NKB * AF;           // Ktil^T T [channel tile][kb of tokens]
  static constexpr size_t MTM = PMAT + (size_t)2 * NTILE * kFragBytes;  // M T    non-zero [row tile][kb], 6 blocks
  static constexpr size_t GAM = MTM + (size_t)6 * kFragBytes;           // Gamma_C (D floats)
  static constexpr size_t RFAC = GAM + sizeof(float) * D;               // EXACT: per-token factors of k, then q
  static constexpr size_t BYTES = (RFAC + (EXACT ? 2 * C * sizeof(float) : 0) + kWorkspaceAlign - 1) /
                                  kWorkspaceAlign * kWorkspaceAlign;
  __device__ __forceinline__ static size_t khat(int rt, int kb) { return KHAT + (size_t)(NKB * rt + kb) * AF; }
  __device__ __forceinline__ static size_t qhat(int rt, int kb) { return QHAT + (size_t)(NKB * rt + kb) * AF; }
  __device__ __forceinline__ static size_t pmat(int t, int kb) { return PMAT + (size_t)(2 * t + kb) * kFragBytes; }
  // M T is lower triangular: row tiles 0 and 1 have k-block 0 only.
  __device__ __forceinline__ static size_t mtm(int rt, int kb) {
    return MTM + (size_t)(rt < 2 ? rt : 2 * rt - 2 + kb) * kFragBytes;
  }
};

// ---------------------------------------------------------------------------
// chunk_local_kernel: every operand of one chunk and head, computed once.
//
// Lane layout: wave w holds token block w (16 tokens) in the matrix-core
// operand layout, lane 16 g + m holding token 16 w + m and channels
// kb*32 + 8g .. +7 of every k-block kb (32 channels at d = 128).  The Gram
// operands of the wave's own block and the Khat and Qhat fragments of the
// record are therefore formed in registers and written without passing
// through LDS.
//
// Decay factors, per channel, as running products of alpha:
//   bp_r   product over the block up to and including token r
//   bs_r   product over the block after token r
//   bt_b   block totals; before / after = products of the totals of the
//          blocks before / after w
//   Gamma_r = before bp_r,   Gamma_C / Gamma_r = bs_r after.
// The in-block products are scans across the 16 lanes m of a row (DPP).
//
// Gram tiles (R, J <= R) of A (k against k) and M (q against k):
//   Gamma_r / Gamma_j = bp_r bs_j prod_{J<b<R} bt_b   (J < R)
//                     = bp_r / bp_j                   (J = R, j <= r)
// Wave R forms row block R from its A operands k bp and q bp and the B
// operands of block J: its own k / bp for J = R, else k bs times the
// in-between block totals, written to LDS by wave J.  1/bp is used only when
// every channel's block total is >= 2^-100; otherwise the block's diagonal
// tiles are recomputed directly.
//
// Then L = I + Diag(beta) A and X = L^-1 (diagonal blocks by forward
// substitution, the others by 16 x 16 block products on the fp32 matrix
// cores), T = X Diag(beta), and (Ktil^T T)^T = T^T Ktil and (M T)^T = T^T M^T
// on the matrix cores.  Their accumulators are written as operand fragments
// directly: lane (g, m) of output tiles 2kb and 2kb+1 holds row m at token
// columns 32kb + 4g + i and 32kb + 16 + 4g + i, which is the k-order the
// state pass uses for U.
// ---------------------------------------------------------------------------

// In-place products within 16-lane rows: x_m <- x_{m -/+ s} x_m.  Lanes whose
// source falls outside the row are disabled by the DPP operation and keep x.
// (The s_nop covers the wait states a DPP read needs after a VALU write.)
#define KDA_DPP_MUL4(CTRL, a, b, c, d)            \
  asm volatile("s_nop 1\n"                        \
               "v_mul_f32_dpp %0, %0, %0 " CTRL "\n" \
               "v_mul_f32_dpp %1, %1, %1 " CTRL "\n" \
               "v_mul_f32_dpp %2, %2, %2 " CTRL "\n" \
               "v_mul_f32_dpp %3, %3, %3 " CTRL "\n" \
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d))

// Inclusive prefix (y) and suffix (z) products across the 16 lanes of a row,
// for eight channels.
__device__ __forceinline__ void row_scans8(float (&y)[8], float (&z)[8]) {
  KDA_DPP_MUL4("row_shr:1", y[0], y[1], y[2], y[3]);
  KDA_DPP_MUL4("row_shr:1", y[4], y[5], y[6], y[7]);
  KDA_DPP_MUL4("row_shl:1", z[0], z[1], z[2], z[3]);
  KDA_DPP_MUL4("row_shl:1", z[4], z[5], z[6], z[7]);
  KDA_DPP_MUL4("row_shr:2", y[0], y[1], y[2], y[3]);
  KDA_DPP_MUL4("row_shr:2", y[4], y[5], y[6], y[7]);
  KDA_DPP_MUL4("row_shl:2", z[0], z[1], z[2], z[3]);
  KDA_DPP_MUL4("row_shl:2", z[4], z[5], z[6], z[7]);
  KDA_DPP_MUL4("row_shr:4", y[0], y[1], y[2], y[3]);
  KDA_DPP_MUL4("row_shr:4", y[4], y[5], y[6], y[7]);
  KDA_DPP_MUL4("row_shl:4", z[0], z[1], z[2], z[3]);
  KDA_DPP_MUL4("row_shl:4", z[4], z[5], z[6], z[7]);
  KDA_DPP_MUL4("row_shr:8", y[0], y[1], y[2], y[3]);
  KDA_DPP_MUL4("row_shr:8", y[4], y[5], y[6], y[7]);
  KDA_DPP_MUL4("row_shl:8", z[0], z[1], z[2], z[3]);
  KDA_DPP_MUL4("row_shl:8", z[4], z[5], z[6], z[7]);
}

// x_m <- z_{m+1} within each row, 1 for the last lane (exclusive suffix).
__device__ __forceinline__ void row_next8(float (&x)[8], const float (&z)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 1.f;
  asm volatile("s_nop 1\n"
               "v_mov_b32_dpp %0, %8 row_shl:1\n"
               "v_mov_b32_dpp %1, %9 row_shl:1\n"
               "v_mov_b32_dpp %2, %10 row_shl:1\n"
               "v_mov_b32_dpp %3, %11 row_shl:1\n"
               "v_mov_b32_dpp %4, %12 row_shl:1\n"
               "v_mov_b32_dpp %5, %13 row_shl:1\n"
               "v_mov_b32_dpp %6, %14 row_shl:1\n"
               "v_mov_b32_dpp %7, %15 row_shl:1\n"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
               : "v"(z[0]), "v"(z[1]), "v"(z[2]), "v"(z[3]), "v"(z[4]), "v"(z[5]), "v"(z[6]), "v"(z[7]));
}

// The same two scans and the exclusive suffix for one value per lane (a
// decay rate shared by every channel of the token).
__device__ __forceinline__ void row_scans1(float &y, float &z) {
  asm volatile("s_nop 1\n"
               "v_mul_f32_dpp %0, %0, %0 row_shr:1\n"
               "v_mul_f32_dpp %1, %1, %1 row_shl:1\n"
               "s_nop 1\n"
               "v_mul_f32_dpp %0, %0, %0 row_shr:2\n"
               "v_mul_f32_dpp %1, %1, %1 row_shl:2\n"
               "s_nop 1\n"
               "v_mul_f32_dpp %0, %0, %0 row_shr:4\n"
               "v_mul_f32_dpp %1, %1, %1 row_shl:4\n"
               "s_nop 1\n"
               "v_mul_f32_dpp %0, %0, %0 row_shr:8\n"
               "v_mul_f32_dpp %1, %1, %1 row_shl:8\n"
               : "+v"(y), "+v"(z));
}

__device__ __forceinline__ float row_next1(float z) {
  float x = 1.f;
  asm volatile("s_nop 1\n"
               "v_mov_b32_dpp %0, %1 row_shl:1\n"
               : "+v"(x)
               : "v"(z));
  return x;
}

template <int D>
struct LocCfg {
  static constexpr int DK = D < 32 ? 32 : D;
  static constexpr int NKB = DK / 32;
  static constexpr int MP = C + 1;   // pitch of s_X (fp32)
  static constexpr int LP = C + 4;   // pitch of s_L and s_M (fp32, 16-byte rows)
  static constexpr int KP = DK + 4;  // pitch of the token-major Ktil staging (fp32)
  // B-operand planes: k bs of blocks 0, 1, 2; block 0 times bt1 and times
  // bt1 bt2; block 1 times bt2.
  static constexpr int NPLANE = 6;
  static constexpr size_t GRAM = (size_t)2 * NPLANE * kFragBytes;  // one k-block, double-buffered
  static constexpr size_t LM = sizeof(float) * (2 * C * LP + 4 * 256);  // s_L, s_M, per-wave Y
  static constexpr size_t KT = sizeof(float) * C * KP;
  static constexpr size_t U = GRAM > LM ? (GRAM > KT ? GRAM : KT) : (LM > KT ? LM : KT);
};

// Plane holding the B operand of Gram tile (R, J < R).
__device__ __forceinline__ int gram_plane(int R, int J) {
  return R - J == 1 ? J : (R - J == 2 ? (J == 0 ? 3 : 5) : 4);
}

// T^T as an A operand for column tile ct and token k-block kb, for the six
// (ct, kb) blocks where T (lower triangular) can be non-zero.
__device__ __forceinline__ int tb_ct(int u) { return u < 4 ? u >> 1 : u - 2; }
__device__ __forceinline__ int tb_kb(int u) { return u < 4 ? u & 1 : 1; }

template <int D, typename TIn, typename P, int GATE, int FORM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void chunk_local_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ alpha,
    const float *__restrict__ beta, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t W, int64_t j0, const int32_t *__restrict__ base,
    char *__restrict__ recs) {
  using Cf = LocCfg<D>;
  // one rate per head with bf16 q/k: the record holds exact k and q (Rec)
  constexpr bool EXACT = GATE == KDA_GATE_HEAD && std::is_same<TIn, __bf16>::value &&
                         std::is_same<P, SplitBF16>::value;
  using Rc = Rec<D, EXACT>;
  using IO = FragIO<P>;
  using Frag = typename P::Frag;
  constexpr int DK = Cf::DK, NKB = Cf::NKB, MP = Cf::MP, LP = Cf::LP, KP = Cf::KP;

  __shared__ __attribute__((aligned(16))) char s_u[Cf::U];  // Gram planes; then L, M, Y; then Ktil
  __shared__ float s_X[C * MP];
  __shared__ __attribute__((aligned(16))) float s_bt[4 * DK];
  __shared__ float s_beta[C];
  __shared__ float s_inv[2][C];  // KDA_INPUT_PREACT: 1 / ||k||, 1 / ||q|| per token
  __shared__ int s_flag[4];
  float *s_L = reinterpret_cast<float *>(s_u);
  float *s_M = s_L + C * LP;
  float *s_kt = reinterpret_cast<float *>(s_u);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  float *s_Yw = s_M + C * LP + 256 * wave;
  // Work item: head h, packed chunk c = j0 + j of the stripe.  Workgroups
  // start in block order, so the stripe's chunks are taken last to first:
  // the records written last, which the XCD's L2 still holds when the state
  // pass starts, are those of the first chunks it reads (4k workload: state
  // pass 141 vs 144-147 us).
  const int h = (int)(blockIdx.x % (unsigned)H);
  const int64_t j = (int64_t)(gridDim.x / (unsigned)H) - 1 - (int64_t)(blockIdx.x / (unsigned)H);
  const int64_t c = j0 + j;
  if (total_tokens <= 0) return;
  int n;
  int64_t cfirst;  // first packed chunk of sequence n
  if (cu == nullptr) {
    const int64_t cps = dense_chunks(seq_len);
    if (c >= (int64_t)N * cps) return;
    n = (int)(c / cps);
    cfirst = n * cps;
  } else {
    if (c >= (int64_t)base[N]) return;
    n = find_seq(base, N, c);
    cfirst = base[n];
  }
  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const ChunkTok ct = chunk_tokens(sstart, slen, c - cfirst, total_tokens);
  const int64_t t0 = ct.t0;
  const int nvalid = ct.valid;
  char *rec = recs + ((size_t)h * W + j) * Rc::BYTES;

  // ---- loads: token 16 w + m, channels kb*32 + 8g .. +7 (rows past the
  // chunk and channels past d are padding: k = q = 0, alpha = 1) ------------
  const int r = 16 * wave + m;
  const bool rv = r < nvalid;
  const int64_t tok = load_token(t0, r, nvalid, total_tokens);
  // In the order of first use: beta (stored to LDS below, so waiting for it
  // must not wait for the rest), alpha (the scans), then k and q.
  const float bv = beta[load_token(t0, tid & (C - 1), nvalid, total_tokens) * H + h];
  Raw8<TIn> kr[NKB], qr[NKB];
  float4 ar0[NKB], ar1[NKB];
  float ah = 1.f;  // KDA_GATE_HEAD: the token's one rate
  if constexpr (GATE == KDA_GATE_HEAD) {
    ah = alpha[tok * H + h];
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int ch = kb * 32 + 8 * g;
      const int64_t off = (tok * H + h) * D + (ch < D ? ch : 0);
      ar0[kb] = *reinterpret_cast<const float4 *>(alpha + off);
      ar1[kb] = *reinterpret_cast<const float4 *>(alpha + off + 4);
    }
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int ch = kb * 32 + 8 * g;
    const int64_t off = (tok * H + h) * D + (ch < D ? ch : 0);
    kr[kb].load(k + off);
    qr[kb].load(q + off);
  }
  for (int e = tid; e < C * MP; e += NT) s_X[e] = 0.f;
  if (tid < C)
    s_beta[tid] = tid < nvalid ? (FORM == KDA_INPUT_PREACT ? strength_from_preact(bv) : bv) : 0.f;
  constexpr bool kPre = FORM == KDA_INPUT_PREACT;
  if constexpr (kPre) {
    if constexpr (GATE == KDA_GATE_HEAD) {
      ah = decay_from_preact(ah);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        ar0[kb].x = decay_from_preact(ar0[kb].x); ar0[kb].y = decay_from_preact(ar0[kb].y);
        ar0[kb].z = decay_from_preact(ar0[kb].z); ar0[kb].w = decay_from_preact(ar0[kb].w);
        ar1[kb].x = decay_from_preact(ar1[kb].x); ar1[kb].y = decay_from_preact(ar1[kb].y);
        ar1[kb].z = decay_from_preact(ar1[kb].z); ar1[kb].w = decay_from_preact(ar1[kb].w);
      }
    }
  }
  // Raw q and k are scaled to unit length: sums of squares over the lane's
  // channels, then over the four lanes (g) that share the token.
  float inv_k = 1.f, inv_q = 1.f;
  if constexpr (kPre) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb * 32 + 8 * g < D) {
        float t[8];
        kr[kb].to_f32(t);
#pragma unroll
        for (int j = 0; j < 8; ++j) sk += t[j] * t[j];
        qr[kb].to_f32(t);
#pragma unroll
        for (int j = 0; j < 8; ++j) sq += t[j] * t[j];
      }
    }
    sk += __shfl_xor(sk, 16);
    sq += __shfl_xor(sq, 16);
    sk += __shfl_xor(sk, 32);
    sq += __shfl_xor(sq, 32);
    inv_k = inv_norm(sk);
    inv_q = inv_norm(sq);
    if (g == 0) {
      s_inv[0][r] = inv_k;
      s_inv[1][r] = inv_q;
    }
  }

  // ---- in-block decay products -------------------------------------------------
  float bp[NKB][8], bs[NKB][8];
  bool tiny = false;
  float hy = rv ? ah : 1.f, hz = hy;  // KDA_GATE_HEAD: one scan, shared by every channel
  if constexpr (GATE == KDA_GATE_HEAD) row_scans1(hy, hz);
  const float hs = GATE == KDA_GATE_HEAD ? row_next1(hz) : 1.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if constexpr (GATE == KDA_GATE_HEAD) {
      // Padding channels (d = 16) keep the token's products: their k and q
      // are zero and Gamma_C is stored for real channels only.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bp[kb][j] = hy;
        bs[kb][j] = hs;
      }
    } else {
      const bool ok = rv && kb * 32 + 8 * g < D;
      const float a[8] = {ar0[kb].x, ar0[kb].y, ar0[kb].z, ar0[kb].w, ar1[kb].x, ar1[kb].y, ar1[kb].z, ar1[kb].w};
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bp[kb][j] = z[j] = ok ? a[j] : 1.f;
      row_scans8(bp[kb], z);
      row_next8(bs[kb], z);
    }
    if (m == 15) {
      *reinterpret_cast<float4 *>(&s_bt[wave * DK + kb * 32 + 8 * g]) =
          make_float4(bp[kb][0], bp[kb][1], bp[kb][2], bp[kb][3]);
      *reinterpret_cast<float4 *>(&s_bt[wave * DK + kb * 32 + 8 * g + 4]) =
          make_float4(bp[kb][4], bp[kb][5], bp[kb][6], bp[kb][7]);
#pragma unroll
      for (int j = 0; j < 8; ++j) tiny = tiny || !(bp[kb][j] >= kTinyBlock);
    }
  }
  const bool block_tiny = __ballot(tiny) != 0;
  if (lane == 0) s_flag[wave] = block_tiny ? 1 : 0;
  __syncthreads();

  // ---- operands and Gram tiles, one k-block at a time --------------------------------
  // Registers: the A operands k bp and q bp and the diagonal B operand k / bp
  // of this block; Khat, Qhat to the record; k bs (times block totals) to the
  // Gram planes of the k-block (double-buffered); Ktil kept for the last step.
  // Wave R accumulates row block R of A and M.
  f32x4 aacc[4], macc[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) aacc[J] = macc[J] = zero4();
  float ktl[NKB][8];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    char *pl = s_u + (size_t)(kb & 1) * Cf::NPLANE * kFragBytes;
    const int cb = kb * 32 + 8 * g;
    float tv[4][8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float4 u0 = *reinterpret_cast<const float4 *>(&s_bt[b * DK + cb]);
      const float4 u1 = *reinterpret_cast<const float4 *>(&s_bt[b * DK + cb + 4]);
      tv[b][0] = u0.x; tv[b][1] = u0.y; tv[b][2] = u0.z; tv[b][3] = u0.w;
      tv[b][4] = u1.x; tv[b][5] = u1.y; tv[b][6] = u1.z; tv[b][7] = u1.w;
    }
    float bef[8], aft[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bef[j] = aft[j] = 1.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < wave) bef[j] *= tv[b][j];
        if (b > wave) aft[j] *= tv[b][j];
      }
    }
    const bool ok = rv && cb < D;
    float kf[8], qf[8];
    kr[kb].to_f32(kf);
    qr[kb].to_f32(qf);
    float xa[8], xq[8], x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kf[j] = ok ? kf[j] * inv_k : 0.f;
      qf[j] = ok ? qf[j] * inv_q : 0.f;
      xa[j] = kf[j] * bp[kb][j];
      xq[j] = qf[j] * bp[kb][j];
    }
    const Frag ka = P::make(xa);
    const Frag qa = P::make(xq);
    if constexpr (EXACT) {
      // k and q as loaded (zero past the chunk), and the token's factors
      // Gamma_r / ||k_r|| and Gamma_r / ||q_r|| (one rate per head: bp and
      // bef are the same in every channel)
      // (a value select per word: a select between the two uint4 objects
      // would take their addresses and move kr, qr to scratch)
      const uint32_t keep = ok ? 0xffffffffu : 0u;
      const uint4 kw = kr[kb].u, qw = qr[kb].u;
      *reinterpret_cast<uint4 *>(rec + Rc::khat(wave, kb) + 16 * lane) =
          make_uint4(kw.x & keep, kw.y & keep, kw.z & keep, kw.w & keep);
      *reinterpret_cast<uint4 *>(rec + Rc::qhat(wave, kb) + 16 * lane) =
          make_uint4(qw.x & keep, qw.y & keep, qw.z & keep, qw.w & keep);
      if (kb == 0 && g == 0) {
        float *rf = reinterpret_cast<float *>(rec + Rc::RFAC);
        const float gr = rv ? bp[0][0] * bef[0] : 0.f;
        rf[16 * wave + m] = gr * inv_k;
        rf[C + 16 * wave + m] = gr * inv_q;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = xa[j] * bef[j];  // Gamma_r k_r
      IO::store(rec + Rc::khat(wave, kb), lane, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = xq[j] * bef[j];  // Gamma_r q_r
      IO::store(rec + Rc::qhat(wave, kb), lane, x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = block_tiny ? 0.f : kf[j] * __builtin_amdgcn_rcpf(bp[kb][j]);
    const Frag ki = P::make(x);
    float xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xb[j] = kf[j] * bs[kb][j];
      ktl[kb][j] = xb[j] * aft[j];  // (Gamma_C / Gamma_r) k_r
    }
    if (wave <= 2) IO::store_frag(pl + (size_t)wave * kFragBytes, lane, P::make(xb));
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = xb[j] * tv[1][j];
      IO::store_frag(pl + (size_t)3 * kFragBytes, lane, P::make(x));
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= tv[2][j];
      IO::store_frag(pl + (size_t)4 * kFragBytes, lane, P::make(x));
      if (m == 0 && cb < D) {  // Gamma_C
        float *gam = reinterpret_cast<float *>(rec + Rc::GAM);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = tv[0][j] * tv[1][j] * tv[2][j] * tv[3][j];
        *reinterpret_cast<float4 *>(gam + cb) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4 *>(gam + cb + 4) = make_float4(x[4], x[5], x[6], x[7]);
      }
    } else if (wave == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = xb[j] * tv[2][j];
      IO::store_frag(pl + (size_t)5 * kFragBytes, lane, P::make(x));
    }
    __syncthreads();  // this k-block's planes are written (and the other buffer is free)
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J < wave) {
        FragRaw raw;
        IO::load(raw, pl + (size_t)gram_plane(wave, J) * kFragBytes, lane);
        const Frag B = IO::frag(raw);
        P::mma(aacc[J], ka, B);
        P::mma(macc[J], qa, B);
      } else if (J == wave) {
        P::mma(aacc[J], ka, ki);
        P::mma(macc[J], qa, ki);
      }
    }
  }
  __syncthreads();  // Gram planes consumed: the region now holds L, M, Y

  // L = I + Diag(beta) A (strictly lower part) and M (lower), row block wave.
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * wave + 4 * g + i, jj = 16 * J + m;
      s_L[rr * LP + jj] = (J <= wave && jj < rr) ? aacc[J][i] * s_beta[rr] : 0.f;
      s_M[rr * LP + jj] = (J <= wave && jj <= rr) ? macc[J][i] : 0.f;
    }
  }
  __syncthreads();

  // Rare path: a 16-token block whose decay underflows 2^-100 in some
  // channel.  Its diagonal tiles of A and M, directly:
  //   sum_c x_rc k_jc prod_{j<s<=r} alpha_sc.
  for (int b = 0; b < 4; ++b) {
    if (s_flag[b] == 0) continue;  // uniform across the workgroup
    if (tid < 136) {
      int rl = 0, rem = tid;
      while (rem > rl) {  // pair index -> (r, j), j <= r, within the block
        rem -= rl + 1;
        ++rl;
      }
      const int jl = rem;
      const int rr = 16 * b + rl, jj = 16 * b + jl;
      float a_acc = 0.f, m_acc = 0.f;
      if (rr < nvalid && jj < nvalid) {
        for (int ch = 0; ch < D; ++ch) {
          float f = 1.f;
          for (int s = jj + 1; s <= rr; ++s) {
            const float as =
                GATE == KDA_GATE_HEAD ? alpha[(t0 + s) * H + h] : alpha[((t0 + s) * H + h) * D + ch];
            f *= kPre ? decay_from_preact(as) : as;
          }
          const int64_t orr = ((t0 + rr) * H + h) * D + ch, ojj = ((t0 + jj) * H + h) * D + ch;
          const float kj = to_f32(k[ojj]) * (kPre ? s_inv[0][jj] : 1.f) * f;
          a_acc += to_f32(k[orr]) * (kPre ? s_inv[0][rr] : 1.f) * kj;
          m_acc += to_f32(q[orr]) * (kPre ? s_inv[1][rr] : 1.f) * kj;
        }
      }
      s_L[rr * LP + jj] = (jl < rl) ? a_acc * s_beta[rr] : 0.f;
      s_M[rr * LP + jj] = m_acc;
    }
    __syncthreads();
  }

  // ---- X = L^-1, blocked by 16 ---------------------------------------------------
  // Diagonal blocks: forward substitution, one column per lane (wave b
  // inverts block b).
  if (lane < 16) {
    const int b = wave, jj = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) s -= s_L[(16 * b + i) * LP + 16 * b + t] * x[t];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s_X[(16 * b + i) * MP + 16 * b + jj] = x[i];
  }
  __syncthreads();
  // Off-diagonal blocks by distance d, block (I, I - d) on wave I:
  //   X_IJ = -X_II sum_{K=J}^{I-1} L_IK X_KJ      (fp32 matrix cores, k = 4s + g)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (wave >= d) {
      const int I = wave, J = wave - d;
      f32x4 y = zero4();
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(s_L[(16 * I + m) * LP + 16 * K + 4 * s + g],
                                                   s_X[(16 * K + 4 * s + g) * MP + 16 * J + m], y, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s_Yw[(4 * g + i) * 16 + m] = y[i];
      f32x4 xv = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xv = __builtin_amdgcn_mfma_f32_16x16x4f32(s_X[(16 * I + m) * MP + 16 * I + 4 * s + g],
                                                  s_Yw[(4 * s + g) * 16 + m], xv, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_X[(16 * I + 4 * g + i) * MP + 16 * J + m] = -xv[i];
    }
    __syncthreads();
  }

  // ---- records: (M T)^T and (Ktil^T T)^T -------------------------------------------
  Frag tb[6];  // T^T: lane (g, m) holds T[kb*32 + 8g + j][16 ct + m]
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int cc = tb_ct(u), kb = tb_kb(u);
    const float bc = s_beta[16 * cc + m];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s_X[(kb * 32 + 8 * g + j) * MP + 16 * cc + m] * bc;
    tb[u] = P::make(x);
  }
  // (M T)^T for row tile wave: B = M^T, lane (g, m) holds M[16 w + m][kb*32 + 8g + j].
  {
    f32x4 acc[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) acc[cc] = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb <= (wave >> 1)) {
        float x[8];
        const float4 u0 = *reinterpret_cast<const float4 *>(&s_M[(16 * wave + m) * LP + kb * 32 + 8 * g]);
        const float4 u1 = *reinterpret_cast<const float4 *>(&s_M[(16 * wave + m) * LP + kb * 32 + 8 * g + 4]);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
        x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
        const Frag Bm = P::make(x);
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          if (tb_kb(u) == kb && tb_ct(u) <= wave) P::mma(acc[tb_ct(u)], tb[u], Bm);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb <= (wave >> 1)) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = acc[2 * kb][i];
          x[4 + i] = acc[2 * kb + 1][i];
        }
        IO::store(rec + Rc::mtm(wave, kb), lane, x);
      }
    }
  }
  __syncthreads();  // L, M consumed: the region now holds Ktil (token-major)
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    *reinterpret_cast<float4 *>(&s_kt[r * KP + kb * 32 + 8 * g]) =
        make_float4(ktl[kb][0], ktl[kb][1], ktl[kb][2], ktl[kb][3]);
    *reinterpret_cast<float4 *>(&s_kt[r * KP + kb * 32 + 8 * g + 4]) =
        make_float4(ktl[kb][4], ktl[kb][5], ktl[kb][6], ktl[kb][7]);
  }
  __syncthreads();
  // (Ktil^T T)^T for channel tiles wave, wave + 4: B = Ktil, lane (g, m)
  // holds Ktil[kb*32 + 8g + j][16 t + m].
  constexpr int PT = (Rc::NTILE + 3) / 4;
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    const int t = wave + 4 * tt;
    if (t < Rc::NTILE) {
      Frag Bk[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = s_kt[(kb * 32 + 8 * g + j) * KP + 16 * t + m];
        Bk[kb] = P::make(x);
      }
      f32x4 acc[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) acc[cc] = zero4();
#pragma unroll
      for (int u = 0; u < 6; ++u) P::mma(acc[tb_ct(u)], tb[u], Bk[tb_kb(u)]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = acc[2 * kb][i];
          x[4 + i] = acc[2 * kb + 1][i];
        }
        IO::store(rec + Rc::pmat(t, kb), lane, x);
      }
    }
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
template <int D, int CT = 1>
struct ScanCfg {
  static constexpr int NW = 8;                   // waves per workgroup
  static constexpr int NTH = 64 * NW;
  static constexpr int VW = 16 * CT;             // value columns per workgroup (CT tiles of 16)
  static constexpr int G = D / VW;               // workgroups per (sequence, head)
  static constexpr int NKB = Rec<D>::NKB;
  static constexpr int NTILE = Rec<D>::NTILE;    // state row tiles
  static_assert(NTILE <= NW, "shape");
};

template <int D, typename TIn, int CT = 1>
struct ScanBuf {
  using Cf = ScanCfg<D, CT>;
  // U waves: V row 16 rt + lane / 4, columns 4 CT (lane & 3) .. + 4 CT - 1
  uint32_t v[CT * 2 * sizeof(TIn) / 2];
  FragRaw mt[2];            // O waves: M T, row tile rt
  FragRaw a[Cf::NKB];       // Khat (U waves) or Qhat (O waves), row tile rt
  FragRaw p[2];             // Ktil^T T, state tile = wave
  float4 gam;               // Gamma_C, rows of state tile = wave
  float4 rf;                // exact records: the factors of rows 16 rt + 4 g .. + 3
  uint32_t tch;             // one word of a record two chunks ahead
};

// Loads of one record, in two groups issued in the two phases of the
// previous chunk: the row-tile operands (group 0) and the rest (group 1).
template <int D, typename TIn, typename P, int CT, bool EXACT>
__device__ __forceinline__ void load_scan_a(ScanBuf<D, TIn, CT> &B, int kk, const char *rec, int wave, int lane,
                                            int rot) {
  using Cf = ScanCfg<D, CT>;
  using Rc = Rec<D, EXACT>;
  // The workgroups of one head read the same record at the same time; each
  // starts at a different k-block (register slot kk holds k-block
  // (kk + rot) mod NKB).
  const int rt = wave & 3;
  const int kb = (kk + rot) % Cf::NKB;
  const char *f = rec + (wave < 4 ? Rc::khat(rt, kb) : Rc::qhat(rt, kb));
  if constexpr (EXACT) {
    B.a[kk].a = *reinterpret_cast<const uint4 *>(f + 16 * lane);  // one exact bf16 plane
  } else {
    FragIO<P>::load(B.a[kk], f, lane);
  }
}

// V of a chunk (U waves), issued with the first row-tile load of the
// previous chunk so that it has arrived before the chunk starts: one load
// per lane, through a buffer descriptor spanning the chunk's valid rows
// (padding rows read 0).  (Offsets are 32-bit: the host requires
// 64 H d 4 < 2^31.)
template <int D, typename TIn, int CT>
__device__ __forceinline__ void load_scan_v(ScanBuf<D, TIn, CT> &B, const TIn *v, int64_t vt0, int valid, int h, int H,
                                            int col0, int wave, int lane) {
  const int rt = wave & 3;
  const uint64_t addr = reinterpret_cast<uint64_t>(v + (vt0 * H + h) * D + col0);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const int nbytes = __builtin_amdgcn_readfirstlane(valid * H * D * (int)sizeof(TIn));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0, nbytes, kBufferWord3);
  const int off = ((16 * rt + (lane >> 2)) * H * D + 4 * CT * (lane & 3)) * (int)sizeof(TIn);
  if constexpr (sizeof(TIn) == 2 && CT == 1) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    B.v[0] = x[0];
    B.v[1] = x[1];
  } else {
#pragma unroll
    for (int j = 0; j < CT * (int)sizeof(TIn) / 4; ++j) {  // 16-byte pieces
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * j, 0, 0);
      B.v[4 * j] = x[0];
      B.v[4 * j + 1] = x[1];
      B.v[4 * j + 2] = x[2];
      B.v[4 * j + 3] = x[3];
    }
  }
}

template <int D, typename TIn, typename P, int CT, bool EXACT>
__device__ __forceinline__ void load_scan_b(ScanBuf<D, TIn, CT> &B, const char *rec, int wave, int lane) {
  using Cf = ScanCfg<D, CT>;
  using Rc = Rec<D, EXACT>;
  using IO = FragIO<P>;
  // M T is loaded by the O waves only (a wave-uniform branch).
  const int rt = wave & 3, g = lane >> 4;
  if (wave >= 4) {
    // (row tiles 0 and 1 use only their k-block 0 block)
    IO::load(B.mt[0], rec + Rc::mtm(rt, 0), lane);
    if (rt >= 2) IO::load(B.mt[1], rec + Rc::mtm(rt, 1), lane);
  }
  const int t = wave < Cf::NTILE ? wave : Cf::NTILE - 1;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) IO::load(B.p[kb], rec + Rc::pmat(t, kb), lane);
  // rows 16 t + 4 g .. + 3, the lane's row group (a vector load: a scalar
  // load here would be waited for at the next barrier, with the LDS stores)
  B.gam = *reinterpret_cast<const float4 *>(rec + Rc::GAM + sizeof(float) * (16 * t + 4 * g));
  if constexpr (EXACT)  // factors of k (U waves) or q (O waves) for rows 16 rt + 4 g .. + 3
    B.rf = *reinterpret_cast<const float4 *>(rec + Rc::RFAC + sizeof(float) * ((wave < 4 ? 0 : C) + 16 * rt + 4 * g));
}

// Two waves per SIMD: the two register sets of record fragments take about
// half of each wave's 256 registers.  CT = 1 or 2 tiles of 16 value columns
// per workgroup: with CT = 2 every record fragment a wave loads serves two
// products, so a head's record is streamed to half as many CUs (batches with
// more workgroups than CUs); with CT = 1 a head's chain spreads over twice
// as many CUs (small batches).
template <int D, typename TIn, typename P, int CT, bool EXACT>
__global__ __launch_bounds__(ScanCfg<D>::NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk_state_kernel(
    const TIn *__restrict__ v, const int32_t *__restrict__ cu, int32_t seq_len, int N, int H,
    int64_t total_tokens, int64_t W, int64_t j0, const int32_t *__restrict__ base,
    const char *__restrict__ recs, const float *S0, float *carry, float *__restrict__ o, float *S_T) {
  using Cf = ScanCfg<D, CT>;
  using Rc = Rec<D, EXACT>;
  using IO = FragIO<P>;
  using Buf = ScanBuf<D, TIn, CT>;
  constexpr int VW = Cf::VW, G = Cf::G, NKB = Cf::NKB, NTILE = Cf::NTILE, NTH = Cf::NTH;
  constexpr int DK = D < 32 ? 32 : D;

  __shared__ Plane<P, VW, DK> Sop;     // S^T in operand form (rows = value columns)
  __shared__ Plane<P, VW, C> Uop;      // U^T in operand form
  __shared__ __attribute__((aligned(16))) float s_ot[4][16][VW + 4];  // o tile of each O wave, row-major
  __shared__ __attribute__((aligned(16))) TIn s_vt[4][16][VW];        // V tile of each U wave, row-major

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
  // varlen: the sequences in the schedule's longest-first order
  const int n = cu != nullptr ? base[N + 1 + (int)(pair / H)] : (int)(pair / H);
  const int h = (int)(pair % H);
  const int64_t nh = (int64_t)n * H + h;  // the (sequence, head) whose state this is
  const int col0 = VW * cg;

  // The sequence's packed chunks in this stripe, [lo, hi).  A sequence with
  // none there has nothing to do, except that the first stripe gives an
  // empty sequence S_T = S0.
  int64_t first, count;
  seq_chunk_range(cu, base, seq_len, n, first, count);
  if (total_tokens <= 0) count = 0;
  const int64_t lo = first > j0 ? first : j0;
  const int64_t hi = first + count < j0 + W ? first + count : j0 + W;
  if (!(lo < hi || (count == 0 && j0 == 0))) return;
  // the state comes from S0 if the sequence starts here, else from the
  // previous stripe; it goes to S_T if the sequence ends here, else on
  const float *sin = lo == first ? S0 : carry;
  float *sout = hi == first + count ? S_T : carry;

  if constexpr (DK > D) {
    for (int e = tid; e < VW * (DK - D); e += NTH) Sop.store(e / (DK - D), D + e % (DK - D), 0.f);
  }
  f32x4 sreg[CT];
  const float *S0p = sin ? sin + (size_t)nh * D * D : nullptr;
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    sreg[t] = zero4();
    if (wave < NTILE) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sreg[t][i] = S0p ? S0p[(size_t)(16 * wave + 4 * g + i) * D + col0 + 16 * t + m] : 0.f;
      Sop.store4(16 * t + m, 16 * wave + 4 * g, sreg[t]);
    }
  }

  // This stripe's chunks of the sequence, numbered within the sequence.
  int64_t sstart, slen;
  seq_range(cu, seq_len, n, sstart, slen);
  const int64_t cbeg = lo - first;
  const int64_t cend = lo < hi ? hi - first : cbeg;

  auto rec_of = [&](int64_t cc) __attribute__((always_inline)) {
    return recs + ((size_t)h * W + (first + cc - j0)) * Rc::BYTES;
  };
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
    load_scan_b<D, TIn, P, CT, EXACT>(B, rec_of(cc), wave, lane);
  };
  auto prefetch_v = [&](int64_t cc, Buf &B) __attribute__((always_inline)) {
    if (uwave) {
      const ChunkTok cn = chunk_tokens(sstart, slen, cc, total_tokens);
      load_scan_v<D, TIn>(B, v, cn.t0, cn.valid, h, H, col0, wave, lane);
    }
  };

  // o of a chunk is stored during the next chunk's first phase by the O
  // waves: the wave's 16 x 16 tile goes through LDS so that each lane stores
  // four consecutive columns of one row, through a buffer descriptor
  // spanning exactly the chunk's valid rows (the hardware drops the stores
  // of padding rows).  (Offsets are 32-bit: the host requires
  // 64 H d 4 < 2^31.)
  f32x4 opend[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) opend[t] = zero4();
  int64_t pend_t0 = 0;
  int pend_valid = 0;
  auto store_o = [&]() __attribute__((always_inline)) {
    // (the base and size are wave-uniform; readfirstlane lets the compiler
    // keep the descriptor in scalar registers)
    const uint64_t addr = reinterpret_cast<uint64_t>(o + (pend_t0 * H + h) * D + col0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int nbytes = __builtin_amdgcn_readfirstlane(pend_valid * H * D * (int)sizeof(float));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<float *>(((uint64_t)hi << 32) | lo), 0, nbytes, kBufferWord3);
    float(*ot)[VW + 4] = s_ot[rt];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) ot[4 * g + i][16 * t + m] = opend[t][i];
    // (one wave writes and reads its own tile: LDS executes a wave's
    // accesses in order)
    __builtin_amdgcn_wave_barrier();
    const int r = lane >> 2, cq = lane & 3;
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      const float4 x = *reinterpret_cast<const float4 *>(&ot[r][4 * CT * cq + 4 * j]);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs,
                                             ((16 * rt + r) * H * D + 4 * CT * cq + 4 * j) * (int)sizeof(float),
                                             0, 0);
    }
  };

  // The loads of the next record are spread over this chunk's two phases,
  // between its matrix-core products, so that each wave keeps computing
  // while its loads queue.
  auto process = [&](int64_t c, const Buf &U, Buf &Nx, int64_t cn) __attribute__((always_inline)) {
    const ChunkTok ct = chunk_tokens(sstart, slen, c, total_tokens);
    const char *rn = rec_of(cn);  // unconditional (the last chunk re-reads itself)

    // Khat S (U waves) or Qhat S (O waves) for row tile rt.  All S operand
    // fragments are read first, so their LDS latency is paid once.
    typename P::Frag Bs[CT][NKB];
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) Bs[t][kk] = Sop.load8(16 * t + m, ((kk + cg) % NKB) * 32 + 8 * g);
    // This chunk's V (U waves) to the accumulator layout through LDS: rows
    // 16 rt + 4 g + i, column 16 t + m.
    float vf[CT][4];
#pragma unroll
    for (int t = 0; t < CT; ++t) vf[t][0] = vf[t][1] = vf[t][2] = vf[t][3] = 0.f;
    if (uwave) {
      TIn *vrow = &s_vt[rt][lane >> 2][4 * CT * (lane & 3)];
      if constexpr (sizeof(TIn) == 2 && CT == 1) {
        *reinterpret_cast<uint2 *>(vrow) = make_uint2(U.v[0], U.v[1]);
      } else {
#pragma unroll
        for (int j = 0; j < CT * (int)sizeof(TIn) / 4; ++j)
          reinterpret_cast<uint4 *>(vrow)[j] = make_uint4(U.v[4 * j], U.v[4 * j + 1], U.v[4 * j + 2], U.v[4 * j + 3]);
      }
      // (one wave writes and reads its own tile: LDS executes a wave's
      // accesses in order)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[t][i] = to_f32(s_vt[rt][4 * g + i][16 * t + m]);
    }
    f32x4 acc[2][CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[0][t] = acc[1][t] = zero4();
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {  // register slot kk holds k-block (kk + cg) mod NKB
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        if constexpr (EXACT) {  // exact bf16 k or q: its lo part is zero
          const auto a = __builtin_bit_cast(bf16x8, U.a[kk].a);
          acc[kk & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Bs[t][kk].hi, acc[kk & 1][t], 0, 0, 0);
          acc[kk & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Bs[t][kk].lo, acc[kk & 1][t], 0, 0, 0);
        } else {
          P::mma(acc[kk & 1][t], IO::frag(U.a[kk]), Bs[t][kk]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_scan_a<D, TIn, P, CT, EXACT>(Nx, kk, rn, wave, lane, cg);
      if (kk == 0) prefetch_v(cn, Nx);
      __builtin_amdgcn_sched_barrier(0);
    }
    Nx.tch = touch(cn + 1 < cend ? cn + 1 : cn);
    if (!uwave) store_o();  // the previous chunk's o, while the U waves form U
    f32x4 ov[CT];
    // (exact records: rows scaled by Gamma_r / ||k_r|| or Gamma_r / ||q_r||)
    const float rfac[4] = {U.rf.x, U.rf.y, U.rf.z, U.rf.w};
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ov[t][i] = acc[0][t][i] + acc[1][t][i];
        if constexpr (EXACT) ov[t][i] *= rfac[i];
      }
    if (uwave) {
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          u[i] = (r < ct.valid ? vf[t][i] : 0.f) - ov[t][i];
        }
        Uop.store4(16 * t + m, 16 * rt + 4 * g, u);
      }
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < CT; ++t) {
      // U as an operand, in the k-order of the Ktil^T T and M T fragments:
      // rows 32kb + 4g .. +3 and 32kb + 16 + 4g .. +3 of column 16 t + m.
      const auto u0 = Uop.load_acc_order(16 * t + m, 0, g);
      const auto u1 = Uop.load_acc_order(16 * t + m, 32, g);
      // S <- Diag(Gamma_C) S + (Ktil^T T) U
      if (wave < NTILE) {
        const float gm[4] = {U.gam.x, U.gam.y, U.gam.z, U.gam.w};
        f32x4 sacc;
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[i] = gm[i] * sreg[t][i];
        P::mma(sacc, IO::frag(U.p[0]), u0);
        P::mma(sacc, IO::frag(U.p[1]), u1);
        sreg[t] = sacc;
        Sop.store4(16 * t + m, 16 * wave + 4 * g, sacc);
      }
      // o = Qhat S + (M T) U
      if (!uwave) {
        P::mma(ov[t], IO::frag(U.mt[0]), u0);
        if (rt >= 2) P::mma(ov[t], IO::frag(U.mt[1]), u1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    prefetch_b(cn, Nx);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < CT; ++t) opend[t] = ov[t];
    pend_t0 = ct.t0;
    pend_valid = uwave ? 0 : ct.valid;
    sink += U.tch;
    __syncthreads();
  };

  if (cbeg < cend) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) load_scan_a<D, TIn, P, CT, EXACT>(bufA, kk, rec_of(cbeg), wave, lane, cg);
    prefetch_v(cbeg, bufA);
    prefetch_b(cbeg, bufA);
    bufA.tch = touch(cbeg);
  }
  __syncthreads();
  // Pairs of chunks (no exit between the two halves, so each half's loads
  // stay where they are issued), then an odd last chunk.
  int64_t c = cbeg;
  for (; c + 1 < cend; c += 2) {
    process(c, bufA, bufB, c + 1);
    process(c + 1, bufB, bufA, c + 2 < cend ? c + 2 : c + 1);
  }
  if (c < cend) process(c, bufA, bufB, c);
  if (!uwave) store_o();
  if (N < 0) o[sink & 1] = 0.f;  // never taken (N >= 0): keeps the touches alive

  // The state after this stripe: the final state, or the carry into the
  // next stripe.
  if (sout != nullptr && wave < NTILE) {
    float *STp = sout + (size_t)nh * D * D;
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) STp[(size_t)(16 * wave + 4 * g + i) * D + col0 + 16 * t + m] = sreg[t][i];
  }
}

template <int D, typename TIn, typename P, int GATE, int FORM>
hipError_t launch_prefill_t(const kda_shape_t &s, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const int32_t *cu,
                            const float *S0, float *o, float *S_T, void *workspace,
                            const PrefillPlan &plan, hipStream_t stream, int phases) {
  char *ws = static_cast<char *>(workspace);
  int32_t *base = reinterpret_cast<int32_t *>(ws);
  char *recs = ws + schedule_bytes(s);
  // the state between stripes: S_T, or the carry area when S_T is NULL
  float *carry = plan.carry_off != 0 ? reinterpret_cast<float *>(ws + plan.carry_off) : S_T;
  const int N = s.num_seqs, H = s.num_heads;
  const int64_t W = plan.W;
  const TIn *qp = static_cast<const TIn *>(q), *kp = static_cast<const TIn *>(k),
            *vp = static_cast<const TIn *>(v);
  // the record layout the chunk-local kernel writes for this gate and dtype
  constexpr bool kExact = GATE == KDA_GATE_HEAD && std::is_same<TIn, __bf16>::value &&
                          std::is_same<P, SplitBF16>::value;
  // Two 16-column tiles per state-pass workgroup once a stripe keeps more
  // one-tile workgroups busy than the chip has CUs (each CU then streams a
  // record for 32 value columns instead of 16); one tile otherwise.  A
  // stripe of W packed chunks keeps about W N / chunks + 1 sequences busy
  // (all of them with one stripe).  (Measured: two tiles win for two dense
  // 4k sequences, 21.0 vs 18.4 M tokens/s; one tile for the eight-sequence
  // varlen batch in 512 MiB stripes, 19.2 vs 17.0.)
  const int64_t pairs8 = ((int64_t)N * H + 7) / 8 * 8;
  int64_t busy = N;
  if (plan.stripes > 1 && plan.chunks > 0) {
    const int64_t est = W * N / plan.chunks + 1;
    busy = est < N ? est : N;
  }
  const bool wide = D >= 32 && busy * H * (D / 16) > kStateWideAbove;
  const int64_t sblocks = pairs8 * (wide ? ScanCfg<D, D >= 32 ? 2 : 1>::G : ScanCfg<D>::G);
  hipError_t e = hipSuccess;
  if ((phases & kPhaseLocal) && cu != nullptr) {  // dense batches compute their table in the kernels
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, cu, N, s.seq_len, base);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int64_t i = 0; i < plan.stripes; ++i) {
    const int64_t j0 = i * W;
    const int64_t wi = plan.chunks - j0 < W ? plan.chunks - j0 : W;  // chunks of this stripe
    if ((phases & kPhaseLocal) && wi > 0) {
      hipLaunchKernelGGL((chunk_local_kernel<D, TIn, P, GATE, FORM>), dim3((unsigned)(wi * H)), dim3(NT), 0,
                         stream, qp, kp, alpha, beta, cu, s.seq_len, N, H, s.total_tokens, W, j0, base, recs);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & kPhaseState) {
      if (wide) {
        hipLaunchKernelGGL((chunk_state_kernel<D, TIn, P, D >= 32 ? 2 : 1, kExact>), dim3((unsigned)sblocks),
                           dim3(ScanCfg<D>::NTH), 0, stream, vp, cu, s.seq_len, N, H, s.total_tokens, W, j0, base,
                           recs, S0, carry, o, S_T);
      } else {
        hipLaunchKernelGGL((chunk_state_kernel<D, TIn, P, 1, kExact>), dim3((unsigned)sblocks), dim3(ScanCfg<D>::NTH), 0,
                           stream, vp, cu, s.seq_len, N, H, s.total_tokens, W, j0, base, recs, S0, carry, o, S_T);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return e;
}

template <typename TIn, int GATE, int FORM>
hipError_t dispatch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                            const float *alpha, const float *beta, const int32_t *cu,
                            const float *S0, float *o, float *S_T, void *ws, const PrefillPlan &pl,
                            hipStream_t st, int ph) {
  // bf16 inputs run the split-bf16 matrix-core path; fp32 inputs (and the
  // 16-wide heads) the fp32 matrix-core path.
  using PB = typename std::conditional<std::is_same<TIn, __bf16>::value, SplitBF16, F32>::type;
  switch (s.d_k) {
    case 16: return launch_prefill_t<16, TIn, F32, GATE, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
    case 32: return launch_prefill_t<32, TIn, PB, GATE, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
    case 64: return launch_prefill_t<64, TIn, PB, GATE, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
    case 128: return launch_prefill_t<128, TIn, PB, GATE, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, int FORM>
hipError_t dispatch_gate(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, const int32_t *cu, const float *S0,
                         float *o, float *S_T, void *ws, const PrefillPlan &pl, hipStream_t st, int ph) {
  if (s.gate == KDA_GATE_HEAD)
    return dispatch_prefill<TIn, KDA_GATE_HEAD, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
  return dispatch_prefill<TIn, KDA_GATE_CHANNEL, FORM>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
}

template <typename TIn>
hipError_t dispatch_form(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, const int32_t *cu, const float *S0,
                         float *o, float *S_T, void *ws, const PrefillPlan &pl, hipStream_t st, int ph) {
  if (s.input_form == KDA_INPUT_PREACT)
    return dispatch_gate<TIn, KDA_INPUT_PREACT>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
  return dispatch_gate<TIn, KDA_INPUT_FINAL>(s, q, k, v, alpha, beta, cu, S0, o, S_T, ws, pl, st, ph);
}

}  // namespace

hipError_t launch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          const float *S0, float *o, float *S_T, void *workspace,
                          const PrefillPlan &plan, hipStream_t stream, int phases) {
  if (s.qkv_dtype == KDA_BF16)
    return dispatch_form<__bf16>(s, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, plan, stream,
                                 phases);
  return dispatch_form<float>(s, q, k, v, alpha, beta, cu_seqlens, S0, o, S_T, workspace, plan, stream,
                              phases);
}

}  // namespace kda
