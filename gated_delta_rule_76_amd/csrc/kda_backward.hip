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
// columns: one workgroup per (sequence, head, column slice).  Lane layout:
// LPC lanes hold one column (64 at d >= 64, i.e. one wave per column; 32 at
// d = 32; one 16-lane DPP row at d = 16), lane rg of a column keeping rows
// rg*RPT .. +RPT-1, so the workgroup has 16 LPC threads (1024 at d >= 64:
// four waves per SIMD, which hide each other's latencies).  Tokens go in
// blocks of CK (16; at d = 128, 12 for bf16 and 8 for fp32 inputs, so that a
// block's states and inputs fit in LDS).  Per workgroup:
//   pass 1  the forward recurrence over the sequence from S0, storing the
//           state at the start of every block (workspace);
//   pass 2  blocks from last to first: re-run the block forward from its
//           checkpoint, keeping every S_{t-1} in LDS (each thread keeps its
//           own elements, so no barrier guards the ring), then the tokens
//           backward with G in registers.
// A block's inputs (k, q, alpha, beta and the slice's v, dO) are staged in
// LDS; the next block's are loaded into registers while the current block
// computes, so the steps never wait on global memory.
// The column sums the recurrences need (X^T k, G^T k) stay inside the wave:
// DPP adds within rows and lane swaps between them, no barrier, so the
// forward steps never synchronise the workgroup.  The row sums over the 16
// columns (dk, dq, dalpha, and dbeta) are outputs only: lane swaps over the
// wave's columns (when it holds more than one), then one LDS round across
// the waves (double-buffered, one barrier per backward token); they are
// per-slice partials, summed over the slices in a fixed order by a second
// kernel (deterministic results).
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// The part of every sequence one launch of the backward covers, and where
// its state, state gradient, checkpoints and partial rows live.
struct BwdPiece {
  int64_t t_off;        // first token of the piece within every sequence
  int64_t plen;         // piece length cap (tokens)
  int64_t slot_stride;  // checkpoint slots per sequence; 0 = packed over the batch
  int64_t row_len;      // partial rows per sequence; 0 = one row per token of the batch
  int64_t rows;         // partial rows per head and column slice (the slice stride / H)
  const float *S_in;    // state at the piece start (NULL = zeros)
  const float *G_in;    // dL/dS at the piece end (NULL = zeros)
  float *G_out;         // dL/dS at the piece start (NULL = not written)
  float *sweep;         // forward sweep only: the state at every multiple of plen, [p-1][N][H][d][d]
};

// (a native vector type: the in-flight block stays in registers)
typedef uint32_t bu32x4 __attribute__((ext_vector_type(4)));
constexpr int kBwdVW = 16;  // value columns per workgroup

template <int D, typename TIn, int GATE>
struct BwdCfg {
  static constexpr int VW = kBwdVW < D ? kBwdVW : D;  // columns per workgroup
  static constexpr int SL = D / VW;                   // column slices per head
  static constexpr int LPC = D >= 64 ? 64 : D >= 32 ? 32 : 16;  // lanes per column
  static constexpr int NT = VW * LPC;                 // threads per workgroup
  static constexpr int RPT = D / LPC;                 // rows per thread
  static constexpr int NW = NT / 64;
  static constexpr int NRED = bwd_row_sums(D, GATE == KDA_GATE_HEAD);  // row sums per token
  static constexpr int NREDP = (NRED + 3) / 4 * 4;                     // LDS row: 16-byte groups
  // lanes of each of the first four waves that add the row sums (pairs)
  static constexpr int RLW = ((NREDP / 2 + 3) / 4 + 1) / 2 * 2;
  static constexpr int EB = GATE == KDA_GATE_HEAD ? 2 * D : 3 * D;     // index of dbeta
  static constexpr int CK = bwd_block(D, sizeof(TIn) == 4);
  static constexpr int DA = GATE == KDA_GATE_HEAD ? 1 : D;  // rates per token
  // 16-byte chunks of one block's rows, and chunks per token row
  static constexpr int KCT = D * (int)sizeof(TIn) / 16;    // k or q
  static constexpr int ACT = GATE == KDA_GATE_HEAD ? 0 : D / 4;
  static constexpr int VCT = VW * (int)sizeof(TIn) / 16;  // v slice
  static constexpr int OCT = VW / 4;                       // dO slice
  static constexpr int NK = CK * KCT, NA = CK * ACT, NV = CK * VCT, NO = CK * OCT;
  static constexpr int PK = (NK + NT - 1) / NT;  // chunks per thread
  static constexpr int PA = (NA + NT - 1) / NT;
  static_assert(VW == 16 && RPT >= 1 && D % LPC == 0 && NV <= NT && NO <= NT, "layout");
  static_assert(NW >= 4 && NW % 2 == 0 && RLW <= 64 && 4 * RLW >= NREDP / 2, "row-sum lanes");
};

// Sum over the 16 lanes of a DPP row, every lane receiving the total
// (xor 1 and xor 2 within quads, then rotations by 4 and 8 within the row).
__device__ __forceinline__ float row16_allsum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)); // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)); // row_ror:8
  return x;
}

// x[lane] + x[lane ^ 16] and x[lane] + x[lane ^ 32], for every lane
// (lane-swap instructions, no LDS).
__device__ __forceinline__ float xor16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the LPC lanes of one column (16: one DPP row; 32: two), and over
// the wave's columns (the other lanes), every lane receiving the total.
template <int LPC>
__device__ __forceinline__ float column_sum(float x) {
  x = row16_allsum(x);
  if constexpr (LPC >= 32) x = xor16_sum(x);
  if constexpr (LPC == 64) x = xor32_sum(x);
  return x;
}
// column_sum of x and of y together.  The first lane swap leaves x's partial
// sums in half of each column's lanes and y's in the other half, so the rest
// of the reduction runs once for both; the last swap hands every lane both.
template <int LPC>
__device__ __forceinline__ void column_sum2(float &x, float &y) {
  if constexpr (LPC == 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float u = row16_allsum(xor16_sum(__uint_as_float(r[0]) + __uint_as_float(r[1])));  // lanes < 32: x
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(u), false, false);
    x = __uint_as_float(b[0]);
    y = __uint_as_float(b[1]);
  } else if constexpr (LPC == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float u = row16_allsum(__uint_as_float(r[0]) + __uint_as_float(r[1]));  // rows 0, 2: x
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
    x = __uint_as_float(b[0]);
    y = __uint_as_float(b[1]);
  } else {
    x = row16_allsum(x);
    y = row16_allsum(y);
  }
}
template <int LPC>
__device__ __forceinline__ float across_columns(float x) {
  if constexpr (LPC == 16) x = xor16_sum(x);
  if constexpr (LPC <= 32) x = xor32_sum(x);
  return x;
}

// Wait until every global load and store this wave issued has completed
// (s_waitcnt vmcnt(0)).  Placed where the next block's prefetch has had a
// whole phase of LDS-only work to arrive: the compiler cannot count the loads
// and stores issued under per-thread conditions, so without it it waits for
// everything right after the prefetch, at the first reuse of a register.
__device__ __forceinline__ void wait_global_ops() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One block's inputs in LDS.
template <int D, typename TIn, int GATE>
struct BlockIn {
  using Cf = BwdCfg<D, TIn, GATE>;
  TIn k[Cf::CK][D];
  TIn q[Cf::CK][D];
  float a[Cf::CK][Cf::DA];
  TIn v[Cf::CK][Cf::VW];
  float dO[Cf::CK][Cf::VW];
  float b[Cf::CK];
};

// The next block's inputs in flight, in registers (16-byte chunks; thread
// tid holds chunks tid, tid + 256, ... of each array).
template <int D, typename TIn, int GATE>
struct BlockRaw {
  using Cf = BwdCfg<D, TIn, GATE>;
  bu32x4 k[Cf::PK], q[Cf::PK], a[Cf::PA > 0 ? Cf::PA : 1], v, o;
  float b, ah;
};

template <int D, typename TIn, int GATE>
__global__ __launch_bounds__((BwdCfg<D, TIn, GATE>::NT)) void bwd_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    int32_t seq_len, int N, int H, int64_t total, const float *__restrict__ dO, float *__restrict__ dv,
    float *__restrict__ ckpt, float *__restrict__ part, const BwdPiece pc) {
  using Cf = BwdCfg<D, TIn, GATE>;
  constexpr int RPT = Cf::RPT, VW = Cf::VW, SL = Cf::SL, NW = Cf::NW, NRED = Cf::NRED, CK = Cf::CK;
  constexpr int NT = Cf::NT, LPC = Cf::LPC;

  __shared__ float s_ring[CK][NT][RPT];  // S_{t-1} of the block's tokens, per thread
  constexpr int NREDP = Cf::NREDP;
  __shared__ __attribute__((aligned(16))) float s_red[2][NW][NREDP];  // per-wave row sums, double-buffered
  __shared__ __attribute__((aligned(16))) BlockIn<D, TIn, GATE> s_in;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid / LPC, rg = tid % LPC;  // column of the slice, row group
  const int r0 = rg * RPT;
  // blockIdx -> work: consecutive workgroups are dealt round-robin to the 8
  // XCDs, so the SL column slices of one (sequence, head) get block indices
  // congruent mod 8.  They share an XCD and its L2, and the rows of k, q and
  // alpha that every slice reads come from HBM once for all of them.  (The
  // grid covers the (sequence, head) pairs rounded up to a multiple of 8.)
  const int id = blockIdx.x;
  const int sl = (id >> 3) % SL;
  const int nh = ((id >> 3) / SL) * 8 + (id & 7);
  if (nh >= N * H) return;
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
  // This launch's piece of the sequence (the forward sweep runs all of it).
  if (pc.sweep == nullptr) {
    const int64_t off = pc.t_off < len ? pc.t_off : len;
    start += off;
    len -= off;
    if (len > pc.plen) len = pc.plen;
  }
  const int64_t nblk = (len + CK - 1) / CK;
  // first checkpoint slot and first partial row of this piece
  const int64_t blk0 = pc.slot_stride > 0 ? (int64_t)n * pc.slot_stride : start / CK + n;
  const int64_t row0 = pc.row_len > 0 ? (int64_t)n * pc.row_len : start;
  const int64_t sbase = (((int64_t)n * H + h) * D) * D;  // [n][h] state offset
  // A checkpoint slot holds the slice as [thread][RPT] (each thread reads back
  // what it wrote).
  auto ck_at = [&](int64_t j) {
    return ckpt + (((blk0 + j) * H + h) * SL + sl) * (int64_t)(D * VW) + tid * RPT;
  };
  // (token row * H + head) of token t of the block starting at tb; tokens past
  // the sequence re-read its last token (their values are never used).
  auto trow = [&](int64_t tb, int t) {
    int64_t tt = tb + t;
    tt = tt < len ? tt : len - 1;
    return (start + tt) * H + h;
  };

  // ---- block inputs: global -> registers -> LDS -----------------------------------
  auto fetch = [&](int64_t tb, BlockRaw<D, TIn, GATE> &R) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < Cf::PK; ++m) {
      const int idx = tid + NT * m;
      if (Cf::NK % NT == 0 || idx < Cf::NK) {
        const int64_t off = trow(tb, idx / Cf::KCT) * D * (int64_t)sizeof(TIn) + (idx % Cf::KCT) * 16;
        R.k[m] = *reinterpret_cast<const bu32x4 *>(reinterpret_cast<const char *>(k) + off);
        R.q[m] = *reinterpret_cast<const bu32x4 *>(reinterpret_cast<const char *>(q) + off);
      }
    }
    if constexpr (Cf::NA > 0) {
#pragma unroll
      for (int m = 0; m < Cf::PA; ++m) {
        const int idx = tid + NT * m;
        if (Cf::NA % NT == 0 || idx < Cf::NA) {
          const int64_t off = trow(tb, idx / Cf::ACT) * D + (idx % Cf::ACT) * 4;
          R.a[m] = *reinterpret_cast<const bu32x4 *>(alpha + off);
        }
      }
    }
    if (tid < Cf::NV) {
      const int64_t off = (trow(tb, tid / Cf::VCT) * D + sl * VW) * (int64_t)sizeof(TIn) + (tid % Cf::VCT) * 16;
      R.v = *reinterpret_cast<const bu32x4 *>(reinterpret_cast<const char *>(v) + off);
    }
    if (tid < Cf::NO)
      R.o = *reinterpret_cast<const bu32x4 *>(dO + trow(tb, tid / Cf::OCT) * D + sl * VW + (tid % Cf::OCT) * 4);
    if (tid < CK) {
      R.b = beta[trow(tb, tid)];
      if constexpr (GATE == KDA_GATE_HEAD) R.ah = alpha[trow(tb, tid)];
    }
  };
  auto stash = [&](const BlockRaw<D, TIn, GATE> &R) __attribute__((always_inline)) {
    char *bk = reinterpret_cast<char *>(&s_in.k[0][0]), *bq = reinterpret_cast<char *>(&s_in.q[0][0]);
#pragma unroll
    for (int m = 0; m < Cf::PK; ++m) {
      const int idx = tid + NT * m;
      if (Cf::NK % NT == 0 || idx < Cf::NK) {
        *reinterpret_cast<bu32x4 *>(bk + 16 * idx) = R.k[m];
        *reinterpret_cast<bu32x4 *>(bq + 16 * idx) = R.q[m];
      }
    }
    if constexpr (Cf::NA > 0) {
#pragma unroll
      for (int m = 0; m < Cf::PA; ++m) {
        const int idx = tid + NT * m;
        if (Cf::NA % NT == 0 || idx < Cf::NA)
          *reinterpret_cast<bu32x4 *>(reinterpret_cast<char *>(&s_in.a[0][0]) + 16 * idx) = R.a[m];
      }
    }
    if (tid < Cf::NV) *reinterpret_cast<bu32x4 *>(reinterpret_cast<char *>(&s_in.v[0][0]) + 16 * tid) = R.v;
    if (tid < Cf::NO) *reinterpret_cast<bu32x4 *>(reinterpret_cast<char *>(&s_in.dO[0][0]) + 16 * tid) = R.o;
    if (tid < CK) {
      s_in.b[tid] = R.b;
      if constexpr (GATE == KDA_GATE_HEAD) s_in.a[tid][0] = R.ah;
    }
  };

  // Token j of the staged block: this thread's rows of k (and q, alpha).
  auto rate = [&](int j, int i) -> float {
    if constexpr (GATE == KDA_GATE_HEAD) {
      return s_in.a[j][0];
    } else {
      return s_in.a[j][r0 + i];
    }
  };

  // ---- pass 1: forward, checkpoint at every block start -----------------------
  // (the forward sweep instead stores the state at every piece start)
  float s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = pc.S_in != nullptr ? pc.S_in[sbase + (int64_t)(r0 + i) * D + col] : 0.f;
  auto fwd_step = [&](int j) __attribute__((always_inline)) {
    float ak[RPT];
    float xk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      s[i] *= rate(j, i);
      ak[i] = to_f32(s_in.k[j][r0 + i]);
      xk += s[i] * ak[i];
    }
    xk = column_sum<LPC>(xk);
    const float w = s_in.b[j] * (to_f32(s_in.v[j][c]) - xk);
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] += ak[i] * w;
  };

  BlockRaw<D, TIn, GATE> R;
  if (nblk > 0) {
    fetch(0, R);
    stash(R);
  }
  for (int64_t b = 0; b < nblk; ++b) {
    __syncthreads();  // block b is in LDS
    // next block needed: b + 1, or (after the last) the one before it for pass 2
    const int64_t nb = b + 1 < nblk ? b + 1 : (b > 0 ? b - 1 : b);
    fetch(nb * CK, R);
    if (pc.sweep == nullptr) {
      float *cp = ck_at(b);
#pragma unroll
      for (int i = 0; i < RPT; ++i) cp[i] = s[i];
    } else if (b > 0 && (b * CK) % pc.plen == 0) {  // (plen is a multiple of CK)
      float *sp = pc.sweep + ((b * CK) / pc.plen - 1) * (int64_t)N * H * D * D + sbase;
#pragma unroll
      for (int i = 0; i < RPT; ++i) sp[(int64_t)(r0 + i) * D + col] = s[i];
    }
    const int nt = (int)(len - b * CK < CK ? len - b * CK : CK);
    // (loops over a block's tokens are unrolled, so LDS addresses are
    // immediate offsets rather than per-lane pointer increments)
#pragma unroll
    for (int j = 0; j < CK; ++j)
      if (j < nt) fwd_step(j);
    wait_global_ops();  // the next block's inputs
    if (b + 1 < nblk) {
      __syncthreads();  // every wave is done with block b
      stash(R);
    }
  }
  if (pc.sweep != nullptr) return;
  // Each thread reads back only the checkpoint elements it wrote.
  __threadfence_block();

  // ---- pass 2: backward ---------------------------------------------------------
  // LDS holds the last block; R holds the one before it.
  float G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) G[i] = pc.G_in != nullptr ? pc.G_in[sbase + (int64_t)(r0 + i) * D + col] : 0.f;
  int par = 0;
  // The checkpoint of the block before is loaded while a block runs.
  float ckn[RPT];
  if (nblk > 0) {
    const float *cp = ck_at(nblk - 1);
#pragma unroll
    for (int i = 0; i < RPT; ++i) ckn[i] = cp[i];
  }
  wait_global_ops();  // (once: so that no load is pending at the loop head)
  for (int64_t b = nblk - 1; b >= 0; --b) {
    const int64_t tb = b * CK;
    const int nt = (int)(len - tb < CK ? len - tb : CK);
    if (b < nblk - 1) {
      __syncthreads();  // every wave is done with block b + 1
      stash(R);
      __syncthreads();
      fetch((b > 0 ? b - 1 : 0) * CK, R);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = ckn[i];
    if (b > 0) {
      const float *cp = ck_at(b - 1);
#pragma unroll
      for (int i = 0; i < RPT; ++i) ckn[i] = cp[i];
    }
    // (this re-run stays a rolled loop: unrolled like the other block loops
    // it made the whole pass 6% slower)
    for (int j = 0; j < CK; ++j) {
      if (j >= nt) break;
#pragma unroll
      for (int i = 0; i < RPT; ++i) s_ring[j][tid][i] = s[i];
      fwd_step(j);
    }
    wait_global_ops();  // the block before: inputs and checkpoint
#pragma unroll
    for (int j = CK - 1; j >= 0; --j) {
      if (j >= nt) continue;
      const int64_t th = (start + tb + j) * H + h;
      const float dOc = s_in.dO[j][c];
      float sp[RPT], X[RPT], kf[RPT];
      float xk = 0.f, gk = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        sp[i] = s_ring[j][tid][i];
        kf[i] = to_f32(s_in.k[j][r0 + i]);
        G[i] += to_f32(s_in.q[j][r0 + i]) * dOc;
        X[i] = rate(j, i) * sp[i];
        xk += X[i] * kf[i];
        gk += G[i] * kf[i];
      }
      column_sum2<LPC>(xk, gk);
      const float bt = s_in.b[j];
      const float w = to_f32(s_in.v[j][c]) - xk;
      const float bw = bt * w, bg = bt * gk;
      dv[th * D + col] = bg;  // (the column's lanes store the same value)
      float dkp[RPT], dqp[RPT], dap[RPT];
      float da_all = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float st = X[i] + kf[i] * bw;  // S_t
        dkp[i] = G[i] * bw - X[i] * bg;
        dqp[i] = st * dOc;
        const float e = G[i] - kf[i] * bg;
        dap[i] = e * sp[i];
        da_all += dap[i];
        G[i] = rate(j, i) * e;
      }
      // Row sums over the slice's 16 columns: the wave's columns by lane
      // swaps (when it holds more than one), then the waves through LDS.
      float *red = s_red[par][wave];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        dkp[i] = across_columns<LPC>(dkp[i]);
        dqp[i] = across_columns<LPC>(dqp[i]);
        if constexpr (GATE != KDA_GATE_HEAD) dap[i] = across_columns<LPC>(dap[i]);
      }
      const float db = across_columns<LPC>(gk * w);
      if (lane < LPC) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          red[r0 + i] = dkp[i];
          red[D + r0 + i] = dqp[i];
          if constexpr (GATE != KDA_GATE_HEAD) red[2 * D + r0 + i] = dap[i];
        }
      }
      if constexpr (GATE == KDA_GATE_HEAD) {
        // one rate per head: dalpha sums over every row and column
        const float da = across_columns<LPC>(column_sum<LPC>(da_all));
        if (lane == 0) red[Cf::EB + 1] = da;
      }
      if (lane == 0) red[Cf::EB] = db;
      __syncthreads();
      // The slice's partial row sums of this token, in one contiguous row.
      float *prow = part + ((int64_t)sl * pc.rows * H + (row0 + tb + j) * H + h) * NRED;
      // Two threads per group of four consecutive sums, each adding half of
      // the waves' rows with 16-byte reads, then one lane exchange; the
      // threads sit in the first four waves, one per SIMD.
      if (wave < 4 && lane < Cf::RLW) {
        const int i = wave * Cf::RLW + lane;
        const int g = i >> 1, p = i & 1;  // (the pair of a group is two adjacent lanes)
        if (g < NREDP / 4) {
          const f32x4 *src = reinterpret_cast<const f32x4 *>(&s_red[par][p * (NW / 2)][4 * g]);
          f32x4 acc = src[0];
#pragma unroll
          for (int w2 = 1; w2 < NW / 2; ++w2) acc += src[w2 * (NREDP / 4)];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[m] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[m]), 0xB1, 0xf, 0xf, false));
          const int e = 4 * g + 2 * p;  // this thread stores sums e and e + 1
          if (e < NRED) prow[e] = p ? acc[2] : acc[0];
          if (e + 1 < NRED) prow[e + 1] = p ? acc[3] : acc[1];
        }
      }
      par ^= 1;
    }
  }
  if (pc.G_out != nullptr) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) pc.G_out[sbase + (int64_t)(r0 + i) * D + col] = G[i];
  }
}

// Partial row -> (token row * H + head) of the batch, or -1 for a row past
// its sequence's piece (never written).  row_len = 0: the rows are the
// batch's token rows.
struct RowMap {
  const int32_t *cu;
  int32_t seq_len;
  int H;
  int64_t total, t_off, plen, row_len;
};

template <bool PIECE>
__device__ __forceinline__ int64_t map_row(const RowMap &m, int64_t r) {
  if constexpr (!PIECE) return r;
  const int64_t tok = r / m.H;
  const int h = (int)(r - tok * m.H);
  const int n = (int)(tok / m.row_len);
  const int64_t lt = tok - (int64_t)n * m.row_len;
  int64_t start, len;
  if (m.cu != nullptr) {
    start = m.cu[n];
    len = (int64_t)m.cu[n + 1] - start;
  } else {
    start = (int64_t)n * m.seq_len;
    len = m.seq_len;
  }
  if (start < 0) start = 0;
  if (start > m.total) start = m.total;
  if (len < 0) len = 0;
  if (len > m.total - start) len = m.total - start;
  const int64_t off = m.t_off < len ? m.t_off : len;
  const int64_t plen = len - off < m.plen ? len - off : m.plen;
  return lt < plen ? (start + off + lt) * m.H + h : -1;
}

// dk, dq, dalpha and dbeta = sums of the per-slice partial rows, slice order
// fixed, scattered to their outputs.  Four consecutive sums per thread when
// every slice starts on a 16-byte boundary, with the loads of all slices in
// flight together.
template <int D, int GATE, bool PIECE>
__device__ __forceinline__ void bwd_put(const RowMap &m, int64_t i, float acc, float *__restrict__ dk,
                                        float *__restrict__ dq, float *__restrict__ dalpha,
                                        float *__restrict__ dbeta) {
  constexpr int NRED = bwd_row_sums(D, GATE == KDA_GATE_HEAD);
  constexpr int EB = GATE == KDA_GATE_HEAD ? 2 * D : 3 * D;
  const int64_t r = i / NRED;
  const int e = (int)(i - r * NRED);
  const int64_t th = map_row<PIECE>(m, r);
  if (th < 0) return;
  if (e < D) {
    dk[th * D + e] = acc;
  } else if (e < 2 * D) {
    dq[th * D + e - D] = acc;
  } else if (e < EB) {
    dalpha[th * D + e - 2 * D] = acc;
  } else if (e == EB) {
    dbeta[th] = acc;
  } else {
    dalpha[th] = acc;  // one rate per head
  }
}

template <int D, int GATE, int SL, bool PIECE>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *__restrict__ part, float *__restrict__ dk,
                                                         float *__restrict__ dq, float *__restrict__ dalpha,
                                                         float *__restrict__ dbeta, int64_t rows, const RowMap m) {
  constexpr int NRED = bwd_row_sums(D, GATE == KDA_GATE_HEAD);
  const int64_t n = rows * NRED;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n % 4 == 0) {
    const float4 *p4 = reinterpret_cast<const float4 *>(part);
    const int64_t n4 = n / 4;
    for (int64_t v = first; v < n4; v += stride) {
      float4 x[SL];
#pragma unroll
      for (int s = 0; s < SL; ++s) {  // (read once: non-temporal loads, 1.5% faster over the call)
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p4 + (int64_t)s * n4 + v));
        x[s] = make_float4(t[0], t[1], t[2], t[3]);
      }
      float4 acc = x[0];
#pragma unroll
      for (int s = 1; s < SL; ++s) {
        acc.x += x[s].x;
        acc.y += x[s].y;
        acc.z += x[s].z;
        acc.w += x[s].w;
      }
      bwd_put<D, GATE, PIECE>(m, 4 * v, acc.x, dk, dq, dalpha, dbeta);
      bwd_put<D, GATE, PIECE>(m, 4 * v + 1, acc.y, dk, dq, dalpha, dbeta);
      bwd_put<D, GATE, PIECE>(m, 4 * v + 2, acc.z, dk, dq, dalpha, dbeta);
      bwd_put<D, GATE, PIECE>(m, 4 * v + 3, acc.w, dk, dq, dalpha, dbeta);
    }
  } else {
    for (int64_t i = first; i < n; i += stride) {
      float x[SL];
#pragma unroll
      for (int s = 0; s < SL; ++s) x[s] = part[(int64_t)s * n + i];
      float acc = x[0];
#pragma unroll
      for (int s = 1; s < SL; ++s) acc += x[s];
      bwd_put<D, GATE, PIECE>(m, i, acc, dk, dq, dalpha, dbeta);
    }
  }
}

template <int D, typename TIn, int GATE>
hipError_t launch_bwd_t(const kda_shape_t &s, const BwdArgs &a, const BwdLayout &L, hipStream_t stream) {
  using Cf = BwdCfg<D, TIn, GATE>;
  char *ws = static_cast<char *>(a.workspace);
  float *ckpt = reinterpret_cast<float *>(ws + L.ckpt_off);
  float *part = reinterpret_cast<float *>(ws + L.part_off);
  float *pstate = reinterpret_cast<float *>(ws + L.pstate_off);
  float *carry = reinterpret_cast<float *>(ws + L.carry_off);
  const int64_t blocks = ((int64_t)s.num_seqs * s.num_heads + 7) / 8 * 8 * Cf::SL;
  const int64_t state = (int64_t)s.num_seqs * s.num_heads * D * D;
  const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k),
            *v = static_cast<const TIn *>(a.v);
  auto run = [&](const BwdPiece &pc) -> hipError_t {
    hipLaunchKernelGGL((bwd_kernel<D, TIn, GATE>), dim3((unsigned)blocks), dim3(Cf::NT), 0, stream, q, k, v,
                       a.alpha, a.beta, a.cu, s.seq_len, s.num_seqs, s.num_heads, s.total_tokens, a.dO, a.dv,
                       ckpt, part, pc);
    return hipGetLastError();
  };
  auto reduce = [&](int64_t rows, const RowMap &m) -> hipError_t {
    const int64_t n = rows * s.num_heads * Cf::NRED;
    if (n <= 0) return hipSuccess;
    const int64_t w = n % 4 == 0 ? n / 4 : n;  // work items (four sums each when aligned)
    const int64_t g = (w + 255) / 256 < 8192 ? (w + 255) / 256 : 8192;
    if (m.row_len == 0) {
      hipLaunchKernelGGL((bwd_reduce_kernel<D, GATE, Cf::SL, false>), dim3((unsigned)g), dim3(256), 0, stream, part,
                         a.dk, a.dq, a.dalpha, a.dbeta, rows * s.num_heads, m);
    } else {
      hipLaunchKernelGGL((bwd_reduce_kernel<D, GATE, Cf::SL, true>), dim3((unsigned)g), dim3(256), 0, stream, part,
                         a.dk, a.dq, a.dalpha, a.dbeta, rows * s.num_heads, m);
    }
    return hipGetLastError();
  };
  hipError_t e;
  if (L.L == 0) {  // the whole sequences at once
    e = run(BwdPiece{0, INT64_MAX, 0, 0, s.total_tokens, a.S0, a.dS_T, a.dS0, nullptr});
    if (e != hipSuccess) return e;
    return reduce(s.total_tokens, RowMap{a.cu, s.seq_len, s.num_heads, s.total_tokens, 0, INT64_MAX, 0});
  }
  // Pieces of L tokens: the forward sweep stores the state at every piece
  // start, then the pieces run from last to first.
  const int64_t P = L.pieces, rows = (int64_t)s.num_seqs * L.L;
  if (P > 1) {
    e = run(BwdPiece{0, L.L, 0, 0, 0, a.S0, nullptr, nullptr, pstate});
    if (e != hipSuccess) return e;
  }
  for (int64_t i = P - 1; i >= 0; --i) {
    const float *S_in = i == 0 ? a.S0 : pstate + (i - 1) * state;
    const float *G_in = i == P - 1 ? a.dS_T : carry;
    float *G_out = i == 0 ? a.dS0 : carry;
    e = run(BwdPiece{i * L.L, L.L, L.L / Cf::CK, L.L, rows, S_in, G_in, G_out, nullptr});
    if (e != hipSuccess) return e;
    e = reduce(rows, RowMap{a.cu, s.seq_len, s.num_heads, s.total_tokens, i * L.L, L.L, L.L});
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TIn, int GATE>
hipError_t bwd_by_dim(const kda_shape_t &s, const BwdArgs &a, const BwdLayout &L, hipStream_t st) {
  switch (s.d_k) {
    case 16: return launch_bwd_t<16, TIn, GATE>(s, a, L, st);
    case 32: return launch_bwd_t<32, TIn, GATE>(s, a, L, st);
    case 64: return launch_bwd_t<64, TIn, GATE>(s, a, L, st);
    case 128: return launch_bwd_t<128, TIn, GATE>(s, a, L, st);
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t bwd_by_gate(const kda_shape_t &s, const BwdArgs &a, const BwdLayout &L, hipStream_t st) {
  if (s.gate == KDA_GATE_HEAD) return bwd_by_dim<TIn, KDA_GATE_HEAD>(s, a, L, st);
  return bwd_by_dim<TIn, KDA_GATE_CHANNEL>(s, a, L, st);
}

}  // namespace

hipError_t launch_backward(const kda_shape_t &s, const BwdArgs &a, const BwdLayout &L, hipStream_t stream) {
  if (s.qkv_dtype == KDA_BF16) return bwd_by_gate<__bf16>(s, a, L, stream);
  return bwd_by_gate<float>(s, a, L, stream);
}

}  // namespace kda
