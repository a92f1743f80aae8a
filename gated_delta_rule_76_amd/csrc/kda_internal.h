// Internal interface between the C ABI (kda_api.cpp) and the kernel
// launchers (kda_decode.hip, kda_prefill.hip).  Not installed; not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kChunk = KDA_CHUNK;  // tokens per prefill chunk

// Per chunk and head the prefill keeps one record of matrix-core operand
// fragments in the workspace (written by the chunk-local phase, streamed by
// the state pass): Khat and Qhat (64 x d, as 4 x d/32 fragments each),
// Ktil^T T (d x 64, d/16 x 2 fragments), the six non-zero fragments of the
// lower-triangular M T (64 x 64) and Gamma_C (d floats).  A fragment is
// 2 KiB: one 16x32 operand block as 64 lanes x 8 values, stored either as
// bf16 hi/lo planes or as fp32.
constexpr size_t kFragBytes = 2048;
constexpr size_t kWorkspaceAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int frag_kblocks(int d) { return (d < 32 ? 32 : d) / 32; }
inline size_t record_frags(int d) {
  return (size_t)(4 * frag_kblocks(d) * 2 + (d / 16) * 2 + 6);
}
inline size_t record_bytes(int d) {
  return align_up(record_frags(d) * kFragBytes + sizeof(float) * (size_t)d, kWorkspaceAlign);
}

// Upper bound on the number of 64-token chunks of a batch: every sequence
// contributes at most one partial chunk.
inline int64_t max_chunks(const kda_shape_t &s) {
  return s.total_tokens / kChunk + (int64_t)s.num_seqs;
}

// Prefill workspace: [chunk table: (N+1) int32, then the sequences by
//                     descending chunk count: N int32; padded to 256 B]
//                    [records: W H, slot h W + c - j0]
//                    [carry: N H d_k d_v floats, only if needed]
// The chunks of the batch are numbered in packed order (sequence after
// sequence; the table holds each sequence's first chunk, built on the device
// for a varlen batch and implied by seq_len for a dense one).  The prefill
// runs in stripes of W consecutive packed chunks: stripe i builds the records
// of chunks j0 = iW .. j0+W-1, then the state pass carries the state of every
// sequence with chunks in the stripe across them.  A sequence that continues
// past the stripe leaves its state in S_T, or when S_T is NULL in the carry
// area, for the next stripe.  So W follows from the workspace the caller
// provides and the workspace need not grow with the context:
//   recommended size  table + (floor(T/64) + N) H records: every chunk in
//                     one stripe (the fastest; what the phase entry points
//                     need)
//   minimum size      table + H records (+ the carry area if S_T is NULL)
inline size_t schedule_bytes(const kda_shape_t &s) {
  return align_up(sizeof(int32_t) * (size_t)(2 * s.num_seqs + 1), kWorkspaceAlign);
}
inline size_t prefill_workspace_bytes(const kda_shape_t &s) {
  return schedule_bytes(s) + (size_t)max_chunks(s) * (size_t)s.num_heads * record_bytes(s.d_k);
}
inline size_t carry_bytes(const kda_shape_t &s) {
  return align_up(sizeof(float) * (size_t)s.num_seqs * (size_t)s.num_heads * (size_t)s.d_k * (size_t)s.d_v,
                  kWorkspaceAlign);
}

struct PrefillPlan {
  int64_t chunks;    // packed chunks to cover (exact for a dense batch, an upper bound for varlen)
  int64_t W;         // packed chunks per stripe (>= 1); 0 = the workspace is too small
  int64_t stripes;   // ceil(chunks / W), at least 1
  size_t carry_off;  // offset of the carry area in the workspace, or 0 = none (S_T carries)
};

inline PrefillPlan prefill_plan(const kda_shape_t &s, bool varlen, bool has_final_state,
                                size_t workspace_bytes) {
  PrefillPlan p{0, 0, 1, 0};
  if (s.num_seqs <= 0 || s.num_heads <= 0) return p;
  const int64_t per_seq = s.seq_len > 0 ? ((int64_t)s.seq_len + kChunk - 1) / kChunk : 0;
  p.chunks = varlen ? max_chunks(s) : (int64_t)s.num_seqs * per_seq;
  const int64_t need = p.chunks > 0 ? p.chunks : 1;
  const size_t table = schedule_bytes(s);
  const size_t rec = (size_t)s.num_heads * record_bytes(s.d_k);  // one packed chunk, all heads
  // grid limit of the chunk-local kernel: W H < 2^31
  const int64_t wmax = ((int64_t)1 << 31) / s.num_heads - 1;
  auto fit = [&](size_t reserve) -> int64_t {
    if (workspace_bytes < table + reserve) return 0;
    int64_t w = (int64_t)((workspace_bytes - table - reserve) / rec);
    return w < need ? (w < wmax ? w : wmax) : (need < wmax ? need : wmax);
  };
  int64_t W = fit(0);
  if (W < need && !has_final_state) {  // several stripes: the carry needs room too
    W = fit(carry_bytes(s));
    p.carry_off = table + (size_t)W * rec;  // records are multiples of 256 B
  }
  if (W <= 0) return p;
  p.W = W;
  p.stripes = (need + W - 1) / W;
  if (p.stripes == 1) p.carry_off = 0;
  return p;
}

hipError_t launch_decode(const kda_shape_t &s, const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta, float *S, float *o,
                         hipStream_t stream);

// s.seq_len tokens per sequence; hist == nullptr advances S in place.
hipError_t launch_decode_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, float *S, float *o, float *hist,
                                hipStream_t stream);

hipError_t launch_commit(const kda_shape_t &s, float *S, const float *hist, const int32_t *accepted,
                         hipStream_t stream);

// s.seq_len tokens per sequence from S, outputs only (S is not written).
hipError_t launch_verify_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, const float *S, float *o,
                                hipStream_t stream);

// S advanced in place by the first accepted[n] (clamped to [0, s.seq_len])
// of each sequence's s.seq_len tokens; no outputs.
hipError_t launch_accept_tokens(const kda_shape_t &s, const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta, float *S, const int32_t *accepted,
                                hipStream_t stream);

// S advanced in place by the first accepted[n] of the previous round's
// tokens (q0 .. beta0), then the outputs of this round's tokens from it (S
// keeps the former).
hipError_t launch_accept_verify_tokens(const kda_shape_t &s, const void *q0, const void *k0, const void *v0,
                                       const float *alpha0, const float *beta0, const int32_t *accepted,
                                       const void *q, const void *k, const void *v, const float *alpha,
                                       const float *beta, float *S, float *o, hipStream_t stream);

// Backward pass.  Workspace: state checkpoints every bwd_block tokens per
// (sequence, head) -- d_k x d_v floats per slot -- then the per-slice
// partial row sums over the d_v / 16 column slices, [slices][rows][H]
// [bwd_row_sums] floats: per (token, head) dk (d), dq (d), then dalpha (d) and
// dbeta, or with one rate per head dbeta and dalpha.  The block is 16 tokens
// at d <= 64; at d = 128, 12 for bf16 inputs and 8 for fp32 ones (the block's
// states and inputs have to fit in LDS).
//
// With the recommended workspace every sequence is one piece: checkpoint
// slots packed over the batch (at most floor(T / block) + N) and one partial
// row per token.  With less, every sequence is cut into pieces of L tokens
// (L a multiple of 48, so of every block size): a forward sweep stores the
// state at each piece start, then the pieces run from last to first, the
// state gradient handed from piece to piece through a carry buffer.  The
// workspace then holds, in this order: the piece-start states [P-1][N][H]
// [d_k][d_v], the carry [N][H][d_k][d_v], checkpoint slots [N][L/block][H]
// and partial rows [slices][N][L][H] -- nothing that grows with the context
// beyond the P-1 piece-start states.
constexpr int bwd_block(int d, bool f32_inputs) { return d >= 128 ? (f32_inputs ? 8 : 12) : 16; }
constexpr int bwd_row_sums(int d, bool head_gate) { return head_gate ? 2 * d + 2 : 3 * d + 1; }
constexpr int64_t kBwdPieceUnit = 48;

struct BwdLayout {
  int64_t pieces;    // P (1: the whole sequences at once)
  int64_t L;         // piece length in tokens (P > 1)
  size_t pstate_off, carry_off, ckpt_off, part_off, bytes;
};

// Layout for pieces of L tokens (L = 0: one piece, the recommended layout).
inline BwdLayout backward_layout(const kda_shape_t &s, bool varlen = true, int64_t L = 0) {
  const size_t d = (size_t)s.d_k, H = (size_t)s.num_heads, T = (size_t)s.total_tokens;
  const size_t N = (size_t)s.num_seqs;
  const size_t slices = d < 16 ? 1 : d / 16;
  const int blk = bwd_block(s.d_k, s.qkv_dtype == KDA_F32);
  const size_t nred = (size_t)bwd_row_sums(s.d_k, s.gate == KDA_GATE_HEAD);
  const size_t state = sizeof(float) * N * H * d * (size_t)s.d_v;  // [N][H][d_k][d_v]
  BwdLayout Lo{1, 0, 0, 0, 0, 0, 0};
  if (L <= 0) {
    const size_t slots = (size_t)(s.total_tokens / blk) + N;
    Lo.ckpt_off = 0;
    Lo.part_off = align_up(sizeof(float) * slots * H * d * (size_t)s.d_v, kWorkspaceAlign);
    Lo.bytes = align_up(Lo.part_off + sizeof(float) * slices * T * H * nred, kWorkspaceAlign);
    return Lo;
  }
  const int64_t maxlen = varlen ? s.total_tokens : (int64_t)s.seq_len;
  Lo.L = L;
  Lo.pieces = maxlen > L ? (maxlen + L - 1) / L : 1;
  Lo.pstate_off = 0;
  Lo.carry_off = align_up((size_t)(Lo.pieces - 1) * state, kWorkspaceAlign);
  Lo.ckpt_off = align_up(Lo.carry_off + state, kWorkspaceAlign);
  Lo.part_off = align_up(Lo.ckpt_off + (size_t)(L / blk) * state, kWorkspaceAlign);
  Lo.bytes = align_up(Lo.part_off + sizeof(float) * slices * N * (size_t)L * H * nred, kWorkspaceAlign);
  return Lo;
}

// The layout a workspace of `bytes` allows: one piece if it holds the
// recommended layout, else the longest pieces that fit (pieces = 0: none).
inline BwdLayout backward_plan(const kda_shape_t &s, bool varlen, size_t bytes) {
  const BwdLayout one = backward_layout(s);
  if (bytes >= one.bytes) return one;
  const int64_t maxlen = varlen ? s.total_tokens : (int64_t)s.seq_len;
  for (int64_t m = (maxlen + kBwdPieceUnit - 1) / kBwdPieceUnit; m >= 1; --m) {
    const BwdLayout Lo = backward_layout(s, varlen, m * kBwdPieceUnit);
    if (Lo.bytes <= bytes) return Lo;
  }
  BwdLayout none{};
  return none;
}

struct BwdArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const int32_t *cu;
  const float *S0, *dO, *dS_T;
  float *dq, *dk, *dv, *dalpha, *dbeta, *dS0;
  void *workspace;
};

// Runs the backward with layout L (backward_plan of the workspace).
hipError_t launch_backward(const kda_shape_t &s, const BwdArgs &a, const BwdLayout &L, hipStream_t stream);

// Prefill phases (bit mask): the chunk table and chunk-local matrices, then
// the sequential state pass.
constexpr int kPhaseLocal = 1;
constexpr int kPhaseState = 2;

// Runs the stripes of `plan` (phases: both, or one of them for a one-stripe
// plan).
hipError_t launch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          const float *S0, float *o, float *S_T, void *workspace,
                          const PrefillPlan &plan, hipStream_t stream, int phases);

}  // namespace kda
