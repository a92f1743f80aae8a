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

// Workspace layout: [chunk base table: (N+1) int32, padded to 256 B]
//                   [records: max_chunks * H * record_bytes(d)]
inline size_t schedule_bytes(const kda_shape_t &s) {
  return align_up(sizeof(int32_t) * (size_t)(s.num_seqs + 1), kWorkspaceAlign);
}
inline size_t prefill_workspace_bytes(const kda_shape_t &s) {
  return schedule_bytes(s) + (size_t)max_chunks(s) * (size_t)s.num_heads * record_bytes(s.d_k);
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

// Backward pass.  Workspace: state checkpoints every bwd_block tokens per
// (sequence, head) -- at most floor(T / bwd_block) + N slots of d_k x d_v
// floats per head -- then the per-slice partial row sums over the d_v / 16
// column slices, [slices][T][H][bwd_row_sums] floats: per (token, head) dk
// (d), dq (d), then dalpha (d) and dbeta, or with one rate per head dbeta and
// dalpha.  The block is 16 tokens at d <= 64; at d = 128, 12 for bf16 inputs
// and 8 for fp32 ones (the block's states and inputs have to fit in LDS).
constexpr int bwd_block(int d, bool f32_inputs) { return d >= 128 ? (f32_inputs ? 8 : 12) : 16; }
constexpr int bwd_row_sums(int d, bool head_gate) { return head_gate ? 2 * d + 2 : 3 * d + 1; }

struct BwdLayout {
  size_t ckpt_off, part_off, bytes;
};

inline BwdLayout backward_layout(const kda_shape_t &s) {
  const size_t d = (size_t)s.d_k, H = (size_t)s.num_heads, T = (size_t)s.total_tokens;
  const size_t slices = d < 16 ? 1 : d / 16;
  const int blk = bwd_block(s.d_k, s.qkv_dtype == KDA_F32);
  const size_t slots = (size_t)(s.total_tokens / blk) + (size_t)s.num_seqs;
  const size_t nred = (size_t)bwd_row_sums(s.d_k, s.gate == KDA_GATE_HEAD);
  BwdLayout L;
  L.ckpt_off = 0;
  L.part_off = align_up(L.ckpt_off + sizeof(float) * slots * H * d * (size_t)s.d_v, kWorkspaceAlign);
  L.bytes = align_up(L.part_off + sizeof(float) * slices * T * H * nred, kWorkspaceAlign);
  return L;
}

struct BwdArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const int32_t *cu;
  const float *S0, *dO, *dS_T;
  float *dq, *dk, *dv, *dalpha, *dbeta, *dS0;
  void *workspace;
};

hipError_t launch_backward(const kda_shape_t &s, const BwdArgs &a, hipStream_t stream);

// Prefill phases (bit mask): the chunk table and chunk-local matrices, then
// the sequential state pass.
constexpr int kPhaseLocal = 1;
constexpr int kPhaseState = 2;

hipError_t launch_prefill(const kda_shape_t &s, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, const int32_t *cu_seqlens,
                          const float *S0, float *o, float *S_T, void *workspace,
                          hipStream_t stream, int phases);

}  // namespace kda
