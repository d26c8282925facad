// Internal declarations shared by the host planner, the C-ABI layer and the
// HIP kernels of the segmented KDA forward pass.
#ifndef KDA_INTERNAL_H_
#define KDA_INTERNAL_H_

#include <cstdint>
#include <vector>

namespace kda {

// Fragment flag bits, as serialised in the plan blob.
constexpr int32_t kFragCarried = 1;  // first fragment of a segment that continues a sequence
constexpr int32_t kFragSegLast = 2;  // ends at its segment's end (its state is B_r)
constexpr int32_t kFragSeqEnd = 4;   // ends at its sequence's end (owns final_state)

// Bytes of one chunk-cache slot per head: T diag(beta) of a 32-token chunk
// as bf16 hi and lo parts (2 x 32 x 32 x 2).
constexpr int kChunkCacheBytes = 4096;

// Backward geometry: 1024-thread workgroups, a persistent fragment launch of
// at most kBwdGrid workgroups, and state checkpoints every
// kBwdCheckpointTokens tokens.
constexpr int kBwdThreads = 1024;          // the fragment launch
constexpr int kBwdSummaryThreads = 256;    // the backward-summary launch
constexpr int kBwdGrid = 256;
constexpr int kBwdCheckpointTokens = 16;

// Largest supported packed token count: a chunk-count times 64 times the head
// count stays far inside 32-bit grid arithmetic.
constexpr int32_t kMaxTokens = (1 << 30);

// Word offsets of the arrays inside the plan blob (see kda_plan_blob()).
// The seg_* arrays describe the pieces (the segments themselves when the plan
// has no pieces); the useg_* offsets the segment-level arrays, which alias
// the piece-level ones when there are no pieces (useg_piece_ptr is then -1).
struct BlobLayout {
  int32_t seg_bounds, seg_first_seq, seg_last_seq, seg_carry_in, seg_transition_live,
      seg_frag_ptr, frag_seq, frag_begin, frag_end, frag_seg, frag_flags, seq_end_seg, frag_order;
  int32_t useg_bounds, useg_carry_in, useg_transition_live, useg_piece_ptr;
};

inline BlobLayout blob_layout(int32_t P, int32_t F, int32_t N, int32_t S, bool pieces) {
  BlobLayout L;
  int32_t o = 4;
  L.seg_bounds = o;          o += P + 1;
  L.seg_first_seq = o;       o += P;
  L.seg_last_seq = o;        o += P;
  L.seg_carry_in = o;        o += P;
  L.seg_transition_live = o; o += P;
  L.seg_frag_ptr = o;        o += P + 1;
  L.frag_seq = o;            o += F;
  L.frag_begin = o;          o += F;
  L.frag_end = o;            o += F;
  L.frag_seg = o;            o += F;
  L.frag_flags = o;          o += F;
  L.seq_end_seg = o;         o += N;
  L.frag_order = o;          o += F;
  if (pieces) {
    o += 1;                  // S
    L.useg_bounds = o;          o += S + 1;
    L.useg_carry_in = o;        o += S;
    L.useg_transition_live = o; o += S;
    L.useg_piece_ptr = o;
  } else {
    L.useg_bounds = L.seg_bounds;
    L.useg_carry_in = L.seg_carry_in;
    L.useg_transition_live = L.seg_transition_live;
    L.useg_piece_ptr = -1;
  }
  return L;
}

}  // namespace kda

struct kda_plan {
  int32_t T = 0, N = 0, S = 0, P = 0, F = 0;   // S segments, P pieces (P = S: no pieces)
  bool pieces = false;
  kda::BlobLayout layout{};
  std::vector<int32_t> blob;
};

#endif  // KDA_INTERNAL_H_
