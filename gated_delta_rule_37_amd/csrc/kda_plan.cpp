// Host-side segment planner for the segmented KDA forward pass.
//
// Builds the contiguous segment plan over packed sequences (inclusionAI/cuLA
// pull request #136 "feat(kda): add cuDNN concatenated-summary Kimi CP",
// Walkthrough, "Packed-shard planning": CPU-only balanced or custom contiguous
// shards over the global sequence boundaries, with input validation) and its
// canonical int32 serialisation, which the device kernels read.  No HIP call
// is made here.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

// Index n such that bounds[n] <= t < bounds[n + 1] (bounds strictly increasing).
int32_t locate(const std::vector<int32_t>& bounds, int32_t t) {
  auto it = std::upper_bound(bounds.begin(), bounds.end(), t);
  return static_cast<int32_t>(it - bounds.begin()) - 1;
}

}  // namespace

extern "C" int kda_plan_segments_pieces(const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_segments,
                                        const int32_t* custom_bounds, int32_t piece_tokens, kda_plan** out) {
  if (cu_seqlens == nullptr || out == nullptr) return KDA_ERR_INVALID_ARG;
  if (num_seqs < 1) return KDA_ERR_BAD_CU_SEQLENS;
  if (cu_seqlens[0] != 0) return KDA_ERR_BAD_CU_SEQLENS;
  for (int32_t n = 0; n < num_seqs; ++n) {
    if (cu_seqlens[n + 1] <= cu_seqlens[n]) return KDA_ERR_BAD_CU_SEQLENS;
  }
  const int32_t T = cu_seqlens[num_seqs];
  // Token offsets times H * 128 stay well inside size_t, but a chunk index
  // times the head count must fit int32 in the launch grid.
  if (T > kda::kMaxTokens) return KDA_ERR_UNSUPPORTED;
  const int32_t S = num_segments;
  if (S < 1 || S > T) return KDA_ERR_BAD_SEGMENTS;
  if (piece_tokens < 0 || piece_tokens % 32 != 0) return KDA_ERR_BAD_SEGMENTS;

  std::vector<int32_t> cu(cu_seqlens, cu_seqlens + num_seqs + 1);
  std::vector<int32_t> b(S + 1);
  if (custom_bounds == nullptr) {
    for (int32_t r = 0; r <= S; ++r) {
      b[r] = static_cast<int32_t>((static_cast<int64_t>(r) * T) / S);
    }
  } else {
    for (int32_t r = 0; r <= S; ++r) b[r] = custom_bounds[r];
    if (b[0] != 0 || b[S] != T) return KDA_ERR_BAD_SEGMENTS;
    for (int32_t r = 0; r < S; ++r) {
      if (b[r + 1] <= b[r]) return KDA_ERR_BAD_SEGMENTS;
    }
  }

  kda_plan* plan = new (std::nothrow) kda_plan;
  if (plan == nullptr) return KDA_ERR_NO_MEMORY;
  try {
    // Pieces: each segment cut every piece_tokens tokens from its start (the
    // last piece shorter); without pieces the pieces are the segments.
    std::vector<int32_t> pb, piece_ptr(S + 1);
    for (int32_t r = 0; r < S; ++r) {
      piece_ptr[r] = static_cast<int32_t>(pb.size());
      pb.push_back(b[r]);
      if (piece_tokens > 0) {
        for (int64_t x = static_cast<int64_t>(b[r]) + piece_tokens; x < b[r + 1]; x += piece_tokens)
          pb.push_back(static_cast<int32_t>(x));
      }
    }
    piece_ptr[S] = static_cast<int32_t>(pb.size());
    pb.push_back(T);
    const int32_t P = static_cast<int32_t>(pb.size()) - 1;
    const bool pieces = P > S;

    plan->T = T;
    plan->N = num_seqs;
    plan->S = S;
    plan->P = P;
    plan->pieces = pieces;
    // carry-in and live flags of a list of bounds (segments or pieces)
    auto flags_of = [&](const std::vector<int32_t>& bb, int32_t R, std::vector<int32_t>& first,
                        std::vector<int32_t>& last, std::vector<int32_t>& carry, std::vector<int32_t>& live) {
      first.resize(R);
      last.resize(R);
      carry.resize(R);
      live.resize(R);
      for (int32_t r = 0; r < R; ++r) {
        first[r] = locate(cu, bb[r]);
        last[r] = locate(cu, bb[r + 1] - 1);
        const bool starts_here = cu[first[r]] == bb[r];
        carry[r] = (r > 0 && !starts_here) ? 1 : 0;
        live[r] = (carry[r] && first[r] == last[r]) ? 1 : 0;
      }
    };
    std::vector<int32_t> first, last, carry, live, frag_ptr(P + 1);
    flags_of(pb, P, first, last, carry, live);
    std::vector<int32_t> f_seq, f_beg, f_end, f_seg, f_flags;
    frag_ptr[0] = 0;
    for (int32_t r = 0; r < P; ++r) {
      for (int32_t n = first[r]; n <= last[r]; ++n) {
        const int32_t lo = std::max(pb[r], cu[n]);
        const int32_t hi = std::min(pb[r + 1], cu[n + 1]);
        int32_t flags = 0;
        if (lo == pb[r] && carry[r]) flags |= kda::kFragCarried;
        if (hi == pb[r + 1]) flags |= kda::kFragSegLast;
        if (hi == cu[n + 1]) flags |= kda::kFragSeqEnd;
        f_seq.push_back(n);
        f_beg.push_back(lo);
        f_end.push_back(hi);
        f_seg.push_back(r);
        f_flags.push_back(flags);
      }
      frag_ptr[r + 1] = static_cast<int32_t>(f_seq.size());
    }
    const int32_t F = static_cast<int32_t>(f_seq.size());
    plan->F = F;
    std::vector<int32_t> end_seg(num_seqs);
    for (int32_t n = 0; n < num_seqs; ++n) end_seg[n] = locate(pb, cu[n + 1] - 1);
    // launch order: longest fragments first (ties by index), so that the long
    // sequential chains are not the last to start
    std::vector<int32_t> order(F);
    for (int32_t f = 0; f < F; ++f) order[f] = f;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      return f_end[x] - f_beg[x] > f_end[y] - f_beg[y];
    });

    std::vector<int32_t>& blob = plan->blob;
    blob.reserve(4 + (P + 1) * 2 + P * 4 + F * 6 + num_seqs + (pieces ? 3 * S + 3 : 0));
    blob.insert(blob.end(), {T, num_seqs, P, F});
    auto append = [&blob](const std::vector<int32_t>& a) { blob.insert(blob.end(), a.begin(), a.end()); };
    append(pb);
    append(first);
    append(last);
    append(carry);
    append(live);
    append(frag_ptr);
    append(f_seq);
    append(f_beg);
    append(f_end);
    append(f_seg);
    append(f_flags);
    append(end_seg);
    append(order);
    if (pieces) {
      std::vector<int32_t> ufirst, ulast, ucarry, ulive;
      flags_of(b, S, ufirst, ulast, ucarry, ulive);
      blob.push_back(S);
      append(b);
      append(ucarry);
      append(ulive);
      append(piece_ptr);
    }
    plan->layout = kda::blob_layout(P, F, num_seqs, S, pieces);
  } catch (const std::bad_alloc&) {
    delete plan;
    return KDA_ERR_NO_MEMORY;
  }
  *out = plan;
  return KDA_OK;
}

extern "C" int kda_plan_segments(const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_segments,
                                 const int32_t* custom_bounds, kda_plan** out) {
  return kda_plan_segments_pieces(cu_seqlens, num_seqs, num_segments, custom_bounds, 0, out);
}

extern "C" int kda_plan_blob(const kda_plan* plan, const int32_t** blob, size_t* n_int32) {
  if (plan == nullptr || blob == nullptr || n_int32 == nullptr) return KDA_ERR_INVALID_ARG;
  *blob = plan->blob.data();
  *n_int32 = plan->blob.size();
  return KDA_OK;
}

extern "C" int kda_plan_info(const kda_plan* plan, int32_t* T, int32_t* N, int32_t* S,
                             int32_t* F) {
  if (plan == nullptr) return KDA_ERR_INVALID_ARG;
  if (T) *T = plan->T;
  if (N) *N = plan->N;
  if (S) *S = plan->S;
  if (F) *F = plan->F;
  return KDA_OK;
}

extern "C" int kda_plan_pieces(const kda_plan* plan, int32_t* P) {
  if (plan == nullptr || P == nullptr) return KDA_ERR_INVALID_ARG;
  *P = plan->P;
  return KDA_OK;
}

extern "C" void kda_plan_destroy(kda_plan* plan) { delete plan; }

extern "C" size_t kda_summary_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V) {
  if (plan == nullptr || H <= 0 || K <= 0 || V <= 0) return 0;
  const size_t per_head = static_cast<size_t>(K) * K + static_cast<size_t>(K) * V;
  return static_cast<size_t>(plan->S) * static_cast<size_t>(H) * per_head * sizeof(float);
}

extern "C" const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_BAD_CU_SEQLENS: return "KDA_ERR_BAD_CU_SEQLENS";
    case KDA_ERR_BAD_SEGMENTS: return "KDA_ERR_BAD_SEGMENTS";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_NO_MEMORY: return "KDA_ERR_NO_MEMORY";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_BUFFER_TOO_SMALL: return "KDA_ERR_BUFFER_TOO_SMALL";
    default: return "KDA_ERR_UNKNOWN";
  }
}
