// Kernel parameter blocks and entry points shared by the C-ABI layer and the
// HIP kernels of the segmented KDA forward pass.
#ifndef KDA_KERNELS_H_
#define KDA_KERNELS_H_

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_internal.h"

namespace kda {

constexpr int kSummaryThreads = 1024;  // kda_chunk_kernel (summaries launch): 16 waves
constexpr int kCarryThreads = 768;    // kda_carry_kernel (carry launch): 12 waves
constexpr int kComposeThreads = 1024;  // kda_compose_kernel workgroup size: 16 waves
constexpr int kComposeColumns = 16;      // state columns per compose workgroup
constexpr int kComposeColumnBlocks = 128 / kComposeColumns;
constexpr int kChainThreads = 768;     // kda_bwd_chain_kernel: 12 waves
constexpr int kGradThreads = 1024;     // kda_bwd_grad_kernel: 16 waves

struct ChunkParams {
  const int32_t* plan;   // device copy of the plan blob
  BlobLayout L;
  int32_t H;             // heads in the tensors (their stride)
  int32_t h0;            // heads [h0, h0 + hn) are this launch's
  int32_t hn;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  float* o;              // [T, H, V], FP32, or BF16 bits when o_bf16 is set
  int32_t o_bf16;
  int32_t gate_floor_on;  // the optional gate lower bound is set
  float gate_floor;       // that bound in log2 units (-inf when not set)
  float* final_state;
  float* transitions;
  float* updates;
  const float* carry;
  const float* init_state;  // per-sequence initial states [N, H, K, V], or null (zero)
  uint16_t* chunk_cache;  // T diag(beta) per chunk of the fragments that end a segment
  // checkpoint launch (the chunked backward): the state entering every chunk,
  // rows scaled by the chunk's anchor, at slot floor(begin / 32) + f + chunk;
  // and per (fragment, head) item 1 where the fragment left the anchored
  // form's range (its checkpoints are not valid), else 0
  float* ckpt;
  int32_t* item_flag;
  int32_t* slot_map;   // per chunk slot: the fragment whose chunk it holds, -1 where none
  float* rv_out;       // per chunk slot: V - Kr R of the chunk, [32 tokens][V] FP32
};

// Chunk cache: slot of chunk `it` of the fragment that ends segment r and
// starts at token b_r is floor(b_r / 32) + r + it (its last slot is below
// ceil(e_r / 32) + r for the segment end e_r, the next segment's first is at
// least floor(e_r / 32) + r + 1, so segments never share one); a slot holds,
// per head, T diag(beta) as
// [hi | lo] x [32 rows] x [32 columns in k-slot order] bf16 = kChunkCacheBytes.
__host__ __device__ inline int64_t chunk_cache_slot(int32_t seg, int32_t frag_begin, int32_t it) {
  return static_cast<int64_t>(frag_begin / 32) + seg + it;
}

struct ComposeParams {
  const int32_t* plan;
  BlobLayout L;
  int32_t H;    // heads in the tensors
  int32_t h0;   // heads [h0, h0 + hn) are composed by this launch
  int32_t hn;
  int32_t S;          // steps of the one chain (compose, reverse): segments or pieces
  int32_t live_off;   // plan word offset of the transition flags of those steps
  int32_t chains;     // fold, piece carry: one chain per segment
  const float* transitions;
  const float* updates;
  float* carry;       // compose, reverse, piece carry: every step's value
  const float* init;  // piece carry: the segments' carry-ins
  float* out_a;       // fold: the segments' transitions
  float* out_b;       // fold: the segments' updates
};

// Backward (kda_backward); its geometry constants are in kda_internal.h.
struct BwdParams {
  const int32_t* plan;
  BlobLayout L;
  int32_t H;              // heads in the tensors
  int32_t h0;             // heads [h0, h0 + hn) are this launch's
  int32_t hn;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const float* h0s;       // initial states [N, H, K, V] or null (zero)
  const float* d_o;       // dL/do [T, H, V]
  const float* dfinal;    // dL/dfinal [N, H, K, V] or null (zero)
  const float* carry;     // the forward's carry-in C_r [S, H, K, V]
  float* esum;            // E_r [S, H, K, V] (written by the summary launch)
  const float* dcarry;    // D_r [S, H, K, V] (the reverse compose of E)
  float* dq;
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;
  float* dh0;             // dL/dh0 [N, H, K, V] or null (not wanted)
  float* ckpt;            // state checkpoints: slot floor(begin/16) + f + j per head
  float* upbuf;           // u and p of every token [T, H, 2, V] (the fragment launch's level 1)
  // chunked path, per chunk slot floor(begin/32) + f + c and head: the
  // anchored state entering the chunk, the anchored cotangent of the state
  // leaving it, T diag(beta); per (fragment, head) the path flag (1: the
  // token-by-token path), per slot its fragment (-1: none)
  const float* ck32;
  float* dcot;
  const uint16_t* tcache;
  const int32_t* iflag;
  int32_t* smap;
  const float* rvbuf;     // per chunk slot: V - Kr R (checkpoint launch), [32][V]
  float* dubuf;           // per chunk slot: dU = P^T dO + Kc D (chain launch), [32][V]
  int32_t nslots;         // chunk slots (slots x hn < 2^31)
};

__global__ void kda_chunk_kernel(ChunkParams p);
__global__ void kda_backward_summary_kernel(BwdParams p);         // kBwdThreads threads
__global__ void kda_backward_summary_narrow_kernel(BwdParams p);  // kBwdSummaryThreads threads
__global__ void kda_backward_forward_kernel(BwdParams p);         // kBwdThreads threads
__global__ void kda_backward_fragment_kernel(BwdParams p);        // kBwdThreads threads
__global__ void kda_carry_kernel(ChunkParams p);
__global__ void kda_ckpt_kernel(ChunkParams p);   // kCarryThreads threads
__global__ void kda_bwd_chain_e_kernel(BwdParams p);   // kChainThreads threads, one per (piece, head)
__global__ void kda_bwd_chain_kernel(BwdParams p);     // kChainThreads threads, one per (fragment, head)
__global__ void kda_bwd_grad_kernel(BwdParams p);      // kGradThreads threads, persistent over (chunk slot, head)
__global__ void kda_compose_kernel(ComposeParams p);
__global__ void kda_compose_reverse_kernel(ComposeParams p);
__global__ void kda_fold_pieces_kernel(ComposeParams p);
__global__ void kda_piece_carry_kernel(ComposeParams p);

}  // namespace kda

#endif  // KDA_KERNELS_H_
