// Internal helpers shared by the HIP kernels of libspectree (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spectree.h"

namespace spectree {

constexpr int kBlockSize = 16;
constexpr int kMaxT = 512;          // tree nodes: ancestor bitsets of 8 x 64 bits
constexpr int kMaxV = 262144;       // rejected-token bitmap of the sampler lives in LDS
// Cache-policy operand of a vector memory instruction: the non-temporal (nt)
// bit, for data read once, which should not displace what the caches hold.
constexpr int kLoadNT = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// A workgroup barrier for data exchanged through LDS only: this wave's LDS
// accesses complete, then the barrier.  Unlike __syncthreads() (a workgroup
// fence, which waits for every outstanding memory access), it leaves direct
// global->LDS loads in flight, so work between their issue and their use
// overlaps their latency.  The LDS it publishes must not be what those loads
// write.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void report(int32_t* status, int b, int32_t bits) {
  if (status != nullptr && bits != 0) atomicOr(status + b, bits);
}

// ---------------------------------------------------------------------------
// launch wrappers implemented in the kernel translation units
// ---------------------------------------------------------------------------

struct AttnPlan {
  int mode;       // 0: fp32 VALU kernel, 2: bf16 tile kernel (> 16 rows), 3: bf16 streaming
                  // kernel (<= 16 rows)
  int rows;       // R = T * G query rows per (sequence, kv head)
  int rt;         // rows per workgroup
  int nrb;        // 16-row blocks per wave
  int n_rt;       // row tiles per (sequence, kv head)
  int splits;     // KV splits per (sequence, kv head)
  int pps;        // pages per split
  long items;     // workgroups of the main kernel (before XCD padding)
  int depth;      // streaming kernel: page slots per wave
  int streamk;    // tile kernel: the stream-K split (ragged batches with more items than resident workgroups)
  int fused;      // spec_tree_write_attn: the write in the attention launch (else two launches)
  size_t ws_bytes;
};

AttnPlan plan_attn(int B, int T, int Hq, int Hkv, int D, int max_blocks, int dtype);

struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* prefix_lens;
  const int32_t* parent;
  void* out;
  int32_t* status;
  void* workspace;
  int B, T, Hq, Hkv, D, max_blocks, num_blocks;
  float scale;
};

hipError_t launch_attn_bf16(const AttnPlan& plan, const AttnLaunch& a, hipStream_t stream);

// The tree's K/V write and the attention in one launch (bf16, head dim 128):
// attn.q holds the queries before rotation; the rotated ones go to the workspace.
struct AttnWriteLaunch {
  AttnLaunch attn;
  const void* k_new;  // [B,T,Hkv,D] keys before rotation
  const void* v_new;  // [B,T,Hkv,D]
  float theta;        // rope base; 0: no rotation
};
AttnPlan plan_attn_write(int B, int T, int Hq, int Hkv, int max_blocks);
hipError_t launch_attn_write(const AttnPlan& plan, const AttnWriteLaunch& w, hipStream_t stream);
void plan_stream(AttnPlan& p, int B, int Hkv, int max_blocks);
hipError_t launch_attn_stream(const AttnPlan& plan, const AttnLaunch& a, hipStream_t stream);
// the same launch with the tree's K/V write (spec_tree_write_attn on a streaming plan)
hipError_t launch_attn_stream_write(const AttnPlan& plan, const AttnWriteLaunch& w, hipStream_t stream);
hipError_t launch_attn_f32(const AttnPlan& plan, const AttnLaunch& a, hipStream_t stream);

struct CompactLaunch {
  void* k;
  void* v;
  const int32_t* block_table;
  const int32_t* prefix_lens;
  const int32_t* accepted;
  const int32_t* num_accepted;
  int32_t* new_lens;
  int32_t* status;
  int B, T, Hkv, D, max_blocks, num_blocks, elem_bytes;
};

struct RejectLaunch {
  const float* logits;
  const float* q;
  const int32_t* tokens;
  const int32_t* parent;
  int B, T, V;
  float temperature;
  int without_replacement;
  uint64_t seed, offset;
  int32_t* accepted;
  int32_t* out_tokens;
  int32_t* num_accepted;
  int32_t* status;
  void* workspace;
  size_t workspace_bytes;
  const CompactLaunch* compact;  // non-null: compact the KV cache along the accepted path in the same launch
  int top_k;    // 1 .. 64: truncate the visited target rows (top-k, then top-p); 0: no truncation
  float top_p;  // > 0; >= 1: top-k only
};

size_t reject_workspace_bytes(int B, int T, int V);
long reject_resident_capacity();  // workgroups of the sampler the current device holds at once (0: unknown)
void reject_plan(int B, int T, int V, long resident, int* team, int* slice);
size_t reject_workspace_zero_bytes();
size_t reject_trunc_workspace_bytes(int B, int T, int V, int top_k);  // sampler with truncation
void reject_trunc_plan(int B, int T, int V, int top_k, long resident, int* team, int* list_len);
constexpr int kTruncTopKMax = 64;  // largest top_k the sampler truncates with
hipError_t launch_reject(const RejectLaunch& a, hipStream_t stream);
size_t reject_static_scratch_bytes();  // size of the allocation-free entry point's device array
hipError_t launch_reject_static(const RejectLaunch& a, hipStream_t stream);  // on that array

hipError_t launch_compact(const CompactLaunch& a, hipStream_t stream);

struct KvWriteLaunch {
  const void* k_new;
  const void* v_new;
  const void* q;  // nullable
  void* q_out;    // where the rotated queries go: q itself (in place) or another [B,T,Hq,D] buffer
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* prefix_lens;
  const int32_t* parent;
  int32_t* status;
  int B, T, Hq, Hkv, D, max_blocks, num_blocks, bf16;
  float theta;
};

hipError_t launch_kv_write(const KvWriteLaunch& a, hipStream_t stream);

struct TruncateLaunch {
  const float* in;
  float* out;  // == in: in place
  int32_t* status;
  int B, T, V;
  float temperature;
  int top_k;
  float top_p;
};

hipError_t launch_truncate(const TruncateLaunch& a, hipStream_t stream);

}  // namespace spectree
