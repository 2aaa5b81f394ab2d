// Selective KV-cache compaction: keep only the accepted root-to-leaf path
// (EAGLE report "Report: Support nextn speculative decoding", important
// implementation detail and the KV-cache rewrite of "Issue: Speculative
// Decoding on vLLM"; SGLang "SpeculativeDecoding", prefix-match eviction).
//
// One workgroup per (sequence, kv head) runs the shared core of compact_dev.h
// on the path the sampler wrote (accepted_nodes, num_accepted).
#include "compact_dev.h"

namespace spectree {
namespace {

__global__ __launch_bounds__(256) void kv_compact_kernel(const CompactLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kCompactStageBytes];
  __shared__ int s_path[kMaxT];
  __shared__ int s_first, s_L;
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;

  if (threadIdx.x == 0) {
    const int L = a.num_accepted[b];
    const bool in = L >= 0 && L < a.T;
    for (int d = 0; in && d <= L; ++d) s_path[d] = a.accepted[static_cast<long>(b) * a.T + d];
    int first = 1 << 30;
    const int err = compact_plan(a, b, a.prefix_lens[b], s_path, in ? L : -1, &first);
    s_first = first;
    s_L = err ? -1 : L;
    if (g == 0) {
      const int Lb = a.prefix_lens[b];
      if (a.new_lens != nullptr) a.new_lens[b] = err ? Lb : Lb + L + 1;
      report(a.status, b, err);
    }
  }
  __syncthreads();
  compact_move(a, b, g, g + 1, a.prefix_lens[b], s_L, s_first, s_path, stage);  // no-op on error, nothing accepted, or a chain
}

}  // namespace

hipError_t launch_compact(const CompactLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_compact_kernel, dim3(static_cast<unsigned>(a.B * a.Hkv)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spectree
