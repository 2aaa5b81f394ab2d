// Selective KV-cache compaction: keep only the accepted root-to-leaf path
// (EAGLE report "Report: Support nextn speculative decoding", important
// implementation detail and the KV-cache rewrite of "Issue: Speculative
// Decoding on vLLM"; SGLang "SpeculativeDecoding", prefix-match eviction).
//
// One workgroup per (sequence, kv head).  The path n_0 = 0 < n_1 < ... < n_L
// has n_d >= d, so row d is a no-op until the first d with n_d != d, and every
// later row moves.  A destination d can be the source of an earlier row d' < d
// (n_d' = d) but never of a later one (n_d'' > d for d'' > d), so rows are
// moved in chunks of increasing d: each chunk is first read completely into
// LDS, then written.  The result equals doing the copies one by one in
// increasing d.
#include "common.h"

namespace spectree {
namespace {

constexpr int kStageBytes = 32768;

__global__ __launch_bounds__(256) void kv_compact_kernel(const CompactLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStageBytes];
  __shared__ int s_path[kMaxT];
  __shared__ int s_first, s_L;
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x;
  const int32_t* bt_b = a.block_table + static_cast<long>(b) * a.max_blocks;

  if (tid == 0) {
    int err = 0;
    int L = a.num_accepted[b];
    int Lb = a.prefix_lens[b];
    if (Lb < 0 || Lb > a.max_blocks * kBlockSize - a.T) err |= SPEC_DEV_LENGTH;
    if (L < 0 || L >= a.T) err |= SPEC_DEV_PATH;
    int first = 1 << 30;
    if (!err) {
      int prev = -1;
      for (int d = 0; d <= L; ++d) {
        const int n = a.accepted[static_cast<long>(b) * a.T + d];
        if ((d == 0 && n != 0) || n <= prev || n >= a.T) {
          err |= SPEC_DEV_PATH;
          break;
        }
        s_path[d] = n;
        if (n != d && first > d) first = d;
        prev = n;
      }
    }
    if (!err) {  // every page a moved row touches must be a valid block
      for (int d = (first < L + 1 ? first : L + 1); d <= L; ++d) {
        const int ps = (Lb + s_path[d]) / kBlockSize, pd = (Lb + d) / kBlockSize;
        const int bs = bt_b[ps], bd = bt_b[pd];
        if (bs < 0 || bs >= a.num_blocks || bd < 0 || bd >= a.num_blocks) {
          err |= SPEC_DEV_BLOCK;
          break;
        }
      }
    }
    s_first = first;
    s_L = err ? -1 : L;
    if (g == 0) {
      if (a.new_lens != nullptr) a.new_lens[b] = err ? Lb : Lb + L + 1;
      report(a.status, b, err);
    }
  }
  __syncthreads();
  const int L = s_L;
  const int first = s_first;
  if (L < 1 || first > L) return;  // error, nothing accepted, or a pure no-op (chain)
  const int Lb = a.prefix_lens[b];

  const int row_bytes = a.D * a.elem_bytes;  // 256 or 512
  const int chunks = row_bytes / 16;         // 16-byte pieces per row
  const int rows_per_stage = kStageBytes / (2 * row_bytes);
  for (int d0 = first; d0 <= L; d0 += rows_per_stage) {
    const int nrows = min(rows_per_stage, L + 1 - d0);
    const int pieces = nrows * chunks;
    for (int i = tid; i < 2 * pieces; i += 256) {
      const int kv = i / pieces, rem = i % pieces;
      const int r = rem / chunks, c = rem % chunks;
      const int src = Lb + s_path[d0 + r];
      const long off = ((static_cast<long>(bt_b[src / kBlockSize]) * a.Hkv + g) * kBlockSize + src % kBlockSize) * row_bytes + c * 16;
      const uint8_t* base = static_cast<const uint8_t*>(kv ? a.v : a.k);
      *reinterpret_cast<u32x4*>(stage + i * 16) = *reinterpret_cast<const u32x4*>(base + off);
    }
    __syncthreads();
    for (int i = tid; i < 2 * pieces; i += 256) {
      const int kv = i / pieces, rem = i % pieces;
      const int r = rem / chunks, c = rem % chunks;
      const int dst = Lb + d0 + r;
      const long off = ((static_cast<long>(bt_b[dst / kBlockSize]) * a.Hkv + g) * kBlockSize + dst % kBlockSize) * row_bytes + c * 16;
      uint8_t* base = static_cast<uint8_t*>(kv ? a.v : a.k);
      *reinterpret_cast<u32x4*>(base + off) = *reinterpret_cast<const u32x4*>(stage + i * 16);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_compact(const CompactLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_compact_kernel, dim3(static_cast<unsigned>(a.B * a.Hkv)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spectree
