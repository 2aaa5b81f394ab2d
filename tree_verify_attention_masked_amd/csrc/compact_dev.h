// Selective KV-cache compaction, the per-(sequence, kv head) core shared by the
// standalone kernel (compact.hip) and the sampler's fused tail (reject.hip):
// keep only the accepted root-to-leaf path (EAGLE report "Report: Support nextn
// speculative decoding", important implementation detail and the KV-cache
// rewrite of "Issue: Speculative Decoding on vLLM"; SGLang
// "SpeculativeDecoding", prefix-match eviction).
//
// The path n_0 = 0 < n_1 < ... < n_L has n_d >= d, so row d is a no-op until
// the first d with n_d != d, and every later row moves.  A destination d can
// be the source of an earlier row d' < d (n_d' = d) but never of a later one
// (n_d'' > d for d'' > d), so rows are moved in chunks of increasing d: each
// chunk is first read completely into LDS, then written.  The result equals
// doing the copies one by one in increasing d.
#pragma once

#include "common.h"

namespace spectree {

constexpr int kCompactStageBytes = 32768;  // LDS staging for one chunk of rows (K and V)

// One thread: checks the prefix length Lb (= prefix_lens[b]), the path
// path[0..L] (0 first, strictly increasing, below T) and every block a moved
// row touches.  Returns the device error bits (0 if the rows may move) and the
// first moved row in *first (> L when nothing moves).
__device__ inline int compact_plan(const CompactLaunch& c, int b, int Lb, const int* path, int L, int* first) {
  int err = 0;
  if (Lb < 0 || Lb > c.max_blocks * kBlockSize - c.T) err |= SPEC_DEV_LENGTH;
  if (L < 0 || L >= c.T) err |= SPEC_DEV_PATH;
  int f = 1 << 30;
  if (!err) {
    int prev = -1;
    for (int d = 0; d <= L; ++d) {
      const int n = path[d];
      if ((d == 0 && n != 0) || n <= prev || n >= c.T) {
        err |= SPEC_DEV_PATH;
        break;
      }
      if (n != d && f > d) f = d;
      prev = n;
    }
  }
  if (!err) {  // every page a moved row touches must be a valid block
    const int32_t* bt_b = c.block_table + static_cast<long>(b) * c.max_blocks;
    for (int d = (f < L + 1 ? f : L + 1); d <= L; ++d) {
      const int ps = (Lb + path[d]) / kBlockSize, pd = (Lb + d) / kBlockSize;
      const int bs = bt_b[ps], bd = bt_b[pd];
      if (bs < 0 || bs >= c.num_blocks || bd < 0 || bd >= c.num_blocks) {
        err |= SPEC_DEV_BLOCK;
        break;
      }
    }
  }
  *first = f;
  return err;
}

// The whole workgroup (256 threads, every thread calls it): moves rows
// first..L of kv heads g0 .. g1-1 of sequence b (prefix length Lb), as planned,
// through `stage` (kCompactStageBytes of LDS).  Rows go in chunks of increasing
// d; a chunk holds those rows of as many heads as the stage takes (heads are
// independent, so their order within a chunk does not matter).  A no-op when
// first > L.
__device__ inline void compact_move(const CompactLaunch& c, int b, int g0, int g1, int Lb, int L, int first,
                                    const int* path, uint8_t* stage) {
  if (L < 1 || first > L || g1 <= g0) return;
  const int32_t* bt_b = c.block_table + static_cast<long>(b) * c.max_blocks;
  const int tid = threadIdx.x;
  const int row_bytes = c.D * c.elem_bytes;  // 256 or 512
  const int chunks = row_bytes / 16;         // 16-byte pieces per row
  const int pair_cap = kCompactStageBytes / (2 * row_bytes);  // (head, row) pairs per stage, K and V
  const int nh = g1 - g0;
  const int rows_per_stage = max(1, pair_cap / nh);
  const int heads_per_stage = min(nh, pair_cap / rows_per_stage);
  for (int d0 = first; d0 <= L; d0 += rows_per_stage) {
    const int nrows = min(rows_per_stage, L + 1 - d0);
    for (int h0 = g0; h0 < g1; h0 += heads_per_stage) {
      const int nhh = min(heads_per_stage, g1 - h0);
      const int per_head = nrows * chunks;
      const int pieces = nhh * per_head;  // per K or V
      for (int i = tid; i < 2 * pieces; i += 256) {
        const int kv = i / pieces, rem = i % pieces;
        const int g = h0 + rem / per_head, rem2 = rem % per_head;
        const int r = rem2 / chunks, ch = rem2 % chunks;
        const int src = Lb + path[d0 + r];
        const long off =
            ((static_cast<long>(bt_b[src / kBlockSize]) * c.Hkv + g) * kBlockSize + src % kBlockSize) * row_bytes +
            ch * 16;
        const uint8_t* base = static_cast<const uint8_t*>(kv ? c.v : c.k);
        *reinterpret_cast<u32x4*>(stage + i * 16) = *reinterpret_cast<const u32x4*>(base + off);
      }
      __syncthreads();
      for (int i = tid; i < 2 * pieces; i += 256) {
        const int kv = i / pieces, rem = i % pieces;
        const int g = h0 + rem / per_head, rem2 = rem % per_head;
        const int r = rem2 / chunks, ch = rem2 % chunks;
        const int dst = Lb + d0 + r;
        const long off =
            ((static_cast<long>(bt_b[dst / kBlockSize]) * c.Hkv + g) * kBlockSize + dst % kBlockSize) * row_bytes +
            ch * 16;
        uint8_t* base = static_cast<uint8_t*>(kv ? c.v : c.k);
        *reinterpret_cast<u32x4*>(base + off) = *reinterpret_cast<const u32x4*>(stage + i * 16);
      }
      __syncthreads();
    }
  }
}

}  // namespace spectree
