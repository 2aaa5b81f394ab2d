// The step before verify attention: the draft tree's K/V rows go into the
// paged cache, the keys and the queries rotated for their tree positions.
//
// Node i of sequence b is at position Lb + depth(i): the tokens are scored in
// one flattened pass ("Report: Support nextn speculative decoding",
// implementation summary, step 3), each at the position it would have along
// its own path (the position_ids of "Issue: Speculative Decoding on vLLM").
// Its K and V rows are written to logical slot Lb + i, where the verify
// attention reads them and from where the compaction later moves the accepted
// ones.  The rotation is RoFormer's rotary position embedding in the
// half-split layout: for j < D/2 the pair (x_j, x_{j + D/2}) at position p
// turns by p * theta^(-2j/D); theta = 0 writes the rows unrotated.
//
// One workgroup per (sequence, chunk of rows): the parent row is staged in LDS
// and every node's depth found by pointer jumping (8 rounds cover T <= 256);
// then each wave takes one row at a time -- a query head, a key head or a value
// head of one node -- with lane j on the pair (j, j + D/2).  Angles, sines and
// cosines are taken in fp64, so positions of any length keep full precision.
#include <math.h>

#include "common.h"

namespace spectree {
namespace {

struct KvArgs {
  const void* k_new;
  const void* v_new;
  void* q;
  void* k_cache;
  void* v_cache;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  int32_t* status;
  int B, T, Hq, Hkv, D, max_blocks, num_blocks;
  int rotate;
  double log2_theta;
};

template <bool kBf16>
__device__ __forceinline__ float ld_elt(const void* p, long i) {
  if constexpr (kBf16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}
template <bool kBf16>
__device__ __forceinline__ void st_elt(void* p, long i, float v) {
  if constexpr (kBf16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

constexpr int kRowsPerBlock = 4;  // one per wave

template <bool kBf16>
__global__ __launch_bounds__(256) void tree_kv_write_kernel(const KvArgs a) {
  __shared__ int s_up[kMaxT], s_dep[kMaxT];
  __shared__ int s_err;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;
  if (tid == 0) s_err = 0;
  __syncthreads();
  if (tid < T) {
    const int p = a.parent[static_cast<long>(b) * T + tid];
    const bool ok = tid == 0 ? p == -1 : (p >= 0 && p < tid);
    s_up[tid] = (tid == 0 || !ok) ? -1 : p;
    s_dep[tid] = tid == 0 ? 0 : 1;
    if (!ok) atomicOr(&s_err, SPEC_DEV_PARENT);
  }
  __syncthreads();
  for (int r = 0; r < 8; ++r) {  // after round r, up = the ancestor 2^(r+1) steps above (or -1)
    int up = -1, dep = 0;
    if (tid < T) {
      up = s_up[tid];
      dep = s_dep[tid];
      if (up >= 0) {
        dep += s_dep[up];
        up = s_up[up];
      }
    }
    __syncthreads();
    if (tid < T) {
      s_up[tid] = up;
      s_dep[tid] = dep;
    }
    __syncthreads();
  }
  const int Lb = a.plen[b];
  int err = s_err;
  if (Lb < 0 || Lb > a.max_blocks * kBlockSize - T) err |= SPEC_DEV_LENGTH;
  if (err) {  // nothing is written for this sequence
    if (tid == 0 && blockIdx.x == 0) report(a.status, b, err);
    return;
  }
  const int per_node = a.Hq + 2 * a.Hkv;  // query heads, key heads, value heads
  const int nrows = T * per_node;
  const int half = a.D >> 1;
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
  for (int row = blockIdx.x * kRowsPerBlock + wave; row < nrows; row += gridDim.x * kRowsPerBlock) {
    const int i = row / per_node, r = row % per_node;
    const void* src;
    void* dst;
    long si, di;
    bool rot;
    if (r < a.Hq) {  // a query head, rotated in place
      if (a.q == nullptr) continue;
      si = di = ((static_cast<long>(b) * T + i) * a.Hq + r) * a.D;
      src = a.q;
      dst = a.q;
      rot = a.rotate != 0;
    } else {
      const bool is_k = r < a.Hq + a.Hkv;
      const int g = r - a.Hq - (is_k ? 0 : a.Hkv);
      const int t = Lb + i;
      const int blk = bt_b[t / kBlockSize];
      if (blk < 0 || blk >= a.num_blocks) {
        if (lane == 0) report(a.status, b, SPEC_DEV_BLOCK);
        continue;
      }
      si = ((static_cast<long>(b) * T + i) * a.Hkv + g) * a.D;
      di = ((static_cast<long>(blk) * a.Hkv + g) * kBlockSize + t % kBlockSize) * a.D;
      src = is_k ? a.k_new : a.v_new;
      dst = is_k ? a.k_cache : a.v_cache;
      rot = is_k && a.rotate != 0;
    }
    if (lane < half) {
      const float x0 = ld_elt<kBf16>(src, si + lane), x1 = ld_elt<kBf16>(src, si + lane + half);
      float y0 = x0, y1 = x1;
      if (rot) {
        const double ang =
            static_cast<double>(Lb + s_dep[i]) * exp2(-(2.0 * lane / a.D) * a.log2_theta);
        const double c = cos(ang), s = sin(ang);
        y0 = static_cast<float>(static_cast<double>(x0) * c - static_cast<double>(x1) * s);
        y1 = static_cast<float>(static_cast<double>(x1) * c + static_cast<double>(x0) * s);
      }
      st_elt<kBf16>(dst, di + lane, y0);
      st_elt<kBf16>(dst, di + lane + half, y1);
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteLaunch& L, hipStream_t stream) {
  KvArgs a{};
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.q = L.q;
  a.k_cache = L.k_cache;
  a.v_cache = L.v_cache;
  a.bt = L.block_table;
  a.plen = L.prefix_lens;
  a.parent = L.parent;
  a.status = L.status;
  a.B = L.B;
  a.T = L.T;
  a.Hq = L.q != nullptr ? L.Hq : 0;
  a.Hkv = L.Hkv;
  a.D = L.D;
  a.max_blocks = L.max_blocks;
  a.num_blocks = L.num_blocks;
  a.rotate = L.theta > 0.0f ? 1 : 0;
  a.log2_theta = L.theta > 0.0f ? log2(static_cast<double>(L.theta)) : 0.0;
  const long rows = static_cast<long>(L.T) * (a.Hq + 2 * a.Hkv);
  const long chunks = std::min<long>((rows + kRowsPerBlock - 1) / kRowsPerBlock, 64);
  const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(L.B));
  if (L.bf16) {
    hipLaunchKernelGGL(tree_kv_write_kernel<true>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(tree_kv_write_kernel<false>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace spectree
