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
// and every node's depth found by pointer jumping (ceil(log2 T) rounds); then
// each wave takes four rows at a time (query, key or value heads of the nodes,
// their loads in flight together), lane j on the pair (j, j + D/2).  Angles,
// sines and cosines are taken in fp64, so positions of any length keep full
// precision.
#include <math.h>

#include "common.h"
#include "rope_dev.h"

namespace spectree {
namespace {

struct KvArgs {
  const void* k_new;
  const void* v_new;
  const void* q;
  void* q_out;
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
constexpr int kUnroll = 4;        // rows per wave in flight together

template <bool kBf16>
__global__ __launch_bounds__(256) void tree_kv_write_kernel(const KvArgs a) {
  __shared__ int s_up[kMaxT], s_dep[kMaxT];
  static_assert(kMaxT <= 512, "two nodes per thread");
  __shared__ int s_err;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;
  const int Lb = a.plen[b];  // loaded on entry, with the parent row
  if (tid == 0) s_err = 0;
  __syncthreads();
  for (int i = tid; i < T; i += 256) {  // T <= 512: two nodes per thread at most
    const int p = a.parent[static_cast<long>(b) * T + i];
    const bool ok = i == 0 ? p == -1 : (p >= 0 && p < i);
    s_up[i] = (i == 0 || !ok) ? -1 : p;
    s_dep[i] = i == 0 ? 0 : 1;
    if (!ok) atomicOr(&s_err, SPEC_DEV_PARENT);
  }
  __syncthreads();
  for (int r = 0; (1 << r) < T; ++r) {  // after round r, up = the ancestor 2^(r+1) steps above (or -1)
    int up[2] = {-1, -1}, dep[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k;
      if (i < T) {
        up[k] = s_up[i];
        dep[k] = s_dep[i];
        if (up[k] >= 0) {
          dep[k] += s_dep[up[k]];
          up[k] = s_up[up[k]];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k;
      if (i < T) {
        s_up[i] = up[k];
        s_dep[i] = dep[k];
      }
    }
    __syncthreads();
  }
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
  // Each wave takes a contiguous run of rows, kUnroll at a time so that their
  // loads are in flight together; consecutive rows mostly belong to one node,
  // whose angles (the same for all its heads) are computed once.
  const int nwaves = gridDim.x * kRowsPerBlock;
  const int rpw = (nrows + nwaves - 1) / nwaves;
  const int r_begin = min(nrows, (blockIdx.x * kRowsPerBlock + wave) * rpw);
  const int r_end = min(nrows, r_begin + rpw);
  int trig_node = -1;  // node whose cosine and sine this lane holds
  double c = 1.0, sn = 0.0;
  // (node, row within the node) of the next row, stepped along the run
  int next_i = r_begin / per_node, next_r = r_begin - next_i * per_node;
  for (int row0 = r_begin; row0 < r_end; row0 += kUnroll) {
    long si[kUnroll], di[kUnroll];
    const void* src[kUnroll];
    void* dst[kUnroll];
    bool live[kUnroll], rot[kUnroll], kvrow[kUnroll];
    int node[kUnroll], blk[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = row0 + u;
      live[u] = false;
      rot[u] = false;
      kvrow[u] = false;
      node[u] = 0;
      blk[u] = 0;
      si[u] = di[u] = 0;
      src[u] = nullptr;
      dst[u] = nullptr;
      if (row >= r_end) continue;
      const int i = next_i, r = next_r;
      if (++next_r == per_node) {
        next_r = 0;
        ++next_i;
      }
      node[u] = i;
      if (r < a.Hq) {  // a query head, rotated in place
        si[u] = di[u] = ((static_cast<long>(b) * T + i) * a.Hq + r) * a.D;
        src[u] = a.q;
        dst[u] = a.q_out;
        rot[u] = a.rotate != 0;
        live[u] = true;
      } else {
        const bool is_k = r < a.Hq + a.Hkv;
        const int g = r - a.Hq - (is_k ? 0 : a.Hkv);
        const int t = Lb + i;
        blk[u] = bt_b[t / kBlockSize];
        si[u] = ((static_cast<long>(b) * T + i) * a.Hkv + g) * a.D;
        di[u] = (static_cast<long>(g) * kBlockSize + t % kBlockSize) * a.D;  // + the block's offset once it is known
        src[u] = is_k ? a.k_new : a.v_new;
        dst[u] = is_k ? a.k_cache : a.v_cache;
        rot[u] = is_k && a.rotate != 0;
        live[u] = true;
        kvrow[u] = true;
      }
    }
    if (lane < half) {
      // unconditional loads, issued back to back (rows past the run read the
      // first row again and store nothing; row0 < r_end, so that one is live)
      float x0[kUnroll], x1[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const void* sp = live[u] ? src[u] : src[0];
        const long sx = live[u] ? si[u] : si[0];
        x0[u] = ld_elt<kBf16>(sp, sx + lane);
        x1[u] = ld_elt<kBf16>(sp, sx + lane + half);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (!live[u]) continue;
        if (kvrow[u]) {
          if (blk[u] < 0 || blk[u] >= a.num_blocks) {
            if (lane == 0) report(a.status, b, SPEC_DEV_BLOCK);
            continue;
          }
          di[u] += static_cast<long>(blk[u]) * a.Hkv * kBlockSize * a.D;
        }
        float y0 = x0[u], y1 = x1[u];
        if (rot[u]) {
          if (node[u] != trig_node) {
            rope_cos_sin(Lb + s_dep[node[u]], lane, a.D, a.log2_theta, &c, &sn);
            trig_node = node[u];
          }
          rope_turn(x0[u], x1[u], c, sn, &y0, &y1);
        }
        st_elt<kBf16>(dst[u], di[u] + lane, y0);
        st_elt<kBf16>(dst[u], di[u] + lane + half, y1);
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteLaunch& L, hipStream_t stream) {
  KvArgs a{};
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.q = L.q;
  a.q_out = L.q_out != nullptr ? L.q_out : const_cast<void*>(L.q);
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
  // about 1024 workgroups in all (each finds the tree's depths once)
  const long per_seq = std::max<long>(1, std::min<long>((rows + kRowsPerBlock - 1) / kRowsPerBlock,
                                                        1024 / std::max(1, L.B)));
  const long chunks = per_seq;
  const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(L.B));
  if (L.bf16) {
    hipLaunchKernelGGL(tree_kv_write_kernel<true>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(tree_kv_write_kernel<false>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace spectree
