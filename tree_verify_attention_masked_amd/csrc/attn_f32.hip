// Tree-masked verify attention, fp32 inputs (head dim 64 or 128): the vector
// ALU path for small fp32 layers.  One 64-lane wave per query row (b, node i,
// head h).  Keys: the prefix 0..Lb-1, then the ancestors-or-self of node i,
// found by walking the parent array upward (the tree_mask of "Report: Support
// nextn speculative decoding", implementation summary step 3).
//
// Keys are taken 64 at a time, one per lane: each lane forms its key's full
// dot product with the query (read from LDS as a broadcast), one cross-lane max
// and one cross-lane sum update the online softmax (fp32, full-precision exp),
// then the lanes switch to owning head dims and accumulate P.V over the chunk's
// keys, whose probabilities and row offsets they read back from LDS.
#include "common.h"

namespace spectree {
namespace {

struct FArgs {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  float* out;
  int32_t* status;
  int B, T, Hq, Hkv, G, max_blocks, num_blocks;
  float scale;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x = fmaxf(x, __shfl_xor(x, w));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x += __shfl_xor(x, w);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const FArgs a) {
  constexpr int E = D / 64;                 // head dims per lane in P.V
  constexpr int kAncWords = kMaxT / 64;     // ancestors held per lane
  __shared__ __attribute__((aligned(16))) float s_q[4][D];
  __shared__ float s_p[4][64];
  __shared__ long s_off[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const long row = static_cast<long>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<long>(a.B) * a.T * a.Hq) return;  // no workgroup barriers below
  const int h = static_cast<int>(row % a.Hq);
  const int node = static_cast<int>((row / a.Hq) % a.T);
  const int b = static_cast<int>(row / (static_cast<long>(a.Hq) * a.T));
  const int g = h / a.G;
  int err = 0;
  int Lb = a.plen[b];
  const int cap = a.max_blocks * kBlockSize - a.T;
  if (Lb < 0 || Lb > cap) {
    err |= SPEC_DEV_LENGTH;
    Lb = Lb < 0 ? 0 : cap;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) s_q[wave][lane * E + e] = a.q[row * D + lane * E + e];
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;

  // ancestors-or-self of `node`: every lane walks the chain; lane k keeps steps
  // k, k + 64, ...; a broken chain keeps what was reached
  int anc[kAncWords];
#pragma unroll
  for (int c = 0; c < kAncWords; ++c) anc[c] = 0;
  int n_anc = 0;
  {
    const int32_t* par = a.parent + static_cast<long>(b) * a.T;
    int j = node;
    for (int steps = 0; steps <= a.T; ++steps) {
#pragma unroll
      for (int c = 0; c < kAncWords; ++c)
        if (n_anc == 64 * c + lane) anc[c] = j;
      ++n_anc;
      const int p = par[j];
      if (j == 0) {
        if (p != -1) err |= SPEC_DEV_PARENT;
        break;
      }
      if (p < 0 || p >= j) {
        err |= SPEC_DEV_PARENT;
        break;
      }
      j = p;
    }
  }

  float m = -INFINITY, l = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  // one chunk: this lane's key at logical position t (if `valid`)
  auto chunk = [&](int t, bool valid) {
    long off = 0;
    if (valid) {
      const int blk = bt_b[t / kBlockSize];
      if (blk < 0 || blk >= a.num_blocks) {
        err |= SPEC_DEV_BLOCK;
        valid = false;
      } else {
        off = ((static_cast<long>(blk) * a.Hkv + g) * kBlockSize + t % kBlockSize) * D;
      }
    }
    float sc = -INFINITY;
    if (valid) {
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(a.k + off + d);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&s_q[wave][d]);
        dot += qv[0] * kv[0] + qv[1] * kv[1] + qv[2] * kv[2] + qv[3] * kv[3];
      }
      sc = dot * a.scale;
    }
    const float cm = wave_max(sc);
    if (cm == -INFINITY) return;  // no valid key in the chunk (uniform)
    const float m_new = fmaxf(m, cm);
    const float alpha = expf(m - m_new);  // 0 while m is -inf
    const float p = valid ? expf(sc - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
    m = m_new;
    s_p[wave][lane] = p;
    s_off[wave][lane] = off;
    __builtin_amdgcn_wave_barrier();
    // branch-free so that the loads of many keys are in flight together; a
    // masked or invalid key (offset 0, in bounds) is selected away, so the NaN
    // that unused cache slots may hold never reaches the sum
#pragma unroll 16
    for (int kk = 0; kk < 64; ++kk) {
      const float pk = s_p[wave][kk];
      const float* vp = a.v + s_off[wave][kk] + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = vp[e];
        o[e] += pk != 0.f ? pk * x : 0.f;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int c0 = 0; c0 < Lb; c0 += 64) chunk(c0 + lane, c0 + lane < Lb);
#pragma unroll
  for (int c = 0; c < kAncWords; ++c)
    if (64 * c < n_anc) chunk(Lb + anc[c], 64 * c + lane < n_anc);

  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = a.out + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) op[e] = o[e] * inv;
  if (lane == 0) report(a.status, b, err);
}

}  // namespace

hipError_t launch_attn_f32(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  FArgs a{};
  a.q = static_cast<const float*>(L.q);
  a.k = static_cast<const float*>(L.k);
  a.v = static_cast<const float*>(L.v);
  a.bt = L.block_table;
  a.plen = L.prefix_lens;
  a.parent = L.parent;
  a.out = static_cast<float*>(L.out);
  a.status = L.status;
  a.B = L.B;
  a.T = L.T;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.max_blocks = L.max_blocks;
  a.num_blocks = L.num_blocks;
  a.scale = L.scale;
  const dim3 grid(static_cast<unsigned>(plan.items));
  if (L.D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spectree
