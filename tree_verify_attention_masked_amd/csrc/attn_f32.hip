// Tree-masked verify attention, fp32 inputs (head dim 64 or 128): the vector
// ALU path for small fp32 layers.  One 64-lane wave per query row (b, node i,
// head h); each lane owns D/64 head dims.  Keys: the prefix 0..Lb-1, then the
// ancestors-or-self of node i found by walking the parent array upward (the
// tree_mask of "Report: Support nextn speculative decoding", implementation
// summary step 3).  Online softmax in fp32 with full-precision exp.
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

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const FArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<long>(a.B) * a.T * a.Hq) return;
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
  float qv[E];
  const float* qp = a.q + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = qp[e];
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;

  float m = -INFINITY, l = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  auto visit = [&](int t) {
    const int blk = bt_b[t / kBlockSize];
    if (blk < 0 || blk >= a.num_blocks) {
      err |= SPEC_DEV_BLOCK;
      return;
    }
    const long off = ((static_cast<long>(blk) * a.Hkv + g) * kBlockSize + t % kBlockSize) * D + lane * E;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) dot += qv[e] * a.k[off + e];
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) dot += __shfl_xor(dot, w);
    const float sc = dot * a.scale;
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * alpha + p * a.v[off + e];
    m = m_new;
  };

  for (int t = 0; t < Lb; ++t) visit(t);
  // ancestors-or-self of `node`, walked upward; a broken chain keeps what was reached
  const int32_t* par = a.parent + static_cast<long>(b) * a.T;
  int j = node;
  for (int steps = 0; steps <= a.T; ++steps) {
    visit(Lb + j);
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
