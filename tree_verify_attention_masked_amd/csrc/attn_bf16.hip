// Tree-masked verify attention, bf16 inputs, head dim 128, gfx950 matrix cores:
// planning for every bf16 shape, and the kernel for many query rows per kv head
// (> 64: wide trees times GQA groups).  Shapes with <= 64 rows use the
// streaming kernel (attn_stream.hip).
//
// Work item = (sequence b, kv head g, KV split s, row tile rt).  The query rows
// of one (b, g) are the T tree nodes times the G query heads of the group
// (row r -> node r / G, head g*G + r % G), so one pass over a KV page serves
// every tree query of the GQA group.  Keys are the logical positions
// 0 .. prefix+T-1 of the sequence, read page by page through the block table;
// keys at prefix + j are tree nodes and are masked by the ancestor-or-self
// bitset of the row's node (the tree_mask of the EAGLE implementation summary
// in "Report: Support nextn speculative decoding").
//
// A workgroup holds 4 waves x NRB blocks of 16 rows.  Per iteration the
// workgroup stages a 64-key tile (4 pages) in LDS -- K in its natural layout,
// V transposed with the keys of each 32-key half paired as (k, k+16) -- while
// the next tile's loads are in flight in registers.  Each wave computes, per
// 32-key half and row block, S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (8
// scores of one row per lane), the online softmax in the log2 domain, and
// O^T += V^T P^T with P packed in the (k, k+16) order.  Splits write
// unnormalised partials (O, m, l); the last workgroup of a (b, g, rt) to finish
// merges them (arrival counter in the workspace, reset by that workgroup).
#include <algorithm>

#include "common.h"

namespace spectree {
namespace {

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;             // keys per iteration (4 pages)
constexpr int kKS = kD + 8;           // LDS row stride of K (bf16), 272 B
constexpr int kVS = kTile + 8;        // LDS row stride of V^T (bf16 slots), 144 B
constexpr int kMaxSplitPages = 1024;  // pages per split (planning keeps below)

struct TArgs2 {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  uint16_t* out;
  int32_t* status;
  float* part_o;       // [items][RT][D]
  float* part_ml;      // [items][RT][2]
  unsigned* counters;  // [B * Hkv * n_rt]
  int B, T, Hq, Hkv, G, R, n_rt, splits, pps, max_blocks, num_blocks;
  long items;
  float sl2;
};

// Ancestor-or-self bitsets (4 x 64 bits per node) from the LDS copy of a parent
// row.  A node whose parent chain is not topological keeps only itself.
__device__ int build_ancestors_lds(const int* par, int T, uint64_t* anc) {
  int err = 0;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    uint64_t w[4] = {0, 0, 0, 0};
    int j = i;
    bool ok = true;
    for (int steps = 0; steps <= T; ++steps) {
      w[j >> 6] |= 1ull << (j & 63);
      const int p = par[j];
      if (j == 0) {
        ok = (p == -1);
        break;
      }
      if (p < 0 || p >= j) {
        ok = false;
        break;
      }
      j = p;
    }
    if (!ok) {
      err = SPEC_DEV_PARENT;
      w[0] = w[1] = w[2] = w[3] = 0;
      w[i >> 6] = 1ull << (i & 63);
    }
    for (int k = 0; k < 4; ++k) anc[i * 4 + k] = w[k];
  }
  return err;
}

template <int NRB>
__global__ __launch_bounds__(256) void attn_tile_kernel(const TArgs2 a) {
  constexpr int RT = 64 * NRB;  // rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * kVS];
  __shared__ uint64_t anc[kMaxT * 4];
  __shared__ int s_par[kMaxT];
  __shared__ int s_blk[kMaxSplitPages];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int quad = lane >> 4;

  // Consecutive workgroup ids are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous run of items so the row tiles of one KV chunk share an L2.
  const long per = (a.items + 7) / 8;
  const long item = static_cast<long>(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= a.items) return;
  const int rt = static_cast<int>(item % a.n_rt);
  long rest = item / a.n_rt;
  const int s = static_cast<int>(rest % a.splits);
  rest /= a.splits;
  const int g = static_cast<int>(rest % a.Hkv);
  const int b = static_cast<int>(rest / a.Hkv);
  const long bgr = (static_cast<long>(b) * a.Hkv + g) * a.n_rt + rt;

  int err = 0;
  int Lb = a.plen[b];
  const int cap = a.max_blocks * kBlockSize - a.T;
  if (Lb < 0 || Lb > cap) {
    err |= SPEC_DEV_LENGTH;
    Lb = Lb < 0 ? 0 : cap;
  }
  const int n_keys = Lb + a.T;
  const int npages = (n_keys + kBlockSize - 1) / kBlockSize;
  const int p0 = s * a.pps;
  const int p1 = min(npages, p0 + a.pps);
  const int kend = min(n_keys, p1 * kBlockSize);
  const int n_it = p1 > p0 ? (p1 - p0 + 3) / 4 : 0;
  const bool tail = n_it > 0 && kend > Lb;

  // the split's block indices and the parent row, staged once in LDS
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
  for (int i = tid; i < p1 - p0; i += 256) {
    const int blk = bt_b[p0 + i];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    if (!ok) err |= SPEC_DEV_BLOCK;
    s_blk[i] = ok ? blk : -1;
  }
  if (tail)
    for (int i = tid; i < a.T; i += 256) s_par[i] = a.parent[static_cast<long>(b) * a.T + i];
  __syncthreads();
  if (tail) err |= build_ancestors_lds(s_par, a.T, anc);

  // query fragments (B operand of S^T): Q[row][c*32 + quad*8 .. +7]
  const int row_base = rt * RT + wave * NRB * 16;
  bf16x8 qf[NRB][4];
  int node_of[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row_base + rb * 16 + l16;
    node_of[rb] = r < a.R ? r / a.G : 0;
    if (r < a.R) {
      const int node = r / a.G, hh = r % a.G;
      const uint16_t* qp = a.q + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + quad * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[rb][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + c * 32));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[rb][c] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  float m_run[NRB], l_run[NRB];
  f32x4 o[NRB][8];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Staging: thread (key kin = tid/16, dims d0 = (tid%16)*8) moves, for each
  // 32-key half st and 16-key quarter h, one 16-byte chunk of K and of V.
  // Loads are unconditional (pages past the split re-read its last page);
  // validity is a flag applied when the chunk is written to LDS.
  const int kin = tid >> 4;
  const int d0 = (tid & 15) * 8;
  u32x4 kr[2][2], vr[2][2];
  bool okr[2][2];
  auto load_tile = [&](int it) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pg = p0 + 4 * it + 2 * st + h;
        const int page = min(pg, max(p1 - 1, p0));
        const int blk = p1 > p0 ? s_blk[page - p0] : -1;
        okr[st][h] = (pg * kBlockSize + kin < kend) && blk >= 0;
        const long off = ((static_cast<long>(max(blk, 0)) * a.Hkv + g) * kBlockSize + kin) * kD + d0;
        kr[st][h] = *reinterpret_cast<const u32x4*>(a.k + off);
        vr[st][h] = *reinterpret_cast<const u32x4*>(a.v + off);
      }
  };
  __syncthreads();  // s_blk and anc are ready
  if (n_it > 0) load_tile(0);

  for (int it = 0; it < n_it; ++it) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4*>(&Ks[(st * 32 + h * 16 + kin) * kKS + d0]) =
            okr[st][h] ? kr[st][h] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t a0 = okr[st][0] ? vr[st][0][e2] : 0u, a1 = okr[st][1] ? vr[st][1][e2] : 0u;
        const uint32_t lo = (a0 & 0xffffu) | (a1 << 16);
        const uint32_t hi = (a0 >> 16) | (a1 & 0xffff0000u);
        const int d = d0 + 2 * e2;
        *reinterpret_cast<uint32_t*>(&Vt[d * kVS + st * 32 + 2 * kin]) = lo;
        *reinterpret_cast<uint32_t*>(&Vt[(d + 1) * kVS + st * 32 + 2 * kin]) = hi;
      }
    }
    __syncthreads();
    if (it + 1 < n_it) load_tile(it + 1);

#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key0 = (p0 + 4 * it + 2 * st) * kBlockSize;
      const bool need_mask = key0 + 32 > Lb || key0 + 32 > kend;
      bf16x8 kf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kf[h][c] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&Ks[(st * 32 + h * 16 + l16) * kKS + c * 32 + quad * 8]));
      bf16x8 pf[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h][c], qf[rb][c], sacc[h], 0, 0, 0);
        // lane holds S[row l16][key h*16 + quad*4 + i]; PV slot j <-> (h = j % 2, i = j / 2)
        float sv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = sacc[h][i] * a.sl2;
            if (need_mask) {
              const int pos = key0 + h * 16 + quad * 4 + i;
              bool ok = pos < kend;
              if (ok && pos >= Lb) {
                const int jj = pos - Lb;
                ok = (anc[node_of[rb] * 4 + (jj >> 6)] >> (jj & 63)) & 1ull;
              }
              x = ok ? x : -INFINITY;
            }
            sv[2 * i + h] = x;
          }
        float mx = sv[0];
#pragma unroll
        for (int j2 = 1; j2 < 8; ++j2) mx = fmaxf(mx, sv[j2]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[rb], mx);
        const bool none = (m_new == -INFINITY);
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        float psum = 0.f;
#pragma unroll
        for (int j2 = 0; j2 < 8; ++j2) {
          const float p = none ? 0.f : __builtin_amdgcn_exp2f(sv[j2] - m_new);
          psum += p;
          pf[rb][j2] = static_cast<__bf16>(p);
        }
        l_run[rb] = l_run[rb] * alpha + psum;
        m_run[rb] = m_new;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[rb][dt] *= alpha;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&Vt[(dt * 16 + l16) * kVS + st * 32 + quad * 8]));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], o[rb][dt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16);
    l_run[rb] += __shfl_xor(l_run[rb], 32);
  }
  report(a.status, b, err);

  const bool direct = (a.splits == 1);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row_base + rb * 16 + l16;
    if (r >= a.R) continue;
    const int rl = r - rt * RT;
    if (direct) {
      const int node = r / a.G, hh = r % a.G;
      uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD;
      const float inv = l_run[rb] > 0.f ? 1.f / l_run[rb] : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t w0 =
            f32_to_bf16(o[rb][dt][0] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[rb][dt][1] * inv)) << 16);
        const uint32_t w1 =
            f32_to_bf16(o[rb][dt][2] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[rb][dt][3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(op + dt * 16 + quad * 4) = u32x2{w0, w1};
      }
    } else {
      float* po = a.part_o + (item * RT + rl) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + quad * 4) = o[rb][dt];
      if (quad == 0) {
        a.part_ml[(item * RT + rl) * 2 + 0] = m_run[rb];
        a.part_ml[(item * RT + rl) * 2 + 1] = l_run[rb];
      }
    }
  }
  if (direct) return;

  // the last workgroup of (b, g, rt) to arrive merges every split
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&a.counters[bgr], 1u);
    s_last = (prev == static_cast<unsigned>(a.splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const long first = (bgr / a.n_rt) * a.splits * a.n_rt + rt;  // item of split 0
  const int dseg = (tid & 15) * 8;
  for (int rl = tid >> 4; rl < RT; rl += 16) {
    const int r = rt * RT + rl;
    if (r >= a.R) break;
    float mstar = -INFINITY, lstar = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp0 = 0; sp0 < a.splits; sp0 += 8) {
      float ms[8], ls[8];
      f32x4 x0[8], x1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        x0[k] = x1[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sp0 + k < a.splits) {
          const long it2 = first + static_cast<long>(sp0 + k) * a.n_rt;
          ms[k] = a.part_ml[(it2 * RT + rl) * 2];
          ls[k] = a.part_ml[(it2 * RT + rl) * 2 + 1];
          const float* po = a.part_o + (it2 * RT + rl) * kD + dseg;
          x0[k] = *reinterpret_cast<const f32x4*>(po);
          x1[k] = *reinterpret_cast<const f32x4*>(po + 4);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (ms[k] == -INFINITY) continue;
        const float m_new = fmaxf(mstar, ms[k]);
        const float fa = __builtin_amdgcn_exp2f(mstar - m_new);
        const float fb = __builtin_amdgcn_exp2f(ms[k] - m_new);
        lstar = lstar * fa + ls[k] * fb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = acc[e] * fa + x0[k][e] * fb;
          acc[4 + e] = acc[4 + e] * fa + x1[k][e] * fb;
        }
        mstar = m_new;
      }
    }
    const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
    const int node = r / a.G, hh = r % a.G;
    uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + dseg;
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wds[e] = f32_to_bf16(acc[2 * e] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * e + 1] * inv)) << 16);
    *reinterpret_cast<u32x4*>(op) = u32x4{wds[0], wds[1], wds[2], wds[3]};
  }
  if (tid == 0) atomicExch(&a.counters[bgr], 0u);
}

template <int NRB>
hipError_t run_tile(const TArgs2& args, hipStream_t stream) {
  const long grid = ((args.items + 7) / 8) * 8;
  hipLaunchKernelGGL((attn_tile_kernel<NRB>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int B, int T, int Hq, int Hkv, int D, int max_blocks, int dtype) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  p.rows = T * G;
  if (dtype == SPEC_F32) {
    p.mode = 0;
    p.rt = 4;
    p.nrb = 0;
    p.n_rt = 0;
    p.splits = 1;
    p.pps = max_blocks;
    p.items = (static_cast<long>(B) * T * Hq + 3) / 4;
    p.ws_bytes = 0;
    return p;
  }
  (void)D;
  if (p.rows <= 64) {
    plan_stream(p, B, Hkv, max_blocks);
    return p;
  }
  // many rows: 128-row tiles, or 256-row tiles from 1024 rows up
  p.mode = 2;
  p.nrb = p.rows >= 1024 ? 4 : 2;
  p.rt = 64 * p.nrb;
  p.n_rt = (p.rows + p.rt - 1) / p.rt;
  const long base = static_cast<long>(B) * Hkv * p.n_rt;
  // ~one workgroup per CU; at least 16 pages (256 keys) per split
  long splits = std::max<long>(1, (256 + base - 1) / base);
  splits = std::min<long>(splits, std::max<long>(1, max_blocks / 16));
  long pps = (max_blocks + splits - 1) / splits;
  pps = (pps + 3) / 4 * 4;
  pps = std::min<long>(pps, kMaxSplitPages);
  splits = (max_blocks + pps - 1) / pps;
  p.pps = static_cast<int>(pps);
  p.splits = static_cast<int>(splits);
  p.items = base * p.splits;
  const size_t head = (static_cast<size_t>(base) * sizeof(unsigned) + 255) / 256 * 256;
  p.ws_bytes = p.splits > 1 ? head + static_cast<size_t>(p.items) * p.rt * (kD + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_attn_bf16(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  if (plan.mode == 3) return launch_attn_stream(plan, L, stream);
  TArgs2 a{};
  a.q = static_cast<const uint16_t*>(L.q);
  a.k = static_cast<const uint16_t*>(L.k);
  a.v = static_cast<const uint16_t*>(L.v);
  a.bt = L.block_table;
  a.plen = L.prefix_lens;
  a.parent = L.parent;
  a.out = static_cast<uint16_t*>(L.out);
  a.status = L.status;
  a.B = L.B;
  a.T = L.T;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.R = plan.rows;
  a.n_rt = plan.n_rt;
  a.splits = plan.splits;
  a.pps = plan.pps;
  a.max_blocks = L.max_blocks;
  a.num_blocks = L.num_blocks;
  a.items = plan.items;
  a.sl2 = L.scale * kLog2e;
  if (plan.splits > 1) {
    const size_t base = static_cast<size_t>(L.B) * L.Hkv * plan.n_rt;
    const size_t head = (base * sizeof(unsigned) + 255) / 256 * 256;
    a.counters = static_cast<unsigned*>(L.workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + head);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rt * kD;
  }
  if (plan.nrb == 4) return run_tile<4>(a, stream);
  return run_tile<2>(a, stream);
}

}  // namespace spectree
