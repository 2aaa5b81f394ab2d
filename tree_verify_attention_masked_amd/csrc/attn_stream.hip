// Tree-masked verify attention for few query rows per kv head (<= 64: chains,
// single-token decode, small trees), bf16, head dim 128.  HBM-bound: the design
// keeps as many KV bytes in flight as possible.
//
// Work item = (sequence b, kv head g, split s of the KV pages).  The rows are
// the T*G (node, query head) pairs of the group (<= 4 blocks of 16).  Each of
// the 4 waves of a workgroup streams its own 32-key tiles (tiles w, w+4, ...):
//   * K goes straight from HBM into the A operand of v_mfma_f32_16x16x32_bf16
//     (lane l holds key l%16, dims c*32 + (l/16)*8 .. +7: 16 contiguous bytes),
//     giving S^T = K Q^T with 8 scores of one row per lane;
//   * V is loaded in its natural layout and transposed through a wave-private
//     LDS region: lane (key k, quad q) writes the pair (V[k][d], V[k+16][d]) as
//     one 32-bit word, so a row of V^T holds the 32 keys in the order
//     k, k+16, k+1, k+17, ...; the scores are packed into the PV operand in the
//     same order, so O^T += V^T P^T needs no other data movement;
//   * loads for the next DEPTH-1 tiles are issued before a tile is computed.
// Keys at prefix + j are tree nodes, masked by the row's ancestor bits (the
// tree_mask of "Report: Support nextn speculative decoding", EAGLE
// implementation summary, step 3).  The four waves merge through LDS; splits
// write partials (O, m, l) and the last workgroup of a (b, g) to finish merges
// them (a per-(b, g) arrival counter in the workspace, reset by that
// workgroup), so the whole call is one launch.
#include <algorithm>

#include "common.h"

namespace spectree {
namespace {

constexpr int kD = 128;
constexpr int kVS = 40;  // V^T row stride in LDS, in bf16 slots (32 keys + 8 pad, 80 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplitPages = 128;  // pages per split (plan_stream never exceeds it)

struct StArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  uint16_t* out;
  int32_t* status;
  float* part_o;       // [items][R][D]
  float* part_ml;      // [items][R][2]
  unsigned* counters;  // [B * Hkv], zero between calls
  int B, T, Hq, Hkv, G, R, splits, pps, max_blocks, num_blocks;
  long items;
  float sl2;
};

// Orders this wave's LDS writes and reads of the V^T region in program order.
// The hardware executes one wave's LDS operations in order, so only the
// compiler has to be kept from moving them across each other; a memory fence
// here would also wait for the prefetched global loads.
__device__ __forceinline__ void wave_lds_fence() { __asm__ volatile("" ::: "memory"); }

// parent_b is the LDS copy of the sequence's parent row.
__device__ int build_ancestors_st(const int* parent_b, int T, uint64_t* anc) {
  int err = 0;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    uint64_t w[4] = {0, 0, 0, 0};
    int j = i;
    bool ok = true;
    for (int steps = 0; steps <= T; ++steps) {
      w[j >> 6] |= 1ull << (j & 63);
      const int p = parent_b[j];
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

struct TileRegs {
  u32x4 k[2][4];  // [16-key half][32-dim chunk]
  u32x4 v[2][4];
  bool ok[2];     // this lane's key of each half is a real key of the split
};

template <int NRB, int DEPTH>
__global__ __launch_bounds__(256) void attn_stream_kernel(const StArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt_all[4 * kD * kVS];  // 40 KB: 4 waves' V^T, later merge space
  __shared__ uint64_t anc[kMaxT * 4];
  __shared__ int s_par[kMaxT];
  __shared__ int s_blk[kMaxSplitPages];  // block index of each page of this split (-1: invalid)
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  uint16_t* vt = vt_all + wave * kD * kVS;

  const long per = (a.items + 7) / 8;
  const long item = static_cast<long>(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= a.items) return;
  const int s = static_cast<int>(item % a.splits);
  const long bg = item / a.splits;
  const int g = static_cast<int>(bg % a.Hkv);
  const int b = static_cast<int>(bg / a.Hkv);

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
  const int n_tiles = p1 > p0 ? (p1 - p0 + 1) / 2 : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;

  // the split's block indices and the parent row, staged once: no dependent global loads later
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
  const bool tail = n_tiles > 0 && kend > Lb;
  for (int i = tid; i < p1 - p0; i += 256) {
    const int blk = bt_b[p0 + i];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    if (!ok) err |= SPEC_DEV_BLOCK;
    s_blk[i] = ok ? blk : -1;
  }
  if (tail)
    for (int i = tid; i < a.T; i += 256) s_par[i] = a.parent[static_cast<long>(b) * a.T + i];
  __syncthreads();
  if (tail) err |= build_ancestors_st(s_par, a.T, anc);
  __syncthreads();

  // query fragments: B operand of S^T, Q[row][c*32 + quad*8 .. +7]
  bf16x8 qf[NRB][4];
  int node_of[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = rb * 16 + l16;
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

  // Loads are unconditional so the compiler can count them: a tile past this
  // wave's range re-reads its last tile, a page past the split its last page
  // (cache hits); such keys are flagged and masked when the tile is computed.
  auto load_tile = [&](int j, TileRegs& t) {  // j-th tile of this wave
    const int tile = wave + 4 * min(j, max(my_tiles - 1, 0));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int page = min(p0 + 2 * tile + h, max(p1 - 1, p0));
      const int pos = (p0 + 2 * tile + h) * kBlockSize + l16;
      const int blk = p1 > p0 ? s_blk[page - p0] : -1;
      t.ok[h] = (j < my_tiles) && (pos < kend) && blk >= 0;
      const long off = ((static_cast<long>(max(blk, 0)) * a.Hkv + g) * kBlockSize + l16) * kD + quad * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t.k[h][c] = *reinterpret_cast<const u32x4*>(a.k + off + c * 32);
        t.v[h][c] = *reinterpret_cast<const u32x4*>(a.v + off + c * 32);
      }
    }
  };

  auto compute_tile = [&](int j, const TileRegs& t) {
    const int tile = wave + 4 * j;
    const int key0 = (p0 + 2 * tile) * kBlockSize;  // logical position of this tile's key 0
    // V^T into this wave's LDS region: word (d, pair k) = (V[k][d], V[k+16][d])
    wave_lds_fence();
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t a0 = t.ok[0] ? t.v[0][c][e2] : 0u, a1 = t.ok[1] ? t.v[1][c][e2] : 0u;
        const uint32_t lo = (a0 & 0xffffu) | (a1 << 16);
        const uint32_t hi = (a0 >> 16) | (a1 & 0xffff0000u);
        const int d = c * 32 + quad * 8 + 2 * e2;
        *reinterpret_cast<uint32_t*>(&vt[d * kVS + 2 * l16]) = lo;
        *reinterpret_cast<uint32_t*>(&vt[(d + 1) * kVS + 2 * l16]) = hi;
      }
    wave_lds_fence();
    const bool need_mask = key0 + 32 > Lb || key0 + 32 > kend;
    bf16x8 pf[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[h][c]), qf[rb][c], sacc[h],
                                                            0, 0, 0);
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
      const bf16x8 vf =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vt[(dt * 16 + l16) * kVS + quad * 8]));
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], o[rb][dt], 0, 0, 0);
    }
  };

  // software pipeline: DEPTH tiles in flight per wave
  TileRegs buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_tile(d, buf[d]);
  for (int j0 = 0; j0 < my_tiles; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      if (j < my_tiles) {
        compute_tile(j, buf[d]);
        load_tile(j + DEPTH, buf[d]);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16);
    l_run[rb] += __shfl_xor(l_run[rb], 32);
  }
  report(a.status, b, err);

  // merge the four waves, 16 rows at a time, through LDS
  float* mo = reinterpret_cast<float*>(vt_all);  // [4][16][128]
  float* ml = mo + 4 * 16 * kD;                  // [4][16][2]
  const int row = tid >> 4;
  const int dseg = (tid & 15) * 8;
  const bool direct = a.splits == 1;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&mo[(wave * 16 + l16) * kD + dt * 16 + quad * 4]) = o[rb][dt];
    if (quad == 0) {
      ml[(wave * 16 + l16) * 2 + 0] = m_run[rb];
      ml[(wave * 16 + l16) * 2 + 1] = l_run[rb];
    }
    __syncthreads();
    const int r = rb * 16 + row;
    if (r < a.R) {
      float mw[4], mstar = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mw[w] = ml[(w * 16 + row) * 2];
        mstar = fmaxf(mstar, mw[w]);
      }
      float lstar = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float wt = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - mstar);
        lstar += wt * ml[(w * 16 + row) * 2 + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wt * mo[(w * 16 + row) * kD + dseg + e];
      }
      if (direct) {
        const int node = r / a.G, hh = r % a.G;
        uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + dseg;
        const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wds[e] = f32_to_bf16(acc[2 * e] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * e + 1] * inv)) << 16);
        *reinterpret_cast<u32x4*>(op) = u32x4{wds[0], wds[1], wds[2], wds[3]};
      } else {
        float* po = a.part_o + (item * a.R + r) * kD + dseg;
        *reinterpret_cast<f32x4*>(po) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(po + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        if ((tid & 15) == 0) {
          a.part_ml[(item * a.R + r) * 2 + 0] = mstar;
          a.part_ml[(item * a.R + r) * 2 + 1] = lstar;
        }
      }
    }
  }
  if (direct) return;

  // the last workgroup of (b, g) to arrive merges every split
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&a.counters[bg], 1u);
    s_last = (prev == static_cast<unsigned>(a.splits - 1));
    if (s_last) __threadfence();
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const long first = bg * a.splits;
  for (int r = row; r < a.R; r += 16) {
    // online merge over the splits, 8 partials' loads in flight at a time
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
          const long it = first + sp0 + k;
          ms[k] = a.part_ml[(it * a.R + r) * 2];
          ls[k] = a.part_ml[(it * a.R + r) * 2 + 1];
          const float* po = a.part_o + (it * a.R + r) * kD + dseg;
          x0[k] = *reinterpret_cast<const f32x4*>(po);
          x1[k] = *reinterpret_cast<const f32x4*>(po + 4);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (ms[k] == -INFINITY) continue;
        const float m_new = fmaxf(mstar, ms[k]);
        const float fa = __builtin_amdgcn_exp2f(mstar - m_new);  // 0 while mstar is -inf
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
  if (tid == 0) atomicExch(&a.counters[bg], 0u);
}

template <int NRB, int DEPTH>
hipError_t run_stream(const StArgs& args, hipStream_t stream) {
  const long grid = ((args.items + 7) / 8) * 8;
  hipLaunchKernelGGL((attn_stream_kernel<NRB, DEPTH>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

// Plan for the streaming kernel: rows <= 64 per (b, g).  Pages per split are a
// multiple of 8 (one 32-key tile per wave and round); a workgroup holds a whole
// CU (one wave per SIMD), so small problems aim for one split per CU; at most
// 128 pages (2048 keys) per split keeps ragged batches balanced.
void plan_stream(AttnPlan& p, int B, int Hkv, int max_blocks) {
  p.mode = 3;
  p.rt = p.rows;
  p.nrb = (p.rows + 15) / 16;
  p.n_rt = 1;
  const long bg = static_cast<long>(B) * Hkv;
  long pps = (static_cast<long>(max_blocks) * bg + 255) / 256;
  pps = std::max<long>(8, std::min<long>(128, pps));
  pps = (pps + 7) / 8 * 8;
  p.pps = static_cast<int>(pps);
  p.splits = static_cast<int>((max_blocks + pps - 1) / pps);
  p.items = bg * p.splits;
  const size_t head = (static_cast<size_t>(bg) * sizeof(unsigned) + 255) / 256 * 256;
  p.ws_bytes = p.splits > 1 ? head + static_cast<size_t>(p.items) * p.rows * (kD + 2) * sizeof(float) : 0;
}

hipError_t launch_attn_stream(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  StArgs a{};
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
  a.splits = plan.splits;
  a.pps = plan.pps;
  a.max_blocks = L.max_blocks;
  a.num_blocks = L.num_blocks;
  a.items = plan.items;
  a.sl2 = L.scale * kLog2e;
  if (plan.splits > 1) {
    const size_t bg = static_cast<size_t>(L.B) * L.Hkv;
    a.counters = static_cast<unsigned*>(L.workspace);
    const size_t head = (bg * sizeof(unsigned) + 255) / 256 * 256;
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + head);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rows * kD;
  }
  switch (plan.nrb) {
    case 1:
      return run_stream<1, 3>(a, stream);
    case 2:
      return run_stream<2, 2>(a, stream);
    case 3:
      return run_stream<3, 1>(a, stream);
    default:
      return run_stream<4, 1>(a, stream);
  }
}

}  // namespace spectree
