// Tree-masked verify attention, bf16 inputs, head dim 128, gfx950 matrix cores.
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
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, one 64-lane wave):
//   S^T[key, row] = K[key, :] . Q[row, :]     A = K from LDS, B = Q in registers
//   O^T[d, row]  += V^T[d, key] . P^T[key, row]
// With S^T as the accumulator every lane holds 8 scores of ONE row, which is
// exactly the B operand the PV product needs, so P never leaves registers; the
// key order inside the 32-wide contraction is permuted identically in V^T.
// V is staged transposed in LDS.  Online softmax runs in the log2 domain.
// Splits write unnormalised partials (O, m, l) that a second kernel merges.
#include <algorithm>

#include "common.h"

namespace spectree {
namespace {

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct BArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  uint16_t* out;
  int32_t* status;
  float* part_o;   // [items, RT, D]
  float* part_ml;  // [items, RT, 2]
  int B, T, Hq, Hkv, G, R, n_rt, splits, pps, max_blocks, num_blocks;
  long items;
  float sl2;  // scale * log2(e)
};

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Ancestor-or-self bitsets of all T nodes of sequence b into LDS (4 x 64 bits
// per node).  A node whose parent chain is not topological keeps only itself.
__device__ int build_ancestors(const int32_t* parent_b, int T, uint64_t* anc) {
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

template <int WR, int WK, int NRB>
__global__ __launch_bounds__(256) void attn_bf16_kernel(const BArgs a) {
  constexpr int TILE = 32 * WK;      // keys staged per iteration
  constexpr int PAGES = TILE / 16;   // pages per iteration
  constexpr int RT = 16 * NRB * WR;  // query rows per workgroup
  constexpr int KSTR = kD + 8;       // LDS row stride of K (elements)
  constexpr int VSTR = TILE + 8;     // LDS row stride of V^T (elements)
  static_assert(WR * WK == 4, "four waves per workgroup");
  static_assert(WK == 1 || NRB == 1, "key-split workgroups hold one row block");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * VSTR];
  __shared__ uint64_t anc[kMaxT * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int n_it = p1 > p0 ? (p1 - p0 + PAGES - 1) / PAGES : 0;
  const int kend = min(n_keys, p1 * kBlockSize);  // keys past the split belong to the next one

  if (n_it > 0 && p1 * kBlockSize > Lb) err |= build_ancestors(a.parent + static_cast<long>(b) * a.T, a.T, anc);

  // query fragments (B operand of S^T): Q[row][c*32 + quad*8 .. +7]
  const int row_base = rt * RT + (WR == 1 ? 0 : wave * NRB * 16);
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
      for (int c = 0; c < 4; ++c) qf[rb][c] = ld_bf16x8(qp + c * 32);
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

  // Each thread moves one 16-byte chunk per page and tensor: key kin, dims d0..d0+7.
  const int kin = tid >> 4;
  const int d0 = (tid & 15) * 8;
  u32x4 kr[PAGES], vr[PAGES];
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
  auto load_tile = [&](int it) {
#pragma unroll
    for (int n = 0; n < PAGES; ++n) {
      const int page = p0 + it * PAGES + n;
      const int pos = page * kBlockSize + kin;
      kr[n] = u32x4{0, 0, 0, 0};
      vr[n] = u32x4{0, 0, 0, 0};
      if (page < p1 && pos < n_keys) {
        const int blk = bt_b[page];
        if (blk < 0 || blk >= a.num_blocks) {
          err |= SPEC_DEV_BLOCK;
        } else {
          const long off = ((static_cast<long>(blk) * a.Hkv + g) * kBlockSize + kin) * kD + d0;
          kr[n] = *reinterpret_cast<const u32x4*>(a.k + off);
          vr[n] = *reinterpret_cast<const u32x4*>(a.v + off);
        }
      }
    }
  };

  if (n_it > 0) load_tile(0);
  const int koff = (WK == 1) ? 0 : wave * 32;
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();
#pragma unroll
    for (int n = 0; n < PAGES; ++n) {
      *reinterpret_cast<u32x4*>(&Ks[(n * 16 + kin) * KSTR + d0]) = kr[n];
      const int col = n * 16 + kin;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Vt[(d0 + 2 * j) * VSTR + col] = static_cast<uint16_t>(vr[n][j] & 0xffffu);
        Vt[(d0 + 2 * j + 1) * VSTR + col] = static_cast<uint16_t>(vr[n][j] >> 16);
      }
    }
    __syncthreads();
    if (it + 1 < n_it) load_tile(it + 1);

    const int sub0 = (p0 + it * PAGES) * kBlockSize + koff;  // logical position of this wave's key 0
    const bool need_mask = sub0 + 32 > Lb || sub0 + 32 > kend;

    bf16x8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < 4; ++c) kf[kt][c] = ld_bf16x8(&Ks[(koff + kt * 16 + l16) * KSTR + c * 32 + quad * 8]);
    bf16x8 vf[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vp = &Vt[(dt * 16 + l16) * VSTR + koff + quad * 4];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
      vf[dt] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }

#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][c], qf[rb][c], sacc[kt], 0, 0, 0);
      float sv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[kt][i] * a.sl2;
          if (need_mask) {
            const int pos = sub0 + kt * 16 + quad * 4 + i;
            bool ok = pos < kend;
            if (ok && pos >= Lb) {
              const int j = pos - Lb;
              ok = (anc[node_of[rb] * 4 + (j >> 6)] >> (j & 63)) & 1ull;
            }
            x = ok ? x : -INFINITY;
          }
          sv[kt * 4 + i] = x;
        }
      float mx = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);
      const bool none = (m_new == -INFINITY);
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      float psum = 0.f;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = none ? 0.f : __builtin_amdgcn_exp2f(sv[j] - m_new);
        psum += p;
        pf[j] = static_cast<__bf16>(p);
      }
      l_run[rb] = l_run[rb] * alpha + psum;
      m_run[rb] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        o[rb][dt] *= alpha;
        o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, o[rb][dt], 0, 0, 0);
      }
    }
  }

  // row sums: the four lanes of a row hold disjoint key subsets
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16);
    l_run[rb] += __shfl_xor(l_run[rb], 32);
  }
  report(a.status, b, err);

  const bool direct = (a.splits == 1);
  if constexpr (WK == 1) {
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
          const uint32_t w0 = f32_to_bf16(o[rb][dt][0] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[rb][dt][1] * inv)) << 16);
          const uint32_t w1 = f32_to_bf16(o[rb][dt][2] * inv) | (static_cast<uint32_t>(f32_to_bf16(o[rb][dt][3] * inv)) << 16);
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
  } else {
    // four waves hold the same 16 rows over disjoint keys: merge through LDS
    __syncthreads();
    float* mo = reinterpret_cast<float*>(Ks);  // [4][16][128]
    float* ml = reinterpret_cast<float*>(Vt);  // [4][16][2]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&mo[(wave * 16 + l16) * kD + dt * 16 + quad * 4]) = o[0][dt];
    if (quad == 0) {
      ml[(wave * 16 + l16) * 2 + 0] = m_run[0];
      ml[(wave * 16 + l16) * 2 + 1] = l_run[0];
    }
    __syncthreads();
    const int row = tid >> 4;
    const int dseg = (tid & 15) * 8;
    const int r = rt * RT + row;
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
        for (int j = 0; j < 8; ++j) acc[j] += wt * mo[(w * 16 + row) * kD + dseg + j];
      }
      const int rl = r - rt * RT;
      if (direct) {
        const int node = r / a.G, hh = r % a.G;
        uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + dseg;
        const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = f32_to_bf16(acc[2 * j] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1] * inv)) << 16);
        *reinterpret_cast<u32x4*>(op) = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        float* po = a.part_o + (item * RT + rl) * kD + dseg;
        *reinterpret_cast<f32x4*>(po) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(po + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        if ((tid & 15) == 0) {
          a.part_ml[(item * RT + rl) * 2 + 0] = mstar;
          a.part_ml[(item * RT + rl) * 2 + 1] = lstar;
        }
      }
    }
  }
}

// Merge the split partials of one (b, g, row tile): O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
template <int RT>
__global__ __launch_bounds__(256) void attn_combine_kernel(const BArgs a) {
  const long bgr = blockIdx.x;  // (b * Hkv + g) * n_rt + rt
  const int rt = static_cast<int>(bgr % a.n_rt);
  const long bg = bgr / a.n_rt;
  const int g = static_cast<int>(bg % a.Hkv);
  const int b = static_cast<int>(bg / a.Hkv);
  const int tid = threadIdx.x;
  const int dq = (tid & 31) * 4;
  for (int rl = tid >> 5; rl < RT; rl += 8) {
    const int r = rt * RT + rl;
    if (r >= a.R) break;
    float mstar = -INFINITY;
    for (int s = 0; s < a.splits; ++s) {
      const long item = (bg * a.splits + s) * a.n_rt + rt;
      mstar = fmaxf(mstar, a.part_ml[(item * RT + rl) * 2]);
    }
    float lstar = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
      const long item = (bg * a.splits + s) * a.n_rt + rt;
      const float ms = a.part_ml[(item * RT + rl) * 2];
      if (ms == -INFINITY) continue;
      const float wt = __builtin_amdgcn_exp2f(ms - mstar);
      lstar += wt * a.part_ml[(item * RT + rl) * 2 + 1];
      acc += wt * *reinterpret_cast<const f32x4*>(a.part_o + (item * RT + rl) * kD + dq);
    }
    const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
    const int node = r / a.G, hh = r % a.G;
    uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + dq;
    const uint32_t w0 = f32_to_bf16(acc[0] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[1] * inv)) << 16);
    const uint32_t w1 = f32_to_bf16(acc[2] * inv) | (static_cast<uint32_t>(f32_to_bf16(acc[3] * inv)) << 16);
    *reinterpret_cast<u32x2*>(op) = u32x2{w0, w1};
  }
}

template <int WR, int WK, int NRB>
hipError_t run(const AttnPlan& plan, const BArgs& args, hipStream_t stream) {
  constexpr int RT = 16 * NRB * WR;
  const long grid = ((args.items + 7) / 8) * 8;
  hipLaunchKernelGGL((attn_bf16_kernel<WR, WK, NRB>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<RT>), dim3(static_cast<unsigned>(static_cast<long>(args.B) * args.Hkv * args.n_rt)),
                     dim3(256), 0, stream, args);
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
  int pages_per_it;
  if (p.rows <= 16) {
    p.mode = 1;
    p.rt = 16;
    p.nrb = 1;
    pages_per_it = 8;
  } else if (p.rows < 1024) {
    p.mode = 2;
    p.rt = 64;
    p.nrb = 1;
    pages_per_it = 2;
  } else {
    p.mode = 2;
    p.rt = 256;
    p.nrb = 4;
    pages_per_it = 2;
  }
  p.n_rt = (p.rows + p.rt - 1) / p.rt;
  const long base = static_cast<long>(B) * Hkv * p.n_rt;
  // Aim for ~1024 workgroups; keep the partial traffic (2 * splits * rows fp32
  // rows per head) under ~1/4 of the KV bytes; splits hold whole iterations.
  const long want = std::max<long>(1, (1024 + base - 1) / base);
  const long kv_keys = static_cast<long>(max_blocks) * kBlockSize;
  long cap = std::max<long>(1, kv_keys / (8L * p.rows));
  if (p.rows >= 1024) cap = std::max<long>(cap, 4);  // matrix-core bound: parallelism first
  long splits = std::min(want, cap);
  int pps = static_cast<int>((max_blocks + splits - 1) / splits);
  pps = ((pps + pages_per_it - 1) / pages_per_it) * pages_per_it;
  splits = (max_blocks + pps - 1) / pps;
  p.pps = pps;
  p.splits = static_cast<int>(splits);
  p.items = base * p.splits;
  p.ws_bytes = p.splits > 1 ? static_cast<size_t>(p.items) * p.rt * (kD + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_attn_bf16(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  BArgs a{};
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
    a.part_o = static_cast<float*>(L.workspace);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rt * kD;
  }
  if (plan.mode == 1) return run<1, 4, 1>(plan, a, stream);
  if (plan.nrb == 1) return run<4, 1, 1>(plan, a, stream);
  return run<4, 1, 4>(plan, a, stream);
}

}  // namespace spectree
