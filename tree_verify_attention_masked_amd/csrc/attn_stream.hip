// Tree-masked verify attention for few query rows per kv head (<= 64: chains,
// single-token decode, small trees), bf16, head dim 128.  HBM-bound: the design
// keeps as many KV bytes in flight per CU as LDS allows.
//
// Work item = (sequence b, kv head g, split s of the KV pages).  The rows are
// the T*G (node, query head) pairs of the group (<= 4 blocks of 16).  Each of
// the 4 waves of a workgroup streams its own pages (s*pps + wave + 4k) through
// a private ring of DEPTH page slots in LDS, filled by direct global->LDS loads
// (global_load_lds_dwordx4), so prefetch depth costs no registers:
//   * K lands key-major with its 16-byte chunks XOR-swizzled by the key, so the
//     A operand of v_mfma_f32_16x16x32_bf16 (lane l: key l%16, dims
//     c*32 + (l/16)*8 .. +7) is one conflict-free ds_read_b128; S^T = K Q^T
//     leaves 4 scores of one row per lane (keys 4*(l/16) + i);
//   * V lands key-major with an even swizzle, and ds_read_b64_tr_b16 (within
//     16 lanes: out[i][m] = mem[addr[i/4 + 4m] + i%4]) turns it into the A
//     operand of v_mfma_f32_16x16x16_bf16 for O^T += V^T P^T, whose B operand
//     is exactly the S^T accumulator layout, so P needs no data movement.
// Keys at prefix + j are tree nodes, masked by the row's ancestor bits (the
// tree_mask of "Report: Support nextn speculative decoding", EAGLE
// implementation summary, step 3); with T <= 64 each node's ancestor set is
// one 64-bit word, built by pointer doubling across the lanes of a wave.  The
// four waves merge through LDS; when a (b, g) spans several splits, each
// writes a partial (O, m, l) and the last one to finish merges them (a
// per-(b, g) arrival counter in the workspace, reset by that workgroup), so
// the whole call is one launch.
#include <algorithm>

#include "common.h"
#include "rope_dev.h"

namespace spectree {
namespace {

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPageBytes = kBlockSize * kD * 2;  // one page of one head: 4 KB
constexpr int kSlotBytes = 2 * kPageBytes;       // K page, then V page
constexpr int kMaxWavePages = 64;                // pages per wave and split (one lane holds each block index)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct StArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  uint16_t* out;
  int32_t* status;
  float* part_o;       // [items][R][D]; within each row, element e of dims 8j..8j+7 at 16e + j
  float* part_ml;      // [items][R][2]
  unsigned* counters;  // [B * Hkv], zero between calls
  int B, T, Hq, Hkv, G, R, splits, pps, max_blocks, num_blocks;
  int reorder;  // order items full splits first (B <= 64, more items than resident workgroups)
  long items;
  float sl2;
  // The tree's K/V write in the same launch (kFused): every item rotates its own
  // queries (q holds them before rotation), and each item whose range holds
  // tree keys first writes its kv head's T key and value rows into the cache.
  const uint16_t* k_new;  // [B,T,Hkv,D] the nodes' keys before rotation
  const uint16_t* v_new;  // [B,T,Hkv,D] their values
  uint16_t* kc;           // = k, = v: the cache the write fills
  uint16_t* vc;
  int rotate;             // rope_theta > 0
  double log2_theta;
};

// Waits until at most n of this wave's vector-memory operations are in flight.
// The compiler does not track the LDS side of direct global->LDS loads, so the
// kernel places these waits itself; the memory clobber keeps LDS accesses on
// their side of the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// vmcnt(8 * n): the loads of the n pages issued after the one to be read may stay in flight.
template <int DEPTH>
__device__ __forceinline__ void wait_pages_after(int n) {
  if constexpr (DEPTH >= 4) {
    if (n >= 3) {
      wait_vm<24>();
      return;
    }
  }
  if constexpr (DEPTH >= 3) {
    if (n >= 2) {
      wait_vm<16>();
      return;
    }
  }
  if constexpr (DEPTH >= 2) {
    if (n >= 1) {
      wait_vm<8>();
      return;
    }
  }
  wait_vm<0>();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

// Eight transposed V^T fragments (ds_read_b64_tr_b16 at the given LDS byte
// addresses), complete on return.  Issued from assembly because the compiler
// would otherwise drain every in-flight direct global->LDS load before them.
__device__ __forceinline__ void read_vt(s16x4 (&v)[8], uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t a4,
                                        uint32_t a5, uint32_t a6, uint32_t a7) {
  __asm__ volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4), "v"(a5), "v"(a6), "v"(a7)
      : "memory");
}

// Split partials cross workgroups (and XCDs, whose L2s are not coherent with
// each other).  They are written and read as relaxed agent-scope atomics
// (write-through stores, coherent loads), so publishing them needs only this
// wave's stores to have completed before the arrival counter is bumped -- no
// write-back or invalidation of the whole L2, which a fence would cost.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NRB, int DEPTH, bool kFused>
__global__ __launch_bounds__(256) void attn_stream_kernel(const StArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4 * DEPTH * kSlotBytes];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int quad = lane >> 4;

  // Items in launch order: splits read disjoint pages, so there is no cache
  // reuse to keep within an XCD, and dealing consecutive items to different
  // XCDs balances ragged batches.  With `reorder`, workgroup ids go first to
  // the full splits of every (b, g), then to each (b, g)'s last split, then to
  // nothing: the long items start first and the short ones fill the tail.
  long item = blockIdx.x;
  if (item >= a.items) return;
  int s = static_cast<int>(item % a.splits);
  int g = static_cast<int>((item / a.splits) % a.Hkv);
  int b = static_cast<int>(item / a.splits / a.Hkv);
  if (a.reorder) {
    int lb = lane < a.B ? a.plen[lane] : 0;
    const int cap = a.max_blocks * kBlockSize - a.T;
    lb = lb < 0 ? 0 : (lb > cap ? cap : lb);
    const int nu = lane < a.B ? (((lb + a.T + kBlockSize - 1) / kBlockSize) + a.pps - 1) / a.pps : 0;
    const int full = lane < a.B ? (nu - 1) * a.Hkv : 0;
    int incl = full;  // inclusive prefix sum over sequences
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) {
      const int o = __shfl_up(incl, w);
      if (lane >= w) incl += o;
    }
    const int F = __shfl(incl, 63);
    const int id = static_cast<int>(blockIdx.x);
    if (id < F) {
      const unsigned long long hit = __ballot(incl > id);
      b = __ffsll(static_cast<long long>(hit)) - 1;
      const int k = id - (__shfl(incl, b) - __shfl(full, b));
      const int nb = __shfl(nu, b) - 1;
      g = k / nb;
      s = k % nb;
    } else if (id - F < a.B * a.Hkv) {
      b = (id - F) / a.Hkv;
      g = (id - F) % a.Hkv;
      s = __shfl(nu, b) - 1;
    } else {
      return;
    }
    item = (static_cast<long>(b) * a.Hkv + g) * a.splits + s;
  }
  const long bg = item / a.splits;

  // Independent prologue loads: prefix length, this wave's block indices (lane
  // k holds page s*pps + wave + 4k), the parent row (lane = node), the queries.
  const int plen_raw = a.plen[b];
  const int wave_pages_max = a.pps / 4;
  const int pg_lane = s * a.pps + wave + 4 * lane;
  int blk = -1;
  if (lane < wave_pages_max && pg_lane < a.max_blocks) blk = a.bt[static_cast<long>(b) * a.max_blocks + pg_lane];
  const int par = lane < a.T ? a.parent[static_cast<long>(b) * a.T + lane] : -1;

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

  int err = 0;
  int Lb = plen_raw;
  const int cap = a.max_blocks * kBlockSize - a.T;
  if (Lb < 0 || Lb > cap) {
    err |= SPEC_DEV_LENGTH;
    Lb = Lb < 0 ? 0 : cap;
  }
  const int n_keys = Lb + a.T;
  const int npages = (n_keys + kBlockSize - 1) / kBlockSize;
  const int n_used = (npages + a.pps - 1) / a.pps;  // splits of this (b, g) that hold keys
  if (s >= n_used) return;
  const int p0 = s * a.pps;
  const int p1 = min(npages, p0 + a.pps);
  const int kend = min(n_keys, p1 * kBlockSize);
  const int n_mine = p1 - p0 > wave ? (p1 - p0 - wave + 3) / 4 : 0;
  {
    const bool real = lane < n_mine;
    const bool bad = real && !(blk >= 0 && blk < a.num_blocks);
    if (__any(bad)) err |= SPEC_DEV_BLOCK;
    blk = (real && !bad) ? blk : -1;
  }

  // Ancestor-or-self words by pointer doubling: lane i follows its parent
  // chain 1, 2, 4, ... steps at a time.  A chain that is not topological (or
  // whose root has a parent) leaves its nodes with only themselves.
  uint64_t anc_row[NRB];
  const bool tail = kend > Lb;
  int dep = 0;  // (fused) depth of node `lane`
  if (tail || kFused) {
    const bool in = lane < a.T;
    const bool valid = in && (lane == 0 ? par == -1 : (par >= 0 && par < lane));
    int j = (lane == 0 || !valid) ? lane : par;
    uint64_t A = 1ull << lane;
    int okc = valid || !in;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      A |= __shfl(A, j);
      okc &= __shfl(okc, j);
      j = __shfl(j, j);
    }
    if (__any(in && !okc)) err |= SPEC_DEV_PARENT;
    if (!okc) A = 1ull << lane;
    dep = __popcll(A) - 1;  // ancestors-or-self, less the node itself
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) anc_row[rb] = __shfl(A, node_of[rb]);
  } else {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) anc_row[rb] = 0;
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

  uint8_t* my_ring = ring + wave * DEPTH * kSlotBytes;
  // Per-lane byte offsets inside a slot.  DMA: instruction t, lane i fills LDS
  // bytes t*1024 + 16 i = key (4t + i/16), position i%16, which holds chunk
  // position ^ key of K, position ^ 2*(key % 8) of V.
  const int dma_key = lane >> 4;
  const int dma_pos = lane & 15;
  // K fragment c: key l16, chunk 4c + quad.
  // V^T fragment dt: key 4*quad + l16/4, dims dt*16 + 4*(l16%4) .. +3.
  const int vkey = 4 * quad + (l16 >> 2);
  uint32_t vt_off[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    vt_off[dt] = vkey * 256 + (((2 * dt + ((l16 & 3) >> 1)) ^ (2 * (vkey & 7))) * 16) + (l16 & 1) * 8;
  auto issue = [&](int k) {  // page k of this wave into slot k % DEPTH; k is wave-uniform
    const int bk = __builtin_amdgcn_readlane(blk, k);
    const long base = (static_cast<long>(bk < 0 ? 0 : bk) * a.Hkv + g) * (kBlockSize * kD);
    uint8_t* slot = my_ring + (k % DEPTH) * kSlotBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 4 * t + dma_key;
      const uint16_t* ks = a.k + base + key * kD + ((dma_pos ^ key) * 8);
      const uint16_t* vs = a.v + base + key * kD + ((dma_pos ^ (2 * (key & 7))) * 8);
      // every page is read by this wave only: non-temporal loads
      __builtin_amdgcn_global_load_lds(ks, slot + t * 1024, 16, 0, kLoadNT);
      __builtin_amdgcn_global_load_lds(vs, slot + kPageBytes + t * 1024, 16, 0, kLoadNT);
    }
  };

  if constexpr (kFused) {
    // Before the ring is filled: the cosines and sines of every node's pairs
    // into it ([T][64] double2, T <= 16 here), the item's queries rotated in
    // registers, and -- on an item whose range holds tree keys -- kv head g's T
    // key (rotated) and value rows written into the cache at slots Lb + i,
    // nothing for a bad parent row or prefix length (as spec_tree_kv_write).
    // The same helpers as spec_tree_kv_write, so the stored bits are the same.
    double2* trig = reinterpret_cast<double2*>(ring);
    if (a.rotate) {
      for (int nd = wave; nd < a.T; nd += 4) {
        const int d = __shfl(dep, nd);
        double c, sn;
        rope_cos_sin(Lb + d, lane, kD, a.log2_theta, &c, &sn);
        trig[nd * 64 + lane] = double2{c, sn};
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const double2* tn = trig + node_of[rb] * 64 + quad * 8;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double2 cs = tn[c * 32 + e];
            float y0, y1;
            rope_turn(static_cast<float>(qf[rb][c][e]), static_cast<float>(qf[rb][c + 2][e]), cs.x, cs.y, &y0, &y1);
            qf[rb][c][e] = __builtin_bit_cast(__bf16, f32_to_bf16(y0));
            qf[rb][c + 2][e] = __builtin_bit_cast(__bf16, f32_to_bf16(y1));
          }
      }
    }
    if (tail && !(err & (SPEC_DEV_PARENT | SPEC_DEV_LENGTH))) {
      for (int row = wave; row < 2 * a.T; row += 4) {  // row 2i: node i's key, 2i + 1: its value
        const int i = row >> 1;
        const bool isv = (row & 1) != 0;
        const uint16_t* src = (isv ? a.v_new : a.k_new) + ((static_cast<long>(b) * a.T + i) * a.Hkv + g) * kD;
        const uint16_t x0 = src[lane], x1 = src[lane + 64];
        const int t = Lb + i;
        const int bk = a.bt[static_cast<long>(b) * a.max_blocks + t / kBlockSize];
        if (bk < 0 || bk >= a.num_blocks) {
          err |= SPEC_DEV_BLOCK;
          continue;
        }
        uint16_t y0 = x0, y1 = x1;
        if (!isv && a.rotate) {
          const double2 cs = trig[i * 64 + lane];
          float f0, f1;
          rope_turn(bf16_to_f32(x0), bf16_to_f32(x1), cs.x, cs.y, &f0, &f1);
          y0 = f32_to_bf16(f0);
          y1 = f32_to_bf16(f1);
        }
        uint16_t* dst = (isv ? a.vc : a.kc) + ((static_cast<long>(bk) * a.Hkv + g) * kBlockSize + t % kBlockSize) * kD;
        dst[lane] = y0;
        dst[lane + 64] = y1;
      }
    }
    __syncthreads();  // the rows are stored (the barrier's fence waits for them) and the table is free
  }

#pragma unroll
  for (int k = 0; k < DEPTH; ++k)
    if (k < n_mine) issue(k);

  for (int k = 0; k < n_mine; ++k) {
    wait_pages_after<DEPTH>(min(n_mine - 1 - k, DEPTH - 1));
    uint8_t* slot = my_ring + (k % DEPTH) * kSlotBytes;
    const int page = p0 + wave + 4 * k;
    const int key0 = page * kBlockSize;
    const int bk = __builtin_amdgcn_readlane(blk, k);
    const int nvalid = bk < 0 ? 0 : min(kBlockSize, kend - key0);
    if (nvalid < kBlockSize) {
      // keys past the split (or a whole invalid page): zero their V rows so that
      // p = 0 never meets a NaN; their scores are masked below
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (4 * t + dma_key >= nvalid)
          *reinterpret_cast<u32x4*>(slot + kPageBytes + (4 * t + dma_key) * 256 + dma_pos * 16) = u32x4{0, 0, 0, 0};
    }
    bf16x8 kf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kf[c] = __builtin_bit_cast(bf16x8,
                                 *reinterpret_cast<const u32x4*>(slot + l16 * 256 + (((4 * c + quad) ^ l16) * 16)));
    s16x4 vf[8];
    {
      const uint32_t vb = lds_addr(slot + kPageBytes);
      read_vt(vf, vb + vt_off[0], vb + vt_off[1], vb + vt_off[2], vb + vt_off[3], vb + vt_off[4], vb + vt_off[5],
              vb + vt_off[6], vb + vt_off[7]);
    }
    wait_lds();  // the slot is in registers: refill it
    if (k + DEPTH < n_mine) issue(k + DEPTH);

    const bool need_mask = nvalid < kBlockSize || key0 + kBlockSize > Lb;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[rb][c], sacc, 0, 0, 0);
      // lane holds S[row l16][key 4*quad + i]
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[i] * a.sl2;
        if (need_mask) {
          const int kin = 4 * quad + i;
          const int pos = key0 + kin;
          bool ok = kin < nvalid;
          if (ok && pos >= Lb) ok = (anc_row[rb] >> (pos - Lb)) & 1ull;
          x = ok ? x : -INFINITY;
        }
        sv[i] = x;
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);
      const bool none = (m_new == -INFINITY);
      bf16x4 pb;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = none ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_new);
        psum += p;
        pb[i] = static_cast<__bf16>(p);
      }
      if (!__all(m_new == m_run[rb])) {  // the running max moved somewhere in the wave: rescale
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[rb][dt] *= alpha;
      }
      l_run[rb] += psum;
      m_run[rb] = m_new;
      const s16x4 pf = __builtin_bit_cast(s16x4, pb);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[dt], pf, o[rb][dt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16);
    l_run[rb] += __shfl_xor(l_run[rb], 32);
  }
  report(a.status, b, err);

  // merge the four waves, 16 rows at a time, through LDS (the rings are drained)
  float* mo = reinterpret_cast<float*>(ring);  // [4][16][128]
  float* ml = mo + 4 * 16 * kD;                // [4][16][2]
  const int row = tid >> 4;
  const int dseg = (tid & 15) * 8;
  const bool direct = n_used == 1;
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
        // element e of dims dseg .. dseg+7 at e*16 + dseg/8: each store instruction writes whole lines
        float* po = a.part_o + (item * a.R + r) * kD + (tid & 15);
#pragma unroll
        for (int e = 0; e < 8; ++e) st_agent(po + e * 16, acc[e]);
        if ((tid & 15) == 0) {
          st_agent(&a.part_ml[(item * a.R + r) * 2 + 0], mstar);
          st_agent(&a.part_ml[(item * a.R + r) * 2 + 1], lstar);
        }
      }
    }
  }
  if (direct) return;

  // the last of the n_used workgroups of (b, g) to arrive merges their partials
  wait_vm<0>();  // this wave's partial stores have reached the coherent level
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&a.counters[bg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<unsigned>(n_used - 1));
  }
  __syncthreads();
  if (!s_last) return;
  const long first = bg * a.splits;
  for (int r = row; r < a.R; r += 16) {
    // online merge over the splits, 8 partials' loads in flight at a time
    float mstar = -INFINITY, lstar = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sp0 = 0; sp0 < n_used; sp0 += 8) {
      float ms[8], ls[8];
      f32x4 x0[8], x1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
        x0[k] = x1[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sp0 + k < n_used) {
          const long it = first + sp0 + k;
          ms[k] = ld_agent(&a.part_ml[(it * a.R + r) * 2]);
          ls[k] = ld_agent(&a.part_ml[(it * a.R + r) * 2 + 1]);
          const float* po = a.part_o + (it * a.R + r) * kD + (tid & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[k][e] = ld_agent(po + e * 16);
            x1[k][e] = ld_agent(po + (4 + e) * 16);
          }
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
  if (tid == 0) __hip_atomic_store(&a.counters[bg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NRB, int DEPTH>
hipError_t run_stream(const StArgs& args, bool fused, hipStream_t stream) {
  const long grid = args.items;
  if (fused)
    hipLaunchKernelGGL((attn_stream_kernel<NRB, DEPTH, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       args);
  else
    hipLaunchKernelGGL((attn_stream_kernel<NRB, DEPTH, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                       stream, args);
  return hipGetLastError();
}

}  // namespace

// Plan for the streaming kernel (the kernel takes up to 64 rows per (b, g); the
// attention planner sends it at most 16, one 16-row block, and only that shape
// is instantiated).  Pages per split are a
// multiple of 4 (one page per wave and round), at most 4 * 64.  A workgroup
// with DEPTH slots per wave holds 4 * DEPTH * 8 KB of LDS, so 160 KB fits
// 160 / (32 DEPTH) of them per CU; the split size minimises the estimated
// makespan: rounds of resident workgroups times (pages per wave + a fixed cost
// of a few pages' time for the prologue latency and the merge).
#ifndef SPEC_STREAM_DEPTH
#define SPEC_STREAM_DEPTH 3
#endif
#ifndef SPEC_STREAM_RAGGED_PPS
#define SPEC_STREAM_RAGGED_PPS 256
#endif
#ifndef SPEC_STREAM_OVERHEAD_PAGES
#define SPEC_STREAM_OVERHEAD_PAGES 3
#endif
void plan_stream(AttnPlan& p, int B, int Hkv, int max_blocks) {
  p.mode = 3;
  p.rt = p.rows;
  p.nrb = (p.rows + 15) / 16;
  p.n_rt = 1;
  p.depth = SPEC_STREAM_DEPTH;
  const long bg = static_cast<long>(B) * Hkv;
  const long per_cu = std::max(1, 160 / (32 * p.depth));
  const long slots = 256 * per_cu;
  long best_pps = 4 * kMaxWavePages;
  double best = 1e30;
  // Much more work than wave slots (batched serving): bounded items, so that
  // ragged sequence lengths leave a short tail.
  const long max_pps =
      static_cast<long>(max_blocks) * bg >= 8 * slots * 64 ? SPEC_STREAM_RAGGED_PPS : 4 * kMaxWavePages;
  for (long pps = 4; pps <= max_pps; pps += 4) {
    const long splits = (max_blocks + pps - 1) / pps;
    const long items = bg * splits;
    const long rounds = (items + slots - 1) / slots;
    const double cost = static_cast<double>(rounds) * (static_cast<double>(pps) / 4 + SPEC_STREAM_OVERHEAD_PAGES);
    if (cost < best - 1e-9) {
      best = cost;
      best_pps = pps;
    }
  }
  p.pps = static_cast<int>(best_pps);
  p.splits = static_cast<int>((max_blocks + best_pps - 1) / best_pps);
  p.items = bg * p.splits;
  const size_t head = (static_cast<size_t>(bg) * sizeof(unsigned) + 255) / 256 * 256;
  p.ws_bytes = p.splits > 1 ? head + static_cast<size_t>(p.items) * p.rows * (kD + 2) * sizeof(float) : 0;
}

static StArgs stream_args(const AttnPlan& plan, const AttnLaunch& L) {
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
  a.reorder = (plan.splits > 1 && L.B <= 64 && plan.items > 256L * std::max(1, 160 / (32 * plan.depth))) ? 1 : 0;
  if (plan.splits > 1) {
    const size_t bg = static_cast<size_t>(L.B) * L.Hkv;
    a.counters = static_cast<unsigned*>(L.workspace);
    const size_t head = (bg * sizeof(unsigned) + 255) / 256 * 256;
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + head);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rows * kD;
  }
  return a;
}

hipError_t launch_attn_stream(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  if (plan.nrb != 1 || plan.depth != SPEC_STREAM_DEPTH) return hipErrorInvalidValue;  // not a planned shape
  return run_stream<1, SPEC_STREAM_DEPTH>(stream_args(plan, L), false, stream);
}

hipError_t launch_attn_stream_write(const AttnPlan& plan, const AttnWriteLaunch& W, hipStream_t stream) {
  if (plan.nrb != 1 || plan.depth != SPEC_STREAM_DEPTH || W.attn.T > 16) return hipErrorInvalidValue;
  StArgs a = stream_args(plan, W.attn);
  a.k_new = static_cast<const uint16_t*>(W.k_new);
  a.v_new = static_cast<const uint16_t*>(W.v_new);
  a.kc = static_cast<uint16_t*>(const_cast<void*>(W.attn.k));
  a.vc = static_cast<uint16_t*>(const_cast<void*>(W.attn.v));
  a.rotate = W.theta > 0.0f ? 1 : 0;
  a.log2_theta = W.theta > 0.0f ? log2(static_cast<double>(W.theta)) : 0.0;
  return run_stream<1, SPEC_STREAM_DEPTH>(a, true, stream);
}

}  // namespace spectree
