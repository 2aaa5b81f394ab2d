// Tree-masked verify attention, bf16 inputs, head dim 128, gfx950 matrix cores:
// planning for every bf16 shape, and the kernel for more than 16 query rows per
// kv head (trees times GQA groups).  Shapes with <= 16 rows (chains, decode,
// small trees) use the streaming kernel (attn_stream.hip).
//
// Work item = (sequence b, kv head g, KV split s, row tile rt).  The query rows
// of one (b, g) are the T tree nodes times the G query heads of the group
// (row r -> node r / G, head g*G + r % G), so one pass over a KV page serves
// every tree query of the GQA group.  Keys are the logical positions
// 0 .. prefix+T-1 of the sequence, read page by page through the block table;
// keys at prefix + j are tree nodes and are masked by the ancestor-or-self
// bitset of the row's node (the tree_mask of the EAGLE implementation summary
// in "Report: Support nextn speculative decoding").  Splits that start past a
// sequence's end exit at once and take no part in its merge.
//
// A workgroup holds 4 waves x NRB blocks of 16 rows (NRB = 1: 64 rows, up to
// 64 rows per kv head; NRB = 2: 128 rows), at most 256 registers per lane, two
// workgroups per CU, so that while one wave of a SIMD waits on its softmax
// chain the other keeps the matrix core busy.  Per iteration the
// workgroup takes a 64-key tile (4 pages of K, 4 of V), each wave bringing one
// page of each straight from HBM into LDS (direct global->LDS loads, double
// buffered, so the next tile streams in while this one is used).  Each wave then
// computes, per 32-key half (a pair of pages) and row block, S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (8 scores of one row per lane), the online softmax in
// the log2 domain, and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16 whose 32-key
// operand holds 4 keys of each page per lane (V^T fragments from
// ds_read_b64_tr_b16).  One split writes the normalised output; several write
// unnormalised partials (O, m, l) and the last workgroup of a (b, g, rt) to
// finish merges them (arrival counter in the workspace, reset by that
// workgroup).
//
// A ragged batch with more items than resident workgroups (64-row tiles, one
// row tile per (b, g)) is instead cut stream-K fashion: the (b, g) are laid end
// to end as tiles plus a fixed cost each, and every resident workgroup takes an
// equal range of that line, so all of them finish together whatever the mix of
// lengths; a (b, g) cut between workgroups is merged like the splits (see
// SkPlan).
#include <algorithm>
#include <cmath>

#include "common.h"
#include "rope_dev.h"

namespace spectree {
namespace {

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr unsigned kFlagSpinLimit = 1u << 24;  // polls of a write item's flag (a few seconds)
constexpr int kPageBytes = kBlockSize * kD * 2;  // one page of one head: 4 KB
constexpr int kTileBytes = 8 * kPageBytes;       // 4 K pages, then 4 V pages: 64 keys
constexpr int kMaxSplitPages = 1024;             // pages per split (planning keeps below)
constexpr int kMaxPiecePages = 1536;             // pages per piece of the stream-K split (64-row tiles)
// The stream-K split weighs each (b, g) as its tiles plus kSkItemUnits tiles'
// worth of fixed cost (block indices and queries, the first tile's latency,
// the ancestor sets, the epilogue) and a write chunk as kSkWriteUnits tiles.
constexpr int kSkItemUnits = 5;
constexpr int kSkWriteUnits = 6;

__device__ __forceinline__ void wait_vm0() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

// Fragments of the two pages of a 32-key half (page A at LDS byte address base,
// page B at base + 4096), complete on return.  Issued from assembly: the compiler
// would otherwise drain every in-flight direct global->LDS load (the next tile)
// before them.
// K: kA[c], kB[c] = ds_read_b128 at base (+4096) + koff[c].
__device__ __forceinline__ void read_k_pair(u32x4 (&kA)[4], u32x4 (&kB)[4], uint32_t base, const uint32_t (&koff)[4]) {
  __asm__ volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %9 offset:4096\n\t"
      "ds_read_b128 %6, %10 offset:4096\n\t"
      "ds_read_b128 %7, %11 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kA[0]), "=&v"(kA[1]), "=&v"(kA[2]), "=&v"(kA[3]), "=&v"(kB[0]), "=&v"(kB[1]), "=&v"(kB[2]), "=&v"(kB[3])
      : "v"(base + koff[0]), "v"(base + koff[1]), "v"(base + koff[2]), "v"(base + koff[3])
      : "memory");
}
// V^T: vA[dt], vB[dt] = ds_read_b64_tr_b16 at base (+4096) + voff[dt].
__device__ __forceinline__ void read_vt_pair(u32x2 (&vA)[8], u32x2 (&vB)[8], uint32_t base,
                                             const uint32_t (&voff)[8]) {
  __asm__ volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %20\n\t"
      "ds_read_b64_tr_b16 %5, %21\n\t"
      "ds_read_b64_tr_b16 %6, %22\n\t"
      "ds_read_b64_tr_b16 %7, %23\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:4096\n\t"
      "ds_read_b64_tr_b16 %13, %21 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vA[0]), "=&v"(vA[1]), "=&v"(vA[2]), "=&v"(vA[3]), "=&v"(vA[4]), "=&v"(vA[5]), "=&v"(vA[6]), "=&v"(vA[7]),
        "=&v"(vB[0]), "=&v"(vB[1]), "=&v"(vB[2]), "=&v"(vB[3]), "=&v"(vB[4]), "=&v"(vB[5]), "=&v"(vB[6]), "=&v"(vB[7])
      : "v"(base + voff[0]), "v"(base + voff[1]), "v"(base + voff[2]), "v"(base + voff[3]), "v"(base + voff[4]),
        "v"(base + voff[5]), "v"(base + voff[6]), "v"(base + voff[7])
      : "memory");
}

__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// max(a, b) for operands that are not NaN, as one v_med3(a, b, pinf) with pinf
// = +inf known only at run time (fmaxf quiets signalling NaNs first, one more
// instruction per operand, and so does the med3 of a constant +inf, which the
// compiler turns back into a max)
__device__ __forceinline__ float max_nn(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr long kWFirst = 12;  // pages of a first-round split, in eighths of a second-round one's
constexpr float kLazyLog2 = 8.f;  // how far (log2 units) a row's max may pass the reference max
constexpr bf16x2 kBf16Ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

// Max / sum over the four lanes l%16 + 16q of a row (VALU lane swaps, no LDS):
// v_permlane16_swap of a value with a copy of itself leaves rows (0,1) and (2,3)
// of the two registers exchanged, so combining them joins lanes l and l^16;
// v_permlane32_swap likewise joins l and l^32.  Written in assembly because,
// given one value for both operands, the compiler keeps only one of the two
// results of the swap builtins.
__device__ __forceinline__ float quad_max(float x) {
  float y;
  __asm__(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(y));
  return x;
}
__device__ __forceinline__ float quad_sum(float x) {
  float y;
  __asm__(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %1"
      : "+v"(x), "=&v"(y));
  return x;
}

struct TArgs2 {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* plen;
  const int32_t* parent;
  uint16_t* out;
  int32_t* status;
  float* part_o;       // [slots][RT][D]: one slot an item, or (stream-K) two a workgroup
  float* part_ml;      // [slots][RT][2]
  unsigned* counters;  // [B * Hkv * n_rt] arrivals, then [unused, workgroups done]
  int B, T, Hq, Hkv, G, R, n_rt, splits, pps, max_blocks, num_blocks;
  int streamk;    // the stream-K split (64-row tiles, one row tile per (b, g), B <= 64)
  int kv_stream;  // every K/V page is read by one item only: load it non-temporally
  long items;
  float sl2;
  float pinf;   // +inf
  int n_first;  // workgroups of the first dispatch round when the grid is two rounds of one a CU, else 0
  // The tree's K/V write in the same launch (stream-K split only): n_write
  // chunks, n_chunks per sequence (chunk_rows of its 2 T Hkv K and V rows
  // each), each claimed before it is written; attention pieces rotate their
  // own queries, and a piece that holds tree keys waits until its sequence's
  // chunks are all written.
  int n_write;             // B * n_chunks
  int n_chunks;            // per sequence: ceil(2 T Hkv / chunk_rows)
  int chunk_rows;          // a multiple of 8, at most 64
  int rotate;              // rope_theta > 0 (`q` holds the queries before rotation)
  double log2_theta;
  const uint16_t* k_new;   // [B,T,Hkv,D] the nodes' keys before rotation
  const uint16_t* v_new;   // [B,T,Hkv,D] their values
  uint16_t* kc;            // = k, = v: the cache the write items fill
  uint16_t* vc;
  unsigned* flags;         // [B]: chunks of the sequence written so far, then [n_write] claim words
};

constexpr int kAncWords = kMaxT / 64;  // words of one node's ancestor-or-self bitset

// Ancestor-or-self bitsets of every node of a parent row, by pointer doubling:
// anc[i] holds the path from i up to, not including, jump[i] (at first {i},
// jump[i] = i's parent); each round joins the set of jump[i] and takes over its
// jump, so ceil(log2(T)) rounds cover every path (a path has at most T nodes).
// A node whose parent is not an earlier node (or the root's is not -1) ends its
// path there.  `jump` is the parent row (overwritten); `anc` holds T x
// kAncWords words.  Every thread of the 256-thread workgroup calls it (T <=
// 512); its barriers wait for LDS only (see lds_barrier), the first one for
// every earlier reader of `jump` and `anc`, the last one publishing `anc`.
__device__ int build_ancestors_lds(int* jump, int T, uint64_t* anc) {
  const int tid = threadIdx.x;
  const int nw = (T + 63) >> 6;
  int err = 0;
  lds_barrier();
  for (int i = tid; i < T; i += 256) {
    const int p = jump[i];
    if (!(i == 0 ? p == -1 : (p >= 0 && p < i))) {
      err = SPEC_DEV_PARENT;
      jump[i] = -1;
    }
#pragma unroll
    for (int w = 0; w < kAncWords; ++w)
      if (w < nw) anc[i * kAncWords + w] = (w == (i >> 6)) ? 1ull << (i & 63) : 0ull;
  }
  const int rounds = T > 1 ? 32 - __clz(T - 1) : 0;
  for (int round = 0; round < rounds; ++round) {
    lds_barrier();  // the last round's writes (or the initial sets) are visible
    uint64_t add[2][kAncWords];
    int nj[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k;
      nj[k] = -2;  // nothing to join
      const int j = i < T ? jump[i] : -1;
      if (j >= 0) {
        nj[k] = jump[j];
#pragma unroll
        for (int w = 0; w < kAncWords; ++w) add[k][w] = w < nw ? anc[j * kAncWords + w] : 0ull;
      }
    }
    lds_barrier();  // every read of this round before any write
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k;
      if (nj[k] != -2) {
#pragma unroll
        for (int w = 0; w < kAncWords; ++w)
          if (w < nw) anc[i * kAncWords + w] |= add[k][w];
        jump[i] = nj[k];
      }
    }
  }
  lds_barrier();
  return err;
}

template <int NRB>
struct TileLds {
  __attribute__((aligned(16))) uint8_t tiles[2 * kTileBytes];  // 2 x (4 K pages, 4 V pages)
  uint64_t anc[64 * NRB * kAncWords];  // the bitsets of the item's nodes (at most one per row)
  int s_par[kMaxT];
  int s_blk[NRB == 1 ? kMaxPiecePages : kMaxSplitPages];
  int s_last, s_next;
};
static_assert(kMaxT * kAncWords * sizeof(uint64_t) <= kTileBytes,
              "the whole tree's bitsets are built in the second tile buffer");

constexpr int kTrigDepths = 27;  // depths whose cosines and sines a fused item tabulates (27 KB of LDS)
constexpr int kTrigOffset = 2 * kMaxT * sizeof(int) + 256;  // the table's place in its 32 KB buffer
static_assert(kTrigOffset + kTrigDepths * 64 * sizeof(double2) <= kTileBytes, "the table fits a tile buffer");

__device__ __forceinline__ void st_agent_u32(uint16_t* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every node's depth by pointer doubling over a parent row in LDS (a node whose
// parent is not an earlier node stops its path there): s_dep[i], with s_up as
// scratch.  Every thread of the 256-thread workgroup calls it (T <= 512); the
// rounds' barriers also publish what the caller wrote to LDS before the call.
__device__ void tree_depths(const int* par, int T, int* s_up, int* s_dep) {
  const int tid = threadIdx.x;
  int pending = 0;
  for (int i = tid; i < T; i += 256) {
    const int p = par[i];
    const bool ok = i == 0 ? p == -1 : (p >= 0 && p < i);
    s_up[i] = (i == 0 || !ok) ? -1 : p;
    s_dep[i] = i == 0 ? 0 : 1;
    pending |= s_up[i] >= 0;
  }
  // each round: up = the ancestor twice as far above (or -1); the rounds end
  // once no node has an ancestor left to jump to (ceil(log2(depth)) of them)
  while (__syncthreads_or(pending)) {
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
    pending = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k;
      if (i < T) {
        s_up[i] = up[k];
        s_dep[i] = dep[k];
        pending |= up[k] >= 0;
      }
    }
  }
}

constexpr int kWalkSteps = 32;  // parent chains walked one step at a time up to this length

// Depths of nodes n0 .. n1 (at most 256 of them) into s_dep: each by walking its
// parent chain when every such chain is at most kWalkSteps long (a bad parent
// ends a chain), else for the whole tree by pointer doubling (tree_depths); and
// their [min, max] into s_rng.  Every thread of the workgroup calls it.
__device__ void node_depths(const int* par, int T, int n0, int n1, int* s_up, int* s_dep, int* s_rng) {
  const int tid = threadIdx.x;
  const int i = n0 + tid;
  int d = 0, j = i;
  if (i <= n1) {
    for (int k = 0; k < kWalkSteps && j > 0; ++k) {
      const int p = par[j];
      if (!(p >= 0 && p < j)) {
        j = 0;
        break;
      }
      j = p;
      ++d;
    }
  }
  if (tid == 0) {
    s_rng[0] = 0x7fffffff;
    s_rng[1] = -1;
  }
  if (__syncthreads_or(i <= n1 && j > 0)) {
    tree_depths(par, T, s_up, s_dep);
  } else if (i <= n1) {
    s_dep[i] = d;
  }
  __syncthreads();
  if (i <= n1) {
    atomicMin(&s_rng[0], s_dep[i]);
    atomicMax(&s_rng[1], s_dep[i]);
  }
  __syncthreads();
}

// Cosine and sine at position p of pair j (out of line: it would take registers from the item).
__device__ __noinline__ double2 trig_direct(int p, int j, double log2_theta) {
  double c, sn;
  rope_cos_sin(p, j, kD, log2_theta, &c, &sn);
  return double2{c, sn};
}

// Cosines and sines of every (depth d in [dmin, dmin + n), pair j < 64) at
// position Lb + d into trig[(d - dmin) * 64 + j], when n <= kTrigDepths (in
// line: a call would make the caller wait for every load in flight).
__device__ __forceinline__ void fill_trig(double2* trig, int Lb, int dmin, int n, double log2_theta) {
  if (n > kTrigDepths) return;
  for (int e = threadIdx.x; e < n * 64; e += 256) {
    double c, sn;
    rope_cos_sin(Lb + dmin + (e >> 6), e & 63, kD, log2_theta, &c, &sn);
    trig[e] = double2{c, sn};
  }
}

__device__ __forceinline__ void trig_of(const double2* trig, int Lb, int dmin, int n, int d, int j, double log2_theta,
                                        double* c, double* sn) {
  const double2 cs = n <= kTrigDepths ? trig[(d - dmin) * 64 + j] : trig_direct(Lb + d, j, log2_theta);
  *c = cs.x;
  *sn = cs.y;
}

// Depth of node i by walking its parent row (a parent that is not an earlier
// node ends the walk there, as in node_depths).
__device__ __forceinline__ int walk_depth(const int* par, int i) {
  int d = 0;
  while (i > 0) {
    const int p = par[i];
    if (!(p >= 0 && p < i)) break;
    i = p;
    ++d;
  }
  return d;
}

// Rotates the lane's query fragments for their rows' positions Lb + depth: the
// fragment holds dims c*32 + quad*8 + e (c < 4, e < 8), so the pairs (j, j +
// 64) of the rotation are (c, c + 2) for c < 2, all within the lane.  Each lane
// walks its rows' parent chains; the cosines and sines of the item's range of
// depths are tabulated in `buf` (a free 32 KB tile buffer) behind LDS-only
// barriers, so a tile already issued stays in flight meanwhile.  The table is
// read until the caller's next barrier.
template <int NRB>
__device__ __forceinline__ void rotate_queries(const TArgs2& a, int Lb, int row_base, int l16, int quad,
                                               const int* par, uint8_t* buf, bf16x8 (&qf)[NRB][4]) {
  int* s_rng = reinterpret_cast<int*>(buf);  // each wave's [min, max] depth of its rows' nodes
  double2* trig = reinterpret_cast<double2*>(buf + kTrigOffset);
  int dep[NRB];
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row_base + rb * 16 + l16;
    dep[rb] = r < a.R ? walk_depth(par, r / a.G) : 0;
    if (r < a.R) {
      lo = min(lo, dep[rb]);
      hi = max(hi, dep[rb]);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  // the item's range from the waves' ranges (plain LDS stores: LDS atomics
  // would wait for the tile in flight)
  if ((threadIdx.x & 63) == 0) {
    s_rng[2 * (threadIdx.x >> 6)] = lo;
    s_rng[2 * (threadIdx.x >> 6) + 1] = hi;
  }
  lds_barrier();
  int dmin = s_rng[0], dmax = s_rng[1];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    dmin = min(dmin, s_rng[2 * w]);
    dmax = max(dmax, s_rng[2 * w + 1]);
  }
  const int n = dmax >= dmin ? dmax - dmin + 1 : 0;
  fill_trig(trig, Lb, dmin, n, a.log2_theta);
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row_base + rb * 16 + l16;
    if (r >= a.R) continue;
    const int d = dep[rb];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 lo4 = __builtin_bit_cast(u32x4, qf[rb][c]), hi4 = __builtin_bit_cast(u32x4, qf[rb][c + 2]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t nlo = 0, nhi = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          double cs, sn;
          trig_of(trig, Lb, dmin, n, d, c * 32 + quad * 8 + 2 * k + h, a.log2_theta, &cs, &sn);
          float y0, y1;
          rope_turn(bf16_to_f32(static_cast<uint16_t>(lo4[k] >> (16 * h))),
                    bf16_to_f32(static_cast<uint16_t>(hi4[k] >> (16 * h))), cs, sn, &y0, &y1);
          nlo |= static_cast<uint32_t>(f32_to_bf16(y0)) << (16 * h);
          nhi |= static_cast<uint32_t>(f32_to_bf16(y1)) << (16 * h);
        }
        lo4[k] = nlo;
        hi4[k] = nhi;
      }
      qf[rb][c] = __builtin_bit_cast(bf16x8, lo4);
      qf[rb][c + 2] = __builtin_bit_cast(bf16x8, hi4);
    }
  }
}

// One 16-key page of K and of V (a kv head's 4 KB each) straight into LDS,
// 16 bytes a lane: bytes t*1024 + 16 i hold key 4t + i/16, chunk position
// i%16, which is chunk position ^ key of K and position ^ 2*(key % 8) of V.
// kAux: the loads' cache policy (kLoadNT for pages no other workgroup reads).
template <int kAux>
__device__ __forceinline__ void load_kv_page(const uint16_t* kp, const uint16_t* vp, uint8_t* kdst, uint8_t* vdst,
                                             int dma_key, int dma_pos) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int key = 4 * t + dma_key;
    __builtin_amdgcn_global_load_lds(kp + key * kD + ((dma_pos ^ key) * 8), kdst + t * 1024, 16, 0, kAux);
    __builtin_amdgcn_global_load_lds(vp + key * kD + ((dma_pos ^ (2 * (key & 7))) * 8), vdst + t * 1024, 16, 0, kAux);
  }
}

// One piece of attention work: the rows of row tile rt of (b, g) against pages
// [p0, p1) of its keys, sequence b's prefix length already clamped to its valid
// range (err: SPEC_DEV_LENGTH if it was not).  Every thread of the workgroup
// calls tile_item_run; it returns at points the whole workgroup reaches
// together, or after its merge.  n_parts pieces of (b, g, rt) hold keys (one: the
// output is written directly); otherwise this piece's partial goes to slot
// pslot, arrivals are counted at counters[bgr], and the last piece to arrive
// merges the partials of slots part_slot(0 .. n_parts - 1).  Every field is
// wave-uniform.
struct Piece {
  int b, g, rt, p0, p1, n_parts;
  long pslot, bgr;
};

template <int NRB>
__device__ __forceinline__ void write_item(const TArgs2& a, int b, int chunk, TileLds<NRB>& L);

template <int NRB, bool kFused, class PartSlot>
__device__ __forceinline__ void tile_item_run(const TArgs2& a, const Piece& pc, int Lb, int err, TileLds<NRB>& L,
                                              PartSlot part_slot) {
  constexpr int RT = 64 * NRB;  // rows per workgroup
  uint8_t* tiles = L.tiles;
  uint64_t* anc = L.anc;
  int* s_par = L.s_par;
  int* s_blk = L.s_blk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int rt = pc.rt, g = pc.g, b = pc.b;
  const int n_keys = Lb + a.T;
  const int p0 = pc.p0, p1 = pc.p1;
  const int kend = min(n_keys, p1 * kBlockSize);
  const int n_it = p1 > p0 ? (p1 - p0 + 3) / 4 : 0;
  const bool tail = n_it > 0 && kend > Lb;

  // The split's block indices and the parent row are staged once in LDS, the
  // query fragments loaded beside them (one memory latency for all three); the
  // first tile is issued as soon as the indices are in, and the ancestor sets
  // are built while it lands.  With the K/V write in the same launch an item
  // that holds tree keys first waits for its sequence's rows (the count is read
  // with the indices), and every item rotates its own queries while its first
  // tile lands.
  unsigned written = 0;
  if (kFused && tail && tid == 0)
    written = __hip_atomic_load(&a.flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
  for (int i = tid; i < p1 - p0; i += 256) {
    const int blk = bt_b[p0 + i];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    if (!ok) err |= SPEC_DEV_BLOCK;
    s_blk[i] = ok ? blk : -1;
  }
  if (tail || (kFused && a.rotate))
    for (int i = tid; i < a.T; i += 256) s_par[i] = a.parent[static_cast<long>(b) * a.T + i];

  // query fragments (B operand of S^T): Q[row][c*32 + quad*8 .. +7]
  const int row_base = rt * RT + wave * NRB * 16;
  const int node0 = (rt * RT) / a.G;  // the item's first node: its rows hold nodes node0 .. node0 + RT - 1 at most
  bf16x8 qf[NRB][4];
  int node_of[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row_base + rb * 16 + l16;
    node_of[rb] = r < a.R ? r / a.G - node0 : 0;  // index among the item's nodes
  }
  auto load_q = [&]() {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = row_base + rb * 16 + l16;
      if (r < a.R) {
        const int node = r / a.G, hh = r % a.G;
        const uint16_t* qp = a.q + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD + quad * 8;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          qf[rb][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + c * 32));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) qf[rb][c] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      }
    }
  };
  load_q();
  float m_run[NRB], l_run[NRB];
  f32x4 o[NRB][8];
  const float lazy = kLazyLog2 / a.sl2;  // scale > 0
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Tiles of 64 keys (4 pages), double-buffered in LDS.  For tile `it`, wave w
  // brings page 4*it + w straight from HBM into LDS (direct global->LDS loads):
  // K key-major with 16-byte chunk c of key k at position c ^ k, V key-major with
  // chunk c at c ^ 2*(k % 8), so the K fragments are conflict-free ds_read_b128
  // and the V^T fragments conflict-free ds_read_b64_tr_b16.  Pages past the split
  // (or with an invalid block) re-read a valid page and are masked; their V rows
  // are zeroed so that p = 0 never meets a NaN.
  const int dma_key = lane >> 4, dma_pos = lane & 15;
  auto tile_page = [&](int it) { return p0 + 4 * it + wave; };
  auto page_block = [&](int pg) { return pg < p1 ? s_blk[pg - p0] : -1; };
  auto issue_tile = [&](int it) {
    const int pg = tile_page(it);
    const int blk = page_block(min(pg, p1 - 1));
    const long base = (static_cast<long>(blk < 0 ? 0 : blk) * a.Hkv + g) * (kBlockSize * kD);
    uint8_t* kdst = tiles + (it & 1) * kTileBytes + wave * kPageBytes;
    uint8_t* vdst = kdst + 4 * kPageBytes;
    if (a.kv_stream)
      load_kv_page<kLoadNT>(a.k + base, a.v + base, kdst, vdst, dma_key, dma_pos);
    else
      load_kv_page<0>(a.k + base, a.v + base, kdst, vdst, dma_key, dma_pos);
  };
  // per-lane LDS offsets of the fragments within one page
  uint32_t k_off[4], vt_off[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_off[c] = l16 * 256 + (((4 * c + quad) ^ l16) * 16);
  {
    const int vkey = 4 * quad + (l16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      vt_off[dt] = vkey * 256 + (((2 * dt + ((l16 & 3) >> 1)) ^ (2 * (vkey & 7))) * 16) + (l16 & 1) * 8;
  }

  if (kFused && tail) {
    // Sequence b's tree rows are written by the chunks' own workgroups first;
    // a chunk nobody has claimed yet (its workgroup not started: the device
    // holding other work) is written here instead, so the wait below always
    // ends (the bound only guards the loop).  The tile buffers are still free.
    if (tid == 0) L.s_next = written < static_cast<unsigned>(a.n_chunks) ? 1 : 0;
    __syncthreads();
    if (L.s_next) {
      unsigned* claim = a.flags + a.B + static_cast<long>(b) * a.n_chunks;
      for (int c = 0; c < a.n_chunks; ++c) {
        __syncthreads();  // every wave has read s_last before it is rewritten
        if (tid == 0)
          L.s_last = __hip_atomic_exchange(claim + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u ? 1 : 0;
        __syncthreads();
        if (L.s_last) write_item<NRB>(a, b, c, L);
      }
    }
  }
  if (kFused && tail && tid == 0) {
    for (unsigned spins = 0; written < static_cast<unsigned>(a.n_chunks); ++spins) {
      if (spins > kFlagSpinLimit) {
        err |= SPEC_DEV_TIMEOUT;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      written = __hip_atomic_load(&a.flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // s_blk and s_par are ready (and, fused, the tree's rows are written)
  if (n_it > 0) issue_tile(0);
  if constexpr (kFused) {
    if (a.rotate) {
      rotate_queries<NRB>(a, Lb, row_base, l16, quad, s_par, tiles + kTileBytes, qf);
    }
  }
  if (tail) {
    // the whole tree's bitsets in tile buffer 1 (first written by tile 1, issued
    // after the loop's first barrier), then the item's nodes' ones into `anc`
    uint64_t* full = reinterpret_cast<uint64_t*>(tiles + kTileBytes);
    err |= build_ancestors_lds(s_par, a.T, full);
    const int nw = (a.T + 63) >> 6;
    for (int e = tid; e < RT * kAncWords; e += 256) {
      const int node = node0 + e / kAncWords, w = e % kAncWords;
      anc[e] = (node < a.T && w < nw) ? full[node * kAncWords + w] : 0ull;
    }
  }

  for (int it = 0; it < n_it; ++it) {
    wait_vm0();  // this wave's page of tile `it` has landed
    {
      const int pg = tile_page(it);
      const int nvalid = page_block(pg) < 0 ? 0 : min(kBlockSize, kend - pg * kBlockSize);
      uint8_t* vpage = tiles + (it & 1) * kTileBytes + 4 * kPageBytes + wave * kPageBytes;
      if (nvalid < kBlockSize) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (4 * t + dma_key >= nvalid)
            *reinterpret_cast<u32x4*>(vpage + (4 * t + dma_key) * 256 + dma_pos * 16) = u32x4{0, 0, 0, 0};
      }
    }
    __syncthreads();  // tile `it` is complete and every wave is done with tile it-1
    if (it + 1 < n_it) issue_tile(it + 1);

    const uint8_t* kt = tiles + (it & 1) * kTileBytes;
    const uint8_t* vt = kt + 4 * kPageBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 32-key halves: pages 2h (A) and 2h+1 (B)
      const int key0 = (p0 + 4 * it + 2 * h) * kBlockSize;
      const bool need_mask = key0 + 32 > Lb || key0 + 32 > kend;
      // Bit t of vis[rb] (before the shift by 4*quad) says whether key key0 + t is
      // visible to the lane's row: prefix keys are, tree keys by the ancestor
      // bitset, keys at or past the split end are not.  Shifts are uniform.
      uint32_t vis[NRB];
      if (need_mask) {
        const int d = key0 - Lb;  // tree index of key0 (negative inside the prefix)
        const int nv = kend - key0;
        const uint32_t endm = nv >= 32 ? 0xFFFFFFFFu : (nv <= 0 ? 0u : ((1u << nv) - 1u));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const uint64_t* an = anc + node_of[rb] * kAncWords;
          uint32_t w;
          if (d >= 0) {
            const int wi = d >> 6, sh = d & 63;
            const uint64_t lo = wi < kAncWords ? an[wi] : 0ull;
            const uint64_t hi = wi + 1 < kAncWords ? an[wi + 1] : 0ull;
            w = static_cast<uint32_t>(sh == 0 ? lo : ((lo >> sh) | (hi << (64 - sh))));
          } else if (d > -32) {
            w = (static_cast<uint32_t>(an[0]) << (-d)) | ((1u << (-d)) - 1u);
          } else {
            w = 0xFFFFFFFFu;
          }
          vis[rb] = (w & endm) >> (4 * quad);
        }
      }
      u32x4 kr[2][4];
      u32x2 vA[8], vB[8];
      read_k_pair(kr[0], kr[1], lds_addr(kt + (2 * h) * kPageBytes), k_off);
      read_vt_pair(vA, vB, lds_addr(vt + (2 * h) * kPageBytes), vt_off);
      bf16x8 kf[2][4];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[pb][c] = __builtin_bit_cast(bf16x8, kr[pb][c]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][c], qf[rb][c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][c], qf[rb][c], sb, 0, 0, 0);
        }
        // lane holds S[row l16][key0 + 4*quad + i] (page A) and [key0 + 16 + 4*quad + i] (page B);
        // PV slot i <-> page A key 4*quad + i, slot 4 + i <-> page B key 4*quad + i.
        // Scores stay unscaled here; the scale enters the exponent.
        float sv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = sa[i];
          sv[4 + i] = sb[i];
        }
        if (need_mask) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = ((vis[rb] >> ((j >> 2) * 16 + (j & 3))) & 1u) ? sv[j] : -INFINITY;
        }
        const float pi = a.pinf;
        float mx = max_nn(max_nn(max_nn(sv[0], sv[1], pi), max_nn(sv[2], sv[3], pi), pi),
                          max_nn(max_nn(sv[4], sv[5], pi), max_nn(sv[6], sv[7], pi), pi), pi);
        mx = quad_max(mx);
        // The reference max m_run moves only when a row's max passes it by more
        // than lazy (kLazyLog2 in the exponent), so each p stays below
        // 2^kLazyLog2 and the accumulators are rescaled rarely: once the first
        // keys have set it, typically never again.
        if (!__all(mx <= m_run[rb] + lazy)) {
          const float m_new = max_nn(m_run[rb], mx, pi);
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run[rb] - m_new) * a.sl2);
          l_run[rb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[rb][dt] *= alpha;
          m_run[rb] = m_new;
        }
        // A row with no visible key so far (m = -inf, every score -inf) takes
        // its exponents against 0, so that each p is exp2(-inf) = 0.
        const float msl = m_run[rb] == -INFINITY ? 0.f : -m_run[rb] * a.sl2;
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], a.sl2, msl)));
        // the row sum adds the bf16 weights the PV product uses, two per v_dot2
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j += 2)
          psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[j], pf[j + 1]}, kBf16Ones, psum, false);
        l_run[rb] += psum;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{vA[dt][0], vA[dt][1], vB[dt][0], vB[dt][1]});
          o[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[rb][dt], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) l_run[rb] = quad_sum(l_run[rb]);
  report(a.status, b, err);

  const bool direct = (pc.n_parts == 1);
  if (direct) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = row_base + rb * 16 + l16;
      if (r >= a.R) continue;
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
    }
    return;
  }

  // Split partials, one 16-row block of 2048 floats per (wave, rb), in the
  // accumulator layout: element i of o[rb][dt] of lane l at (dt*4 + i)*64 + l, so
  // that each store (and each load of the merge) covers 64 consecutive floats.
  // Partials are read by another workgroup, possibly on another XCD (whose L2 is
  // not coherent with this one): they are written and read as relaxed agent-scope
  // atomics, and the arrival counter is bumped once this workgroup's stores have
  // completed -- no fence, which would write back and invalidate the whole L2.
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int blk16 = wave * NRB + rb;
    float* pb = a.part_o + (pc.pslot * RT + blk16 * 16) * kD + lane;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st_agent(pb + (dt * 4 + i) * 64, o[rb][dt][i]);
    if (quad == 0) {
      st_agent(&a.part_ml[(pc.pslot * RT + blk16 * 16 + l16) * 2 + 0], m_run[rb] * a.sl2);  // log2 units
      st_agent(&a.part_ml[(pc.pslot * RT + blk16 * 16 + l16) * 2 + 1], l_run[rb]);
    }
  }
  wait_vm0();  // this wave's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&a.counters[pc.bgr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L.s_last = (prev == static_cast<unsigned>(pc.n_parts - 1));
  }
  __syncthreads();
  if (!L.s_last) return;

  // The last workgroup of (b, g, rt) merges every piece: wave w takes the 16-row
  // blocks w, w+4, ..., each lane the elements it would hold in the accumulator
  // layout, with the loads of KS pieces in flight at a time.
  constexpr int KS = NRB <= 2 ? 2 : 4;  // splits whose loads are in flight together
  for (int blk16 = wave; blk16 < RT / 16; blk16 += 4) {
    const int r = rt * RT + blk16 * 16 + l16;
    if (rt * RT + blk16 * 16 >= a.R) break;
    float mstar = -INFINITY, lstar = 0.f, acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    for (int sp0 = 0; sp0 < pc.n_parts; sp0 += KS) {
      float ms[KS], ls[KS], x[KS][32];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        ms[k] = -INFINITY;
        ls[k] = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) x[k][e] = 0.f;
        if (sp0 + k < pc.n_parts) {
          const long it2 = part_slot(sp0 + k);
          ms[k] = ld_agent(&a.part_ml[(it2 * RT + blk16 * 16 + l16) * 2 + 0]);
          ls[k] = ld_agent(&a.part_ml[(it2 * RT + blk16 * 16 + l16) * 2 + 1]);
          const float* pb = a.part_o + (it2 * RT + blk16 * 16) * kD + lane;
#pragma unroll
          for (int e = 0; e < 32; ++e) x[k][e] = ld_agent(pb + e * 64);
        }
      }
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        if (ms[k] == -INFINITY) continue;
        const float m_new = fmaxf(mstar, ms[k]);
        const float fa = __builtin_amdgcn_exp2f(mstar - m_new);  // 0 while mstar is -inf
        const float fb = __builtin_amdgcn_exp2f(ms[k] - m_new);
        lstar = lstar * fa + ls[k] * fb;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] = acc[e] * fa + x[k][e] * fb;
        mstar = m_new;
      }
    }
    if (r < a.R) {
      const int node = r / a.G, hh = r % a.G;
      uint16_t* op = a.out + ((static_cast<long>(b) * a.T + node) * a.Hq + g * a.G + hh) * kD;
      const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t w0 = f32_to_bf16(acc[dt * 4 + 0] * inv) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[dt * 4 + 1] * inv)) << 16);
        const uint32_t w1 = f32_to_bf16(acc[dt * 4 + 2] * inv) |
                            (static_cast<uint32_t>(f32_to_bf16(acc[dt * 4 + 3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(op + dt * 16 + quad * 4) = u32x2{w0, w1};
      }
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[pc.bgr], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The stream-K split of a ragged batch (64-row tiles, one row tile per (b, g),
// B <= 64).  Every (b, g) is laid end to end in (b, g) order as kSkItemUnits +
// tiles units (tiles of 64 keys), so that the units measure time whatever the
// mix of lengths; workgroup w takes units [u0(w), u0(w + 1)).  A (b, g) cut
// between workgroups runs as pieces whose partials the last piece to arrive
// merges.  With the fused K/V write, which spreads the n_write = q G + r write
// chunks over the workgroups (about q + 1 on the first r), ranges are shorter
// by kSkWriteUnits (W) per chunk: the first r workgroups take len1 = base -
// W (q + 1) units, the others len2 = base - W q, base = ceil((U + n_write W) /
// G).  Lane b of every wave holds sequence b.
struct SkPlan {
  int lb, np, tiles, errlen, incl;  // lane b: clamped prefix length, pages, tiles, error bit, running units
  int U, r, len1, len2;             // all units; the ranges' two lengths
};

__device__ __forceinline__ SkPlan sk_plan(const TArgs2& a, int n_write) {
  const int lane = threadIdx.x & 63;
  SkPlan p;
  const bool in = lane < a.B;
  const int raw = in ? a.plen[lane] : 0;
  const int cap = a.max_blocks * kBlockSize - a.T;
  p.errlen = (in && (raw < 0 || raw > cap)) ? SPEC_DEV_LENGTH : 0;
  p.lb = raw < 0 ? 0 : (raw > cap ? cap : raw);
  p.np = in ? (p.lb + a.T + kBlockSize - 1) / kBlockSize : 0;
  p.tiles = (p.np + 3) / 4;
  int incl = in ? a.Hkv * (kSkItemUnits + p.tiles) : 0;
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) {
    const int o = __shfl_up(incl, w);
    if (lane >= w) incl += o;
  }
  p.incl = incl;
  p.U = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  const int G = static_cast<int>(gridDim.x);
  const int q = n_write / G;
  p.r = n_write % G;
  int W = kSkWriteUnits;
  int base = (p.U + n_write * W + G - 1) / G;
  if (base - W * (q + 1) < 1) {  // (tiny batches: no allowance for the write)
    W = 0;
    base = (p.U + G - 1) / G;
  }
  p.len1 = base - W * (q + 1);
  p.len2 = base - W * q;
  return p;
}

// First unit of workgroup w's range (clamped to U) and the workgroup whose range holds unit u < U.
__device__ __forceinline__ int sk_u0(const SkPlan& p, int w) {
  const int u = w <= p.r ? w * p.len1 : p.r * p.len1 + (w - p.r) * p.len2;
  return min(u, p.U);
}
__device__ __forceinline__ int sk_w_of(const SkPlan& p, int u) {
  const int k = p.r * p.len1;
  return u < k ? u / p.len1 : p.r + (u - k) / p.len2;
}

// Write item (b, chunk) of the fused launch: rows chunk*C .. chunk*C + C - 1 (C =
// chunk_rows, a multiple of 8 up to 64) of sequence b's 2 T Hkv tree rows, row
// 2 (i Hkv + g) + k being node i's key (k = 0), rotated for position Lb +
// depth(i), or value (k = 1) of kv head g, into the cache at slot Lb + i.
// Stores are agent-scope atomics (written through to memory, like the split
// partials), so items on any die that read the tree's keys see them once the
// sequence's count of written chunks is complete.  A bad parent row or prefix
// length writes nothing; a bad block index skips that slot.  Either way the
// chunk is counted.
template <int NRB>
__device__ __forceinline__ void write_item(const TArgs2& a, int b, int chunk, TileLds<NRB>& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;
  int* s_up = reinterpret_cast<int*>(L.tiles);
  int* s_dep = s_up + kMaxT;
  int* s_rng = s_dep + kMaxT;
  double2* trig = reinterpret_cast<double2*>(L.tiles + kTrigOffset);
  const int n_rows = 2 * T * a.Hkv;
  const int r0 = chunk * a.chunk_rows, r1 = min(n_rows, r0 + a.chunk_rows);
  // the chunk's rows first (they depend on nothing): half-wave h takes rows
  // r0 + h, r0 + h + 8, ..., lane l the pairs (2l, 2l + 64) and (2l + 1, 2l + 65)
  // as two 32-bit words, all in flight while the depths are found
  constexpr int kU = 8;
  const int hl = lane & 31;
  const int first = r0 + wave * 2 + (lane >> 5);
  uint32_t x0[kU], x1[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int r = min(first + 8 * u, r1 - 1);
    const int pr = r >> 1, i = pr / a.Hkv, g = pr % a.Hkv;
    const uint16_t* src = ((r & 1) ? a.v_new : a.k_new) + ((static_cast<long>(b) * T + i) * a.Hkv + g) * kD;
    x0[u] = *reinterpret_cast<const uint32_t*>(src + 2 * hl);
    x1[u] = *reinterpret_cast<const uint32_t*>(src + 64 + 2 * hl);
  }
  const int Lb = a.plen[b];
  int err = (Lb < 0 || Lb > a.max_blocks * kBlockSize - T) ? SPEC_DEV_LENGTH : 0;
  for (int i = tid; i < T; i += 256) {
    const int p = a.parent[static_cast<long>(b) * T + i];
    if (!(i == 0 ? p == -1 : (p >= 0 && p < i))) err |= SPEC_DEV_PARENT;
    L.s_par[i] = p;
  }
  const bool bad = __syncthreads_or(err != 0);  // also publishes s_par
  report(a.status, b, err);
  const bool rotate = a.rotate && !bad;
  int dmin = 0, n = 0;
  if (rotate) {
    node_depths(L.s_par, T, (r0 >> 1) / a.Hkv, ((r1 - 1) >> 1) / a.Hkv, s_up, s_dep, s_rng);
    dmin = s_rng[0];
    n = s_rng[1] - s_rng[0] + 1;
    fill_trig(trig, Lb, dmin, n, a.log2_theta);
    __syncthreads();
  }
  if (!bad) {
    const int32_t* bt_b = a.bt + static_cast<long>(b) * a.max_blocks;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = first + 8 * u;
      if (r >= r1) break;
      const int pr = r >> 1, i = pr / a.Hkv, g = pr % a.Hkv;
      const int t = Lb + i;
      const int blk = bt_b[t / kBlockSize];
      if (blk < 0 || blk >= a.num_blocks) {
        if (hl == 0) report(a.status, b, SPEC_DEV_BLOCK);
        continue;
      }
      uint16_t* dst = ((r & 1) ? a.vc : a.kc) + ((static_cast<long>(blk) * a.Hkv + g) * kBlockSize + t % kBlockSize) * kD;
      uint32_t y0 = x0[u], y1 = x1[u];
      if (rotate && !(r & 1)) {
        const int d = s_dep[i];
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          double cs, sn;
          trig_of(trig, Lb, dmin, n, d, 2 * hl + h, a.log2_theta, &cs, &sn);
          float r_0, r_1;
          rope_turn(bf16_to_f32(static_cast<uint16_t>(x0[u] >> (16 * h))),
                    bf16_to_f32(static_cast<uint16_t>(x1[u] >> (16 * h))), cs, sn, &r_0, &r_1);
          lo |= static_cast<uint32_t>(f32_to_bf16(r_0)) << (16 * h);
          hi |= static_cast<uint32_t>(f32_to_bf16(r_1)) << (16 * h);
        }
        y0 = lo;
        y1 = hi;
      }
      st_agent_u32(dst + 2 * hl, y0);
      st_agent_u32(dst + 64 + 2 * hl, y1);
    }
  }
  wait_vm0();  // this wave's stores have completed
  __syncthreads();
  if (tid == 0) __hip_atomic_fetch_add(&a.flags[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kFused: the launch also writes the tree's K/V rows (stream-K split, 64-row
// tiles only).
template <int NRB, bool kFused>
__global__ __launch_bounds__(256, NRB <= 2 ? 2 : 1) void attn_tile_kernel(const TArgs2 a) {
  __shared__ TileLds<NRB> L;
  const int tid = threadIdx.x;
  static_assert(!kFused || NRB == 1, "the fused launch runs 64-row tiles");
  if constexpr (NRB == 1) {
    if (kFused || a.streamk) {
      // The stream-K split (see SkPlan): write chunks w, w + G, ... first, then
      // the pieces of this workgroup's range of units, in (b, g) order.  Each
      // chunk is claimed before it is written (a claim word a chunk), and a
      // piece holding tree keys that finds its sequence's rows unwritten takes
      // over the chunks nobody has claimed before it waits for the rest (see
      // tile_item_run), so every wait ends whatever else the device holds.
      const int n_write = kFused ? a.n_write : 0;
      const SkPlan p = sk_plan(a, n_write);
      const int G = static_cast<int>(gridDim.x), w = static_cast<int>(blockIdx.x);
      if constexpr (kFused) {
        unsigned* claim = a.flags + a.B;
        for (int j = w; j < n_write; j += G) {
          if (tid == 0)
            L.s_next = __hip_atomic_exchange(claim + j, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u ? 1 : 0;
          __syncthreads();
          const bool mine = L.s_next != 0;
          __syncthreads();  // every wave has read s_next before it is rewritten
          if (mine) {
            write_item<NRB>(a, j / a.n_chunks, j % a.n_chunks, L);
            __syncthreads();  // the chunk's LDS is free again
          }
        }
      }
      // The range is taken from its end: its last piece is the head of a (b, g)
      // (no tree keys) and its first the end of one (tree keys), so pieces that
      // need the tree's rows come late, when the chunks are long written.
      const int lane = tid & 63;
      const int u_begin = sk_u0(p, w);
      int u = sk_u0(p, w + 1);  // units [u_begin, u) are still to do
      while (u > u_begin) {
        // the (b, g) holding unit u - 1: sequence b from the running sums, then its kv head
        const int b =
            __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(__ballot(lane < a.B && p.incl > u - 1))) - 1);
        const int incl_b = __builtin_amdgcn_readlane(p.incl, b);
        const int tiles_b = __builtin_amdgcn_readlane(p.tiles, b);
        const int per = kSkItemUnits + tiles_b;
        const int start_b = incl_b - a.Hkv * per;
        const int g = (u - 1 - start_b) / per;
        const int s_bg = start_b + g * per;
        const int f = s_bg + kSkItemUnits, e = f + tiles_b;  // the (b, g)'s tile units
        const int t0 = max(u_begin, f) - f, t1 = min(u, e) - f;
        if (t1 > t0) {
          Piece pc;
          pc.b = b;
          pc.g = g;
          pc.rt = 0;
          pc.p0 = 4 * t0;
          pc.p1 = min(__builtin_amdgcn_readlane(p.np, b), 4 * t1);
          const int w_first = sk_w_of(p, f);
          pc.n_parts = sk_w_of(p, e - 1) - w_first + 1;
          // two partial slots a workgroup: its first piece, its last one (the pieces between are whole (b, g))
          pc.pslot = 2L * w + (sk_u0(p, w) >= s_bg ? 0 : 1);
          pc.bgr = static_cast<long>(b) * a.Hkv + g;
          tile_item_run<NRB, kFused>(a, pc, __builtin_amdgcn_readlane(p.lb, b), __builtin_amdgcn_readlane(p.errlen, b), L,
                                     [&](int k) {
                                       const int ww = w_first + k;
                                       return 2L * ww + (sk_u0(p, ww) >= s_bg ? 0 : 1);
                                     });
          __syncthreads();  // every wave is done with the piece's LDS
        }
        u = s_bg;
      }
      // the last workgroup to leave resets the write flags and claims for the next call
      unsigned* done = a.counters + static_cast<long>(a.B) * a.Hkv * a.n_rt + 1;
      if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        L.s_last = (prev == static_cast<unsigned>(G - 1));
      }
      __syncthreads();
      if (L.s_last) {
        if constexpr (kFused)
          for (int i = tid; i < a.B + n_write; i += 256)  // flags, then claim words
            __hip_atomic_store(&a.flags[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
  }
  // One item (b, g, KV split, row tile) a workgroup.  Consecutive workgroup ids
  // are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of items
  // so the row tiles of one KV chunk share an L2.
  const long per = (a.items + 7) / 8;
  const long item = static_cast<long>(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (item >= a.items) return;
  const int rt = static_cast<int>(item % a.n_rt);
  long rest = item / a.n_rt;
  const int s = static_cast<int>(rest % a.splits);
  rest /= a.splits;
  const int g = static_cast<int>(rest % a.Hkv);
  const int b = static_cast<int>(rest / a.Hkv);
  int Lb = a.plen[b], err = 0;
  const int cap = a.max_blocks * kBlockSize - a.T;
  if (Lb < 0 || Lb > cap) {
    err |= SPEC_DEV_LENGTH;
    Lb = Lb < 0 ? 0 : cap;
  }
  const int npages = (Lb + a.T + kBlockSize - 1) / kBlockSize;
  const long first = (static_cast<long>(b) * a.Hkv + g) * a.splits * a.n_rt + rt;  // item of split 0
  int n_used = (npages + a.pps - 1) / a.pps;  // splits of this (b, g) that hold keys
  int p0 = s * a.pps, p1 = min(npages, p0 + a.pps);
  if (a.n_first > 0 && npages >= 16 * a.splits) {
    // The grid is two rounds of one workgroup a CU.  A CU's first workgroup
    // runs ahead of the one dispatched onto it second (its older waves win the
    // SIMD arbiter), so the splits of first-round workgroups get kWFirst/8 the
    // pages of the others.  Integer weights, so every workgroup of the
    // (b, g, rt) finds the same boundaries, rounded down to whole 64-key tiles
    // (a partial tile costs a whole one); each split spans at least
    // npages / (2 splits) >= 8 pages before rounding, so none is empty.
    // When all of them fall in one round the equal splits stay.
    long before = 0, total = 0, mine = 0;
    int n_early = 0;
    for (int k = 0; k < a.splits; ++k) {
      const long it = first + static_cast<long>(k) * a.n_rt;
      const long wg = (it % per) * 8 + it / per;  // the workgroup that runs item it
      const long w = wg < a.n_first ? kWFirst : 8;
      n_early += wg < a.n_first ? 1 : 0;
      if (k < s) before += w;
      if (k == s) mine = w;
      total += w;
    }
    if (n_early > 0 && n_early < a.splits) {
      p0 = static_cast<int>(npages * before / total) & ~3;
      p1 = s == a.splits - 1 ? npages : static_cast<int>(npages * (before + mine) / total) & ~3;
      n_used = a.splits;
    }
  }
  if (s >= n_used) return;
  Piece pc;
  pc.b = b;
  pc.g = g;
  pc.rt = rt;
  pc.p0 = p0;
  pc.p1 = p1;
  pc.n_parts = n_used;
  pc.pslot = item;
  pc.bgr = (static_cast<long>(b) * a.Hkv + g) * a.n_rt + rt;
  tile_item_run<NRB, kFused>(a, pc, Lb, err, L, [&](int k) { return first + static_cast<long>(k) * a.n_rt; });
}

// Workgroups of attn_tile_kernel<NRB, kFused> the current device holds at once
// (occupancy per CU times the CU count), queried once per device.
template <int NRB, bool kFused>
long tile_capacity() {
  static long cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_tile_kernel<NRB, kFused>, 256, 0) != hipSuccess)
    return 0;
  const long cap = static_cast<long>(cus) * per_cu;
  if (dev < 64) cache[dev] = cap;
  return cap;
}

template <int NRB>
hipError_t run_tile(const TArgs2& args_in, hipStream_t stream) {
  TArgs2 args = args_in;
  const long grid = ((args.items + 7) / 8) * 8;
  // Weighted splits (see the kernel) when the grid is two rounds of one
  // workgroup a CU and the longest weighted split still fits the block-index
  // buffer (a weighted split holds at most kWFirst/8 of pps pages).
  int dev = 0, cus = 0;
  const long cap = tile_capacity<NRB, false>();
  const long max_pages = sizeof(TileLds<NRB>::s_blk) / sizeof(int);
  args.n_first = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                                              hipSuccess &&
      cap == 2L * cus && grid > cus && grid <= cap && static_cast<long>(args.pps) * kWFirst <= 8 * max_pages) {
    // only where some (b, g, rt) has splits in both rounds (the kernel's own test)
    const long per = (args.items + 7) / 8, n_bgr = static_cast<long>(args.B) * args.Hkv * args.n_rt;
    bool mixed = false;
    for (long bgr = 0; bgr < n_bgr && !mixed; ++bgr) {
      const long first = (bgr / args.n_rt) * args.splits * args.n_rt + bgr % args.n_rt;
      int n_early = 0;
      for (int k = 0; k < args.splits; ++k) {
        const long it = first + static_cast<long>(k) * args.n_rt;
        n_early += (it % per) * 8 + it / per < cus ? 1 : 0;
      }
      mixed = n_early > 0 && n_early < args.splits;
    }
    if (mixed) args.n_first = cus;
  }
  hipLaunchKernelGGL((attn_tile_kernel<NRB, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

#ifndef SPEC_TILE_RAGGED_PPS
#define SPEC_TILE_RAGGED_PPS 256
#endif
// Tile-kernel shape of p.rows query rows per (sequence, kv head): 64-row tiles
// up to 64 rows, else 128-row tiles; two workgroups per CU.
static void plan_tile(AttnPlan& p, int B, int Hkv, int max_blocks) {
  p.mode = 2;
  p.nrb = p.rows <= 64 ? 1 : 2;
  p.rt = 64 * p.nrb;
  p.n_rt = (p.rows + p.rt - 1) / p.rt;
  const long base = static_cast<long>(B) * Hkv * p.n_rt;
  // ~two workgroups per CU; at least 16 pages (256 keys) per split
  long splits = std::max<long>(1, (512 + base - 1) / base);
  // long sequences of a ragged batch: at most 512 pages per split, so the
  // longest ones do not set the makespan alone
  splits = std::max<long>(splits, (max_blocks + 511) / 512);
  splits = std::min<long>(splits, std::max<long>(1, max_blocks / 16));
  // a ragged batch with more items than resident workgroups (512: two per CU)
  // takes the stream-K split, whose partials need two slots a resident
  // workgroup: at least 1024 items' worth of workspace; its splits are then only
  // the fallback's (no occupancy figure), cut so that no item sets the makespan alone
  p.streamk = (p.nrb == 1 && p.n_rt == 1 && B <= 64 && base * splits > 512 && max_blocks <= kMaxPiecePages) ? 1 : 0;
  if (p.streamk) {
    splits = std::max<long>(splits, (max_blocks + SPEC_TILE_RAGGED_PPS - 1) / SPEC_TILE_RAGGED_PPS);
    splits = std::max<long>(splits, (1024 + base - 1) / base);
  }
  long pps = (max_blocks + splits - 1) / splits;
  pps = (pps + 3) / 4 * 4;
  pps = std::min<long>(pps, kMaxSplitPages);
  splits = (max_blocks + pps - 1) / pps;
  p.pps = static_cast<int>(pps);
  p.splits = static_cast<int>(splits);
  p.items = base * p.splits;
}

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
  if (p.rows <= 16) {  // chains, decode, small trees: the streaming kernel
    plan_stream(p, B, Hkv, max_blocks);
    return p;
  }
  plan_tile(p, B, Hkv, max_blocks);
  const size_t head = (static_cast<size_t>(p.items / p.splits + 2) * sizeof(unsigned) + 255) / 256 * 256;  // + the exit counter
  p.ws_bytes = p.splits > 1 ? head + static_cast<size_t>(p.items) * p.rt * (kD + 2) * sizeof(float) : 0;
  return p;
}

// The tree's K/V write and the attention: one launch of the tile kernel where
// its work is cut stream-K fashion (64-row tiles over a ragged batch with more
// items than resident workgroups), the write chunks spread over the
// workgroups; there the workspace holds arrival counters, [unused, workgroups
// done], one count of written chunks per sequence, one claim word per chunk,
// then the partials.  Any other shape takes two launches, which measured faster
// there: the write (rotated queries into the workspace), then the attention of
// spec_tree_attn.
constexpr int kWriteChunkRows = 64;  // rows of a write chunk: few workgroups carry the write's latency
static size_t fused_head_bytes(int B, int T, int Hkv, size_t arrivals) {
  const size_t chunks = static_cast<size_t>(B) * ((2 * T * Hkv + kWriteChunkRows - 1) / kWriteChunkRows);
  return ((arrivals + 2 + static_cast<size_t>(B) + chunks) * sizeof(unsigned) + 255) / 256 * 256;
}

AttnPlan plan_attn_write(int B, int T, int Hq, int Hkv, int max_blocks) {
  AttnPlan p = plan_attn(B, T, Hq, Hkv, kD, max_blocks, SPEC_BF16);
  if (p.mode == 2 && p.nrb == 1 && p.streamk && p.splits > 1) {
    p.fused = 1;
    const size_t head = fused_head_bytes(B, T, Hkv, static_cast<size_t>(p.items / p.splits));
    p.ws_bytes = head + static_cast<size_t>(p.items) * p.rt * (kD + 2) * sizeof(float);
    return p;
  }
  if (p.mode == 3 && T <= 16) {  // the streaming kernel writes and rotates in its own launch
    p.fused = 1;
    return p;
  }
  p.ws_bytes += (static_cast<size_t>(B) * T * Hq * kD * sizeof(uint16_t) + 255) / 256 * 256;
  return p;
}

static TArgs2 tile_args(const AttnPlan& plan, const AttnLaunch& L) {
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
  // With one row tile per (b, g) each K/V page is read by one item; with several,
  // the row tiles of a KV chunk find it in L2 (streaming loads made the 16-tile
  // Sequoia-scale layer slower), so only the former load non-temporally.
  a.kv_stream = plan.n_rt == 1;
  a.sl2 = L.scale * kLog2e;
  a.pinf = INFINITY;
  return a;
}

hipError_t launch_attn_bf16(const AttnPlan& plan, const AttnLaunch& L, hipStream_t stream) {
  if (plan.mode == 3) return launch_attn_stream(plan, L, stream);
  TArgs2 a = tile_args(plan, L);
  if (plan.splits > 1) {
    const size_t base = static_cast<size_t>(L.B) * L.Hkv * plan.n_rt;
    const size_t head = (static_cast<size_t>(base + 2) * sizeof(unsigned) + 255) / 256 * 256;
    a.counters = static_cast<unsigned*>(L.workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + head);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rt * kD;
  }
  if (plan.nrb == 1) {
    if (plan.streamk && plan.splits > 1) {  // the stream-K split over one round of resident workgroups
      const long cap = tile_capacity<1, false>();
      if (cap > 0) {
        a.streamk = 1;
        const long grid = std::min<long>(cap, plan.items / 2);  // two partial slots a workgroup
        hipLaunchKernelGGL((attn_tile_kernel<1, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
        return hipGetLastError();
      }
    }
    return run_tile<1>(a, stream);
  }
  return run_tile<2>(a, stream);
}

hipError_t launch_attn_write(const AttnPlan& plan, const AttnWriteLaunch& W, hipStream_t stream) {
  const AttnLaunch& L = W.attn;
  char* ws = static_cast<char*>(L.workspace);
  if (plan.fused && plan.mode == 3) return launch_attn_stream_write(plan, W, stream);
  if (!plan.fused) {  // two launches: the write (queries rotated into the workspace), the attention
    const size_t qbytes = (static_cast<size_t>(L.B) * L.T * L.Hq * kD * sizeof(uint16_t) + 255) / 256 * 256;
    KvWriteLaunch K{};
    K.k_new = W.k_new;
    K.v_new = W.v_new;
    K.q = L.q;
    K.q_out = ws;
    K.k_cache = const_cast<void*>(L.k);
    K.v_cache = const_cast<void*>(L.v);
    K.block_table = L.block_table;
    K.prefix_lens = L.prefix_lens;
    K.parent = L.parent;
    K.status = L.status;
    K.B = L.B;
    K.T = L.T;
    K.Hq = L.Hq;
    K.Hkv = L.Hkv;
    K.D = L.D;
    K.max_blocks = L.max_blocks;
    K.num_blocks = L.num_blocks;
    K.bf16 = 1;
    K.theta = W.theta;
    const hipError_t e = launch_kv_write(K, stream);
    if (e != hipSuccess) return e;
    AttnLaunch L2 = L;
    L2.q = ws;
    L2.workspace = ws + qbytes;
    return launch_attn_bf16(plan, L2, stream);
  }
  TArgs2 a = tile_args(plan, L);
  const size_t base = static_cast<size_t>(L.B) * L.Hkv * plan.n_rt;
  const size_t head = fused_head_bytes(L.B, L.T, L.Hkv, base);
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.flags = a.counters + base + 2;
  if (plan.splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws + head);
    a.part_ml = a.part_o + static_cast<size_t>(plan.items) * plan.rt * kD;
  }
  a.k_new = static_cast<const uint16_t*>(W.k_new);
  a.v_new = static_cast<const uint16_t*>(W.v_new);
  a.kc = static_cast<uint16_t*>(const_cast<void*>(L.k));
  a.vc = static_cast<uint16_t*>(const_cast<void*>(L.v));
  a.rotate = W.theta > 0.0f ? 1 : 0;
  a.log2_theta = W.theta > 0.0f ? std::log2(static_cast<double>(W.theta)) : 0.0;
  a.streamk = 1;
  const long cap = tile_capacity<1, true>();
  if (cap <= 0) return hipErrorInvalidDevice;
  // chunks of the write: 64 rows, so that few workgroups carry the write's
  // latency (smaller chunks on every workgroup measured slower)
  a.chunk_rows = kWriteChunkRows;
  a.n_chunks = (2 * L.T * L.Hkv + a.chunk_rows - 1) / a.chunk_rows;
  a.n_write = L.B * a.n_chunks;
  // one round of resident workgroups, two partial slots each
  const long grid = std::min<long>(cap, plan.items / 2);
  hipLaunchKernelGGL((attn_tile_kernel<1, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace spectree
