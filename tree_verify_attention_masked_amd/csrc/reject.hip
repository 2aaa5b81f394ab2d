// Tree rejection sampling on the GPU.
//
// The rule ("Speculative Decoding" notes, "Draft Token Validation"): a drafted
// token x is accepted iff r * q(x) < p(x) for a uniform r in [0, 1); after a
// rejection the target becomes the residual max(0, p - q) renormalised, and a
// node whose children are all rejected (or a leaf) ends with one draw from the
// current target.  Siblings are tried in turn; the Sequoia variant ("Sequoia:
// Scalable and Robust Speculative Decoding" summary, "Robust Sampling") also
// removes each rejected token from q and renormalises q.
//
// One kernel.  Each sequence is walked by a TEAM of NW workgroups; member w
// owns the contiguous vocabulary slice [w*S, (w+1)*S) and keeps the slices of
// the rows it works on in LDS.  Every member replays the same walk (same
// inputs, same Philox draws, merges done by one wave in a fixed order, so the
// same decisions); vocabulary-wide quantities are merged from the members'
// slice partials, exchanged through the workspace at a team barrier:
//   * row statistics of node u: max logit, first argmax, sum exp((l-max)/t)
//     in fp64 -- rows 0..E-1 before the walk, deeper rows when reached;
//   * the residual after j rejections, kept in closed form
//         p~_j(x) = max(p(x) - C_j(x) q(x), 0) / N_j,
//     one coefficient C_j for every token still in q and a frozen coefficient
//     per token removed from q (without replacement), q~_j = s_j q on the
//     tokens still in q.  Each rejection is one pass over the slice that
//     publishes the slice mass of the new residual, scanned over per-thread
//     contiguous segments in index order;
//   * the final draw: after a rejection the last pass already holds the
//     scanned weights; for a bonus draw the slice masses of p follow from the
//     row statistics.  The member whose range holds u * total finds the token
//     inside its slice.
// Members exchange records through tagged slots (one per exchange and member,
// written once per call): a reader polls the slots themselves until every one
// carries this call's tag, with a bounded wait.
// Decisions are taken in fp64 from the fp32 inputs.  Uniforms: Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, SC'11), key (seed lo, seed hi), counter (node,
// b, purpose + 2*(offset >> 32), offset lo); u = (word0 >> 8) * 2^-24.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "compact_dev.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxEager = 8;     // rows whose statistics are taken before the walk
constexpr int kMaxTeam = 64;     // workgroups per sequence (one wave merges their partials)
constexpr int kDeepTeam = 32;    // at most this many for trees with deeper rows (more than 16 nodes)
constexpr int kEagerCap = 8192;  // floats of eager-row logit slices kept in LDS
constexpr int kSmallTree = 256;  // trees up to this many nodes: the kernel with the larger eager space
constexpr int kEagerCapBig = 7680;  // eager-slice floats beside the node arrays of a larger tree
constexpr int kSliceCap = 8192;  // floats of the current row's logits / draft probs kept in LDS
constexpr int kHeaderBytes = 256;  // workspace header: word 0 exit counter of the grid, word 1 call epoch
constexpr unsigned kSpinLimit = 1u << 24;
constexpr long kUnboundedResidency = 1L << 40;

struct Rec {
  float m;   // slice max logit (-inf if none)
  int idx;   // first index of the max; -1 if the slice holds NaN or +inf
  double z;  // sum over the slice of exp((l - m) / t), or a slice mass
};

struct Slot {
  unsigned long long w[4];  // (tag << 32) | 32 bits of a Rec: m, idx, z high, z low
};

struct Team {
  int NW, S, ld, E;  // members, slice length, LDS row stride (S rounded up to 4), eager rows (0 to 8)
};

// Team size: up to 64 members (32 for trees of more than 16 nodes), about 256
// workgroups in all, at least 512 vocabulary entries per member, and never more
// workgroups than the device can hold at once (`resident`): members of a team
// wait for each other, so a team larger than one member needs the whole grid
// resident; when even two members per sequence do not fit, each sequence gets
// a single member, which waits for nobody.
Team team_shape(int B, int T, int V, long resident) {
  Team t;
  int nw = std::max(1, std::min(T > 16 ? kDeepTeam : kMaxTeam, 256 / std::max(B, 1)));
  nw = std::min(nw, std::max(1, (V + 511) / 512));
  if (static_cast<long>(nw) * B > resident) {
    nw = static_cast<int>(std::max(1L, std::min<long>(nw, resident / std::max(B, 1))));
    if (nw < 2) nw = 1;
  }
  t.NW = nw;
  t.S = (V + nw - 1) / nw;
  t.ld = (t.S + 3) & ~3;
  int e = std::min(T, kMaxEager);
  const int cap = T <= kSmallTree ? kEagerCap : kEagerCapBig;
  e = t.ld > cap ? 0 : std::min(e, cap / t.ld);  // >= 1 when the slice fits a tree of up to kSmallTree nodes
  // 5 to 7 rows cost each wave a second row scan; they pay only where the eager
  // space is what limits the count (trees of more than kSmallTree nodes)
  t.E = T > kSmallTree ? e : (e >= 8 ? 8 : e >= 4 ? 4 : e >= 2 ? 2 : e);
  return t;
}

// ---------------------------------------------------------------------------
// Philox4x32-10: ten rounds of the multiply/xor bijection, key bumped by the
// Weyl increments between rounds.  Only output word 0 is used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox4x32_10_w0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                     uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ double draw_uniform(uint64_t seed, uint64_t offset, int b, int node, int purpose) {
  const uint32_t w = philox4x32_10_w0(static_cast<uint32_t>(node), static_cast<uint32_t>(b),
                                      static_cast<uint32_t>(purpose) + 2u * static_cast<uint32_t>(offset >> 32),
                                      static_cast<uint32_t>(offset), static_cast<uint32_t>(seed),
                                      static_cast<uint32_t>(seed >> 32));
  return static_cast<double>(w >> 8) * (1.0 / 16777216.0);
}

__device__ __forceinline__ bool bad_logit(float v) { return isnan(v) || v == INFINITY; }

// e^x for N arguments at once, meant for x <= 0 (softmax terms); arguments are
// clamped to [-746, 709], so -inf and NaN give a finite value the caller masks.
// Cody-Waite reduction x = n ln2 + r, |r| <= ln2/2, with ln2 split into a part
// of 24 significant bits (n * hi exact) and the rest; e^r by its Taylor
// polynomial to degree 13 (truncation below 5e-18), evaluated by Horner's rule
// for all N arguments in lockstep so their dependency chains overlap; scaled by 2^n.
template <int N>
__device__ __forceinline__ void exp_lockstep(double (&x)[N]) {
  constexpr double kLog2e = 1.4426950408889634074;
  constexpr double kLn2Hi = 0.693145751953125;          // ln 2 rounded to 24 bits
  constexpr double kLn2Lo = 1.4286068203094172321e-06;  // ln 2 - kLn2Hi
  constexpr double kF[14] = {1.0,
                             1.0,
                             1.0 / 2,
                             1.0 / 6,
                             1.0 / 24,
                             1.0 / 120,
                             1.0 / 720,
                             1.0 / 5040,
                             1.0 / 40320,
                             1.0 / 362880,
                             1.0 / 3628800,
                             1.0 / 39916800,
                             1.0 / 479001600,
                             1.0 / 6227020800.0};
  double r[N], p[N];
  int k[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const double xv = fmin(fmax(x[j], -746.0), 709.0);
    const double kd = rint(xv * kLog2e);
    r[j] = fma(-kd, kLn2Lo, fma(-kd, kLn2Hi, xv));
    k[j] = static_cast<int>(kd);
    p[j] = kF[13];
  }
#pragma unroll
  for (int d = 12; d >= 0; --d)
#pragma unroll
    for (int j = 0; j < N; ++j) p[j] = fma(p[j], r[j], kF[d]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = ldexp(p[j], k[j]);
}

__device__ __forceinline__ double exp1(double x) {
  double v[1] = {x};
  exp_lockstep<1>(v);
  return v[0];
}

struct TArgs {
  const float* logits;
  const float* q;
  const int32_t* tokens;
  const int32_t* parent;
  int32_t* accepted;
  int32_t* out_tokens;
  int32_t* num_accepted;
  int32_t* status;
  unsigned* hdr;   // workspace header: [0] exit counter of the grid, [1] call epoch
  unsigned long long* slot_words;  // every 64-bit word of the workspace after the header
  long n_slot_words;               // (cleared when the epoch wraps)
  Slot* eager;     // [B][NW][max(E,1)]: statistics of the eager rows
  Slot* part;      // [B][part_rows][NW]: one row of slots per later exchange
  int part_rows;
  int T, V, NW, S, ld, E, greedy, wr;
  double inv_tau;
  uint64_t seed, offset;
  int fuse;         // compact the KV cache along the accepted path after the walk
  CompactLaunch c;  // its arguments (accepted / num_accepted unused: the path is in LDS)
  // truncation of the visited target rows (trunc != 0: top_k in 1 .. kTopKMax)
  int trunc, top_k;     // K
  int kc_e, q_e;        // eager rows: first-list length (<= K), parts a member's slice is cut into
  int kc_d, q_d;        // later rows: the same
  double top_p;         // >= 1: top-k only
  unsigned long long* lists;  // [B][list_blocks][top_k + 2] tagged words: the lists of each row (see the kernel)
  int list_blocks;
};

// Records cross workgroups (the team spans XCDs, whose L2s are not coherent
// with each other) through slots written once per call.  Each of a slot's four
// 64-bit words carries the call's tag in its high half and 32 bits of the
// record in its low half, and is written and read as one relaxed agent-scope
// atomic (write-through store, coherent load; naturally aligned 64-bit
// accesses are single-copy atomic).  A reader that finds the tag in all four
// words therefore holds the whole record: no arrival counter, no wait for the
// writer's stores to complete, no fence (which would write back and invalidate
// the whole L2), and no second round trip to read the record after a barrier.
// Tags are never 0, so a zero-filled workspace holds no valid slot.
__device__ __forceinline__ void put_slot(Slot* p, const Rec& r, uint32_t tag) {
  const unsigned long long t = static_cast<unsigned long long>(tag) << 32;
  const unsigned long long zb = static_cast<unsigned long long>(__double_as_longlong(r.z));
  __hip_atomic_store(&p->w[0], t | __float_as_uint(r.m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->w[1], t | static_cast<uint32_t>(r.idx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->w[2], t | (zb >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->w[3], t | (zb & 0xFFFFFFFFull), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave, every lane active: lane w < NW waits until slot base[h][w * stride]
// of each of the NR rows h carries `tag`, and returns member w's records
// (lanes >= NW get `dflt`).  The wait is bounded: past kSpinLimit polls lane 0
// sets *fail and the records are not to be used.
template <int NR>
__device__ __forceinline__ void get_slots(const Slot* const (&base)[NR], int stride, int NW, uint32_t tag,
                                          const Rec& dflt, Rec (&out)[NR], int* fail) {
  const int lane = threadIdx.x & 63;
  unsigned long long w[NR][4];
  bool ok = lane >= NW;
  unsigned spins = 0;
  for (;;) {
    if (!ok) {
#pragma unroll
      for (int h = 0; h < NR; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[h][k] = __hip_atomic_load(const_cast<unsigned long long*>(&base[h][lane * stride].w[k]), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      ok = true;
#pragma unroll
      for (int h = 0; h < NR; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) ok = ok && static_cast<uint32_t>(w[h][k] >> 32) == tag;
    }
    if (__all(ok)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) *fail = 1;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    if (lane < NW) {
      out[h].m = __uint_as_float(static_cast<uint32_t>(w[h][0]));
      out[h].idx = static_cast<int>(static_cast<uint32_t>(w[h][1]));
      out[h].z = __longlong_as_double(static_cast<long long>(((w[h][2] & 0xFFFFFFFFull) << 32) |
                                                             (w[h][3] & 0xFFFFFFFFull)));
    } else {
      out[h] = dflt;
    }
  }
}

// Starts copying rows [r * src_stride + i], r < nrows, i < n, of global memory
// into LDS dst[r * ld + i] (ld a multiple of 4) with direct global->LDS loads:
// lane i of an instruction writes LDS word(s) i of the instruction's base, so
// the copy needs no registers.  When the rows are 16-byte aligned one
// instruction moves 256 consecutive floats (16 bytes a lane) and the last n % 4
// elements of a row go 4 bytes a lane; otherwise every instruction moves 64
// floats.  Instructions are dealt to the waves round-robin by a running count
// (no division in the issue loop).  The data may be read after this wave's
// vector-memory counter has drained and a workgroup barrier.
__device__ __forceinline__ void stage_dma(float* dst, const float* src, int ld, long src_stride, int nrows, int n) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && ((src_stride & 3) == 0);
  int j = 0;
  if (vec) {
    const int n4 = n & ~3;
    const int per_row = (n4 + 255) >> 8;
    for (int r = 0; r < nrows; ++r)
      for (int c = 0; c < per_row; ++c, ++j)
        if ((j & (kWaves - 1)) == wave) {
          const int i = c * 256 + lane * 4;
          if (i < n4) __builtin_amdgcn_global_load_lds(src + r * src_stride + i, dst + r * ld + c * 256, 16, 0, 0);
        }
    if (n4 < n)
      for (int r = 0; r < nrows; ++r, ++j)
        if ((j & (kWaves - 1)) == wave && lane < n - n4)
          __builtin_amdgcn_global_load_lds(src + r * src_stride + n4 + lane, dst + r * ld + n4, 4, 0, 0);
  } else {
    const int per_row = (n + 63) >> 6;
    for (int r = 0; r < nrows; ++r)
      for (int c = 0; c < per_row; ++c, ++j)
        if ((j & (kWaves - 1)) == wave) {
          const int i = c * 64 + lane;
          if (i < n) __builtin_amdgcn_global_load_lds(src + r * src_stride + i, dst + r * ld + c * 64, 4, 0, 0);
        }
  }
}

__device__ __forceinline__ void wait_dma() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Four consecutive slice elements at p (16-byte aligned in LDS); from global
// memory only the first `valid` are read.
template <bool kLds>
__device__ __forceinline__ f32x4 load4(const float* p, int valid) {
  if constexpr (kLds) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid) v[e] = p[e];
    return v;
  }
}

// Cross-lane steps through DPP (a few cycles each, instead of an LDS round trip
// per shuffle).  A wave-wide inclusive scan is row_shr 1, 2, 4, 8 within each
// row of 16 lanes, then row_bcast:15 into rows 1 and 3 and row_bcast:31 into
// rows 2 and 3; lanes without a source keep `old` (the operation's identity).
// Every lane of the wave must be active.
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143, kWaveShr1 = 0x138;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL, ROWS>(__builtin_bit_cast(int, old), __builtin_bit_cast(int, x)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double old, double x) {
  const long long o = __builtin_bit_cast(long long, old), v = __builtin_bit_cast(long long, x);
  const int lo = dpp_i<CTRL, ROWS>(static_cast<int>(o), static_cast<int>(v));
  const int hi = dpp_i<CTRL, ROWS>(static_cast<int>(o >> 32), static_cast<int>(v >> 32));
  return __builtin_bit_cast(double, (static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
__device__ __forceinline__ float lane63_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const long long v = __builtin_bit_cast(long long, x);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), l);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), l);
  return __builtin_bit_cast(double, (static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// (max, lowest index of the max) combined with the value DPP brings in.
template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(float& m, int& i) {
  const float om = dpp_f<CTRL, ROWS>(-INFINITY, m);
  const int oi = dpp_i<CTRL, ROWS>(0x7fffffff, i);
  const bool take = om > m || (om == m && oi < i);  // selects, not branches
  m = take ? om : m;
  i = take ? oi : i;
}

// Max with the lowest index on ties over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  argmax_step<kShr1, 0xF>(m, i);
  argmax_step<kShr2, 0xF>(m, i);
  argmax_step<kShr4, 0xF>(m, i);
  argmax_step<kShr8, 0xF>(m, i);
  argmax_step<kBcast15, 0xA>(m, i);
  argmax_step<kBcast31, 0xC>(m, i);
  m = lane63_f(m);
  i = __builtin_amdgcn_readlane(i, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_d<kShr1, 0xF>(0.0, v);
  v += dpp_d<kShr2, 0xF>(0.0, v);
  v += dpp_d<kShr4, 0xF>(0.0, v);
  v += dpp_d<kShr8, 0xF>(0.0, v);
  v += dpp_d<kBcast15, 0xA>(0.0, v);
  v += dpp_d<kBcast31, 0xC>(0.0, v);
  return v;
}

// The previous lane's value (lane 0: `first`).
__device__ __forceinline__ double wave_shift_up(double v, double first) { return dpp_d<kWaveShr1, 0xF>(first, v); }

// Running (max, first argmax, sum of exp((l - max) / t) relative to the running
// max) of NR rows, row r at base[r * stride + i], over the 4-element chunks
// c0, c0 + step, ... (< nc) of a slice of n elements (global index v0 + i).
// Consecutive lanes take consecutive chunks, so each LDS read instruction
// covers one contiguous run (no bank conflicts); chunks are visited in
// increasing order, so the index kept is the first of the lane's max.  A NaN or
// +inf pins the row's max at +inf with index -1.
template <int NR, bool kLds>
__device__ __forceinline__ void scan_chunks(const float* base, int stride, int n, int v0, double inv_tau, int c0, int nc,
                                            int step, bool noz, float (&mx)[NR], int (&ix)[NR], double (&z)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mx[r] = -INFINITY;
    ix[r] = 0x7fffffff;
    z[r] = 0.0;
  }
  for (int c = c0; c < nc; c += step) {
    f32x4 v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = load4<kLds>(base + r * stride + 4 * c, n - 4 * c);
    float cm[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      cm[r] = mx[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // a NaN or +inf pins the row's max at +inf with index -1
        const bool in = 4 * c + e < n;
        const float x = v[r][e];
        const bool bad = in && bad_logit(x);
        const bool take = (in && x > cm[r]) || bad;
        cm[r] = take ? (bad ? INFINITY : x) : cm[r];
        ix[r] = take ? (bad ? -1 : v0 + 4 * c + e) : ix[r];
      }
    }
    if (!noz) {
      double t[5 * NR];  // the chunk's terms, then the factor rescaling the running sum
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[4 * r + e] = (static_cast<double>(v[r][e]) - static_cast<double>(cm[r])) * inv_tau;
        t[4 * NR + r] = (static_cast<double>(mx[r]) - static_cast<double>(cm[r])) * inv_tau;
      }
      exp_lockstep<5 * NR>(t);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        double zz = (mx[r] == -INFINITY) ? 0.0 : z[r] * t[4 * NR + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) zz += (4 * c + e < n) ? t[4 * r + e] : 0.0;
        z[r] = zz;
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) mx[r] = cm[r];
  }
}

// Statistics of R rows whose slices are rows[r * ld + i], i < n: slice max, its
// first index (-1 if the slice holds NaN or +inf) and the sum of
// exp((l - max) / t), into out[0 .. R-1].  One pass per thread over every
// kThreads-th 4-element chunk keeps a running (max, first argmax, sum of exp
// relative to the running max) per row; the partials go to LDS (`scratch`, at
// least R * kThreads * 16 bytes) and wave w then reduces row w over all threads,
// so each wave's dependency chain covers one row, not R.
template <int R, bool kLds>
__device__ __forceinline__ void slice_stats_rows(const float* rows, int ld, int n, int v0, bool greedy, double inv_tau,
                                                 Rec* out, void* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* pm = static_cast<float*>(scratch);
  int* pi = reinterpret_cast<int*>(pm + R * kThreads);
  double* pz = reinterpret_cast<double*>(pi + R * kThreads);
  const int nc = (n + 3) >> 2;
  float mx[R];
  int ix[R];
  double z[R];
  scan_chunks<R, kLds>(rows, ld, n, v0, inv_tau, tid, nc, kThreads, greedy, mx, ix, z);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pm[r * kThreads + tid] = mx[r];
    pi[r * kThreads + tid] = ix[r];
    pz[r * kThreads + tid] = z[r];
  }
  __syncthreads();
  for (int r = wave; r < R; r += kWaves) {
    constexpr int K = kThreads / 64;
    float m = -INFINITY, ms[K];
    int i = 0x7fffffff;
    double zs[K];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {  // ties keep the lower index
      ms[k] = pm[r * kThreads + k * 64 + lane];
      const int ik = pi[r * kThreads + k * 64 + lane];
      zs[k] = pz[r * kThreads + k * 64 + lane];
      bad |= ik < 0;
      const bool take = ms[k] > m || (ms[k] == m && ik < i);
      m = take ? ms[k] : m;
      i = take ? ik : i;
    }
    bad = __any(bad);
    wave_argmax(m, i);
    double zl = 0.0;
    if (!greedy && !bad && m != -INFINITY) {
      double f[K];
#pragma unroll
      for (int k = 0; k < K; ++k) f[k] = (static_cast<double>(ms[k]) - static_cast<double>(m)) * inv_tau;
      exp_lockstep<K>(f);
#pragma unroll
      for (int k = 0; k < K; ++k) zl += (ms[k] == -INFINITY) ? 0.0 : zs[k] * f[k];
    }
    const double zt = readlane_d(wave_incl_scan(zl), 63);
    if (lane == 0) {
      out[r].m = m;
      out[r].idx = bad ? -1 : (i == 0x7fffffff ? v0 : i);
      out[r].z = zt;
    }
  }
  __syncthreads();
}

// Statistics of R = 4 or 8 rows (as slice_stats_rows) with every row owned by
// one wave: wave w takes row w and, for R = 8, row w + 4; lane l scans chunks
// l, l + 64, ... of the row and the wave reduces its rows at once, with no
// partials in LDS and no workgroup barrier before the reduction.
template <int R>
__device__ __forceinline__ void slice_stats_rows_by_wave(const float* rows, int ld, int n, int v0, bool greedy,
                                                         double inv_tau, int E, Rec* out) {
  static_assert(R % kWaves == 0, "whole rows per wave");
  constexpr int RPW = R / kWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nc = (n + 3) >> 2;
  float mx[RPW];
  int ix[RPW];
  double z[RPW];
  // rows wave, wave + 4, ... of the E staged ones; a wave past the last one
  // scans row E - 1 again (its record is not published)
  if (RPW == 1 || wave + kWaves < E)
    scan_chunks<RPW, true>(rows + min(wave, E - 1) * ld, kWaves * ld, n, v0, inv_tau, lane, nc, 64, greedy, mx, ix, z);
  else
    scan_chunks<RPW, true>(rows + min(wave, E - 1) * ld, 0, n, v0, inv_tau, lane, nc, 64, greedy, mx, ix, z);
  float m[RPW];
  int arg[RPW];
  bool bad[RPW];
  double f[RPW];
#pragma unroll
  for (int h = 0; h < RPW; ++h) {
    bad[h] = __any(ix[h] < 0);
    m[h] = mx[h];
    arg[h] = ix[h];
    wave_argmax(m[h], arg[h]);  // ties keep the lower index
    f[h] = (static_cast<double>(mx[h]) - static_cast<double>(m[h])) * inv_tau;
  }
  exp_lockstep<RPW>(f);
#pragma unroll
  for (int h = 0; h < RPW; ++h) {
    const double zl = (!greedy && !bad[h] && m[h] != -INFINITY && mx[h] != -INFINITY) ? z[h] * f[h] : 0.0;
    const double zt = readlane_d(wave_incl_scan(zl), 63);
    if (lane == 0) {
      const int r = wave + h * kWaves;
      out[r].m = m[h];
      out[r].idx = bad[h] ? -1 : (arg[h] == 0x7fffffff ? v0 : arg[h]);
      out[r].z = zt;
    }
  }
  __syncthreads();
}

// Merges the members' statistics of one row in one wave (lane w < NW holds
// member w's record): max logit, first argmax, 1/z with z summed in member order,
// error bits, and each member's share of p (slice mass of p, for a draw from p).
__device__ __forceinline__ void merge_row(const Rec& r, bool member, bool greedy, double inv_tau, float* m_out,
                                          double* iz_out, int* arg_out, int* err_out, double* mass_out) {
  const int lane = threadIdx.x & 63;
  const bool badr = member && r.idx < 0;
  float m = r.m;
  int arg = badr ? 0x7fffffff : r.idx;
  wave_argmax(m, arg);
  double zl = 0.0;
  if (!greedy && member && r.m != -INFINITY) zl = r.z * exp1((static_cast<double>(r.m) - m) * inv_tau);
  const double zt = readlane_d(wave_incl_scan(zl), 63);  // member-order sum
  const bool anybad = __any(badr);
  const double iz = 1.0 / zt;
  if (member) mass_out[lane] = greedy ? 0.0 : zl * iz;
  if (lane == 0) {
    int err = 0;
    if (anybad) err |= SPEC_DEV_NONFINITE;
    if (!greedy && !(zt > 0.0)) err |= SPEC_DEV_EMPTY;
    *err_out = err;
    *m_out = m;
    *iz_out = iz;
    *arg_out = arg;
  }
}

// ---------------------------------------------------------------------------
// Top-k / top-p truncation of the target rows the walk visits (the Sequoia
// summary's top-p robustness table verifies against a nucleus-truncated
// target; the rules come from Fan et al. 2018 and Holtzman et al. 2020).  Row u
// keeps {x : l(x) >= t_u}: t_u is the K-th largest logit, then, for top_p < 1,
// the largest kept value v whose set {l >= v} holds top_p of the kept mass of
// softmax(l / temperature); equal logits are never split.  Dropped tokens get
// p = 0 in the accept tests, the residuals and the final draws.
//
// Each member lists the kc largest values of its slice of the row (kc <= K):
// t_w = its kc-th largest, e_w = how many of its elements equal t_w, and its
// values above t_w.  Every element >= t_w of member w is then listed or
// counted, so the union of the lists is complete above L = max_w t_w; when the
// union holds at least K entries >= L, the global K-th largest lies there
// (and is found by bisection over order-preserving keys, counting the union).
// Otherwise (a slice held more than kc of the row's top values) the members
// exchange their full K-lists, for which the union always suffices.
// ---------------------------------------------------------------------------
constexpr int kTopKMax = kTruncTopKMax;  // top_k taken inside the walk
constexpr int kCandCap = 256;            // elements gathered for a slice's exact selection
constexpr int kWaveSel = kSliceCap / kWaves;  // LDS floats of selection scratch per wave
constexpr int kListPoll = 16;             // list words a thread polls at a time
constexpr uint32_t kNoValue = 0x7FC00000u;  // NaN: a list word that is never counted

// The selection helpers below are real calls (inlining them three times over
// would spill the walk's registers); their pointers carry the address space,
// so that their LDS and global accesses compile to LDS and global instructions
// instead of generic (flat) ones.
typedef __attribute__((address_space(3))) float lds_f;
typedef __attribute__((address_space(3))) int lds_i;
typedef __attribute__((address_space(3))) uint32_t lds_u;
typedef __attribute__((address_space(3))) double lds_d;
typedef __attribute__((address_space(3))) f32x4 lds_f4;
typedef __attribute__((address_space(1))) unsigned long long gbl_u64;
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds(T* p) {
  return (__attribute__((address_space(3))) T*)(p);
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gbl(T* p) {
  return (__attribute__((address_space(1))) T*)(p);
}
template <bool kLds>
__device__ __forceinline__ auto row_ptr(const float* p) {
  if constexpr (kLds)
    return (const lds_f*)(p);
  else
    return (const __attribute__((address_space(1))) float*)(p);
}
// a slice row: LDS or global memory
template <bool kLds>
using RowPtr = typename std::conditional<kLds, const lds_f*, const __attribute__((address_space(1))) float*>::type;
template <bool kLds>
__device__ __forceinline__ f32x4 row4(RowPtr<kLds> p, int valid) {
  if constexpr (kLds) {
    return *reinterpret_cast<const lds_f4*>(p);
  } else {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid) v[e] = p[e];
    return v;
  }
}

static_assert(kCandCap + kTopKMax <= kWaveSel, "a wave's selection scratch holds its candidates and its list");

// Order-preserving 32-bit keys of floats (-0 taken as +0), and back.
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float okey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += dpp_i<kShr1, 0xF>(0, v);
  v += dpp_i<kShr2, 0xF>(0, v);
  v += dpp_i<kShr4, 0xF>(0, v);
  v += dpp_i<kShr8, 0xF>(0, v);
  v += dpp_i<kBcast15, 0xA>(0, v);
  v += dpp_i<kBcast31, 0xC>(0, v);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) { return __builtin_amdgcn_readlane(wave_incl_scan_i(v), 63); }
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// The value of lane ^ J: within a row of 16 lanes by DPP (quad permutes for
// 1 and 2, row shifts for 4 and 8), across rows by ds_bpermute.
template <int J>
__device__ __forceinline__ int xor_lane_i(int x) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (J == 4 || J == 8) {
    const int up = __builtin_amdgcn_update_dpp(x, x, 0x100 + J, 0xF, 0xF, false);  // row_shl: from lane + J
    const int dn = __builtin_amdgcn_update_dpp(x, x, 0x110 + J, 0xF, 0xF, false);  // row_shr: from lane - J
    return (threadIdx.x & J) ? dn : up;
  } else {
    return __shfl_xor(x, J);
  }
}
template <int J>
__device__ __forceinline__ float xor_lane_f(float x) {
  return __builtin_bit_cast(float, xor_lane_i<J>(__builtin_bit_cast(int, x)));
}
template <int J>
__device__ __forceinline__ double xor_lane_d(double x) {
  const long long v = __builtin_bit_cast(long long, x);
  const int lo = xor_lane_i<J>(static_cast<int>(v));
  const int hi = xor_lane_i<J>(static_cast<int>(v >> 32));
  return __builtin_bit_cast(double, (static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
// One compare-exchange step of a bitonic sort of the wave's 64 values, largest
// first (K: the size of the blocks being merged, J: the partner distance); the
// payload w moves with its value; equal values stay where they are.
template <int K, int J, bool kPay>
__device__ __forceinline__ void bitonic_step(float& v, double& w) {
  const int lane = threadIdx.x & 63;
  const float ov = xor_lane_f<J>(v);
  const bool lower = (lane & J) == 0;
  const bool desc = (lane & K) == 0;
  const bool take = (lower == desc) ? ov > v : ov < v;
  if constexpr (kPay) {
    const double ow = xor_lane_d<J>(w);
    w = take ? ow : w;
  }
  v = take ? ov : v;
}
template <bool kPay>
__device__ __forceinline__ void wave_sort_desc(float& v, double& w) {
  bitonic_step<2, 1, kPay>(v, w);
  bitonic_step<4, 2, kPay>(v, w);
  bitonic_step<4, 1, kPay>(v, w);
  bitonic_step<8, 4, kPay>(v, w);
  bitonic_step<8, 2, kPay>(v, w);
  bitonic_step<8, 1, kPay>(v, w);
  bitonic_step<16, 8, kPay>(v, w);
  bitonic_step<16, 4, kPay>(v, w);
  bitonic_step<16, 2, kPay>(v, w);
  bitonic_step<16, 1, kPay>(v, w);
  bitonic_step<32, 16, kPay>(v, w);
  bitonic_step<32, 8, kPay>(v, w);
  bitonic_step<32, 4, kPay>(v, w);
  bitonic_step<32, 2, kPay>(v, w);
  bitonic_step<32, 1, kPay>(v, w);
  bitonic_step<64, 32, kPay>(v, w);
  bitonic_step<64, 16, kPay>(v, w);
  bitonic_step<64, 8, kPay>(v, w);
  bitonic_step<64, 4, kPay>(v, w);
  bitonic_step<64, 2, kPay>(v, w);
  bitonic_step<64, 1, kPay>(v, w);
}
// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// LDS scratch of one wave's selections (floats from its base):
//   slice top-k:   [0, 576) each lane's candidates (kLaneSlots a lane, then a
//                  slot that takes the rest), [576, 832) the candidates packed,
//                  [832, 896) the list;
//   row threshold: [0, 512) entry values, [512, 1024) their multiplicities,
//                  [1024, 2048) their masses, then prefix sums (fp64), holding
//                  before them the histogram [1024, 1280) and the kept entries
//                  [1280, 1408).
constexpr int kLaneSlots = 8, kSlotStride = kLaneSlots + 1;
constexpr int kSelPacked = 576, kSelList = 832, kSelScratch = 1024;  // (a slice top-k's whole scratch)
constexpr int kPairCap = 512;
constexpr int kThrMult = 512, kThrMass = 1024, kThrHist = 1024, kThrKept = 1280, kThrKeptIdx = 1344;
static_assert(64 * kSlotStride <= kSelPacked && kSelPacked + kCandCap <= kSelList && kSelList + 64 <= kSelScratch &&
                  4 * kSelScratch <= kEagerCapBig &&
                  kThrMult + kPairCap <= kThrMass && kThrMass + 2 * kPairCap <= kWaveSel &&
                  kThrHist + 256 <= kThrKept && kThrKeptIdx + 64 <= kThrMass + 2 * kPairCap,
              "selection scratch layout");

// Four chunks of four elements a lane per step (chunks c, c + 64, c + 128,
// c + 192), their loads issued together; elements past the slice read -inf.
template <bool kLds>
__device__ __forceinline__ void load_chunks4(RowPtr<kLds> row, int n, int nc, int c, f32x4 (&v)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cu = c + 64 * u;
    v[u] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (cu < nc) v[u] = row4<kLds>(row + 4 * cu, n - 4 * cu);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[u][e] = 4 * cu + e < n ? v[u][e] : -INFINITY;
  }
}

// The kc largest values of one slice (n elements at `row`, LDS when kLds),
// one wave: t = the kc-th largest value (-inf when the slice holds fewer than
// kc values above -inf), e = how many elements equal it, and the a values
// above it (fewer than kc; every value above -inf when t is -inf) at
// sc + kSelList, in a fixed order (lane by lane, each lane's in index order).
// NaN elements are passed over (the row's statistics report them).  Fast
// path: t0, the kc-th largest of the lanes' maxima, has kc elements at or
// above it, so the answer is >= t0; each lane keeps its elements >= t0 (about
// kc in all for most rows), they are packed and ranked.  When a lane holds
// more than kLaneSlots of them or all hold more than kCandCap (flat rows, many
// ties), the answer is found by bisection over order-preserving keys between t0
// and the slice's max, counting the slice.  The passes over the slice are
// branch-free (a selected element is written to its lane's next slot, any
// other to the lane's spare slot).
struct SliceTop {
  float t;
  int e, a;
};

template <bool kLds>
__device__ __forceinline__ SliceTop wave_slice_topk(RowPtr<kLds> row, int n, int kc, lds_f* sc) {
  const int lane = threadIdx.x & 63;
  const int nc = (n + 3) >> 2;
  lds_f* slots = sc + lane * kSlotStride;
  lds_f* packed = sc + kSelPacked;
  lds_f* list = sc + kSelList;
  float mx = -INFINITY;
  for (int c = lane; c < nc; c += 256) {
    f32x4 v[4];
    load_chunks4<kLds>(row, n, nc, c, v);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[u][e]);  // NaN passed over
  }
  float srt = mx;  // the kc-th largest lane maximum (-inf when fewer than kc are finite)
  double none = 0.0;
  wave_sort_desc<false>(srt, none);
  const float t0 = readlane_f(srt, kc - 1);
  int cnt = 0;  // this lane's elements >= t0 (above -inf); the first kLaneSlots kept
  for (int c = lane; c < nc; c += 256) {
    f32x4 v[4];
    load_chunks4<kLds>(row, n, nc, c, v);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = v[u][e];
        const bool sel = x >= t0 && x > -INFINITY;
        slots[sel ? min(cnt, kLaneSlots) : kLaneSlots] = x;
        cnt += sel ? 1 : 0;
      }
  }
  const int incl = wave_incl_scan_i(cnt);
  const int C = __builtin_amdgcn_readlane(incl, 63);
  if (!__any(cnt > kLaneSlots) && C <= kCandCap) {
    for (int k = 0; k < cnt; ++k) packed[incl - cnt + k] = slots[k];
    if (C < kc) {  // fewer than kc values above -inf: all of them
      for (int i = lane; i < C; i += 64) list[i] = packed[i];
      return SliceTop{-INFINITY, 0, C};
    }
    const int Cp = (C + 15) & ~15;
    for (int i = C + lane; i < Cp; i += 64) packed[i] = __uint_as_float(kNoValue);
    bool found = false;
    float tv = 0.f;
    for (int i = lane; i < C; i += 64) {
      const float vi = packed[i];
      int g = 0, q = 0;
      for (int j = 0; j < Cp; j += 16) {
        f32x4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const lds_f4*>(packed + j + 4 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            g += w[u][k] > vi ? 1 : 0;
            q += w[u][k] == vi ? 1 : 0;
          }
      }
      if (g < kc && kc <= g + q) {
        found = true;
        tv = vi;
      }
    }
    // some candidate is the kc-th largest (the elements >= t0 are all packed)
    const float t = readlane_f(tv, __ffsll(static_cast<long long>(__ballot(found))) - 1);
    int a = 0, ne = 0;
    for (int i0 = 0; i0 < C; i0 += 64) {
      const int i = i0 + lane;
      const float v = i < C ? packed[i] : __uint_as_float(kNoValue);
      const bool up = v > t;
      ne += v == t ? 1 : 0;
      const unsigned long long bm = __ballot(up);
      if (up) list[a + lanes_below(bm)] = v;
      a += __builtin_popcountll(bm);
    }
    return SliceTop{t, wave_sum_i(ne), a};
  }
  // slow path: bisection for the largest key x with #{elements >= x} >= kc (count_ge(t0) >= kc)
  auto count_ge = [&](float x) {
    int c = 0;
    for (int cc = lane; cc < nc; cc += 256) {
      f32x4 v[4];
      load_chunks4<kLds>(row, n, nc, cc, v);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) c += (v[u][e] >= x && v[u][e] > -INFINITY) ? 1 : 0;
    }
    return wave_sum_i(c);
  };
  uint32_t lo = okey(t0), hi = okey(wave_max_f(mx));
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo + 1u) >> 1);
    if (count_ge(okey_value(mid)) >= kc)
      lo = mid;
    else
      hi = mid - 1u;
  }
  const float t = okey_value(lo);
  // the values above t (fewer than kc) lane by lane, each lane's in index order, and the count equal to t
  int mine = 0, ne = 0;
  for (int c = lane; c < nc; c += 256) {
    f32x4 v[4];
    load_chunks4<kLds>(row, n, nc, c, v);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mine += v[u][e] > t ? 1 : 0;
        ne += v[u][e] == t ? 1 : 0;
      }
  }
  const int inc2 = wave_incl_scan_i(mine);
  int pos = inc2 - mine;
  for (int c = lane; c < nc && pos < inc2; c += 256) {
    f32x4 v[4];
    load_chunks4<kLds>(row, n, nc, c, v);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v[u][e] > t) {
          if (pos < kTopKMax) list[pos] = v[u][e];
          ++pos;
        }
  }
  return SliceTop{t, wave_sum_i(ne), __builtin_amdgcn_readlane(inc2, 63)};
}

// A member's list (one wave): LW tagged 64-bit words, like the slots -- word 0
// t_w, word 1 e_w, words 2 .. 2 + a the values above t_w, NaN after them.
__device__ __forceinline__ void put_list(unsigned long long* dst, int LW, const SliceTop& st, const float* list,
                                         uint32_t tag) {
  const int lane = threadIdx.x & 63;
  const unsigned long long tg = static_cast<unsigned long long>(tag) << 32;
  for (int j = lane; j < LW; j += 64) {
    uint32_t p = kNoValue;
    if (j == 0)
      p = __float_as_uint(st.t);
    else if (j == 1)
      p = static_cast<uint32_t>(st.e);
    else if (j - 2 < st.a)
      p = __float_as_uint(list[j - 2]);
    __hip_atomic_store(dst + j, tg | p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The whole workgroup: the lists of nblk consecutive (row, member) blocks of
// LW words (stride LWS words in the workspace) into U[blk * LW + j], each word
// polled until it carries `tag` (bounded like get_slots), kListPoll words a
// thread at a time.  Ends with a barrier.
__device__ __forceinline__ void get_lists(const gbl_u64* src, int LWS, int LW, int nblk, uint32_t tag,
                                                    lds_u* U, lds_i* fail) {
  const int tid = threadIdx.x;
  const int nwords = nblk * LW;
  const float inv = 1.0f / static_cast<float>(LW);
  for (int base = 0; base < nwords; base += kListPoll * kThreads) {
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kListPoll; ++k)
      if (base + tid + k * kThreads < nwords) pending |= 1u << k;
    unsigned spins = 0;
    for (;;) {
      unsigned long long w[kListPoll];
#pragma unroll
      for (int k = 0; k < kListPoll; ++k) {
        w[k] = 0ull;
        if ((pending >> k) & 1u) {
          const int i = base + tid + k * kThreads;
          const int blk = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
          w[k] = __hip_atomic_load(const_cast<gbl_u64*>(src + static_cast<long>(blk) * LWS + (i - blk * LW)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int k = 0; k < kListPoll; ++k)
        if (((pending >> k) & 1u) && static_cast<uint32_t>(w[k] >> 32) == tag) {
          U[base + tid + k * kThreads] = static_cast<uint32_t>(w[k]);
          pending &= ~(1u << k);
        }
      if (!__syncthreads_or(pending != 0u)) break;
      if (++spins > kSpinLimit) {
        if (tid == 0) *fail = 1;
        __syncthreads();
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// Threads t .. of nt (whole waves, t counted from the first of them): the
// words of get_lists, each thread polling its own until they carry `tag`
// (bounded like get_slots), with no barrier: the caller's barrier publishes U.
__device__ __forceinline__ void poll_lists(const gbl_u64* src, int LWS, int LW, int nblk, uint32_t tag, lds_u* U,
                                           lds_i* fail, int t, int nt) {
  const int nwords = nblk * LW;
  const float inv = 1.0f / static_cast<float>(LW);
  for (int base = 0; base < nwords; base += kListPoll * nt) {
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kListPoll; ++k)
      if (base + t + k * nt < nwords) pending |= 1u << k;
    unsigned spins = 0;
    while (__any(pending != 0u)) {
      unsigned long long w[kListPoll];
#pragma unroll
      for (int k = 0; k < kListPoll; ++k) {
        w[k] = 0ull;
        if ((pending >> k) & 1u) {
          const int i = base + t + k * nt;
          const int blk = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
          w[k] = __hip_atomic_load(const_cast<gbl_u64*>(src + static_cast<long>(blk) * LWS + (i - blk * LW)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int k = 0; k < kListPoll; ++k)
        if (((pending >> k) & 1u) && static_cast<uint32_t>(w[k] >> 32) == tag) {
          U[base + t + k * nt] = static_cast<uint32_t>(w[k]);
          pending &= ~(1u << k);
        }
      if (++spins > kSpinLimit) {
        *fail = 1;
        return;
      }
      if (__any(pending != 0u)) __builtin_amdgcn_s_sleep(1);
    }
  }
}

// The row's lists: NB blocks of LW words in U (block b: t_b, e_b, then the
// values above t_b, NaN after them), member w owning blocks w*Q .. w*Q+Q-1
// (its slice cut into Q parts in index order).  An entry is a listed value
// (multiplicity 1) or a block's t_b group (multiplicity e_b; none when t_b is
// -inf).  Word i of U: block i / LW (taken in fp32, exact for these sizes).
struct ListWord {
  float v;  // NaN: no entry
  int mult, blk;
};
__device__ __forceinline__ ListWord list_word(const lds_u* U, int nw, int LW, float inv, int i) {
  const int ic = min(i, nw - 1);
  const float w0 = __uint_as_float(U[ic]);
  const int w1 = static_cast<int>(U[min(ic + 1, nw - 1)]);  // (a t_b word is never the last)
  const int b = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
  const int j = i - b * LW;
  const bool head = j == 0 && w0 > -INFINITY;
  const bool val = j >= 2;
  ListWord e;
  e.v = (i < nw && (head || val)) ? w0 : __uint_as_float(kNoValue);
  e.mult = head ? w1 : 1;
  e.blk = b;
  return e;
}

// Member shares of the kept mass when the entries above L outnumber the
// scratch: bisection for the K-th largest over the list words, the kept
// entries by a pass over them, each member's mass summed over its blocks'
// words in order.  (Rare: a union far larger than the lists usually are.)
__device__ __forceinline__ void wave_row_threshold_slow(const lds_u* U, int NB, int Q, int NW, int LW, float L, int W,
                                                        int K, double top_p, float m, double inv_tau, lds_f* sc,
                                                        lds_f* thr, lds_d* iz_out, lds_d* mass) {
  const int lane = threadIdx.x & 63;
  const int nw = NB * LW;
  const float inv = 1.0f / static_cast<float>(LW);
  auto count_ge = [&](float x) {
    int c = 0;
    for (int i = lane; i < nw; i += 64) {
      const ListWord e = list_word(U, nw, LW, inv, i);
      c += e.v >= x ? e.mult : 0;
    }
    return wave_sum_i(c);
  };
  float tk = -INFINITY;
  if (W >= K) {
    uint32_t lo = okey(L), hi = okey(m);
    while (lo < hi) {
      const uint32_t mid = lo + ((hi - lo + 1u) >> 1);
      if (count_ge(okey_value(mid)) >= K)
        lo = mid;
      else
        hi = mid - 1u;
    }
    tk = okey_value(lo);
  }
  lds_f* kv = sc;
  int ngt = 0, ntie = 0;
  for (int i0 = 0; i0 < nw; i0 += 64) {
    const ListWord e = list_word(U, nw, LW, inv, i0 + lane);
    const bool up = e.v > tk;
    ntie += e.v == tk ? e.mult : 0;
    const unsigned long long bm = __ballot(up);
    if (up) kv[ngt + lanes_below(bm)] = e.v;
    ngt += __builtin_popcountll(bm);
  }
  ntie = wave_sum_i(ntie);
  float ev = -INFINITY;
  double em = 0.0;
  const double tk_mass = tk > -INFINITY ? exp1((static_cast<double>(tk) - static_cast<double>(m)) * inv_tau) : 0.0;
  if (lane < ngt) {
    ev = kv[lane];
    em = exp1((static_cast<double>(ev) - static_cast<double>(m)) * inv_tau);
  } else if (lane == ngt && ntie > 0) {
    ev = tk;
    em = static_cast<double>(ntie) * tk_mass;
  }
  float t = tk;
  if (top_p < 1.0) {
    wave_sort_desc<true>(ev, em);
    const double cum = wave_incl_scan(em);
    const double zk = readlane_d(cum, 63);
    const unsigned long long hb = __ballot(ev > -INFINITY && cum / zk >= top_p);
    if (hb) t = readlane_f(ev, __ffsll(static_cast<long long>(hb)) - 1);
  }
  double share = 0.0;
  if (lane < NW)
    for (int i = lane * Q * LW; i < (lane + 1) * Q * LW; ++i) {
      const ListWord e = list_word(U, nw, LW, inv, i);
      if (e.v >= t) share += static_cast<double>(e.mult) * exp1((static_cast<double>(e.v) - static_cast<double>(m)) * inv_tau);
    }
  const double z = readlane_d(wave_incl_scan(share), 63);
  const double iz = 1.0 / z;
  if (lane < NW) mass[lane] = share * iz;
  if (lane == 0) {
    *thr = t;
    *iz_out = iz;
  }
}

// The row's threshold from its lists (one wave).  m: the row's max logit
// (finite).  Writes *thr, *iz (1 / kept mass of exp((l - m) / t)) and mass[w]
// (member w's share of the kept mass), all in fixed orders so that every
// member gets the same values; or sets *fb when the lists were too short
// (their lengths below K only).  sc: the wave's selection scratch.  The lanes
// take the list words in turn: the entries >= L = max t_b are packed in word
// order (block by block) by ballots; the K-th largest is found by rounds of a
// 256-bin histogram of their keys, each round keeping the bin where the
// running weight from the top reaches K (at most four rounds for 32-bit
// keys); the kept entries (fewer than K above it, then its group) are sorted
// by value across the lanes and their masses scanned for top-p; the members'
// shares are differences of one prefix sum over the packed entries.
constexpr int kMultBits = 24;  // a packed entry: multiplicity (< 2^24) | block << 24
__device__ __forceinline__ void wave_row_threshold(lds_u* U, int NB, int Q, int NW, int LW, int K,
                                                             double top_p, float m, double inv_tau, lds_f* sc,
                                                             lds_f* thr, lds_d* iz_out, lds_d* mass, lds_i* fb) {
  const int lane = threadIdx.x & 63;
  float tmax = -INFINITY;
  for (int b = lane; b < NB; b += 64) tmax = fmaxf(tmax, __uint_as_float(U[b * LW]));
  const float L = wave_max_f(tmax);
  const int nw = NB * LW;
  const float inv = 1.0f / static_cast<float>(LW);
  lds_f* pv = sc;
  lds_u* pm = reinterpret_cast<lds_u*>(sc + kThrMult);
  lds_d* pw = reinterpret_cast<lds_d*>(sc + kThrMass);
  constexpr uint32_t kMultMask = (1u << kMultBits) - 1u;
  // pack the entries >= L in word order (four words a lane read at once)
  int P = 0, wsum = 0;
  for (int i0 = 0; i0 < nw; i0 += 256) {
    ListWord e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = list_word(U, nw, LW, inv, i0 + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool keep = e[u].v >= L;  // (NaN never)
      wsum += keep ? e[u].mult : 0;
      const unsigned long long bm = __ballot(keep);
      const int pos = P + lanes_below(bm);
      if (keep && pos < kPairCap) {
        pv[pos] = e[u].v;
        pm[pos] = static_cast<uint32_t>(e[u].mult) | (static_cast<uint32_t>(e[u].blk) << kMultBits);
      }
      P += __builtin_popcountll(bm);
    }
  }
  const int W = wave_sum_i(wsum);
  if (L > -INFINITY && W < K) {  // the K-th largest may lie below some block's t_b
    if (lane == 0) *fb = 1;
    return;
  }
  if (lane == 0) *fb = 0;
  if (P > kPairCap) {
    wave_row_threshold_slow(U, NB, Q, NW, LW, L, W, K, top_p, m, inv_tau, sc, thr, iz_out, mass);
    return;
  }
  // the K-th largest entry (weighted): keys in [lo, hi], `above` the weight over hi
  float tk = -INFINITY;
  if (W >= K) {
    lds_u* hist = reinterpret_cast<lds_u*>(sc + kThrHist);
    uint32_t lo = okey(L), hi = okey(m);
    int above = 0;
    while (lo < hi) {
      const uint32_t range = hi - lo;
      const int sh = range < 256u ? 0 : 24 - __builtin_clz(range);  // (range >> sh) < 256
#pragma unroll
      for (int k = 0; k < 4; ++k) hist[lane + 64 * k] = 0u;
      for (int i = lane; i < P; i += 64) {
        const uint32_t key = okey(pv[i]);
        if (key >= lo && key <= hi)
          __hip_atomic_fetch_add(&hist[(hi - key) >> sh], pm[i] & kMultMask, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
      // lane l holds bins 4l .. 4l+3 (bin 0 = the highest keys)
      int h[4], hs = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = static_cast<int>(hist[4 * lane + k]);
        hs += h[k];
      }
      const int hin = wave_incl_scan_i(hs);
      int run = above + hin - hs, bin = -1, before = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool here = bin < 0 && run + h[k] >= K;
        bin = here ? 4 * lane + k : bin;
        before = here ? run : before;
        run += h[k];
      }
      const unsigned long long hb = __ballot(bin >= 0);  // some bin reaches K (W >= K)
      const int src = __ffsll(static_cast<long long>(hb)) - 1;
      const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(bin, src));
      above = __builtin_amdgcn_readlane(before, src);
      const uint32_t nhi = hi - (b << sh);
      const uint32_t span = (1u << sh) - 1u;  // keys of the bin: [nhi - span, nhi] within [lo, hi]
      lo = (nhi - lo >= span) ? nhi - span : lo;
      hi = nhi;
    }
    tk = okey_value(lo);
  }
  // kept entries, one a lane: those above tk (fewer than K, in entry order), then tk's group
  lds_f* kv = sc + kThrKept;
  lds_i* kidx = reinterpret_cast<lds_i*>(sc + kThrKeptIdx);
  int ngt = 0, ntie = 0;
  for (int i0 = 0; i0 < P; i0 += 64) {
    const int i = i0 + lane;
    const float v = i < P ? pv[i] : __uint_as_float(kNoValue);
    const bool up = v > tk;
    ntie += (i < P && v == tk) ? static_cast<int>(pm[i] & kMultMask) : 0;
    const unsigned long long bm = __ballot(up);
    if (up) {
      kv[ngt + lanes_below(bm)] = v;
      kidx[ngt + lanes_below(bm)] = i;
    }
    ngt += __builtin_popcountll(bm);
  }
  ntie = wave_sum_i(ntie);
  float ev = -INFINITY;
  double em = 0.0;
  int my_idx = -1;
  if (lane < ngt) {
    ev = kv[lane];
    my_idx = kidx[lane];
    em = exp1((static_cast<double>(ev) - static_cast<double>(m)) * inv_tau);
  }
  const double tk_mass = tk > -INFINITY ? exp1((static_cast<double>(tk) - static_cast<double>(m)) * inv_tau) : 0.0;
  if (lane == ngt && ntie > 0) {
    ev = tk;
    em = static_cast<double>(ntie) * tk_mass;
  }
  float t = tk;
  const int nent = ngt + (ntie > 0 ? 1 : 0);
  if (top_p < 1.0) {
    // each kept entry: the mass of the entries above it and equal to it (LDS broadcast, entry order)
    lds_f* kvv = sc + kThrKept;
    lds_d* kvm = reinterpret_cast<lds_d*>(sc + kThrHist);
    kvv[lane] = lane < nent ? ev : __uint_as_float(kNoValue);
    kvm[lane] = lane < nent ? em : 0.0;
    const double zk = readlane_d(wave_incl_scan(lane < nent ? em : 0.0), 63);
    double above = 0.0, same = 0.0;
    for (int j = 0; j < nent; j += 4) {
      const f32x4 v4 = *reinterpret_cast<const lds_f4*>(kvv + j);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double mq = kvm[j + q];
        above += v4[q] > ev ? mq : 0.0;
        same += v4[q] == ev ? mq : 0.0;
      }
    }
    const bool hit = lane < nent && above / zk < top_p && (above + same) / zk >= top_p;
    const unsigned long long hb = __ballot(hit);
    if (hb) t = readlane_f(ev, __ffsll(static_cast<long long>(hb)) - 1);
    // (none: the kept mass summed short of top_p by rounding; the top-k set stays)
  }
  // the kept mass (the members' shares are taken when a draw needs them: wave_row_shares)
  const double z = readlane_d(wave_incl_scan((lane < nent && ev >= t) ? em : 0.0), 63);
  (void)mass;
  (void)Q;
  (void)NW;
  (void)my_idx;
  (void)pw;
  if (lane == 0) {
    *thr = t;
    *iz_out = 1.0 / z;
  }
}

// The members' shares of a row's kept mass (one wave), for a draw from the
// row's truncated target: the entries >= t of its lists (NB blocks of LW words,
// Q a member), 64 at a time in word order, their masses computed a lane each
// and summed member by member in word order.  sc: 192 floats of scratch.
__device__ __forceinline__ void wave_row_shares(const lds_u* U, int NB, int Q, int NW, int LW, float t, float m,
                                                double inv_tau, double iz, lds_f* sc, lds_d* mass) {
  const int lane = threadIdx.x & 63;
  const int nw = NB * LW;
  const float inv = 1.0f / static_cast<float>(LW);
  lds_i* gb = reinterpret_cast<lds_i*>(sc);
  lds_d* gw = reinterpret_cast<lds_d*>(sc + 64);
  double share = 0.0;
  int n_in = 0;
  auto flush = [&]() {
    for (int j = 0; j < n_in; j += 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool mine = j + q < n_in && gb[j + q] == lane;
        share += mine ? gw[j + q] : 0.0;
      }
    }
    n_in = 0;
  };
  for (int i0 = 0; i0 < nw; i0 += 64) {
    const ListWord e = list_word(U, nw, LW, inv, i0 + lane);
    const bool keep = e.v >= t;
    const unsigned long long bm = __ballot(keep);
    const int cnt = __builtin_popcountll(bm);
    if (n_in + cnt > 64) flush();
    if (keep) {
      const int pos = n_in + lanes_below(bm);
      gb[pos] = e.blk / Q;
      gw[pos] = static_cast<double>(e.mult) * exp1((static_cast<double>(e.v) - static_cast<double>(m)) * inv_tau);
    }
    n_in += cnt;
  }
  flush();
  if (lane < NW) mass[lane] = share * iz;
}

// kFits: the slice (S <= kSliceCap floats) lives in LDS, so every slice access is an
// LDS access; otherwise the slices are read from global memory where they lie.
// kTree: the largest tree (kSmallTree, or kMaxT with a smaller eager space, so
// that the node arrays fit beside it in the 160 KB of LDS).
template <bool kFits, int kTree>
__global__ __launch_bounds__(kThreads) void reject_team_kernel(const TArgs a) {
  constexpr int kEager = kTree <= kSmallTree ? kEagerCap : kEagerCapBig;
  static_assert(kTree <= 2 * kThreads, "two nodes per thread at most");
  __shared__ __attribute__((aligned(16))) float eager_l[kEager];  // logit slices of rows 0 .. E-1, stride ld
  __shared__ __attribute__((aligned(16))) float eager_q[kEager];  // their draft-probability slices
  __shared__ __attribute__((aligned(16))) float cur_lbuf[kSliceCap];
  __shared__ __attribute__((aligned(16))) float cur_qbuf[kSliceCap];
  __shared__ int16_t first_child[kTree], next_sib[kTree];
  __shared__ int s_par[kTree], s_tok[kTree], s_path[kTree];
  __shared__ float s_lx[kTree], s_qx[kTree];  // logit / draft prob of node c's token in its parent's row
  __shared__ int rej_tok[kTree];
  __shared__ double s_ru[kTree], s_fu[kTree];  // accept draw of node c, final draw at node u
  __shared__ double rej_c[kTree];
  __shared__ __attribute__((aligned(16))) double row_partials[2 * kThreads];  // one row's statistics partials
  __shared__ Rec s_rec[kMaxEager];
  // merged statistics of the eager rows (index r < E) and of the current deeper row (index kMaxEager)
  __shared__ float e_m[kMaxEager + 1];
  __shared__ double e_iz[kMaxEager + 1];
  __shared__ int e_arg[kMaxEager + 1], e_err[kMaxEager + 1];
  __shared__ double e_mass[(kMaxEager + 1) * kMaxTeam];  // each member's share of p
  __shared__ double sh_incl[kWaves];
  __shared__ double s_lastmass[kMaxTeam];  // the members' slice masses of the last residual pass
  __shared__ int sh_err, sh_fail, sh_len, sh_u, sh_c, sh_x, sh_state, sh_nrej, sh_emit_local, sh_owner, sh_arg;
  __shared__ double sh_m, sh_iz, sh_C, sh_Cold, sh_N, sh_s, sh_lo, sh_target, sh_total;
  // truncation threshold of each eager row and of the current deeper row, and
  // whether its lists were too short (a second round with K-lists follows)
  __shared__ float s_thr[kMaxEager + 1];
  __shared__ int s_tfb[kMaxEager + 1];
  __shared__ int s_tsh[kMaxEager + 1];  // the row's member shares of its kept mass are in e_mass already
  __shared__ int s_dnb, s_dq, s_dlw;    // the current later row's lists in eager_l: blocks, parts, words

  const int NW = a.NW;
  const int b = blockIdx.x / NW;
  const int wg = blockIdx.x % NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V, S = a.S, E = a.E, ld = a.ld;
  const int v0 = min(V, wg * S), v1 = min(V, v0 + S);
  const int n = v1 - v0;
  // this thread's contiguous run of 4-element chunks of the slice: elements [i0, i1)
  const int nc = (n + 3) >> 2;
  const int per = (nc + kThreads - 1) / kThreads;
  const int c0 = min(nc, tid * per), c1 = min(nc, c0 + per);
  const int i0 = min(n, 4 * c0), i1 = min(n, 4 * c1);
  const float* lg_b = a.logits + static_cast<long>(b) * T * V;
  const float* q_b = a.q + static_cast<long>(b) * T * V;
  Slot* eager = a.eager + static_cast<long>(b) * NW * max(E, 1);
  Slot* part = a.part + static_cast<long>(b) * a.part_rows * NW;
  int xrow = 0;  // the next row of part slots (one per exchange after the eager one)
  // the call's tag: the workspace's epoch (advanced by the last workgroup of the grid to leave) + 1
  const uint32_t epoch = __hip_atomic_load(a.hdr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tag = epoch + 1u;
  // truncation: this sequence's lists, LWS words a block.  Eager rows: E rows
  // of NW * q_e blocks (member w's slice cut into q_e parts, one a wave);
  // later rows: a row of NW * q_d blocks each; second rounds (K-lists of whole
  // slices): a row of NW blocks each.  Block of member w, part q: w * q + q.
  const int LWS = a.top_k + 2;
  const int NBe = NW * a.q_e, NBd = NW * a.q_d, LWe = a.kc_e + 2, LWd = a.kc_d + 2;
  unsigned long long* const lists_b = a.trunc ? a.lists + static_cast<long>(b) * a.list_blocks * LWS : nullptr;
  unsigned long long* const lists_d = lists_b + static_cast<long>(8) * NW * LWS;
  unsigned long long* const lists_s = lists_d + static_cast<long>(T) * 4 * NW * LWS;
  int drow = 0, srow = 0;  // rows of later first lists and of second rounds used so far
  // the rows' sums of exp((l - max) / t) are not needed when greedy, nor when truncating (the threshold
  // gives the kept mass): the statistics then take the max and its index only
  const bool no_z = a.greedy || a.trunc;
  // part q of Q of a slice of n elements (a multiple of 4 long, so that parts stay 16-byte aligned)
  auto part_of = [&](int q, int Q, int* len) __attribute__((always_inline)) {
    const int nq = (n + 4 * Q - 1) / (4 * Q) * 4;
    const int s0 = min(n, q * nq);
    *len = min(n, s0 + nq) - s0;
    return s0;
  };
  // row r's threshold from the lists in U (NB blocks, Q a member; one wave, sc
  // its selection scratch), unless the row's statistics already failed (then
  // nothing is kept back)
  auto row_threshold = [&](int r, uint32_t* U, int NB, int Q, int LW, float* sc) __attribute__((always_inline)) {
    if (e_err[r] == 0 && isfinite(e_m[r])) {
      wave_row_threshold(lds(U), NB, Q, NW, LW, a.top_k, a.top_p, e_m[r], a.inv_tau, lds(sc), lds(&s_thr[r]),
                         lds(&e_iz[r]), lds(&e_mass[r * kMaxTeam]), lds(&s_tfb[r]));
    } else if (lane == 0) {
      s_thr[r] = -INFINITY;
      s_tfb[r] = 0;
      if (e_err[r] == 0) e_err[r] = SPEC_DEV_EMPTY;  // (the max is -inf: nothing to keep)
    }
  };
  // row r's member shares of its kept mass (one wave; sc: 192 floats)
  auto row_shares = [&](int r, uint32_t* U, int NB, int Q, int LW, float* sc) __attribute__((always_inline)) {
    if (e_err[r] == 0 && isfinite(e_m[r]))
      wave_row_shares(lds(U), NB, Q, NW, LW, s_thr[r], e_m[r], a.inv_tau, e_iz[r], lds(sc),
                      lds(&e_mass[r * kMaxTeam]));
    if (lane == 0) s_tsh[r] = 1;
  };
  // (whole workgroup) the members' K-lists of row r, whose first lists were too
  // short, and its threshold from them; slice: this member's slice of the row
  auto second_round = [&](int r, const float* slice, uint32_t* U, float* sc) __attribute__((always_inline)) {
    if (srow >= T + kMaxEager) {  // more exchanges than planned: cannot happen for a valid tree
      if (tid == 0) sh_fail = 1;
      __syncthreads();
      return;
    }
    unsigned long long* const row = lists_s + static_cast<long>(srow) * NW * LWS;
    if (wave == 0) {
      const SliceTop st = wave_slice_topk<kFits>(row_ptr<kFits>(slice), n, a.top_k, lds(sc));
      put_list(row + static_cast<long>(wg) * LWS, LWS, st, sc + kSelList, tag);
    }
    get_lists(gbl(row), LWS, LWS, NW, tag, lds(U), lds(&sh_fail));
    ++srow;
    if (!sh_fail && wave == 0) {
      row_threshold(r, U, NW, 1, LWS, sc);
      row_shares(r, U, NW, 1, LWS, sc);
    }
    __syncthreads();
  };

  // tree and tokens (nodes tid and tid + kThreads) and the eager logit and
  // draft slices, which depend on nothing else: all in flight together
  const int pv = a.parent[static_cast<long>(b) * T + min(tid, T - 1)];
  const int tv = a.tokens[static_cast<long>(b) * T + min(tid, T - 1)];
  int pv2 = -1, tv2 = 0;
  if (kTree > kThreads && tid + kThreads < T) {
    pv2 = a.parent[static_cast<long>(b) * T + tid + kThreads];
    tv2 = a.tokens[static_cast<long>(b) * T + tid + kThreads];
  }
  const int c_lb = a.fuse ? a.c.prefix_lens[b] : 0;  // the compaction's prefix length, loaded early
  if constexpr (kFits) {  // (E = 0 for a larger tree whose slice is too long for the eager space)
    stage_dma(eager_l, lg_b + v0, ld, V, E, n);
    if (!a.greedy) stage_dma(eager_q, q_b + v0, ld, V, E, n);
  }
  // the Philox uniforms of every node depend on none of the loads in flight:
  // drawn while they land
  if (!a.greedy)
    for (int i = tid; i < T; i += kThreads) {
      s_ru[i] = draw_uniform(a.seed, a.offset, b, i, 0);
      s_fu[i] = draw_uniform(a.seed, a.offset, b, i, 1);
    }
  if constexpr (kFits) wait_dma();
  if (tid < T) {
    s_par[tid] = pv;
    s_tok[tid] = tv;
  }
  if (kTree > kThreads && tid + kThreads < T) {
    s_par[tid + kThreads] = pv2;
    s_tok[tid + kThreads] = tv2;
  }
  if (tid == 0) {
    sh_err = 0;
    sh_fail = 0;
    sh_len = 1;
    s_path[0] = 0;
    sh_u = 0;
    sh_nrej = 0;
    sh_emit_local = -1;
    sh_owner = 0;
  }
  if (T <= 64) {
    // Checks and the child lists in wave 0, lane i = node i: the children of u
    // are the lanes whose parent is u (one ballot per node), first_child[i] is
    // the lowest of i's, next_sib[i] the lowest of its parent's above i.  (tid 0
    // initialised sh_err above, earlier in this wave's program order.)
    if (wave == 0) {
      const bool in = lane < T;
      const bool ok = in && (lane == 0 ? pv == -1 : (pv >= 0 && pv < lane));
      int err = 0;
      if (in && !ok) err |= SPEC_DEV_PARENT;
      if (in && lane > 0 && ok && (tv < 0 || tv >= V)) err |= SPEC_DEV_TOKEN;
      const bool child = in && lane > 0 && ok;
      unsigned long long mine = 0;
      for (int u = 0; u < T; ++u) {
        const unsigned long long m = __ballot(child && pv == u);
        if (lane == u) mine = m;
      }
      const unsigned long long sibs = __shfl(mine, child ? pv : 0);
      const unsigned long long later = sibs & ~((2ull << lane) - 1ull);  // siblings after this node
      if (in) {
        first_child[lane] = static_cast<int16_t>(mine ? __ffsll(static_cast<long long>(mine)) - 1 : -1);
        next_sib[lane] = static_cast<int16_t>(child && later ? __ffsll(static_cast<long long>(later)) - 1 : -1);
      }
      if (err) atomicOr(&sh_err, err);
    }
    __syncthreads();
  } else {
    __syncthreads();
    // Checks and the child lists: bit c of kids[p] is set for
    // every child c of p (an LDS atomic per node), so first_child[i] (the first c
    // whose parent is i) and next_sib[i] (the first c > i sharing i's parent) are
    // lowest-set-bit lookups, with no scan over the tree.  kids lives in cur_qbuf,
    // which is first written when a deeper row is staged.
    constexpr int kKW = kTree / 32;  // bitset words per parent
    static_assert(kTree * kKW <= kSliceCap, "the child bitsets fit the current-row draft buffer");
    const int nkw = (T + 31) >> 5;   // words in use
    uint32_t* kids = reinterpret_cast<uint32_t*>(cur_qbuf);
    for (int i = tid; i < T * kKW; i += kThreads)
      if ((i & (kKW - 1)) < nkw) kids[i] = 0u;
    __syncthreads();
    {
      int err = 0;
      for (int i = tid; i < T; i += kThreads) {
        const int p = s_par[i];
        const bool ok = (i == 0) ? p == -1 : (p >= 0 && p < i);
        if (!ok) err |= SPEC_DEV_PARENT;
        if (i > 0 && ok && (s_tok[i] < 0 || s_tok[i] >= V)) err |= SPEC_DEV_TOKEN;
        if (i > 0 && ok) atomicOr(&kids[p * kKW + (i >> 5)], 1u << (i & 31));
      }
      if (err) atomicOr(&sh_err, err);
    }
    __syncthreads();
    for (int i = tid; i < T; i += kThreads) {
      int fc = -1;
      for (int w = 0; w < nkw && fc < 0; ++w) {
        const uint32_t m = kids[i * kKW + w];
        if (m) fc = w * 32 + __builtin_ctz(m);
      }
      const int p = s_par[i];
      int ns = -1;
      if (i > 0 && p >= 0 && p < i) {
        for (int w = (i + 1) >> 5; w < nkw && ns < 0; ++w) {
          uint32_t m = kids[p * kKW + w];
          if (w == ((i + 1) >> 5)) m &= 0xFFFFFFFFu << ((i + 1) & 31);
          if (m) ns = w * 32 + __builtin_ctz(m);
        }
      }
      first_child[i] = static_cast<int16_t>(fc);
      next_sib[i] = static_cast<int16_t>(ns);
    }
    __syncthreads();
  }

  int emitted = -1;  // greedy argmax, known to every member
  if (sh_err == 0) {
    // accept-test operands of every drafted node (logit and draft probability of
    // its token in its parent's row): loaded just before the first team barrier,
    // whose latency they share, and stored to LDS after it
    const int cx = 1 + tid, cx2 = 1 + tid + kThreads;  // nodes cx2 only in trees of more than kThreads + 1
    const int nd = min(cx, T - 1);  // lanes past the tree re-read a valid node (or element 0)
    const long off = nd >= 1 ? static_cast<long>(s_par[nd]) * V + s_tok[nd] : 0;
    const bool two = kTree > kThreads && cx2 < T;
    const long off2 = two ? static_cast<long>(s_par[cx2]) * V + s_tok[cx2] : 0;
    // statistics of the first E rows, from their LDS slices (landed before the tree build's barrier)
    if (kFits && E > 0) {
      switch (E) {
        case 1:
          slice_stats_rows<1, true>(eager_l, ld, n, v0, no_z, a.inv_tau, s_rec, cur_lbuf);
          break;
        case 2:
          slice_stats_rows<2, true>(eager_l, ld, n, v0, no_z, a.inv_tau, s_rec, cur_lbuf);
          break;
        case 4:
        case 3:
          slice_stats_rows_by_wave<4>(eager_l, ld, n, v0, no_z, a.inv_tau, E, s_rec);
          break;
        default:  // 5 to 8
          slice_stats_rows_by_wave<8>(eager_l, ld, n, v0, no_z, a.inv_tau, E, s_rec);
          break;
      }
      if (tid < E) put_slot(&eager[wg * E + tid], s_rec[tid], tag);
      const float lx = lg_b[off];
      const float qx = (a.greedy ? lg_b : q_b)[off];
      const float lx2 = two ? lg_b[off2] : 0.f;
      const float qx2 = two ? (a.greedy ? lg_b : q_b)[off2] : 0.f;
      if (a.trunc) {  // this member's first lists of the eager rows: (row, part) pairs dealt to the waves
        float* sc = cur_qbuf + wave * kWaveSel;
        for (int task = wave; task < E * a.q_e; task += kWaves) {
          const int r = task / a.q_e, q = task - r * a.q_e;
          int len;
          const int s0 = part_of(q, a.q_e, &len);
          const SliceTop st = wave_slice_topk<kFits>(row_ptr<kFits>(eager_l + r * ld + s0), len, a.kc_e, lds(sc));
          put_list(lists_b + (static_cast<long>(r) * NBe + wg * a.q_e + q) * LWS, LWe, st, sc + kSelList, tag);
        }
      }
      // gather every member's eager rows (wave w: rows w and w + 4) and merge them, member order
      const Rec none = Rec{-INFINITY, 0x7fffffff, 0.0};
      if (wave + kWaves < E) {
        const Slot* const rows2[2] = {eager + wave, eager + wave + kWaves};
        Rec rr[2];
        get_slots<2>(rows2, E, NW, tag, none, rr, &sh_fail);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          merge_row(rr[h], lane < NW, no_z, a.inv_tau, &e_m[wave + h * kWaves], &e_iz[wave + h * kWaves],
                    &e_arg[wave + h * kWaves], &e_err[wave + h * kWaves], &e_mass[(wave + h * kWaves) * kMaxTeam]);
      } else if (wave < E) {
        const Slot* const rows1[1] = {eager + wave};
        Rec rr[1];
        get_slots<1>(rows1, E, NW, tag, none, rr, &sh_fail);
        merge_row(rr[0], lane < NW, no_z, a.inv_tau, &e_m[wave], &e_iz[wave], &e_arg[wave], &e_err[wave],
                  &e_mass[wave * kMaxTeam]);
      }
      if (cx < T) {
        s_lx[cx] = lx;
        s_qx[cx] = qx;
      }
      if (two) {
        s_lx[cx2] = lx2;
        s_qx[cx2] = qx2;
      }
      __syncthreads();
      if (a.trunc) {  // every member's lists of the eager rows, then their thresholds
        uint32_t* U = reinterpret_cast<uint32_t*>(cur_lbuf);
        get_lists(gbl(lists_b), LWS, LWe, E * NBe, tag, lds(U), lds(&sh_fail));
        if (!sh_fail) {
          for (int r = wave; r < E; r += kWaves) {
            row_threshold(r, U + r * NBe * LWe, NBe, a.q_e, LWe, cur_qbuf + wave * kWaveSel);
            if (lane == 0) s_tsh[r] = 0;
          }
          __syncthreads();
          bool any_fb = false;
          for (int r = 0; r < E; ++r) any_fb = any_fb || s_tfb[r] != 0;
          if (any_fb) {  // a second round overwrites these lists: take every other row's shares first
            for (int r = wave; r < E; r += kWaves)
              if (!s_tfb[r]) row_shares(r, U + r * NBe * LWe, NBe, a.q_e, LWe, cur_qbuf + wave * kWaveSel);
            __syncthreads();
          }
          for (int r = 0; r < E && !sh_fail; ++r)
            if (s_tfb[r]) second_round(r, eager_l + r * ld, U, cur_qbuf);
        }
      }
    } else {
      if (cx < T) {
        s_lx[cx] = lg_b[off];
        s_qx[cx] = (a.greedy ? lg_b : q_b)[off];
      }
      if (two) {
        s_lx[cx2] = lg_b[off2];
        s_qx[cx2] = (a.greedy ? lg_b : q_b)[off2];
      }
      __syncthreads();
    }

    for (;;) {  // one iteration per visited node
      if (sh_fail) break;
      const int u = sh_u;
      const bool has_kids = first_child[u] >= 0;
      // this node's logit slice (LDS when it fits) and, if it has children, its draft slice
      const float* cl;
      const float* cq;
      if constexpr (kFits) {
        if (u < E) {
          cl = eager_l + u * ld;
          cq = eager_q + u * ld;
        } else {
          stage_dma(cur_lbuf, lg_b + static_cast<long>(u) * V + v0, ld, 0, 1, n);
          if (!a.greedy && has_kids) stage_dma(cur_qbuf, q_b + static_cast<long>(u) * V + v0, ld, 0, 1, n);
          wait_dma();
          cl = cur_lbuf;
          cq = cur_qbuf;
        }
      } else {
        cl = lg_b + static_cast<long>(u) * V + v0;
        cq = q_b + static_cast<long>(u) * V + v0;
      }
      __syncthreads();
      if (u >= E) {  // a deeper row: its statistics now
        slice_stats_rows<1, kFits>(cl, ld, n, v0, no_z, a.inv_tau, s_rec, row_partials);
        if (xrow >= a.part_rows) {  // more exchanges than planned: cannot happen for a valid tree
          if (tid == 0) sh_fail = 1;
          break;
        }
        Slot* xs = part + xrow * NW;
        ++xrow;
        if (tid == 0) put_slot(&xs[wg], s_rec[0], tag);
        if (a.trunc && wave < a.q_d && drow < T) {  // this member's first lists of the row, a part a wave
          float* sc = eager_q + wave * kSelScratch;    // (the eager buffers are free now)
          int len;
          const int s0 = part_of(wave, a.q_d, &len);
          const SliceTop st = wave_slice_topk<kFits>(row_ptr<kFits>(cl + s0), len, a.kc_d, lds(sc));
          put_list(lists_d + (static_cast<long>(drow) * NBd + wg * a.q_d + wave) * LWS, LWd, st, sc + kSelList, tag);
        }
        if (wave == 0) {
          const Slot* const rows1[1] = {xs};
          Rec r[1];
          get_slots<1>(rows1, 1, NW, tag, Rec{-INFINITY, 0x7fffffff, 0.0}, r, &sh_fail);
          merge_row(r[0], lane < NW, no_z, a.inv_tau, &e_m[kMaxEager], &e_iz[kMaxEager], &e_arg[kMaxEager],
                    &e_err[kMaxEager], &e_mass[kMaxEager * kMaxTeam]);
        } else if (a.trunc && drow < T) {  // meanwhile the other waves read every member's lists of the row
          poll_lists(gbl(lists_d + static_cast<long>(drow) * NBd * LWS), LWS, LWd, NBd, tag,
                     lds(reinterpret_cast<uint32_t*>(eager_l)), lds(&sh_fail), tid - 64, kThreads - 64);
        }
        __syncthreads();
        if (sh_fail) break;
        if (a.trunc) {  // the row's threshold from the lists
          if (drow >= T) {  // more rows than the tree has: cannot happen for a valid tree
            if (tid == 0) sh_fail = 1;
            break;
          }
          uint32_t* U = reinterpret_cast<uint32_t*>(eager_l);
          ++drow;
          if (wave == 0) {
            row_threshold(kMaxEager, U, NBd, a.q_d, LWd, eager_q);
            if (lane == 0) {
              s_tsh[kMaxEager] = 0;
              s_dnb = NBd;
              s_dq = a.q_d;
              s_dlw = LWd;
            }
          }
          __syncthreads();
          if (s_tfb[kMaxEager]) {
            second_round(kMaxEager, cl, U, eager_q);
            if (sh_fail) break;
          }
        }
      }
      const int er = u < E ? u : kMaxEager;  // this row's merged statistics
      const float thr = a.trunc ? s_thr[er] : -INFINITY;  // kept: logits >= thr
      if (tid == 0) {
        sh_err |= e_err[er];
        sh_m = e_m[er];
        sh_iz = e_iz[er];
        sh_arg = e_arg[er];
        sh_C = 0.0;
        sh_N = 1.0;
        sh_s = 1.0;
        sh_nrej = 0;
        sh_c = first_child[u];
      }
      __syncthreads();
      if (sh_err) break;
      if (a.greedy) {
        if (tid == 0) {
          int c = first_child[u];
          while (c >= 0 && s_tok[c] != sh_arg) c = next_sib[c];
          if (c >= 0) {
            s_path[sh_len++] = c;
            sh_u = c;
          }
          sh_state = c >= 0 ? 1 : 0;
        }
        __syncthreads();
        if (sh_state == 1) continue;
        emitted = sh_arg;
        break;
      }
      const double m = sh_m, iz = sh_iz;
      // current residual weights of the 4 slice elements 4c .. 4c+3 (logits lv, draft probabilities qv)
      auto weight4 = [&](const f32x4& lv, const f32x4& qv, int c, double (&w)[4]) {
        if (!(lv[0] >= thr || lv[1] >= thr || lv[2] >= thr || lv[3] >= thr)) {  // all truncated: p = 0, weight 0
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = 0.0;
          return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (static_cast<double>(lv[e]) - m) * a.inv_tau;
        exp_lockstep<4>(w);
        const double C = sh_C;
        const int nrej = sh_nrej;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = lv[e] >= thr ? w[e] * iz : 0.0;  // a truncated token has p = 0
          if (nrej > 0 || C != 0.0) {
            const int x = v0 + 4 * c + e;
            double cx = C;
            for (int k = 0; k < nrej; ++k)
              if (rej_tok[k] == x) cx = rej_c[k];
            w[e] = fmax(w[e] - cx * static_cast<double>(qv[e]), 0.0);
          }
        }
      };
      // publish the slice mass of the current weights, scanned in index order
      double excl = 0.0, incl = 0.0;  // this thread's range within the slice
      auto scan_slice = [&](bool check_q) -> bool {
        double mine = 0.0;
        bool badq = false;
        for (int c = c0; c < c1; ++c) {
          const f32x4 lv = load4<kFits>(cl + 4 * c, n - 4 * c);
          const f32x4 qv = load4<kFits>(cq + 4 * c, n - 4 * c);
          double w[4];
          weight4(lv, qv, c, w);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = 4 * c + e < n;
            if (check_q) badq |= in && isnan(qv[e]);
            mine += in ? w[e] : 0.0;
          }
        }
        badq = __syncthreads_or(badq);
        incl = wave_incl_scan(mine);
        if (lane == 63) sh_incl[wave] = incl;
        __syncthreads();
        double before = 0.0;
        for (int w = 0; w < wave; ++w) before += sh_incl[w];
        incl += before;
        excl = wave_shift_up(incl, before);  // lane 0: the waves before it
        return badq;
      };
      bool scanned = false;  // s_lastmass holds the members' slice masses of the current weights
      // try the children of u in turn
      for (;;) {
        if (tid == 0) {
          const int c = sh_c;
          if (c < 0) {
            sh_state = 0;  // no untried child: final draw at u
          } else {
            const int x = s_tok[c];
            const double px = s_lx[c] >= thr ? exp1((static_cast<double>(s_lx[c]) - m) * a.inv_tau) * iz : 0.0;
            const float qf = s_qx[c];
            if (isnan(qf)) sh_err |= SPEC_DEV_NONFINITE;
            const double qx = static_cast<double>(qf);
            int k = 0;
            while (k < sh_nrej && rej_tok[k] != x) ++k;
            const bool removed = k < sh_nrej;
            const double cx = removed ? rej_c[k] : sh_C;
            const double pt = fmax(px - cx * qx, 0.0) / sh_N;
            const double qt = removed ? 0.0 : sh_s * qx;
            const double r = s_ru[c];
            sh_x = x;
            if (r * qt < pt) {
              sh_state = 1;  // accept
            } else {
              sh_state = 2;  // reject: the residual uses C' = C + N s for the tokens still in q
              sh_Cold = sh_C;
              sh_C = sh_C + sh_N * sh_s;
            }
          }
        }
        __syncthreads();
        if (sh_state != 2 || sh_err) break;
        const bool badq = scan_slice(true);
        if (xrow >= a.part_rows) {
          if (tid == 0) sh_fail = 1;
          break;
        }
        Slot* xs = part + xrow * NW;
        ++xrow;
        if (tid == kThreads - 1) {
          Rec r;
          r.m = 0.f;
          r.idx = badq ? -1 : 0;
          r.z = incl;  // slice mass: the last thread's inclusive sum
          put_slot(&xs[wg], r, tag);
        }
        if (wave == 0) {
          const Slot* const rows1[1] = {xs};
          Rec rr[1];
          get_slots<1>(rows1, 1, NW, tag, Rec{0.f, 0, 0.0}, rr, &sh_fail);
          const Rec r = rr[0];
          s_lastmass[lane] = r.z;  // kept for the final draw
          const double tot = wave_incl_scan(r.z);
          const bool anybad = __any(lane < NW && r.idx < 0);
          if (lane == 63) {
            if (anybad) sh_err |= SPEC_DEV_NONFINITE;
            if (tot > 0.0) {
              sh_N = tot;
            } else {
              sh_C = sh_Cold;  // zero residual mass: p~ stays as it was
            }
            if (a.wr) {
              const int x = sh_x;
              int k = 0;
              while (k < sh_nrej && rej_tok[k] != x) ++k;
              if (k == sh_nrej) {
                const double q_old = sh_s * static_cast<double>(s_qx[sh_c]);
                rej_tok[sh_nrej] = x;
                rej_c[sh_nrej] = sh_C;
                ++sh_nrej;
                if (q_old < 1.0) sh_s = sh_s / (1.0 - q_old);
              }
            }
            sh_total = tot;
            sh_c = next_sib[sh_c];
          }
        }
        __syncthreads();
        if (sh_fail) break;
        scanned = sh_total > 0.0;
      }
      if (sh_err || sh_fail) break;
      if (sh_state == 1) {
        if (tid == 0) {
          s_path[sh_len++] = sh_c;
          sh_u = sh_c;
        }
        __syncthreads();
        continue;
      }
      // final draw at u: inverse CDF of the current weights in index order
      const bool bonus = (sh_C == 0.0 && sh_nrej == 0);  // no rejection here: the weights are p
      if (!scanned) {
        scan_slice(false);
        if (!bonus) {  // a zero-mass residual left earlier weights in place: publish them
          if (xrow >= a.part_rows) {
            if (tid == 0) sh_fail = 1;
            break;
          }
          Slot* xs = part + xrow * NW;
          ++xrow;
          if (tid == kThreads - 1) put_slot(&xs[wg], Rec{0.f, 0, incl}, tag);
          if (wave == 0) {
            const Slot* const rows1[1] = {xs};
            Rec rr[1];
            get_slots<1>(rows1, 1, NW, tag, Rec{0.f, 0, 0.0}, rr, &sh_fail);
            s_lastmass[lane] = rr[0].z;
          }
          __syncthreads();
          if (sh_fail) break;
        }
      }
      if (a.trunc && !scanned && bonus && wave == 0 && !s_tsh[er]) {  // this row's shares, from its lists
        if (er < E)
          row_shares(er, reinterpret_cast<uint32_t*>(cur_lbuf) + er * NBe * LWe, NBe, a.q_e, LWe,
                     reinterpret_cast<float*>(row_partials));
        else
          row_shares(er, reinterpret_cast<uint32_t*>(eager_l), s_dnb, s_dq, s_dlw, reinterpret_cast<float*>(row_partials));
      }
      if (wave == 0) {
        double mass = 0.0;
        if (scanned || !bonus) {  // the masses gathered by the last exchange
          mass = s_lastmass[lane];
        } else if (lane < NW) {
          mass = e_mass[er * kMaxTeam + lane];
        }
        const double inc = wave_incl_scan(mass);
        const double exc = wave_shift_up(inc, 0.0);
        const double total = readlane_d(inc, 63);
        const double uu = s_fu[u];
        const double target = uu * total;
        const bool here = lane < NW && exc <= target && target < inc;
        const unsigned long long hit = __ballot(here);
        const unsigned long long nz = __ballot(lane < NW && mass > 0.0);
        const int owner = hit ? (__ffsll(static_cast<long long>(hit)) - 1)
                              : (nz ? (63 - __clzll(static_cast<long long>(nz))) : 0);
        const double lo = readlane_d(exc, owner);
        if (lane == 0) {
          if (!(total > 0.0)) sh_err |= SPEC_DEV_EMPTY;
          sh_owner = owner;
          sh_lo = lo;
          sh_target = target;
        }
      }
      __syncthreads();
      if (wg == sh_owner && sh_err == 0) {
        const double t_lo = sh_lo + excl, t_hi = sh_lo + incl;
        const double target = sh_target;
        const bool last_nonempty = i1 > i0 && i1 == n;
        if ((t_lo <= target && target < t_hi) || (last_nonempty && target >= t_hi)) {
          double run = t_lo;
          int pick = -1, lastnz = -1;
          for (int c = c0; c < c1 && pick < 0; ++c) {
            const f32x4 lv = load4<kFits>(cl + 4 * c, n - 4 * c);
            const f32x4 qv = load4<kFits>(cq + 4 * c, n - 4 * c);
            double w[4];
            weight4(lv, qv, c, w);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * c + e;
              if (pick >= 0 || i >= n) continue;
              if (w[e] > 0.0) lastnz = i;
              run += w[e];
              if (run > target) pick = i;
            }
          }
          const int k = pick >= 0 ? pick : lastnz;
          if (k >= 0) sh_emit_local = v0 + k;
        }
      }
      __syncthreads();
      // the drawn token goes to member 0, the only member that writes outputs:
      // the owner publishes it in this exchange's slot, member 0 waits for it
      if (xrow >= a.part_rows) {
        if (tid == 0) sh_fail = 1;
        break;
      }
      Slot* xs = part + xrow * NW;
      ++xrow;
      if (sh_owner != 0 && sh_err == 0) {
        if (wg == sh_owner && tid == 0) put_slot(&xs[wg], Rec{0.f, sh_emit_local, 0.0}, tag);
        if (wg == 0 && wave == 0) {
          const Slot* const one[1] = {xs + sh_owner};
          Rec rr[1];
          get_slots<1>(one, 1, 1, tag, Rec{0.f, -1, 0.0}, rr, &sh_fail);
          if (lane == 0) sh_emit_local = rr[0].idx;
        }
        __syncthreads();
      }
      break;
    }
  }
  __syncthreads();
  if (sh_fail && tid == 0) atomicOr(&sh_err, SPEC_DEV_TIMEOUT);
  __syncthreads();

  // Outputs and compaction: member 0 alone writes every output of the
  // sequence and moves its KV rows, from its own view of the walk, so the
  // results are one member's decisions even when another member's wait ran
  // out (the others write nothing).
  const int err = sh_err;
  const int L = err ? 0 : sh_len - 1;
  if (wg == 0) {
    if (tid == 0) {
      int32_t* acc_b = a.accepted + static_cast<long>(b) * T;
      int32_t* out_b = a.out_tokens + static_cast<long>(b) * T;
      for (int i = 0; i < T; ++i) {
        acc_b[i] = (i == 0) ? 0 : ((!err && i <= L) ? s_path[i] : -1);
        out_b[i] = (!err && i < L) ? s_tok[s_path[i + 1]] : -1;
      }
      if (!err) out_b[L] = a.greedy ? emitted : sh_emit_local;
      a.num_accepted[b] = L;
      report(a.status, b, err);
    }
    if (a.fuse) {
      // KV compaction along the path (s_path[0..L]; L = 0 after a sampler
      // error, which leaves the cache as it is), every kv head, through the
      // (now free) current-row LDS buffer
      if (tid == 0) {
        int first = 1 << 30;
        const int cerr = compact_plan(a.c, b, c_lb, s_path, L, &first);
        sh_c = cerr ? -1 : L;  // the walk is over: its scratch words are free
        sh_x = first;
        if (a.c.new_lens != nullptr) a.c.new_lens[b] = cerr ? c_lb : c_lb + L + 1;
        report(a.status, b, cerr);
      }
      __syncthreads();
      compact_move(a.c, b, 0, a.c.Hkv, c_lb, sh_c, sh_x, s_path, reinterpret_cast<uint8_t*>(cur_lbuf));
    }
  }
  // Leave.  The last workgroup of the grid out resets the exit counter and
  // advances the workspace's epoch, so the next call's tag differs from every
  // tag written before, whatever shape the earlier calls had: a slot is valid
  // only for the call that wrote it.  When the next tag would be 0 (after
  // 2^32 - 1 calls) the epoch starts again at 0, and this workgroup first clears
  // every word of the workspace after the header, so no slot written in an
  // earlier cycle can carry a later tag.
  if (tid == 0) {
    const unsigned prev = atomicAdd(a.hdr, 1u);
    sh_state = (prev == gridDim.x - 1u) ? 1 : 0;
  }
  __syncthreads();
  if (sh_state == 1) {
    unsigned next = epoch + 1u;
    if (next == 0xFFFFFFFFu) {
      next = 0u;
      for (long i = tid; i < a.n_slot_words; i += kThreads)
        __hip_atomic_store(a.slot_words + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (tid == 0) {
      atomicExch(a.hdr, 0u);
      atomicExch(a.hdr + 1, next);
    }
  }
}

}  // namespace

// Exchanges after the eager one: at most one per visited row past the eager
// rows (<= T), one per rejected child (<= T - 1), one final republish and the
// drawn token.
int part_rows(int T) { return 2 * T + 2; }

size_t reject_workspace_bytes(int B, int T, int V) {
  const Team t = team_shape(B, T, V, kUnboundedResidency);  // the largest team any device gets
  return kHeaderBytes + static_cast<size_t>(B) * t.NW * (std::max(t.E, 1) + part_rows(T)) * sizeof(Slot);
}

size_t reject_workspace_zero_bytes() { return kHeaderBytes; }

// Parts a member's slice of n logits is cut into when the selection takes
// `rows` rows at once (a part a wave, four waves a workgroup): long slices are
// split so that their passes run on several waves, while a row keeps at most
// 64 blocks.
static int slice_parts(int n, int rows, int NW) {
  int q = n >= 2048 ? 4 : (n >= 1024 ? 2 : 1);
  while (q > 1 && NW * q > 64) q >>= 1;  // (more blocks make the threshold's union longer than the passes save)
  return std::max(1, std::min(q, kWaves / std::max(rows, 1)));
}

// Length of the first lists of NB blocks for top-k K: about twice a block's
// expected share of the top K plus a margin (so that a second round is rare),
// bounded so that `rows` rows of lists fit `cap` words of the LDS buffer that
// merges them.
static int first_list_len(int NB, int K, int rows, int cap) {
  int kc = std::min(K, (2 * K + NB - 1) / NB + 6);
  while (kc > 1 && rows * NB * (kc + 2) > cap) --kc;
  return kc;
}

struct TruncPlan {
  int kc_e, q_e, kc_d, q_d;
};
static TruncPlan trunc_plan(const Team& t, int K) {
  TruncPlan p;
  p.q_e = slice_parts(t.S, t.E, t.NW);
  p.kc_e = first_list_len(t.NW * p.q_e, K, std::max(t.E, 1), kSliceCap);
  p.q_d = slice_parts(t.S, 1, t.NW);
  p.kc_d = first_list_len(t.NW * p.q_d, K, 1, kEagerCapBig);
  return p;
}

// List blocks per sequence: the eager rows' (at most 8 NW), a row of at most
// 4 NW for each later row, a row of NW for each second round (at most T + 8).
static long list_blocks(int NW, int T) { return static_cast<long>(NW) * (5L * T + 16); }

size_t reject_trunc_workspace_bytes(int B, int T, int V, int top_k) {
  const Team t = team_shape(B, T, V, kUnboundedResidency);  // the largest team any device gets
  const size_t slots = static_cast<size_t>(B) * t.NW * (kMaxEager + part_rows(T)) * sizeof(Slot);
  const size_t lists = static_cast<size_t>(B) * list_blocks(t.NW, T) * (top_k + 2) * sizeof(unsigned long long);
  return kHeaderBytes + slots + lists;
}

void reject_trunc_plan(int B, int T, int V, int top_k, long resident, int* team, int* list_len) {
  const Team t = team_shape(B, T, V, resident);
  *team = t.NW;
  *list_len = trunc_plan(t, top_k).kc_d;
}

// Workgroups of the sampler kernel the current device holds at once: its
// occupancy per CU (LDS bound: one) times the CU count, queried once per
// device.
long reject_resident_capacity() {
  static long cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu[4] = {0, 0, 0, 0};
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu[0], reject_team_kernel<true, kSmallTree>, kThreads, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu[1], reject_team_kernel<false, kSmallTree>, kThreads, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu[2], reject_team_kernel<true, kMaxT>, kThreads, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu[3], reject_team_kernel<false, kMaxT>, kThreads, 0) !=
          hipSuccess)
    return 0;
  const long cap = static_cast<long>(cus) * std::min(std::min(per_cu[0], per_cu[1]), std::min(per_cu[2], per_cu[3]));
  if (dev < 64) cache[dev] = cap;
  return cap;
}

void reject_plan(int B, int T, int V, long resident, int* team, int* slice) {
  const Team t = team_shape(B, T, V, resident);
  *team = t.NW;
  *slice = t.S;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the sampler's workspace as a
// file-scope device array, one copy per GPU, held until the process ends.  It
// starts zero-filled (static storage); every completed call leaves it ready for
// the next call of any shape (the epoch protocol above), so it is never
// cleared again.  In host code `scratch` names a host-side stand-in: its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of this device's copy of `scratch`, looked up at the first
// call on the device; nullptr (with *err set) if the lookup fails.
static void* scratch_address(hipError_t* err) {
  static void* addr[kMaxDevices];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || p == nullptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

size_t reject_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t launch_reject_static(const RejectLaunch& L_in, hipStream_t stream) {
  hipError_t err = hipSuccess;
  void* p = scratch_address(&err);
  if (p == nullptr) return err;
  RejectLaunch L = L_in;
  L.workspace = p;
  L.workspace_bytes = kStaticScratchBytes;
  return launch_reject(L, stream);
}

hipError_t launch_reject(const RejectLaunch& L, hipStream_t stream) {
  const long resident = reject_resident_capacity();
  if (resident <= 0) return hipErrorInvalidDevice;
  const Team t = team_shape(L.B, L.T, L.V, resident);
  const bool greedy = (L.temperature == 0.0f);
  TArgs a{};
  a.logits = L.logits;
  a.q = L.q;
  a.tokens = L.tokens;
  a.parent = L.parent;
  a.accepted = L.accepted;
  a.out_tokens = L.out_tokens;
  a.num_accepted = L.num_accepted;
  a.status = L.status;
  a.hdr = static_cast<unsigned*>(L.workspace);
  a.slot_words = reinterpret_cast<unsigned long long*>(static_cast<char*>(L.workspace) + kHeaderBytes);
  a.n_slot_words = static_cast<long>((L.workspace_bytes - kHeaderBytes) / sizeof(unsigned long long));
  a.eager = reinterpret_cast<Slot*>(static_cast<char*>(L.workspace) + kHeaderBytes);
  a.part = a.eager + static_cast<size_t>(L.B) * t.NW * std::max(t.E, 1);
  a.part_rows = part_rows(L.T);
  a.T = L.T;
  a.V = L.V;
  a.NW = t.NW;
  a.S = t.S;
  a.ld = t.ld;
  a.E = t.E;
  a.greedy = greedy;
  a.wr = L.without_replacement ? 1 : 0;
  a.inv_tau = greedy ? 0.0 : 1.0 / static_cast<double>(L.temperature);
  a.seed = L.seed;
  a.offset = L.offset;
  a.fuse = L.compact != nullptr;
  if (a.fuse) a.c = *L.compact;
  a.trunc = (!greedy && L.top_k > 0) ? 1 : 0;
  a.top_k = 1;
  a.kc_e = a.kc_d = a.q_e = a.q_d = 1;
  a.top_p = 1.0;
  if (a.trunc) {
    if (L.top_k > kTopKMax) return hipErrorInvalidValue;
    const TruncPlan tp = trunc_plan(t, L.top_k);
    a.top_k = L.top_k;
    a.kc_e = tp.kc_e;
    a.q_e = tp.q_e;
    a.kc_d = tp.kc_d;
    a.q_d = tp.q_d;
    a.top_p = static_cast<double>(L.top_p);
    a.list_blocks = static_cast<int>(list_blocks(t.NW, L.T));
    a.lists = reinterpret_cast<unsigned long long*>(a.part + static_cast<size_t>(L.B) * a.part_rows * t.NW);
    const size_t used = static_cast<size_t>(reinterpret_cast<char*>(a.lists) - static_cast<char*>(L.workspace)) +
                        static_cast<size_t>(L.B) * a.list_blocks * (a.top_k + 2) * sizeof(unsigned long long);
    if (used > L.workspace_bytes) return hipErrorInvalidValue;
  }
  const dim3 grid(static_cast<unsigned>(L.B * t.NW));
  const bool fits = t.ld <= kSliceCap;
  if (L.T <= kSmallTree) {
    if (fits)
      hipLaunchKernelGGL((reject_team_kernel<true, kSmallTree>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((reject_team_kernel<false, kSmallTree>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (fits)
      hipLaunchKernelGGL((reject_team_kernel<true, kMaxT>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((reject_team_kernel<false, kMaxT>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace spectree
