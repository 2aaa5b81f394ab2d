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
                                            int step, float (&mx)[NR], int (&ix)[NR], double (&z)[NR]) {
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
      mx[r] = cm[r];
    }
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
  scan_chunks<R, kLds>(rows, ld, n, v0, inv_tau, tid, nc, kThreads, mx, ix, z);
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
    scan_chunks<RPW, true>(rows + min(wave, E - 1) * ld, kWaves * ld, n, v0, inv_tau, lane, nc, 64, mx, ix, z);
  else
    scan_chunks<RPW, true>(rows + min(wave, E - 1) * ld, 0, n, v0, inv_tau, lane, nc, 64, mx, ix, z);
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
          slice_stats_rows<1, true>(eager_l, ld, n, v0, a.greedy, a.inv_tau, s_rec, cur_lbuf);
          break;
        case 2:
          slice_stats_rows<2, true>(eager_l, ld, n, v0, a.greedy, a.inv_tau, s_rec, cur_lbuf);
          break;
        case 4:
        case 3:
          slice_stats_rows_by_wave<4>(eager_l, ld, n, v0, a.greedy, a.inv_tau, E, s_rec);
          break;
        default:  // 5 to 8
          slice_stats_rows_by_wave<8>(eager_l, ld, n, v0, a.greedy, a.inv_tau, E, s_rec);
          break;
      }
      if (tid < E) put_slot(&eager[wg * E + tid], s_rec[tid], tag);
      const float lx = lg_b[off];
      const float qx = (a.greedy ? lg_b : q_b)[off];
      const float lx2 = two ? lg_b[off2] : 0.f;
      const float qx2 = two ? (a.greedy ? lg_b : q_b)[off2] : 0.f;
      // gather every member's eager rows (wave w: rows w and w + 4) and merge them, member order
      const Rec none = Rec{-INFINITY, 0x7fffffff, 0.0};
      if (wave + kWaves < E) {
        const Slot* const rows2[2] = {eager + wave, eager + wave + kWaves};
        Rec rr[2];
        get_slots<2>(rows2, E, NW, tag, none, rr, &sh_fail);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          merge_row(rr[h], lane < NW, a.greedy, a.inv_tau, &e_m[wave + h * kWaves], &e_iz[wave + h * kWaves],
                    &e_arg[wave + h * kWaves], &e_err[wave + h * kWaves], &e_mass[(wave + h * kWaves) * kMaxTeam]);
      } else if (wave < E) {
        const Slot* const rows1[1] = {eager + wave};
        Rec rr[1];
        get_slots<1>(rows1, E, NW, tag, none, rr, &sh_fail);
        merge_row(rr[0], lane < NW, a.greedy, a.inv_tau, &e_m[wave], &e_iz[wave], &e_arg[wave], &e_err[wave],
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
        slice_stats_rows<1, kFits>(cl, ld, n, v0, a.greedy, a.inv_tau, s_rec, row_partials);
        if (xrow >= a.part_rows) {  // more exchanges than planned: cannot happen for a valid tree
          if (tid == 0) sh_fail = 1;
          break;
        }
        Slot* xs = part + xrow * NW;
        ++xrow;
        if (tid == 0) put_slot(&xs[wg], s_rec[0], tag);
        if (wave == 0) {
          const Slot* const rows1[1] = {xs};
          Rec r[1];
          get_slots<1>(rows1, 1, NW, tag, Rec{-INFINITY, 0x7fffffff, 0.0}, r, &sh_fail);
          merge_row(r[0], lane < NW, a.greedy, a.inv_tau, &e_m[kMaxEager], &e_iz[kMaxEager], &e_arg[kMaxEager],
                    &e_err[kMaxEager], &e_mass[kMaxEager * kMaxTeam]);
        }
        __syncthreads();
        if (sh_fail) break;
      }
      const int er = u < E ? u : kMaxEager;  // this row's merged statistics
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
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (static_cast<double>(lv[e]) - m) * a.inv_tau;
        exp_lockstep<4>(w);
        const double C = sh_C;
        const int nrej = sh_nrej;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] *= iz;
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
            const double px = exp1((static_cast<double>(s_lx[c]) - m) * a.inv_tau) * iz;
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
