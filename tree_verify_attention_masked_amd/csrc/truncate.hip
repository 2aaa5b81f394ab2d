// Top-k / top-p truncation of the target logits before the acceptance tests.
//
// The Sequoia summary ("Sequoia: Scalable and Robust Speculative Decoding",
// the top-p robustness table) verifies against a nucleus-truncated target.
// Definitions (outside the pages): top-k keeps the k largest logits (Fan et
// al. 2018), top-p the smallest set of most probable tokens whose mass under
// softmax(logits / temperature) reaches top_p (Holtzman et al. 2020).  As a
// threshold rule, so that equal logits are never split: keep {x : l(x) >= t},
// t the k-th largest logit for top-k and, for top-p, the largest logit value
// v whose set {l >= v} holds at least top_p of the mass.  Both rules: top-k
// first, top-p over the top-k set renormalised.  Temperature 0: the nucleus
// is the set tied at the maximum.  Dropped logits become -inf, so the sampler
// gives them probability 0 everywhere; -inf inputs are outside every set.
//
// One workgroup of 1024 threads per row (sequence b, node u); a row of up to
// 32768 logits is staged in LDS once, longer rows are re-read from global
// memory (L2) in each pass.  The threshold is found by value-domain
// bucketing: the current value range [lo, hi] is cut into 1024 equal buckets
// (bucket index monotone in the value, so the buckets are ordered like the
// values); a histogram of the measure (count for top-k, mass for top-p) and
// its prefix sum find the bucket in which the running measure from the top
// reaches the target.  A bucket of at most 512 elements is finished exactly
// (each candidate sums the measure above and equal to it); a crowded bucket
// becomes the next range.  Masses are exp((l - max)/tau): the exponent in
// fp64, 2^(its fraction) in fp32, the power of two exact (relative error
// about 1e-7 per element), summed in fp64.
#include <math.h>

#include "common.h"

namespace spectree {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = kThreads;  // one bucket per thread in the prefix sum
constexpr int kCand = 512;       // exact finish when the chosen bucket holds at most this many
constexpr int kLdsV = 32768;     // rows up to this length live in LDS (128 KB)
constexpr int kMaxRounds = 64;   // each round narrows the range 1024-fold or ends the search

struct TrArgs {
  const float* in;
  float* out;
  int32_t* status;
  int T, V;
  float tau;
  int top_k;
  float top_p;
  double c;  // log2(e) / tau (tau > 0)
  int in_place;
};

// exp((l - m) / tau) = 2^x with x = (l - m) * log2(e) / tau.
__device__ __forceinline__ double weight(float l, float m, double c) {
  const double x = (static_cast<double>(l) - static_cast<double>(m)) * c;
  if (!(x > -1070.0)) return 0.0;
  const double n = rint(x);
  return ldexp(static_cast<double>(exp2f(static_cast<float>(x - n))), static_cast<int>(n));
}

// Bucket of a value in [lo, hi] (hi > lo): 0 for hi, kBins - 1 for lo;
// non-increasing in the value.
__device__ __forceinline__ int bucket(float l, double hi, double s) {
  const double x = (hi - static_cast<double>(l)) * s;
  return x >= static_cast<double>(kBins - 1) ? kBins - 1 : static_cast<int>(x);
}

struct Shared {
  unsigned cnt[kBins];
  double meas[kBins];  // bucket measure, then its inclusive prefix sum
  float cv[kCand];
  double cm[kCand];
  double red_d[kWaves];
  float red_f[2][kWaves];
  int red_i[2][kWaves];
  int sel, n, found;
  double a_sel;
  float t, tmin;
  float tmax[kThreads];  // per-thread maxima of the row
};

// Sums in a fixed order, so every thread gets the same value on every run.
__device__ __forceinline__ double block_sum(double v, Shared& sh, int lane, int wave) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) sh.red_d[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += sh.red_d[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ void block_minmax(float& mn, float& mx, Shared& sh, int lane, int wave) {
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    sh.red_f[0][wave] = mn;
    sh.red_f[1][wave] = mx;
  }
  __syncthreads();
  mn = INFINITY;
  mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mn = fminf(mn, sh.red_f[0][w]);
    mx = fmaxf(mx, sh.red_f[1][w]);
  }
  __syncthreads();
}

template <bool kLds>
struct Row {
  const float* g;
  const float* s;
  __device__ __forceinline__ float operator[](int i) const {
    if constexpr (kLds) {
      return s[i];
    } else {
      return g[i];
    }
  }
};

// For a candidate value v: the measure of the listed entries above v and equal
// to v, and whether a listed entry lies below v.  The list is padded to a
// multiple of 8 with (-inf, 0), which is never above, equal to or counted
// below a finite v; eight entries are read at a time.
constexpr int kPad = 8;
__device__ __forceinline__ void rank_in_list(const Shared& sh, int ncp, float v, double& a, double& e,
                                             bool& lower) {
  a = 0.0;
  e = 0.0;
  lower = false;
  for (int k = 0; k < ncp; k += kPad) {
    float w[kPad];
    double mm[kPad];
#pragma unroll
    for (int j = 0; j < kPad; ++j) {
      w[j] = sh.cv[k + j];
      mm[j] = sh.cm[k + j];
    }
#pragma unroll
    for (int j = 0; j < kPad; ++j) {
      a += w[j] > v ? mm[j] : 0.0;
      e += w[j] == v ? mm[j] : 0.0;
      lower |= w[j] < v && w[j] != -INFINITY;
    }
  }
}

// f(i, row[i]) for every i < V owned by this thread, kU loads in flight at a
// time (a row's pass would otherwise wait out one memory latency per element).
constexpr int kU = 16;
template <typename R, typename F>
__device__ __forceinline__ void for_row(const R& row, int V, int tid, F&& f) {
  for (int base = 0; base < V; base += kThreads * kU) {
    float v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + j * kThreads + tid;
      v[j] = i < V ? row[i] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = base + j * kThreads + tid;
      if (i < V) f(i, v[j]);
    }
  }
}

// The largest value t in [lo, hi] with measure{lo <= l, l >= t} >= target,
// given that the measure above hi (none, on entry) is below the target.
// mass = false: the measure is the count; true: the mass weight(l, m, c).
// keep_top: when the chosen bucket and everything above it fit the candidate
// list (and nothing lies above the range), gather all of them, so that the
// list then holds every element >= the returned threshold (*listed = count,
// else 0).
template <typename R>
__device__ float select_threshold(const R row, int V, bool mass, double target, float lo, float hi,
                                  float m, double c, Shared& sh, int tid, int lane, int wave, bool keep_top,
                                  int* listed) {
  *listed = 0;
  double above = 0.0;  // measure of the considered elements above the current range
  for (int round = 0; round < kMaxRounds; ++round) {
    if (!(lo < hi)) return lo;  // one value left: the target lies within its measure
    const double dhi = hi, s = static_cast<double>(kBins) / (static_cast<double>(hi) - static_cast<double>(lo));
    sh.cnt[tid] = 0;
    sh.meas[tid] = 0.0;
    if (tid == 0) {
      sh.sel = -1;
      sh.n = 0;
      sh.found = 0;
    }
    __syncthreads();
    for_row(row, V, tid, [&](int, float l) {
      if (l >= lo && l <= hi) {
        const int k = bucket(l, dhi, s);
        atomicAdd(&sh.cnt[k], 1u);
        if (mass) atomicAdd(&sh.meas[k], weight(l, m, c));
      }
    });
    __syncthreads();
    // inclusive prefix sum over the buckets (value-descending order), one bucket per thread
    const unsigned cj = sh.cnt[tid];
    const double mj = mass ? sh.meas[tid] : static_cast<double>(cj);
    double inc = mj;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double u = __shfl_up(inc, o);
      if (lane >= o) inc += u;
    }
    if (lane == 63) sh.red_d[wave] = inc;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += sh.red_d[w];
    inc += off;
    sh.meas[tid] = inc;
    __syncthreads();
    const double exc = tid ? sh.meas[tid - 1] : 0.0;
    if (cj > 0 && above + exc < target && above + inc >= target) {
      sh.sel = tid;
      sh.a_sel = above + exc;
    }
    __syncthreads();
    const int sel = sh.sel;
    const double a_sel = sh.a_sel;
    const unsigned n = sel >= 0 ? sh.cnt[sel] : 0u;
    __syncthreads();  // read by everyone before they change
    if (sel < 0) return lo;  // rounding left the target above the whole range: keep all of it
    const bool whole = keep_top && above == 0.0 && a_sel + n <= static_cast<double>(kCand);
    above = whole ? 0.0 : a_sel;
    // value bounds of the chosen bucket, one bucket width wider on each side: a
    // single compare drops nearly every element before the exact bucket test
    float vlo = static_cast<float>(dhi - (sel + 2.0) / s);
    if (static_cast<double>(vlo) > dhi - (sel + 2.0) / s) vlo = nextafterf(vlo, -INFINITY);
    float vhi = static_cast<float>(dhi - (sel - 1.0) / s);
    if (static_cast<double>(vhi) < dhi - (sel - 1.0) / s) vhi = nextafterf(vhi, INFINITY);
    if (whole) vhi = INFINITY;
    if (n <= static_cast<unsigned>(kCand)) {
      for_row(row, V, tid, [&](int, float l) {
        if (l >= vlo && l <= vhi && l >= lo && l <= hi &&
            (whole ? bucket(l, dhi, s) <= sel : bucket(l, dhi, s) == sel)) {
          const int k = atomicAdd(&sh.n, 1);
          if (k < kCand) {  // always: the same test counted at most kCand of them
            sh.cv[k] = l;
            sh.cm[k] = mass ? weight(l, m, c) : 1.0;
          }
        }
      });
      __syncthreads();
      const int nc = min(sh.n, kCand);
      const int ncp = (nc + kPad - 1) / kPad * kPad;
      if (tid >= nc && tid < ncp) {
        sh.cv[tid] = -INFINITY;
        sh.cm[tid] = 0.0;
      }
      __syncthreads();
      if (tid < nc) {
        const float v = sh.cv[tid];
        double a, e;
        bool lower;
        rank_in_list(sh, ncp, v, a, e, lower);
        if (above + a < target && above + a + e >= target) {
          sh.t = v;  // every candidate equal to v writes the same value
          sh.found = 1;
        }
        if (!lower) sh.tmin = v;
      }
      __syncthreads();
      const float res = sh.found ? sh.t : sh.tmin;  // not found: rounding again, keep the whole bucket
      __syncthreads();
      if (whole) *listed = nc;
      return res;
    }
    // crowded bucket: its elements' range is the next range
    float nlo = INFINITY, nhi = -INFINITY;
    for_row(row, V, tid, [&](int, float l) {
      if (l >= vlo && l <= vhi && l >= lo && l <= hi && bucket(l, dhi, s) == sel) {
        nlo = fminf(nlo, l);
        nhi = fmaxf(nhi, l);
      }
    });
    block_minmax(nlo, nhi, sh, lane, wave);
    lo = nlo;
    hi = nhi;
  }
  return lo;
}

template <bool kLds>
__global__ __launch_bounds__(kThreads) void truncate_kernel(const TrArgs a) {
  __shared__ float s_row[kLds ? kLdsV : 1];
  __shared__ Shared sh;
  const long r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V;
  const float* in = a.in + r * V;
  float* out = a.out + r * V;
  Row<kLds> row{in, s_row};

  // pass 1: stage the row, its finite range, its finite count, NaN / +inf
  float mn = INFINITY, mx = -INFINITY;
  int nfin = 0, bad = 0;
  for_row(in, V, tid, [&](int i, float l) {
    if constexpr (kLds) s_row[i] = l;
    bad |= (isnan(l) || l == INFINITY) ? 1 : 0;
    if (l != -INFINITY) {
      mn = fminf(mn, l);
      mx = fmaxf(mx, l);
      ++nfin;
    }
  });
#pragma unroll
  for (int o = 32; o; o >>= 1) {
    nfin += __shfl_xor(nfin, o);
    bad |= __shfl_xor(bad, o);
  }
  if (lane == 0) {
    sh.red_i[0][wave] = nfin;
    sh.red_i[1][wave] = bad;
  }
  const float my_max = mx;               // this thread's largest finite logit (-inf if none)
  block_minmax(mn, mx, sh, lane, wave);  // its barriers also publish red_i
  nfin = 0;
  bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    nfin += sh.red_i[0][w];
    bad |= sh.red_i[1][w];
  }

  float t = -INFINITY;  // keep l >= t
  if (bad) {
    if (tid == 0) report(a.status, static_cast<int>(r / a.T), SPEC_DEV_NONFINITE);
  } else if (nfin > 0) {
    int listed = 0;  // > 0: the candidate list holds every element >= t
    if (a.top_k > 0 && a.top_k < nfin) {
      bool done = false;
      if (a.top_k <= kThreads) {
        // The k-th largest of the per-thread maxima bounds the k-th largest logit from below
        // (those k maxima are k elements of the row).  When every logit at or above the
        // bound fits the candidate list, the threshold is read off the list, which then
        // holds the whole top; otherwise the search below runs over the row.
        sh.tmax[tid] = my_max;
        __syncthreads();
        int unused;
        const float bound = select_threshold(Row<true>{nullptr, sh.tmax}, kThreads, false,
                                             static_cast<double>(a.top_k), mn, mx, mx, a.c, sh, tid, lane, wave,
                                             false, &unused);
        if (tid == 0) sh.n = 0;
        __syncthreads();
        for_row(row, V, tid, [&](int, float l) {
          if (l >= bound) {
            const int k = atomicAdd(&sh.n, 1);
            if (k < kCand) sh.cv[k] = l;
          }
        });
        __syncthreads();
        const int n = sh.n;
        if (n <= kCand) {
          const int ncp = (n + kPad - 1) / kPad * kPad;
          if (tid < ncp) sh.cm[tid] = tid < n ? 1.0 : 0.0;
          if (tid >= n && tid < ncp) sh.cv[tid] = -INFINITY;
          if (tid == 0) sh.found = 0;
          __syncthreads();
          if (tid < n) {
            double above, eq;
            bool lower;
            rank_in_list(sh, ncp, sh.cv[tid], above, eq, lower);
            const double k = static_cast<double>(a.top_k);
            if (above < k && above + eq >= k) {
              sh.t = sh.cv[tid];
              sh.found = 1;
            }
          }
          __syncthreads();
          t = sh.found ? sh.t : bound;  // always found: the list holds every logit >= the k-th largest
          listed = (a.top_p < 1.0f && a.tau > 0.0f) ? n : 0;
          __syncthreads();
          done = true;
        }
      }
      if (!done) {
        t = select_threshold(row, V, false, static_cast<double>(a.top_k), mn, mx, mx, a.c, sh, tid, lane, wave,
                             a.top_p < 1.0f && a.tau > 0.0f, &listed);
      }
    }
    if (a.top_p < 1.0f) {
      if (a.tau == 0.0f) {
        t = mx;
      } else if (listed > 0) {
        // top-p over the top-k set, all of it in the list: masses, their sum, and
        // each candidate's mass above and equal to it
        if (tid < listed) sh.cm[tid] = sh.cv[tid] >= t ? weight(sh.cv[tid], mx, a.c) : 0.0;
        __syncthreads();
        const double z = block_sum(tid < listed ? sh.cm[tid] : 0.0, sh, lane, wave);
        const double target = static_cast<double>(a.top_p) * z;
        if (tid == 0) sh.found = 0;
        __syncthreads();
        if (tid < listed && sh.cv[tid] >= t) {
          const float v = sh.cv[tid];
          double above, eq;
          bool lower;
          rank_in_list(sh, (listed + kPad - 1) / kPad * kPad, v, above, eq, lower);
          if (above < target && above + eq >= target) {
            sh.t = v;
            sh.found = 1;
          }
        }
        __syncthreads();
        if (sh.found) t = sh.t;  // not found: rounding left top_p above the total, keep the top-k set
        __syncthreads();
      } else {
        const float lo = t == -INFINITY ? mn : t;
        double z = 0.0;
        for_row(row, V, tid, [&](int, float l) {
          if (l >= lo) z += weight(l, mx, a.c);
        });
        z = block_sum(z, sh, lane, wave);
        int unused;
        t = select_threshold(row, V, true, static_cast<double>(a.top_p) * z, lo, mx, mx, a.c, sh, tid,
                                   lane, wave, false, &unused);
      }
    }
  }
  // write: dropped entries become -inf; out of place, the kept ones are copied
  if (a.in_place) {
    if (t != -INFINITY) {
      for_row(row, V, tid, [&](int i, float l) {
        if (l < t && l != -INFINITY) out[i] = -INFINITY;
      });
    }
  } else {
    for_row(row, V, tid, [&](int i, float l) { out[i] = l < t ? -INFINITY : l; });
  }
}

}  // namespace

hipError_t launch_truncate(const TruncateLaunch& L, hipStream_t stream) {
  TrArgs a{};
  a.in = L.in;
  a.out = L.out;
  a.status = L.status;
  a.T = L.T;
  a.V = L.V;
  a.tau = L.temperature;
  a.top_k = L.top_k;
  a.top_p = L.top_p;
  a.c = L.temperature > 0.0f ? 1.4426950408889634 / static_cast<double>(L.temperature) : 0.0;
  a.in_place = L.in == L.out ? 1 : 0;
  const long rows = static_cast<long>(L.B) * L.T;
  if (rows == 0) return hipSuccess;
  if (L.V <= kLdsV) {
    truncate_kernel<true><<<dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, stream>>>(a);
  } else {
    truncate_kernel<false><<<dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace spectree
