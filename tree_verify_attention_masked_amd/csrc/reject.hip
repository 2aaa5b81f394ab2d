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
// Two kernels:
//   row_stats: per (row, 4096-token chunk) the max logit and the first index
//     holding it, and sum exp((l - max) / temperature) in fp64.
//   walk: one 1024-thread workgroup per sequence walks the tree.  The target
//     row of the current node is p(x) = exp((l_x - m) / t) / Z.  The residual
//     after j rejections is kept in closed form,
//         p~_j(x) = max(p(x) - C_j(x) q(x), 0) / N_j,
//     with one coefficient C_j for every token not yet removed from q and a
//     frozen coefficient for each removed token (at most one per rejected
//     sibling), and q~_j(x) = s_j q(x) for tokens still in q.  Each rejection
//     costs one vocabulary-wide fp64 reduction for N_{j+1}; no V-sized state
//     is stored.  Decisions are taken in fp64.
// Uniforms come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with
// key (seed lo, seed hi) and counter (node, b, purpose + 2*(offset >> 32),
// offset lo); u = (word0 >> 8) * 2^-24.
#include "common.h"

namespace spectree {
namespace {

constexpr int kChunk = 4096;
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;

struct RowStat {
  float m;   // max logit of the chunk (-inf if all -inf)
  int idx;   // first index holding m; -1 if the chunk holds NaN or +inf
  double z;  // sum over the chunk of exp((l - m) / temperature)
};

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

// ---------------------------------------------------------------------------
// row statistics
// ---------------------------------------------------------------------------
struct SArgs {
  const float* logits;
  RowStat* stats;
  int V, nchunks, greedy;
  double inv_tau;
};

__global__ __launch_bounds__(256) void row_stats_kernel(const SArgs a) {
  __shared__ float s_m[4];
  __shared__ int s_i[4];
  __shared__ double s_z[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x % a.nchunks;
  const long row = blockIdx.x / a.nchunks;
  const float* lr = a.logits + row * a.V;
  const int x0 = c * kChunk, x1 = min(a.V, x0 + kChunk);

  float mx = -INFINITY;
  int ix = 0x7fffffff;
  bool bad = false;
  for (int x = x0 + tid; x < x1; x += 256) {
    const float v = lr[x];
    bad |= bad_logit(v);
    if (v > mx) {  // strictly greater: a thread keeps its first index of the max
      mx = v;
      ix = x;
    }
  }
  // max with lowest index on ties
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const float om = __shfl_xor(mx, w);
    const int oi = __shfl_xor(ix, w);
    if (om > mx || (om == mx && oi < ix)) {
      mx = om;
      ix = oi;
    }
  }
  bad = __any(bad);
  if (lane == 0) {
    s_m[wave] = mx;
    s_i[wave] = bad ? -1 : ix;
  }
  __syncthreads();
  float m = s_m[0];
  int idx = s_i[0];
  bool anybad = s_i[0] < 0;
  for (int w = 1; w < 4; ++w) {
    anybad |= s_i[w] < 0;
    if (s_m[w] > m || (s_m[w] == m && s_i[w] < idx)) {
      m = s_m[w];
      idx = s_i[w];
    }
  }
  double z = 0.0;
  if (!a.greedy && m != -INFINITY && !anybad) {
    const double md = static_cast<double>(m);
    for (int x = x0 + tid; x < x1; x += 256) z += exp((static_cast<double>(lr[x]) - md) * a.inv_tau);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) z += __shfl_xor(z, w);
    if (lane == 0) s_z[wave] = z;
    __syncthreads();
    z = s_z[0] + s_z[1] + s_z[2] + s_z[3];
  }
  if (tid == 0) {
    RowStat st;
    st.m = m;
    st.idx = anybad ? -1 : (idx == 0x7fffffff ? x0 : idx);
    st.z = z;
    a.stats[row * a.nchunks + c] = st;
  }
}

// ---------------------------------------------------------------------------
// tree walk
// ---------------------------------------------------------------------------
struct WArgs {
  const float* logits;
  const float* q;
  const int32_t* tokens;
  const int32_t* parent;
  const RowStat* stats;
  int32_t* accepted;
  int32_t* out_tokens;
  int32_t* num_accepted;
  int32_t* status;
  int T, V, nchunks, greedy, wr;
  double inv_tau;
  uint64_t seed, offset;
};

__device__ double block_sum(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kWalkWaves; ++w) t += red[w];  // fixed order: every thread gets the same value
  return t;
}

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(const WArgs a) {
  __shared__ int16_t first_child[kMaxT], next_sib[kMaxT];
  __shared__ int s_tok[kMaxT], s_path[kMaxT];
  __shared__ uint32_t rej_bits[kMaxV / 32];
  __shared__ int rej_tok[kMaxT];
  __shared__ double rej_c[kMaxT];
  __shared__ double red[kWalkWaves];
  __shared__ double sh_incl[kWalkWaves];
  __shared__ int sh_err, sh_len, sh_u, sh_c, sh_x, sh_state, sh_nrej, sh_emit;
  __shared__ double sh_m, sh_iz, sh_C, sh_N, sh_s;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int T = a.T, V = a.V;
  const int32_t* par = a.parent + static_cast<long>(b) * T;
  const int32_t* tk = a.tokens + static_cast<long>(b) * T;

  for (int i = tid; i < (V + 31) / 32; i += kWalkThreads) rej_bits[i] = 0u;
  if (tid == 0) {
    int err = 0;
    for (int i = 0; i < T; ++i) {
      first_child[i] = -1;
      next_sib[i] = -1;
      s_tok[i] = tk[i];
    }
    if (par[0] != -1) err |= SPEC_DEV_PARENT;
    for (int i = T - 1; i >= 1; --i) {  // prepend in decreasing order: child lists come out increasing
      const int p = par[i];
      if (p < 0 || p >= i) {
        err |= SPEC_DEV_PARENT;
        continue;
      }
      if (s_tok[i] < 0 || s_tok[i] >= V) err |= SPEC_DEV_TOKEN;
      next_sib[i] = first_child[p];
      first_child[p] = static_cast<int16_t>(i);
    }
    sh_err = err;
    sh_len = 1;
    s_path[0] = 0;
    sh_u = 0;
    sh_emit = -1;
    sh_nrej = 0;
  }
  __syncthreads();

  if (sh_err == 0 && a.greedy) {
    if (tid == 0) {
      int u = 0;
      for (;;) {
        const RowStat* st = a.stats + (static_cast<long>(b) * T + u) * a.nchunks;
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool bad = false;
        for (int c = 0; c < a.nchunks; ++c) {
          bad |= st[c].idx < 0;
          if (st[c].m > best || (st[c].m == best && st[c].idx < bi)) {
            best = st[c].m;
            bi = st[c].idx;
          }
        }
        if (bad) {
          sh_err |= SPEC_DEV_NONFINITE;
          break;
        }
        int c = first_child[u];
        while (c >= 0 && s_tok[c] != bi) c = next_sib[c];
        if (c < 0) {
          sh_emit = bi;
          break;
        }
        s_path[sh_len++] = c;
        u = c;
      }
    }
  } else if (sh_err == 0) {
    for (;;) {  // one iteration per visited node
      if (tid == 0) {
        const int u = sh_u;
        const RowStat* st = a.stats + (static_cast<long>(b) * T + u) * a.nchunks;
        float m = -INFINITY;
        bool bad = false;
        for (int c = 0; c < a.nchunks; ++c) {
          bad |= st[c].idx < 0;
          m = fmaxf(m, st[c].m);
        }
        double z = 0.0;
        for (int c = 0; c < a.nchunks; ++c)
          if (st[c].m != -INFINITY) z += st[c].z * exp((static_cast<double>(st[c].m) - m) * a.inv_tau);
        if (bad) sh_err |= SPEC_DEV_NONFINITE;
        if (!(z > 0.0)) sh_err |= SPEC_DEV_EMPTY;
        sh_m = m;
        sh_iz = 1.0 / z;
        sh_C = 0.0;
        sh_N = 1.0;
        sh_s = 1.0;
        for (int k = 0; k < sh_nrej; ++k) rej_bits[rej_tok[k] >> 5] &= ~(1u << (rej_tok[k] & 31));
        sh_nrej = 0;
        sh_c = first_child[u];
      }
      __syncthreads();
      if (sh_err) break;
      const float* lrow = a.logits + (static_cast<long>(b) * T + sh_u) * V;
      const float* qrow = a.q + (static_cast<long>(b) * T + sh_u) * V;
      // try the children of u in turn
      for (;;) {
        if (tid == 0) {
          const int c = sh_c;
          if (c < 0) {
            sh_state = 0;  // no untried child: final draw at u
          } else {
            const int x = s_tok[c];
            const double px = exp((static_cast<double>(lrow[x]) - sh_m) * a.inv_tau) * sh_iz;
            const float qf = qrow[x];
            if (isnan(qf)) sh_err |= SPEC_DEV_NONFINITE;
            const double qx = static_cast<double>(qf);
            const bool removed = (rej_bits[x >> 5] >> (x & 31)) & 1u;
            double cx = sh_C;
            if (removed)
              for (int k = 0; k < sh_nrej; ++k)
                if (rej_tok[k] == x) cx = rej_c[k];
            const double ax = fmax(px - cx * qx, 0.0);
            const double pt = ax / sh_N;
            const double qt = removed ? 0.0 : sh_s * qx;
            const double r = draw_uniform(a.seed, a.offset, b, c, 0);
            sh_x = x;
            sh_state = (r * qt < pt) ? 1 : 2;  // 1 accept, 2 reject
          }
        }
        __syncthreads();
        if (sh_state != 2 || sh_err) break;
        // residual after rejecting sh_x: C' = C + N s for tokens still in q
        const double Cp = sh_C + sh_N * sh_s;
        const double iz = sh_iz, m = sh_m;
        double part = 0.0;
        bool badq = false;
        for (int x = tid; x < V; x += kWalkThreads) {
          const float qf = qrow[x];
          badq |= isnan(qf);
          const double p = exp((static_cast<double>(lrow[x]) - m) * a.inv_tau) * iz;
          part += fmax(p - Cp * static_cast<double>(qf), 0.0);
        }
        if (badq) sh_err |= SPEC_DEV_NONFINITE;  // benign race: every writer sets the same bit
        const double mass = block_sum(part, red);
        if (tid == 0) {
          double tot = mass;
          for (int k = 0; k < sh_nrej; ++k) {  // removed tokens keep their frozen coefficient
            const int y = rej_tok[k];
            const double py = exp((static_cast<double>(lrow[y]) - m) * a.inv_tau) * iz;
            const double qy = static_cast<double>(qrow[y]);
            tot += fmax(py - rej_c[k] * qy, 0.0) - fmax(py - Cp * qy, 0.0);
          }
          if (tot > 0.0) {
            sh_C = Cp;
            sh_N = tot;
          }
          if (a.wr) {
            const int x = sh_x;
            const bool removed = (rej_bits[x >> 5] >> (x & 31)) & 1u;
            if (!removed) {
              const double q_old = sh_s * static_cast<double>(qrow[x]);
              rej_bits[x >> 5] |= 1u << (x & 31);
              rej_tok[sh_nrej] = x;
              rej_c[sh_nrej] = sh_C;
              ++sh_nrej;
              if (q_old < 1.0) sh_s = sh_s / (1.0 - q_old);
            }
          }
          sh_c = next_sib[sh_c];
        }
        __syncthreads();
      }
      if (sh_err) break;
      if (sh_state == 1) {
        if (tid == 0) {
          s_path[sh_len++] = sh_c;
          sh_u = sh_c;
        }
        __syncthreads();
        continue;
      }
      // final draw at u: inverse CDF of w(x) = max(p(x) - C(x) q(x), 0) in index order
      const double uu = draw_uniform(a.seed, a.offset, b, sh_u, 1);
      const int seg = (V + kWalkThreads - 1) / kWalkThreads;
      const int x0 = min(V, tid * seg), x1 = min(V, x0 + seg);
      const double C = sh_C, iz = sh_iz, m = sh_m;
      auto weight = [&](int x) -> double {
        const double p = exp((static_cast<double>(lrow[x]) - m) * a.inv_tau) * iz;
        double cx = C;
        if ((rej_bits[x >> 5] >> (x & 31)) & 1u)
          for (int k = 0; k < sh_nrej; ++k)
            if (rej_tok[k] == x) cx = rej_c[k];
        return fmax(p - cx * static_cast<double>(qrow[x]), 0.0);
      };
      double mine = 0.0;
      for (int x = x0; x < x1; ++x) mine += weight(x);
      // inclusive scan of the per-thread sums in thread order
      const int lane = tid & 63, wave = tid >> 6;
      double incl = mine;
#pragma unroll
      for (int w = 1; w < 64; w <<= 1) {
        const double o = __shfl_up(incl, w);
        if (lane >= w) incl += o;
      }
      if (lane == 63) sh_incl[wave] = incl;
      __syncthreads();
      double before = 0.0;
      for (int w = 0; w < wave; ++w) before += sh_incl[w];
      double total = 0.0;
      for (int w = 0; w < kWalkWaves; ++w) total += sh_incl[w];
      incl += before;
      double excl = __shfl_up(incl, 1);
      if (lane == 0) excl = before;
      const double target = uu * total;
      if (tid == 0 && !(total > 0.0)) sh_err |= SPEC_DEV_EMPTY;
      if (total > 0.0 && excl <= target && target < incl) {
        double acc = excl;
        int pick = -1, last = -1;
        for (int x = x0; x < x1; ++x) {
          const double w = weight(x);
          if (w > 0.0) last = x;
          acc += w;
          if (acc > target) {
            pick = x;
            break;
          }
        }
        sh_emit = pick >= 0 ? pick : last;
      }
      __syncthreads();
      break;
    }
  }
  __syncthreads();

  if (tid == 0) {
    int32_t* acc_b = a.accepted + static_cast<long>(b) * T;
    int32_t* out_b = a.out_tokens + static_cast<long>(b) * T;
    const int err = sh_err;
    const int L = err ? 0 : sh_len - 1;
    for (int i = 0; i < T; ++i) {
      acc_b[i] = (i <= L) ? (err ? (i == 0 ? 0 : -1) : s_path[i]) : -1;
      out_b[i] = -1;
    }
    if (!err) {
      for (int d = 1; d <= L; ++d) out_b[d - 1] = s_tok[s_path[d]];
      out_b[L] = sh_emit;
    }
    a.num_accepted[b] = L;
    report(a.status, b, err);
  }
}

}  // namespace

size_t reject_workspace_bytes(int B, int T, int V) {
  const int nchunks = (V + kChunk - 1) / kChunk;
  return static_cast<size_t>(B) * T * nchunks * sizeof(RowStat);
}

hipError_t launch_reject(const RejectLaunch& L, hipStream_t stream) {
  const int nchunks = (L.V + kChunk - 1) / kChunk;
  const bool greedy = (L.temperature == 0.0f);
  const double inv_tau = greedy ? 0.0 : 1.0 / static_cast<double>(L.temperature);
  RowStat* stats = static_cast<RowStat*>(L.workspace);
  SArgs s{};
  s.logits = L.logits;
  s.stats = stats;
  s.V = L.V;
  s.nchunks = nchunks;
  s.greedy = greedy;
  s.inv_tau = inv_tau;
  const long rows = static_cast<long>(L.B) * L.T;
  hipLaunchKernelGGL(row_stats_kernel, dim3(static_cast<unsigned>(rows * nchunks)), dim3(256), 0, stream, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  WArgs w{};
  w.logits = L.logits;
  w.q = L.q;
  w.tokens = L.tokens;
  w.parent = L.parent;
  w.stats = stats;
  w.accepted = L.accepted;
  w.out_tokens = L.out_tokens;
  w.num_accepted = L.num_accepted;
  w.status = L.status;
  w.T = L.T;
  w.V = L.V;
  w.nchunks = nchunks;
  w.greedy = greedy;
  w.wr = L.without_replacement ? 1 : 0;
  w.inv_tau = inv_tau;
  w.seed = L.seed;
  w.offset = L.offset;
  hipLaunchKernelGGL(walk_kernel, dim3(static_cast<unsigned>(L.B)), dim3(kWalkThreads), 0, stream, w);
  return hipGetLastError();
}

}  // namespace spectree
