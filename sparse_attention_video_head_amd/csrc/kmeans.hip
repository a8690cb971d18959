// k-means over the Q tokens or the K tokens of every head ("Sparse VideoGen2"
// wiki summary, Method, stage (1); Key claims, §4.3 / Fig. 7(a)):
//   * k-means++ seeding (Arthur & Vassilvitskii 2007) when no cached
//     centroids are given,
//   * Lloyd rounds: assignment to the nearest centroid, then centroid = mean of
//     its members (the counting sort of sort.hip groups the members).
#include <limits.h>

#include <algorithm>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

// ======================================================================
// k-means++ seeding
// ======================================================================
// Counter-based uniforms: splitmix64 (Steele, Lea & Flood, OOPSLA 2014), one
// output of the state seed ^ (problem * 2^32 + pick), top 53 bits * 2^-53.
__device__ __forceinline__ uint64_t splitmix64_dev(uint64_t state) {
  uint64_t z = state + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double seed_uniform(uint64_t seed, int problem, int pick) {
  const uint64_t x = seed ^ (((uint64_t)(uint32_t)problem << 32) + (uint64_t)(uint32_t)pick);
  return (double)(splitmix64_dev(x) >> 11) * 0x1.0p-53;
}


// ||x - c||^2 as the fp64 sum of fp64 squared differences: the differences of
// bf16 or fp32 values are exact in fp64, and so are the squares of bf16
// differences, so the result equals the plain fp64 definition up to the
// order of the additions.  `c` holds the centre in fp64.
template <typename T, int D> struct ExactDist;
template <int D> struct ExactDist<uint16_t, D> {
  static __device__ __forceinline__ double run(const uint16_t* x, const double* c) {
    const u32x4_t* xv = reinterpret_cast<const u32x4_t*>(x);
    double acc = 0.0;
#pragma unroll 4
    for (int q = 0; q < D / 8; ++q) {
      const u32x4_t v = xv[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d0 = (double)bf16_lo(v[e]) - c[8 * q + 2 * e];
        const double d1 = (double)bf16_hi(v[e]) - c[8 * q + 2 * e + 1];
        acc = fma(d0, d0, acc);
        acc = fma(d1, d1, acc);
      }
    }
    return acc;
  }
};
template <int D> struct ExactDist<float, D> {
  static __device__ __forceinline__ double run(const float* x, const double* c) {
    double acc = 0.0;
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
      const double df = (double)x[e] - c[e];
      acc = fma(df, df, acc);
    }
    return acc;
  }
};

// k-means++ runs as two kernels per pick so that every problem's tokens are
// spread over the whole chip and the kernel boundaries order the picks:
//   k_seed_update(k)  all tokens: D2 = min(D2, ||x - c_k||^2), then 256-token
//                     block sums of D2 (4 consecutive tokens per lane);
//   k_seed_sample(k)  one work-group per problem: pick k+1 by inverse-CDF
//                     sampling over the block sums, then the distances from
//                     pick k+1 to every earlier pick for the next update.
// Per token the state is D2 (exact fp64) and the nearest pick's number as a
// 16-bit index (n <= 4096; 10 bytes, streamed once per pick).  A pick c can lower D2(x) only if ||c - c_near||^2 < 4 D2(x)
// (triangle inequality, Elkan 2003), so other tokens are skipped without
// reading x; the skip leaves D2 equal to evaluating every token.  The tokens
// that pass the test (typically 10-30%, scattered over nearly every wave) are
// compacted per work-group and each candidate row is read by 16 lanes, so
// only candidate rows are fetched and no lane idles on a skipped token.
constexpr int kSeedTPL = 4;
constexpr int kSeedBlk = kWave * kSeedTPL;            // 256 tokens per sampling block
constexpr int kSeedWavesPerWG = 4;
constexpr int kSeedWG = kSeedWavesPerWG * kSeedBlk;   // 1024 tokens per work-group
constexpr int kSeedGroup = 16;                        // lanes per candidate row
constexpr int kSeedUnroll = 4;                        // candidate rows in flight per group
constexpr int kSeedCcLds = 1024;                      // earlier picks whose distances fit the LDS copy

__device__ __forceinline__ int first_pick(uint64_t seed, int p, int N) {
  return min((int)(seed_uniform(seed, p, 0) * (double)N), N - 1);
}

// The slice of one row that lane `sub` of a 16-lane group holds: elements
// [sub * E, (sub + 1) * E), E = D / 16, as 32-bit words.
template <typename T, int D> struct RowSlice {
  static constexpr int E = D / kSeedGroup;
  static constexpr int W = E * (int)sizeof(T) / 4;
  static_assert(W == 2 || W % 4 == 0, "slice of 8 or 16k bytes");
  uint32_t w[W];
  __device__ __forceinline__ void load(const T* row, int sub) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(row + sub * E);
    if constexpr (W == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      w[0] = v.x;
      w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < W / 4; ++q) {
        const u32x4_t v = reinterpret_cast<const u32x4_t*>(src)[q];
        w[4 * q] = v[0];
        w[4 * q + 1] = v[1];
        w[4 * q + 2] = v[2];
        w[4 * q + 3] = v[3];
      }
    }
  }
  __device__ __forceinline__ float elem(int e) const {
    if constexpr (sizeof(T) == 2) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    else return __uint_as_float(w[e]);
  }
};

// Sum over the 16 lanes of a group by an xor butterfly.  Each step adds the
// same two values in both partner lanes and IEEE addition commutes, so every
// lane of the group ends with the identical sum.
template <typename F>
__device__ __forceinline__ F group16_sum(F v) {
#pragma unroll
  for (int m = kSeedGroup / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Pick 0: D2 and nearest pick of every token, and the block sums.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_seed_first(
    const T* __restrict__ X, int N, int n, uint64_t seed, double* __restrict__ D2g,
    int32_t* __restrict__ Ag, int32_t* __restrict__ picks, double* __restrict__ bsum,
    float* __restrict__ C0, int32_t* __restrict__ seed_index) {
  __shared__ double s_cd[D];
  const int p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const T* Xp = X + (size_t)p * N * D;
  const int nblk = (N + kSeedBlk - 1) / kSeedBlk;
  const int t = first_pick(seed, p, N);
  for (int e = tid; e < D; e += 256) {
    const float v = Elem<T>::get(Xp, (size_t)t * D + e);
    s_cd[e] = (double)v;
    if (blockIdx.x == 0) C0[(size_t)p * n * D + e] = v;
  }
  if (blockIdx.x == 0 && tid == 0) {
    picks[(size_t)p * n] = t;
    if (seed_index) seed_index[(size_t)p * n] = t;
  }
  __syncthreads();
  const int b = blockIdx.x * kSeedWavesPerWG + wave;
  if (b >= nblk) return;
  const int t0 = b * kSeedBlk + kSeedTPL * lane;
  double d2[kSeedTPL];
#pragma unroll 1
  for (int i = 0; i < kSeedTPL; ++i) {
    d2[i] = 0.0;
    const int tok = t0 + i;
    if (tok < N) {
      const T* xr = Xp + (size_t)tok * D;
      d2[i] = ExactDist<T, D>::run(xr, s_cd);
      D2g[(size_t)p * N + tok] = d2[i];
      reinterpret_cast<uint16_t*>(Ag)[(size_t)p * N + tok] = 0;
    }
  }
  const double lsum = ((d2[0] + d2[1]) + d2[2]) + d2[3];
  const double inc = wave_inclusive_scan(lsum);
  if (lane == kWave - 1) bsum[(size_t)p * nblk + b] = inc;
}

// Pick k >= 1 (its row is already in C0[k]): lower D2 and the nearest pick
// where the new pick is closer, then the block sums.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_seed_update(
    const T* __restrict__ X, int N, int n, int k, double* __restrict__ D2g, int32_t* __restrict__ Ag,
    const float* __restrict__ C0, const double* __restrict__ ccg, double* __restrict__ bsum) {
  using Slice = RowSlice<T, D>;
  constexpr int E = Slice::E;
  constexpr int NG = 256 / kSeedGroup;              // candidate groups per work-group
  constexpr bool kBF16 = sizeof(T) == 2;
  __shared__ float s_c[D];
  __shared__ double s_cd[D];
  __shared__ double s_d2[kSeedWG];
  __shared__ uint16_t s_list[kSeedWG];
  __shared__ double s_cc[kSeedCcLds];
  __shared__ int s_nc;
  const int p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const T* Xp = X + (size_t)p * N * D;
  double* D2 = D2g + (size_t)p * N;
  uint16_t* A = reinterpret_cast<uint16_t*>(Ag) + (size_t)p * N;
  const double* cc = ccg + (size_t)p * n;
  const int nblk = (N + kSeedBlk - 1) / kSeedBlk;

  // ---- the state of this lane's 4 tokens and the skip test; nothing here
  // waits on the new pick's row, so both loads are in flight together
  const int b = blockIdx.x * kSeedWavesPerWG + wave;
  const int tb = blockIdx.x * kSeedWG;               // first token of the work-group
  const int l0 = wave * kSeedBlk + kSeedTPL * lane;  // first local token of the lane
  const int t0 = tb + l0;
  double d2[kSeedTPL];
  int a[kSeedTPL];
  // 16-byte state loads need every problem's arrays 16-byte aligned
  if ((N % kSeedTPL) == 0 && t0 + kSeedTPL <= N) {
    const double2 d01 = *reinterpret_cast<const double2*>(D2 + t0);
    const double2 d23 = *reinterpret_cast<const double2*>(D2 + t0 + 2);
    const uint2 av = *reinterpret_cast<const uint2*>(A + t0);
    d2[0] = d01.x; d2[1] = d01.y; d2[2] = d23.x; d2[3] = d23.y;
    a[0] = (int)(av.x & 0xffffu); a[1] = (int)(av.x >> 16); a[2] = (int)(av.y & 0xffffu); a[3] = (int)(av.y >> 16);
  } else {
#pragma unroll
    for (int i = 0; i < kSeedTPL; ++i) {
      const bool ok = t0 + i < N;
      d2[i] = ok ? D2[t0 + i] : 0.0;
      a[i] = ok ? A[t0 + i] : 0;
    }
  }
  for (int e = tid; e < D; e += 256) {
    const float v = C0[((size_t)p * n + k) * D + e];
    s_c[e] = v;
    s_cd[e] = (double)v;
  }
  // the distances from the new pick to the earlier ones, staged in LDS with
  // the state loads (one memory round trip instead of a dependent gather)
  const bool cc_lds = k <= kSeedCcLds;
  if (cc_lds)
    for (int e = tid; e < k; e += 256) s_cc[e] = cc[e];
  if (tid == 0) s_nc = 0;
#pragma unroll
  for (int i = 0; i < kSeedTPL; ++i) s_d2[l0 + i] = d2[i];
  __syncthreads();
  unsigned m = 0;
#pragma unroll
  for (int i = 0; i < kSeedTPL; ++i) {
    const int ai = clampi(a[i], 0, k - 1);
    const double cai = cc_lds ? s_cc[ai] : cc[ai];
    if (t0 + i < N && cai < 4.0 * d2[i] * (1.0 + 0x1p-20)) m |= 1u << i;
  }
  float cn = 0.f;
  if (kBF16) {
    for (int e = lane; e < D; e += kWave) cn = fmaf(s_c[e], s_c[e], cn);
    cn = wave_sum(cn);
  }
  // ---- compaction of the candidates into s_list
  {
    const int cnt = __popc(m);
    const int inc = wave_inclusive_scan(cnt);
    const int wtot = __shfl(inc, kWave - 1);
    int base = 0;
    if (lane == 0 && wtot > 0) base = atomicAdd(&s_nc, wtot);
    int pos = __shfl(base, 0) + inc - cnt;
#pragma unroll
    for (int i = 0; i < kSeedTPL; ++i)
      if ((m >> i) & 1u) s_list[pos++] = (uint16_t)(l0 + i);
  }
  __syncthreads();

  // ---- candidates: 16 lanes per row, kSeedUnroll rows in flight per group
  const int nc = s_nc;
  const int grp = tid / kSeedGroup, sub = tid % kSeedGroup;
  for (int c0 = grp; c0 < nc; c0 += NG * kSeedUnroll) {
    Slice r[kSeedUnroll];
    int loc[kSeedUnroll];
#pragma unroll
    for (int j = 0; j < kSeedUnroll; ++j) {
      const int ci = c0 + j * NG;
      loc[j] = ci < nc ? (int)s_list[ci] : -1;
      if (loc[j] >= 0) r[j].load(Xp + (size_t)(tb + loc[j]) * D, sub);
    }
#pragma unroll
    for (int j = 0; j < kSeedUnroll; ++j) {
      if (loc[j] < 0) continue;                      // uniform over the group
      const double dv = s_d2[loc[j]];
      bool go = true;
      if (kBF16) {
        // fp32 screen: each bf16 x bf16 product is exact in fp32 and the D
        // additions, in any order, err by at most D 2^-24 sum|x_i c_i|
        // <= D 2^-25 (xn + cn); with the rounding of xn, cn and the final
        // additions the screen is off by less than 2e-5 (xn + cn) at D = 128
        float dot = 0.f, x_n = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xe = r[j].elem(e);
          dot = fmaf(xe, s_c[sub * E + e], dot);
          x_n = fmaf(xe, xe, x_n);
        }
        dot = group16_sum(dot);
        x_n = group16_sum(x_n);
        const float approx = x_n + cn - 2.f * dot;
        go = approx <= (float)dv + 5e-5f * (x_n + cn) + 1e-30f;
      }
      if (go) {
        // exact: differences and squares in fp64, the same order in every run
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double df = (double)r[j].elem(e) - s_cd[sub * E + e];
          acc = fma(df, df, acc);
        }
        acc = group16_sum(acc);
        if (acc < dv && sub == 0) {
          D2[tb + loc[j]] = acc;
          A[tb + loc[j]] = (uint16_t)k;
          s_d2[loc[j]] = acc;
        }
      }
    }
  }
  __syncthreads();

  // ---- block sums of the updated D2 (the same order as for pick 0)
  if (b < nblk) {
    const double lsum = ((s_d2[l0] + s_d2[l0 + 1]) + s_d2[l0 + 2]) + s_d2[l0 + 3];
    const double inc = wave_inclusive_scan(lsum);
    if (lane == kWave - 1) bsum[(size_t)p * nblk + b] = inc;
  }
}

// Pick k+1 of problem blockIdx.x: the smallest token whose running D2 sum
// exceeds u_{k+1} * sum D2 (block sums, then the 256 tokens of the block).
// Then ||c_{k+1} - c_a||^2 for every earlier pick a, from the centroid rows.
// kSampleSplit work-groups per problem take the same (deterministic) pick and
// share the distances; work-group 0 alone writes the pick.  The work-groups are
// small (4 waves) so that they find room on CUs that the other side's update
// kernel still occupies: with the Q and K sides on two streams, one side's
// sampler then overlaps the other side's update.
constexpr int kSampleThreads = 256;
constexpr int kSampleSplit = 8;

template <typename T, int D>
__global__ __launch_bounds__(kSampleThreads) void k_seed_sample(
    const T* __restrict__ X, int N, int n, int k, uint64_t seed, const double* __restrict__ D2g,
    const double* __restrict__ bsum, int32_t* __restrict__ picks, double* __restrict__ ccg,
    float* __restrict__ C0, int32_t* __restrict__ seed_index) {
  __shared__ double s_red[17];
  __shared__ double s_cd[D];
  __shared__ int s_blk, s_last, s_pick;
  __shared__ double s_resid;
  const int p = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const T* Xp = X + (size_t)p * N * D;
  const double* D2 = D2g + (size_t)p * N;
  const int nblk = (N + kSeedBlk - 1) / kSeedBlk;
  const double* bs = bsum + (size_t)p * nblk;
  if (tid == 0) {
    s_blk = INT_MAX;
    s_last = -1;
  }
  const int per = (nblk + kSampleThreads - 1) / kSampleThreads;
  const int b0 = min(tid * per, nblk), b1 = min(b0 + per, nblk);
  double loc = 0.0;
  for (int b = b0; b < b1; ++b) loc += bs[b];
  double total;
  const double excl = block_exclusive_scan(loc, s_red, &total);
  const double u = seed_uniform(seed, p, k + 1);
  const double target = u * total;
  int found = INT_MAX;
  double resid = 0.0;
  if (total > 0.0) {
    double run = excl;
    for (int b = b0; b < b1; ++b) {
      const double nxt = run + bs[b];
      if (found == INT_MAX && run <= target && target < nxt) {
        found = b;
        resid = target - run;
      }
      run = nxt;
    }
    if (found != INT_MAX) atomicMin(&s_blk, found);
    for (int b = b1 - 1; b >= b0; --b)
      if (bs[b] > 0.0) {
        atomicMax(&s_last, b);
        break;
      }
  }
  __syncthreads();
  if (found != INT_MAX && found == s_blk) s_resid = resid;
  __syncthreads();
  if (wave == 0) {
    int pick;
    if (!(total > 0.0)) {
      pick = min((int)(u * (double)N), N - 1);
    } else {
      int b = s_blk;
      bool exact = true;
      if (b == INT_MAX) {
        b = s_last;
        exact = false;
      }
      b = clampi(b, 0, nblk - 1);
      const int t0 = b * kSeedBlk + kSeedTPL * lane;
      double d2[kSeedTPL];
#pragma unroll
      for (int i = 0; i < kSeedTPL; ++i) d2[i] = t0 + i < N ? D2[t0 + i] : 0.0;
      const double lsum = ((d2[0] + d2[1]) + d2[2]) + d2[3];
      const double inc = wave_inclusive_scan(lsum);
      const double before = __shfl_up(inc, 1);
      const double resid_b = s_resid;
      const uint64_t above = exact ? __ballot(inc > resid_b) : 0ull;
      int owner;
      if (above) {
        owner = __ffsll((unsigned long long)above) - 1;
      } else {
        const uint64_t pos = __ballot(lsum > 0.0);
        owner = pos ? 63 - __clzll((long long)pos) : 0;
      }
      int cand = -1, last_pos = -1;
      double run = lane == 0 ? 0.0 : before;
#pragma unroll
      for (int i = 0; i < kSeedTPL; ++i) {
        run += d2[i];
        if (d2[i] > 0.0) last_pos = t0 + i;
        if (cand < 0 && above && run > resid_b) cand = t0 + i;
      }
      if (cand < 0) cand = last_pos;
      pick = __shfl(cand, owner);
    }
    if (lane == 0) s_pick = clampi(pick, 0, N - 1);
  }
  __syncthreads();
  const int t = s_pick;
  for (int e = tid; e < D; e += kSampleThreads) {
    const float v = Elem<T>::get(Xp, (size_t)t * D + e);
    s_cd[e] = (double)v;
    if (blockIdx.y == 0) C0[((size_t)p * n + k + 1) * D + e] = v;
  }
  if (blockIdx.y == 0 && tid == 0) {
    picks[(size_t)p * n + k + 1] = t;
    if (seed_index) seed_index[(size_t)p * n + k + 1] = t;
  }
  __syncthreads();
  // distances from the new pick to picks 0..k from the rows of C0 (which hold
  // the picked tokens exactly): 16 lanes per row, fp64 differences and squares
  constexpr int E = D / kSeedGroup;                 // floats per lane
  const int sub = tid % kSeedGroup;
  const int grp = (tid / kSeedGroup) * kSampleSplit + (int)blockIdx.y;
  constexpr int NG = kSampleThreads / kSeedGroup * kSampleSplit;
  for (int a0 = grp; a0 <= k; a0 += NG * kSeedUnroll) {
    float v[kSeedUnroll][E];
#pragma unroll
    for (int j = 0; j < kSeedUnroll; ++j) {
      const int a = a0 + j * NG;
      if (a <= k) {
        const float* cr = C0 + ((size_t)p * n + a) * D + sub * E;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 f = reinterpret_cast<const float4*>(cr)[q];
          v[j][4 * q] = f.x; v[j][4 * q + 1] = f.y; v[j][4 * q + 2] = f.z; v[j][4 * q + 3] = f.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kSeedUnroll; ++j) {
      const int a = a0 + j * NG;
      if (a > k) break;                              // uniform over the group
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double df = (double)v[j][e] - s_cd[sub * E + e];
        acc = fma(df, df, acc);
      }
      acc = group16_sum(acc);
      if (sub == 0) ccg[(size_t)p * n + a] = acc;
    }
  }
}

hipError_t launch_kmeanspp(const void* x, bool bf16, int bh, int N, int d, int n, uint64_t seed,
                           double* d2_ws, int32_t* near_ws, float* centroids, int32_t* seed_index,
                           int32_t* picks_ws, double* cc_ws, double* bsum_ws, hipStream_t s) {
  const int nblk = (N + kSeedBlk - 1) / kSeedBlk;
  const dim3 ug((nblk + kSeedWavesPerWG - 1) / kSeedWavesPerWG, bh);
#define SVG2_SEED(T, D)                                                                                   \
  for (int k = 0; k < n; ++k) {                                                                         \
    if (k == 0)                                                                                         \
      hipLaunchKernelGGL((k_seed_first<T, D>), ug, dim3(256), 0, s, static_cast<const T*>(x), N, n,     \
                         seed, d2_ws, near_ws, picks_ws, bsum_ws, centroids, seed_index);               \
    else                                                                                                \
      hipLaunchKernelGGL((k_seed_update<T, D>), ug, dim3(256), 0, s, static_cast<const T*>(x), N, n, k, \
                         d2_ws, near_ws, centroids, cc_ws, bsum_ws);                                    \
    if (k + 1 < n)                                                                                      \
      hipLaunchKernelGGL((k_seed_sample<T, D>), dim3(bh, kSampleSplit), dim3(kSampleThreads), 0, s, static_cast<const T*>(x), N, \
                         n, k, seed, d2_ws, bsum_ws, picks_ws, cc_ws, centroids, seed_index);           \
  }
  if (bf16) {
    if (d == 128) { SVG2_SEED(uint16_t, 128) } else { SVG2_SEED(uint16_t, 64) }
  } else {
    if (d == 128) { SVG2_SEED(float, 128) } else { SVG2_SEED(float, 64) }
  }
#undef SVG2_SEED
  return hipGetLastError();
}

// The first Lloyd assignment after k-means++ seeding: the seeding state
// already holds, for every token, the pick nearest to it by the exact fp64
// distance (ties to the earlier pick, i.e. the smaller centroid number), and
// the centroids of that round are exactly the picked rows.  So that round's
// labels are the state's nearest-pick numbers, and the assignment is skipped.
__global__ __launch_bounds__(256) void k_labels_from_picks(const uint16_t* __restrict__ near, size_t total,
                                                           int32_t* __restrict__ labels) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x)
    labels[i] = (int32_t)near[i];
}

hipError_t launch_labels_from_seeding(const int32_t* near_ws, int bh, int N, int32_t* labels, hipStream_t s) {
  const size_t total = (size_t)bh * N;
  const int grid = (int)std::min<size_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(k_labels_from_picks, dim3(grid), dim3(256), 0, s, reinterpret_cast<const uint16_t*>(near_ws),
                     total, labels);
  return hipGetLastError();
}

// ======================================================================
// Lloyd assignment
// ======================================================================
// c = c_hi + c_lo with both halves bf16 (|c - c_hi - c_lo| <= 2^-18 |c|), and
// ||c||^2 in fp32, for the bf16 matrix-core distance contraction.  Each
// problem's rows are padded to a multiple of kCentroidPad: padding rows are
// zero with ||c||^2 = +inf, so they are never the nearest centroid.
__global__ __launch_bounds__(256) void k_prep_centroids(const float* __restrict__ c, int bh, int n, int npad,
                                                        int d, uint16_t* __restrict__ hi,
                                                        uint16_t* __restrict__ lo,
                                                        float* __restrict__ cn, SortStart st) {
  // The round's counting sort starts from zero: the near-tie lists and the
  // chunk histograms the assignment adds its labels to (a grid-stride pass,
  // four ints per store).
  {
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t words = st.hist_words / 4;
    int4* h4 = reinterpret_cast<int4*>(st.hist);
    for (size_t i = gid; i < words; i += nthreads) h4[i] = make_int4(0, 0, 0, 0);
    for (size_t i = words * 4 + gid; i < st.hist_words; i += nthreads) st.hist[i] = 0;
    for (size_t i = gid; i < (size_t)bh; i += nthreads) st.fix_count[i] = 0;
  }
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= bh * npad) return;
  const int p = row / npad, j = row % npad;
  if (j >= n) {
    for (int e = lane; e < d; e += kWave) {
      hi[(size_t)row * d + e] = 0;
      lo[(size_t)row * d + e] = 0;
    }
    if (lane == 0) cn[row] = __builtin_inff();
    return;
  }
  const float* src = c + ((size_t)p * n + j) * d;
  // ||c||^2: the squares of fp32 values are exact in fp64 and the sum of at
  // most 128 of them errs by ~1e-14 relative, so the stored fp32 norm is
  // within one fp32 rounding (2^-24 relative) of the exact one
  double acc = 0.0;
  for (int e = lane; e < d; e += kWave) {
    const float v = src[e];
    const uint16_t h = f32_to_bf16(v);
    const uint16_t l = f32_to_bf16(v - bf16_to_f32(h));
    hi[(size_t)row * d + e] = h;
    lo[(size_t)row * d + e] = l;
    acc = fma((double)v, (double)v, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) cn[row] = (float)acc;
}

hipError_t launch_prep_centroids(const float* c, int bh, int n, int d, uint16_t* c_hi,
                                 uint16_t* c_lo, float* c_norm, const SortStart& st, hipStream_t s) {
  const int npad = centroid_rows(n);
  const int rows = bh * npad;
  hipLaunchKernelGGL(k_prep_centroids, dim3((rows + 3) / 4), dim3(256), 0, s, c, bh, n, npad, d, c_hi, c_lo,
                     c_norm, st);
  return hipGetLastError();
}

// bf16 inputs: argmin_c ||c||^2 - 2 x.c on matrix cores.  The MFMA computes
// S^T = C x X^T (centroids as rows, tokens as columns) so that each lane holds
// 16 centroid distances of ONE token and the argmin is mostly in-lane.
// A work-group holds 512 tokens (4 waves x 4 blocks of 32) in registers and
// streams the centroids through a 4-deep LDS ring of 32-centroid chunks (bf16
// hi and lo rows plus ||c||^2), filled by direct global -> LDS loads three
// chunks ahead; the rows' 16-byte chunks are XOR-swizzled by row % 16 so that
// the operand reads are conflict-free without padding.
//
// Exact labels.  The matrix-core distance of token x to centroid c,
// a(c) = fl(||c||^2) - 2 acc(x, c_hi + c_lo), differs from the exact
// ||c||^2 - 2 x.c by at most
//   E(x) = 2 (2^-18 + g256) (1 + 2^-8) ||x|| cmax + 2u (cmax^2 + ||x|| cmax)
// with u = 2^-24, g256 = 256u / (1 - 256u) (the fp32 accumulation of 256
// exact products in any order), 2^-18 the relative error of c_hi + c_lo, and
// cmax the largest centroid norm of the problem (||c||^2 is rounded once from
// fp64).  So when the second-smallest a exceeds the smallest by more than
// 2E, the smallest is the true nearest centroid.  Otherwise the token is a
// near tie: it is appended, with its smallest a, to the problem's fix list,
// and a second launch of this kernel (FIX) re-walks the centroids for the
// listed tokens, keeps every centroid whose a is within 2E of that smallest
// value (the true nearest is among them), and decides between those with
// exact fp64 distances (ties to the lowest index).
constexpr int kAsgTB = 4;                 // 32-token blocks per wave (the near-tie pass: 1)
constexpr int kAsgCB = kCentroidPad;      // centroids per LDS chunk
constexpr int asg_tb(bool fix) { return fix ? 1 : kAsgTB; }
constexpr int asg_tok(bool fix) { return 4 * asg_tb(fix) * 32; }   // tokens per work-group
constexpr int kFixCand = 16;              // candidate centroids kept per listed token

// s_waitcnt immediates (vmcnt only; expcnt and lgkmcnt not waited for)
constexpr int asg_wait_vm(int n) { return 0xF70 | n; }

__device__ __forceinline__ void lds_barrier_asg() {
  __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}

// Error bound E(x) of a matrix-core distance (see above), rounded up.
__device__ __forceinline__ float asg_error_bound(float xn, float cmax2) {
  const float xnorm = sqrtf(xn) * (1.f + 1e-5f);
  const float cmax = sqrtf(cmax2) * (1.f + 1e-6f);
  return 3.85e-5f * xnorm * cmax + 1.2e-7f * cmax2;
}

struct AsgFix {
  int32_t* count;         // [bh] near ties listed this round
  int32_t* token;         // [bh, N] listed tokens
  float* dmin;            // [bh, N] their smallest matrix-core distance
  const float* C;         // [bh, n, D] fp32 centroids (the exact values)
  int32_t* hist;          // [bh, sort_chunks(N), n] label counts per counting-sort chunk
};

template <int D, bool FIX>
__global__ __launch_bounds__(256, 2) void k_assign_bf16(const uint16_t* __restrict__ X, int N, int n,
                                                        const uint16_t* __restrict__ Chi,
                                                        const uint16_t* __restrict__ Clo,
                                                        const float* __restrict__ Cn,
                                                        int32_t* __restrict__ labels,
                                                        float* __restrict__ min_dist, AsgFix fx) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
  typedef __attribute__((address_space(3))) float lds_f32_t;
  constexpr int KS = D / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = kWave / CPR;           // rows per load instruction
  constexpr int INS = kAsgCB / 4 / RPI;      // load instructions per wave per half
  static_assert(INS >= 1 && kAsgCB == 32, "chunk geometry");
  // ring slot j: hi rows [0, CB*D), lo rows [CB*D, 2*CB*D), then CB norms
  constexpr int SLOT = 2 * kAsgCB * D + 2 * kAsgCB;   // uint16 elements
  constexpr int kAsgTB = asg_tb(FIX);        // this pass's token blocks per wave
  constexpr int kAsgTok = asg_tok(FIX);
  __shared__ __attribute__((aligned(16))) uint16_t sC0[SLOT], sC1[SLOT], sC2[SLOT], sC3[SLOT];
  // FIX: candidate centroids per listed token (token slot = wave, block, column)
  __shared__ int32_t s_cand[FIX ? kAsgTok * kFixCand : 1];
  __shared__ int32_t s_ncand[FIX ? kAsgTok : 1];

  const int p = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 31, half = lane >> 5;
  const uint16_t* Xp = X + (size_t)p * N * D;
  const int npad = centroid_rows(n);
  const int nchunk = npad / kAsgCB;
  const uint16_t* Hp = Chi + (size_t)p * npad * D;
  const uint16_t* Lp = Clo + (size_t)p * npad * D;
  const float* Np = Cn + (size_t)p * npad;
  // FIX: this work-group's share of the list, kAsgTok entries at a time
  const int nfix = FIX ? min(fx.count[p], N) : 0;
  int li0 = FIX ? (int)blockIdx.x * kAsgTok : 0;
  if (FIX && li0 >= nfix) return;

  // this lane's part of a chunk load: row 8 wave + RPI q + lane / CPR,
  // 16-byte slot lane % CPR holding source chunk (lane % CPR) ^ (row % 16)
  uint32_t loff[INS];
#pragma unroll
  for (int q = 0; q < INS; ++q) {
    const int r = 8 * wave + RPI * q + lane / CPR;
    loff[q] = (uint32_t)(r * D + ((lane % CPR) ^ (r & (CPR - 1) & 15)) * 8) * 2u;
  }
  // loads chunk `ch` (clamped to the last one: past the end the slot is
  // filled but never read) into a ring slot
  auto load_chunk = [&](int ch, uint16_t* slot) __attribute__((always_inline)) {
    ch = min(ch, nchunk - 1);
    const uint32_t cbase = (uint32_t)ch * (uint32_t)(kAsgCB * D * 2);
    lds_u16_t* dst = (lds_u16_t*)(lds_void_t*)(void*)slot;
#pragma unroll
    for (int q = 0; q < INS; ++q) {
      lds_u16_t* d = dst + (8 * wave + RPI * q) * D;
      __builtin_amdgcn_global_load_lds((const void*)((const char*)Hp + cbase + loff[q]), (lds_void_t*)d, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)((const char*)Lp + cbase + loff[q]),
                                       (lds_void_t*)(d + kAsgCB * D), 16, 0, 0);
    }
    if (wave == 0 && lane < kAsgCB)
      __builtin_amdgcn_global_load_lds((const void*)(Np + (size_t)ch * kAsgCB + lane),
                                       (lds_void_t*)(dst + 2 * kAsgCB * D), 4, 0, 0);
  };

  for (;;) {
    // tokens of this lane's blocks: consecutive tokens, or (FIX) listed ones
    // with the candidate bound
    const int tok0 = (int)blockIdx.x * kAsgTok + wave * (kAsgTB * 32) + col;
    int tokf[FIX ? kAsgTB : 1];
    float thr[FIX ? kAsgTB : 1];
    auto tok = [&](int tb) __attribute__((always_inline)) -> int {
      if constexpr (FIX) return tokf[tb];
      else return tok0 + tb * 32 < N ? tok0 + tb * 32 : -1;
    };
    if constexpr (FIX) {
#pragma unroll
      for (int tb = 0; tb < kAsgTB; ++tb) {
        const int li = li0 + wave * (kAsgTB * 32) + tb * 32 + col;
        tokf[tb] = li < nfix ? clampi(fx.token[(size_t)p * N + li], 0, N - 1) : -1;
        thr[tb] = li < nfix ? fx.dmin[(size_t)p * N + li] : -__builtin_inff();
      }
    }
    if constexpr (FIX) {
      for (int i = threadIdx.x; i < kAsgTok; i += 256) s_ncand[i] = 0;
    }

    bf16x8_t xb[kAsgTB][KS];
    float xn[kAsgTB];
#pragma unroll
    for (int tb = 0; tb < kAsgTB; ++tb) {
      float acc = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (tok(tb) >= 0) v = *reinterpret_cast<const u32x4_t*>(Xp + (size_t)tok(tb) * D + ks * 16 + half * 8);
        xb[tb][ks] = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = bf16_lo(v[e]), a1 = bf16_hi(v[e]);
          acc = fmaf(a0, a0, fmaf(a1, a1, acc));
        }
      }
      xn[tb] = acc + __shfl_xor(acc, 32);
    }

    float best[kAsgTB], best2[kAsgTB];
    int bidx[kAsgTB];
#pragma unroll
    for (int tb = 0; tb < kAsgTB; ++tb) {
      best[tb] = __builtin_inff();
      best2[tb] = __builtin_inff();
      bidx[tb] = 0;
    }
    // operand row col: its chunk (2 ks + half) sits at (2 ks + half) ^ (col % 16)
    const int arow = col * D, aswz = col & (CPR - 1) & 15;

    auto compute = [&](const uint16_t* slot, int c0) __attribute__((always_inline)) {
      const lds_u16_t* sh = (const lds_u16_t*)(const lds_void_t*)(const void*)slot;
      const lds_f32_t* sn = (const lds_f32_t*)(sh + 2 * kAsgCB * D);
      f32x16_t acc[kAsgTB];
#pragma unroll
      for (int tb = 0; tb < kAsgTB; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[tb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int aoff = arow + (((2 * ks + half) ^ aswz) * 8);
        const bf16x8_t ah = *(const __attribute__((address_space(3))) bf16x8_t*)(sh + aoff);
        const bf16x8_t al = *(const __attribute__((address_space(3))) bf16x8_t*)(sh + kAsgCB * D + aoff);
#pragma unroll
        for (int tb = 0; tb < kAsgTB; ++tb) {
          acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[tb][ks], acc[tb], 0, 0, 0);
          acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[tb][ks], acc[tb], 0, 0, 0);
        }
      }
      // lane (col, half) holds centroid rows (i/4)*8 + half*4 + i%4 of the chunk
#pragma unroll
      for (int tb = 0; tb < kAsgTB; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (i / 4) * 8 + half * 4 + (i % 4);
          const float dist = sn[r] - 2.f * acc[tb][i];
          if constexpr (FIX) {
            if (dist <= thr[tb]) {
              const int ts = wave * (kAsgTB * 32) + tb * 32 + col;
              const int k = atomicAdd(&s_ncand[ts], 1);
              if (k < kFixCand) s_cand[ts * kFixCand + k] = c0 + r;
            }
          } else {
            // second smallest: with best <= best2, the median of the three
            best2[tb] = __builtin_amdgcn_fmed3f(dist, best[tb], best2[tb]);
            if (dist < best[tb]) {
              best[tb] = dist;
              bidx[tb] = c0 + r;
            }
          }
        }
    };

    // cmax^2: the largest ||c||^2 of the problem's real rows
    auto cmax_sq = [&]() __attribute__((always_inline)) -> float {
      float cm = 0.f;
      for (int r = lane; r < n; r += kWave) cm = fmaxf(cm, Np[r]);
      return wave_max(cm);
    };
    if constexpr (FIX) {
      const float cm = cmax_sq();
#pragma unroll
      for (int tb = 0; tb < kAsgTB; ++tb)
        if (tok(tb) >= 0) thr[tb] += 2.02f * asg_error_bound(xn[tb], cm);
      __syncthreads();                           // s_ncand cleared
    }

    // prologue: chunks 0..2 in flight, chunk 0 landed
    load_chunk(0, sC0);
    load_chunk(1, sC1);
    load_chunk(2, sC2);
    constexpr int kLoadsPerChunk = 2 * INS + 1;   // wave 0 issues one more (the norms)
    if (wave == 0) __builtin_amdgcn_s_waitcnt(asg_wait_vm(2 * kLoadsPerChunk));
    else __builtin_amdgcn_s_waitcnt(asg_wait_vm(4 * INS));
    lds_barrier_asg();
    // chunk c: compute slot c % 4, load chunk c + 3 into slot (c + 3) % 4 (the
    // slot of chunk c - 1, which every wave finished before the last barrier),
    // then wait only for chunk c + 1, the next one computed: chunks c + 2 and
    // c + 3 stay in flight.  The first chunk of each trip loads after computing
    // (at the loop head the compiler's tracking of the loads is lost and it
    // would wait for all of them).
    int c = 0;
    auto iter = [&](auto late, const uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) -> bool {
      if constexpr (!decltype(late)::value) load_chunk(c + 3, nxt);
      compute(cur, c * kAsgCB);
      if constexpr (decltype(late)::value) load_chunk(c + 3, nxt);
      if (wave == 0) __builtin_amdgcn_s_waitcnt(asg_wait_vm(2 * kLoadsPerChunk));
      else __builtin_amdgcn_s_waitcnt(asg_wait_vm(4 * INS));
      lds_barrier_asg();
      return ++c < nchunk;
    };
    constexpr std::true_type late{};
    constexpr std::false_type early{};
    while (iter(late, sC0, sC3) && iter(early, sC1, sC0) && iter(early, sC2, sC1) && iter(early, sC3, sC2)) {
    }
    __builtin_amdgcn_s_waitcnt(0xF70);           // no chunk load outlives the loop

    if constexpr (!FIX) {
      const float cmax2 = cmax_sq();
#pragma unroll
      for (int tb = 0; tb < kAsgTB; ++tb) {
        const float ob = __shfl_xor(best[tb], 32);
        const float ob2 = __shfl_xor(best2[tb], 32);
        const int oi = __shfl_xor(bidx[tb], 32);
        // second smallest of the two halves' (best, best2) pairs
        best2[tb] = fminf(fmaxf(best[tb], ob), fminf(best2[tb], ob2));
        if (ob < best[tb] || (ob == best[tb] && oi < bidx[tb])) {
          best[tb] = ob;
          bidx[tb] = oi;
        }
        const int t = tok(tb);
        const bool tie = t >= 0 && half == 0 && !(best2[tb] - best[tb] > 2.02f * asg_error_bound(xn[tb], cmax2));
        if (half == 0 && t >= 0) {
          labels[(size_t)p * N + t] = bidx[tb];
          if (min_dist) min_dist[(size_t)p * N + t] = fmaxf(xn[tb] + best[tb], 0.f);
          // the counting sort's histogram of this chunk (integer adds: exact)
          atomicAdd(&fx.hist[((size_t)p * sort_chunks(N) + t / kSortChunk) * n + bidx[tb]], 1);
        }
        // near ties to the fix list: one counter bump per wave
        const uint64_t m = __ballot(tie);
        if (m) {
          int base = 0;
          if (lane == __ffsll((unsigned long long)m) - 1) base = atomicAdd(&fx.count[p], __popcll(m));
          base = __shfl(base, __ffsll((unsigned long long)m) - 1);
          if (tie) {
            const int k = base + __popcll(m & ((1ull << lane) - 1ull));
            fx.token[(size_t)p * N + k] = t;
            fx.dmin[(size_t)p * N + k] = best[tb];
          }
        }
      }
      return;
    } else {
      __syncthreads();                           // every candidate recorded
      // exact fp64 decision between the candidates (all centroids if they
      // overflowed the list): differences and squares of bf16 / fp32 values are
      // exact in fp64; ties go to the lowest index
      const float* Cp = fx.C + (size_t)p * n * D;
#pragma unroll 1
      for (int tb = 0; tb < kAsgTB; ++tb) {
        const int t = tok(tb);
        if (half != 0 || t < 0) continue;
        const int ts = wave * (kAsgTB * 32) + tb * 32 + col;
        const int nc = s_ncand[ts];
        const bool all = nc > kFixCand;
        const int m = all ? n : nc;
        const uint16_t* xr = Xp + (size_t)t * D;
        double bd = __builtin_inf();
        int bi = 0x7fffffff;
        for (int k = 0; k < m; ++k) {
          const int cj = all ? k : s_cand[ts * kFixCand + k];
          if ((unsigned)cj >= (unsigned)n) continue;
          const float* cr = Cp + (size_t)cj * D;
          double acc = 0.0;
#pragma unroll 4
          for (int q = 0; q < D / 8; ++q) {
            const u32x4_t v = reinterpret_cast<const u32x4_t*>(xr)[q];
            const float4 c0 = reinterpret_cast<const float4*>(cr)[2 * q];
            const float4 c1 = reinterpret_cast<const float4*>(cr)[2 * q + 1];
            const double e0 = (double)bf16_lo(v[0]) - c0.x, e1 = (double)bf16_hi(v[0]) - c0.y;
            const double e2 = (double)bf16_lo(v[1]) - c0.z, e3 = (double)bf16_hi(v[1]) - c0.w;
            const double e4 = (double)bf16_lo(v[2]) - c1.x, e5 = (double)bf16_hi(v[2]) - c1.y;
            const double e6 = (double)bf16_lo(v[3]) - c1.z, e7 = (double)bf16_hi(v[3]) - c1.w;
            acc = fma(e0, e0, acc); acc = fma(e1, e1, acc); acc = fma(e2, e2, acc); acc = fma(e3, e3, acc);
            acc = fma(e4, e4, acc); acc = fma(e5, e5, acc); acc = fma(e6, e6, acc); acc = fma(e7, e7, acc);
          }
          if (acc < bd || (acc == bd && cj < bi)) {
            bd = acc;
            bi = cj;
          }
        }
        if (m > 0) {
          const int old = labels[(size_t)p * N + t];
          labels[(size_t)p * N + t] = bi;
          if (min_dist) min_dist[(size_t)p * N + t] = (float)bd;
          if (old != bi) {
            // move the token between its chunk's histogram bins
            int32_t* hrow = fx.hist + ((size_t)p * sort_chunks(N) + t / kSortChunk) * n;
            atomicSub(&hrow[clampi(old, 0, n - 1)], 1);
            atomicAdd(&hrow[bi], 1);
          }
        }
      }
      li0 += (int)gridDim.x * kAsgTok;
      if (li0 >= nfix) return;
      __syncthreads();                           // s_ncand and the ring are reused
    }
  }
}

// fp32 inputs: exact-difference distances in fp64 on the vector ALUs.
template <int D>
__global__ __launch_bounds__(256) void k_assign_f32(const float* __restrict__ X, int N, int n,
                                                    const float* __restrict__ C,
                                                    int32_t* __restrict__ labels,
                                                    float* __restrict__ min_dist) {
  constexpr int CB = 32;
  __shared__ float sh_c[CB * D];
  const int p = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const float* xr = X + ((size_t)p * N + min(t, N - 1)) * D;
  float x[D];
#pragma unroll
  for (int e = 0; e < D; ++e) x[e] = xr[e];
  double best = __builtin_inf();
  int bidx = 0;
  const float* Cp = C + (size_t)p * n * D;
  for (int c0 = 0; c0 < n; c0 += CB) {
    __syncthreads();
    for (int v = threadIdx.x; v < CB * D; v += 256) sh_c[v] = (c0 + v / D < n) ? Cp[(size_t)c0 * D + v] : 0.f;
    __syncthreads();
    const int cend = min(CB, n - c0);
    for (int r = 0; r < cend; ++r) {
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        const double df = (double)x[e] - (double)sh_c[r * D + e];
        acc += df * df;
      }
      if (acc < best) {
        best = acc;
        bidx = c0 + r;
      }
    }
  }
  if (t < N) {
    labels[(size_t)p * N + t] = bidx;
    if (min_dist) min_dist[(size_t)p * N + t] = (float)best;
  }
}

hipError_t launch_assign(const void* x, bool bf16, int bh, int N, int d, int n, const float* c,
                         const uint16_t* c_hi, const uint16_t* c_lo, const float* c_norm,
                         int32_t* labels, float* min_dist, const AsgFixWs& fw, hipStream_t s) {
  if (bf16) {
    const AsgFix fx{fw.count, fw.token, fw.dmin, c, fw.hist};
    const dim3 grid((N + asg_tok(false) - 1) / asg_tok(false), bh);
    // the near-tie pass: enough work-groups per problem (128 tokens each) for
    // a quarter of the tokens in one sweep over the centroids, so that the
    // few percent of near ties finish in one sweep latency; work-groups past
    // the list's end exit at once, and each loops if the list is longer
    const dim3 gfix((N + 4 * asg_tok(true) - 1) / (4 * asg_tok(true)), bh);
    const uint16_t* xt = static_cast<const uint16_t*>(x);
    if (d == 128) {
      hipLaunchKernelGGL((k_assign_bf16<128, false>), grid, dim3(256), 0, s, xt, N, n, c_hi, c_lo, c_norm, labels,
                         min_dist, fx);
      hipLaunchKernelGGL((k_assign_bf16<128, true>), gfix, dim3(256), 0, s, xt, N, n, c_hi, c_lo, c_norm, labels,
                         min_dist, fx);
    } else {
      hipLaunchKernelGGL((k_assign_bf16<64, false>), grid, dim3(256), 0, s, xt, N, n, c_hi, c_lo, c_norm, labels,
                         min_dist, fx);
      hipLaunchKernelGGL((k_assign_bf16<64, true>), gfix, dim3(256), 0, s, xt, N, n, c_hi, c_lo, c_norm, labels,
                         min_dist, fx);
    }
  } else {
    const dim3 grid((N + 255) / 256, bh);
    if (d == 128)
      hipLaunchKernelGGL(k_assign_f32<128>, grid, dim3(256), 0, s, static_cast<const float*>(x), N, n, c,
                         labels, min_dist);
    else
      hipLaunchKernelGGL(k_assign_f32<64>, grid, dim3(256), 0, s, static_cast<const float*>(x), N, n, c,
                         labels, min_dist);
  }
  return hipGetLastError();
}

// ======================================================================
// Lloyd update: centroid = mean of members (segmented over the sorted order)
// ======================================================================
// Centroid c = mean of the rows perm[offsets[c] .. offsets[c+1]).
// Cluster sizes are heavy-tailed, so the work is cut along the sorted order
// instead of per cluster: work-group k sums the rows of sorted positions
// [512 k, 512 (k+1)), one cluster segment after the other, and writes one
// fp64 partial sum per (cluster c, chunk k) to slot c + k (unique, because
// every cluster is a contiguous, increasing range of the sorted order).  A
// second kernel adds each cluster's partials in chunk order.  Every sum runs
// in a fixed order, so the result is the same run to run.
// MOVE (1: same dtype, 2: E4M3 from bf16): the rows read at sorted position
// r are also stored to row r of mv.x_out (and, when mv.y is given, row
// perm[r] of y to row r of mv.y_out): the permutation into cluster blocks
// rides on the reads the update makes anyway.
template <typename T, int D, int MOVE>
__global__ __launch_bounds__(256) void k_centroid_partial(const T* __restrict__ X, int N, int n,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets,
                                                          double* __restrict__ partial, MeanMove mv) {
  static_assert(MOVE != 2 || sizeof(T) == 2, "E4M3 rows from bf16 only");
  constexpr int EPV = 16 / sizeof(T);          // elements per 16-byte vector
  constexpr int VPR = D / EPV;                 // lanes per row
  constexpr int G = 256 / VPR;                 // row groups
  constexpr int U = MOVE ? 8 : 4;              // rows in flight per lane (more when moving rows)
  __shared__ double red[G][D];
  __shared__ int32_t s_perm[kMeanChunk];
  __shared__ int s_c0;
  const int p = blockIdx.y, k = blockIdx.x;
  const int chunks = gridDim.x;
  const int j0 = k * kMeanChunk, j1 = min(j0 + kMeanChunk, N);
  const int32_t* off = offsets + (size_t)p * (n + 1);
  const int32_t* pp = perm + (size_t)p * N;
  for (int j = threadIdx.x; j < j1 - j0; j += blockDim.x) s_perm[j] = clampi(pp[j0 + j], 0, N - 1);
  if (threadIdx.x == 0) {
    // the cluster holding position j0: the largest c < n with offsets[c] <= j0
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= j0) lo = mid; else hi = mid - 1;
    }
    s_c0 = lo;
  }
  __syncthreads();
  const int cv = threadIdx.x % VPR, g = threadIdx.x / VPR;
  const T* Xp = X + (size_t)p * N * D + cv * EPV;
  // destinations: element offset of this lane's 16 source bytes (E4M3: 8 bytes)
  using OutT = typename std::conditional<MOVE == 2, uint8_t, T>::type;
  const size_t o_lane = (size_t)p * N * D + cv * EPV;
  OutT* Xq = MOVE ? static_cast<OutT*>(mv.x_out) + o_lane : nullptr;
  const T* Yp = MOVE && mv.y ? static_cast<const T*>(mv.y) + o_lane : nullptr;
  OutT* Yq = MOVE && mv.y ? static_cast<OutT*>(mv.y_out) + o_lane : nullptr;
  float rx = 1.f, ry = 1.f;
  if constexpr (MOVE == 2) {
    const int bh = (int)gridDim.y;
    rx = quant_ratio(mv.amax[p]);
    if (Yp) ry = quant_ratio(mv.amax[bh + p]);
    if (k == 0 && threadIdx.x == 0) {
      mv.x_scale[p] = quant_scale(mv.amax[p]);
      if (Yp) mv.y_scale[p] = quant_scale(mv.amax[bh + p]);
    }
  }
  double* part = partial + (size_t)p * (n + chunks) * D;
  int c = s_c0, pos = j0;
  while (pos < j1 && c < n) {
    const int end = min(max(off[c + 1], pos), j1);
    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
    for (int i = pos + g; i < end; i += G * U) {
      u32x4_t v[U], w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = i + u * G;
        if (r < end) {
          const size_t src = (size_t)s_perm[r - j0] * D;
          v[u] = *reinterpret_cast<const u32x4_t*>(Xp + src);
          if (MOVE && Yp) w[u] = *reinterpret_cast<const u32x4_t*>(Yp + src);
        }
      }
      if constexpr (MOVE) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = i + u * G;
          if (r < end) {
            if constexpr (MOVE == 2) {
              *reinterpret_cast<uint2*>(Xq + (size_t)r * D) = quant8_bf16(v[u], rx);
              if (Yp) *reinterpret_cast<uint2*>(Yq + (size_t)r * D) = quant8_bf16(w[u], ry);
            } else {
              *reinterpret_cast<u32x4_t*>(Xq + (size_t)r * D) = v[u];
              if (Yp) *reinterpret_cast<u32x4_t*>(Yq + (size_t)r * D) = w[u];
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i + u * G >= end) break;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16_lo(v[u][e]);
            acc[2 * e + 1] += (double)bf16_hi(v[u][e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(v[u][e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) red[g][cv * EPV + e] = acc[e];
    __syncthreads();
    if (end > pos && threadIdx.x < D) {
      double sum = 0.0;
#pragma unroll
      for (int q = 0; q < G; ++q) sum += red[q][threadIdx.x];
      part[(size_t)(c + k) * D + threadIdx.x] = sum;
    }
    __syncthreads();
    pos = max(end, pos);
    // next cluster holding `pos` (empty clusters end where they start)
    ++c;
    while (c < n && off[c + 1] <= pos) ++c;
  }
}

template <int D>
__global__ __launch_bounds__(D) void k_centroid_finish(int n, int chunks, const int32_t* __restrict__ offsets,
                                                       const double* __restrict__ partial,
                                                       float* __restrict__ C) {
  const int c = blockIdx.x, p = blockIdx.y;
  const int32_t* off = offsets + (size_t)p * (n + 1);
  const int a = off[c], b = off[c + 1];
  if (b <= a) return;                          // empty cluster keeps its centroid
  const double* part = partial + (size_t)p * (n + chunks) * D;
  const int k0 = a / kMeanChunk, k1 = (b - 1) / kMeanChunk;
  double sum = 0.0;
  for (int k = k0; k <= k1; ++k) sum += part[(size_t)(c + k) * D + threadIdx.x];
  C[((size_t)p * n + c) * D + threadIdx.x] = (float)(sum / (double)(b - a));
}

template <typename T, int D>
void centroid_mean_t(const void* x, int bh, int N, int n, const int32_t* perm, const int32_t* offsets,
                     double* partial_ws, float* c, hipStream_t s, const MeanMove& mv, int mode) {
  const int chunks = mean_chunks(N);
  const dim3 grid(chunks, bh);
  const T* xt = static_cast<const T*>(x);
  if (mode == 0) {
    hipLaunchKernelGGL((k_centroid_partial<T, D, 0>), grid, dim3(256), 0, s, xt, N, n, perm, offsets, partial_ws, mv);
  } else if (mode == 1) {
    hipLaunchKernelGGL((k_centroid_partial<T, D, 1>), grid, dim3(256), 0, s, xt, N, n, perm, offsets, partial_ws, mv);
  } else if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((k_centroid_partial<T, D, 2>), grid, dim3(256), 0, s, xt, N, n, perm, offsets, partial_ws, mv);
  }
  hipLaunchKernelGGL((k_centroid_finish<D>), dim3(n, bh), dim3(D), 0, s, n, chunks, offsets, partial_ws, c);
}

hipError_t launch_centroid_mean(const void* x, bool bf16, int bh, int N, int d, int n,
                                const int32_t* perm, const int32_t* offsets, double* partial_ws, float* c,
                                hipStream_t s, const MeanMove& mv) {
  const int mode = !mv.x_out ? 0 : (mv.amax ? 2 : 1);
  if (mode == 2 && !bf16) return hipErrorInvalidValue;
  if (bf16) {
    if (d == 128) centroid_mean_t<uint16_t, 128>(x, bh, N, n, perm, offsets, partial_ws, c, s, mv, mode);
    else centroid_mean_t<uint16_t, 64>(x, bh, N, n, perm, offsets, partial_ws, c, s, mv, mode);
  } else {
    if (d == 128) centroid_mean_t<float, 128>(x, bh, N, n, perm, offsets, partial_ws, c, s, mv, mode);
    else centroid_mean_t<float, 64>(x, bh, N, n, perm, offsets, partial_ws, c, s, mv, mode);
  }
  return hipGetLastError();
}

}  // namespace svg2
