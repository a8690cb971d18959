// Block-sparse attention over variable-sized cluster blocks ("Sparse
// VideoGen2" wiki summary, Method, stage (4); Key claims, §4.3 / Fig. 7(b)).
//
// Work item = (problem, Q-cluster i, 128-row slab of that cluster).  The key
// list of item i is the concatenation of the key ranges of its selected
// K-clusters; it is walked in tiles of 64 keys that may straddle cluster
// boundaries, so the only padding is the tail of the whole list (and of the
// query slab), not a round-up of every cluster to a fixed block size.
//
// bf16 kernel, one wave = 32 query rows, 4 waves share each K/V tile in LDS:
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, K tile from LDS, Q in registers
//   online softmax     fp32, base 2 (scale * log2 e folded in), per lane: one
//                      query, 32 keys; one cross-half exchange for the max
//   O^T += V^T P^T     P re-used straight from the S accumulator (no shuffle):
//                      the key order inside each 16-key MFMA step is permuted,
//                      and V^T is staged in LDS in the same permuted order.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace svg2 {

constexpr int kAttnBM = 128;     // query rows per work item (bf16 kernel)
constexpr int kAttnBN = 64;      // keys per tile
constexpr int kAttnF32BM = 64;   // query rows per work item (fp32 kernel)

int attn_block_rows(bool bf16) { return bf16 ? kAttnBM : kAttnF32BM; }

// ---------------------------------------------------------------- planning
// One work-group per problem: the list of (cluster, slab) items.
__global__ __launch_bounds__(1024) void k_attn_plan(const int32_t* __restrict__ q_off, int n_q, int N,
                                                    int bm, int max_items,
                                                    int32_t* __restrict__ item_count,
                                                    int32_t* __restrict__ items) {
  __shared__ int32_t scratch[17];
  const int p = blockIdx.x;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  int nb[4];
  int local = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * threadIdx.x + e;
    nb[e] = 0;
    if (i < n_q) {
      const int a = clampi(qo[i], 0, N), b = clampi(qo[i + 1], a, N);
      nb[e] = (b - a + bm - 1) / bm;
    }
    local += nb[e];
  }
  int total;
  int base = block_exclusive_scan(local, scratch, &total);
  int32_t* it = items + (size_t)p * max_items;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * threadIdx.x + e;
    for (int r = 0; r < nb[e] && base < max_items; ++r, ++base) it[base] = i | (r << 12);
  }
  if (threadIdx.x == 0) item_count[p] = min(total, max_items);
}

// Walks the concatenated key ranges of the selected clusters; all threads of a
// work-group advance the same cursor (uniform control flow).
struct KeyCursor {
  const int32_t* sel;
  const int32_t* koff;
  int nsel, n_k, N;
  int next, pos, rem;

  __device__ __forceinline__ void init(const int32_t* s, const int32_t* ko, int ns, int nk, int n) {
    sel = s; koff = ko; nsel = ns; n_k = nk; N = n;
    next = 0; pos = 0; rem = 0;
  }
  __device__ __forceinline__ void open_ranges() {
    while (rem == 0 && next < nsel) {
      const int j = sel[next++];
      if ((unsigned)j >= (unsigned)n_k) continue;
      const int a = clampi(koff[j], 0, N);
      pos = a;
      rem = clampi(koff[j + 1], a, N) - a;
    }
  }
  // Fills up to `tile` keys; slot_of[e] (this thread's slots) get key indices
  // or -1.  Returns the number of keys in the tile; *contiguous tells that the
  // tile is full and inside one key range (key = first key + slot).
  template <int NS>
  __device__ __forceinline__ int fill(int tile, const int (&slot_of)[NS], int (&key)[NS], bool* contiguous) {
    open_ranges();
    if (rem >= tile) {
#pragma unroll
      for (int e = 0; e < NS; ++e) key[e] = slot_of[e] >= 0 ? pos + slot_of[e] : -1;
      pos += tile;
      rem -= tile;
      *contiguous = true;
      return tile;
    }
    *contiguous = false;
#pragma unroll
    for (int e = 0; e < NS; ++e) key[e] = -1;
    int filled = 0;
    while (filled < tile) {
      if (rem == 0) {
        if (next >= nsel) break;
        const int j = sel[next++];
        if ((unsigned)j >= (unsigned)n_k) continue;
        const int a = clampi(koff[j], 0, N);
        const int b = clampi(koff[j + 1], a, N);
        pos = a;
        rem = b - a;
        continue;
      }
      const int take = min(rem, tile - filled);
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const int s = slot_of[e] - filled;
        if (s >= 0 && s < take) key[e] = pos + s;
      }
      filled += take;
      pos += take;
      rem -= take;
    }
    return filled;
  }
};

// ---------------------------------------------------------------- bf16
// Lazy rescaling: the exponentials use a reference max m_ref that only moves
// when a tile's max exceeds it by more than kLazyTau (log2 units), so P stays
// <= 2^kLazyTau and O / l are rescaled rarely.  The result is the same
// softmax; only the intermediate scaling differs.
constexpr float kLazyTau = 8.f;

// Work items are taken in an order that keeps consecutive items (same
// Q-cluster, same head) on one XCD: work-groups are dispatched round-robin
// over the 8 XCDs, so block b runs item (b % 8) * per_xcd + b / 8.
constexpr int kXcds = 8;

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int N, const int32_t* __restrict__ q_off, int n_q, const int32_t* __restrict__ k_off, int n_k,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx, float scale_log2,
    uint16_t* __restrict__ O, float* __restrict__ lse, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ items, int max_items, int bh) {
  constexpr int BN = kAttnBN;
  constexpr int KS = D / 16;           // 16-wide k-steps of Q.K
  constexpr int DT = D / 32;           // 32-row tiles of O^T
  constexpr int KLD = D + 8;           // K tile row stride (elements)
  constexpr int VLD = BN + 8;          // V^T tile row stride (elements)
  constexpr int VPR = D / 8;           // 16-byte vectors per row
  constexpr int VUNITS = (BN / 8) * VPR;        // 8x8 transpose blocks of V
  constexpr int KUNITS = BN * VPR / 8;          // 8-vector groups of K
  static_assert(VUNITS + KUNITS <= 256, "one load unit per thread");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VLD];

  const int total = max_items * bh;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int logical = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (logical >= total) return;
  const int p = logical / max_items, slot = logical % max_items;
  if (slot >= item_count[p]) return;
  const int item = items[(size_t)p * max_items + slot];
  const int ci = item & 0xfff, rb = item >> 12;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  const int qa = clampi(qo[ci], 0, N), qb = clampi(qo[ci + 1], qa, N);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int col = lane & 31, half = lane >> 5;
  const int row0 = qa + rb * kAttnBM + wave * 32;
  const bool active = row0 < qb;                 // this wave has query rows
  const int row = row0 + col;
  const bool row_ok = row < qb;
  const size_t base = (size_t)p * N * D;

  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row_ok) v = *reinterpret_cast<const u32x4_t*>(Q + base + (size_t)row * D + ks * 16 + half * 8);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  // this thread's load unit: a V transpose block (key group g, column chunk c)
  // or a group of 8 K vectors
  const bool is_v = tid < VUNITS;
  const bool is_k = !is_v && tid < VUNITS + KUNITS;
  const int vc = tid % VPR, vg = tid / VPR;
  const int ku = tid - VUNITS;
  int slot_of[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (is_v) {
      // group g = (kk, h) holds keys 16kk + 4h + {0..3} and 16kk + 8 + 4h + {0..3}
      const int kk = vg >> 1, h = vg & 1;
      slot_of[e] = 16 * kk + 8 * (e >> 2) + 4 * h + (e & 3);
    } else if (is_k) {
      slot_of[e] = (ku + KUNITS * e) / VPR;
    } else {
      slot_of[e] = -1;
    }
  }
  // element offset of this thread's vector inside a key row
  const int vec_off = is_v ? vc * 8 : (ku % VPR) * 8;
  const uint16_t* src = (is_v ? V : K) + base + vec_off;

  KeyCursor cur;
  cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
           clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N);

  u32x4_t rg[8];
  auto load_tile = [&](const int (&key)[8], bool contiguous) {
    if (!(is_v || is_k)) return;
    if (contiguous) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rg[e] = *reinterpret_cast<const u32x4_t*>(src + (size_t)key[e] * D);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rg[e] = u32x4_t{0u, 0u, 0u, 0u};
        if (key[e] >= 0) rg[e] = *reinterpret_cast<const u32x4_t*>(src + (size_t)key[e] * D);
      }
    }
  };
  // registers -> LDS buffer (V transposed into the permuted key order)
  auto store_tile = [&](int buf) {
    if (is_v) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = __builtin_amdgcn_perm(rg[2 * q + 1][x >> 1], rg[2 * q][x >> 1], sel);
        const int d = vc * 8 + x;
        *reinterpret_cast<u32x4_t*>(&sV[buf][d * VLD + (vg ^ ((d >> 4) & 7)) * 8]) = w;
      }
    } else if (is_k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = ku + KUNITS * e;
        *reinterpret_cast<u32x4_t*>(&sK[buf][(v / VPR) * KLD + (v % VPR) * 8]) = rg[e];
      }
    }
  };

  float m_ref = -__builtin_inff();
  f32x16_t o[DT], lsum;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) lsum[i] = 0.f;
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  int key[8];
  bool contiguous;
  int filled = cur.fill<8>(BN, slot_of, key, &contiguous);
  if (filled > 0) {
    load_tile(key, contiguous);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  while (filled > 0) {
    // prefetch the next tile while this one is computed
    bool next_contig;
    const int next_filled = cur.fill<8>(BN, slot_of, key, &next_contig);
    if (next_filled > 0) load_tile(key, next_contig);

    if (active) {
      const uint16_t* kb = sK[buf];
      const uint16_t* vb = sV[buf];
      // ---- S^T = K Q^T for 2 sub-tiles of 32 keys
      f32x16_t s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&kb[(st * 32 + col) * KLD + ks * 16 + half * 8]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[st], 0, 0, 0);
        }
      }
      // ---- online softmax; lane holds keys st*32 + (i/4)*8 + half*4 + i%4
      if (filled < BN) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ks = st * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            if (ks >= filled) s[st][i] = -__builtin_inff();
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
      {
        // lanes i and i+32 hold the same query: combine their maxima
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
      }
      if (mx > m_ref + kLazyTau) {
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mx);
#pragma unroll
        for (int i = 0; i < 16; ++i) lsum[i] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        m_ref = mx;
      }
      const float neg = -m_ref;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = __builtin_amdgcn_exp2f(fmaf(s[st][i], scale_log2, neg));

      // ---- O^T += V^T P^T, 4 k-steps of 16 keys
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int st = kk >> 1, sub = kk & 1;
        u32x4_t pw;
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = pack_bf16x2(s[st][8 * sub + 2 * q], s[st][8 * sub + 2 * q + 1]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
        const int blk = 2 * kk + half;
        // row sums of the bf16 P on the matrix core: an all-ones A operand
        lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb, lsum, 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = dt * 32 + col;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&vb[d * VLD + ((blk ^ ((d >> 4) & 7)) * 8)]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[dt], 0, 0, 0);
        }
      }
    }
    if (next_filled > 0) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    filled = next_filled;
  }

  // every row of the ones-product holds the sum over all keys of the tile
  const float l_tot = lsum[0];
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = O + base + (size_t)row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
        w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 32 + g * 8 + half * 4) = w;
      }
    if (lse && half == 0)
      lse[(size_t)p * N + row] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * 0.69314718055994531f
                                            : -__builtin_inff();
  }
}

// ---------------------------------------------------------------- fp32
// fp32 inputs: two threads per query row (each owns half of the head dim),
// keys staged 32 at a time in LDS, exact fp32 online softmax per key.
template <int D>
__global__ __launch_bounds__(128) void k_attn_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V, int N,
    const int32_t* __restrict__ q_off, int n_q, const int32_t* __restrict__ k_off, int n_k,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx, float scale,
    float* __restrict__ O, float* __restrict__ lse, const int32_t* __restrict__ item_count,
    const int32_t* __restrict__ items, int max_items) {
  constexpr int BN = 32;
  constexpr int H = D / 2;
  __shared__ float sK[BN * D];
  __shared__ float sV[BN * D];
  const int p = blockIdx.y;
  if ((int)blockIdx.x >= item_count[p]) return;
  const int item = items[(size_t)p * max_items + blockIdx.x];
  const int ci = item & 0xfff, rb = item >> 12;
  const int32_t* qo = q_off + (size_t)p * (n_q + 1);
  const int qa = clampi(qo[ci], 0, N), qb = clampi(qo[ci + 1], qa, N);
  const int tid = threadIdx.x;
  const int row = qa + rb * kAttnF32BM + tid / 2;
  const int hh = tid & 1;
  const bool row_ok = row < qb;
  const size_t base = (size_t)p * N * D;
  float q[H], o[H];
#pragma unroll
  for (int e = 0; e < H; ++e) {
    q[e] = row_ok ? Q[base + (size_t)row * D + hh * H + e] : 0.f;
    o[e] = 0.f;
  }
  // each thread loads BN*D/128 floats of K and of V per tile
  constexpr int PER = BN * D / 128;
  int slot_of[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) slot_of[e] = (tid + 128 * e) / D;
  KeyCursor cur;
  cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
           clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N);
  float m_run = -__builtin_inff(), l_run = 0.f;
  for (;;) {
    int key[PER];
    bool contiguous;
    const int filled = cur.fill<PER>(BN, slot_of, key, &contiguous);
    if (filled == 0) break;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int f = tid + 128 * e;
      const int c = f % D;
      sK[f] = key[e] >= 0 ? K[base + (size_t)key[e] * D + c] : 0.f;
      sV[f] = key[e] >= 0 ? V[base + (size_t)key[e] * D + c] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < filled; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < H; ++e) part = fmaf(q[e], sK[j * D + hh * H + e], part);
      const float sc = (part + __shfl_xor(part, 1)) * scale;
      const float m_new = fmaxf(m_run, sc);
      const float corr = expf(m_run - m_new);
      const float pe = expf(sc - m_new);
      l_run = l_run * corr + pe;
#pragma unroll
      for (int e = 0; e < H; ++e) o[e] = fmaf(pe, sV[j * D + hh * H + e], o[e] * corr);
      m_run = m_new;
    }
  }
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int e = 0; e < H; ++e) O[base + (size_t)row * D + hh * H + e] = o[e] * inv;
    if (lse && hh == 0) lse[(size_t)p * N + row] = l_run > 0.f ? m_run + logf(l_run) : -__builtin_inff();
  }
}

hipError_t launch_varblock_attn(const void* q, const void* k, const void* v, bool bf16, int bh,
                                int N, int d, const int32_t* q_off, int n_q, const int32_t* k_off,
                                int n_k, const int32_t* sel_count, const int32_t* sel_idx,
                                float scale, void* out, float* lse, int32_t* item_count_ws,
                                int32_t* items_ws, hipStream_t s) {
  const int bm = attn_block_rows(bf16);
  const int max_items = attn_max_items(N, n_q, bm);
  hipLaunchKernelGGL(k_attn_plan, dim3(bh), dim3(1024), 0, s, q_off, n_q, N, bm, max_items, item_count_ws,
                     items_ws);
  const dim3 grid(max_items, bh);
  const int total = max_items * bh;
  const dim3 grid_x((total + kXcds - 1) / kXcds * kXcds);
  if (bf16) {
    const float sl2 = scale * 1.4426950408889634f;
#define SVG2_ATTN(D)                                                                                  \
  hipLaunchKernelGGL(k_attn_bf16<D>, grid_x, dim3(256), 0, s, static_cast<const uint16_t*>(q),        \
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N, q_off, n_q, \
                     k_off, n_k, sel_count, sel_idx, sl2, static_cast<uint16_t*>(out), lse,          \
                     item_count_ws, items_ws, max_items, bh)
    if (d == 128) SVG2_ATTN(128); else SVG2_ATTN(64);
#undef SVG2_ATTN
  } else {
#define SVG2_ATTN(D)                                                                                   \
  hipLaunchKernelGGL(k_attn_f32<D>, grid, dim3(128), 0, s, static_cast<const float*>(q),               \
                     static_cast<const float*>(k), static_cast<const float*>(v), N, q_off, n_q, k_off, \
                     n_k, sel_count, sel_idx, scale, static_cast<float*>(out), lse, item_count_ws,    \
                     items_ws, max_items)
    if (d == 128) SVG2_ATTN(128); else SVG2_ATTN(64);
#undef SVG2_ATTN
  }
  return hipGetLastError();
}

}  // namespace svg2
