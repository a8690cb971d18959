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

// Work-groups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Items are handed out in chunks of kXcdChunk consecutive items per
// XCD, so the slabs of one Q-cluster (which read the same key list) share an
// XCD and its L2, while all XCDs still advance through the same head at the
// same time (its K/V stays in the last-level cache):
//   block b -> item ((b / 8 / C) * 8 + b % 8) * C + (b / 8) % C,  C = kXcdChunk
// which is a bijection on [0, grid) when grid is a multiple of 8 C.
constexpr int kXcds = 8;
constexpr int kXcdChunk = 4;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

template <typename Tp>
__device__ __forceinline__ lds_u16_t* to_lds(Tp* p) {
  return (lds_u16_t*)(lds_void_t*)(void*)p;
}

// K and V tiles sit row-major in LDS, 64 keys x D, with the 16-byte chunks of
// each row XOR-swizzled (no padding, so they can be filled by direct
// global -> LDS loads):
//   K: chunk c of row r at c ^ (r % 16)      (conflict-free 16-byte reads of
//      one chunk across 16 consecutive rows)
//   V: chunk c of row r at c ^ 2 (r % 4)      (conflict-free transposing reads
//      of 4 rows x 32 bytes)
template <int D> struct TileGeom {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static __device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (CPR - 1) & 15); }
  static __device__ __forceinline__ int v_chunk(int r, int c) { return c ^ (2 * (r & 3)); }
};

// One tile = 64 rows.  Each wave fills 16 rows of K and of V with 4 + 4
// direct-to-LDS loads of 16 bytes per lane (lane -> row 4q + lane/16, slot
// lane%16 of the row); rows past the key list load key 0 (never weighted:
// their scores are masked to -inf).
template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t* Kp, const uint16_t* Vp, lds_u16_t* sk, lds_u16_t* sv,
                                         const int (&key)[4], int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = kWave / CPR;                  // rows per instruction (4 at D=128)
  constexpr int INS = 16 / RPI;                     // instructions per 16 rows
#pragma unroll
  for (int q = 0; q < INS; ++q) {
    const int r = 16 * wave + RPI * q + lane / CPR;
    const int phys = lane % CPR;
    const size_t krow = (size_t)max(key[q], 0) * D;
    const uint16_t* ksrc = Kp + krow + TileGeom<D>::k_chunk(r, phys) * 8;
    const uint16_t* vsrc = Vp + krow + TileGeom<D>::v_chunk(r, phys) * 8;
    lds_u16_t* kdst = sk + (16 * wave + RPI * q) * D;
    lds_u16_t* vdst = sv + (16 * wave + RPI * q) * D;
    __builtin_amdgcn_global_load_lds((const void*)ksrc, (lds_void_t*)kdst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)vsrc, (lds_void_t*)vdst, 16, 0, 0);
  }
}

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
  constexpr int CPR = D / 8;
  constexpr int RPI = kWave / CPR;
  constexpr int INS = 16 / RPI;
  static_assert(INS <= 4, "key slots per lane");
  __shared__ __attribute__((aligned(16))) uint16_t sK0[BN * D], sK1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[BN * D], sV1[BN * D];

  const int total = max_items * bh;
  const int jx = (int)(blockIdx.x / kXcds), xx = (int)(blockIdx.x % kXcds);
  const int logical = ((jx / kXcdChunk) * kXcds + xx) * kXcdChunk + jx % kXcdChunk;
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
  const uint16_t* Kp = K + base;
  const uint16_t* Vp = V + base;

  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row_ok) v = *reinterpret_cast<const u32x4_t*>(Q + base + (size_t)row * D + ks * 16 + half * 8);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  // this lane's tile rows (one per direct-to-LDS load)
  int slot_of[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) slot_of[q] = q < INS ? 16 * wave + RPI * q + lane / CPR : -1;

  KeyCursor cur;
  cur.init(sel_idx + ((size_t)p * n_q + ci) * n_k, k_off + (size_t)p * (n_k + 1),
           clampi(sel_count[(size_t)p * n_q + ci], 0, n_k), n_k, N);

  float m_ref = -__builtin_inff();
  f32x16_t o[DT], lsum;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) lsum[i] = 0.f;
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  // per-lane LDS offsets (elements) of this lane's operand reads
  // K (S^T = K Q^T): row st*32 + col, chunk 2 ks + half
  // V^T (transposing read): rows kb + (lane%16)/4, columns d0 + 4 (lane%4)
  const int vr = (lane & 15) >> 2;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto compute = [&](const lds_u16_t* kb, const lds_u16_t* vb, int filled) {
    // ---- S^T = K Q^T for 2 sub-tiles of 32 keys
    f32x16_t s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
      const int r = st * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const __attribute__((address_space(3))) bf16x8_t*)(
            kb + r * D + TileGeom<D>::k_chunk(r, 2 * ks + half) * 8);
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

    // ---- O^T += V^T P^T, 4 k-steps of 16 keys; key order inside a step:
    // position h*8 + e <-> key 16 kk + 8 (e/4) + 4 h + e%4
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int st = kk >> 1, sub = kk & 1;
      u32x4_t pw;
#pragma unroll
      for (int q = 0; q < 4; ++q) pw[q] = pack_bf16x2(s[st][8 * sub + 2 * q], s[st][8 * sub + 2 * q + 1]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
      lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb, lsum, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int c0 = dt * 32 + vcol;                       // column (element)
        const int ra = 16 * kk + 4 * half + vr;              // keys 16kk + 4h + {0..3}
        const int rb2 = ra + 8;                              // keys 16kk + 8 + 4h + {0..3}
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vb + ra * D + TileGeom<D>::v_chunk(ra, c0 >> 3) * 8 + (c0 & 7)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vb + rb2 * D + TileGeom<D>::v_chunk(rb2, c0 >> 3) * 8 + (c0 & 7)));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[dt], 0, 0, 0);
      }
    }
  };

  lds_u16_t* k0 = to_lds(sK0);
  lds_u16_t* k1 = to_lds(sK1);
  lds_u16_t* v0 = to_lds(sV0);
  lds_u16_t* v1 = to_lds(sV1);

  int key[4];
  bool contiguous;
  int filled = cur.fill<4>(BN, slot_of, key, &contiguous);
  if (filled > 0) dma_tile<D>(Kp, Vp, k0, v0, key, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // two tiles per trip so that each LDS buffer is a distinct static array
  while (filled > 0) {
    int nf = cur.fill<4>(BN, slot_of, key, &contiguous);
    if (nf > 0) dma_tile<D>(Kp, Vp, k1, v1, key, wave, lane);
    if (active) compute(k0, v0, filled);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    filled = nf;
    if (filled <= 0) break;
    nf = cur.fill<4>(BN, slot_of, key, &contiguous);
    if (nf > 0) dma_tile<D>(Kp, Vp, k0, v0, key, wave, lane);
    if (active) compute(k1, v1, filled);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    filled = nf;
  }

  // every row of the ones-product holds the sum over all keys seen
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
  constexpr int span = kXcds * kXcdChunk;
  const dim3 grid_x((total + span - 1) / span * span);
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
