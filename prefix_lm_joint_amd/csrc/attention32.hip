// Grouped-query attention at head_dim 256 with 8 query heads per KV head on
// 32x32x16 matrix-core steps, gfx950: the prefill over the pooled K/V and the
// cached suffix decode.
//
// What is computed ("π0.5 vs MM-DiT joint attention", first section; "VLA 代码精读"
// §1.5, §1.6): per (sample, query token, head) one softmax over every visible key
// of the concatenated pool, query head h reading KV head floor(h*Hkv/Hq); masked
// keys are excluded by selection (score -inf before the maximum, weight 0).
//
// Organisation:
//   * A wave owns 32 query rows = 4 tokens x 8 heads, so every K/V element it
//     reads from LDS serves 8 heads and each matrix-core operand fragment feeds a
//     32 x 32 product: half the LDS bytes per flop of 16-row tiles.  A workgroup
//     is four waves (128 rows = 16 tokens), one per SIMD, each holding its Q
//     fragments (64 registers) and its fp32 O^T (128 registers) for the whole
//     key loop.
//   * Products are transposed: S^T = K Q^T (A = K from LDS, B = Q^T from
//     registers), then O^T += V^T P^T with P^T taken straight from the S^T
//     accumulators.  In the 32x32 accumulator a lane holds 16 keys of ONE query
//     row (lane l: row l % 32, keys 8(i/4) + 4(l/32) + i%4), so a row's
//     statistics live in two lanes (l and l ^ 32).  The P^T operand of the
//     product over keys 16a..16a+15 is the lane's own elements 8a..8a+7 when the
//     contraction index k = 8(l/32) + t stands for key 16a + 4(l/32) + (t&3) +
//     8(t>>2); the V^T operand is read in that key order by two transposing LDS
//     reads (ds_read_b64_tr_b16) of 4 keys each.
//   * K/V tiles of 32 keys go from global memory straight into LDS (buffer loads
//     with the LDS destination) over four stages; every wave issues a quarter of
//     a tile's loads, spread through its products.  LDS rows are unpadded;
//     16-byte chunks are XOR-swizzled by row (K: chunk ^ (r & 15), for 16 lanes
//     reading 16 rows at one chunk; V: chunk ^ 4(r & 3), for 32 lanes reading 4
//     rows x 64 bytes transposed), applied to the global source chunk each lane
//     fetches, so both operand reads are bank-conflict free.
//   * Softmax in base 2 against a per-row reference maximum fixed at the row's
//     first tile with a visible key; weights may exceed 1 and the final 1/l
//     removes the reference.  If a row's maximum ends more than kGrowth above
//     it, the workgroup redoes its tiles with the true maximum.  Row sums add the
//     bf16 weights that multiply V (v_dot2 with ones).
//   * Step i runs tile i-1's PV and tile i+1's scores on the matrix cores, with
//     tile i's weights computed between them, while tile i+2 streams in.
#include "attention32.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace {

using namespace pi_engine;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int D = 256;
constexpr int G = 8;              // query heads per KV head
constexpr int ROWS_W = 32;        // query rows per wave
constexpr int NW = 4;             // waves per workgroup
constexpr int ROWS = NW * ROWS_W; // 128
constexpr int TOK = ROWS / G;     // 16 query tokens per workgroup
constexpr int THREADS = NW * 64;
constexpr int kLoadsPerWave = (TK * D * 2 / 1024) / NW;   // 1 KB loads of each tensor per wave and tile: 4
constexpr float kGrowth = 64.0f;
constexpr int kMaxSplit32 = 16;

struct Stage {
  alignas(16) __bf16 k[TK * D];
  alignas(16) __bf16 v[TK * D];
  alignas(16) uint32_t w[64];     // per-key mask words (lanes >= 32 land as zeros)
};

__device__ __forceinline__ int fk(int r) { return r & 15; }
__device__ __forceinline__ int fv(int r) { return 4 * (r & 3); }

// Per-lane byte offsets computed once.
//   kr[j]: K fragment j (j < 8; j + 8 is kr[j] + 256): key row l % 32, logical chunk 2j + l/32.
//   vr[c]: V^T fragment of d chunk c (c < 4; c + 4 is vr[c] + 256), key half 0, first read;
//          key half a and read e add (16a + 8e) rows.
//   ld_k/ld_v[n], ld_row[n]: this wave's n-th 1 KB load of a tile (rows 2N, 2N+1 with
//          N = wave * 4 + n), the source chunk pre-swizzled.
struct Lanes {
  uint32_t kr[8];
  uint32_t vr[4];
  uint32_t ld_k[kLoadsPerWave], ld_v[kLoadsPerWave];
  int ld_row[kLoadsPerWave];
};

__device__ __forceinline__ Lanes make_lanes(int tsb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  Lanes lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) lo.kr[j] = (uint32_t)(r * D * 2 + 16 * ((2 * j + h) ^ fk(r)));
  const int g16 = (lane >> 4) & 1, jj = lane & 15;
  const int vrow = 4 * h + (jj >> 2);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int lchunk = 4 * c + 2 * g16 + ((jj & 3) >> 1);
    lo.vr[c] = (uint32_t)(vrow * D * 2 + 16 * (lchunk ^ fv(vrow)) + 8 * (jj & 1));
  }
#pragma unroll
  for (int n = 0; n < kLoadsPerWave; ++n) {
    const int row = 2 * (wave * kLoadsPerWave + n) + (lane >> 5);
    const int p = lane & 31;
    lo.ld_row[n] = row;
    lo.ld_k[n] = (uint32_t)row * (uint32_t)tsb + 16u * (uint32_t)(p ^ fk(row));
    lo.ld_v[n] = (uint32_t)row * (uint32_t)tsb + 16u * (uint32_t)(p ^ fv(row));
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ const T* at_bytes(const void* base, uint32_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

__device__ __forceinline__ bf16x8 read_k(const Stage& s, const Lanes& lo, int j) {
  return *at_bytes<bf16x8>(s.k, lo.kr[j & 7] + (j >> 3) * 256u);
}

// V^T fragment for product slot j: d chunk j / 2, key half j % 2.
__device__ __forceinline__ bf16x8 read_v(const Stage& s, const Lanes& lo, int j) {
  const int c = j >> 1, a = j & 1;
  const __bf16* p = at_bytes<__bf16>(s.v, lo.vr[c & 3]) + (c >> 2) * 128 + 16 * a * D;
  const bf16x4 x0 = lds_read_tr4(p);
  const bf16x4 x1 = lds_read_tr4(p + 8 * D);
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-wave state: Q^T fragments, O^T, and the row statistics of this lane's row
// (m: reference maximum in base 2, the same in lanes l and l ^ 32; mobs: this
// lane's running maximum of its raw scores; l: this lane's sum of its weights).
struct State {
  bf16x8 qf[16];
  f32x16 o[8];
  float m, mobs, l;
  uint32_t wq;
  bool all_set;
};

__device__ __forceinline__ void init_state(State& st) {
  st.m = -INFINITY;
  st.mobs = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[c][i] = 0.f;
  st.all_set = false;
}

__device__ __forceinline__ float xhalf_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }

// Visibility of a tile's keys for this lane's row, when a kernel can form it
// without the per-pair rule: bit k set if key k of the tile is visible.
struct VisWord {
  uint32_t w;
};

// Softmax, branchy part (tile i, before its weights): the per-pair rule of a
// PARTIAL tile, and until every row of the wave has a reference maximum, the
// maxima of rows that lack one.
//   words(q): the key words of this lane's keys 8q + 4(lane/32) .. + 3 of the tile,
//             or a VisWord of the whole tile (then called once).
// A masked score becomes -inf; with a VisWord each element costs a bit-field
// extract (0 or all ones) and a bit-field insert of -inf.
template <typename Words>
__device__ __forceinline__ void softmax_pre(State& st, f32x16& s, int cls, uint32_t forbid, float scale_log2,
                                            Words words) {
  if (cls == PI_TILE_PARTIAL) {
    if constexpr (std::is_same<decltype(words(0)), VisWord>::value) {
      const uint32_t mh = words(0).w >> (4 * ((threadIdx.x >> 5) & 1));
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int bit = 8 * q + e;
          const uint32_t keep = (uint32_t)((int32_t)(mh << (31 - bit)) >> 31);
          s[4 * q + e] = __uint_as_float((__float_as_uint(s[4 * q + e]) & keep) | (0xFF800000u & ~keep));
        }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w = words(q);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!pair_visible(st.wq, w[e], forbid)) s[4 * q + e] = -INFINITY;
      }
    }
  }
  if (!st.all_set) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    const float mt = xhalf_max(mx) * scale_log2;
    st.m = (st.m == -INFINITY) ? mt : st.m;
    st.all_set = __ballot(st.m == -INFINITY) == 0ull;
  }
}

// A key tile as the loop sees it: d = tile index | class << 16 (| 1 << 24 for a
// decode suffix tile), m = its key-validity bitmap (w unused).
struct TileDesc {
  uint32_t d, m, w;
};

__device__ __forceinline__ int tile_cls(const TileDesc& t) { return (int)((t.d >> 16) & 0xFFu); }

// This wave's loads of one K/V tile, prepared once per step so that issuing one in
// a product slot is a single instruction: the two buffer resources (K and V of the
// sample, built once per kernel), the tile's byte offset from them (scalar, the
// loads' soffset) and the per-lane offsets of the wave's 2 * kLoadsPerWave loads,
// out of range (zeros) for keys outside the tile's validity mask.
struct LoadPlan {
  i32x4 rk, rv;
  uint32_t soff;
  uint32_t off[2 * kLoadsPerWave];
  uint32_t wo;        // prefill: this lane's offset of the key-word load (out of range: none)
};

template <typename LN>
__device__ __forceinline__ LoadPlan plan_kv(const LN& lo, const i32x4& rk, const i32x4& rv, int key0, int tsb,
                                           uint32_t keymask, bool live) {
  LoadPlan pl;
  pl.rk = rk;
  pl.rv = rv;
  pl.soff = (uint32_t)__builtin_amdgcn_readfirstlane(key0) * (uint32_t)tsb;
  // keys to fetch (uniform): every key of a full tile, none past the end
  const uint32_t fetch = live ? __builtin_amdgcn_readfirstlane(keymask) : 0u;
  if (fetch == 0xFFFFFFFFu) {
#pragma unroll
    for (int n = 0; n < kLoadsPerWave; ++n) {
      pl.off[n] = lo.ld_k[n];
      pl.off[kLoadsPerWave + n] = lo.ld_v[n];
    }
  } else {
#pragma unroll
    for (int n = 0; n < kLoadsPerWave; ++n) {
      const bool ok = (fetch >> lo.ld_row[n]) & 1u;
      pl.off[n] = ok ? lo.ld_k[n] : kOOB;
      pl.off[kLoadsPerWave + n] = ok ? lo.ld_v[n] : kOOB;
    }
  }
  return pl;
}

__device__ __forceinline__ void issue_planned(Stage* __restrict__ sg, const LoadPlan& pl, int n) {
  const bool isv = n >= kLoadsPerWave;
  const int nn = isv ? n - kLoadsPerWave : n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __bf16* dst = (isv ? sg->v : sg->k) + (size_t)(wave * kLoadsPerWave + nn) * 512;
  pi_buffer_load_lds(isv ? pl.rv : pl.rk, lds_u32(dst), 16, (int)pl.off[n], (int)pl.soff, 0, 0);
}

// One pipeline step (its parts do not depend on one another):
//   the branchy softmax part of tile i (mask words in cs);
//   PV:  O^T += V^T P^T for tile i-1 (weights pp, V in vs);
//   QK:  S^T = K Q^T for tile i+1 (K in ks) into sn;
//   weights of tile i (sc -> pn), the row sums and the lane maxima;
//   this wave's loads of tile i+2 into ld (plan pl), one per slot in the first half.
// Slot j holds product j of both.  A wave issues in order, so anything in a slot
// that waits on a result produced in the same slot stalls the products behind it;
// every chain is therefore spread over slots: the LDS reads run AH slots ahead of
// their products, and weight j is scaled in slot j-1, exponentiated in slot j,
// rounded to bf16 (as a pair) two slots later and summed into the row sum two
// slots after that.  Empty asm statements pin each result to its slot (left
// alone, the compiler sinks all of them below the last product).  The four
// stages are distinct, and saying so (restrict) lets the compiler see that the
// LDS reads do not depend on the loads in flight.
//   words(cs, t, q): key words of the lane's keys of tile i (descriptor t; see softmax_pre);
//   issue_words(ld, pl): the key-word load of tile i+2, if the kernel has one;
//   mid(): work for the next step (its load plan), run halfway, under the products.
template <bool PV, typename Words, typename IssueWords, typename Mid>
__device__ __forceinline__ void step_block(const Stage* __restrict__ vs, const Stage* __restrict__ cs,
                                           const Stage* __restrict__ ks, Stage* __restrict__ ld, const Lanes& lo,
                                           State& st, const bf16x8 (&pp)[2], f32x16& sc, bf16x8 (&pn)[2],
                                           f32x16& sn, const TileDesc& tcur, uint32_t forbid, float scale_log2,
                                           const LoadPlan& pl, Words words, IssueWords issue_words, Mid mid) {
  constexpr int AH = 3;
  softmax_pre(st, sc, tile_cls(tcur), forbid, scale_log2, [&](int q) { return words(cs, tcur, q); });
  issue_words(ld, pl);
  const float m_use = (st.m == -INFINITY) ? 0.f : st.m;
  bf16x8 vb[AH], kb[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if constexpr (PV) vb[j] = read_v(*vs, lo, j);
    kb[j] = read_k(*ks, lo, j);
  }
  float x[16], e[16];
  bf16x2 pk[8];
  bf16x2 ones;
  ones[0] = f2bf(1.0f);
  ones[1] = f2bf(1.0f);
  float mloc = st.mobs;
  x[0] = fmaf(sc[0], scale_log2, -m_use);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if constexpr (PV) st.o[j >> 1] = mfma32(vb[j % AH], pp[j & 1], st.o[j >> 1]);
    sn = mfma32(kb[j % AH], st.qf[j], j == 0 ? f32x16{} : sn);
    if (j + AH < 16) {
      if constexpr (PV) vb[j % AH] = read_v(*vs, lo, j + AH);
      kb[j % AH] = read_k(*ks, lo, j + AH);
    }
    e[j] = __builtin_amdgcn_exp2f(x[j]);
    asm volatile("" : "+v"(e[j]));
    if (j + 1 < 16) {
      x[j + 1] = fmaf(sc[j + 1], scale_log2, -m_use);
      asm volatile("" : "+v"(x[j + 1]));
    }
    if (j & 1) {
      mloc = fmaxf(mloc, fmaxf(sc[j - 1], sc[j]));
      asm volatile("" : "+v"(mloc));
    }
    if (j >= 3 && (j & 1)) {            // pair (j-3, j-2), exponentiated one and two slots ago
      const int pr = (j - 3) >> 1;
      pk[pr][0] = f2bf(e[j - 3]);
      pk[pr][1] = f2bf(e[j - 2]);
      asm volatile("" : "+v"(pk[pr]));
    }
    if (j >= 5 && (j & 1)) {            // the pair rounded two slots ago
      const int pr = (j - 5) >> 1;
      st.l = __builtin_amdgcn_fdot2_f32_bf16(pk[pr], ones, st.l, false);
      asm volatile("" : "+v"(st.l));
    }
    if (j < kLoadsPerWave * 2) issue_planned(ld, pl, j);   // early, so they land before the next barrier
    if (j == 8) mid();
    __builtin_amdgcn_sched_barrier(0);
  }
  // the next tile's scores stay in vector registers: the products write them there
  // and the next step's weights read them without a copy out of the accumulators
  asm volatile("" : "+v"(sn));
  // the last pairs
  pk[7][0] = f2bf(e[14]);
  pk[7][1] = f2bf(e[15]);
  st.l = __builtin_amdgcn_fdot2_f32_bf16(pk[6], ones, st.l, false);
  st.l = __builtin_amdgcn_fdot2_f32_bf16(pk[7], ones, st.l, false);
#pragma unroll
  for (int pr = 0; pr < 8; ++pr) {
    pn[pr >> 2][2 * (pr & 3)] = pk[pr][0];
    pn[pr >> 2][2 * (pr & 3) + 1] = pk[pr][1];
  }
  st.mobs = mloc;
}

__device__ __forceinline__ void pv_last(const Stage& vs, const Lanes& lo, State& st, const bf16x8 (&pp)[2]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) st.o[j >> 1] = mfma32(read_v(vs, lo, j), pp[j & 1], st.o[j >> 1]);
}


// Tile loop over tiles [i_lo, i_hi); tile j lives in stage (j - i_lo) % 4, and the
// loop is unrolled by four so every step names its stages statically.  The four
// stages are four separate LDS objects: the compiler then sees that a step's
// reads never touch the stage its loads are filling (with one array indexed at
// run time it makes every transposing read after a load wait for that load).
// Step i: barrier (this wave's loads of tile i+1 have landed; every wave is past
// step i-1, so the stage of tile i-2 is free), then the block above with tile
// i+2's loads spread through it.  Past the end, loads keep going to the free
// stage with every key out of range (zeros, no memory traffic) and the scores of
// the missing tile are computed and dropped, which keeps the block free of
// branches.
//   desc(j): tile j's descriptor (LDS reads only)
//   plan(t, live): this wave's load plan of tile t (registers only)
//   words(stage, q), issue_words(stage, plan): see step_block
//   prep(): row work that needs the Q registers, once the first loads are out
template <typename Desc, typename Plan, typename Words, typename IssueWords, typename Prep>
__device__ __forceinline__ void run_tiles(Stage& s0, Stage& s1, Stage& s2, Stage& s3, const Lanes& lo, State& st,
                                          int i_lo, int i_hi, Desc desc, Plan plan, Words words,
                                          IssueWords issue_words, Prep prep, uint32_t forbid, float scale_log2) {
  if (i_lo >= i_hi) return;
  auto clamp = [&](int i) { return i < i_hi ? i : i_lo; };
  {
    const LoadPlan p0 = plan(desc(i_lo), true);
    issue_words(&s0, p0);
#pragma unroll
    for (int n = 0; n < 2 * kLoadsPerWave; ++n) issue_planned(&s0, p0, n);
    const bool two = i_lo + 1 < i_hi;
    const LoadPlan p1 = plan(desc(clamp(i_lo + 1)), two);
    issue_words(&s1, p1);
#pragma unroll
    for (int n = 0; n < 2 * kLoadsPerWave; ++n) issue_planned(&s1, p1, n);
  }
  prep();
  // descriptors of tiles i, i+1 and i+3 and the load plan of tile i+2, for step i = i_lo
  TileDesc t_cur = desc(i_lo);
  TileDesc t_n1 = desc(clamp(i_lo + 1));
  TileDesc t_n3 = desc(clamp(i_lo + 3));
  LoadPlan pl = plan(desc(clamp(i_lo + 2)), i_lo + 2 < i_hi);
  __syncthreads();      // the first two tiles have landed
  f32x16 sc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) sc = mfma32(read_k(s0, lo, j), st.qf[j], sc);
  bf16x8 pp[2];
  // Step i: tile i+2's loads go out on the plan made during step i-1; halfway
  // through, the plan of tile i+3 is made from its descriptor, read in step i-1;
  // tile i+4's descriptor is read at the start.
  auto step = [&](auto pv, int i, Stage& prev, Stage& cur, Stage& nxt, Stage& ld) {
    __syncthreads();      // tile i+1 has landed; every wave is done with tile i-2
    const TileDesc t_n4 = desc(clamp(i + 4));
    const TileDesc t3 = t_n3;
    LoadPlan pl_next;
    bf16x8 pn[2];
    f32x16 sn;
    step_block<decltype(pv)::value>(&prev, &cur, &nxt, &ld, lo, st, pp, sc, pn, sn, t_cur, forbid,
                                    scale_log2, pl, words, issue_words,
                                    [&]() { pl_next = plan(t3, i + 3 < i_hi); });
    t_cur = t_n1;
    t_n1 = desc(clamp(i + 2));
    t_n3 = t_n4;
    pl = pl_next;
    pp[0] = pn[0];
    pp[1] = pn[1];
    sc = sn;
  };
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;
  step(NoPV{}, i_lo, s3, s0, s1, s2);
  for (int i = i_lo + 1; i < i_hi; i += 4) {
    step(WithPV{}, i, s0, s1, s2, s3);
    if (i + 1 < i_hi) step(WithPV{}, i + 1, s1, s2, s3, s0);
    if (i + 2 < i_hi) step(WithPV{}, i + 2, s2, s3, s0, s1);
    if (i + 3 < i_hi) step(WithPV{}, i + 3, s3, s0, s1, s2);
  }
  const int last = (i_hi - 1 - i_lo) & 3;
  pv_last(last == 0 ? s0 : last == 1 ? s1 : last == 2 ? s2 : s3, lo, st, pp);
}

// True if this lane's row maximum (its raw scores, both halves, scaled to base 2
// here, once) grew past the reference by more than kGrowth.
__device__ __forceinline__ bool needs_rerun(State& st, float scale_log2) {
  st.mobs = xhalf_max(st.mobs) * scale_log2;
  return st.mobs > st.m + kGrowth;
}

// Reset for the second pass: the reference becomes the row's true maximum.
__device__ __forceinline__ void reset_for_rerun(State& st) {
  st.m = st.mobs;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[c][i] = 0.f;
  st.all_set = true;
}

// Q^T fragments of this lane's row (row-major [.., d] at `qrow`): fragment j holds
// d = 16 j + 8 (lane / 32) .. + 7.
__device__ __forceinline__ void load_q_row(State& st, const __bf16* qrow) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.qf[j] = *reinterpret_cast<const bf16x8*>(qrow + 16 * j + 8 * h);
}

// The same from the operand tile layout (tiled_offset) of a matrix of width d:
// row `row` of that matrix.
__device__ __forceinline__ void load_q_tiled(State& st, const __bf16* q, int64_t row) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.qf[j] = *reinterpret_cast<const bf16x8*>(q + tiled_offset(row, 16 * j + 8 * h, D));
}

// Rotary embedding of the lane's Q row in registers: pairs (i, i + 128) sit in
// fragments j and j + 8 at the same element; pair i = 16 j + 8 (lane / 32) + e.
__device__ __forceinline__ void rotate_q(State& st, int pos, const double* inv_freq) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, sn;
      rope_cos_sin(pos, inv_freq[16 * j + 8 * h + e], c, sn);
      const float a = bf2f(st.qf[j][e]), b = bf2f(st.qf[j + 8][e]);
      st.qf[j][e] = f2bf(a * c - b * sn);
      st.qf[j + 8][e] = f2bf(b * c + a * sn);
    }
}

// Output store of the wave's 32 rows held transposed in accumulators (element
// 4q + e of acc[c] in lane l: row l % 32, d = 32 c + 8 q + 4 (l / 32) + e), each
// value times `mul`, rounded to bf16, staged through LDS: the wave writes its rows
// into `buf` (32 rows x 512 bytes; 16-byte chunk x of row r at chunk x ^ r), then
// reads them back a row per half-wave, so that every global store writes two
// whole rows in 16-byte pieces (each cache line from one instruction instead of
// from eight).
//   dst(r, x) -> where d = 8x .. 8x + 7 of the wave's row r go (nullptr: no row).
// The caller makes sure no wave still reads `buf` and no load still fills it.
template <typename Dst>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[8], float mul, __bf16* buf, Dst dst) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
  char* base = reinterpret_cast<char*>(buf);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = f2bf(acc[c][4 * q + e] * mul);
      *reinterpret_cast<bf16x4*>(base + r * 512 + 16 * ((4 * c + q) ^ r) + 8 * h) = v;
    }
  const int x = lane & 31;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = 2 * i + h;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(base + rr * 512 + 16 * (x ^ rr));
    __bf16* p = dst(rr, x);
    if (p != nullptr) *reinterpret_cast<bf16x8*>(p) = v;
  }
}

// Key-split epilogue: the unnormalised partial O^T of the wave's 32 rows in
// accumulator lane order (each store 1 KB contiguous), and (m, l) per row.
// chunk = (group * n_qblk + qblk) * NW + wave; split s at s * n_chunks + chunk.
__device__ __forceinline__ void store_partials(const State& st, float l_row, float* __restrict__ opart,
                                               float* __restrict__ mlpart, int64_t n_chunks, int64_t chunk, int split) {
  const int lane = threadIdx.x & 63;
  const int64_t at = split * n_chunks + chunk;
  f32x4* dst = reinterpret_cast<f32x4*>(opart) + at * 32 * 64 + lane;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {st.o[c][4 * q], st.o[c][4 * q + 1], st.o[c][4 * q + 2], st.o[c][4 * q + 3]};
      __builtin_nontemporal_store(v, &dst[(4 * c + q) * 64]);
    }
  if (lane < 32) {
    mlpart[at * 64 + 2 * lane] = st.m;
    mlpart[at * 64 + 2 * lane + 1] = l_row;
  }
}

// ---------------------------------------------------------------------------
// Prefill: one group per (sample, KV head, key split), n_qblk blocks of 16 query
// tokens each, XCD-placed.  The workgroup reads its 16-token row of the mask's
// tile table and compacts its non-EMPTY key tiles into an LDS list.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill32_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                 __bf16* __restrict__ o, int B, int L, int Hq, int Hkv, float scale_log2,
                 const uint32_t* __restrict__ tok, const uint8_t* __restrict__ tiles, int n_qt, int n_kt,
                 uint32_t forbid, Placement place, int n_split, float* __restrict__ opart,
                 float* __restrict__ mlpart, const int32_t* __restrict__ rope_pos, double rope_log2_base,
                 float* __restrict__ lse) {
  __shared__ Stage stage0, stage1, stage2, stage3;
  __shared__ uint32_t kmask[kMaxTiles];
  __shared__ uint32_t tlist[kMaxTiles];
  __shared__ u32x2 tdesc[kMaxTiles];      // (tile | class << 16, key-validity bitmap) of list entry i
  __shared__ double rope_if[D / 2];
  __shared__ int tcount;
  int grp, qblk;
  if (!xcd_place(place, grp, qblk)) return;
  if (rope_pos != nullptr)
    for (int i = threadIdx.x; i < D / 2; i += THREADS) rope_if[i] = rope_inv_freq(i, D, rope_log2_base);
  const int group = grp / n_split, split = grp % n_split;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = qblk * TOK;
  const uint32_t* tk = tok + (size_t)b * L;

  query_block_tiles(tk, L, tiles + (size_t)b * n_qt * n_kt, n_qt, n_kt, tok0, TOK, NW, kmask, tlist, &tcount);

  // this lane's row: token t, head h (rows past the last token read token 0 and are
  // never stored); the Q loads go out after the setup's reads (measured: issuing
  // them first, so the setup's waits cover them too, costs 2-3 %)
  const int row = wave * ROWS_W + (lane & 31);
  const int t = tok0 + row / G;
  const int hq = kvh * G + row % G;
  const bool row_ok = t < L;
  State st;
  init_state(st);
  st.wq = row_ok ? tk[t] : 0u;
  load_q_row(st, q + (((int64_t)b * L + (row_ok ? t : 0)) * Hq + hq) * D);
  __syncthreads();
  const int count = tcount;
  // one 8-byte descriptor per list entry, so the loop fetches a tile's with a single read
  for (int i = threadIdx.x; i < count; i += THREADS) {
    const uint32_t d = tlist[i];
    tdesc[i] = u32x2{d, kmask[d & 0xFFFFu]};
  }
  __syncthreads();

  const __bf16* k0 = k + ((size_t)b * L * Hkv + kvh) * D;
  const __bf16* v0 = v + ((size_t)b * L * Hkv + kvh) * D;
  const i32x4 rw = make_rsrc(tk);
  const i32x4 rk0 = make_rsrc(k0), rv0 = make_rsrc(v0);
  const int tsb = Hkv * D * 2;
  const Lanes lo = make_lanes(tsb);
  auto desc = [&](int i) {
    const u32x2 dm = tdesc[i];
    return TileDesc{dm[0], dm[1], 0u};
  };
  auto plan = [&](const TileDesc& td, bool live) {
    const int key0 = (int)(td.d & 0xFFFFu) * TK;
    LoadPlan pl = plan_kv(lo, rk0, rv0, key0, tsb, td.m, live);
    pl.wo = (live && lane < TK && key0 + lane < L) ? (uint32_t)(key0 + lane) * 4u : kOOB;
    return pl;
  };
  // the tile's key words: one small load by wave 0, with its K/V loads
  auto issue_words = [&](Stage* sg, const LoadPlan& pl) {
    if (wave == 0) pi_buffer_load_lds(rw, lds_u32(&sg->w[0]), 4, (int)pl.wo, 0, 0, 0);
  };
  auto words = [&](const Stage* cs, const TileDesc&, int q) {
    return *reinterpret_cast<const u32x4*>(&cs->w[8 * q + 4 * (lane >> 5)]);
  };
  const int i_lo = (int)((int64_t)count * split / n_split);
  const int i_hi = (int)((int64_t)count * (split + 1) / n_split);
  bool rotated = rope_pos == nullptr;
  auto prep = [&]() {
    if (rotated) return;
    rotate_q(st, rope_pos[(int64_t)b * L + min(t, L - 1)], rope_if);
    rotated = true;
  };
  auto run = [&]() { run_tiles(stage0, stage1, stage2, stage3, lo, st, i_lo, i_hi, desc, plan, words, issue_words, prep, forbid,
              scale_log2);
  };
  run();
  if (__syncthreads_or(needs_rerun(st, scale_log2))) {
    reset_for_rerun(st);
    run();
  }
  const float l_row = st.l + __shfl_xor(st.l, 32);
  if (n_split == 1) {
    if (lse != nullptr && lane < 32 && row_ok)
      lse[((int64_t)b * L + t) * Hq + hq] =
          l_row > 0.f ? (st.m + log2f(l_row)) * 0.6931471805599453f : -INFINITY;
    // the stages are free once every wave is past its last read and its (dead) loads have landed
    wait_vmem();
    __syncthreads();
    __bf16* buf = wave == 0 ? stage0.k : wave == 1 ? stage0.v : wave == 2 ? stage1.k : stage1.v;
    // the wave's rows are 4 consecutive tokens x this KV head's 8 query heads
    store_rows_staged(st.o, l_row > 0.f ? 1.f / l_row : 0.f, buf, [&](int r, int x) -> __bf16* {
      const int tr = tok0 + (wave * ROWS_W + r) / G;
      return tr < L ? o + (((int64_t)b * L + tr) * Hq + kvh * G + r % G) * D + 8 * x : nullptr;
    });
    return;
  }
  const int64_t n_chunks = (int64_t)B * Hkv * place.n_sub * NW;
  store_partials(st, l_row, opart, mlpart, n_chunks, ((int64_t)group * place.n_sub + qblk) * NW + wave, split);
}

// ---------------------------------------------------------------------------
// Cached suffix decode (Hq = 8, Hkv = 1): one group per (sample, key split),
// n_qblk blocks of 16 suffix tokens each, XCD-placed.  Keys: the valid prefix
// slots of the cache layer, then the suffix's own K/V; query / key words reuse
// the prefill rule with bid 0 for every prefix slot and 1 + cumsum(suffix_ar)
// for suffix tokens.  Fully padded cache tiles are never fetched.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode32_kernel(const __bf16* __restrict__ ck, const __bf16* __restrict__ cv,
                const uint8_t* __restrict__ prefix_mask, int cap, int P,
                const __bf16* __restrict__ qs, const __bf16* __restrict__ ks, const __bf16* __restrict__ vs,
                const uint8_t* __restrict__ suffix_ar, int B, int S, float scale_log2,
                __bf16* __restrict__ os, int tiled, Placement place, int n_split, float* __restrict__ opart,
                float* __restrict__ mlpart, int rope, double rope_log2_base) {
  __shared__ Stage stage0, stage1, stage2, stage3;
  __shared__ uint32_t sbid[128];
  __shared__ int send[128];        // end of suffix token u's block: the first later block start, or S
  __shared__ uint32_t pmask[kMaxTiles];
  __shared__ u32x2 tdesc[kMaxTiles];      // (tile | class << 16 | suffix << 24, key-validity bitmap)
  __shared__ double rope_if[D / 2];
  __shared__ int tcount;
  int grp, qblk;
  if (!xcd_place(place, grp, qblk)) return;
  if (rope)
    for (int i = threadIdx.x; i < D / 2; i += THREADS) rope_if[i] = rope_inv_freq(i, D, rope_log2_base);
  const int b = grp / n_split, split = grp % n_split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = qblk * TOK;
  const int n_pt = (P + TK - 1) / TK;
  const int n_st = (S + TK - 1) / TK;

  // this lane's row; its Q loads go out first and stay in flight through the setup
  const int row = wave * ROWS_W + (lane & 31);
  const int t = tok0 + row / G;
  const int hq = row % G;
  const bool row_ok = t < S;
  State st;
  init_state(st);
  if (tiled) {
    // this sample's queries: rows t*8 + head of a tile-layout matrix of width 256,
    // padded to whole 16-row blocks; blocks past the padding read block 0
    const int padded = (S * G + 15) / 16 * 16;
    int r = tok0 * G + row;
    if (r >= padded) r &= 15;
    load_q_tiled(st, qs, (int64_t)b * padded + r);
  } else {
    load_q_row(st, qs + (((int64_t)b * S + (row_ok ? t : 0)) * G + hq) * D);
  }
  // the suffix's block flags (S <= 128), then the validity bitmap of the prefix
  // slots, one 32-bit word per tile, the bytes of up to eight rounds loaded
  // before the first ballot: one memory latency for all of the setup's reads
  int a0 = lane < S ? (suffix_ar[lane] != 0) : 0;
  int a1 = lane + 64 < S ? (suffix_ar[lane + 64] != 0) : 0;
  const uint8_t* pm = prefix_mask + (size_t)b * cap;
  for (int base0 = wave * 64; base0 < n_pt * TK; base0 += 8 * THREADS) {
    bool valid[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int slot = base0 + u * THREADS + lane;
      valid[u] = slot < P && pm[slot] != 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = base0 + u * THREADS;
      if (base >= n_pt * TK) break;
      const unsigned long long bal = __ballot(valid[u]);
      if (lane == 0) pmask[base / TK] = (uint32_t)bal;
      if (lane == 32 && base / TK + 1 < n_pt) pmask[base / TK + 1] = (uint32_t)(bal >> 32);
    }
  }
  // suffix block ids: inclusive cumsum of the flags, by wave 0; and the end of
  // each token's block (the first flagged position after it, or S), from a
  // suffix minimum of the flagged positions
  if (wave == 0) {
    constexpr int kNone = 1 << 20;
    int p0 = a0 ? lane : kNone, p1 = a1 ? lane + 64 : kNone;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v0 = __shfl_down(p0, off), v1 = __shfl_down(p1, off);
      if (lane + off < 64) {
        p0 = min(p0, v0);
        p1 = min(p1, v1);
      }
    }
    const int min_hi = __shfl(p1, 0);          // first flag in [64, 128)
    const int n0 = __shfl_down(p0, 1), n1 = __shfl_down(p1, 1);
    send[lane] = min(S, lane == 63 ? min_hi : min(n0, min_hi));
    send[lane + 64] = min(S, lane == 63 ? kNone : n1);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u0 = __shfl_up(a0, off), u1 = __shfl_up(a1, off);
      if (lane >= off) {
        a0 += u0;
        a1 += u1;
      }
    }
    const int tot0 = __shfl(a0, 63);
    sbid[lane] = 1u | ((uint32_t)(1 + a0) << 3);
    sbid[lane + 64] = 1u | ((uint32_t)(1 + tot0 + a1) << 3);
  }
  __syncthreads();
  // compact tile list: non-empty prefix tiles, then the suffix tiles
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base < n_pt + n_st; base += 64) {
      const int i = base + lane;
      uint32_t m = 0u, d = 0u;
      if (i < n_pt) {
        m = pmask[i];
        d = (uint32_t)i | ((uint32_t)(m == 0xFFFFFFFFu ? PI_TILE_FULL : PI_TILE_PARTIAL) << 16);
      } else if (i < n_pt + n_st) {
        const int nv = min(TK, S - (i - n_pt) * TK);
        m = nv == TK ? 0xFFFFFFFFu : ((1u << nv) - 1u);
        d = (uint32_t)(i - n_pt) | ((uint32_t)PI_TILE_PARTIAL << 16) | (1u << 24);
      }
      const unsigned long long bal = __ballot(m != 0u);
      if (m != 0u) {
        const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
        tdesc[pos] = u32x2{d, m};
      }
      cnt += __popcll(bal);
    }
    if (lane == 0) tcount = cnt;
  }
  __syncthreads();
  st.wq = row_ok ? sbid[t] : 0u;
  // the suffix keys this row sees: [0, lim) (block ids never decrease along the suffix)
  const int lim = row_ok ? send[t] : 0;
  const int i_lo = (int)((int64_t)tcount * split / n_split);
  const int i_hi = (int)((int64_t)tcount * (split + 1) / n_split);

  const __bf16* k0 = ck + (size_t)b * cap * D;
  const __bf16* v0 = cv + (size_t)b * cap * D;
  const __bf16* ks0 = ks + (size_t)b * S * D;
  const __bf16* vs0 = vs + (size_t)b * S * D;
  const i32x4 rk0 = make_rsrc(k0), rv0 = make_rsrc(v0), rks = make_rsrc(ks0), rvs = make_rsrc(vs0);
  const Lanes lo = make_lanes(D * 2);
  auto desc = [&](int i) {
    const u32x2 dm = tdesc[i];
    return TileDesc{dm[0], dm[1], 0u};
  };
  auto plan = [&](const TileDesc& td, bool live) {
    const uint32_t d = __builtin_amdgcn_readfirstlane(td.d);   // uniform: the resources are picked in scalars
    const int key0 = (int)(d & 0xFFFFu) * TK;
    const bool suffix = (d >> 24) & 1u;
    LoadPlan pl = plan_kv(lo, suffix ? rks : rk0, suffix ? rvs : rv0, key0, D * 2, td.m, live);
    pl.wo = kOOB;
    return pl;
  };
  auto issue_words = [](Stage*, const LoadPlan&) {};
  // visibility of the current tile's keys (masked tiles only): a cache slot is seen
  // by every row of the suffix if it is valid; suffix key u by the rows whose block
  // ends past u
  auto words = [&](const Stage*, const TileDesc& tl, int) {
    const uint32_t d = tl.d;
    if ((d >> 24) & 1u) {
      const int lj = lim - TK * (int)(d & 0xFFFFu);
      return VisWord{lj >= TK ? 0xFFFFFFFFu : lj <= 0 ? 0u : (1u << lj) - 1u};
    }
    return VisWord{row_ok ? tl.m : 0u};
  };
  bool rotated = !rope;
  auto prep = [&]() {
    if (rotated) return;
    int n_valid = 0;
    for (int w = lane; w < n_pt; w += 64) n_valid += __popc(pmask[w]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n_valid += __shfl_xor(n_valid, off);
    rotate_q(st, n_valid + t, rope_if);
    rotated = true;
  };
  auto run = [&]() { run_tiles(stage0, stage1, stage2, stage3, lo, st, i_lo, i_hi, desc, plan, words, issue_words, prep, 0u,
              scale_log2);
  };
  run();
  if (__syncthreads_or(needs_rerun(st, scale_log2))) {
    reset_for_rerun(st);
    run();
  }
  const float l_row = st.l + __shfl_xor(st.l, 32);
  if (n_split == 1) {
    wait_vmem();
    __syncthreads();
    __bf16* buf = wave == 0 ? stage0.k : wave == 1 ? stage0.v : wave == 2 ? stage1.k : stage1.v;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    // the wave's rows: 4 consecutive suffix tokens x 8 heads
    if (tiled) {
      store_rows_staged(st.o, inv, buf, [&](int r, int x) -> __bf16* {
        const int tr = tok0 + (wave * ROWS_W + r) / G;
        return tr < S ? os + tiled_offset((int64_t)b * S + tr, (r % G) * D + 8 * x, G * D) : nullptr;
      });
    } else {
      store_rows_staged(st.o, inv, buf, [&](int r, int x) -> __bf16* {
        const int tr = tok0 + (wave * ROWS_W + r) / G;
        return tr < S ? os + (((int64_t)b * S + tr) * G + r % G) * D + 8 * x : nullptr;
      });
    }
    return;
  }
  const int64_t n_chunks = (int64_t)B * place.n_sub * NW;
  store_partials(st, l_row, opart, mlpart, n_chunks, ((int64_t)b * place.n_sub + qblk) * NW + wave, split);
}

// Merge the key splits of one 32-row chunk: O = sum_s 2^(m_s - M) O_s / sum_s
// 2^(m_s - M) l_s, M = max_s m_s.  One wave per (chunk, 32-wide d chunk), four
// waves per workgroup; every lane merges its row's 16 values of the d chunk.
__global__ void __launch_bounds__(256)
combine32_kernel(const float* __restrict__ opart, const float* __restrict__ mlpart, __bf16* __restrict__ out,
                 int o_tiled, int64_t n_chunks, int n_qblk, int L, int Hq, int n_split, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t chunk = blockIdx.x >> 1;
  const int c = (blockIdx.x & 1) * 4 + (threadIdx.x >> 6);
  if (chunk >= n_chunks) return;
  const int wave_in = (int)(chunk % NW);
  const int64_t gq = chunk / NW;               // group * n_qblk + qblk
  const int qblk = (int)(gq % n_qblk);
  const int64_t group = gq / n_qblk;           // sample * Hkv + kv head
  const int Hkv = Hq / G;
  const int64_t b = group / Hkv;
  const int kvh = (int)(group % Hkv);
  const int row = wave_in * ROWS_W + (lane & 31);
  const int t = qblk * TOK + row / G;
  const int hq = kvh * G + row % G;
  const int h = lane >> 5;
  // every split's (m, l) and the first eight splits' O values are loaded before
  // the first use, so the merge waits on one memory latency (two past 8 splits)
  constexpr int kBatch = 8;
  static_assert(kMaxSplit32 == 2 * kBatch, "two batches of splits");
  float ms[kMaxSplit32], ls[kMaxSplit32];
#pragma unroll
  for (int sp = 0; sp < kMaxSplit32; ++sp) {
    const int64_t at = sp * n_chunks + chunk;
    ms[sp] = sp < n_split ? mlpart[at * 64 + 2 * (lane & 31)] : -INFINITY;
    ls[sp] = sp < n_split ? mlpart[at * 64 + 2 * (lane & 31) + 1] : 0.f;
  }
  f32x4 acc[4] = {};
  float Ls = 0.f, M = -INFINITY;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half * kBatch >= n_split) break;
    f32x4 op[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sp = half * kBatch + u;
      const f32x4* src = reinterpret_cast<const f32x4*>(opart) + (sp * n_chunks + chunk) * 32 * 64 + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        op[u][q] = sp < n_split ? __builtin_nontemporal_load(&src[(4 * c + q) * 64]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (half == 0) {
#pragma unroll
      for (int sp = 0; sp < kMaxSplit32; ++sp) M = fmaxf(M, ms[sp]);
    }
    if (M == -INFINITY) break;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sp = half * kBatch + u;
      const float w = (ms[sp] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[sp] - M);
      Ls += w * ls[sp];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += w * op[u][q];
    }
  }
  if (t >= L) return;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  if (lse != nullptr && c == 0 && h == 0)
    lse[(b * L + t) * Hq + hq] = Ls > 0.f ? (M + log2f(Ls)) * 0.6931471805599453f : -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f2bf(acc[q][e] * inv);
    const int d = 32 * c + 8 * q + 4 * h;
    __bf16* dst = o_tiled ? out + tiled_offset(b * L + t, hq * D + d, Hq * D) : out + ((b * L + t) * Hq + hq) * D + d;
    *reinterpret_cast<bf16x4*>(dst) = v;
  }
}

// Key splits: enough workgroups to cover the chip (about 256), each split with
// at least min_tiles key tiles, at most 16 splits.
int splits_for(int groups, int n_qblk, int tiles, int min_tiles) {
  const int by_chip = 256 / std::max(1, groups * n_qblk);
  return std::max(1, std::min({kMaxSplit32, by_chip, tiles / min_tiles}));
}

size_t split_bytes(int groups, int n_qblk, int splits) {
  if (splits <= 1) return 0;
  const size_t chunks = (size_t)splits * groups * n_qblk * NW;
  return pi::align_up(chunks * 32 * 256 * sizeof(float), 256) + chunks * 64 * sizeof(float);
}

// ---------------------------------------------------------------------------
// dQ of the attention backward on the same engine (Hq = 8, Hkv = 1): the
// forward's step with the softmax replaced by the weights of the backward.  Per
// query row (this lane's row of the wave's 32): P = exp2(c2 S - lse2) from the
// row's log-sum-exp (no running maximum), dS = P (dP - Dr), dQ = scale sum_j
// dS_j k_j.  Per 32-key tile: S^T = K Q^T and dP^T = V dO^T (row-wise reads of
// K and V, Q^T and dO^T from registers), then dQ^T += K^T dS^T with dS^T taken
// straight from the accumulators as the forward's P^T, and K^T from two
// transposing reads of the K tile.  K is read both ways, so its tile takes a
// swizzle that serves both (dqsw); V is only read row-wise (fk).
// ---------------------------------------------------------------------------

// Logical 16-byte chunk x of K row r sits at x ^ dqsw(r): over r & 15 every value
// once, rows r and r + 8 differ in chunk bit 3 (row-wise read), and each aligned
// group of 4 rows differs in chunk bits 2-3 (the transposing read's 4 rows x 64
// bytes then cover all 64 banks).
__device__ __forceinline__ int dqsw(int r) { return (((r & 3) ^ ((r >> 2) & 2)) << 2) | ((r >> 2) & 3); }

// Per-lane byte offsets (lane l, h = l / 32):
//   kr[j] / vr[j]: row-wise A fragment j (< 8; j + 8 is + 256 bytes) of K / V: row
//                  l % 32, logical chunk 2j + h.
//   tr[c][e]: transposing read e of the K^T fragment of d chunk c (< 4; c + 4 is
//             + 256 bytes): keys 8e + 4h .. + 3, column 32c + l % 32 (key half a
//             adds 16 keys: dqsw sees only r & 15).
//   ld_k / ld_v / ld_row: this wave's loads, as in Lanes.
struct DqLanes {
  uint32_t kr[8], vr[8];
  uint32_t tr[4][2];
  uint32_t ld_k[kLoadsPerWave], ld_v[kLoadsPerWave];
  int ld_row[kLoadsPerWave];
};

__device__ __forceinline__ DqLanes make_dq_lanes(int tsb) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  DqLanes lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo.kr[j] = (uint32_t)(r * D * 2 + 16 * ((2 * j + h) ^ dqsw(r)));
    lo.vr[j] = (uint32_t)(r * D * 2 + 16 * ((2 * j + h) ^ fk(r)));
  }
  const int g16 = (lane >> 4) & 1, jj = lane & 15;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int kr = 8 * e + 4 * h + (jj >> 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int x = 4 * c + 2 * g16 + ((jj & 3) >> 1);
      lo.tr[c][e] = (uint32_t)(kr * D * 2 + 16 * (x ^ dqsw(kr)) + 8 * (jj & 1));
    }
  }
#pragma unroll
  for (int n = 0; n < kLoadsPerWave; ++n) {
    const int row = 2 * (wave * kLoadsPerWave + n) + (lane >> 5);
    const int p = lane & 31;
    lo.ld_row[n] = row;
    lo.ld_k[n] = (uint32_t)row * (uint32_t)tsb + 16u * (uint32_t)(p ^ dqsw(row));
    lo.ld_v[n] = (uint32_t)row * (uint32_t)tsb + 16u * (uint32_t)(p ^ fk(row));
  }
  return lo;
}

__device__ __forceinline__ bf16x8 dq_read_k(const Stage& s, const DqLanes& lo, int j) {
  return *at_bytes<bf16x8>(s.k, lo.kr[j & 7] + (j >> 3) * 256u);
}
__device__ __forceinline__ bf16x8 dq_read_v(const Stage& s, const DqLanes& lo, int j) {
  return *at_bytes<bf16x8>(s.v, lo.vr[j & 7] + (j >> 3) * 256u);
}
// K^T fragment for product slot j: d chunk j / 2, key half j % 2.
__device__ __forceinline__ bf16x8 dq_read_kt(const Stage& s, const DqLanes& lo, int j) {
  const int c = j >> 1, a = j & 1;
  const char* base = reinterpret_cast<const char*>(s.k) + (c >> 2) * 256 + a * (16 * D * 2);
  const bf16x4 x0 = lds_read_tr4(reinterpret_cast<const __bf16*>(base + lo.tr[c & 3][0]));
  const bf16x4 x1 = lds_read_tr4(reinterpret_cast<const __bf16*>(base + lo.tr[c & 3][1]));
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per wave: Q^T and dO^T fragments of this lane's row (as State::qf), dQ^T in
// the accumulator layout (chunk c, element i: d = 32c + 8(i/4) + 4h + i%4), the
// row's lse2 (base 2; +inf: no visible key) and Dr, and its query word.
struct DqState {
  bf16x8 qf[16], of[16];
  f32x16 acc[8];
  float l2, dr;
  uint32_t wq;
};

// One dQ step: S^T and dP^T of tile i+1 (K, V in `ks`), dQ^T += K^T dS^T of tile
// i-1 (K of `vs`, dS^T in pp), and tile i's weights from sc / dc (mask words in
// `cs`), with this wave's loads of tile i+2 into `ld` and the next plan (mid)
// halfway.  Weight j: scaled in slot j-1, exponentiated in slot j, multiplied
// by (dP - Dr) in slot j+1, rounded to bf16 as a pair two slots after that.
template <bool PV, typename Words, typename IssueWords, typename Mid>
__device__ __forceinline__ void dq_block(const Stage* __restrict__ vs, const Stage* __restrict__ cs,
                                         const Stage* __restrict__ ks, Stage* __restrict__ ld, const DqLanes& lo,
                                         DqState& st, const bf16x8 (&pp)[2], f32x16& sc, const f32x16& dc,
                                         bf16x8 (&pn)[2], f32x16& sn, f32x16& dn, const TileDesc& tcur,
                                         uint32_t forbid, float c2, const LoadPlan& pl, Words words,
                                         IssueWords issue_words, Mid mid) {
  constexpr int AH = 2;
  if (tile_cls(tcur) == PI_TILE_PARTIAL) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = words(cs, tcur, q);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!pair_visible(st.wq, w[e], forbid)) sc[4 * q + e] = -INFINITY;
    }
  }
  issue_words(ld, pl);
  bf16x8 tb[AH], kb[AH], vb[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if constexpr (PV) tb[j] = dq_read_kt(*vs, lo, j);
    kb[j] = dq_read_k(*ks, lo, j);
    vb[j] = dq_read_v(*ks, lo, j);
  }
  float x[16], e[16];
  bf16x2 pk[8];
  x[0] = fmaf(sc[0], c2, -st.l2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if constexpr (PV) st.acc[j >> 1] = mfma32(tb[j % AH], pp[j & 1], st.acc[j >> 1]);
    sn = mfma32(kb[j % AH], st.qf[j], j == 0 ? f32x16{} : sn);
    dn = mfma32(vb[j % AH], st.of[j], j == 0 ? f32x16{} : dn);
    if (j + AH < 16) {
      if constexpr (PV) tb[j % AH] = dq_read_kt(*vs, lo, j + AH);
      kb[j % AH] = dq_read_k(*ks, lo, j + AH);
      vb[j % AH] = dq_read_v(*ks, lo, j + AH);
    }
    e[j] = __builtin_amdgcn_exp2f(x[j]);
    asm volatile("" : "+v"(e[j]));
    if (j + 1 < 16) {
      x[j + 1] = fmaf(sc[j + 1], c2, -st.l2);
      asm volatile("" : "+v"(x[j + 1]));
    }
    if (j >= 1) {
      e[j - 1] *= dc[j - 1] - st.dr;
      asm volatile("" : "+v"(e[j - 1]));
    }
    if (j >= 3 && (j & 1)) {            // pair (j-3, j-2)
      const int pr = (j - 3) >> 1;
      pk[pr][0] = f2bf(e[j - 3]);
      pk[pr][1] = f2bf(e[j - 2]);
      asm volatile("" : "+v"(pk[pr]));
    }
    if (j < kLoadsPerWave * 2) issue_planned(ld, pl, j);
    if (j == 8) mid();
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("" : "+v"(sn));
  asm volatile("" : "+v"(dn));
  e[15] *= dc[15] - st.dr;
  pk[6][0] = f2bf(e[12]);
  pk[6][1] = f2bf(e[13]);
  pk[7][0] = f2bf(e[14]);
  pk[7][1] = f2bf(e[15]);
#pragma unroll
  for (int pr = 0; pr < 8; ++pr) {
    pn[pr >> 2][2 * (pr & 3)] = pk[pr][0];
    pn[pr >> 2][2 * (pr & 3) + 1] = pk[pr][1];
  }
}

// The dQ tile loop, organised as run_tiles: tile j in stage (j - i_lo) % 4, tile
// i+2 loading during step i, descriptors and plans one step ahead.
template <typename Desc, typename Plan, typename Words, typename IssueWords>
__device__ __forceinline__ void dq_tiles(Stage& s0, Stage& s1, Stage& s2, Stage& s3, const DqLanes& lo, DqState& st,
                                         int i_lo, int i_hi, Desc desc, Plan plan, Words words,
                                         IssueWords issue_words, uint32_t forbid, float c2) {
  if (i_lo >= i_hi) return;
  auto clamp = [&](int i) { return i < i_hi ? i : i_lo; };
  {
    const LoadPlan p0 = plan(desc(i_lo), true);
    issue_words(&s0, p0);
#pragma unroll
    for (int n = 0; n < 2 * kLoadsPerWave; ++n) issue_planned(&s0, p0, n);
    const bool two = i_lo + 1 < i_hi;
    const LoadPlan p1 = plan(desc(clamp(i_lo + 1)), two);
    issue_words(&s1, p1);
#pragma unroll
    for (int n = 0; n < 2 * kLoadsPerWave; ++n) issue_planned(&s1, p1, n);
  }
  TileDesc t_cur = desc(i_lo);
  TileDesc t_n1 = desc(clamp(i_lo + 1));
  TileDesc t_n3 = desc(clamp(i_lo + 3));
  LoadPlan pl = plan(desc(clamp(i_lo + 2)), i_lo + 2 < i_hi);
  __syncthreads();      // the first two tiles have landed
  f32x16 sc = {}, dc = {};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sc = mfma32(dq_read_k(s0, lo, j), st.qf[j], sc);
    dc = mfma32(dq_read_v(s0, lo, j), st.of[j], dc);
  }
  bf16x8 pp[2];
  auto step = [&](auto pv, int i, Stage& prev, Stage& cur, Stage& nxt, Stage& ld) {
    __syncthreads();      // tile i+1 has landed; every wave is done with tile i-2
    const TileDesc t_n4 = desc(clamp(i + 4));
    const TileDesc t3 = t_n3;
    LoadPlan pl_next;
    bf16x8 pn[2];
    f32x16 sn, dn;
    dq_block<decltype(pv)::value>(&prev, &cur, &nxt, &ld, lo, st, pp, sc, dc, pn, sn, dn, t_cur, forbid, c2, pl,
                                  words, issue_words, [&]() { pl_next = plan(t3, i + 3 < i_hi); });
    t_cur = t_n1;
    t_n1 = desc(clamp(i + 2));
    t_n3 = t_n4;
    pl = pl_next;
    pp[0] = pn[0];
    pp[1] = pn[1];
    sc = sn;
    dc = dn;
  };
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;
  step(NoPV{}, i_lo, s3, s0, s1, s2);
  for (int i = i_lo + 1; i < i_hi; i += 4) {
    step(WithPV{}, i, s0, s1, s2, s3);
    if (i + 1 < i_hi) step(WithPV{}, i + 1, s1, s2, s3, s0);
    if (i + 2 < i_hi) step(WithPV{}, i + 2, s2, s3, s0, s1);
    if (i + 3 < i_hi) step(WithPV{}, i + 3, s3, s0, s1, s2);
  }
  const int last = (i_hi - 1 - i_lo) & 3;
  const Stage& sl = last == 0 ? s0 : last == 1 ? s1 : last == 2 ? s2 : s3;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.acc[j >> 1] = mfma32(dq_read_kt(sl, lo, j), pp[j & 1], st.acc[j >> 1]);
}

// One workgroup per (sample, block of 16 query tokens), XCD-placed per sample
// (q, dO, dq [B, L, 8, 256]; k, v [B, L, 1, 256]; lse2, dr [B, L, 8]).  Rows of
// padded tokens take zero Q and dO, rows past the last token read token 0 and
// are never stored.
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
dq32_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
            const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dr,
            __bf16* __restrict__ dq, int L, float scale, float c2, const uint32_t* __restrict__ tok,
            const uint8_t* __restrict__ tiles, int n_qt, int n_kt, uint32_t forbid, Placement place) {
  __shared__ Stage stage0, stage1, stage2, stage3;
  __shared__ uint32_t kmask[kMaxTiles];
  __shared__ uint32_t tlist[kMaxTiles];
  __shared__ u32x2 tdesc[kMaxTiles];
  __shared__ int tcount;
  int b, qblk;
  if (!xcd_place(place, b, qblk)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = qblk * TOK;
  const uint32_t* tk = tok + (size_t)b * L;

  query_block_tiles(tk, L, tiles + (size_t)b * n_qt * n_kt, n_qt, n_kt, tok0, TOK, NW, kmask, tlist, &tcount);

  const int row = wave * ROWS_W + (lane & 31);
  const int t = tok0 + row / G;
  const int hq = row % G;
  const bool row_ok = t < L;
  DqState st;
  {
    const int64_t r = ((int64_t)b * L + (row_ok ? t : 0)) * G + hq;
    st.wq = row_ok ? tk[t] : 0u;
    const bool live = (st.wq & 1u) != 0u;
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(q + r * D + 16 * j + 8 * h);
      const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + r * D + 16 * j + 8 * h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st.qf[j][e] = live ? a[e] : f2bf(0.f);
        st.of[j][e] = live ? d[e] : f2bf(0.f);
      }
    }
    st.l2 = lse2[r];
    st.dr = dr[r];
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[c] = f32x16{};
  }
  __syncthreads();
  const int count = tcount;
  for (int i = threadIdx.x; i < count; i += THREADS) {
    const uint32_t d = tlist[i];
    tdesc[i] = u32x2{d, kmask[d & 0xFFFFu]};
  }
  __syncthreads();

  const i32x4 rw = make_rsrc(tk);
  const i32x4 rk0 = make_rsrc(k + (size_t)b * L * D), rv0 = make_rsrc(v + (size_t)b * L * D);
  const int tsb = D * 2;
  const DqLanes lo = make_dq_lanes(tsb);
  auto desc = [&](int i) {
    const u32x2 dm = tdesc[i];
    return TileDesc{dm[0], dm[1], 0u};
  };
  auto plan = [&](const TileDesc& td, bool live) {
    const int key0 = (int)(td.d & 0xFFFFu) * TK;
    LoadPlan pl = plan_kv(lo, rk0, rv0, key0, tsb, td.m, live);
    pl.wo = (live && lane < TK && key0 + lane < L) ? (uint32_t)(key0 + lane) * 4u : kOOB;
    return pl;
  };
  auto issue_words = [&](Stage* sg, const LoadPlan& pl) {
    if (wave == 0) pi_buffer_load_lds(rw, lds_u32(&sg->w[0]), 4, (int)pl.wo, 0, 0, 0);
  };
  auto words = [&](const Stage* cs, const TileDesc&, int qq) {
    return *reinterpret_cast<const u32x4*>(&cs->w[8 * qq + 4 * (lane >> 5)]);
  };
  dq_tiles(stage0, stage1, stage2, stage3, lo, st, 0, count, desc, plan, words, issue_words, forbid, c2);
  // the stages are free once every wave is past its last read and its (dead) loads have landed
  wait_vmem();
  __syncthreads();
  __bf16* buf = wave == 0 ? stage0.k : wave == 1 ? stage0.v : wave == 2 ? stage1.k : stage1.v;
  store_rows_staged(st.acc, scale, buf, [&](int r, int x) -> __bf16* {
    const int tr = tok0 + (wave * ROWS_W + r) / G;
    return tr < L ? dq + (((int64_t)b * L + tr) * G + r % G) * D + 8 * x : nullptr;
  });
}

// ---------------------------------------------------------------------------
// dK, dV on the 32 x 32 x 16 engine (key-major).  A workgroup owns 64 keys of one
// sample as two pairs of waves, 32 keys per pair; the query rows stream through
// four stages, 32 rows (4 tokens x 8 heads) per step.  In a pair, wave A holds
// its keys' K^T fragments and dV^T, wave B their V^T fragments and dK^T:
//   A: S = Q K^T (row-wise Q reads), P = exp2(S c2 - lse2) on the visible pairs,
//      dV^T += dO^T P (transposing dO reads); P goes to B through LDS, in fp32;
//   B: dP = dO V^T (row-wise dO reads), dS = P (dP - Dr), dK^T += Q^T dS
//      (transposing Q reads).
// Lane l of either wave holds key l % 32 and query rows 8(i/4) + 4(l/32) + i%4 of
// its S / dP accumulator, which is the B-operand layout of the dV / dK products
// once their A operands (the transposing reads) order the rows the same way.
// Step m: A runs dV += dO^T(m-1) P(m-1) and S(m+1) slot by slot while it turns
// S(m) into P(m) (written to the exchange slot of tile m); B reads P(m-1)
// (written by A in step m-1), forms dS(m-1) while its dP(m) products start, and
// runs dK += Q^T(m-1) dS(m-1) eight slots behind them.  A step touches tiles
// m-1, m and m+1 while tile m+2 loads: four stages.  Steps run for m = 0 .. n,
// the first without the dV / dK products, the last with its S / dP dropped.
// ---------------------------------------------------------------------------
constexpr int kKeys32 = 64;                       // keys per workgroup
constexpr int kMaxQTiles32 = kMaxTiles * TK / PI_MASK_TILE_Q;

// A stage: Q rows (t.k) and dO rows (t.v) of 32 query rows, their query words
// (t.w), lse2 and Dr (lanes >= 32 of their loads land as zeros).
struct BwStage {
  Stage t;
  alignas(16) float lse2[64];
  alignas(16) float dr[64];
};

// Per-lane byte offsets: row-wise fragment j (< 8; j + 8 is + 256 bytes) of a
// tile: row l % 32, logical chunk 2j + h; transposing reads as DqLanes::tr; the
// wave's loads: rows 8 wave + 2 jj + h of the tile, chunk l % 32, pre-swizzled.
struct BwLanes {
  uint32_t kr[8];
  uint32_t tr[4][2];
  uint32_t ld[4];
};

__device__ __forceinline__ BwLanes make_bw_lanes() {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  BwLanes lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) lo.kr[j] = (uint32_t)(r * D * 2 + 16 * ((2 * j + h) ^ dqsw(r)));
  const int g16 = (lane >> 4) & 1, jj = lane & 15;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int kr = 8 * e + 4 * h + (jj >> 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int x = 4 * c + 2 * g16 + ((jj & 3) >> 1);
      lo.tr[c][e] = (uint32_t)(kr * D * 2 + 16 * (x ^ dqsw(kr)) + 8 * (jj & 1));
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 8 * wave + 2 * n + h;
    lo.ld[n] = (uint32_t)row * (uint32_t)(D * 2) + 16u * (uint32_t)(r ^ dqsw(row));
  }
  return lo;
}

__device__ __forceinline__ bf16x8 bw_read_row(const __bf16* tile, const BwLanes& lo, int j) {
  return *at_bytes<bf16x8>(tile, lo.kr[j & 7] + (j >> 3) * 256u);
}
// Transposed fragment for product slot j: d chunk j / 2, query-row half j % 2.
__device__ __forceinline__ bf16x8 bw_read_tr(const __bf16* tile, const BwLanes& lo, int j) {
  const int c = j >> 1, a = j & 1;
  const char* base = reinterpret_cast<const char*>(tile) + (c >> 2) * 256 + a * (16 * D * 2);
  const bf16x4 x0 = lds_read_tr4(reinterpret_cast<const __bf16*>(base + lo.tr[c & 3][0]));
  const bf16x4 x1 = lds_read_tr4(reinterpret_cast<const __bf16*>(base + lo.tr[c & 3][1]));
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Register state of one wave: B-operand fragments of its 32 keys (K for A, V for
// B; fragment j holds d = 16 j + 8 h .. + 7 of key l % 32), the dV^T or dK^T
// accumulators (chunk c, element i: d = 32 c + 8(i/4) + 4h + i%4), the key's word,
// the carried product of the next tile (S or dP) and the bf16 weights of tile i
// (A: P(i)).
struct BwWave {
  bf16x8 f[16];
  f32x16 acc[8];
  f32x16 nx;
  bf16x8 pp[2];
  uint32_t wk;
};

// The visibility of this lane's 16 (row, key) pairs of a PARTIAL tile.
__device__ __forceinline__ uint32_t bw_visible(const BwStage& st, uint32_t wk, uint32_t forbid, bool partial) {
  if (!partial) return 0xFFFFu;
  const int h = (threadIdx.x >> 5) & 1;
  uint32_t vis = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 wq = *reinterpret_cast<const u32x4*>(&st.t.w[8 * q + 4 * h]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (pair_visible(wq[e], wk, forbid)) vis |= 1u << (4 * q + e);
  }
  return vis;
}

// One step m of wave A (tiles m-1, m, m+1 in `pst`, `cst`, `nst`): dV^T +=
// dO^T(m-1) P(m-1) (PV; P(m-1) in w.pp), S(m+1) = Q(m+1) K^T into w.nx, and the
// weights P(m) from S(m) (w.nx on entry) with tile m's statistics, spread over
// the product slots as in the forward step (scaled in slot j-1, exponentiated in
// slot j, rounded as a pair two slots later); P(m) goes to w.pp and, in fp32, to
// the exchange slot `xo`.
template <bool PV>
__device__ __forceinline__ void bw_step_a(const BwStage& pst, const BwStage& cst, const BwStage& nst,
                                          const BwLanes& lo, BwWave& w, bool partial_cur, uint32_t forbid, float c2,
                                          f32x4* __restrict__ xo) {
  constexpr int AH = 3;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  f32x4 l2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) l2[q] = *reinterpret_cast<const f32x4*>(&cst.lse2[8 * q + 4 * h]);
  const uint32_t vis = bw_visible(cst, w.wk, forbid, partial_cur);
  bf16x8 qb[AH], tb[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    qb[j] = bw_read_row(nst.t.k, lo, j);
    if constexpr (PV) tb[j] = bw_read_tr(pst.t.v, lo, j);
  }
  const f32x16 sc = w.nx;
  float x[16], e[16];
  bf16x2 pk[8];
  f32x16 sn = {};
  x[0] = fmaf(sc[0], c2, -l2[0][0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if constexpr (PV) w.acc[j >> 1] = mfma32(tb[j % AH], w.pp[j & 1], w.acc[j >> 1]);
    sn = mfma32(qb[j % AH], w.f[j], sn);
    if (j + AH < 16) {
      if constexpr (PV) tb[j % AH] = bw_read_tr(pst.t.v, lo, j + AH);
      qb[j % AH] = bw_read_row(nst.t.k, lo, j + AH);
    }
    e[j] = ((vis >> j) & 1u) ? __builtin_amdgcn_exp2f(x[j]) : 0.f;
    asm volatile("" : "+v"(e[j]));
    if (j + 1 < 16) {
      x[j + 1] = fmaf(sc[j + 1], c2, -l2[(j + 1) >> 2][(j + 1) & 3]);
      asm volatile("" : "+v"(x[j + 1]));
    }
    if (j >= 3 && (j & 1)) {            // pair (j-3, j-2)
      const int pr = (j - 3) >> 1;
      pk[pr][0] = f2bf(e[j - 3]);
      pk[pr][1] = f2bf(e[j - 2]);
      asm volatile("" : "+v"(pk[pr]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  pk[6][0] = f2bf(e[12]);
  pk[6][1] = f2bf(e[13]);
  pk[7][0] = f2bf(e[14]);
  pk[7][1] = f2bf(e[15]);
#pragma unroll
  for (int pr = 0; pr < 8; ++pr) {
    w.pp[pr >> 2][2 * (pr & 3)] = pk[pr][0];
    w.pp[pr >> 2][2 * (pr & 3) + 1] = pk[pr][1];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) xo[q * 64 + lane] = f32x4{e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]};
  w.nx = sn;
}

// One step m of wave B (tiles m-1, m in `pst`, `cst`): with PV, dS(m-1) =
// P(m-1) (dP(m-1) - Dr) from the exchange slot `xi`, w.nx (dP(m-1)) and tile
// m-1's Dr, and dK^T += Q^T(m-1) dS(m-1) eight slots behind; dP(m) = dO(m) V^T
// into w.nx.
template <bool PV>
__device__ __forceinline__ void bw_step_b(const BwStage& pst, const BwStage& cst, const BwLanes& lo, BwWave& w,
                                          const f32x4* __restrict__ xi) {
  constexpr int AH = 3;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  f32x4 pv[4], d4[4];
  if constexpr (PV) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pv[q] = xi[q * 64 + lane];
      d4[q] = *reinterpret_cast<const f32x4*>(&pst.dr[8 * q + 4 * h]);
    }
  }
  bf16x8 ob[AH], tb[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    ob[j] = bw_read_row(cst.t.v, lo, j);
    if constexpr (PV) tb[j] = bw_read_tr(pst.t.k, lo, j);
  }
  const f32x16 dc = w.nx;
  bf16x8 dsp[2];
  f32x16 dn = {};
  __builtin_amdgcn_sched_barrier(0);
  // slot j: product j of dP(m); in slots 4..7 (once the exchanged weights have
  // arrived) dS weights 4(j-4) .. +3; product j - 8 of dK^T once they are packed
  constexpr int DS0 = 4, DK0 = 8;
#pragma unroll
  for (int j = 0; j < 16 + DK0; ++j) {
    if (j < 16) {
      dn = mfma32(ob[j % AH], w.f[j], dn);
      if (j + AH < 16) ob[j % AH] = bw_read_row(cst.t.v, lo, j + AH);
    }
    if constexpr (PV) {
      if (j >= DS0 && j < DS0 + 4) {
        const int q = j - DS0;
#pragma unroll
        for (int e = 0; e < 4; ++e) dsp[q >> 1][4 * (q & 1) + e] = f2bf(pv[q][e] * (dc[4 * q + e] - d4[q][e]));
      }
      if (j >= DK0) {
        const int jk = j - DK0;
        w.acc[jk >> 1] = mfma32(tb[jk % AH], dsp[jk & 1], w.acc[jk >> 1]);
        if (jk + AH < 16) tb[jk % AH] = bw_read_tr(pst.t.k, lo, jk + AH);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  w.nx = dn;
}

// One workgroup per (sample, block of 64 keys), XCD-placed per sample; the
// query tiles (16 tokens) with a visible pair for any key of the block are
// listed up front (class merged over the block's two key tiles), each is four
// steps of 4 tokens.  Rows of padded tokens and rows past the last token load
// as zeros: their dO and dS rows are zero, so they add exactly nothing.  Keys
// past the end read key 0 and are never stored; a padded key's K and V are
// zeros and its pairs are masked (its tiles are PARTIAL).
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
dkdv32_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
              const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dr,
              __bf16* __restrict__ dk, __bf16* __restrict__ dv, int L, float scale, float c2,
              const uint32_t* __restrict__ tok, const uint8_t* __restrict__ tiles, int n_qt, int n_kt,
              uint32_t forbid, Placement place) {
  __shared__ BwStage st0, st1, st2, st3;
  __shared__ f32x4 xch[2][2][4 * 64];     // [slot][pair]: P of a tile, lane-ordered
  __shared__ uint32_t qlist[kMaxQTiles32];
  __shared__ uint32_t qvalid[kMaxTiles];
  __shared__ int qcount;
  int b, kblk;
  if (!xcd_place(place, b, kblk)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int role = __builtin_amdgcn_readfirstlane(wave & 1), pair = __builtin_amdgcn_readfirstlane(wave >> 1);
  const int key0 = kblk * kKeys32;
  const uint32_t* tk = tok + (size_t)b * L;
  token_bitmap(tk, L, n_kt, NW, qvalid);
  if (wave == 0) {
    const uint8_t* trow = tiles + (size_t)b * n_qt * n_kt;
    const int kt_lo = key0 / TK, kt_hi = min(n_kt, (key0 + kKeys32 + TK - 1) / TK);
    int cnt = 0;
    for (int base = 0; base < n_qt; base += 64) {
      const int qt = base + lane;
      int cls = 0;
      if (qt < n_qt) {
        cls = -1;
        for (int kt = kt_lo; kt < kt_hi; ++kt) {
          const int cl = trow[(size_t)qt * n_kt + kt];
          cls = (cls < 0) ? cl : (cls == cl ? cls : PI_TILE_PARTIAL);
        }
      }
      const unsigned long long bal = __ballot(cls > 0);
      if (cls > 0) qlist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (uint32_t)qt | ((uint32_t)cls << 16);
      cnt += __popcll(bal);
    }
    if (lane == 0) qcount = cnt;
  }
  BwWave w;
  const int key = key0 + 32 * pair + (lane & 31);
  const bool ok = key < L;
  {
    const int64_t r = (int64_t)b * L + (ok ? key : 0);
    w.wk = ok ? tk[key] : 0u;
    const bool live = (w.wk & 1u) != 0u;
    const __bf16* src = (role == 0 ? k : v) + r * D + 8 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(src + 16 * j);
#pragma unroll
      for (int e = 0; e < 8; ++e) w.f[j][e] = live ? a[e] : f2bf(0.f);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) w.acc[c] = f32x16{};
  }
  __syncthreads();
  const int n = 4 * qcount;
  const BwLanes lo = make_bw_lanes();
  const float* lse2_b = lse2 + (size_t)b * L * G;
  const float* dr_b = dr + (size_t)b * L * G;
  const __bf16* q_b = q + (size_t)b * L * G * D;
  const __bf16* o_b = dout + (size_t)b * L * G * D;
  auto partial = [&](int i) { return (int)((qlist[i >> 2] >> 16) & 0xFFu) == PI_TILE_PARTIAL; };
  // this wave's loads of step i: the 8 rows of token t0 + wave of Q and dO, and the
  // statistics of the 32 rows (wave 0 the query words, 1 lse2, 2 Dr)
  auto issue = [&](int i, BwStage& sg) {
    const int t0 = (int)(qlist[i >> 2] & 0xFFFFu) * PI_MASK_TILE_Q + (i & 3) * 4;
    const int tw = t0 + wave;
    const bool in = (qvalid[tw >> 5] >> (tw & 31)) & 1u;
    const int64_t at = (int64_t)__builtin_amdgcn_readfirstlane(t0) * G * D * 2;
    const i32x4 rq = make_rsrc(reinterpret_cast<const char*>(q_b) + at);
    const i32x4 ro = make_rsrc(reinterpret_cast<const char*>(o_b) + at);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t off = in ? lo.ld[jj] : kOOB;
      pi_buffer_load_lds(rq, lds_u32(&sg.t.k[(8 * wave + 2 * jj) * D]), 16, (int)off, 0, 0, 0);
      pi_buffer_load_lds(ro, lds_u32(&sg.t.v[(8 * wave + 2 * jj) * D]), 16, (int)off, 0, 0, 0);
    }
    const bool row_in = lane < 32 && t0 + (lane >> 3) < L;
    if (wave == 0) {
      const uint32_t off = row_in ? (uint32_t)(t0 + (lane >> 3)) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(tk), lds_u32(&sg.t.w[0]), 4, (int)off, 0, 0, 0);
    } else if (wave == 1) {
      const uint32_t off = row_in ? (uint32_t)(t0 * G + lane) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(lse2_b), lds_u32(&sg.lse2[0]), 4, (int)off, 0, 0, 0);
    } else if (wave == 2) {
      const uint32_t off = row_in ? (uint32_t)(t0 * G + lane) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(dr_b), lds_u32(&sg.dr[0]), 4, (int)off, 0, 0, 0);
    }
  };
  // The two roles run separate copies of the loop (the same barriers in the
  // same order), so each keeps only its own values in registers.
  auto run = [&](auto role_tag) {
    constexpr int R = decltype(role_tag)::value;
    if (n <= 0) return;
    issue(0, st0);
    if (n > 1) issue(1, st1);
    wait_vmem();
    __syncthreads();      // tiles 0 and 1 have landed
    // prologue: A forms S(0)
    if constexpr (R == 0) {
      f32x16 x0 = {};
#pragma unroll
      for (int j = 0; j < 16; ++j) x0 = mfma32(bw_read_row(st0.t.k, lo, j), w.f[j], x0);
      w.nx = x0;
    }
    // Step m: barrier (tile m+1 has landed; every wave is done with step m-1, so
    // the stage of tile m-2 and the exchange slot A writes in this step are free),
    // then this wave's loads of tile m+2 and its half of the pair's work.
    auto step = [&](auto pv, int m, BwStage& prv, BwStage& cur, BwStage& nxt, BwStage& ld) {
      constexpr bool PV = decltype(pv)::value;
      wait_vmem();
      __syncthreads();
      if (m + 2 < n) issue(m + 2, ld);
      if constexpr (R == 0)
        bw_step_a<PV>(prv, cur, nxt, lo, w, m < n && partial(m), forbid, c2, &xch[m & 1][pair][0]);
      else
        bw_step_b<PV>(prv, cur, lo, w, &xch[(m + 1) & 1][pair][0]);
    };
    using NoPV = std::integral_constant<bool, false>;
    using WithPV = std::integral_constant<bool, true>;
    step(NoPV{}, 0, st3, st0, st1, st2);
    for (int m = 1; m <= n; m += 4) {
      step(WithPV{}, m, st0, st1, st2, st3);
      if (m + 1 <= n) step(WithPV{}, m + 1, st1, st2, st3, st0);
      if (m + 2 <= n) step(WithPV{}, m + 2, st2, st3, st0, st1);
      if (m + 3 <= n) step(WithPV{}, m + 3, st3, st0, st1, st2);
    }
  };
  if (role == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  // outputs through a free stage: dV (A waves) and dK (B waves), 32 key rows each
  wait_vmem();
  __syncthreads();
  __bf16* buf = wave == 0 ? st0.t.k : wave == 1 ? st0.t.v : wave == 2 ? st1.t.k : st1.t.v;
  __bf16* out = role == 0 ? dv : dk;
  store_rows_staged(w.acc, role == 0 ? 1.f : scale, buf, [&](int r, int x) -> __bf16* {
    const int kr = key0 + 32 * pair + r;
    return kr < L ? out + ((int64_t)b * L + kr) * D + 8 * x : nullptr;
  });
}

}  // namespace

namespace pi32 {

int prefill_splits(int B, int Hkv, int L) {
  const int n_qblk = (L + TOK - 1) / TOK;
  return splits_for(B * Hkv, n_qblk, (L + TK - 1) / TK, 2);
}

size_t prefill_split_bytes(int B, int Hkv, int L, int splits) {
  return split_bytes(B * Hkv, (L + TOK - 1) / TOK, splits);
}

pi_status prefill(const void* q, const void* k, const void* v, void* o, int B, int L, int Hq, int Hkv, float scale,
                  const pi_mask* m, float rope_base, float* lse, void* split_ws, size_t split_avail,
                  hipStream_t s) {
  const int n_qblk = (L + TOK - 1) / TOK;
  int splits = prefill_splits(B, Hkv, L);
  if (split_ws == nullptr || split_avail < prefill_split_bytes(B, Hkv, L, splits)) splits = 1;
  const Placement place = make_placement(B * Hkv * splits, n_qblk);
  const int64_t grid = placement_grid(place);
  PI_REQUIRE(grid < (1ll << 31), PI_ERR_UNSUPPORTED, "prefill: grid too large");
  const size_t chunks = (size_t)splits * B * Hkv * n_qblk * NW;
  float* opart = splits > 1 ? static_cast<float*>(split_ws) : nullptr;
  float* mlpart = splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(split_ws) +
                                                        pi::align_up(chunks * 32 * 256 * sizeof(float), 256))
                             : nullptr;
  prefill32_kernel<<<(unsigned)grid, THREADS, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), B, L, Hq, Hkv, scale * 1.4426950408889634f, m->tok, m->tiles, m->n_qt, m->n_kt,
      m->forbid_bits, place, splits, opart, mlpart, rope_base > 0.f ? m->pos : nullptr,
      rope_base > 0.f ? log2((double)rope_base) : 0.0, splits > 1 ? nullptr : lse);
  pi_status st = pi::check_launch("prefill32_kernel");
  if (st != PI_OK || splits == 1) return st;
  const int64_t n_chunks = (int64_t)B * Hkv * n_qblk * NW;
  combine32_kernel<<<(unsigned)(n_chunks * 2), 256, 0, s>>>(opart, mlpart, static_cast<__bf16*>(o), 0, n_chunks,
                                                              n_qblk, L, Hq, splits, lse);
  return pi::check_launch("combine32_kernel");
}

int decode_splits(int B, int S, int len) {
  const int n_qblk = (S + TOK - 1) / TOK;
  return splits_for(B, n_qblk, (len + TK - 1) / TK + (S + TK - 1) / TK, 2);
}

size_t decode_split_bytes(int B, int S, int splits) { return split_bytes(B, (S + TOK - 1) / TOK, splits); }

pi_status decode(const pi_kv_cache* cache, const __bf16* ckl, const __bf16* cvl, const void* q_s, const void* k_s,
                 const void* v_s, const uint8_t* suffix_ar, int B, int S, float scale, float rope_base, void* o_s,
                 bool tiled, void* split_ws, size_t split_avail, hipStream_t s) {
  const int n_qblk = (S + TOK - 1) / TOK;
  int splits = decode_splits(B, S, cache->len);
  if (split_ws == nullptr || split_avail < decode_split_bytes(B, S, splits)) splits = 1;
  const size_t chunks = (size_t)splits * B * n_qblk * NW;
  float* opart = splits > 1 ? static_cast<float*>(split_ws) : nullptr;
  float* mlpart = splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(split_ws) +
                                                        pi::align_up(chunks * 32 * 256 * sizeof(float), 256))
                             : nullptr;
  const Placement place = make_placement(B * splits, n_qblk);
  const bool rope = rope_base > 0.f;
  decode32_kernel<<<(unsigned)placement_grid(place), THREADS, 0, s>>>(
      ckl, cvl, cache->prefix_mask, cache->capacity, cache->len, static_cast<const __bf16*>(q_s),
      static_cast<const __bf16*>(k_s), static_cast<const __bf16*>(v_s), suffix_ar, B, S,
      scale * 1.4426950408889634f, static_cast<__bf16*>(o_s), tiled ? 1 : 0, place, splits, opart, mlpart,
      rope ? 1 : 0, rope ? log2((double)rope_base) : 0.0);
  pi_status st = pi::check_launch("decode32_kernel");
  if (st != PI_OK || splits == 1) return st;
  const int64_t n_chunks = (int64_t)B * n_qblk * NW;
  combine32_kernel<<<(unsigned)(n_chunks * 2), 256, 0, s>>>(opart, mlpart, static_cast<__bf16*>(o_s),
                                                              tiled ? 1 : 0, n_chunks, n_qblk, S, G, splits, nullptr);
  return pi::check_launch("combine32_kernel");
}

pi_status dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse2, const float* dr,
               void* dk, void* dv, int B, int L, float scale, const pi_mask* m, hipStream_t s) {
  const Placement place = make_placement(B, (L + kKeys32 - 1) / kKeys32);
  const int64_t grid = placement_grid(place);
  PI_REQUIRE(grid < (1ll << 31), PI_ERR_UNSUPPORTED, "dkdv: grid too large");
  dkdv32_kernel<<<(unsigned)grid, THREADS, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<const __bf16*>(dout), lse2, dr, static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), L, scale,
      scale * 1.4426950408889634f, m->tok, m->tiles, m->n_qt, m->n_kt, m->forbid_bits, place);
  return pi::check_launch("dkdv32_kernel");
}

pi_status dq(const void* q, const void* k, const void* v, const void* dout, const float* lse2, const float* dr, void* dq,
             int B, int L, float scale, const pi_mask* m, hipStream_t s) {
  const Placement place = make_placement(B, (L + TOK - 1) / TOK);
  const int64_t grid = placement_grid(place);
  PI_REQUIRE(grid < (1ll << 31), PI_ERR_UNSUPPORTED, "dq: grid too large");
  dq32_kernel<<<(unsigned)grid, THREADS, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<const __bf16*>(dout), lse2, dr, static_cast<__bf16*>(dq), L, scale, scale * 1.4426950408889634f,
      m->tok, m->tiles, m->n_qt, m->n_kt, m->forbid_bits, place);
  return pi::check_launch("dq32_kernel");
}

}  // namespace pi32
