// Masked grouped-query attention over one shared KV pool, gfx950.
//
// What is computed ("π0.5 vs MM-DiT joint attention", first section; "VLA 代码精读"
// §1.5, §1.6): per (sample, query token, head) one softmax over every visible key
// of the concatenated prefix+suffix pool, query head h reading KV head
// floor(h*Hkv/Hq).  Masked keys are excluded by selection (score -inf before the
// maximum, weight exactly 0).
//
// Kernel organisation (one engine for prefill and cached decode):
//   * A workgroup owns NW waves x NR row tiles x 16 query rows.  With one KV head
//     and 8 query heads a row is a (token, head) pair: a 16-row tile holds two
//     tokens x 8 heads, so every K/V element loaded serves 8 heads.
//   * K/V tiles of 32 keys go from global memory straight into LDS (buffer loads
//     with the LDS destination: no registers, no VALU) over four stages, one
//     barrier per tile: one block per step runs tile i-1's PV, tile i+1's scores
//     and tile i's softmax while tile i+2 streams in.  A padded or masked-out key is given an
//     out-of-range offset, which the buffer unit turns into zeros: whatever a
//     padded slot holds never reaches a product.
//   * LDS rows are unpadded; 16-byte chunks are XOR-swizzled by row so that both
//     matrix-core operand reads are bank-conflict free (the swizzle is applied to
//     the global source chunk each lane fetches).
//   * Products are computed transposed: S^T = K Q^T (A = K from LDS, B = Q held in
//     registers), then O^T += V^T P^T with P^T taken straight from the S^T
//     accumulators.  The V^T operand is read with the transposing LDS load
//     (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
//     (i % 4) of the 4 elements addressed by lanes 4k + i/4, k = 0..3, so pointing
//     lane j at row 4g + j/4, columns 4*(j%4).. of the V tile hands lane i the
//     values of 4 keys at one d -- the keys its S^T accumulators cover.
//   * Softmax in base 2 against a per-row reference maximum fixed at the row's
//     first visible tile (see kMaxGrowth); the accumulators are never rescaled in
//     the loop.
//   * Key tiles classified EMPTY by the mask builder are skipped; FULL tiles skip
//     the per-pair rule.  Workgroups of one (sample, KV head) are placed on one
//     XCD so their K/V reads share that XCD's L2.
#include "attention32.h"
#include "common.h"
#include "engine.h"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace {

using namespace pi_engine;

template <int D, int G, int NR, int NW>
struct Cfg {
  static constexpr int ROWS_W = NR * 16;
  static constexpr int ROWS = NW * ROWS_W;
  static constexpr int TOK = ROWS / G;        // query tokens per workgroup
  static constexpr int NWT = NW + 1;             // NW compute waves and one load wave
  static constexpr int THREADS = NWT * PI_WAVE;
  static_assert(ROWS % G == 0, "rows must cover whole tokens");
  static_assert(D == 256 || D == 64, "head dim 256 or 64");
};

// Per-wave state of the online softmax.  m is each row's reference maximum
// (scores already multiplied by scale*log2(e)), fixed at the row's first tile
// with a visible key and the same in the four lanes that share a row; mobs is
// this lane's running maximum over its own scores (reduced across the row only
// at the end); l is the row sums of the weights, accumulated on the matrix cores
// as 1^T P^T (so every lane of a row holds the row's sum in l[r][0]); all_set is
// true once every row of the wave has its reference.
template <int D, int NR>
struct WaveState {
  bf16x8 qf[NR][D / 32];
  f32x4 o[NR][D / 16];
  f32x4 l[NR];
  float m[NR];
  float mobs[NR];
  uint32_t wq[NR];
  bool all_set;
};

// Weights are exp2(score - m) against a reference maximum m fixed at a row's
// first tile with a visible key, so the accumulators never need rescaling inside
// the loop (a rescale there would force the compiler to shuttle all of O between
// accumulation and vector registers every tile).  Later scores may exceed m: the
// weights then grow above 1, exactly representable up to 2^127 in bf16 and fp32,
// and the final division by l makes the result independent of m.  If a row's
// true maximum ends more than kMaxGrowth above m, the workgroup reruns its tiles
// once with m set to that true maximum (never the case for unit-variance inputs).
constexpr float kMaxGrowth = 64.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offsets, within a stage, of this lane's LDS operand reads; computed once.
//   K (S^T = K Q^T, A operand): lane (c, g) reads key row kt*16 + c, logical chunk
//     4 ds + g; the swizzle term f_K(row) is the same for kt = 0 and 1, so kt = 1
//     is a fixed +16 rows.
//   V (transposing read): rows 4g + c/4 (+16 for the second read, same swizzle
//     term), logical chunk 2 dt + (c & 3) / 2, half c & 1.
template <int D>
struct LaneOffsets {
  uint32_t k[D / 32];
  uint32_t v[D / 16];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets() {
  using T = Tile<D>;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  LaneOffsets<D> lo;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) lo.k[ds] = 2u * (uint32_t)(c * D + 8 * ((4 * ds + g) ^ T::fk(c)));
  const int vr = 4 * g + (c >> 2);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    lo.v[dt] = 2u * (uint32_t)(vr * D + 4 * (c & 1) + 8 * ((2 * dt + ((c & 3) >> 1)) ^ T::fv(vr)));
  return lo;
}

template <typename T>
__device__ __forceinline__ const T* at_bytes(const void* base, uint32_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

// S^T = K Q^T for one 32-key tile (the scores of this wave's rows).
template <int D, int NR>
__device__ __forceinline__ void qk_tile(const Stage<D>& sm, const LaneOffsets<D>& lo, const WaveState<D, NR>& st,
                                        f32x4 (&s)[NR][2]) {
  constexpr uint32_t HALF = 16u * D * 2u;   // bytes of 16 rows
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[r][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 a = *at_bytes<bf16x8>(sm.k, lo.k[ds] + kt * HALF);
#pragma unroll
      for (int r = 0; r < NR; ++r) s[r][kt] = mfma16x16x32(a, st.qf[r][ds], s[r][kt]);
    }
  }
}

// Softmax of one tile, branchy part (on the scores S^T of tile i, before the
// step's block): the per-pair mask of a PARTIAL tile, and until every row of the
// wave has a reference maximum, the row maxima (one cross-lane reduction) for
// rows that lack one.
template <int D, int NR>
__device__ __forceinline__ void softmax_pre(const Stage<D>& sm, WaveState<D, NR>& st, f32x4 (&s)[NR][2], int cls,
                                            uint32_t forbid, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const float NEG_INF = -INFINITY;
  if (cls == PI_TILE_PARTIAL) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wk = sm.w[kt * 16 + 4 * g + i];
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (!pair_visible(st.wq[r], wk, forbid)) s[r][kt][i] = NEG_INF;
      }
  }
  if (!st.all_set) {
    bool have_all = true;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float mx = NEG_INF;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[r][kt][i]);
      const float mt = group4_max(mx * scale_log2);
      st.m[r] = (st.m[r] == NEG_INF) ? mt : st.m[r];
      have_all &= st.m[r] != NEG_INF;
    }
    st.all_set = __ballot(!have_all) == 0ull;
  }
}

// One pipeline step's block.  Its three parts do not depend on one another:
//   PV (if PV):  O^T += V^T P^T and l += 1^T P^T for tile i-1 (weights pf_prev,
//                V from `vst`);
//   QK:          S^T = K Q^T for tile i+1 (K from `kst`) into s_nxt;
//   softmax:     the bf16 weights of tile i against the rows' reference maxima
//                (s_cur -> pf_new) and the lane maxima for the growth check.
// The products run in D/16 slots, each holding fragment j of both; the LDS reads
// run AH fragments ahead of their products, and scheduling barriers between
// slots keep that order.  The softmax follows the products: with two waves per
// SIMD it overlaps the other wave's products.
template <int D, int NR, bool PV>
__device__ __forceinline__ void step_block(const Stage<D>& vst, const Stage<D>& cst, const Stage<D>& kst,
                                           const LaneOffsets<D>& lo, WaveState<D, NR>& st,
                                           const bf16x8 (&pf_prev)[NR], f32x4 (&s_cur)[NR][2],
                                           bf16x8 (&pf_new)[NR], f32x4 (&s_nxt)[NR][2], int cls, uint32_t forbid,
                                           float scale_log2) {
  constexpr uint32_t HALF = 16u * D * 2u;   // bytes of 16 rows
  constexpr int NS = D / 16;                // slots = V fragments = K fragments
  constexpr int AH = NS >= 8 ? 3 : 2;       // read-ahead, in fragments
  const float NEG_INF = -INFINITY;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s_nxt[r][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto read_v = [&](int j) -> bf16x8 {
    const bf16x4 lo4 = lds_read_tr4(at_bytes<__bf16>(vst.v, lo.v[j]));
    const bf16x4 hi4 = lds_read_tr4(at_bytes<__bf16>(vst.v, lo.v[j] + HALF));
    return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto read_k = [&](int j) -> bf16x8 { return *at_bytes<bf16x8>(kst.k, lo.k[j >> 1] + (j & 1) * HALF); };
  bf16x8 vbuf[AH], kbuf[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if constexpr (PV) vbuf[j] = read_v(j);
    kbuf[j] = read_k(j);
  }
  if constexpr (PV) {
    bf16x8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = f2bf(1.0f);
#pragma unroll
    for (int r = 0; r < NR; ++r) st.l[r] = mfma16x16x32(ones, pf_prev[r], st.l[r]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int ds = j >> 1, kt = j & 1;
    if constexpr (PV) {
#pragma unroll
      for (int r = 0; r < NR; ++r) st.o[r][j] = mfma16x16x32(vbuf[j % AH], pf_prev[r], st.o[r][j]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) s_nxt[r][kt] = mfma16x16x32(kbuf[j % AH], st.qf[r][ds], s_nxt[r][kt]);
    if (j + AH < NS) {
      if constexpr (PV) vbuf[j % AH] = read_v(j + AH);
      kbuf[j % AH] = read_k(j + AH);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // tile i's mask and first-tile bookkeeping (cst: its stage), after the products
  // so a wave starts on the matrix cores right after the barrier
  softmax_pre<D, NR>(cst, st, s_cur, cls, forbid, scale_log2);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    // a row that has seen no visible key keeps m = -inf: use 0 so masked weights are exp2(-inf) = 0
    const float m_use = (st.m[r] == NEG_INF) ? 0.f : st.m[r];
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx = fmaxf(mx, s_cur[r][kt][i]);
        pf_new[r][4 * kt + i] = f2bf(fast_exp2(fmaf(s_cur[r][kt][i], scale_log2, -m_use)));
      }
    st.mobs[r] = fmaxf(st.mobs[r], mx * scale_log2);
  }
}

// O^T += V^T P^T and l += 1^T P^T for one tile (the pipeline's last PV).
template <int D, int NR>
__device__ __forceinline__ void pv_last(const Stage<D>& vst, const LaneOffsets<D>& lo, WaveState<D, NR>& st,
                                        const bf16x8 (&pf)[NR]) {
  constexpr uint32_t HALF = 16u * D * 2u;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = f2bf(1.0f);
#pragma unroll
  for (int r = 0; r < NR; ++r) st.l[r] = mfma16x16x32(ones, pf[r], st.l[r]);
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const bf16x4 lo4 = lds_read_tr4(at_bytes<__bf16>(vst.v, lo.v[j]));
    const bf16x4 hi4 = lds_read_tr4(at_bytes<__bf16>(vst.v, lo.v[j] + HALF));
    const bf16x8 va = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int r = 0; r < NR; ++r) st.o[r][j] = mfma16x16x32(va, pf[r], st.o[r][j]);
  }
}

constexpr int kStages = 4;

// A key tile as the loop sees it: d = tile index | class << 16 (| 1 << 24 for a
// decode suffix tile), m = its key-validity bitmap, w = this thread's key word
// for the tile (decode only).  Read from the workgroup's LDS tile list a step
// before it is needed, so no LDS round trip sits between a step's barrier and
// its loads.
struct TileDesc {
  uint32_t d, m, w;
};

__device__ __forceinline__ int tile_cls(const TileDesc& t) { return (int)((t.d >> 16) & 0xFFu); }

// Tile loop shared by both kernels, software-pipelined over four LDS stages
// (tile j lives in stage (j - i_lo) % 4; the loop is unrolled by four so every
// LDS address is a per-lane offset plus a constant).  One wave of the workgroup
// (`loader`) issues every global->LDS load; the others only compute.  Step i:
//   loader:   waits for its loads of tile i+1, passes the barrier, issues tile i+2
//             into the stage of tile i-2;
//   compute:  passes the barrier, then one block with tile i-1's PV and tile
//             i+1's scores (its K is already in LDS) on the matrix cores, then
//             tile i's mask, first-tile bookkeeping and weights.
// A tile's V is read one step after its weights are made, hence the fourth stage.
// Loads queued at the texture unit then stall only the loader, never a wave on
// the matrix cores.
//   desc(j): tile j's descriptor (LDS reads only)
//   issue(t, stage): all loads of tile t into `stage` (the loader's job)
//   prep(): once the first loads are out, work on the Q rows (the rotary
//     embedding); it must be idempotent, the loop may run twice
template <int D, int NR, typename Desc, typename Issue, typename Prep>
__device__ __forceinline__ void run_tiles(Stage<D> (&stage)[kStages], const LaneOffsets<D>& lo,
                                          WaveState<D, NR>& st, int i_lo, int i_hi, bool loader, Desc desc,
                                          Issue issue, Prep prep, uint32_t forbid, float scale_log2) {
  if (i_lo >= i_hi) return;
  if (loader) {
    issue(desc(i_lo), stage[0]);
    if (i_lo + 1 < i_hi) issue(desc(i_lo + 1), stage[1]);
    wait_vmem();
    __syncthreads();
    for (int i = i_lo; i < i_hi; ++i) {
      const bool more = i + 2 < i_hi;
      const TileDesc t = desc(more ? i + 2 : i);
      wait_vmem();          // tile i+1 has landed
      __syncthreads();      // ... and every wave is done with tiles i-2 and below
      if (more) issue(t, stage[(i + 2 - i_lo) & 3]);
    }
    return;
  }
  TileDesc t_cur = desc(i_lo), t_nxt = t_cur;
  if (i_lo + 1 < i_hi) t_nxt = desc(i_lo + 1);
  prep();               // row work that needs the Q registers, while the first tiles load
  wait_vmem();          // the Q loads
  __syncthreads();
  f32x4 s_cur[NR][2];
  qk_tile<D, NR>(stage[0], lo, st, s_cur);
  bf16x8 pf[NR];
  // step i; the last step also computes scores against whatever stage `nxt`
  // holds and discards them, which keeps the block free of branches
  auto step = [&](auto pv, int i, Stage<D>& prev, Stage<D>& cur, Stage<D>& nxt) {
    __syncthreads();      // tile i+1 has landed; every wave is done with tile i-2
    bf16x8 pf_new[NR];
    f32x4 s_nxt[NR][2];
    step_block<D, NR, decltype(pv)::value>(prev, cur, nxt, lo, st, pf, s_cur, pf_new, s_nxt, tile_cls(t_cur), forbid,
                                           scale_log2);
    t_cur = t_nxt;
    if (i + 2 < i_hi) t_nxt = desc(i + 2);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      pf[r] = pf_new[r];
      s_cur[r][0] = s_nxt[r][0];
      s_cur[r][1] = s_nxt[r][1];
    }
  };
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;
  step(NoPV{}, i_lo, stage[3], stage[0], stage[1]);
  for (int i = i_lo + 1; i < i_hi; i += 4) {
    step(WithPV{}, i, stage[0], stage[1], stage[2]);
    if (i + 1 < i_hi) step(WithPV{}, i + 1, stage[1], stage[2], stage[3]);
    if (i + 2 < i_hi) step(WithPV{}, i + 2, stage[2], stage[3], stage[0]);
    if (i + 3 < i_hi) step(WithPV{}, i + 3, stage[3], stage[0], stage[1]);
  }
  // the last tile's PV (its stage is not overwritten: no load is issued past i_hi)
  pv_last<D, NR>(stage[(i_hi - 1 - i_lo) & 3], lo, st, pf);
}

// True if a row's maximum grew past its reference by more than kMaxGrowth (the
// lane maxima are reduced across each row here, once).
template <int D, int NR>
__device__ __forceinline__ bool needs_rerun(WaveState<D, NR>& st) {
  bool bad = false;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.mobs[r] = group4_max(st.mobs[r]);
    bad |= st.mobs[r] > st.m[r] + kMaxGrowth;
  }
  return bad;
}

template <int D, int NR>
__device__ __forceinline__ void reset_for_rerun(WaveState<D, NR>& st) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.m[r] = st.mobs[r];
    st.l[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.o[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.all_set = true;
}

template <int D, int NR>
__device__ __forceinline__ void init_state(WaveState<D, NR>& st) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.m[r] = -INFINITY;
    st.mobs[r] = -INFINITY;
    st.l[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.o[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.all_set = false;
}

// Normalise and store O rows.  dst(r, dt) gives where the lane's four values
// d = 16 dt + 4 g .. + 3 of row tile r go, or nullptr for a row with no output.
template <int D, int NR, typename Dst>
__device__ __forceinline__ void store_rows(WaveState<D, NR>& st, Dst dst) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float l = st.l[r][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      __bf16* p = dst(r, dt);
      if (p == nullptr) continue;
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f2bf(st.o[r][dt][i] * inv);
      *reinterpret_cast<bf16x4*>(p) = v;
    }
  }
}

// Row-major output rows (row_base[r] = output row or nullptr).
template <int D>
struct RowMajorDst {
  __bf16* const* row_base;
  __device__ __forceinline__ __bf16* operator()(int r, int dt) const {
    return row_base[r] ? row_base[r] + dt * 16 + 4 * ((threadIdx.x & 63) >> 4) : nullptr;
  }
};

// Key-split epilogue: the unnormalised fp32 partial O of each 16-row tile,
// stored in the accumulator's own lane order so every store writes 1 KB
// contiguous, plus (reference max, weight sum) per row.  Chunk (16 rows) index:
// ((group * n_qblk + qblk) * NW + wave) * NR + r; split s of n_chunks at
// s * n_chunks + chunk.
template <int D, int NR, int NW>
__device__ __forceinline__ void store_partials(const WaveState<D, NR>& st, float* __restrict__ opart,
                                               float* __restrict__ mlpart, int64_t n_chunks, int64_t group,
                                               int n_qblk, int qblk, int split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int64_t chunk = ((group * n_qblk + qblk) * NW + wave) * NR + r;
    const int64_t at = split * n_chunks + chunk;
    f32x4* dst = reinterpret_cast<f32x4*>(opart) + at * (D / 16) * 64 + lane;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) __builtin_nontemporal_store(st.o[r][dt], &dst[dt * 64]);   // read once, by the merge
    if (g == 0) {
      mlpart[at * 32 + 2 * c] = st.m[r];
      mlpart[at * 32 + 2 * c + 1] = st.l[r][0];
    }
  }
}

// Row setup: Q fragments into registers and the output row; with `words`, also
// the row's query word (else set later by set_row_words).  Issued first thing so
// the Q loads are in flight while the workgroup builds its tile list.
// q_tiled (decode only, G == Hq): this sample's queries as rows t*G + head of a
// matrix in the operand tile layout, padded to whole 16-row blocks, so each
// fragment is one contiguous 1 KB load.
template <int D, int G, int NR, int ROWS_W>
__device__ __forceinline__ void load_rows(WaveState<D, NR>& st, __bf16** row_base, const __bf16* __restrict__ q,
                                          __bf16* __restrict__ o, int64_t tok_base, int ntok, int Hq, int head0,
                                          int tok0, const uint32_t* words,
                                          const __bf16* __restrict__ q_tiled = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = wave * ROWS_W + r * 16 + c;
    const int t = tok0 + row / G;
    const int h = head0 + row % G;
    const bool ok = t < ntok;
    if (words != nullptr) st.wq[r] = ok ? words[t] : 0u;
    // Rows past the last token (ok false) load token 0's values instead of
    // zeros: they are never stored, and leaving the loaded registers untouched
    // keeps the loads in flight until the first product needs them.
    if (q_tiled != nullptr) {
      int r0 = tok0 * G + wave * ROWS_W + r * 16;     // first row of the block, wave-uniform
      if (r0 >= ntok * G) r0 = 0;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(q_tiled) + (int64_t)(r0 / 16) * (D / 32) * 64 + lane;
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) st.qf[r][ds] = src[ds * 64];
    } else {
      const __bf16* qrow = q + ((tok_base + (ok ? t : 0)) * Hq + h) * D;
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) st.qf[r][ds] = *reinterpret_cast<const bf16x8*>(qrow + ds * 32 + 8 * g);
    }
    row_base[r] = ok ? o + ((tok_base + t) * Hq + h) * D : nullptr;
  }
}

template <int D, int G, int NR, int ROWS_W>
__device__ __forceinline__ void set_row_words(WaveState<D, NR>& st, int ntok, int tok0, const uint32_t* words) {
  const int c = threadIdx.x & 15, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int t = tok0 + (wave * ROWS_W + r * 16 + c) / G;
    st.wq[r] = t < ntok ? words[t] : 0u;
  }
}

// Rotary embedding of this lane's Q rows in registers (pairs (i, i + D/2): the
// lane's fragments ds and ds + D/64 hold them at the same offsets), row r at
// position pos[r]; inv_freq: the D/2 pair frequencies in LDS.
template <int D, int NR>
__device__ __forceinline__ void rotate_q(WaveState<D, NR>& st, const int (&pos)[NR], const double* inv_freq) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int ds = 0; ds < D / 64; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, sn;
        rope_cos_sin(pos[r], inv_freq[ds * 32 + 8 * g + e], c, sn);
        const float a = bf2f(st.qf[r][ds][e]), b = bf2f(st.qf[r][ds + D / 64][e]);
        st.qf[r][ds][e] = f2bf(a * c - b * sn);
        st.qf[r][ds + D / 64][e] = f2bf(b * c + a * sn);
      }
}

// ---------------------------------------------------------------------------
// Prefill: one group per (sample, KV head), n_qblk query blocks each, XCD-placed.
// Up front the workgroup computes every key tile's validity bitmap and compacts
// its non-EMPTY tiles into an LDS list; the loop then streams tile i+1 into the
// other LDS stage while tile i is computed.
// ---------------------------------------------------------------------------
template <int D, int G, int NR, int NW>
__global__ void __launch_bounds__((NW + 1) * 64)
prefill_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
               __bf16* __restrict__ o, int B, int L, int Hq, int Hkv, float scale_log2,
               const uint32_t* __restrict__ tok, const uint8_t* __restrict__ tiles, int n_qt, int n_kt,
               uint32_t forbid, Placement place, int n_split, float* __restrict__ opart,
               float* __restrict__ mlpart, const int32_t* __restrict__ rope_pos, double rope_log2_base,
               float* __restrict__ lse) {
  using C = Cfg<D, G, NR, NW>;
  __shared__ Stage<D> stage[kStages];
  __shared__ uint32_t kmask[kMaxTiles];
  __shared__ uint32_t tlist[kMaxTiles];
  __shared__ double rope_if[D / 2];
  __shared__ int tcount;
  int grp, qblk;
  if (!xcd_place(place, grp, qblk)) return;
  if (rope_pos != nullptr)
    for (int i = threadIdx.x; i < D / 2; i += C::NWT * 64) rope_if[i] = rope_inv_freq(i, D, rope_log2_base);
  const int group = grp / n_split, split = grp % n_split;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool loader = wave == NW;   // the last wave issues the K/V loads and computes nothing
  const int tok0 = qblk * C::TOK;
  const uint32_t* tk = tok + (size_t)b * L;

  // the Q loads go out first, with the setup's own reads, so one memory latency
  // covers them all (the barrier below waits for every load in flight)
  WaveState<D, NR> st;
  init_state(st);
  __bf16* row_base[NR];
  if (!loader) load_rows<D, G, NR, C::ROWS_W>(st, row_base, q, o, (int64_t)b * L, L, Hq, kvh * G, tok0, tk);
  query_block_tiles(tk, L, tiles + (size_t)b * n_qt * n_kt, n_qt, n_kt, tok0, C::TOK, C::NWT, kmask, tlist,
                    &tcount);
  __syncthreads();
  const int count = tcount;

  const __bf16* k0 = k + ((size_t)b * L * Hkv + kvh) * D;
  const __bf16* v0 = v + ((size_t)b * L * Hkv + kvh) * D;
  const i32x4 rw = make_rsrc(tk);
  const int tsb = Hkv * D * 2;
  const LaneOffsets<D> lo = lane_offsets<D>();
  auto desc = [&](int i) {
    const uint32_t d = tlist[i];
    return TileDesc{d, kmask[d & 0xFFFFu], 0u};
  };
  auto issue = [&](const TileDesc& t, Stage<D>& sg) {
    const int key0 = (int)(t.d & 0xFFFFu) * TK;
    issue_kv<D>(sg, kv_lanes<D>(tsb), k0, v0, key0, tsb, t.m);
    const uint32_t off = (lane < TK && key0 + lane < L) ? (uint32_t)(key0 + lane) * 4u : kOOB;
    pi_buffer_load_lds(rw, lds_u32(&sg.w[0]), 4, (int)off, 0, 0, 0);
  };
  // this workgroup's share of the tile list (all of it when the keys are not split)
  const int i_lo = (int)((int64_t)count * split / n_split);
  const int i_hi = (int)((int64_t)count * (split + 1) / n_split);
  bool rotated = rope_pos == nullptr;
  auto prep = [&]() {
    if (rotated) return;
    int p[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int t = tok0 + (wave * C::ROWS_W + r * 16 + (lane & 15)) / G;
      p[r] = rope_pos[(int64_t)b * L + min(t, L - 1)];
    }
    rotate_q<D, NR>(st, p, rope_if);
    rotated = true;
  };
  auto run = [&]() {
    run_tiles<D, NR>(stage, lo, st, i_lo, i_hi, loader, desc, issue, prep, forbid, scale_log2);
  };
  run();
  if (__syncthreads_or(needs_rerun(st))) {
    reset_for_rerun(st);
    run();
  }
  if (loader) return;
  if (n_split == 1) {
    if (lse != nullptr && lane < 16) {
      // natural-log log-sum-exp of the row's visible scaled scores (-inf with none)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int row = wave * C::ROWS_W + r * 16 + lane;
        const int t = tok0 + row / G;
        if (t < L)
          lse[((int64_t)b * L + t) * Hq + kvh * G + row % G] =
              st.l[r][0] > 0.f ? (st.m[r] + log2f(st.l[r][0])) * 0.6931471805599453f : -INFINITY;
      }
    }
    store_rows<D, NR>(st, RowMajorDst<D>{row_base});
    return;
  }
  store_partials<D, NR, NW>(st, opart, mlpart, (int64_t)B * Hkv * place.n_sub * NW * NR, group, place.n_sub, qblk,
                            split);
}

// ---------------------------------------------------------------------------
// Cached suffix decode (Hq = 8, Hkv = 1, d = 256): one group per (sample, key
// split), n_qblk query blocks each, XCD-placed.  Keys: valid prefix slots of the cache layer, then the suffix's own
// K/V.  Query/key words reuse the prefill rule with bid 0 for every prefix slot
// and 1 + cumsum(suffix_ar) for suffix tokens.  The per-tile validity of the
// prefix slots is read once up front, so fully padded tiles are never fetched
// and padded slots inside a tile are neither read nor used.  With n_split > 1
// the workgroup covers a contiguous share of the tile list and writes an
// unnormalised partial for decode_combine_kernel.
// ---------------------------------------------------------------------------
template <int D, int G, int NR, int NW>
__global__ void __launch_bounds__((NW + 1) * 64)
decode_kernel(const __bf16* __restrict__ ck, const __bf16* __restrict__ cv,
              const uint8_t* __restrict__ prefix_mask, int cap, int P,
              const __bf16* __restrict__ qs, const __bf16* __restrict__ ks, const __bf16* __restrict__ vs,
              const uint8_t* __restrict__ suffix_ar, int B, int S, float scale_log2,
              __bf16* __restrict__ os, int tiled, Placement place, int n_split, float* __restrict__ opart,
              float* __restrict__ mlpart, int rope, double rope_log2_base) {
  using C = Cfg<D, G, NR, NW>;
  constexpr int Hq = G;
  __shared__ Stage<D> stage[kStages];
  __shared__ uint32_t sbid[128];
  __shared__ uint32_t pmask[kMaxTiles];
  __shared__ uint32_t tlist[kMaxTiles];
  __shared__ uint32_t tmask[kMaxTiles];
  __shared__ double rope_if[D / 2];
  __shared__ int tcount;
  int grp, qblk;
  if (!xcd_place(place, grp, qblk)) return;
  if (rope)
    for (int i = threadIdx.x; i < D / 2; i += C::NWT * 64) rope_if[i] = rope_inv_freq(i, D, rope_log2_base);
  const int b = grp / n_split, split = grp % n_split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool loader = wave == NW;   // the last wave issues the K/V loads and computes nothing
  const int tok0 = qblk * C::TOK;
  const int n_pt = (P + TK - 1) / TK;
  const int n_st = (S + TK - 1) / TK;

  // the Q loads and all of the setup's reads (the suffix's block flags, the prefix
  // slots' validity bytes, up to eight rounds before the first ballot) go out
  // before any wait: one memory latency for the whole setup
  WaveState<D, NR> st;
  init_state(st);
  __bf16* row_base[NR];
  const __bf16* q_tiled = tiled ? qs + (int64_t)b * ((S * G + 15) / 16 * 16) * D : nullptr;
  if (!loader) load_rows<D, G, NR, C::ROWS_W>(st, row_base, qs, os, (int64_t)b * S, S, Hq, 0, tok0, nullptr, q_tiled);
  int a0 = lane < S ? (suffix_ar[lane] != 0) : 0;
  int a1 = lane + 64 < S ? (suffix_ar[lane + 64] != 0) : 0;
  // validity bitmap of the prefix slots, one 32-bit word per tile
  const uint8_t* pm = prefix_mask + (size_t)b * cap;
  for (int base0 = wave * 64; base0 < n_pt * TK; base0 += 8 * C::NWT * 64) {
    bool valid[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int slot = base0 + u * C::NWT * 64 + lane;
      valid[u] = slot < P && pm[slot] != 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = base0 + u * C::NWT * 64;
      if (base >= n_pt * TK) break;
      const unsigned long long bal = __ballot(valid[u]);
      if (lane == 0) pmask[base / TK] = (uint32_t)bal;
      if (lane == 32 && base / TK + 1 < n_pt) pmask[base / TK + 1] = (uint32_t)(bal >> 32);
    }
  }
  // suffix block ids: inclusive cumsum of the flags (S <= 128), computed by wave 0
  if (wave == 0) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int u0 = __shfl_up(a0, off), u1 = __shfl_up(a1, off);
      if (lane >= off) { a0 += u0; a1 += u1; }
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
      uint32_t m = 0u, desc = 0u;
      if (i < n_pt) {
        m = pmask[i];
        const bool full = (m == 0xFFFFFFFFu);
        desc = (uint32_t)i | ((uint32_t)(full ? PI_TILE_FULL : PI_TILE_PARTIAL) << 16);
      } else if (i < n_pt + n_st) {
        const int nv = min(TK, S - (i - n_pt) * TK);
        m = nv == TK ? 0xFFFFFFFFu : ((1u << nv) - 1u);
        desc = (uint32_t)(i - n_pt) | ((uint32_t)PI_TILE_PARTIAL << 16) | (1u << 24);
      }
      const unsigned long long bal = __ballot(m != 0u);
      if (m != 0u) {
        const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
        tlist[pos] = desc;
        tmask[pos] = m;
      }
      cnt += __popcll(bal);
    }
    if (lane == 0) tcount = cnt;
  }
  __syncthreads();
  // this workgroup's share of the tile list (all of it when the keys are not split)
  const int i_lo = (int)((int64_t)tcount * split / n_split);
  const int i_hi = (int)((int64_t)tcount * (split + 1) / n_split);

  if (!loader) set_row_words<D, G, NR, C::ROWS_W>(st, S, tok0, sbid);

  const __bf16* k0 = ck + (size_t)b * cap * D;
  const __bf16* v0 = cv + (size_t)b * cap * D;
  const __bf16* ks0 = ks + (size_t)b * S * D;
  const __bf16* vs0 = vs + (size_t)b * S * D;
  const LaneOffsets<D> lo = lane_offsets<D>();
  auto desc = [&](int i) {
    const uint32_t d = tlist[i], m = tmask[i];
    uint32_t w = 0u;
    if (lane < TK) {
      const int key0 = (int)(d & 0xFFFFu) * TK;
      const uint32_t bit = (m >> lane) & 1u;
      w = ((d >> 24) & 1u) ? (bit ? sbid[key0 + lane] : 0u) : bit;
    }
    return TileDesc{d, m, w};
  };
  auto issue = [&](const TileDesc& t, Stage<D>& sg) {
    const int key0 = (int)(t.d & 0xFFFFu) * TK;
    const bool suffix = (t.d >> 24) & 1u;
    issue_kv<D>(sg, kv_lanes<D>(D * 2), suffix ? ks0 : k0, suffix ? vs0 : v0, key0, D * 2, t.m);
    if (lane < TK) sg.w[lane] = t.w;
  };
  // suffix token t sits at position (valid prefix slots) + t
  bool rotated = !rope;
  auto prep = [&]() {
    if (rotated) return;
    int n_valid = 0;
    for (int w = lane; w < n_pt; w += 64) n_valid += __popc(pmask[w]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n_valid += __shfl_xor(n_valid, off);
    int p[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) p[r] = n_valid + tok0 + (wave * C::ROWS_W + r * 16 + (lane & 15)) / G;
    rotate_q<D, NR>(st, p, rope_if);
    rotated = true;
  };
  auto run = [&]() {
    run_tiles<D, NR>(stage, lo, st, i_lo, i_hi, loader, desc, issue, prep, 0u, scale_log2);
  };
  run();
  if (__syncthreads_or(needs_rerun(st))) {
    reset_for_rerun(st);
    run();
  }
  if (loader) return;
  if (n_split == 1) {
    if (tiled) {
      const int c = lane & 15, g = lane >> 4;
      auto dst = [&](int r, int dt) -> __bf16* {
        const int row = wave * C::ROWS_W + r * 16 + c;
        const int t = tok0 + row / G;
        if (t >= S) return nullptr;
        return os + tiled_offset((int64_t)b * S + t, (row % G) * D + dt * 16 + 4 * g, G * D);
      };
      store_rows<D, NR>(st, dst);
    } else {
      store_rows<D, NR>(st, RowMajorDst<D>{row_base});
    }
    return;
  }
  store_partials<D, NR, NW>(st, opart, mlpart, (int64_t)B * place.n_sub * NW * NR, b, place.n_sub, qblk, split);
}

// Merge the key splits of a decode or GQA 8:1 prefill: for each (sample, token, head) row,
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.  The
// split kernel stored each 16-row chunk's partial in accumulator lane order; here four
// workgroups share a chunk and each wave merges one 16-wide slice of d, issuing
// the loads of all splits at once (1 KB contiguous per load).
constexpr int kMaxSplit = 16;

template <int NR, int NW>
__global__ void __launch_bounds__(256)
decode_combine_kernel(const float* __restrict__ opart, const float* __restrict__ mlpart,
                      __bf16* __restrict__ os, int o_tiled, int B, int S, int n_qblk, int n_split,
                      float* __restrict__ lse) {
  constexpr int D = 256, G = 8, TOK = NR * NW * 16 / G;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t chunk = blockIdx.x >> 2;
  const int dt = (blockIdx.x & 3) * 4 + (threadIdx.x >> 6);
  const int64_t n_chunks = (int64_t)B * n_qblk * NW * NR;
  const int r = (int)(chunk % NR);
  const int w_dec = (int)((chunk / NR) % NW);
  const int64_t bq = chunk / (NR * NW);
  const int qblk = (int)(bq % n_qblk);
  const int64_t b = bq / n_qblk;
  const int row = w_dec * 16 * NR + r * 16 + c;
  const int t = qblk * TOK + row / G;
  const int head = row % G;
  float m[kMaxSplit], l[kMaxSplit];
  f32x4 op[kMaxSplit];
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {
    m[sp] = -INFINITY;
    l[sp] = 0.f;
    op[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (sp < n_split) {
      const int64_t at = sp * n_chunks + chunk;
      m[sp] = mlpart[at * 32 + 2 * c];
      l[sp] = mlpart[at * 32 + 2 * c + 1];
      op[sp] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(opart) + (at * (D / 16) + dt) * 64 + lane);
    }
    M = fmaxf(M, m[sp]);
  }
  if (t >= S) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) {
      const float w = (m[sp] == -INFINITY) ? 0.f : fast_exp2(m[sp] - M);
      L += w * l[sp];
      acc += w * op[sp];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (lse != nullptr && dt == 0 && g == 0)
    lse[(b * S + t) * G + head] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = f2bf(acc[i] * inv);
  __bf16* dst = o_tiled ? os + tiled_offset(b * S + t, head * D + dt * 16 + 4 * g, G * D)
                        : os + ((b * S + t) * G + head) * D + dt * 16 + 4 * g;
  *reinterpret_cast<bf16x4*>(dst) = v;
}

// ---------------------------------------------------------------------------
// Cached suffix decode of a few samples (the single-robot sampler), built for
// latency.  Each workgroup of NW waves owns query block qblk of one sample and
// at most kStages key tiles (a contiguous share of the sample's tile sequence:
// the prefix tiles 0 .. ceil(len/32)-1, then the suffix tiles), all resident in
// LDS at once.  So everything a workgroup reads goes out in the first few
// instructions, before any wait: its K/V tiles (direct to LDS, each wave a
// quarter of every tile), its Q rows, the validity bytes of its prefix slots and
// the suffix's block flags; one memory latency later the whole share is there.
// The loads take the static key range (prefix slots < len, suffix tokens < S;
// beyond it they land as zeros).  Padded prefix slots inside that range are
// found from the validity bytes once they arrive: their V rows are zeroed in LDS
// and their scores masked, so no padded K/V reaches an output, NaN included.
// With every score of the share in registers, the softmax takes each row's exact
// maximum over the share: no reference maximum, no second pass.  The partials
// (key split) use the layout decode_combine_kernel<NR, NW> merges.
// ---------------------------------------------------------------------------
template <int D, int G, int NR, int NW>
__global__ void __launch_bounds__(NW * 64)
decode_small_kernel(const __bf16* __restrict__ ck, const __bf16* __restrict__ cv,
                    const uint8_t* __restrict__ prefix_mask, int cap, int P,
                    const __bf16* __restrict__ qs, const __bf16* __restrict__ ks, const __bf16* __restrict__ vs,
                    const uint8_t* __restrict__ suffix_ar, int B, int S, float scale_log2,
                    __bf16* __restrict__ os, int tiled, Placement place, int n_split, float* __restrict__ opart,
                    float* __restrict__ mlpart, int rope, double rope_log2_base) {
  using T = Tile<D>;
  constexpr int ROWS_W = NR * 16;
  constexpr int TOK = NW * ROWS_W / G;
  constexpr int JW = T::INSTS / NW;         // load instructions per tensor tile and wave
  static_assert(T::INSTS % NW == 0, "a tile's loads split evenly over the waves");
  __shared__ Stage<D> stage[kStages];
  __shared__ uint32_t sbid[128];
  __shared__ double rope_if[D / 2];
  int grp, qblk;
  if (!xcd_place(place, grp, qblk)) return;
  const int b = grp / n_split, split = grp % n_split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int tok0 = qblk * TOK;
  const int n_pt = (P + TK - 1) / TK;
  const int nt = n_pt + (S + TK - 1) / TK;
  const int i_lo = (int)((int64_t)nt * split / n_split);
  const int n = (int)((int64_t)nt * (split + 1) / n_split) - i_lo;   // <= kStages (the launcher's rule)

  // 1. this wave's quarter of every K/V tile of the share, static key range
  const __bf16* k0 = ck + (size_t)b * cap * D;
  const __bf16* v0 = cv + (size_t)b * cap * D;
  const __bf16* ks0 = ks + (size_t)b * S * D;
  const __bf16* vs0 = vs + (size_t)b * S * D;
  uint32_t smask[kStages];
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    smask[t] = 0u;
    if (t >= n) continue;
    const int i = i_lo + t;
    const bool suf = i >= n_pt;
    const int key0 = (suf ? i - n_pt : i) * TK;
    const int left = (suf ? S : P) - key0;
    smask[t] = left >= TK ? 0xFFFFFFFFu : ((1u << left) - 1u);
    const int64_t at = (int64_t)key0 * D * 2;
    const i32x4 rk = make_rsrc(reinterpret_cast<const char*>(suf ? ks0 : k0) + at);
    const i32x4 rv = make_rsrc(reinterpret_cast<const char*>(suf ? vs0 : v0) + at);
    const int p = lane % T::CHR;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int j = wave * JW + jj;
      const int r = j * T::RPI + lane / T::CHR;
      uint32_t ok = (uint32_t)r * (D * 2) + 16u * (uint32_t)(p ^ T::fk(r));
      uint32_t ov = (uint32_t)r * (D * 2) + 16u * (uint32_t)(p ^ T::fv(r));
      if (!((smask[t] >> r) & 1u)) ok = ov = kOOB;
      pi_buffer_load_lds(rk, lds_u32(&stage[t].k[j * T::RPI * D]), 16, (int)ok, 0, 0, 0);
      pi_buffer_load_lds(rv, lds_u32(&stage[t].v[j * T::RPI * D]), 16, (int)ov, 0, 0, 0);
    }
  }
  // 2. the Q rows
  WaveState<D, NR> st;
  init_state(st);
  __bf16* row_base[NR];
  const __bf16* q_tiled = tiled ? qs + (int64_t)b * ((S * G + 15) / 16 * 16) * D : nullptr;
  load_rows<D, G, NR, ROWS_W>(st, row_base, qs, os, (int64_t)b * S, S, G, 0, tok0, nullptr, q_tiled);
  // 3. validity of the share's prefix slots (lanes < 32: one slot of each tile)
  const uint8_t* pm = prefix_mask + (size_t)b * cap;
  uint32_t pv[kStages];
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    const int i = i_lo + t;
    const int key = i * TK + lane;
    pv[t] = (t < n && i < n_pt && lane < TK && key < P) ? pm[key] : 0u;
  }
  int n_valid = 0;   // valid prefix slots (the suffix's rotary positions start there)
  if (rope) {
    for (int j = lane; j < P; j += 64) n_valid += pm[j] != 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n_valid += __shfl_xor(n_valid, off);
    for (int i = threadIdx.x; i < D / 2; i += NW * 64) rope_if[i] = rope_inv_freq(i, D, rope_log2_base);
  }
  // 4. suffix block ids: inclusive cumsum of suffix_ar (S <= 128), wave 0
  if (wave == 0) {
    int a0 = lane < S ? (suffix_ar[lane] != 0) : 0;
    int a1 = lane + 64 < S ? (suffix_ar[lane + 64] != 0) : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int u0 = __shfl_up(a0, off), u1 = __shfl_up(a1, off);
      if (lane >= off) { a0 += u0; a1 += u1; }
    }
    const int tot0 = __shfl(a0, 63);
    sbid[lane] = 1u | ((uint32_t)(1 + a0) << 3);
    sbid[lane + 64] = 1u | ((uint32_t)(1 + tot0 + a1) << 3);
  }
  wait_vmem();
  __syncthreads();      // every wave's tiles have landed; sbid is written

  // 5. per tile: the dynamic validity, the key words (written by wave 0), the
  // padded slots inside the loaded range (V rows zeroed: 0 * NaN would be NaN)
  int cls[kStages];
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    cls[t] = PI_TILE_FULL;
    if (t >= n) continue;
    const int i = i_lo + t;
    const bool suf = i >= n_pt;
    uint32_t dyn, w = 0u;
    if (!suf) {
      dyn = (uint32_t)__ballot(pv[t] != 0u);
      w = (dyn >> (lane & 31)) & 1u;
    } else {
      dyn = smask[t];
      const int u = (i - n_pt) * TK + (lane & 31);
      w = ((dyn >> (lane & 31)) & 1u) ? sbid[u] : 0u;
    }
    cls[t] = (!suf && dyn == 0xFFFFFFFFu) ? PI_TILE_FULL : PI_TILE_PARTIAL;
    if (wave == 0 && lane < TK) stage[t].w[lane] = w;
    for (uint32_t zz = smask[t] & ~dyn; zz != 0u; zz &= zz - 1u) {
      const int r = __builtin_ctz(zz);
      if (r % NW == wave) reinterpret_cast<u32x2*>(&stage[t].v[r * D])[lane] = u32x2{0u, 0u};
    }
  }
  __syncthreads();      // key words and zeroed rows are visible

  // 6. scores of the share, each row's exact maximum, weights, PV
  set_row_words<D, G, NR, ROWS_W>(st, S, tok0, sbid);
  if (rope) {
    int pos[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) pos[r] = n_valid + tok0 + (wave * ROWS_W + r * 16 + (lane & 15)) / G;
    rotate_q<D, NR>(st, pos, rope_if);
  }
  const LaneOffsets<D> lo = lane_offsets<D>();
  const float NEG_INF = -INFINITY;
  f32x4 sc[kStages][NR][2];
  float mx[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) mx[r] = NEG_INF;
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    if (t >= n) continue;
    qk_tile<D, NR>(stage[t], lo, st, sc[t]);
    if (cls[t] == PI_TILE_PARTIAL) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wk = stage[t].w[kt * 16 + 4 * g + i];
#pragma unroll
          for (int r = 0; r < NR; ++r)
            if (!pair_visible(st.wq[r], wk, 0u)) sc[t][r][kt][i] = NEG_INF;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx[r] = fmaxf(mx[r], sc[t][r][kt][i]);
  }
  float m_use[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.m[r] = group4_max(mx[r] * scale_log2);
    // a row with no visible key in the share keeps m = -inf; 0 makes its weights exp2(-inf) = 0
    m_use[r] = st.m[r] == NEG_INF ? 0.f : st.m[r];
  }
#pragma unroll
  for (int t = 0; t < kStages; ++t) {
    if (t >= n) continue;
    bf16x8 pf[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pf[r][4 * kt + i] = f2bf(fast_exp2(fmaf(sc[t][r][kt][i], scale_log2, -m_use[r])));
    pv_last<D, NR>(stage[t], lo, st, pf);
  }

  // 7. output rows, or the partials of the key split
  if (n_split == 1) {
    if (tiled) {
      const int c = lane & 15;
      auto dst = [&](int r, int dt) -> __bf16* {
        const int row = wave * ROWS_W + r * 16 + c;
        const int t = tok0 + row / G;
        if (t >= S) return nullptr;
        return os + tiled_offset((int64_t)b * S + t, (row % G) * D + dt * 16 + 4 * g, G * D);
      };
      store_rows<D, NR>(st, dst);
    } else {
      store_rows<D, NR>(st, RowMajorDst<D>{row_base});
    }
    return;
  }
  store_partials<D, NR, NW>(st, opart, mlpart, (int64_t)B * place.n_sub * NW * NR, b, place.n_sub, qblk, split);
}

// K/V rows of tokens [0, P) into cache layer slices; one thread per 16 bytes.
__global__ void cache_write_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                   u32x4* __restrict__ ck, u32x4* __restrict__ cv, int L, int cap, int P,
                                   int row_chunks, int64_t total) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int64_t ch = id % row_chunks;
  const int64_t t = (id / row_chunks) % P;
  const int64_t b = id / ((int64_t)row_chunks * P);
  const int64_t src = (b * L + t) * row_chunks + ch;
  const int64_t dst = (b * cap + t) * row_chunks + ch;
  ck[dst] = k[src];
  cv[dst] = v[src];
}

// Append n_new tokens per sample (grid.y = sample) at slots [len, len + n_new) of a
// cache layer: K (rotated at (valid slots before len) + t when log2_base != 0), V,
// and their validity bytes.  One thread per 8 rotary pairs (16 bytes of each half)
// of one (token, head) row.
__global__ void __launch_bounds__(256)
cache_append_kernel(const bf16x8* __restrict__ k_new, const bf16x8* __restrict__ v_new, bf16x8* __restrict__ ck,
                    bf16x8* __restrict__ cv, uint8_t* __restrict__ pm, int cap, int len, int n_new, int Hkv, int d,
                    double log2_base) {
  __shared__ double inv_freq[256];
  __shared__ int n_valid;
  const int b = blockIdx.y;
  const int half8 = d / 16;                      // 16-byte chunks per half row
  const bool rope = log2_base != 0.0;
  if (threadIdx.x == 0) n_valid = 0;
  if (rope)
    for (int i = threadIdx.x; i < d / 2; i += blockDim.x) inv_freq[i] = rope_inv_freq(i, d, log2_base);
  __syncthreads();
  if (rope) {
    int cnt = 0;
    for (int t = threadIdx.x; t < len; t += blockDim.x) cnt += pm[(int64_t)b * cap + t] != 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&n_valid, cnt);
    __syncthreads();
  }
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)n_new * Hkv * half8) return;
  const int j = (int)(id % half8);
  const int64_t row = id / half8;                 // t * Hkv + h
  const int t = (int)(row / Hkv);
  const int64_t src = ((int64_t)b * n_new * Hkv + row) * (d / 8);
  const int64_t dst = (((int64_t)b * cap + len) * Hkv + row) * (d / 8);
  bf16x8 lo = k_new[src + j], hi = k_new[src + half8 + j];
  if (rope) {
    const int p = n_valid + t;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, sn;
      rope_cos_sin(p, inv_freq[8 * j + e], c, sn);
      const float a = bf2f(lo[e]), bb = bf2f(hi[e]);
      lo[e] = f2bf(a * c - bb * sn);
      hi[e] = f2bf(bb * c + a * sn);
    }
  }
  ck[dst + j] = lo;
  ck[dst + half8 + j] = hi;
  cv[dst + j] = v_new[src + j];
  cv[dst + half8 + j] = v_new[src + half8 + j];
  if (j == 0 && row % Hkv == 0) pm[(int64_t)b * cap + len + t] = 1;
}

// Launch shapes (compute waves; every workgroup has one more wave that issues the
// K/V loads).  GQA 8:1 at d = 256: seven waves of one 16-row tile (14 query
// tokens x 8 heads per workgroup), eight waves in all, two per SIMD.  The
// decode's 51-token suffix fits four such workgroups with 5 padded tokens.
constexpr int kNR256 = 1, kNW256 = 7;
constexpr int kNWdec = 7;
// A single-token (autoregressive) decode: one compute wave, one 16-row tile
// holding the token's 8 heads (the other 8 rows idle); the key split supplies
// the parallelism.
constexpr int kNWar = 1;
// MHA at d = 64: seven waves of one row tile (about 110 registers, so two
// workgroups share a CU).
constexpr int kNR64 = 1, kNW64 = 7;
using CfgG8 = Cfg<256, 8, kNR256, kNW256>;
using CfgDec = Cfg<256, 8, kNR256, kNWdec>;
// A decode of a few samples (at most 16 query blocks of seven waves) takes
// workgroups of three compute waves: twice the workgroups over the same splits,
// each with a shorter chain (measured: 3 % off the B = 1 control step; at B = 64
// it would halve the work per workgroup launch and run 2x slower).
constexpr int kNWdecS = 3;
using CfgDecS = Cfg<256, 8, kNR256, kNWdecS>;
// The latency-lean decode of a few samples (decode_small_kernel): four waves of
// one 16-row tile (8 query tokens per workgroup), at most kStages key tiles each.
constexpr int kNWsmall = 4;
using CfgSmall = Cfg<256, 8, kNR256, kNWsmall>;
using CfgAr = Cfg<256, 8, kNR256, kNWar>;

template <int D, int G, int NR, int NW>
pi_status launch_prefill(const void* q, const void* k, const void* v, void* o, int B, int L, int Hq, int Hkv,
                         float scale, const pi_mask* m, int n_split, float* opart, float* mlpart,
                         float rope_base, float* lse, hipStream_t s) {
  using C = Cfg<D, G, NR, NW>;
  const int n_qblk = (L + C::TOK - 1) / C::TOK;
  const Placement place = make_placement(B * Hkv * n_split, n_qblk);
  const int64_t grid = placement_grid(place);
  PI_REQUIRE(grid < (1ll << 31), PI_ERR_UNSUPPORTED, "prefill: grid too large");
  const float scale_log2 = scale * 1.4426950408889634f;
  prefill_kernel<D, G, NR, NW><<<(unsigned)grid, C::THREADS, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), B, L, Hq, Hkv, scale_log2, m->tok, m->tiles, m->n_qt, m->n_kt, m->forbid_bits,
      place, n_split, opart, mlpart, rope_base > 0.f ? m->pos : nullptr,
      rope_base > 0.f ? log2((double)rope_base) : 0.0, lse);
  return pi::check_launch("prefill_kernel");
}

// Key splits for a decode of B samples: enough workgroups to cover the chip
// (about 256) while giving each split at least two key tiles.
// (min_tiles: the fewest key tiles a split gets; three for the small-batch shape.)
template <typename C>
int decode_splits_for(int B, int S, int len, int min_tiles = 2) {
  const int n_qblk = (S + C::TOK - 1) / C::TOK;
  const int tiles = (len + TK - 1) / TK + (S + TK - 1) / TK;
  const int by_chip = 256 / std::max(1, B * n_qblk);
  return std::max(1, std::min({kMaxSplit, by_chip, tiles / min_tiles}));
}
bool small_decode(int B, int S) { return S > 1 && B * ((S + CfgDec::TOK - 1) / CfgDec::TOK) <= 16; }
// decode_small_kernel: key tiles of a sample (prefix slots, then suffix tokens)
// and its key split: twelve splits (measured at B = 1 against 8, 10 and 16: the
// partials the merge reads against each workgroup's chain), at least one tile
// each, at most kStages each, at most kMaxSplit (the merge's limit; a longer cache
// takes the streaming kernel).
constexpr int kSmallSplits = 12;
int small_tiles(int S, int len) { return (len + TK - 1) / TK + (S + TK - 1) / TK; }
int small_splits(int S, int len) {
  const int nt = small_tiles(S, len);
  return std::min(kMaxSplit, std::max((nt + kStages - 1) / kStages, std::min(kSmallSplits, nt)));
}

// Key splits for a GQA 8:1 prefill of B samples of L tokens (same rule as the
// decode's, over the prefill's query blocks).
int prefill_splits(int B, int L) {
  const int n_qblk = (L + CfgG8::TOK - 1) / CfgG8::TOK;
  const int tiles = (L + TK - 1) / TK;
  const int by_chip = 256 / std::max(1, B * n_qblk);
  return std::max(1, std::min({kMaxSplit, by_chip, tiles / 2}));
}

// Workspace of a key split over S query tokens per sample (fp32 partial chunks
// of 16 rows x 256 d, then (m, l) per row), for a launch configuration C.
template <typename C>
size_t split_ws_bytes(int B, int S, int splits) {
  if (splits <= 1) return 0;
  const int n_qblk = (S + C::TOK - 1) / C::TOK;
  const size_t chunks = (size_t)splits * B * n_qblk * C::ROWS / 16;
  return pi::align_up(chunks * 16 * 256 * sizeof(float), 256) + chunks * 32 * sizeof(float);
}

// Bytes of the rotated suffix K a decode with the rotary embedding keeps in its workspace.
size_t rope_ks_bytes(int B, int S) { return pi::align_up((size_t)B * S * 256 * 2, 256); }

// Decode workspace: [rotated suffix K (rotary embedding only)] [key-split partials
// of whichever kernel a cache of len slots takes].
size_t decode_split_bytes(int B, int S, int len) {
  if (S == 1) return split_ws_bytes<CfgAr>(B, S, decode_splits_for<CfgAr>(B, S, len));
  if (small_decode(B, S))
    return std::max(split_ws_bytes<CfgSmall>(B, S, small_splits(S, len)),
                    split_ws_bytes<CfgDecS>(B, S, decode_splits_for<CfgDecS>(B, S, len, 3)));
  return pi32::decode_split_bytes(B, S, pi32::decode_splits(B, S, len));
}
size_t decode_ws_bytes(int B, int S, int Hq, int len) {
  (void)Hq;
  return rope_ks_bytes(B, S) + decode_split_bytes(B, S, len);
}

}  // namespace

size_t pi::decode_workspace_max(int B, int S, int Hq) {
  // the longest cache takes the most splits
  return decode_ws_bytes(B, S, Hq, kMaxTiles * TK);
}

// Bytes of the rotated K a prefill with the rotary embedding keeps in its workspace.
static size_t rope_k_bytes(int B, int L, int Hkv, int d) { return pi::align_up((size_t)B * L * Hkv * d * 2, 256); }

extern "C" size_t pi_prefill_workspace_bytes(int B, int L, int Hq, int Hkv, int d) {
  if (B < 1 || L < 1) return 0;
  if (Hq == 8 && Hkv == 1 && d == 256)
    return rope_k_bytes(B, L, Hkv, d) + pi32::prefill_split_bytes(B, Hkv, L, pi32::prefill_splits(B, Hkv, L));
  if (Hq == Hkv && d == 64) return rope_k_bytes(B, L, Hkv, d);
  return 0;
}

extern "C" pi_status pi_joint_attn_prefill(const void* q, const void* k, const void* v, int B, int L, int Hq,
                                           int Hkv, int d, float scale, float rope_base, const pi_mask* mask,
                                           void* o, float* lse, const pi_kv_cache* cache, int layer,
                                           void* workspace, size_t workspace_bytes, pi_stream stream) {
  PI_REQUIRE(q && k && v && o && mask, PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: null pointer");
  PI_REQUIRE(pi::aligned16(q) && pi::aligned16(k) && pi::aligned16(v) && pi::aligned16(o), PI_ERR_INVALID_ARG,
             "pi_joint_attn_prefill: tensors must be 16-byte aligned");
  PI_REQUIRE(B >= 1 && L >= 1, PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: B=%d L=%d", B, L);
  PI_REQUIRE(mask->B == B && mask->N == L && mask->tok && mask->tiles, PI_ERR_INVALID_ARG,
             "pi_joint_attn_prefill: mask built for B=%d N=%d, call has B=%d L=%d", mask->B, mask->N, B, L);
  PI_REQUIRE(scale > 0.f && isfinite(scale), PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: scale must be > 0");
  PI_REQUIRE(rope_base == 0.f || (rope_base > 1.f && isfinite(rope_base)), PI_ERR_INVALID_ARG,
             "pi_joint_attn_prefill: rope_base must be 0 (off) or > 1");
  PI_REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, PI_ERR_INVALID_ARG,
             "pi_joint_attn_prefill: Hq=%d must be a multiple of Hkv=%d", Hq, Hkv);
  PI_REQUIRE(L <= kMaxTiles * TK, PI_ERR_UNSUPPORTED, "pi_joint_attn_prefill: L=%d exceeds %d tokens", L,
             kMaxTiles * TK);
  const bool gqa8 = (Hq == 8 && Hkv == 1 && d == 256);
  const bool mha64 = (Hq == Hkv && d == 64);
  PI_REQUIRE(gqa8 || mha64, PI_ERR_UNSUPPORTED,
             "pi_joint_attn_prefill: unsupported (Hq=%d, Hkv=%d, d=%d); supported: (8,1,256) and (H,H,64)", Hq,
             Hkv, d);
  PI_REQUIRE((int64_t)L * Hkv * d * 2 < 0x7FFFFFF0ll, PI_ERR_UNSUPPORTED,
             "pi_joint_attn_prefill: one sample's K/V exceeds 2 GiB");
  if (cache) {
    PI_REQUIRE(cache->k && cache->v, PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: cache has null k/v");
    PI_REQUIRE(cache->B == B && cache->Hkv == Hkv && cache->d == d && layer >= 0 && layer < cache->layers &&
                   cache->len >= 1 && cache->len <= L && cache->len <= cache->capacity,
               PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: cache shape does not match (layer %d)", layer);
  }
  const bool rope = rope_base > 0.f;
  // workspace: [rotated K (with the rotary embedding)] [key-split partials]
  const size_t rot_bytes = rope ? rope_k_bytes(B, L, Hkv, d) : 0;
  PI_REQUIRE(!rope || (workspace != nullptr && workspace_bytes >= rot_bytes), PI_ERR_WORKSPACE,
             "pi_joint_attn_prefill: the rotary embedding needs pi_prefill_workspace_bytes() of workspace");
  PI_REQUIRE(workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_joint_attn_prefill: workspace must be 256-byte aligned");
  PI_REQUIRE(!rope || mask->pos, PI_ERR_INVALID_ARG, "pi_joint_attn_prefill: mask has no positions");
  hipStream_t s = static_cast<hipStream_t>(stream);
  pi_status st;
  const void* kk = k;
  if (rope) {
    st = pi::rope_rows(k, workspace, (int64_t)B * L, Hkv, d, mask->pos, rope_base, s);
    if (st != PI_OK) return st;
    kk = workspace;
  }
  char* split_ws = workspace ? static_cast<char*>(workspace) + rot_bytes : nullptr;
  const size_t split_avail = workspace ? workspace_bytes - rot_bytes : 0;
  if (gqa8) {
    st = pi32::prefill(q, kk, v, o, B, L, Hq, Hkv, scale, mask, rope_base, lse, split_ws, split_avail, s);
  } else {
    st = launch_prefill<64, 1, kNR64, kNW64>(q, kk, v, o, B, L, Hq, Hkv, scale, mask, 1, nullptr, nullptr,
                                             rope_base, lse, s);
  }
  if (st != PI_OK || !cache) return st;
  const int row_chunks = Hkv * d / 8;
  const int64_t total = (int64_t)B * cache->len * row_chunks;
  const size_t layer_elems = (size_t)B * cache->capacity * Hkv * d;
  __bf16* ckl = static_cast<__bf16*>(cache->k) + (size_t)layer * layer_elems;
  __bf16* cvl = static_cast<__bf16*>(cache->v) + (size_t)layer * layer_elems;
  const int threads = 256;
  // the cache keeps rotated keys: a decode reads them as they are
  cache_write_kernel<<<(unsigned)((total + threads - 1) / threads), threads, 0, s>>>(
      static_cast<const u32x4*>(kk), static_cast<const u32x4*>(v), reinterpret_cast<u32x4*>(ckl),
      reinterpret_cast<u32x4*>(cvl), L, cache->capacity, cache->len, row_chunks, total);
  return pi::check_launch("cache_write_kernel");
}

extern "C" size_t pi_decode_workspace_bytes(int B, int S, int Hq, int len) {
  if (B < 1 || S < 1 || Hq < 1 || len < 0) return 0;
  return decode_ws_bytes(B, S, Hq, len);
}

namespace {

// Launch the decode with NWD waves per workgroup (split partials in split_ws when
// split_avail allows a key split), then the merge of the splits.
template <int NWD>
pi_status launch_decode(const pi_kv_cache* cache, const __bf16* ckl, const __bf16* cvl, const void* q_s,
                        const void* k_s, const void* v_s, const uint8_t* suffix_ar, int B, int S, float scale,
                        float rope_base, void* o_s, bool tiled, char* split_ws, size_t split_avail, hipStream_t s) {
  using C = Cfg<256, 8, kNR256, NWD>;
  const int n_qblk = (S + C::TOK - 1) / C::TOK;
  int splits = decode_splits_for<C>(B, S, cache->len, NWD == kNWdecS ? 3 : 2);
  if (split_ws == nullptr || split_avail < split_ws_bytes<C>(B, S, splits)) splits = 1;   // one pass per sample
  const size_t chunks = (size_t)splits * B * n_qblk * NWD * kNR256;
  float* opart = splits > 1 ? reinterpret_cast<float*>(split_ws) : nullptr;
  float* mlpart = splits > 1 ? reinterpret_cast<float*>(split_ws + pi::align_up(chunks * 16 * 256 * sizeof(float), 256))
                             : nullptr;
  const Placement place = make_placement(B * splits, n_qblk);
  const bool rope = rope_base > 0.f;
  decode_kernel<256, 8, kNR256, NWD><<<(unsigned)placement_grid(place), C::THREADS, 0, s>>>(
      ckl, cvl, cache->prefix_mask, cache->capacity, cache->len, static_cast<const __bf16*>(q_s),
      static_cast<const __bf16*>(k_s), static_cast<const __bf16*>(v_s), suffix_ar, B, S,
      scale * 1.4426950408889634f, static_cast<__bf16*>(o_s), tiled ? 1 : 0, place, splits, opart, mlpart,
      rope ? 1 : 0, rope ? log2((double)rope_base) : 0.0);
  pi_status st = pi::check_launch("decode_kernel");
  if (st != PI_OK || splits == 1) return st;
  decode_combine_kernel<kNR256, NWD><<<(unsigned)(chunks / splits * 4), 256, 0, s>>>(
      opart, mlpart, static_cast<__bf16*>(o_s), tiled ? 1 : 0, B, S, n_qblk, splits, nullptr);
  return pi::check_launch("decode_combine_kernel");
}

// The few-sample decode (decode_small_kernel) when the cache's tiles fit its
// shares (at most kStages tiles per split) and the partials fit the workspace;
// false: not launched, the caller takes the streaming kernel.
bool try_decode_small(pi_status& st, const pi_kv_cache* cache, const __bf16* ckl, const __bf16* cvl,
                      const void* q_s, const void* k_s, const void* v_s, const uint8_t* suffix_ar, int B, int S,
                      float scale, float rope_base, void* o_s, bool tiled, char* split_ws, size_t split_avail,
                      hipStream_t s) {
  using C = CfgSmall;
  const int nt = small_tiles(S, cache->len);
  int splits = small_splits(S, cache->len);
  if (nt > kStages * splits) return false;
  if (splits > 1 && (split_ws == nullptr || split_avail < split_ws_bytes<C>(B, S, splits))) {
    if (nt > kStages) return false;
    splits = 1;   // without room for the partials, a short cache still fits one share
  }
  const int n_qblk = (S + C::TOK - 1) / C::TOK;
  const size_t chunks = (size_t)splits * B * n_qblk * kNWsmall * kNR256;
  float* opart = splits > 1 ? reinterpret_cast<float*>(split_ws) : nullptr;
  float* mlpart = splits > 1 ? reinterpret_cast<float*>(split_ws + pi::align_up(chunks * 16 * 256 * sizeof(float), 256))
                             : nullptr;
  const Placement place = make_placement(B * splits, n_qblk);
  const bool rope = rope_base > 0.f;
  decode_small_kernel<256, 8, kNR256, kNWsmall><<<(unsigned)placement_grid(place), kNWsmall * 64, 0, s>>>(
      ckl, cvl, cache->prefix_mask, cache->capacity, cache->len, static_cast<const __bf16*>(q_s),
      static_cast<const __bf16*>(k_s), static_cast<const __bf16*>(v_s), suffix_ar, B, S,
      scale * 1.4426950408889634f, static_cast<__bf16*>(o_s), tiled ? 1 : 0, place, splits, opart, mlpart,
      rope ? 1 : 0, rope ? log2((double)rope_base) : 0.0);
  st = pi::check_launch("decode_small_kernel");
  if (st != PI_OK || splits == 1) return true;
  decode_combine_kernel<kNR256, kNWsmall><<<(unsigned)(chunks / splits * 4), 256, 0, s>>>(
      opart, mlpart, static_cast<__bf16*>(o_s), tiled ? 1 : 0, B, S, n_qblk, splits, nullptr);
  st = pi::check_launch("decode_combine_kernel");
  return true;
}

}  // namespace

pi_status pi::decode_layer(const pi_kv_cache* cache, int layer, const void* q_s, const void* k_s, const void* v_s,
                           const uint8_t* suffix_ar, int B, int S, int Hq, float scale, float rope_base, void* o_s,
                           bool tiled, void* workspace, size_t workspace_bytes, hipStream_t s) {
  PI_REQUIRE(cache && q_s && k_s && v_s && suffix_ar && o_s, PI_ERR_INVALID_ARG,
             "pi_suffix_decode_step: null pointer");
  PI_REQUIRE(cache->k && cache->v && cache->prefix_mask, PI_ERR_INVALID_ARG,
             "pi_suffix_decode_step: cache has null pointers");
  PI_REQUIRE(pi::aligned16(q_s) && pi::aligned16(k_s) && pi::aligned16(v_s) && pi::aligned16(o_s) &&
                 pi::aligned16(cache->k) && pi::aligned16(cache->v),
             PI_ERR_INVALID_ARG, "pi_suffix_decode_step: tensors must be 16-byte aligned");
  PI_REQUIRE(B >= 1 && S >= 1 && S <= 128, PI_ERR_INVALID_ARG, "pi_suffix_decode_step: B=%d S=%d (S <= 128)", B, S);
  PI_REQUIRE(cache->B == B && layer >= 0 && layer < cache->layers && cache->len >= 0 &&
                 cache->len <= cache->capacity,
             PI_ERR_INVALID_ARG, "pi_suffix_decode_step: cache/layer mismatch (layer %d of %d, B %d vs %d)", layer,
             cache->layers, cache->B, B);
  PI_REQUIRE(scale > 0.f && isfinite(scale), PI_ERR_INVALID_ARG, "pi_suffix_decode_step: scale must be > 0");
  PI_REQUIRE(rope_base == 0.f || (rope_base > 1.f && isfinite(rope_base)), PI_ERR_INVALID_ARG,
             "pi_suffix_decode_step: rope_base must be 0 (off) or > 1");
  PI_REQUIRE((cache->len + TK - 1) / TK + (S + TK - 1) / TK <= kMaxTiles, PI_ERR_UNSUPPORTED,
             "pi_suffix_decode_step: cache length %d too long", cache->len);
  PI_REQUIRE(Hq == 8 && cache->Hkv == 1 && cache->d == 256, PI_ERR_UNSUPPORTED,
             "pi_suffix_decode_step: supported heads are Hq=8, Hkv=1, d=256 (got %d, %d, %d)", Hq, cache->Hkv,
             cache->d);
  PI_REQUIRE(workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_suffix_decode_step: workspace must be 256-byte aligned");
  const bool rope = rope_base > 0.f;
  const size_t rot_bytes = rope ? rope_ks_bytes(B, S) : 0;
  PI_REQUIRE(!rope || (workspace != nullptr && workspace_bytes >= rot_bytes), PI_ERR_WORKSPACE,
             "pi_suffix_decode_step: the rotary embedding needs pi_decode_workspace_bytes() of workspace");
  const void* kk = k_s;
  if (rope) {
    // the cache holds keys rotated by the prefill; the suffix keys are rotated here
    const pi_status st = pi::rope_suffix(k_s, workspace, B, S, 1, 256, cache->prefix_mask, cache->capacity,
                                         cache->len, rope_base, s);
    if (st != PI_OK) return st;
    kk = workspace;
  }
  char* split_ws = workspace ? static_cast<char*>(workspace) + rot_bytes : nullptr;
  const size_t split_avail = workspace ? workspace_bytes - rot_bytes : 0;
  const size_t layer_elems = (size_t)B * cache->capacity * 256;
  const __bf16* ckl = static_cast<const __bf16*>(cache->k) + (size_t)layer * layer_elems;
  const __bf16* cvl = static_cast<const __bf16*>(cache->v) + (size_t)layer * layer_elems;
  if (S == 1)
    return launch_decode<kNWar>(cache, ckl, cvl, q_s, kk, v_s, suffix_ar, B, S, scale, rope_base, o_s, tiled,
                                split_ws, split_avail, s);
  if (small_decode(B, S)) {
    pi_status st = PI_OK;
    if (try_decode_small(st, cache, ckl, cvl, q_s, kk, v_s, suffix_ar, B, S, scale, rope_base, o_s, tiled, split_ws,
                         split_avail, s))
      return st;
    return launch_decode<kNWdecS>(cache, ckl, cvl, q_s, kk, v_s, suffix_ar, B, S, scale, rope_base, o_s, tiled,
                                  split_ws, split_avail, s);
  }
  return pi32::decode(cache, ckl, cvl, q_s, kk, v_s, suffix_ar, B, S, scale, rope_base, o_s, tiled, split_ws,
                      split_avail, s);
}

extern "C" pi_status pi_suffix_decode_step(const pi_kv_cache* cache, int layer, const void* q_s, const void* k_s,
                                           const void* v_s, const uint8_t* suffix_ar, int B, int S, int Hq,
                                           float scale, float rope_base, void* o_s, void* workspace,
                                           size_t workspace_bytes, pi_stream stream) {
  return pi::decode_layer(cache, layer, q_s, k_s, v_s, suffix_ar, B, S, Hq, scale, rope_base, o_s, false,
                          workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Allocation-free cached decode for callers that cannot allocate (code under
// graph capture, tight serving loops): the decode's scratch (the rotated suffix
// keys and the key-split partials) lives in one file-scope device array per
// GPU instead of a caller workspace.  Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol); its device address
// is looked up once per device with that device current and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PI_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)

// The scratch address on the device that owns `stream` (the current device for
// the null stream), looked up on the first call there.
pi_status scratch_address(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) {
    dev = cur;
    if (stream != nullptr) e = hipStreamGetDevice(stream, &dev);
  }
  PI_REQUIRE(e == hipSuccess, PI_ERR_HIP, "pi_suffix_decode_step_noalloc: no device for the stream: %s",
             hipGetErrorString(e));
  PI_REQUIRE(dev >= 0 && dev < kMaxDevices, PI_ERR_UNSUPPORTED, "pi_suffix_decode_step_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    PI_REQUIRE(e == hipSuccess && p != nullptr, PI_ERR_HIP,
               "pi_suffix_decode_step_noalloc: scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PI_OK;
}
}  // namespace

extern "C" pi_status pi_suffix_decode_step_noalloc(const pi_kv_cache* cache, int layer, const void* q_s,
                                                   const void* k_s, const void* v_s, const uint8_t* suffix_ar,
                                                   int B, int S, int Hq, float scale, float rope_base, void* o_s,
                                                   pi_stream stream) {
  PI_REQUIRE(B >= 1 && S >= 1 && S <= 128, PI_ERR_INVALID_ARG, "pi_suffix_decode_step_noalloc: B=%d S=%d (S <= 128)",
             B, S);
  const size_t rot = rope_base > 0.f ? rope_ks_bytes(B, S) : 0;
  PI_REQUIRE(rot <= PI_NOALLOC_SCRATCH_BYTES, PI_ERR_UNSUPPORTED,
             "pi_suffix_decode_step_noalloc: the rotated suffix keys of B=%d x S=%d need %zu bytes, more than the "
             "%zu-byte scratch", B, S, rot, (size_t)PI_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const pi_status st = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (st != PI_OK) return st;
  // the scratch stands in for a workspace of its size: the key split runs when its
  // partials fit (as it would with that workspace), otherwise the call runs unsplit
  return pi::decode_layer(cache, layer, q_s, k_s, v_s, suffix_ar, B, S, Hq, scale, rope_base, o_s, false, ws,
                          PI_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

extern "C" pi_status pi_kv_cache_append(const pi_kv_cache* cache, int layer, const void* k_new, const void* v_new,
                                        int n_new, float rope_base, pi_stream stream) {
  PI_REQUIRE(cache && k_new && v_new, PI_ERR_INVALID_ARG, "pi_kv_cache_append: null pointer");
  PI_REQUIRE(cache->k && cache->v && cache->prefix_mask, PI_ERR_INVALID_ARG,
             "pi_kv_cache_append: cache has null pointers");
  PI_REQUIRE(pi::aligned16(k_new) && pi::aligned16(v_new) && pi::aligned16(cache->k) && pi::aligned16(cache->v),
             PI_ERR_INVALID_ARG, "pi_kv_cache_append: tensors must be 16-byte aligned");
  PI_REQUIRE(layer >= 0 && layer < cache->layers && cache->B >= 1 && cache->B <= 65535, PI_ERR_INVALID_ARG,
             "pi_kv_cache_append: layer %d of %d, B %d", layer, cache->layers, cache->B);
  PI_REQUIRE(n_new >= 1 && cache->len >= 0 && cache->len + n_new <= cache->capacity, PI_ERR_INVALID_ARG,
             "pi_kv_cache_append: %d tokens after %d do not fit %d slots", n_new, cache->len, cache->capacity);
  PI_REQUIRE(cache->Hkv >= 1 && cache->d >= 16 && cache->d <= 512 && cache->d % 16 == 0, PI_ERR_UNSUPPORTED,
             "pi_kv_cache_append: Hkv=%d d=%d", cache->Hkv, cache->d);
  PI_REQUIRE(rope_base == 0.f || (rope_base > 1.f && isfinite(rope_base)), PI_ERR_INVALID_ARG,
             "pi_kv_cache_append: rope_base must be 0 (off) or > 1");
  const int d = cache->d, Hkv = cache->Hkv;
  const size_t layer_elems = (size_t)cache->B * cache->capacity * Hkv * d;
  bf16x8* ckl = reinterpret_cast<bf16x8*>(static_cast<__bf16*>(cache->k) + (size_t)layer * layer_elems);
  bf16x8* cvl = reinterpret_cast<bf16x8*>(static_cast<__bf16*>(cache->v) + (size_t)layer * layer_elems);
  const int64_t per_b = (int64_t)n_new * Hkv * (d / 16);
  const dim3 grid((unsigned)((per_b + 255) / 256), (unsigned)cache->B);
  // the prefix_mask is const for the attention calls, which only read it; the append owns these slots
  cache_append_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const bf16x8*>(k_new), static_cast<const bf16x8*>(v_new), ckl, cvl,
      const_cast<uint8_t*>(cache->prefix_mask), cache->capacity, cache->len, n_new, Hkv, d,
      rope_base > 0.f ? log2((double)rope_base) : 0.0);
  return pi::check_launch("cache_append_kernel");
}
