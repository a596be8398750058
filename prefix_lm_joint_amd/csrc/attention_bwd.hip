// Backward of the masked grouped-query joint attention (Hq = 8, Hkv = 1, d = 256), gfx950.
//
// What is computed ("VLA 代码精读 — OpenPI & StarVLA" §1.5: training runs the
// same joint forward under the block mask and differentiates the loss through
// it): for an upstream gradient dO of the output, per query row (b, t, h) with
// visible keys J (all rows read the one KV head),
//   P_j  = exp(scale q.k_j - lse)         lse: the row's log-sum-exp (the forward keeps it)
//   dP_j = dO.v_j,   Dr = dO.O = sum_j P_j dP_j
//   dS_j = P_j (dP_j - Dr)
//   dQ   = scale sum_j dS_j k_j,   dK_j += scale dS_j q,   dV_j += P_j dO.
// Masked pairs get P = 0 by selection; a row with no visible key contributes
// nothing.  With the rotary embedding the kernels run on the rotated Q and K
// and the gradients of the unrotated inputs are the rotated ones turned back by
// the negated positions (the rotation is orthogonal).
//
// Kernels:
//   * bwd_prep_kernel: Dr of every row from the bf16 O and dO (fp32 sum), and
//     the row's lse in base 2 (+inf for a row with no visible key, whose
//     weights then come out exactly 0).
//   * dq32_kernel (attention32.hip, pi32::dq): query-major, on the forward's
//     32 x 32 x 16 engine: 4 waves x 32 rows (16 tokens x 8 heads) per
//     workgroup with Q and dO rows in registers.  Per 32-key tile: S^T = K Q^T
//     and dP^T = V dO^T (row-wise reads of K and V), dS^T elementwise from the
//     row's lse2 and Dr, dQ^T += K^T dS^T (transposing reads of K, dS^T straight
//     from the accumulators as the forward's P^T).
//   * dkdv_kernel: key-major, the same engine with queries and keys swapped: 4
//     waves x 16 keys per workgroup with K and V rows in registers, tiles of 32
//     query rows (4 tokens x 8 heads) of Q, dO and the row statistics streamed
//     over four LDS stages.  Per tile: S^T = Q K^T and dP^T = dO V^T (row-wise
//     reads), P^T and dS^T elementwise, dV^T += dO^T P^T and dK^T += Q^T dS^T
//     (transposing reads).  The fp32 dK and dV of 16 keys x 256 take 128
//     registers per lane, so each wave runs alone on its SIMD with the whole
//     register file and issues its share of the tile loads itself.
//   * dkdv_kernel's tiles are swizzled with f_U, so one copy in LDS serves both
//     the row-wise and the transposing read without bank conflicts.
// Each pipeline step runs one block on the matrix cores: the transposed
// products of tile i-1 and the row-wise products of tile i+1, then the
// elementwise work of tile i; tile i+2 streams in meanwhile.
#include "common.h"
#include "engine.h"
#include "attention32.h"

#include <math.h>

#include <type_traits>

namespace {

using namespace pi_engine;

constexpr int BD = 256;                       // head dim
constexpr int BG = 8;                         // query heads (the KV head is shared)
constexpr uint32_t kHalf = 16u * BD * 2u;     // bytes of 16 tile rows
constexpr float kLog2e = 1.4426950408889634f;
using T256 = Tile<BD>;

// Per-lane byte offsets of the operand reads within a tile, computed once.
//   row(ds): row-wise read, rows c (+16 rows: + kHalf), logical chunk 4 ds + g
//            (A[c][32 ds + 8 g ..] of a 16-row block)
//   tr(dt):  transposing read, rows 4g + c/4 (+16 rows: + kHalf), columns
//            16 dt + 4 (c % 4) ..; hands lane (c, g) column 16 dt + c of rows
//            4g .. 4g+3 (and 16 + 4g ..), the k slots of the accumulator layout.
// f_U < 16 flips only the low four chunk bits, so the upper half of a row (chunks
// 16..31) is the lower half's offset + 256 bytes: only half the offsets are kept.
struct BwdOffsets {
  uint32_t row_[BD / 64];
  uint32_t tr_[BD / 32];
  __device__ __forceinline__ uint32_t row(int ds) const { return row_[ds & 3] + (uint32_t)(ds >> 2) * 256u; }
  __device__ __forceinline__ uint32_t tr(int dt) const { return tr_[dt & 7] + (uint32_t)(dt >> 3) * 256u; }
};
static_assert(BD == 256, "offset halves assume rows of 32 chunks");

__device__ __forceinline__ BwdOffsets bwd_offsets() {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  BwdOffsets lo;
#pragma unroll
  for (int ds = 0; ds < BD / 64; ++ds) lo.row_[ds] = 2u * (uint32_t)(c * BD + 8 * ((4 * ds + g) ^ T256::fu(c)));
  const int vr = 4 * g + (c >> 2);
#pragma unroll
  for (int dt = 0; dt < BD / 32; ++dt)
    lo.tr_[dt] = 2u * (uint32_t)(vr * BD + 4 * (c & 1) + 8 * ((2 * dt + ((c & 3) >> 1)) ^ T256::fu(vr)));
  return lo;
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 read_row(const __bf16* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + off);
}
__device__ __forceinline__ bf16x8 read_tr(const __bf16* tile, uint32_t off) {
  const bf16x4 lo4 = lds_read_tr4(reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(tile) + off));
  const bf16x4 hi4 =
      lds_read_tr4(reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(tile) + off + kHalf));
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Row statistics: Dr = dO . O and lse2 = lse * log2(e); for a row with no
// visible key (lse = -inf) Dr = 0 and lse2 = +inf.
// 32 lanes per row, 8 elements each.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout, const float* __restrict__ lse,
                float* __restrict__ lse2, float* __restrict__ dr, int64_t rows) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
  const int l = threadIdx.x & 31;
  if (row >= rows) return;   // whole 32-lane groups leave together
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * BD + l * 8);
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * BD + l * 8);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(bf2f(a[i]), bf2f(b[i]), s);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (l == 0) {
    const float x = lse[row];
    const bool none = x == -INFINITY;
    dr[row] = none ? 0.f : s;     // a key-less row adds nothing, whatever its dO holds
    lse2[row] = none ? INFINITY : x * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV (key-major).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int entry_cls(uint32_t e) { return (int)((e >> 16) & 0xFFu); }

constexpr int kNWk = 4;                                    // waves, 16 keys each
constexpr int kKeyBlk = kNWk * 16;                         // keys per workgroup
constexpr int kMaxQTiles = kMaxTiles * TK / PI_MASK_TILE_Q;
static_assert(PI_MASK_TILE_Q == 16, "a query tile is four 4-token steps");

// A stage: 32 query rows (4 tokens x 8 heads) of Q (t.k) and dO (t.v), each
// row's query word (t.w), lse2 and Dr (lanes >= 32 of their loads land as zeros).
struct DkvStage {
  Stage<BD> t;
  alignas(16) float lse2[64];
  alignas(16) float dr[64];
};

struct DkvWave {
  bf16x8 kf[BD / 32], vf[BD / 32];   // B operands: K and V of key c, d = 32 ds + 8 g ..
  f32x4 dk[BD / 16], dv[BD / 16];     // dK^T, dV^T [16 j + 4 g + i][key c]
  uint32_t wk;
};

// S^T = Q K^T and dP^T = dO V^T of one tile (the pipeline's first).
__device__ __forceinline__ void dkv_products(const DkvStage& st, const BwdOffsets& lo, const DkvWave& w,
                                             f32x4 (&s)[2], f32x4 (&dp)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) s[h] = dp[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < BD / 16; ++j) {
    s[j & 1] = mfma16x16x32(read_row(st.t.k, lo.row(j >> 1) + (j & 1) * kHalf), w.kf[j >> 1], s[j & 1]);
    dp[j & 1] = mfma16x16x32(read_row(st.t.v, lo.row(j >> 1) + (j & 1) * kHalf), w.vf[j >> 1], dp[j & 1]);
  }
}

// One dK/dV step's block: dV^T += dO^T P^T and dK^T += Q^T dS^T for tile i-1
// (transposing reads of `pst`), S^T = Q K^T and dP^T = dO V^T for tile i+1
// (row-wise reads of `nst`), and P^T and dS^T of tile i (statistics in `cst`),
// one weight per two slots (exponential in the even slot, dS and the bf16
// roundings in the odd one) under the products.  Lane (c, g) holds rows
// 16 h + 4 g + i for key c, packed as the B operands of dV^T += dO^T P^T and
// dK^T += Q^T dS^T.
template <bool PV>
__device__ __forceinline__ void dkv_block(const DkvStage& pst, const DkvStage& cst, const DkvStage& nst,
                                          const BwdOffsets& lo, DkvWave& w, const bf16x8& pfp, const bf16x8& dsp,
                                          const f32x4 (&s)[2], const f32x4 (&dp)[2], bf16x8& pf_new,
                                          bf16x8& ds_new, f32x4 (&s_n)[2], f32x4 (&dp_n)[2], int cls,
                                          uint32_t forbid, float c2) {
  constexpr int NS = BD / 16, AH = 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) s_n[h] = dp_n[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto rq = [&](int j) { return read_row(nst.t.k, lo.row(j >> 1) + (j & 1) * kHalf); };
  auto ro = [&](int j) { return read_row(nst.t.v, lo.row(j >> 1) + (j & 1) * kHalf); };
  auto tq = [&](int j) { return read_tr(pst.t.k, lo.tr(j)); };
  auto to = [&](int j) { return read_tr(pst.t.v, lo.tr(j)); };
  // tile i's row statistics and the visibility of this lane's 8 (row, key) pairs
  const int g = (threadIdx.x & 63) >> 4;
  f32x4 l2[2], d2[2];
  uint32_t vis = 0xFFu;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    l2[h] = *reinterpret_cast<const f32x4*>(&cst.lse2[16 * h + 4 * g]);
    d2[h] = *reinterpret_cast<const f32x4*>(&cst.dr[16 * h + 4 * g]);
    if (cls == PI_TILE_PARTIAL) {
      const u32x4 wq = *reinterpret_cast<const u32x4*>(&cst.t.w[16 * h + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!pair_visible(wq[i], w.wk, forbid)) vis &= ~(1u << (4 * h + i));
    }
  }
  bf16x8 qb[AH], ob[AH], tqb[AH], tob[AH];
#pragma unroll
  for (int j = 0; j < AH; ++j) {
    if constexpr (PV) {
      tob[j] = to(j);
      tqb[j] = tq(j);
    }
    qb[j] = rq(j);
    ob[j] = ro(j);
  }
  float pe[8];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    if constexpr (PV) {
      w.dv[j] = mfma16x16x32(tob[j % AH], pfp, w.dv[j]);
      w.dk[j] = mfma16x16x32(tqb[j % AH], dsp, w.dk[j]);
    }
    s_n[j & 1] = mfma16x16x32(qb[j % AH], w.kf[j >> 1], s_n[j & 1]);
    dp_n[j & 1] = mfma16x16x32(ob[j % AH], w.vf[j >> 1], dp_n[j & 1]);
    if (j + AH < NS) {
      if constexpr (PV) {
        tob[j % AH] = to(j + AH);
        tqb[j % AH] = tq(j + AH);
      }
      qb[j % AH] = rq(j + AH);
      ob[j % AH] = ro(j + AH);
    }
    const int e = j >> 1, h = e >> 2, i = e & 3;
    if ((j & 1) == 0) {
      const float p = hw_exp2(fmaf(s[h][i], c2, -l2[h][i]));
      pe[e] = ((vis >> e) & 1u) ? p : 0.f;
      asm volatile("" : "+v"(pe[e]));
    } else {
      pf_new[e] = f2bf(pe[e]);
      ds_new[e] = f2bf(pe[e] * (dp[h][i] - d2[h][i]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ void dkv_last(const DkvStage& pst, const BwdOffsets& lo, DkvWave& w, const bf16x8& pfp,
                                         const bf16x8& dsp) {
#pragma unroll
  for (int j = 0; j < BD / 16; ++j) {
    w.dv[j] = mfma16x16x32(read_tr(pst.t.v, lo.tr(j)), pfp, w.dv[j]);
    w.dk[j] = mfma16x16x32(read_tr(pst.t.k, lo.tr(j)), dsp, w.dk[j]);
  }
}

// The dK/dV tile loop: four stages, one barrier per tile; every wave issues its
// share of tile i+2's loads right after step i's barrier.  The four stages are
// four LDS objects and every step names the one its loads fill, so the compiler
// sees that the step's reads of the other three do not depend on the loads in
// flight (with one array, or a stage picked at run time, it made the first
// read after the loads wait for them, every step).
template <typename Desc, typename Issue>
__device__ __forceinline__ void dkv_tiles(DkvStage& s0, DkvStage& s1, DkvStage& s2, DkvStage& s3,
                                          const BwdOffsets& lo, DkvWave& w, int n, Desc desc, Issue issue,
                                          uint32_t forbid, float c2) {
  if (n <= 0) return;
  issue(0, s0);
  if (n > 1) issue(1, s1);
  int cls_cur = entry_cls(desc(0)), cls_nxt = n > 1 ? entry_cls(desc(1)) : 0;
  wait_vmem();          // the K/V rows and this wave's share of tiles 0 and 1
  __syncthreads();
  f32x4 s[2], dp[2];
  dkv_products(s0, lo, w, s, dp);
  bf16x8 pfp, dsp;
#pragma unroll
  for (int e = 0; e < 8; ++e) pfp[e] = dsp[e] = f2bf(0.f);
  auto step = [&](auto pv, int i, DkvStage& prev, DkvStage& cur, DkvStage& nxt, DkvStage& ld) {
    wait_vmem();          // this wave's loads of tile i+1
    __syncthreads();      // everyone's; and every wave is done with tile i-2
    if (i + 2 < n) issue(i + 2, ld);
    bf16x8 pf_new, ds_new;
    f32x4 s_n[2], dp_n[2];
    dkv_block<decltype(pv)::value>(prev, cur, nxt, lo, w, pfp, dsp, s, dp, pf_new, ds_new, s_n, dp_n, cls_cur,
                                   forbid, c2);
    cls_cur = cls_nxt;
    if (i + 2 < n) cls_nxt = entry_cls(desc(i + 2));
    pfp = pf_new;
    dsp = ds_new;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = s_n[h];
      dp[h] = dp_n[h];
    }
  };
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;
  step(NoPV{}, 0, s3, s0, s1, s2);
  for (int i = 1; i < n; i += 4) {
    step(WithPV{}, i, s0, s1, s2, s3);
    if (i + 1 < n) step(WithPV{}, i + 1, s1, s2, s3, s0);
    if (i + 2 < n) step(WithPV{}, i + 2, s2, s3, s0, s1);
    if (i + 3 < n) step(WithPV{}, i + 3, s3, s0, s1, s2);
  }
  const int last = (n - 1) & 3;
  dkv_last(last == 0 ? s0 : last == 1 ? s1 : last == 2 ? s2 : s3, lo, w, pfp, dsp);
}

// One workgroup per (sample, block of 64 keys), XCD-placed per sample.  Up
// front wave 0 lists the 16-token query tiles with a visible pair for any key
// of the block (class merged over the block's two key tiles); each listed tile
// is four steps of 4 tokens.  Rows of padded tokens and rows past the last token
// load as zeros (their statistics give P = 0, Dr = 0): they add exactly zero.
__global__ void __launch_bounds__(kNWk * 64)
dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
            const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dr,
            __bf16* __restrict__ dk, __bf16* __restrict__ dv, int L, float scale, float c2,
            const uint32_t* __restrict__ tok, const uint8_t* __restrict__ tiles, int n_qt, int n_kt,
            uint32_t forbid, Placement place) {
  __shared__ DkvStage st0, st1, st2, st3;
  __shared__ uint32_t qlist[kMaxQTiles];
  __shared__ uint32_t qvalid[kMaxTiles];
  __shared__ int qcount;
  int b, kblk;
  if (!xcd_place(place, b, kblk)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int key0 = kblk * kKeyBlk;
  const uint32_t* tk = tok + (size_t)b * L;
  token_bitmap(tk, L, n_kt, kNWk, qvalid);
  if (wave == 0) {
    const uint8_t* trow = tiles + (size_t)b * n_qt * n_kt;
    const int kt_lo = key0 / TK, kt_hi = min(n_kt, (key0 + kKeyBlk + TK - 1) / TK);
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
  DkvWave w;
  const int key = key0 + wave * 16 + c;
  const bool ok = key < L;
  {
    // keys past the end read key 0 and are never stored; a padded key's K and V
    // are replaced by zeros so nothing it holds reaches a product
    const int64_t r = (int64_t)b * L + (ok ? key : 0);
    w.wk = ok ? tk[key] : 0u;
    const bool live = (w.wk & 1u) != 0u;
#pragma unroll
    for (int ds = 0; ds < BD / 32; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(k + r * BD + ds * 32 + 8 * g);
      const bf16x8 d = *reinterpret_cast<const bf16x8*>(v + r * BD + ds * 32 + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w.kf[ds][e] = live ? a[e] : f2bf(0.f);
        w.vf[ds][e] = live ? d[e] : f2bf(0.f);
      }
    }
#pragma unroll
    for (int j = 0; j < BD / 16; ++j) w.dk[j] = w.dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const int n = 4 * qcount;
  // this wave's loads: rows 8 wave .. 8 wave + 7 of the tile (the 8 heads of its
  // token), two rows per instruction, source chunks pre-swizzled with f_U
  uint32_t roff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = 8 * wave + 2 * jj + (lane >> 5), p = lane & 31;
    roff[jj] = (uint32_t)r * (BD * 2u) + 16u * (uint32_t)(p ^ T256::fu(r));
  }
  const float* lse2_b = lse2 + (size_t)b * L * BG;
  const float* dr_b = dr + (size_t)b * L * BG;
  const __bf16* q_b = q + (size_t)b * L * BG * BD;
  const __bf16* o_b = dout + (size_t)b * L * BG * BD;
  auto desc = [&](int i) { return qlist[i >> 2]; };
  auto issue = [&](int i, DkvStage& sg) {
    const int t0 = (int)(qlist[i >> 2] & 0xFFFFu) * PI_MASK_TILE_Q + (i & 3) * 4;   // first token
    const int tw = t0 + wave;                                                         // this wave's token
    const bool in = (qvalid[tw >> 5] >> (tw & 31)) & 1u;   // in range and valid, else zeros
    const int64_t at = (int64_t)__builtin_amdgcn_readfirstlane(t0) * BG * BD * 2;
    const i32x4 rq = make_rsrc(reinterpret_cast<const char*>(q_b) + at);
    const i32x4 ro = make_rsrc(reinterpret_cast<const char*>(o_b) + at);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t off = in ? roff[jj] : kOOB;
      pi_buffer_load_lds(rq, lds_u32(&sg.t.k[(8 * wave + 2 * jj) * BD]), 16, (int)off, 0, 0, 0);
      pi_buffer_load_lds(ro, lds_u32(&sg.t.v[(8 * wave + 2 * jj) * BD]), 16, (int)off, 0, 0, 0);
    }
    // statistics of the 32 rows: wave 0 the query words, 1 lse2, 2 Dr
    const bool row_in = lane < 32 && t0 + (lane >> 3) < L;
    if (wave == 0) {
      const uint32_t off = row_in ? (uint32_t)(t0 + (lane >> 3)) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(tk), lds_u32(&sg.t.w[0]), 4, (int)off, 0, 0, 0);
    } else if (wave == 1) {
      const uint32_t off = row_in ? (uint32_t)(t0 * BG + lane) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(lse2_b), lds_u32(&sg.lse2[0]), 4, (int)off, 0, 0, 0);
    } else if (wave == 2) {
      const uint32_t off = row_in ? (uint32_t)(t0 * BG + lane) * 4u : kOOB;
      pi_buffer_load_lds(make_rsrc(dr_b), lds_u32(&sg.dr[0]), 4, (int)off, 0, 0, 0);
    }
  };
  const BwdOffsets lo = bwd_offsets();
  dkv_tiles(st0, st1, st2, st3, lo, w, n, desc, issue, forbid, c2);
  if (!ok) return;
  const int64_t r = ((int64_t)b * L + key) * BD + 4 * g;
#pragma unroll
  for (int j = 0; j < BD / 16; ++j) {
    bf16x4 xk, xv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xk[i] = f2bf(w.dk[j][i] * scale);
      xv[i] = f2bf(w.dv[j][i]);
    }
    *reinterpret_cast<bf16x4*>(dk + r + 16 * j) = xk;
    *reinterpret_cast<bf16x4*>(dv + r + 16 * j) = xv;
  }
}

size_t stats_bytes(int B, int L) { return pi::align_up((size_t)B * L * BG * sizeof(float), 256); }

// With the rotary embedding: rotated Q [B, L, 8, 256] and K [B, L, 1, 256] (bf16)
// and the negated positions [B, L] the gradients are rotated back with.
size_t rope_bytes(int B, int L) {
  return pi::align_up((size_t)B * L * BG * BD * 2, 256) + pi::align_up((size_t)B * L * BD * 2, 256) +
         pi::align_up((size_t)B * L * sizeof(int32_t), 256);
}

__global__ void negate_kernel(const int32_t* __restrict__ pos, int32_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = -pos[i];
}

}  // namespace

extern "C" size_t pi_attn_backward_workspace_bytes(int B, int L, int Hq, int Hkv, int d, float rope_base) {
  if (B < 1 || L < 1 || Hq != BG || Hkv != 1 || d != BD) return 0;
  return 2 * stats_bytes(B, L) + (rope_base > 0.f ? rope_bytes(B, L) : 0);
}

extern "C" pi_status pi_joint_attn_backward(const void* q, const void* k, const void* v, const void* o,
                                            const void* dout, const float* lse, int B, int L, int Hq, int Hkv,
                                            int d, float scale, float rope_base, const pi_mask* mask, void* dq,
                                            void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                            pi_stream stream) {
  PI_REQUIRE(q && k && v && o && dout && lse && mask && dq && dk && dv, PI_ERR_INVALID_ARG,
             "pi_joint_attn_backward: null pointer");
  PI_REQUIRE(pi::aligned16(q) && pi::aligned16(k) && pi::aligned16(v) && pi::aligned16(o) && pi::aligned16(dout) &&
                 pi::aligned16(dq) && pi::aligned16(dk) && pi::aligned16(dv) &&
                 (reinterpret_cast<uintptr_t>(lse) & 3u) == 0,
             PI_ERR_INVALID_ARG, "pi_joint_attn_backward: tensors must be 16-byte aligned (lse 4-byte)");
  PI_REQUIRE(B >= 1 && L >= 1, PI_ERR_INVALID_ARG, "pi_joint_attn_backward: B=%d L=%d", B, L);
  PI_REQUIRE(mask->B == B && mask->N == L && mask->tok && mask->tiles, PI_ERR_INVALID_ARG,
             "pi_joint_attn_backward: mask built for B=%d N=%d, call has B=%d L=%d", mask->B, mask->N, B, L);
  PI_REQUIRE(scale > 0.f && isfinite(scale), PI_ERR_INVALID_ARG, "pi_joint_attn_backward: scale must be > 0");
  PI_REQUIRE(Hq == BG && Hkv == 1 && d == BD, PI_ERR_UNSUPPORTED,
             "pi_joint_attn_backward: unsupported (Hq=%d, Hkv=%d, d=%d); supported: (8,1,256)", Hq, Hkv, d);
  PI_REQUIRE(L <= kMaxTiles * TK, PI_ERR_UNSUPPORTED, "pi_joint_attn_backward: L=%d exceeds %d tokens", L,
             kMaxTiles * TK);
  PI_REQUIRE(rope_base == 0.f || (rope_base > 1.f && isfinite(rope_base)), PI_ERR_INVALID_ARG,
             "pi_joint_attn_backward: rope_base must be 0 (off) or > 1");
  PI_REQUIRE(rope_base == 0.f || mask->pos, PI_ERR_INVALID_ARG, "pi_joint_attn_backward: mask has no positions");
  const size_t need = pi_attn_backward_workspace_bytes(B, L, Hq, Hkv, d, rope_base);
  PI_REQUIRE(workspace != nullptr && workspace_bytes >= need, PI_ERR_WORKSPACE,
             "pi_joint_attn_backward: needs %zu workspace bytes, got %zu", need, workspace_bytes);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_joint_attn_backward: workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* lse2 = static_cast<float*>(workspace);
  float* dr = reinterpret_cast<float*>(static_cast<char*>(workspace) + stats_bytes(B, L));
  const int64_t rows = (int64_t)B * L * BG;
  pi_status st;
  // the rotary embedding: the kernels below see the rotated Q and K; the
  // gradients of the unrotated inputs are the rotated ones turned back by -p
  const bool rope = rope_base > 0.f;
  char* rw = static_cast<char*>(workspace) + 2 * stats_bytes(B, L);
  void* q_rot = rw;
  void* k_rot = rw + pi::align_up((size_t)B * L * BG * BD * 2, 256);
  int32_t* neg_pos = reinterpret_cast<int32_t*>(static_cast<char*>(k_rot) + pi::align_up((size_t)B * L * BD * 2, 256));
  if (rope) {
    if ((st = pi::rope_rows(q, q_rot, (int64_t)B * L, BG, BD, mask->pos, rope_base, s)) != PI_OK) return st;
    if ((st = pi::rope_rows(k, k_rot, (int64_t)B * L, 1, BD, mask->pos, rope_base, s)) != PI_OK) return st;
    q = q_rot;
    k = k_rot;
  }
  const float c2 = scale * kLog2e;
  bwd_prep_kernel<<<(unsigned)((rows * 32 + 255) / 256), 256, 0, s>>>(
      static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse, lse2, dr, rows);
  if ((st = pi::check_launch("bwd_prep_kernel")) != PI_OK) return st;
  const Placement pk = make_placement(B, (L + kKeyBlk - 1) / kKeyBlk);
  dkdv_kernel<<<(unsigned)placement_grid(pk), kNWk * 64, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<const __bf16*>(dout), lse2, dr, static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), L, scale, c2,
      mask->tok, mask->tiles, mask->n_qt, mask->n_kt, mask->forbid_bits, pk);
  st = pi::check_launch("dkdv_kernel");
  if (st != PI_OK) return st;
  if ((st = pi32::dq(q, k, v, dout, lse2, dr, dq, B, L, scale, mask, s)) != PI_OK || !rope) return st;
  const int64_t n = (int64_t)B * L;
  negate_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(mask->pos, neg_pos, n);
  if ((st = pi::check_launch("negate_kernel")) != PI_OK) return st;
  if ((st = pi::rope_rows(dq, dq, n, BG, BD, neg_pos, rope_base, s)) != PI_OK) return st;
  return pi::rope_rows(dk, dk, n, 1, BD, neg_pos, rope_base, s);
}
