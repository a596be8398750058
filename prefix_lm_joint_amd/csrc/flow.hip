// Euler flow-matching sampler and the stand-in velocity net, gfx950.
//
// Sampler ("VLA 代码精读 — OpenPI & StarVLA" §1.2, §1.6): x starts at the noise,
// dt = -1/N, step k evaluates the velocity at t_k = 1 + k*dt and sets
// x <- x + dt*v; t runs from 1 (noise) to 0 (action).
//
// Stand-in velocity net (random weights; the pages show only the shapes: a state
// token and 50 action tokens projected to the expert width, the expert's
// 8-head / 1-KV-head / d=256 attention over the cached prefix plus the suffix,
// and an output projection back to the action dim):
//   h[:,0]   = r(state) W_state^T + b_state
//   h[:,1+i] = r(x_i) W_in^T + b_in + t * w_time
//   per cache layer l: a = r(h); q,k,v = r(a W_{q,k,v}^T / rms(a)); o = r(decode_l); h += o W_o^T
//   v = a[:,1:] W_out^T / rms(a[:,1:]) + b_out            (a = r(h) after the last layer)
// r() is rounding to bf16; every matrix product runs on the matrix cores with
// bf16 operands and fp32 accumulation.  rms(a) = sqrt(mean(a^2) + 1e-6) is the
// per-stream RMS norm ahead of the projections ("π0.5 vs MM-DiT joint attention",
// first section), taken on the same bf16 activations the product reads; being a
// per-row scalar it is applied to the accumulator.
//
// Layout: the residual stream h stays fp32 row-major; next to it every producer
// of h also writes a = r(h) in the operand tile layout (tiled_offset), the
// decode writes its output in that layout too, and the weights are repacked into
// it once per call, so every operand fragment a GEMM wave needs is one
// contiguous 1 KB load.
#include "common.h"

#include <math.h>

namespace {

enum { EPI_QKV = 0, EPI_RESID = 1, EPI_VEL = 2, EPI_EULER = 3 };

struct GemmArgs {
  const __bf16* a;     // activations [M (padded to 64) x K], operand tile layout
  const __bf16* w;     // weights [N (padded to 16) x K], operand tile layout
  int M, N, K;
  int n1, n2;          // EPI_QKV: output column split q | k | v
  __bf16* o0;          // EPI_QKV outputs: q in the decode's tile layout, k / v row-major
  __bf16* o1;
  __bf16* o2;
  float* out;          // EPI_RESID: h [M x N] fp32; EPI_VEL / EPI_EULER: [B*H x N]
  __bf16* a_out;       // EPI_RESID: r(h) in tile layout, row width N
  int S;               // tokens per sample (row m % S == 0 is the state token)
  const float* bias;   // EPI_VEL / EPI_EULER
  float dt;            // EPI_EULER
};

constexpr float kRmsEps = 1e-6f;

// Epilogue of four consecutive output columns nb .. nb+3 of row m (r: the
// product, already divided by the row's rms when the product normalises).
template <int EPI>
__device__ __forceinline__ void finish_store(const GemmArgs& p, int m, int nb, f32x4 r) {
  if constexpr (EPI == EPI_QKV) {
    // q in the decode's tile layout (rows t*8 + head per sample, padded to 16),
    // k and v row-major
    __bf16* dst;
    if (nb < p.n1) {
      const int64_t qrow = (int64_t)(m / p.S) * ((p.S * 8 + 15) / 16 * 16) + (m % p.S) * 8 + nb / 256;
      dst = p.o0 + tiled_offset(qrow, nb % 256, 256);
    } else if (nb < p.n1 + p.n2) dst = p.o1 + (int64_t)m * p.n2 + (nb - p.n1);
    else dst = p.o2 + (int64_t)m * (p.N - p.n1 - p.n2) + (nb - p.n1 - p.n2);
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f2bf(r[i]);
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else if constexpr (EPI == EPI_RESID) {
    // h += o W_o^T, and r(h) for the next projection (N is a multiple of 64)
    f32x4* dst = reinterpret_cast<f32x4*>(p.out + (int64_t)m * p.N + nb);
    f32x4 hv = *dst;
    hv += r;
    *dst = hv;
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f2bf(hv[i]);
    *reinterpret_cast<bf16x4*>(p.a_out + tiled_offset(m, nb, p.N)) = v;
  } else {
    const int j = m % p.S;
    if (j == 0) return;                            // state token: no velocity
    float* dst = p.out + ((int64_t)(m / p.S) * (p.S - 1) + j - 1) * p.N + nb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (nb + i >= p.N) break;
      if constexpr (EPI == EPI_VEL) dst[i] = r[i] + p.bias[nb + i];
      else dst[i] += p.dt * (r[i] + p.bias[nb + i]);
    }
  }
}

// out[m][n] = sum_k A[m][k] W[n][k]  (divided by rms(A[m]) when NORM).
//
// Workgroup tile TN = 16*NT columns x 64 rows.  The NWV waves split the
// contraction into NWV contiguous ranges and each computes the whole tile over
// its range, KB k-steps at a time: all of a batch's fragment loads (one 1 KB
// contiguous read each, from the tile layout) are issued before the first wait.
// The partial tiles are summed through LDS.  Small batches (M = 51 rows per
// sample) use 16-column tiles and sixteen waves, so many workgroups each wait on
// one short batch of loads.  Products are computed transposed (A operand =
// weights, B operand = activations) so a lane holds four consecutive output
// columns of one row.
template <int EPI, bool NORM, int NT, int NWV, int MF>
__global__ void __launch_bounds__(NWV * 64) gemm_kernel(GemmArgs p) {
  constexpr int TN = 16 * NT;
  constexpr int TM = 16 * MF;                    // rows per workgroup: MF 16-row fragments
  constexpr int PS = TN + 4;                     // LDS row stride (floats) of a partial tile
  constexpr int KB = 4;                          // k-steps of loads in flight
  __shared__ float part[NWV][TM * PS];
  __shared__ float ssp[NWV][TM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM;
  const int kb = p.K / 32;

  // fragment (row block, k-step) of a tile-layout matrix
  const bf16x8* wt = reinterpret_cast<const bf16x8*>(p.w) + (int64_t)(n0 / 16) * kb * 64 + lane;
  const bf16x8* at = reinterpret_cast<const bf16x8*>(p.a) + (int64_t)(m0 / 16) * kb * 64 + lane;

  f32x4 acc[NT][MF];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) ss[j] = 0.f;

  const int per = (kb + NWV - 1) / NWV;
  const int ks_lo = wave * per, ks_hi = min(kb, ks_lo + per);
  for (int ks0 = ks_lo; ks0 < ks_hi; ks0 += KB) {
    bf16x8 wf[KB][NT], af[KB][MF];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const bool live = ks0 + u < ks_hi;          // uniform over the wave
#pragma unroll
      for (int j = 0; j < NT; ++j)
        wf[u][j] = (live && n0 + 16 * j < p.N) ? wt[((int64_t)j * kb + ks0 + u) * 64] : bf16x8{};
#pragma unroll
      for (int j = 0; j < MF; ++j) af[u][j] = live ? at[((int64_t)j * kb + ks0 + u) * 64] : bf16x8{};
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch is issued before the first wait
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < MF; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = bf2f(af[u][j][i]);
            ss[j] += x * x;
          }
      }
#pragma unroll
      for (int jn = 0; jn < NT; ++jn)
#pragma unroll
        for (int jm = 0; jm < MF; ++jm) acc[jn][jm] = mfma16x16x32(wf[u][jn], af[u][jm], acc[jn][jm]);
    }
  }

  // partial tiles and partial row sums of squares to LDS
#pragma unroll
  for (int jn = 0; jn < NT; ++jn)
#pragma unroll
    for (int jm = 0; jm < MF; ++jm)
      *reinterpret_cast<f32x4*>(&part[wave][(16 * jm + c) * PS + 16 * jn + 4 * g]) = acc[jn][jm];
  if constexpr (NORM) {
#pragma unroll
    for (int jm = 0; jm < MF; ++jm) {
      const float t = group4_sum(ss[jm]);
      if (g == 0) ssp[wave][16 * jm + c] = t;
    }
  }
  __syncthreads();

  // finish: each task is four consecutive columns of one row
  for (int task = threadIdx.x; task < TM * TN / 4; task += NWV * 64) {
    const int ml = task / (TN / 4);
    const int nl = 4 * (task % (TN / 4));
    const int m = m0 + ml, nb = n0 + nl;
    if (m >= p.M || nb >= p.N) continue;
    f32x4 r = *reinterpret_cast<const f32x4*>(&part[0][ml * PS + nl]);
#pragma unroll
    for (int w = 1; w < NWV; ++w) r += *reinterpret_cast<const f32x4*>(&part[w][ml * PS + nl]);
    if constexpr (NORM) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) t += ssp[w][ml];
      r *= rsqrtf(t / (float)p.K + kRmsEps);
    }
    finish_store<EPI>(p, m, nb, r);
  }
}

// Products of many rows (a batch of samples: M > 256, N a multiple of 256, K of
// 128): workgroup tile 64 rows x 256 columns, four waves each owning 64 columns
// of all 64 rows (4 x 4 products of 16 x 16 per k-step of 32).  A wave streams
// its own fragments, the tile's four A fragments (the same for the four waves,
// shared through the L1) and its four W fragments, kWideAhead k-steps ahead of
// its products, so no LDS stage and no barrier sits in the loop.  Tiles go to
// the XCDs in contiguous runs of a grouped order (eight row tiles, columns
// fastest), so each XCD's L2 holds about eight row tiles of A and eight column
// blocks of W.  With NORM, wave w also sums the squares of row block w.
constexpr int kWideAhead = 4;

template <int EPI, bool NORM>
__global__ void __launch_bounds__(256) gemm_wide_kernel(GemmArgs p) {
  constexpr int P = kWideAhead;
  __shared__ float ssq[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int n_mt = (p.M + 63) / 64, n_nt = p.N / 256, T = n_mt * n_nt;
  const int per = (T + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= T) return;
  const int gsz = 8 * n_nt;
  const int grp = t / gsz, rem = t % gsz;
  const int rows_in_grp = min(8, n_mt - grp * 8);
  const int mt = grp * 8 + rem % rows_in_grp, nt = rem / rows_in_grp;
  const int m0 = mt * 64, n0 = nt * 256 + 64 * wave;
  const int kb = p.K / 32;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  const bf16x8* at = reinterpret_cast<const bf16x8*>(p.a) + (int64_t)(m0 / 16) * kb * 64 + lane;
  const bf16x8* wt = reinterpret_cast<const bf16x8*>(p.w) + (int64_t)(n0 / 16) * kb * 64 + lane;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  bf16x8 af[P][4], wf[P][4];
  auto load = [&](int slot, int ks) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      af[slot][j] = at[((int64_t)j * kb + ks) * 64];
      wf[slot][j] = wt[((int64_t)j * kb + ks) * 64];
    }
  };
#pragma unroll
  for (int u = 0; u < P; ++u) load(u, u);
  for (int ks0 = 0; ks0 < kb; ks0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == wv) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float x = bf2f(af[u][j][i]);
              ss += x * x;
            }
          }
      }
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm) acc[jn][jm] = mfma16x16x32(wf[u][jn], af[u][jm], acc[jn][jm]);
      if (ks0 + u + P < kb) load(u, ks0 + u + P);
    }
  }
  float inv[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (NORM) {
    const float tsum = group4_sum(ss);
    if (g == 0) ssq[16 * wave + c] = tsum;
    __syncthreads();
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) inv[jm] = rsqrtf(ssq[16 * jm + c] / (float)p.K + kRmsEps);
  }
#pragma unroll
  for (int jm = 0; jm < 4; ++jm) {
    const int m = m0 + 16 * jm + c;
    if (m >= p.M) continue;
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) finish_store<EPI>(p, m, n0 + 16 * jn + 4 * g, acc[jn][jm] * inv[jm]);
  }
}

// Suffix tokens: row m = b*S + j; j = 0 the state token, j >= 1 action j-1.
// Contraction length is the action dim (<= 64): plain fp32 dot products.  Writes
// h (fp32, row-major) and r(h) (tile layout).
__global__ void __launch_bounds__(256)
embed_kernel(const float* __restrict__ x, const float* __restrict__ state, const __bf16* __restrict__ w_state,
             const float* __restrict__ b_state, const __bf16* __restrict__ w_in, const float* __restrict__ b_in,
             const float* __restrict__ w_time, float t, float* __restrict__ h, __bf16* __restrict__ a,
             int H, int A, int W) {
  __shared__ float in[64];
  const int m = blockIdx.y;
  const int S = H + 1;
  const int b = m / S, j = m % S;
  const float* src = (j == 0) ? state + (int64_t)b * A : x + ((int64_t)b * H + (j - 1)) * A;
  if (threadIdx.x < A) in[threadIdx.x] = bf2f(f2bf(src[threadIdx.x]));
  __syncthreads();
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= W) return;
  const __bf16* wr = (j == 0 ? w_state : w_in) + (int64_t)n * A;
  float acc = 0.f;
  for (int k = 0; k < A; ++k) acc += in[k] * bf2f(wr[k]);
  acc += (j == 0) ? b_state[n] : (b_in[n] + t * w_time[n]);
  h[(int64_t)m * W + n] = acc;
  a[tiled_offset(m, n, W)] = f2bf(acc);
}

// Weights [rows x K] row-major -> operand tile layout at row offset row0 of a
// matrix with rows_pad rows; rows in [rows, rows_pad) are zero.  One thread per
// 8 elements.
__global__ void repack_kernel(const __bf16* __restrict__ src, __bf16* __restrict__ dst, int rows, int rows_pad,
                              int row0, int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int k8 = K / 8;
  if (i >= (int64_t)rows_pad * k8) return;
  const int r = (int)(i / k8), k = (int)(i % k8) * 8;
  const bf16x8 v = r < rows ? *reinterpret_cast<const bf16x8*>(src + (int64_t)r * K + k) : bf16x8{};
  *reinterpret_cast<bf16x8*>(dst + tiled_offset(row0 + r, k, K)) = v;
}

// Zero the pad rows [S*Hq, pad16(S*Hq)) of each sample's queries in the decode's
// tile layout (width d).  No product writes them, yet the decode reads them as
// whole 16-row blocks: left as they were, leftover values would reach the
// scores of rows that are never stored (and could make the softmax redo a
// workgroup for nothing).  One thread per element.
__global__ void zero_q_pad_kernel(__bf16* __restrict__ q, int rows, int rows_pad, int d, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int per = (rows_pad - rows) * d;
  const int64_t b = i / per;
  const int j = (int)(i % per);
  q[tiled_offset(b * rows_pad + rows + j / d, j % d, d)] = f2bf(0.f);
}

__global__ void euler_kernel(float* __restrict__ x, const float* __restrict__ v, float dt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i4 = 4 * i;
  if (i4 + 3 < n) {
    f32x4 xv = *reinterpret_cast<const f32x4*>(x + i4);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(v + i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[e] = xv[e] + dt * vv[e];
    *reinterpret_cast<f32x4*>(x + i4) = xv;
  } else {
    for (int64_t e = i4; e < n; ++e) x[e] = x[e] + dt * v[e];
  }
}

// Tile choice.  A small batch (at most 256 rows) runs sixteen waves per workgroup
// splitting the contraction, so each wave waits on a single short batch of loads,
// and tiles chosen for what one CU reads: 16 x 16 tiles when the columns are few
// (the output projection back to the width: 256 workgroups, each with a quarter of
// the activations), 32 x 32 when they are many (the QKV projection: 160
// workgroups reading 64 KB of weights and 64 KB of activations each; measured
// against 16 x 64 and 64 x 16: 4 % and 8 % faster at B = 1).  A batch of samples
// (more rows) takes the wide tiles of gemm_wide_kernel (at B = 64: the QKV
// product 36.9 -> 27.4 us, the output projection 31.5 -> 28.4 us against 64 x 64
// tiles of four waves splitting the contraction, which remain for other shapes).
template <int EPI, bool NORM>
pi_status gemm(const GemmArgs& a, hipStream_t s, const char* name) {
  if (a.M <= 256 && (a.N + 15) / 16 * ((a.M + 63) / 64) < 128) {
    dim3 grid((a.N + 15) / 16, (a.M + 15) / 16);
    gemm_kernel<EPI, NORM, 1, 16, 1><<<grid, 1024, 0, s>>>(a);
  } else if (a.M <= 256) {
    dim3 grid((a.N + 31) / 32, (a.M + 31) / 32);
    gemm_kernel<EPI, NORM, 2, 16, 2><<<grid, 1024, 0, s>>>(a);
  } else if (a.N % 256 == 0 && a.K % (32 * kWideAhead) == 0) {
    const int tiles = (a.M + 63) / 64 * (a.N / 256);
    gemm_wide_kernel<EPI, NORM><<<(unsigned)((tiles + 7) / 8 * 8), 256, 0, s>>>(a);
  } else {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    gemm_kernel<EPI, NORM, 4, 4, 4><<<grid, 256, 0, s>>>(a);
  }
  return pi::check_launch(name);
}

struct FlowWs {
  float* h;           // residual stream [Mpad x W] fp32
  __bf16* a;          // r(h), tile layout [Mpad x W]
  __bf16* q;          // queries, the decode's tile layout [B x pad16(S*Hq) x d]
  __bf16 *k, *v;      // suffix keys / values, row-major [B*S x Hkv*d]
  __bf16* o;          // decode output, tile layout [Mpad x Hq*d]
  __bf16* w_qkv;      // repacked weights, tile layout
  __bf16* w_o;
  __bf16* w_out;
  float* vel;
  void* dec;          // decode key-split partials
  size_t dec_bytes;
  size_t total;
};

inline int pad64(int m) { return (m + 63) / 64 * 64; }
inline int pad16(int m) { return (m + 15) / 16 * 16; }

FlowWs flow_layout(const pi_velocity_net* n, int B, int H, char* base) {
  const size_t S = (size_t)H + 1;
  const size_t M = B * S, Mp = pad64((int)M);
  const size_t nq = (size_t)n->Hq * n->d, nkv = (size_t)n->Hkv * n->d, W = n->width;
  size_t off = 0;
  FlowWs w;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = pi::align_up(off + bytes, 256);
    return base ? base + at : nullptr;
  };
  w.h = reinterpret_cast<float*>(take(sizeof(float) * Mp * W));
  w.a = reinterpret_cast<__bf16*>(take(2 * Mp * W));
  w.q = reinterpret_cast<__bf16*>(take(2 * B * (size_t)pad16((int)S * n->Hq) * n->d));
  w.k = reinterpret_cast<__bf16*>(take(2 * M * nkv));
  w.v = reinterpret_cast<__bf16*>(take(2 * M * nkv));
  w.o = reinterpret_cast<__bf16*>(take(2 * Mp * nq));
  w.w_qkv = reinterpret_cast<__bf16*>(take(2 * (nq + 2 * nkv) * W));
  w.w_o = reinterpret_cast<__bf16*>(take(2 * W * nq));
  w.w_out = reinterpret_cast<__bf16*>(take(2 * (size_t)pad16(n->action_dim) * W));
  w.vel = reinterpret_cast<float*>(take(sizeof(float) * B * H * n->action_dim));
  w.dec_bytes = pi::decode_workspace_max(B, (int)S, n->Hq);
  w.dec = w.dec_bytes ? take(w.dec_bytes) : nullptr;
  w.total = off;
  return w;
}

pi_status check_net(const pi_velocity_net* n, const pi_kv_cache* cache, const uint8_t* suffix_ar,
                    const float* state, int B, int H, int A, const char* who) {
  PI_REQUIRE(n && cache && suffix_ar && state, PI_ERR_INVALID_ARG, "%s: null pointer", who);
  PI_REQUIRE(n->w_state && n->b_state && n->w_in && n->b_in && n->w_time && n->w_q && n->w_k && n->w_v &&
                 n->w_o && n->w_out && n->b_out,
             PI_ERR_INVALID_ARG, "%s: velocity net has a null weight", who);
  PI_REQUIRE(pi::aligned16(n->w_q) && pi::aligned16(n->w_k) && pi::aligned16(n->w_v) && pi::aligned16(n->w_o) &&
                 pi::aligned16(n->w_out),
             PI_ERR_INVALID_ARG, "%s: weights must be 16-byte aligned", who);
  PI_REQUIRE(n->Hq == 8 && n->Hkv == 1 && n->d == 256, PI_ERR_UNSUPPORTED,
             "%s: velocity net heads must be Hq=8, Hkv=1, d=256", who);
  PI_REQUIRE(n->width >= 64 && n->width % 64 == 0, PI_ERR_UNSUPPORTED, "%s: width %d must be a multiple of 64",
             who, n->width);
  PI_REQUIRE(A == n->action_dim && A >= 1 && A <= 64, PI_ERR_INVALID_ARG, "%s: action dim %d (net %d, max 64)",
             who, A, n->action_dim);
  PI_REQUIRE(B >= 1 && H >= 1 && H + 1 <= 128, PI_ERR_INVALID_ARG, "%s: B=%d H=%d (H+1 <= 128)", who, B, H);
  PI_REQUIRE(cache->B == B && cache->Hkv == 1 && cache->d == 256 && cache->layers >= 1 && cache->k && cache->v &&
                 cache->prefix_mask && cache->len >= 0 && cache->len <= cache->capacity,
             PI_ERR_INVALID_ARG, "%s: cache does not match the net / batch", who);
  return PI_OK;
}

pi_status repack(const void* src, __bf16* dst, int rows, int rows_pad, int row0, int K, hipStream_t s) {
  const int64_t n = (int64_t)rows_pad * (K / 8);
  repack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const __bf16*>(src), dst, rows, rows_pad,
                                                              row0, K);
  return pi::check_launch("repack_kernel");
}

// Weights into the operand tile layout (once per sampler or velocity call).
pi_status repack_weights(const pi_velocity_net* n, const FlowWs& w, hipStream_t s) {
  const int W = n->width, nq = n->Hq * n->d, nkv = n->Hkv * n->d;
  pi_status st = repack(n->w_q, w.w_qkv, nq, nq, 0, W, s);
  if (st == PI_OK) st = repack(n->w_k, w.w_qkv, nkv, nkv, nq, W, s);
  if (st == PI_OK) st = repack(n->w_v, w.w_qkv, nkv, nkv, nq + nkv, W, s);
  if (st == PI_OK) st = repack(n->w_o, w.w_o, W, W, 0, nq, s);
  if (st == PI_OK) st = repack(n->w_out, w.w_out, n->action_dim, pad16(n->action_dim), 0, W, s);
  return st;
}

// Once per call: zero the pad rows of the tiled queries (see zero_q_pad_kernel).
pi_status clear_q_pad(const pi_velocity_net* n, const FlowWs& w, int B, int S, hipStream_t s) {
  const int rows = S * n->Hq, rows_pad = pad16(rows);
  if (rows_pad == rows) return PI_OK;
  const int64_t total = (int64_t)B * (rows_pad - rows) * n->d;
  zero_q_pad_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(w.q, rows, rows_pad, n->d, total);
  return pi::check_launch("zero_q_pad_kernel");
}

// v = net(x, t) into `vel` (EPI_VEL) or fused x += dt*v (EPI_EULER, vel ignored).
template <int EPI>
pi_status run_net(const pi_velocity_net* n, const pi_kv_cache* cache, const uint8_t* suffix_ar,
                  const float* state, float* x, float t, float dt, float* vel, int B, int H, int A,
                  const FlowWs& w, hipStream_t s) {
  const int S = H + 1, W = n->width;
  const int M = B * S;
  const int nq = n->Hq * n->d, nkv = n->Hkv * n->d;
  const float scale = 1.0f / sqrtf((float)n->d);
  {
    dim3 grid((W + 255) / 256, M);
    embed_kernel<<<grid, 256, 0, s>>>(x, state, static_cast<const __bf16*>(n->w_state), n->b_state,
                                      static_cast<const __bf16*>(n->w_in), n->b_in, n->w_time, t, w.h, w.a, H, A, W);
    pi_status st = pi::check_launch("embed_kernel");
    if (st != PI_OK) return st;
  }
  for (int layer = 0; layer < cache->layers; ++layer) {
    GemmArgs g{};
    g.a = w.a;
    g.w = w.w_qkv;
    g.M = M;
    g.N = nq + 2 * nkv;
    g.K = W;
    g.n1 = nq;
    g.n2 = nkv;
    g.o0 = w.q;
    g.o1 = w.k;
    g.o2 = w.v;
    g.S = S;
    pi_status st = gemm<EPI_QKV, true>(g, s, "gemm_qkv");
    if (st != PI_OK) return st;
    st = pi::decode_layer(cache, layer, w.q, w.k, w.v, suffix_ar, B, S, n->Hq, scale, 0.f, w.o, true, w.dec, w.dec_bytes,
                          s);
    if (st != PI_OK) return st;
    GemmArgs go{};
    go.a = w.o;
    go.w = w.w_o;
    go.M = M;
    go.N = W;
    go.K = nq;
    go.out = w.h;
    go.a_out = w.a;
    st = gemm<EPI_RESID, false>(go, s, "gemm_out_resid");
    if (st != PI_OK) return st;
  }
  // velocity over every token row; the epilogue drops the state token rows
  GemmArgs gv{};
  gv.a = w.a;
  gv.w = w.w_out;
  gv.M = M;
  gv.N = A;
  gv.K = W;
  gv.S = S;
  gv.bias = n->b_out;
  gv.dt = dt;
  if (EPI == EPI_EULER) {
    gv.out = x;
    return gemm<EPI_EULER, true>(gv, s, "gemm_velocity_euler");
  }
  gv.out = vel;
  return gemm<EPI_VEL, true>(gv, s, "gemm_velocity");
}

}  // namespace

extern "C" pi_status pi_euler_update(float* x, const float* v, float dt, int64_t n, pi_stream stream) {
  PI_REQUIRE(x && v, PI_ERR_INVALID_ARG, "pi_euler_update: null pointer");
  PI_REQUIRE(n >= 0, PI_ERR_INVALID_ARG, "pi_euler_update: n=%lld", (long long)n);
  PI_REQUIRE(pi::aligned16(x) && pi::aligned16(v), PI_ERR_INVALID_ARG, "pi_euler_update: 16-byte alignment");
  if (n == 0) return PI_OK;
  const int64_t threads = 256, n4 = (n + 3) / 4;
  euler_kernel<<<(unsigned)((n4 + threads - 1) / threads), (unsigned)threads, 0, static_cast<hipStream_t>(stream)>>>(
      x, v, dt, n);
  return pi::check_launch("euler_kernel");
}

extern "C" size_t pi_flow_workspace_bytes(const pi_velocity_net* net, int B, int H) {
  if (!net || B < 1 || H < 1) return 0;
  return flow_layout(net, B, H, nullptr).total;
}

extern "C" pi_status pi_velocity_eval(const pi_velocity_net* net, const pi_kv_cache* cache, const uint8_t* suffix_ar,
                                      const float* state, const float* x, float t, float* vel, int B, int H, int A,
                                      void* workspace, size_t workspace_bytes, pi_stream stream) {
  pi_status st = check_net(net, cache, suffix_ar, state, B, H, A, "pi_velocity_eval");
  if (st != PI_OK) return st;
  PI_REQUIRE(x && vel && workspace, PI_ERR_INVALID_ARG, "pi_velocity_eval: null pointer");
  FlowWs w = flow_layout(net, B, H, static_cast<char*>(workspace));
  PI_REQUIRE(workspace_bytes >= w.total, PI_ERR_WORKSPACE, "pi_velocity_eval: workspace %zu < %zu", workspace_bytes,
             w.total);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_velocity_eval: workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = repack_weights(net, w, s);
  if (st == PI_OK) st = clear_q_pad(net, w, B, H + 1, s);
  if (st != PI_OK) return st;
  return run_net<EPI_VEL>(net, cache, suffix_ar, state, const_cast<float*>(x), t, 0.f, vel, B, H, A, w, s);
}

extern "C" pi_status pi_flow_sample(const pi_velocity_net* net, const pi_kv_cache* cache, const uint8_t* suffix_ar,
                                    const float* state, const float* v_const, float* x, int B, int H, int A,
                                    int num_steps, void* workspace, size_t workspace_bytes, pi_stream stream) {
  PI_REQUIRE(x, PI_ERR_INVALID_ARG, "pi_flow_sample: null x");
  PI_REQUIRE(num_steps >= 1, PI_ERR_INVALID_ARG, "pi_flow_sample: num_steps=%d", num_steps);
  PI_REQUIRE(B >= 1 && H >= 1 && A >= 1, PI_ERR_INVALID_ARG, "pi_flow_sample: B=%d H=%d A=%d", B, H, A);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double dt = -1.0 / num_steps;
  if (!net) {
    PI_REQUIRE(v_const, PI_ERR_INVALID_ARG, "pi_flow_sample: constant-velocity mode needs v_const");
    for (int k = 0; k < num_steps; ++k) {
      pi_status st = pi_euler_update(x, v_const, (float)dt, (int64_t)B * H * A, stream);
      if (st != PI_OK) return st;
    }
    return PI_OK;
  }
  pi_status st = check_net(net, cache, suffix_ar, state, B, H, A, "pi_flow_sample");
  if (st != PI_OK) return st;
  PI_REQUIRE(workspace, PI_ERR_INVALID_ARG, "pi_flow_sample: null workspace");
  FlowWs w = flow_layout(net, B, H, static_cast<char*>(workspace));
  PI_REQUIRE(workspace_bytes >= w.total, PI_ERR_WORKSPACE, "pi_flow_sample: workspace %zu < %zu", workspace_bytes,
             w.total);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_flow_sample: workspace must be 256-byte aligned");
  st = repack_weights(net, w, s);
  if (st == PI_OK) st = clear_q_pad(net, w, B, H + 1, s);
  if (st != PI_OK) return st;
  for (int k = 0; k < num_steps; ++k) {
    const float t = (float)(1.0 + k * dt);
    st = run_net<EPI_EULER>(net, cache, suffix_ar, state, x, t, (float)dt, nullptr, B, H, A, w, s);
    if (st != PI_OK) return st;
  }
  return PI_OK;
}
