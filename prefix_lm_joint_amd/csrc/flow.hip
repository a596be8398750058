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
//   per cache layer l: a = r(h); q,k,v = r(a W_{q,k,v}^T / rms(h)); o = r(decode_l); h += o W_o^T
//   v = r(h[:,1:]) W_out^T / rms(h[:,1:]) + b_out
// r() is rounding to bf16; every matrix product runs on the matrix cores with
// bf16 operands and fp32 accumulation.  rms(h) = sqrt(mean(h^2) + 1e-6) is the
// per-stream RMS norm ahead of the projections ("π0.5 vs MM-DiT joint attention",
// first section); being a per-row scalar it is applied to the accumulator, and the
// GEMM that reads the fp32 row of h accumulates its sum of squares on the way.
#include "common.h"

#include <math.h>

namespace {

// Physical row of logical row m: (m / div) * stride + off + m % div.
struct RowMap {
  int div, stride, off;
  __device__ __forceinline__ int64_t operator()(int m) const {
    return (int64_t)(m / div) * stride + off + (m % div);
  }
};

enum { EPI_QKV = 0, EPI_RESID = 1, EPI_VEL = 2, EPI_EULER = 3 };

struct GemmArgs {
  const void* a;       // activations, fp32 or bf16, row stride K
  RowMap amap;
  const __bf16* w0;    // weight rows [0, n1)
  const __bf16* w1;    // weight rows [n1, n1 + n2)
  const __bf16* w2;    // weight rows [n1 + n2, N)
  int n1, n2;
  int M, N, K;
  __bf16* o0;          // EPI_QKV outputs, row strides n1, n2, N - n1 - n2
  __bf16* o1;
  __bf16* o2;
  float* out;          // EPI_RESID / EPI_VEL / EPI_EULER output, row stride N
  RowMap omap;
  const float* bias;   // EPI_VEL / EPI_EULER
  float dt;            // EPI_EULER
};

// 8 consecutive elements of a row as bf16 (zero past K); `ss` accumulates the
// sum of squares of the unrounded values.
template <typename T>
__device__ __forceinline__ bf16x8 load_frag(const T* row, int k, int K, bool vec_ok, float& ss) {
  bf16x8 r;
  if (vec_ok && k + 8 <= K) {
    if constexpr (sizeof(T) == 2) {
      r = *reinterpret_cast<const bf16x8*>(row + k);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + k);
      const f32x4 b = *reinterpret_cast<const f32x4*>(row + k + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r[i] = f2bf(a[i]);
        r[i + 4] = f2bf(b[i]);
        ss += a[i] * a[i] + b[i] * b[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = (k + i < K) ? (float)row[k + i] : 0.f;
      r[i] = f2bf(f);
      ss += f * f;
    }
  }
  return r;
}

constexpr float kRmsEps = 1e-6f;

// out[m][n] = sum_k r(A[m][k]) W[n][k]  (divided by rms(A[m]) when NORM).
//
// Workgroup tile TN = 16*NT columns x 64 rows.  The NWV waves split the
// contraction into NWV contiguous ranges and each computes the whole tile over
// its range, with KB k-steps of loads in flight at a time; the partial tiles are
// summed through LDS.  Small batches (M = 51 rows per sample) use narrow tiles and
// sixteen waves, so many workgroups each wait on one short chain of loads instead
// of a few workgroups serialising on memory latency.  Products are computed
// transposed (A operand = weights, B operand = activations) so a lane holds four
// consecutive output columns of one row.
template <int EPI, typename TA, bool NORM, int NT, int NWV>
__global__ void __launch_bounds__(NWV * 64) gemm_kernel(GemmArgs p) {
  constexpr int TN = 16 * NT;
  constexpr int PS = TN + 4;                     // LDS row stride (floats) of a partial tile
  constexpr int KB = sizeof(TA) == 2 ? 4 : 2;    // k-steps of loads in flight
  __shared__ float part[NWV][64 * PS];
  __shared__ float ssp[NWV][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * 64;
  const bool vec_ok = (p.K & 7) == 0;

  const __bf16* wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = n0 + 16 * j + c;
    wok[j] = n < p.N;
    const __bf16* base = p.w0;
    int nn = n;
    if (n >= p.n1 + p.n2) { base = p.w2; nn = n - p.n1 - p.n2; }
    else if (n >= p.n1) { base = p.w1; nn = n - p.n1; }
    wrow[j] = base + (int64_t)(wok[j] ? nn : 0) * p.K;
  }
  const TA* arow[4];
  bool aok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 16 * j + c;
    aok[j] = m < p.M;
    arow[j] = static_cast<const TA*>(p.a) + (aok[j] ? p.amap(m) : 0) * p.K;
  }

  f32x4 acc[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  float ss_w = 0.f;

  const int ksteps = (p.K + 31) / 32;
  const int per = (ksteps + NWV - 1) / NWV;
  const int ks_lo = wave * per, ks_hi = min(ksteps, ks_lo + per);
  for (int ks0 = ks_lo; ks0 < ks_hi; ks0 += KB) {
    bf16x8 wf[KB][NT], af[KB][4];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = (ks0 + u) * 32 + 8 * g;
      const bool live = ks0 + u < ks_hi;
#pragma unroll
      for (int j = 0; j < NT; ++j) wf[u][j] = (live && wok[j]) ? load_frag(wrow[j], k, p.K, vec_ok, ss_w) : bf16x8{};
#pragma unroll
      for (int j = 0; j < 4; ++j) af[u][j] = (live && aok[j]) ? load_frag(arow[j], k, p.K, vec_ok, ss[j]) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int jn = 0; jn < NT; ++jn)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm) acc[jn][jm] = mfma16x16x32(wf[u][jn], af[u][jm], acc[jn][jm]);
  }
  (void)ss_w;

  // partial tiles and partial row sums of squares to LDS
#pragma unroll
  for (int jn = 0; jn < NT; ++jn)
#pragma unroll
    for (int jm = 0; jm < 4; ++jm)
      *reinterpret_cast<f32x4*>(&part[wave][(16 * jm + c) * PS + 16 * jn + 4 * g]) = acc[jn][jm];
  if constexpr (NORM) {
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) {
      const float t = group4_sum(ss[jm]);
      if (g == 0) ssp[wave][16 * jm + c] = t;
    }
  }
  __syncthreads();

  // finish: each task is four consecutive columns of one row
  for (int task = threadIdx.x; task < 16 * TN; task += NWV * 64) {
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
    if constexpr (EPI == EPI_QKV) {
      __bf16* dst;
      if (nb < p.n1) dst = p.o0 + (int64_t)m * p.n1 + nb;
      else if (nb < p.n1 + p.n2) dst = p.o1 + (int64_t)m * p.n2 + (nb - p.n1);
      else dst = p.o2 + (int64_t)m * (p.N - p.n1 - p.n2) + (nb - p.n1 - p.n2);
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f2bf(r[i]);
      *reinterpret_cast<bf16x4*>(dst) = v;
    } else {
      float* dst = p.out + p.omap(m) * p.N + nb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (nb + i >= p.N) break;
        if constexpr (EPI == EPI_RESID) dst[i] += r[i];
        else if constexpr (EPI == EPI_VEL) dst[i] = r[i] + p.bias[nb + i];
        else dst[i] += p.dt * (r[i] + p.bias[nb + i]);
      }
    }
  }
}

// Suffix tokens: row m = b*S + j; j = 0 the state token, j >= 1 action j-1.
// Contraction length is the action dim (<= 64): plain fp32 dot products.
__global__ void __launch_bounds__(256)
embed_kernel(const float* __restrict__ x, const float* __restrict__ state, const __bf16* __restrict__ w_state,
             const float* __restrict__ b_state, const __bf16* __restrict__ w_in, const float* __restrict__ b_in,
             const float* __restrict__ w_time, float t, float* __restrict__ h, int H, int A, int W) {
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

// Tile choice: 16-column tiles with sixteen waves splitting the contraction for
// the few rows of a small batch (each wave then waits on a single short batch of
// loads), 64 x 64 tiles with four waves once the rows alone give enough
// workgroups.
template <int EPI, typename TA, bool NORM>
pi_status gemm(const GemmArgs& a, hipStream_t s, const char* name) {
  if (a.M <= 256) {
    dim3 grid((a.N + 15) / 16, (a.M + 63) / 64);
    gemm_kernel<EPI, TA, NORM, 1, 16><<<grid, 1024, 0, s>>>(a);
  } else {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    gemm_kernel<EPI, TA, NORM, 4, 4><<<grid, 256, 0, s>>>(a);
  }
  return pi::check_launch(name);
}

struct FlowWs {
  float* h;
  __bf16 *q, *k, *v, *o;
  float* vel;
  void* dec;          // decode key-split partials
  size_t dec_bytes;
  size_t total;
};

FlowWs flow_layout(const pi_velocity_net* n, int B, int H, char* base) {
  const size_t S = (size_t)H + 1;
  size_t off = 0;
  FlowWs w;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = pi::align_up(off + bytes, 256);
    return base ? base + at : nullptr;
  };
  w.h = reinterpret_cast<float*>(take(sizeof(float) * B * S * n->width));
  w.q = reinterpret_cast<__bf16*>(take(2 * B * S * n->Hq * n->d));
  w.k = reinterpret_cast<__bf16*>(take(2 * B * S * n->Hkv * n->d));
  w.v = reinterpret_cast<__bf16*>(take(2 * B * S * n->Hkv * n->d));
  w.o = reinterpret_cast<__bf16*>(take(2 * B * S * n->Hq * n->d));
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
                                      static_cast<const __bf16*>(n->w_in), n->b_in, n->w_time, t, w.h, H, A, W);
    pi_status st = pi::check_launch("embed_kernel");
    if (st != PI_OK) return st;
  }
  for (int layer = 0; layer < cache->layers; ++layer) {
    GemmArgs g{};
    g.a = w.h;
    g.amap = RowMap{M, 0, 0};
    g.w0 = static_cast<const __bf16*>(n->w_q);
    g.w1 = static_cast<const __bf16*>(n->w_k);
    g.w2 = static_cast<const __bf16*>(n->w_v);
    g.n1 = nq;
    g.n2 = nkv;
    g.M = M;
    g.N = nq + 2 * nkv;
    g.K = W;
    g.o0 = w.q;
    g.o1 = w.k;
    g.o2 = w.v;
    pi_status st = gemm<EPI_QKV, float, true>(g, s, "gemm_qkv");
    if (st != PI_OK) return st;
    st = pi_suffix_decode_step(cache, layer, w.q, w.k, w.v, suffix_ar, B, S, n->Hq, scale, w.o, w.dec, w.dec_bytes,
                               s);
    if (st != PI_OK) return st;
    GemmArgs go{};
    go.a = w.o;
    go.amap = RowMap{M, 0, 0};
    go.w0 = go.w1 = go.w2 = static_cast<const __bf16*>(n->w_o);
    go.n1 = W;
    go.n2 = 0;
    go.M = M;
    go.N = W;
    go.K = nq;
    go.out = w.h;
    go.omap = RowMap{M, 0, 0};
    st = gemm<EPI_RESID, __bf16, false>(go, s, "gemm_out_resid");
    if (st != PI_OK) return st;
  }
  GemmArgs gv{};
  gv.a = w.h;
  gv.amap = RowMap{H, S, 1};  // action tokens of sample b are h rows b*S + 1 ..
  gv.w0 = gv.w1 = gv.w2 = static_cast<const __bf16*>(n->w_out);
  gv.n1 = A;
  gv.n2 = 0;
  gv.M = B * H;
  gv.N = A;
  gv.K = W;
  gv.bias = n->b_out;
  gv.omap = RowMap{B * H, 0, 0};
  gv.dt = dt;
  if (EPI == EPI_EULER) {
    gv.out = x;
    return gemm<EPI_EULER, float, true>(gv, s, "gemm_velocity_euler");
  }
  gv.out = vel;
  return gemm<EPI_VEL, float, true>(gv, s, "gemm_velocity");
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
  return run_net<EPI_VEL>(net, cache, suffix_ar, state, const_cast<float*>(x), t, 0.f, vel, B, H, A, w,
                          static_cast<hipStream_t>(stream));
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
  for (int k = 0; k < num_steps; ++k) {
    const float t = (float)(1.0 + k * dt);
    st = run_net<EPI_EULER>(net, cache, suffix_ar, state, x, t, (float)dt, nullptr, B, H, A, w, s);
    if (st != PI_OK) return st;
  }
  return PI_OK;
}
