// One π0.5 joint transformer layer around the joint attention, gfx950.
//
// What is computed ("π0.5 vs MM-DiT joint attention", first section; "VLA 代码精读
// — OpenPI & StarVLA" §1.4, §2.7): two streams, the prefix (VLM) stream and the
// action expert, each with its own norm, fused QKV projection, output projection
// and FFN; their Q/K/V are concatenated along the tokens into one pool, one
// masked softmax runs over it (pi_joint_attn_prefill), and the output is split
// back.  Per stream, with n(h) = h / sqrt(mean(h^2) + 1e-6):
//   a = r(n(h) * gamma1)                      plain stream
//   a = r(n(h) * (1 + scale1) + shift1)        adaptive stream, [shift1 | scale1] = r(silu(c)) W_mod1^T
//   q | k | v = r(a W_qkv^T);  o = r(attention);  h += o W_o^T
//   b = the second norm of h (gamma2 or mod2);  h += r(gelu(b W_up^T)) W_down^T
// r() rounds to bf16 (the matrix cores take bf16 operands); h stays fp32.
//
// Kernels:
//   * gemm_nt_kernel: C = A W^T for row-major bf16 A [M, K] and W [N, K] with fp32
//     accumulation, on the matrix cores.  A workgroup owns a 256 (N) x 256 (M)
//     tile (256 x 128 for few rows) with 8 waves of 64 x 128 (64 x 64); K
//     advances 64 at a time through two (three) LDS stages filled by
//     direct-to-LDS buffer loads.  Each load instruction fetches 8 operand rows
//     x 128 bytes (whole cache lines) into a row-swizzled LDS image whose
//     fragment reads are free of bank conflicts, and every fragment read feeds
//     four (W) or eight (A) products.  Products are computed
//     transposed (A operand = W rows, B operand = A rows) so a lane ends with
//     four consecutive output columns of one row for the epilogue: bf16 store,
//     gelu, residual add into fp32, fp32 store, or the QKV scatter into the
//     joint pool.  A rows can be read through a row map (the joint pool's rows
//     of one stream).
//   * norm_kernel: one wave per row, the RMS norm with the per-channel scale or
//     the per-sample modulation, bf16 output.
//   * silu_kernel: the conditioning's silu, bf16.
#include "common.h"
#include "engine.h"

#include <math.h>

namespace {

using namespace pi_engine;

constexpr int GN = 256, GK = 64;                // workgroup tile N and k step (the M tile is a parameter)
constexpr int GW = 8;                           // waves: 4 along N x 2 along M
constexpr int kRowBytes = GK * 2;               // one operand row's k step: a full 128-byte line
constexpr int kFragBytes = 16 * kRowBytes;      // 16 rows of the LDS image
constexpr int kGroupM = 4;                      // m tiles per group of the tile order
template <int GM>
struct GTile {
  static constexpr int StageBytes = (GN + GM) * kRowBytes;        // 64, 48 or 40 KB (GM 256, 128, 64)
  static constexpr int Stages = GM == 256 ? 2 : 3;                // 128 or 144 KB of LDS
  static constexpr int WLoads = GN / 8 / GW;                      // 1 KB (8-row) loads per wave and step: W
  static constexpr int ALoads = GM / 8 / GW;                      //                                        A
  static constexpr int Loads = WLoads + ALoads;
  static constexpr int MI = GM / 32;                              // A fragments per wave (its GM/2 rows)
  static_assert(Loads < 16, "vmcnt field");
};

// LDS image of an operand tile: row r (128 bytes, 8 chunks of 16) holds logical
// chunk x at physical chunk x ^ swz(r); with swz(r) = (r >> 1) & 7 the fragment
// read (16 rows x one chunk per 16-lane group) measures no bank conflicts.
__host__ __device__ constexpr int swz(int r) { return (r >> 1) & 7; }

enum { E_BF16 = 0, E_GELU = 1, E_RESID = 2, E_F32 = 3, E_QKV = 4 };

// Row map of the A operand: row m of the product reads row (m / T) * S + off + m % T
// of the A buffer (T = M, S = 0, off = 0 for a plain matrix).
struct RowMap {
  int T, S, off;
  __host__ __device__ int64_t operator()(int64_t m) const { return (m / T) * S + off + m % T; }
};

struct GemmParams {
  const __bf16* a;     // [rows, K]
  const __bf16* w;     // [N, K]
  int M, N, K;
  RowMap amap;
  void* out;           // E_BF16 / E_GELU: bf16 [M, N]; E_RESID: fp32 [M, N] (+=); E_F32: fp32 [M, N]
  // E_QKV: q [B, Ntot, nq], k / v [B, Ntot, nkv]; stream row m = (b, t) goes to joint row b*Ntot + tok_off + t
  __bf16 *q, *k, *v;
  int nq, nkv, T, Ntot, tok_off;
  int n_mt, n_nt;      // tile counts
  float* split_ws;     // few-row split-contraction partials (kSplitWsBytes), or null: no split
  int splits;
  float* tsplit_ws;    // tiled split-contraction partials (kTiledSplitBytes), or null: no split
  int tsplit;
};

__device__ __forceinline__ float gelu_exact(float x) { return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f)); }

template <int EPI>
__device__ __forceinline__ void gemm_store(const GemmParams& p, int64_t m, int n, const f32x4& acc) {
  if constexpr (EPI == E_RESID) {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + m * p.N + n);
    *dst = *dst + acc;
  } else if constexpr (EPI == E_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + m * p.N + n) = acc;
  } else {
    bf16x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = f2bf(EPI == E_GELU ? gelu_exact(acc[i]) : acc[i]);
    __bf16* dst;
    if constexpr (EPI == E_QKV) {
      const int64_t row = (m / p.T) * p.Ntot + p.tok_off + m % p.T;
      if (n < p.nq) dst = p.q + row * p.nq + n;
      else if (n < p.nq + p.nkv) dst = p.k + row * p.nkv + (n - p.nq);
      else dst = p.v + row * p.nkv + (n - p.nq - p.nkv);
    } else {
      dst = static_cast<__bf16*>(p.out) + m * p.N + n;
    }
    *reinterpret_cast<bf16x4*>(dst) = x;
  }
}

// vmcnt <= n for n in {0, L} (L loads per wave and step); expcnt and lgkmcnt
// left at their maxima
template <int L>
__device__ __forceinline__ void wait_vmem_le(int n) {
  if (n >= L) __builtin_amdgcn_s_waitcnt(0x0F70 | L);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier without the memory fence __syncthreads() carries: that
// fence waits for every outstanding load of the wave (vmcnt 0), which would
// drain the loads of the steps ahead.  Here each wave has waited for exactly its
// own loads of the current step, and the previous stage's LDS reads have all
// been consumed by products before a wave arrives, so the bare barrier (with
// compiler-level memory ordering around it) is enough.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int EPI, int GM>
__global__ void __launch_bounds__(GW * 64) gemm_nt_kernel(GemmParams p) {
  using G = GTile<GM>;
  constexpr int NS = G::Stages;
  __shared__ __attribute__((aligned(16))) char smem[NS * G::StageBytes];
  // XCD-aware tile order: the workgroups of one XCD take a contiguous run of
  // tiles, and within it groups of kGroupM m tiles x all n tiles, m fastest, so
  // the ~32 workgroups an XCD runs at once cover 4 m tiles x 8 n tiles and share
  // both operands' k windows in that XCD's L2
  const int total = p.n_mt * p.n_nt;
  const int chunk = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= chunk || lin >= total) return;
  const int gsize = kGroupM * p.n_nt;
  const int first_m = (lin / gsize) * kGroupM;
  const int gm = min(p.n_mt - first_m, kGroupM);
  const int mt = first_m + (lin % gsize) % gm, nt = (lin % gsize) / gm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wn = wave & 3, wm = wave >> 2;
  // split contraction (blockIdx.y of p.tsplit): this workgroup's k steps
  const int nk_all = p.K / GK;
  const int per = (nk_all + p.tsplit - 1) / p.tsplit;
  const int kz0 = (int)blockIdx.y * per;
  const int nk = min(nk_all, kz0 + per) - kz0;
  // Loads: each instruction fetches 8 rows x 128 bytes (lane L: row L / 8,
  // physical chunk L % 8, so the source chunk is (L % 8) ^ swz(row)); this wave
  // takes W rows 8 (WLoads wave + j) .. and A rows 8 (ALoads wave + j) ..
  const i32x4 rw = make_rsrc(p.w + (int64_t)nt * GN * p.K + (int64_t)kz0 * GK);
  const i32x4 ra = make_rsrc(p.a + (int64_t)kz0 * GK);
  const uint32_t kb = (uint32_t)p.K * 2u;
  uint32_t ow[G::WLoads], oa[G::ALoads];
#pragma unroll
  for (int j = 0; j < G::WLoads; ++j) {
    const int r = 8 * (G::WLoads * wave + j) + (lane >> 3);
    ow[j] = (uint32_t)r * kb + 16u * (uint32_t)((lane & 7) ^ swz(r));
  }
#pragma unroll
  for (int j = 0; j < G::ALoads; ++j) {
    const int r = 8 * (G::ALoads * wave + j) + (lane >> 3);
    const int64_t am = (int64_t)mt * GM + r;
    oa[j] = am < p.M ? (uint32_t)(p.amap(am) * p.K * 2 + 16 * ((lane & 7) ^ swz(r))) : kOOB;
  }
  auto issue = [&](int i) {
    char* st = smem + (i % NS) * G::StageBytes;
    const int so = __builtin_amdgcn_readfirstlane(i * GK * 2);
#pragma unroll
    for (int j = 0; j < G::WLoads; ++j)
      pi_buffer_load_lds(rw, lds_u32(st + 8 * (G::WLoads * wave + j) * kRowBytes), 16, (int)ow[j], so, 0, 0);
#pragma unroll
    for (int j = 0; j < G::ALoads; ++j)
      pi_buffer_load_lds(ra, lds_u32(st + (GN + 8 * (G::ALoads * wave + j)) * kRowBytes), 16, (int)oa[j], so, 0,
                         0);
  };
  // fragment reads: lane (c, g) reads row 16 f + c, logical chunk 4 kk + g; the
  // swizzle term of row 16 f + c is swz(c) for every f
  uint32_t lo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) lo[kk] = (uint32_t)(c * kRowBytes + 16 * ((4 * kk + g) ^ swz(c)));
  f32x4 acc[4][G::MI];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < G::MI; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < NS - 1 && j < nk; ++j) issue(j);
  for (int i = 0; i < nk; ++i) {
    wait_vmem_le<G::Loads>(G::Loads * min(nk - 1 - i, NS - 2));   // this wave's loads of step i have landed
    step_barrier();                          // everyone's; and every wave is done with step i - 1
    if (i + NS - 1 < nk) issue(i + NS - 1);  // into the stage of step i - 1
    const char* st = smem + (i % NS) * G::StageBytes;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 wf[4], af[G::MI];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wf[j] = *reinterpret_cast<const bf16x8*>(st + (4 * wn + j) * kFragBytes + lo[kk]);
#pragma unroll
      for (int j = 0; j < G::MI; ++j)
        af[j] = *reinterpret_cast<const bf16x8*>(st + GN * kRowBytes + (G::MI * wm + j) * kFragBytes + lo[kk]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < G::MI; ++b) acc[a][b] = mfma16x16x32(wf[a], af[b], acc[a][b]);
    }
  }
  // acc[a][b][i] = C[m = mt*GM + (GM/2) wm + 16 b + c][n = nt*256 + 64 wn + 16 a + 4 g + i]
#pragma unroll
  for (int b = 0; b < G::MI; ++b) {
    const int64_t m = (int64_t)mt * GM + (GM / 2) * wm + 16 * b + c;
    if (m >= p.M) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int n = nt * GN + 64 * wn + 16 * a + 4 * g;
      if (p.tsplit > 1)
        *reinterpret_cast<f32x4*>(p.tsplit_ws + ((int64_t)blockIdx.y * p.M + m) * p.N + n) = acc[a][b];
      else
        gemm_store<EPI>(p, m, n, acc[a][b]);
    }
  }
}

// Sum of the tiled split partials (in split order) through the epilogue; one
// thread per four columns of a row.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_tsplit_reduce_kernel(GemmParams p) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t quads = (int64_t)p.M * (p.N / 4);
  if (q >= quads) return;
  const int64_t m = q / (p.N / 4);
  const int n = (int)(q % (p.N / 4)) * 4;
  const int64_t plane = (int64_t)p.M * p.N;
  f32x4 r = *reinterpret_cast<const f32x4*>(p.tsplit_ws + m * p.N + n);
  for (int z = 1; z < p.tsplit; ++z) r += *reinterpret_cast<const f32x4*>(p.tsplit_ws + z * plane + m * p.N + n);
  gemm_store<EPI>(p, m, n, r);
}

// RMS norm of one fp32 row of width W (a multiple of 256, at most 4096) per wave:
// a = r(n(h) * gamma) (gamma != null) or r(n(h) * (1 + scale) + shift) with
// [shift | scale] = mod[b] (fp32 [B, 2W], b = row / T).
__global__ void __launch_bounds__(256)
norm_kernel(const float* __restrict__ h, __bf16* __restrict__ a, int64_t rows, int W, const float* __restrict__ gamma,
            const float* __restrict__ mod, int T) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;   // whole waves leave together
  const f32x4* src = reinterpret_cast<const f32x4*>(h + row * W);
  const int nv = W / 256;    // f32x4 per lane
  f32x4 x[16];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nv) {
      x[j] = src[j * 64 + lane];
      ss += x[j][0] * x[j][0] + x[j][1] * x[j][1] + x[j][2] * x[j][2] + x[j][3] * x[j][3];
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss / (float)W + 1e-6f);
  const float* shift = mod != nullptr ? mod + (row / T) * 2 * W : nullptr;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nv) {
      const int col = (j * 64 + lane) * 4;
      bf16x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float n = x[j][i] * inv;
        y[i] = f2bf(gamma != nullptr ? n * gamma[col + i] : n * (1.0f + shift[W + col + i]) + shift[col + i]);
      }
      *reinterpret_cast<bf16x4*>(a + row * W + col) = y;
    }
  }
}

__global__ void silu_kernel(const float* __restrict__ c, __bf16* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = c[i];
  y[i] = f2bf(x / (1.0f + expf(-x)));
}

// C = A W^T for few rows (M <= kSmallM): a workgroup owns 16 output columns of up
// to 64 rows and its 16 waves split the contraction, each over a contiguous range
// of 32-wide k steps, four steps of fragment loads in flight (16 bytes per lane
// straight from the row-major operands); the partial tiles are summed through
// LDS and the sum goes through the same epilogues as the tiled kernel.  With few
// rows the tiled kernel would have a handful of workgroups each walking all of K.
// With few column tiles the contraction is also split across workgroups
// (blockIdx.z): each stores its 64 x 16 partial and gemm_split_reduce_kernel sums
// them in split order (deterministic) through the epilogue.
constexpr int kSmallM = 256, kSmallWaves = 16, kSmallKB = 4;
constexpr int kMaxSplitTiles = 512;                              // splits x tiles
constexpr size_t kSplitWsBytes = (size_t)kMaxSplitTiles * 64 * 16 * 4;
constexpr size_t kTiledSplitBytes = (size_t)32 << 20;              // tiled split partials (M x N x splits fp32)

// MF: 16-row fragments per workgroup (4: 64-row tiles, with the optional split of
// the contraction; 1: 16-row tiles, no split, eight k steps of loads in flight).
template <int EPI, int MF>
__global__ void __launch_bounds__(kSmallWaves * 64) gemm_small_kernel(GemmParams p) {
  constexpr int KB = MF == 1 ? 2 * kSmallKB : kSmallKB;
  __shared__ float part[kSmallWaves][16 * MF * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * MF;
  const int ks_all = p.K / 32;
  const int kz = (ks_all + p.splits - 1) / p.splits;            // this split's k steps
  const int kz_lo = blockIdx.z * kz, ks = min(ks_all, kz_lo + kz) - kz_lo;
  const int per = (ks + kSmallWaves - 1) / kSmallWaves;
  const int k_lo = kz_lo + wave * per, k_hi = kz_lo + min(ks, wave * per + per);
  // this lane's operand rows: W row n0 + c; A rows m0 + 16 j + c (through the row map), or none
  const __bf16* wrow = p.w + (int64_t)(n0 + c) * p.K + 8 * g;
  const __bf16* arow[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    const int64_t m = m0 + 16 * j + c;
    arow[j] = m < p.M ? p.a + p.amap(m) * p.K + 8 * g : nullptr;
  }
  f32x4 acc[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = k_lo; k0 < k_hi; k0 += KB) {
    bf16x8 wf[KB], af[KB][MF];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const bool live = k0 + u < k_hi;     // uniform over the wave
      wf[u] = live ? *reinterpret_cast<const bf16x8*>(wrow + 32 * (k0 + u)) : bf16x8{};
#pragma unroll
      for (int j = 0; j < MF; ++j)
        af[u][j] = (live && arow[j]) ? *reinterpret_cast<const bf16x8*>(arow[j] + 32 * (k0 + u)) : bf16x8{};
    }
    __builtin_amdgcn_sched_barrier(0);     // the batch's loads all go out before the first wait
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int j = 0; j < MF; ++j) acc[j] = mfma16x16x32(wf[u], af[u][j], acc[j]);
  }
  // acc[j][i] = C[m0 + 16 j + c][n0 + 4 g + i]
#pragma unroll
  for (int j = 0; j < MF; ++j)
    *reinterpret_cast<f32x4*>(&part[wave][(16 * j + c) * 16 + 4 * g]) = acc[j];
  __syncthreads();
  if (threadIdx.x < 64 * MF) {
    const int ml = threadIdx.x >> 2, nl = 4 * (threadIdx.x & 3);
    const int64_t m = m0 + ml;
    f32x4 r = *reinterpret_cast<const f32x4*>(&part[0][ml * 16 + nl]);
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) r += *reinterpret_cast<const f32x4*>(&part[w][ml * 16 + nl]);
    if (MF == 4 && p.splits > 1) {
      const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
      const int64_t at = (blockIdx.z * (int64_t)gridDim.x * gridDim.y + tile) * 1024 + ml * 16 + nl;
      *reinterpret_cast<f32x4*>(p.split_ws + at) = r;
    } else if (m < p.M) {
      gemm_store<EPI>(p, m, n0 + nl, r);
    }
  }
}

// Sum of the split partials (in split order) through the epilogue; grid as the
// split kernel's x, y; 256 threads, each four columns of one row.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_split_reduce_kernel(GemmParams p) {
  const int ml = threadIdx.x >> 2, nl = 4 * (threadIdx.x & 3);
  const int64_t m = (int64_t)blockIdx.y * 64 + ml;
  if (m >= p.M) return;
  const int64_t tiles = (int64_t)gridDim.x * gridDim.y;
  const int64_t at = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 1024 + ml * 16 + nl;
  f32x4 r = *reinterpret_cast<const f32x4*>(p.split_ws + at);
  for (int z = 1; z < p.splits; ++z) r += *reinterpret_cast<const f32x4*>(p.split_ws + z * tiles * 1024 + at);
  gemm_store<EPI>(p, m, blockIdx.x * 16 + nl, r);
}

// 256 x 256 tiles once the rows alone give a few hundred workgroups, else 256 x 128;
// the split-contraction kernel for few rows.  With few rows and few column tiles
// (the output projection and the FFN down product back to the width) 16-row
// tiles fill the chip instead of a split contraction, so no reduce kernel follows.
template <int EPI>
pi_status launch_gemm(GemmParams p, hipStream_t s) {
  if (p.M <= kSmallM && (p.N / 16) * ((p.M + 63) / 64) < 128) {
    p.splits = 1;
    const dim3 grid((unsigned)(p.N / 16), (unsigned)((p.M + 15) / 16), 1);
    gemm_small_kernel<EPI, 1><<<grid, kSmallWaves * 64, 0, s>>>(p);
    return pi::check_launch("gemm_small_kernel");
  }
  if (p.M <= kSmallM) {
    // split the contraction across workgroups when the column tiles alone leave
    // most of the chip idle and every split keeps at least 16 k steps of 32
    const int tiles = (p.N / 16) * ((p.M + 63) / 64);
    int splits = 1;
    if (p.split_ws != nullptr)
      while (splits < 8 && tiles * splits * 2 <= 256 && p.K / 32 >= 16 * splits * 2 &&
             tiles * splits * 2 <= kMaxSplitTiles)
        splits *= 2;
    p.splits = splits;
    const dim3 grid((unsigned)(p.N / 16), (unsigned)((p.M + 63) / 64), (unsigned)splits);
    gemm_small_kernel<EPI, 4><<<grid, kSmallWaves * 64, 0, s>>>(p);
    pi_status st = pi::check_launch("gemm_small_kernel");
    if (st != PI_OK || splits == 1) return st;
    gemm_split_reduce_kernel<EPI><<<dim3(grid.x, grid.y), 256, 0, s>>>(p);
    return pi::check_launch("gemm_split_reduce_kernel");
  }
  // the M tile: 256 once the rows alone give a few hundred workgroups, else 128, or
  // 64 when 128-row tiles would leave most of the 256 compute units idle
  const int gm = p.M >= 8192 ? 256 : ((p.M + 127) / 128 * (p.N / GN) >= 256 ? 128 : 64);
  p.n_mt = (p.M + gm - 1) / gm;
  p.n_nt = p.N / GN;
  const int total = p.n_mt * p.n_nt;
  const int grid = (total + 7) / 8 * 8;
  // split the contraction when the tiles leave more than half the compute units
  // idle and each split keeps at least 32 k steps of 64 (measured: an 848-row FFN
  // down product of 112 tiles gains 4-way; a 3200-row one of 200 tiles loses 2-way)
  int ts = 1;
  if (p.tsplit_ws != nullptr && total < 128)
    while (ts < 4 && total * ts * 2 <= 512 && p.K / GK >= 32 * ts * 2 &&
           (size_t)p.M * p.N * ts * 2 * 4 <= kTiledSplitBytes)
      ts *= 2;
  p.tsplit = ts;
  const dim3 g3((unsigned)grid, (unsigned)ts);
  if (gm == 256) gemm_nt_kernel<EPI, 256><<<g3, GW * 64, 0, s>>>(p);
  else if (gm == 128) gemm_nt_kernel<EPI, 128><<<g3, GW * 64, 0, s>>>(p);
  else gemm_nt_kernel<EPI, 64><<<g3, GW * 64, 0, s>>>(p);
  pi_status st = pi::check_launch("gemm_nt_kernel");
  if (st != PI_OK || ts == 1) return st;
  const int64_t quads = (int64_t)p.M * (p.N / 4);
  gemm_tsplit_reduce_kernel<EPI><<<(unsigned)((quads + 255) / 256), 256, 0, s>>>(p);
  return pi::check_launch("gemm_tsplit_reduce_kernel");
}

constexpr int LHq = 8, LHkv = 1, LD = 256, LQKV = (LHq + 2 * LHkv) * LD;

struct LayerWs {
  __bf16 *a, *q, *k, *v, *o, *u, *sc;
  float *mod, *gsplit, *tsplit;
  void* attn;
  size_t attn_bytes, total;
};

// attn_bytes: the attention's own workspace (the joint prefill's or the cached decode's)
LayerWs layer_ws(int B, int Np, int Ne, int Wp, int We, int Fp, int Fe, size_t attn_bytes, char* base) {
  const int64_t N = (int64_t)Np + Ne;
  const int64_t rows_max = (int64_t)B * (Np > Ne ? Np : Ne);
  const int64_t wmax = Wp > We ? Wp : We;
  const int64_t fmax = (int64_t)B * Np * Fp > (int64_t)B * Ne * Fe ? (int64_t)B * Np * Fp : (int64_t)B * Ne * Fe;
  LayerWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = pi::align_up(off + bytes, 256);
    return base ? base + at : nullptr;
  };
  w.a = reinterpret_cast<__bf16*>(take(rows_max * wmax * 2));
  w.q = reinterpret_cast<__bf16*>(take(B * N * LHq * LD * 2));
  w.k = reinterpret_cast<__bf16*>(take(B * N * LHkv * LD * 2));
  w.v = reinterpret_cast<__bf16*>(take(B * N * LHkv * LD * 2));
  w.o = reinterpret_cast<__bf16*>(take(B * N * LHq * LD * 2));
  w.u = reinterpret_cast<__bf16*>(take(fmax * 2));
  w.sc = reinterpret_cast<__bf16*>(take((size_t)B * wmax * 2));
  w.mod = reinterpret_cast<float*>(take((size_t)2 * B * 2 * wmax * 4));
  w.gsplit = reinterpret_cast<float*>(take(kSplitWsBytes));
  w.tsplit = rows_max > kSmallM ? reinterpret_cast<float*>(take(kTiledSplitBytes)) : nullptr;
  w.attn_bytes = attn_bytes;
  w.attn = take(w.attn_bytes);
  w.total = off;
  return w;
}

bool stream_ok(const pi_layer_stream* s) {
  if (s == nullptr || !s->w_qkv || !s->w_o || !s->w_up || !s->w_down) return false;
  if (s->width < 256 || s->width > 4096 || s->width % 256 || s->ffn < 256 || s->ffn > 65536 || s->ffn % 256)
    return false;
  const bool plain = s->norm1 && s->norm2, ada = s->mod1 && s->mod2;
  return plain != ada;
}

// One stream's half of the layer before the attention: norm 1 and the QKV scatter.
// mod_T: rows per modulation row (T: one per sample; B * T: one shared by all)
pi_status stream_qkv(const pi_layer_stream* sw, const float* h, int B, int T, int Ntot, int tok_off,
                     const float* mod, const LayerWs& w, hipStream_t s, int mod_T = 0) {
  const int64_t rows = (int64_t)B * T;
  norm_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(h, w.a, rows, sw->width, sw->norm1, sw->norm1 ? nullptr : mod,
                                                          mod_T ? mod_T : T);
  pi_status st = pi::check_launch("norm_kernel");
  if (st != PI_OK) return st;
  GemmParams p{};
  p.a = w.a;
  p.w = static_cast<const __bf16*>(sw->w_qkv);
  p.M = (int)rows;
  p.N = LQKV;
  p.K = sw->width;
  p.amap = RowMap{(int)rows, 0, 0};
  p.q = w.q;
  p.k = w.k;
  p.v = w.v;
  p.nq = LHq * LD;
  p.nkv = LHkv * LD;
  p.T = T;
  p.Ntot = Ntot;
  p.tok_off = tok_off;
  p.split_ws = w.gsplit;
  p.tsplit_ws = w.tsplit;
  return launch_gemm<E_QKV>(p, s);
}

// One stream's half after the attention: output projection, norm 2, FFN.
pi_status stream_out(const pi_layer_stream* sw, float* h, int B, int T, int Ntot, int tok_off, const float* mod,
                     const LayerWs& w, hipStream_t s, int mod_T = 0) {
  const int64_t rows = (int64_t)B * T;
  GemmParams p{};
  p.a = w.o;
  p.w = static_cast<const __bf16*>(sw->w_o);
  p.M = (int)rows;
  p.N = sw->width;
  p.K = LHq * LD;
  p.amap = RowMap{T, Ntot, tok_off};
  p.out = h;
  p.split_ws = w.gsplit;
  p.tsplit_ws = w.tsplit;
  pi_status st = launch_gemm<E_RESID>(p, s);
  if (st != PI_OK) return st;
  norm_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(h, w.a, rows, sw->width, sw->norm2,
                                                          sw->norm2 ? nullptr : mod, mod_T ? mod_T : T);
  if ((st = pi::check_launch("norm_kernel")) != PI_OK) return st;
  GemmParams up{};
  up.a = w.a;
  up.w = static_cast<const __bf16*>(sw->w_up);
  up.M = (int)rows;
  up.N = sw->ffn;
  up.K = sw->width;
  up.amap = RowMap{(int)rows, 0, 0};
  up.out = w.u;
  up.split_ws = w.gsplit;
  up.tsplit_ws = w.tsplit;
  if ((st = launch_gemm<E_GELU>(up, s)) != PI_OK) return st;
  GemmParams dn{};
  dn.a = w.u;
  dn.w = static_cast<const __bf16*>(sw->w_down);
  dn.M = (int)rows;
  dn.N = sw->width;
  dn.K = sw->ffn;
  dn.amap = RowMap{(int)rows, 0, 0};
  dn.out = h;
  dn.split_ws = w.gsplit;
  dn.tsplit_ws = w.tsplit;
  return launch_gemm<E_RESID>(dn, s);
}

// The two modulations [shift | scale] (fp32 [B, 2W] each) of an adaptive stream.
pi_status stream_mod(const pi_layer_stream* sw, const float* cond, int B, const LayerWs& w, hipStream_t s) {
  const int64_t n = (int64_t)B * sw->width;
  silu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(cond, w.sc, n);
  pi_status st = pi::check_launch("silu_kernel");
  if (st != PI_OK) return st;
  for (int j = 0; j < 2; ++j) {
    GemmParams p{};
    p.a = w.sc;
    p.w = static_cast<const __bf16*>(j == 0 ? sw->mod1 : sw->mod2);
    p.M = B;
    p.N = 2 * sw->width;
    p.K = sw->width;
    p.amap = RowMap{B, 0, 0};
    p.out = w.mod + (size_t)j * B * 2 * sw->width;
    p.split_ws = w.gsplit;
    if ((st = launch_gemm<E_F32>(p, s)) != PI_OK) return st;
  }
  return PI_OK;
}

// The expert stream's layer in the cached form: norm 1, QKV, the suffix decode
// against cache layer `layer`, output projection, norm 2 and FFN (h updated in place).
// shared_mods: the two modulations ([2W] fp32 each, at shared_mods[0] and [1]) shared
// by every sample, when the caller has them already; else null (computed here from
// cond [B, W], one per sample).
pi_status expert_layer(const pi_layer_stream* sw, const pi_kv_cache* cache, int layer, float* h, const float* cond,
                       const uint8_t* suffix_ar, int B, int S, float scale, const LayerWs& w, hipStream_t s,
                       const float* const* shared_mods = nullptr) {
  pi_status st = PI_OK;
  if (sw->mod1 && !shared_mods && (st = stream_mod(sw, cond, B, w, s)) != PI_OK) return st;
  const float* mod1 = shared_mods ? shared_mods[0] : w.mod;
  const float* mod2 = shared_mods ? shared_mods[1] : w.mod + (size_t)B * 2 * sw->width;
  const int mod_T = shared_mods ? B * S : S;
  if ((st = stream_qkv(sw, h, B, S, S, 0, mod1, w, s, mod_T)) != PI_OK) return st;
  st = pi_suffix_decode_step(cache, layer, w.q, w.k, w.v, suffix_ar, B, S, LHq, scale, 0.f, w.o, w.attn, w.attn_bytes,
                             s);
  if (st != PI_OK) return st;
  return stream_out(sw, h, B, S, S, 0, mod2, w, s, mod_T);
}

}  // namespace

extern "C" size_t pi_joint_layer_workspace_bytes(const pi_layer_stream* prefix, const pi_layer_stream* expert, int B,
                                                 int Np, int Ne) {
  if (!stream_ok(prefix) || !stream_ok(expert) || B < 1 || Np < 0 || Ne < 0 || Np + Ne < 1) return 0;
  return layer_ws(B, Np, Ne, prefix->width, expert->width, prefix->ffn, expert->ffn,
                  pi_prefill_workspace_bytes(B, Np + Ne, LHq, LHkv, LD), nullptr).total;
}

namespace {
pi_status joint_layer(const pi_layer_stream* prefix, const pi_layer_stream* expert, float* h_p, float* h_e,
                      const float* cond, int B, int Np, int Ne, float scale, const pi_mask* mask,
                      const pi_kv_cache* cache, int layer, void* workspace, size_t workspace_bytes,
                      pi_stream stream);
}  // namespace

extern "C" pi_status pi_joint_layer_forward(const pi_layer_stream* prefix, const pi_layer_stream* expert, float* h_p,
                                            float* h_e, const float* cond, int B, int Np, int Ne, float scale,
                                            const pi_mask* mask, void* workspace, size_t workspace_bytes,
                                            pi_stream stream) {
  return joint_layer(prefix, expert, h_p, h_e, cond, B, Np, Ne, scale, mask, nullptr, 0, workspace, workspace_bytes,
                     stream);
}

extern "C" size_t pi_prefix_layer_workspace_bytes(const pi_layer_stream* prefix, int B, int Np) {
  return pi_joint_layer_workspace_bytes(prefix, prefix, B, Np, 0);
}

extern "C" pi_status pi_prefix_layer_forward(const pi_layer_stream* prefix, float* h_p, const float* cond, int B,
                                             int Np, float scale, const pi_mask* mask, const pi_kv_cache* cache,
                                             int layer, void* workspace, size_t workspace_bytes, pi_stream stream) {
  PI_REQUIRE(cache != nullptr, PI_ERR_INVALID_ARG, "pi_prefix_layer_forward: null cache");
  PI_REQUIRE(cache->len == Np, PI_ERR_INVALID_ARG,
             "pi_prefix_layer_forward: the cache must hold exactly the Np = %d prefix tokens (len %d)", Np,
             cache->len);
  // the whole cache contract here, so that nothing is launched for a call the attention would reject
  PI_REQUIRE(cache->k && cache->v && cache->B == B && cache->Hkv == LHkv && cache->d == LD && layer >= 0 &&
                 layer < cache->layers && Np >= 1 && Np <= cache->capacity,
             PI_ERR_INVALID_ARG, "pi_prefix_layer_forward: cache does not match (B=%d, layer %d of %d, %d slots)", B,
             layer, cache->layers, cache->capacity);
  return joint_layer(prefix, prefix, h_p, nullptr, cond, B, Np, 0, scale, mask, cache, layer, workspace,
                     workspace_bytes, stream);
}

namespace {
pi_status joint_layer(const pi_layer_stream* prefix, const pi_layer_stream* expert, float* h_p, float* h_e,
                      const float* cond, int B, int Np, int Ne, float scale, const pi_mask* mask,
                      const pi_kv_cache* cache, int layer, void* workspace, size_t workspace_bytes,
                      pi_stream stream) {
  PI_REQUIRE(stream_ok(prefix) && stream_ok(expert), PI_ERR_INVALID_ARG,
             "pi_joint_layer_forward: a stream needs w_qkv, w_o, w_up, w_down, a width and ffn that are multiples "
             "of 256 (width <= 4096), and either norm1 + norm2 or mod1 + mod2");
  PI_REQUIRE(B >= 1 && Np >= 0 && Ne >= 0 && Np + Ne >= 1, PI_ERR_INVALID_ARG, "pi_joint_layer_forward: B=%d Np=%d Ne=%d",
             B, Np, Ne);
  PI_REQUIRE((Np == 0 || h_p) && (Ne == 0 || h_e) && mask, PI_ERR_INVALID_ARG, "pi_joint_layer_forward: null pointer");
  PI_REQUIRE(pi::aligned16(h_p) && pi::aligned16(h_e), PI_ERR_INVALID_ARG,
             "pi_joint_layer_forward: h_p / h_e must be 16-byte aligned");
  const bool need_cond = (Np > 0 && prefix->mod1) || (Ne > 0 && expert->mod1);
  PI_REQUIRE(!need_cond || cond, PI_ERR_INVALID_ARG, "pi_joint_layer_forward: an adaptive norm needs cond");
  PI_REQUIRE(!(prefix->mod1 && expert->mod1), PI_ERR_UNSUPPORTED,
             "pi_joint_layer_forward: at most one stream may use the adaptive norm");
  const int N = Np + Ne;
  PI_REQUIRE(N <= kMaxTiles * TK, PI_ERR_UNSUPPORTED, "pi_joint_layer_forward: %d tokens exceed %d", N,
             kMaxTiles * TK);
  PI_REQUIRE(mask->B == B && mask->N == N, PI_ERR_INVALID_ARG,
             "pi_joint_layer_forward: mask built for B=%d N=%d, call has B=%d N=%d", mask->B, mask->N, B, N);
  PI_REQUIRE(scale > 0.f && isfinite(scale), PI_ERR_INVALID_ARG, "pi_joint_layer_forward: scale must be > 0");
  // 32-bit buffer offsets: every operand a GEMM reads stays below 2 GiB
  const int64_t rows = (int64_t)B * (Np > Ne ? Np : Ne);
  const int64_t big = (int64_t)B * N * LHq * LD * 2;
  const int64_t ub = rows * (prefix->ffn > expert->ffn ? prefix->ffn : expert->ffn) * 2;
  const int64_t ab = rows * (prefix->width > expert->width ? prefix->width : expert->width) * 2;
  PI_REQUIRE(big < 0x7FFF0000ll && ub < 0x7FFF0000ll && ab < 0x7FFF0000ll, PI_ERR_UNSUPPORTED,
             "pi_joint_layer_forward: an activation exceeds 2 GiB");
  const size_t attn_bytes = pi_prefill_workspace_bytes(B, N, LHq, LHkv, LD);
  const LayerWs need = layer_ws(B, Np, Ne, prefix->width, expert->width, prefix->ffn, expert->ffn, attn_bytes, nullptr);
  PI_REQUIRE(workspace && workspace_bytes >= need.total, PI_ERR_WORKSPACE,
             "pi_joint_layer_forward: needs %zu workspace bytes, got %zu", need.total, workspace_bytes);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_joint_layer_forward: workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LayerWs w = layer_ws(B, Np, Ne, prefix->width, expert->width, prefix->ffn, expert->ffn, attn_bytes,
                             static_cast<char*>(workspace));
  pi_status st = PI_OK;
  // modulations of the adaptive stream(s): mod1 at w.mod, mod2 after it
  // (only a stream with tokens needs its modulation; cond may be null otherwise)
  const pi_layer_stream* ada = (Ne > 0 && expert->mod1) ? expert : ((Np > 0 && prefix->mod1) ? prefix : nullptr);
  if (ada && (st = stream_mod(ada, cond, B, w, s)) != PI_OK) return st;
  const int wa = ada ? ada->width : 0;
  const float* mod1 = w.mod;
  const float* mod2 = w.mod + (size_t)B * 2 * wa;
  if (Np > 0 && (st = stream_qkv(prefix, h_p, B, Np, N, 0, mod1, w, s)) != PI_OK) return st;
  if (Ne > 0 && (st = stream_qkv(expert, h_e, B, Ne, N, Np, mod1, w, s)) != PI_OK) return st;
  st = pi_joint_attn_prefill(w.q, w.k, w.v, B, N, LHq, LHkv, LD, scale, 0.f, mask, w.o, nullptr, cache, layer,
                             w.attn, w.attn_bytes, stream);
  if (st != PI_OK) return st;
  if (Np > 0 && (st = stream_out(prefix, h_p, B, Np, N, 0, mod2, w, s)) != PI_OK) return st;
  if (Ne > 0 && (st = stream_out(expert, h_e, B, Ne, N, Np, mod2, w, s)) != PI_OK) return st;
  return PI_OK;
}
}  // namespace

extern "C" size_t pi_expert_layer_decode_workspace_bytes(const pi_layer_stream* expert, int B, int S, int len) {
  if (!stream_ok(expert) || B < 1 || S < 1 || len < 0) return 0;
  return layer_ws(B, 0, S, expert->width, expert->width, expert->ffn, expert->ffn,
                  pi_decode_workspace_bytes(B, S, LHq, len), nullptr).total;
}

extern "C" pi_status pi_expert_layer_decode(const pi_layer_stream* expert, const pi_kv_cache* cache, int layer,
                                            float* h_e, const float* cond, const uint8_t* suffix_ar, int B, int S,
                                            float scale, void* workspace, size_t workspace_bytes, pi_stream stream) {
  PI_REQUIRE(stream_ok(expert), PI_ERR_INVALID_ARG,
             "pi_expert_layer_decode: the stream needs w_qkv, w_o, w_up, w_down, a width and ffn that are multiples "
             "of 256 (width <= 4096), and either norm1 + norm2 or mod1 + mod2");
  PI_REQUIRE(cache && h_e && suffix_ar, PI_ERR_INVALID_ARG, "pi_expert_layer_decode: null pointer");
  PI_REQUIRE(B >= 1 && S >= 1 && cache->B == B && cache->Hkv == LHkv && cache->d == LD && layer >= 0 &&
                 layer < cache->layers,
             PI_ERR_INVALID_ARG, "pi_expert_layer_decode: cache / shape mismatch (B=%d S=%d layer %d)", B, S, layer);
  PI_REQUIRE(S <= 128 && cache->k && cache->v && cache->prefix_mask && cache->len >= 0 &&
                 cache->len <= cache->capacity,
             PI_ERR_INVALID_ARG, "pi_expert_layer_decode: S=%d (<= 128) or the cache (len %d of %d slots) is invalid",
             S, cache->len, cache->capacity);
  PI_REQUIRE((cache->len + TK - 1) / TK + (S + TK - 1) / TK <= kMaxTiles, PI_ERR_UNSUPPORTED,
             "pi_expert_layer_decode: cache length %d too long", cache->len);
  PI_REQUIRE(pi::aligned16(h_e), PI_ERR_INVALID_ARG, "pi_expert_layer_decode: h_e must be 16-byte aligned");
  PI_REQUIRE(!expert->mod1 || cond, PI_ERR_INVALID_ARG, "pi_expert_layer_decode: an adaptive norm needs cond");
  PI_REQUIRE(scale > 0.f && isfinite(scale), PI_ERR_INVALID_ARG, "pi_expert_layer_decode: scale must be > 0");
  PI_REQUIRE((int64_t)B * S * expert->ffn * 2 < 0x7FFF0000ll && (int64_t)B * S * LHq * LD * 2 < 0x7FFF0000ll,
             PI_ERR_UNSUPPORTED, "pi_expert_layer_decode: an activation exceeds 2 GiB");
  const size_t attn_bytes = pi_decode_workspace_bytes(B, S, LHq, cache->len);
  const LayerWs need = layer_ws(B, 0, S, expert->width, expert->width, expert->ffn, expert->ffn, attn_bytes, nullptr);
  PI_REQUIRE(workspace && workspace_bytes >= need.total, PI_ERR_WORKSPACE,
             "pi_expert_layer_decode: needs %zu workspace bytes, got %zu", need.total, workspace_bytes);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "pi_expert_layer_decode: workspace must be 256-byte aligned");
  const LayerWs w = layer_ws(B, 0, S, expert->width, expert->width, expert->ffn, expert->ffn, attn_bytes,
                             static_cast<char*>(workspace));
  return expert_layer(expert, cache, layer, h_e, cond, suffix_ar, B, S, scale, w, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// π0.5's action expert at its true shape driving the Euler sampler ("VLA 代码精读"
// §1.2, §1.4, §1.6):
//   c_k = r(silu(r(emb(t_k)) W_t1^T + b_t1)) W_t2^T + b_t2     (one row per step, every sample)
//   h = r(x) W_in^T + b_in;  h = expert_layer_l(h, c_k) for l < layers (cache layer l)
//   v = r(final adaptive norm of h) W_out^T + b_out;  x += dt v
// emb(t)[j] = sin(2 pi t / p_j), emb(t)[W/2 + j] = cos(2 pi t / p_j), with
// p_j = 4e-3 * 1000^(j / (W/2 - 1)).  The embedding, the MLP's activation and the
// final norm are readings of the pages.
// ---------------------------------------------------------------------------
namespace {

// Row k of the time embedding at t = t0 + k*dt (double precision, then bf16).
__global__ void time_embed_kernel(double t0, double dt, int n, int W, __bf16* __restrict__ emb) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int half = W / 2;
  if (i >= n * half) return;
  const int k = i / half, j = i % half;
  const double t = t0 + k * dt;
  const double period = 4e-3 * pow(1000.0, (double)j / (double)(half - 1));
  const double ang = 6.283185307179586 * t / period;
  emb[(int64_t)k * W + j] = f2bf((float)sin(ang));
  emb[(int64_t)k * W + half + j] = f2bf((float)cos(ang));
}

// in fp32 [n, W] + bias: act = 1: bf16 silu(.) into out_b [n, W]; act = 0: fp32
// into out_f, row k repeated `rep` times (rows k*rep .. k*rep + rep - 1).
__global__ void bias_act_kernel(const float* __restrict__ in, const float* __restrict__ bias, int n, int W, int act,
                                __bf16* __restrict__ out_b, float* __restrict__ out_f, int rep) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * W) return;
  const int k = (int)(i / W), j = (int)(i % W);
  const float y = in[i] + bias[j];
  if (act) {
    out_b[i] = f2bf(y / (1.0f + expf(-y)));
  } else {
    for (int r = 0; r < rep; ++r) out_f[((int64_t)k * rep + r) * W + j] = y;
  }
}

// h[m][n] = sum_a r(x[m][a]) w_in[n][a] + b_in[n]  (A <= 256; one row per block.y)
__global__ void __launch_bounds__(256)
action_embed_kernel(const float* __restrict__ x, const __bf16* __restrict__ w_in, const float* __restrict__ b_in,
                    float* __restrict__ h, int A, int W) {
  __shared__ float xs[256];
  const int64_t m = blockIdx.y;
  if (threadIdx.x < A) xs[threadIdx.x] = bf2f(f2bf(x[m * A + threadIdx.x]));
  __syncthreads();
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= W) return;
  const __bf16* wr = w_in + (int64_t)n * A;
  float acc = 0.f;
  for (int a = 0; a < A; ++a) acc += xs[a] * bf2f(wr[a]);
  h[m * W + n] = acc + b_in[n];
}

// dst [rows_pad, K] = src [rows, K] with zero rows after (one thread per 8 elements)
__global__ void pad_rows_kernel(const __bf16* __restrict__ src, __bf16* __restrict__ dst, int rows, int rows_pad,
                                int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int k8 = K / 8;
  if (i >= (int64_t)rows_pad * k8) return;
  const int r = (int)(i / k8), k = (int)(i % k8) * 8;
  *reinterpret_cast<bf16x8*>(dst + (int64_t)r * K + k) =
      r < rows ? *reinterpret_cast<const bf16x8*>(src + (int64_t)r * K + k) : bf16x8{};
}

// v = vel[m][a] + b_out[a] (vel fp32 [M, 256]); euler: x[m][a] += dt v, else out[m][a] = v
__global__ void velocity_out_kernel(const float* __restrict__ vel, const float* __restrict__ b_out,
                                    float* __restrict__ x, float* __restrict__ out, int64_t M, int A, float dt,
                                    int euler) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * A) return;
  const int64_t m = i / A;
  const int a = (int)(i % A);
  const float v = vel[m * 256 + a] + b_out[a];
  if (euler) x[i] += dt * v;
  else out[i] = v;
}

constexpr int kMaxSteps = 1000;

// The conditioning c is the same for every sample of a step, and so is every
// norm's modulation: mods holds all of a call's, computed once: for matrix i
// (layer l's norm j at i = 2 l + j, the final norm at i = 2 layers) and step k,
// [shift | scale] at mods + (i * steps + k) * 2W.
struct ExpertFlowWs {
  LayerWs layer;
  __bf16 *emb, *u, *wout, *sc;
  float *t1, *cond, *h, *vel, *mods;
  size_t total;
};

ExpertFlowWs expert_flow_ws(int W, int F, int L, int B, int H, int n_steps, size_t attn_bytes, char* base) {
  ExpertFlowWs w{};
  w.layer = layer_ws(B, 0, H, W, W, F, F, attn_bytes, base);
  size_t off = w.layer.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = pi::align_up(off + bytes, 256);
    return base ? base + at : nullptr;
  };
  const int64_t M = (int64_t)B * H;
  w.emb = reinterpret_cast<__bf16*>(take((size_t)n_steps * W * 2));
  w.u = reinterpret_cast<__bf16*>(take((size_t)n_steps * W * 2));
  w.wout = reinterpret_cast<__bf16*>(take((size_t)256 * W * 2));
  w.t1 = reinterpret_cast<float*>(take((size_t)n_steps * W * 4));
  w.cond = reinterpret_cast<float*>(take((size_t)n_steps * W * 4));
  w.h = reinterpret_cast<float*>(take((size_t)M * W * 4));
  w.vel = reinterpret_cast<float*>(take((size_t)M * 256 * 4));
  w.sc = reinterpret_cast<__bf16*>(take((size_t)n_steps * W * 2));
  w.mods = reinterpret_cast<float*>(take((size_t)(2 * L + 1) * n_steps * 2 * W * 4));
  w.total = off;
  return w;
}

int expert_ffn_max(const pi_expert_net* n) {
  int f = 256;
  for (int l = 0; l < n->layers; ++l) f = n->layer[l].ffn > f ? n->layer[l].ffn : f;
  return f;
}

bool expert_net_ok(const pi_expert_net* n) {
  if (n == nullptr || n->layer == nullptr || n->layers < 1) return false;
  if (n->width < 256 || n->width > 4096 || n->width % 256 || n->action_dim < 1 || n->action_dim > 256) return false;
  if (!n->w_in || !n->b_in || !n->w_t1 || !n->b_t1 || !n->w_t2 || !n->b_t2 || !n->mod_f || !n->w_out || !n->b_out)
    return false;
  // matrices read 16 bytes per lane (the GEMMs' buffer loads, the out-projection's padding copy)
  if (!pi::aligned16(n->w_t1) || !pi::aligned16(n->w_t2) || !pi::aligned16(n->mod_f) || !pi::aligned16(n->w_out))
    return false;
  for (int l = 0; l < n->layers; ++l) {
    const pi_layer_stream& sl = n->layer[l];
    if (!stream_ok(&sl) || !sl.mod1 || sl.width != n->width) return false;
    if (!pi::aligned16(sl.w_qkv) || !pi::aligned16(sl.w_o) || !pi::aligned16(sl.w_up) || !pi::aligned16(sl.w_down) ||
        !pi::aligned16(sl.mod1) || !pi::aligned16(sl.mod2))
      return false;
  }
  return true;
}

// Conditioning rows c_k for t_k = t0 + k*dt, k < steps, and from them every norm's
// modulation of every step.
pi_status expert_cond(const pi_expert_net* n, double t0, double dt, int steps, const ExpertFlowWs& w,
                      hipStream_t s) {
  const int W = n->width;
  const int half = W / 2;
  time_embed_kernel<<<(unsigned)((steps * half + 255) / 256), 256, 0, s>>>(t0, dt, steps, W, w.emb);
  pi_status st = pi::check_launch("time_embed_kernel");
  if (st != PI_OK) return st;
  for (int j = 0; j < 2; ++j) {
    GemmParams p{};
    p.a = j == 0 ? w.emb : w.u;
    p.w = static_cast<const __bf16*>(j == 0 ? n->w_t1 : n->w_t2);
    p.M = steps;
    p.N = W;
    p.K = W;
    p.amap = RowMap{steps, 0, 0};
    p.out = w.t1;
    p.split_ws = w.layer.gsplit;
    if ((st = launch_gemm<E_F32>(p, s)) != PI_OK) return st;
    const int64_t cnt = (int64_t)steps * W;
    bias_act_kernel<<<(unsigned)((cnt + 255) / 256), 256, 0, s>>>(w.t1, j == 0 ? n->b_t1 : n->b_t2, steps, W,
                                                                 j == 0 ? 1 : 0, w.u, w.cond, 1);
    if ((st = pi::check_launch("bias_act_kernel")) != PI_OK) return st;
  }
  // every norm's [shift | scale] = r(silu(c)) mod^T for all steps at once
  const int64_t rows = steps;
  silu_kernel<<<(unsigned)((rows * W + 255) / 256), 256, 0, s>>>(w.cond, w.sc, rows * W);
  if ((st = pi::check_launch("silu_kernel")) != PI_OK) return st;
  for (int i = 0; i <= 2 * n->layers; ++i) {
    GemmParams p{};
    p.a = w.sc;
    p.w = static_cast<const __bf16*>(i == 2 * n->layers ? n->mod_f
                                     : (i % 2 == 0 ? n->layer[i / 2].mod1 : n->layer[i / 2].mod2));
    p.M = (int)rows;
    p.N = 2 * W;
    p.K = W;
    p.amap = RowMap{(int)rows, 0, 0};
    p.out = w.mods + (size_t)i * rows * 2 * W;
    p.split_ws = w.layer.gsplit;
    if ((st = launch_gemm<E_F32>(p, s)) != PI_OK) return st;
  }
  return PI_OK;
}

// One velocity evaluation with conditioning rows `cond` [B, W]: into `vel` (euler
// = false) or fused x += dt v.
pi_status expert_velocity(const pi_expert_net* n, const pi_kv_cache* cache, const uint8_t* suffix_ar, float* x,
                          int k, int steps, float* vel, float dt, bool euler, int B, int H, const ExpertFlowWs& w,
                          hipStream_t s) {
  const int W = n->width, A = n->action_dim;
  const int64_t M = (int64_t)B * H;
  action_embed_kernel<<<dim3((unsigned)((W + 255) / 256), (unsigned)M), 256, 0, s>>>(
      x, static_cast<const __bf16*>(n->w_in), n->b_in, w.h, A, W);
  pi_status st = pi::check_launch("action_embed_kernel");
  if (st != PI_OK) return st;
  const float scale = 1.0f / 16.0f;   // 1 / sqrt(head_dim 256)
  auto mod_at = [&](int i) { return w.mods + ((size_t)i * steps + k) * 2 * W; };
  for (int l = 0; l < n->layers; ++l) {
    const float* mods[2] = {mod_at(2 * l), mod_at(2 * l + 1)};
    if ((st = expert_layer(&n->layer[l], cache, l, w.h, nullptr, suffix_ar, B, H, scale, w.layer, s, mods)) != PI_OK)
      return st;
  }
  norm_kernel<<<(unsigned)((M + 3) / 4), 256, 0, s>>>(w.h, w.layer.a, M, W, nullptr, mod_at(2 * n->layers), (int)M);
  if ((st = pi::check_launch("norm_kernel")) != PI_OK) return st;
  GemmParams po{};
  po.a = w.layer.a;
  po.w = w.wout;
  po.M = (int)M;
  po.N = 256;
  po.K = W;
  po.amap = RowMap{(int)M, 0, 0};
  po.out = w.vel;
  po.split_ws = w.layer.gsplit;
  if ((st = launch_gemm<E_F32>(po, s)) != PI_OK) return st;
  velocity_out_kernel<<<(unsigned)((M * A + 255) / 256), 256, 0, s>>>(w.vel, n->b_out, x, vel, M, A, dt,
                                                                       euler ? 1 : 0);
  return pi::check_launch("velocity_out_kernel");
}

// Shared checks of the two entry points; fills *w on success.
pi_status expert_setup(const pi_expert_net* n, const pi_kv_cache* cache, const uint8_t* suffix_ar, const float* x,
                       int B, int H, int A, int steps, void* workspace, size_t workspace_bytes, ExpertFlowWs* w,
                       const char* who) {
  PI_REQUIRE(expert_net_ok(n), PI_ERR_INVALID_ARG,
             "%s: the net needs every weight (matrices 16-byte aligned), 1 <= layers, a width that is a multiple "
             "of 256 (<= 4096), action_dim in [1, 256], and layers of that width with adaptive norms (mod1 + mod2)",
             who);
  PI_REQUIRE(cache && suffix_ar && x, PI_ERR_INVALID_ARG, "%s: null pointer", who);
  PI_REQUIRE(A == n->action_dim, PI_ERR_INVALID_ARG, "%s: A=%d but the net's action_dim is %d", who, A,
             n->action_dim);
  PI_REQUIRE(B >= 1 && H >= 1 && H <= 128, PI_ERR_INVALID_ARG, "%s: B=%d H=%d (1 <= H <= 128)", who, B, H);
  PI_REQUIRE(steps >= 1 && steps <= kMaxSteps, PI_ERR_INVALID_ARG, "%s: num_steps=%d (1..%d)", who, steps,
             kMaxSteps);
  PI_REQUIRE(cache->B == B && cache->Hkv == LHkv && cache->d == LD && cache->layers >= n->layers && cache->k &&
                 cache->v && cache->prefix_mask && cache->len >= 0 && cache->len <= cache->capacity,
             PI_ERR_INVALID_ARG, "%s: the cache must have B=%d, one KV head of d=256, at least %d layers and a valid "
             "length", who, B, n->layers);
  PI_REQUIRE((cache->len + TK - 1) / TK + (H + TK - 1) / TK <= kMaxTiles, PI_ERR_UNSUPPORTED,
             "%s: cache length %d too long", who, cache->len);
  const int F = expert_ffn_max(n);
  PI_REQUIRE((int64_t)B * H * F * 2 < 0x7FFF0000ll && (int64_t)B * H * LHq * LD * 2 < 0x7FFF0000ll &&
                 (int64_t)B * H * n->width * 4 < 0x7FFF0000ll,
             PI_ERR_UNSUPPORTED, "%s: an activation exceeds 2 GiB", who);
  const size_t attn_bytes = pi_decode_workspace_bytes(B, H, LHq, cache->len);
  const ExpertFlowWs need = expert_flow_ws(n->width, F, n->layers, B, H, steps, attn_bytes, nullptr);
  PI_REQUIRE(workspace && workspace_bytes >= need.total, PI_ERR_WORKSPACE, "%s: needs %zu workspace bytes, got %zu",
             who, need.total, workspace_bytes);
  PI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PI_ERR_INVALID_ARG,
             "%s: workspace must be 256-byte aligned", who);
  *w = expert_flow_ws(n->width, F, n->layers, B, H, steps, attn_bytes, static_cast<char*>(workspace));
  return PI_OK;
}

pi_status expert_pad_out(const pi_expert_net* n, const ExpertFlowWs& w, hipStream_t s) {
  const int64_t cnt = (int64_t)256 * (n->width / 8);
  pad_rows_kernel<<<(unsigned)((cnt + 255) / 256), 256, 0, s>>>(static_cast<const __bf16*>(n->w_out), w.wout,
                                                                 n->action_dim, 256, n->width);
  return pi::check_launch("pad_rows_kernel");
}

}  // namespace

extern "C" size_t pi_expert_flow_workspace_bytes(const pi_expert_net* net, int B, int H, int len, int num_steps) {
  if (!expert_net_ok(net) || B < 1 || H < 1 || H > 128 || len < 0 || num_steps < 1 || num_steps > kMaxSteps)
    return 0;
  return expert_flow_ws(net->width, expert_ffn_max(net), net->layers, B, H, num_steps,
                        pi_decode_workspace_bytes(B, H, LHq, len), nullptr)
      .total;
}

extern "C" pi_status pi_expert_velocity_eval(const pi_expert_net* net, const pi_kv_cache* cache,
                                             const uint8_t* suffix_ar, const float* x, float t, float* vel, int B,
                                             int H, int A, void* workspace, size_t workspace_bytes, pi_stream stream) {
  ExpertFlowWs w;
  pi_status st = expert_setup(net, cache, suffix_ar, x, B, H, A, 1, workspace, workspace_bytes, &w,
                              "pi_expert_velocity_eval");
  if (st != PI_OK) return st;
  PI_REQUIRE(vel != nullptr, PI_ERR_INVALID_ARG, "pi_expert_velocity_eval: null vel");
  PI_REQUIRE(isfinite(t), PI_ERR_INVALID_ARG, "pi_expert_velocity_eval: t must be finite");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = expert_pad_out(net, w, s)) != PI_OK) return st;
  if ((st = expert_cond(net, (double)t, 0.0, 1, w, s)) != PI_OK) return st;
  return expert_velocity(net, cache, suffix_ar, const_cast<float*>(x), 0, 1, vel, 0.f, false, B, H, w, s);
}

extern "C" pi_status pi_expert_flow_sample(const pi_expert_net* net, const pi_kv_cache* cache,
                                           const uint8_t* suffix_ar, float* x, int B, int H, int A, int num_steps,
                                           void* workspace, size_t workspace_bytes, pi_stream stream) {
  ExpertFlowWs w;
  pi_status st = expert_setup(net, cache, suffix_ar, x, B, H, A, num_steps, workspace, workspace_bytes, &w,
                              "pi_expert_flow_sample");
  if (st != PI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double dt = -1.0 / num_steps;
  if ((st = expert_pad_out(net, w, s)) != PI_OK) return st;
  if ((st = expert_cond(net, 1.0, dt, num_steps, w, s)) != PI_OK) return st;
  for (int k = 0; k < num_steps; ++k) {
    st = expert_velocity(net, cache, suffix_ar, x, k, num_steps, nullptr, (float)dt, true, B, H, w, s);
    if (st != PI_OK) return st;
  }
  return PI_OK;
}
