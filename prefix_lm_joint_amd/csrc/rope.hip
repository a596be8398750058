// Rotary position embedding of Q or K rows, gfx950.
//
// What is computed ("VLA 代码精读 — OpenPI & StarVLA", §3.2: π0 keeps the rotary
// embedding built into its LLM; §1.5 and §1.6: the token positions): every head of
// a token at position p is rotated pairwise, dimension i < d/2 with i + d/2, by
// p * base^(-2i/d) radians (the formula is a reading; the pages name the method
// only).  V is never rotated.
//
// One thread takes 8 pairs of one (token, head) row: a 16-byte load from each
// half, fp32 arithmetic, bf16 results.  The pairs' frequencies are computed once
// per workgroup into LDS in fp64.
#include "common.h"

#include <math.h>

namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeMaxD = 512;

// x, y: bf16 [rows, d] with rows = tokens * H (y may alias x).  Position of row r:
//   positions given (DECODE false): pos[r / H];
//   decode suffix (DECODE true): per sample b (rows of b: [b*S*H, (b+1)*S*H)),
//     (valid slots among prefix_mask[b, 0 .. P)) + token index within the suffix.
template <bool DECODE>
__global__ void __launch_bounds__(kRopeThreads)
rope_kernel(const bf16x8* x, bf16x8* y, const int32_t* __restrict__ pos,
            int64_t rows, int H, int d, double log2_base, const uint8_t* __restrict__ prefix_mask, int cap,
            int P, int S) {
  __shared__ double inv_freq[kRopeMaxD / 2];
  __shared__ int n_valid;
  const int half = d / 2, per_row = half / 8;
  for (int i = threadIdx.x; i < half; i += kRopeThreads) inv_freq[i] = rope_inv_freq(i, d, log2_base);
  int64_t t0 = (int64_t)blockIdx.x * kRopeThreads;
  int b = 0;
  if (DECODE) {
    // grid.y = sample; this block's threads cover rows of sample b only
    b = blockIdx.y;
    if (threadIdx.x == 0) n_valid = 0;
    __syncthreads();
    int cnt = 0;
    const uint8_t* pm = prefix_mask + (int64_t)b * cap;
    for (int s = threadIdx.x; s < P; s += kRopeThreads) cnt += pm[s] != 0;
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&n_valid, cnt);
  }
  __syncthreads();
  const int64_t tid = t0 + threadIdx.x;
  const int64_t n_thr = DECODE ? (int64_t)S * H * per_row : rows * per_row;
  if (tid >= n_thr) return;
  const int64_t row = (DECODE ? (int64_t)b * S * H : 0) + tid / per_row;
  const int j = (int)(tid % per_row);
  const int64_t tok = row / H;
  const int p = DECODE ? n_valid + (int)(tok - (int64_t)b * S) : pos[tok];
  const int64_t base = row * (d / 8);          // in 8-element chunks
  const bf16x8 lo = x[base + j];
  const bf16x8 hi = x[base + per_row + j];
  bf16x8 ylo, yhi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c, s;
    rope_cos_sin(p, inv_freq[8 * j + e], c, s);
    const float a = bf2f(lo[e]), bb = bf2f(hi[e]);
    ylo[e] = f2bf(a * c - bb * s);
    yhi[e] = f2bf(bb * c + a * s);
  }
  y[base + j] = ylo;
  y[base + per_row + j] = yhi;
}

}  // namespace

namespace pi {

pi_status rope_rows(const void* x, void* y, int64_t tokens, int H, int d, const int32_t* pos, float base,
                    hipStream_t s) {
  const int64_t rows = tokens * H;
  const int64_t threads = rows * (d / 16);
  if (threads == 0) return PI_OK;
  rope_kernel<false><<<(unsigned)((threads + kRopeThreads - 1) / kRopeThreads), kRopeThreads, 0, s>>>(
      static_cast<const bf16x8*>(x), static_cast<bf16x8*>(y), pos, rows, H, d, log2((double)base), nullptr, 0,
      0, 0);
  return check_launch("rope_kernel");
}

pi_status rope_suffix(const void* x, void* y, int B, int S, int H, int d, const uint8_t* prefix_mask, int cap,
                      int P, float base, hipStream_t s) {
  const int64_t threads = (int64_t)S * H * (d / 16);
  if (threads == 0) return PI_OK;
  const dim3 grid((unsigned)((threads + kRopeThreads - 1) / kRopeThreads), (unsigned)B);
  rope_kernel<true><<<grid, kRopeThreads, 0, s>>>(static_cast<const bf16x8*>(x), static_cast<bf16x8*>(y), nullptr,
                                                  (int64_t)B * S * H, H, d, log2((double)base), prefix_mask, cap, P,
                                                  S);
  return check_launch("rope_kernel");
}

}  // namespace pi

extern "C" pi_status pi_rope_apply(const void* x, void* y, int B, int L, int H, int d, const int32_t* pos,
                                   float base, pi_stream stream) {
  PI_REQUIRE(x && y && pos, PI_ERR_INVALID_ARG, "pi_rope_apply: null pointer");
  PI_REQUIRE(pi::aligned16(x) && pi::aligned16(y), PI_ERR_INVALID_ARG, "pi_rope_apply: x and y must be 16-byte aligned");
  PI_REQUIRE(B >= 1 && L >= 1 && H >= 1, PI_ERR_INVALID_ARG, "pi_rope_apply: B=%d L=%d H=%d", B, L, H);
  PI_REQUIRE(d >= 16 && d <= kRopeMaxD && d % 16 == 0, PI_ERR_UNSUPPORTED,
             "pi_rope_apply: d=%d must be a multiple of 16 in [16, %d]", d, kRopeMaxD);
  PI_REQUIRE(base > 1.f && std::isfinite(base), PI_ERR_INVALID_ARG, "pi_rope_apply: base must be > 1");
  return pi::rope_rows(x, y, (int64_t)B * L, H, d, pos, base, static_cast<hipStream_t>(stream));
}
