// Device and host helpers shared by the gfx950 kernels of the joint-attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pi_joint.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define PI_WAVE 64

// ---------------------------------------------------------------------------
// Matrix-core tile 16x16x32, bf16 operands, fp32 accumulate (v_mfma_f32_16x16x32_bf16).
// Lane l (g = l / 16, c = l % 16):
//   A operand (16 rows x 32 k):   A[c][8g .. 8g+7]
//   B operand (32 k x 16 cols):   B[8g .. 8g+7][c]
//   C/D       (16 x 16):          C[4g + i][c], i = 0..3
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 f2bf(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ float bf2f(__bf16 h) { return static_cast<float>(h); }

__device__ __forceinline__ bf16x8 cvt8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = f2bf(f[i]);
  return r;
}

// Butterfly reductions across the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Packed per-token mask word: bit0 valid, bits1-2 segment, bits3.. block id.
__device__ __forceinline__ bool pair_visible(uint32_t wq, uint32_t wk, uint32_t forbid) {
  bool both_valid = (wq & wk & 1u) != 0u;
  bool block_ok = (wk >> 3) <= (wq >> 3);
  uint32_t bit = 4u * ((wq >> 1) & 3u) + ((wk >> 1) & 3u);
  bool banned = (forbid >> bit) & 1u;
  return both_valid && block_ok && !banned;
}

// Rotary position embedding, rotate-half pairs (i, i + d/2): pair i turns by
// p * base^(-2i/d) radians at position p.  inv_freq = base^(-2i/d) in fp64; the
// angle is reduced to a fraction of a turn in fp64 and handed to the hardware
// sine/cosine, which take their argument in turns.
__device__ __forceinline__ double rope_inv_freq(int i, int d, double log2_base) {
  return exp2(-(2.0 * (double)i / (double)d) * log2_base);
}
__device__ __forceinline__ void rope_cos_sin(int p, double inv_freq, float& c, float& s) {
  const double turns = (double)p * inv_freq * 0.15915494309189535;   // / (2 pi)
  const float fr = (float)(turns - rint(turns));                         // [-0.5, 0.5]
  c = __builtin_amdgcn_cosf(fr);
  s = __builtin_amdgcn_sinf(fr);
}

// Matrix-core operand tile layout of an [R x K] bf16 matrix (K a multiple of 32,
// R padded to a multiple of 16): 16 x 32 tiles stored row-block major; inside a
// tile, lane 16 * ((k % 32) / 8) + r % 16 holds the 8 elements of row r starting
// at k - k % 8.  A wave then loads a whole operand fragment (A[c][8g..8g+7] of
// lane 16g + c) as one contiguous 1 KB read.
__host__ __device__ inline int64_t tiled_offset(int64_t r, int k, int K) {
  return ((r >> 4) * (K >> 5) + (k >> 5)) * 512 + (((k & 31) >> 3) * 16 + (r & 15)) * 8 + (k & 7);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace pi {
void set_error(const char* fmt, ...);
pi_status check_launch(const char* what);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
// Rotary embedding of tokens x H rows of d (bf16, y may alias x), token t at pos[t].
pi_status rope_rows(const void* x, void* y, int64_t tokens, int H, int d, const int32_t* pos, float base,
                    hipStream_t stream);
// The same for a decode suffix [B, S, H, d]: token t of sample b sits at
// (valid slots among prefix_mask[b, 0 .. P)) + t.
pi_status rope_suffix(const void* x, void* y, int B, int S, int H, int d, const uint8_t* prefix_mask, int cap,
                      int P, float base, hipStream_t stream);
// Largest decode workspace any cache length can ask for at this batch shape.
size_t decode_workspace_max(int B, int S, int Hq);
// Cached suffix decode of one layer.  q_s and o_s are row-major [B, S, Hq, d],
// or with `tiled` both are in the operand tile layout (tiled_offset): q_s as the
// rows t*Hq + head of each sample, each sample's rows padded to whole 16-row
// blocks; o_s as the [B*S x Hq*d] matrix.
pi_status decode_layer(const pi_kv_cache* cache, int layer, const void* q_s, const void* k_s, const void* v_s,
                       const uint8_t* suffix_ar, int B, int S, int Hq, float scale, float rope_base, void* o_s,
                       bool tiled, void* workspace, size_t workspace_bytes, hipStream_t stream);
}  // namespace pi

#define PI_REQUIRE(cond, code, ...)     \
  do {                                   \
    if (!(cond)) {                       \
      ::pi::set_error(__VA_ARGS__);      \
      return (code);                     \
    }                                    \
  } while (0)
