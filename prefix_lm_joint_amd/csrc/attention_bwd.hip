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
//   * dkdv32_kernel (attention32.hip, pi32::dkdv): key-major on the same engine:
//     two pairs of waves per workgroup, 32 keys per pair, with K (one wave) and
//     V (the other) rows in registers and tiles of 32 query rows (4 tokens x 8
//     heads) of Q, dO and the row statistics streamed over four LDS stages.  One
//     wave of a pair forms S = Q K^T, P and dV^T += dO^T P, the other dP =
//     dO V^T, dS = P (dP - Dr) with P passed through LDS, and dK^T += Q^T dS.
#include "common.h"
#include "engine.h"
#include "attention32.h"

#include <math.h>

namespace {

using namespace pi_engine;

constexpr int BD = 256;                       // head dim
constexpr int BG = 8;                         // query heads (the KV head is shared)
constexpr float kLog2e = 1.4426950408889634f;

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
  bwd_prep_kernel<<<(unsigned)((rows * 32 + 255) / 256), 256, 0, s>>>(
      static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse, lse2, dr, rows);
  if ((st = pi::check_launch("bwd_prep_kernel")) != PI_OK) return st;
  if ((st = pi32::dkdv(q, k, v, dout, lse2, dr, dk, dv, B, L, scale, mask, s)) != PI_OK) return st;
  if ((st = pi32::dq(q, k, v, dout, lse2, dr, dq, B, L, scale, mask, s)) != PI_OK || !rope) return st;
  const int64_t n = (int64_t)B * L;
  negate_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(mask->pos, neg_pos, n);
  if ((st = pi::check_launch("negate_kernel")) != PI_OK) return st;
  if ((st = pi::rope_rows(dq, dq, n, BG, BD, neg_pos, rope_base, s)) != PI_OK) return st;
  return pi::rope_rows(dk, dk, n, 1, BD, neg_pos, rope_base, s);
}
